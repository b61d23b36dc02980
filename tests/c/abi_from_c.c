/* A plain C99 caller of libep.so, built with gcc against include/ep.h: the
 * header is a C header and the library's host-only entry points (sizes,
 * argument checks, status strings) behave as documented when called from C.
 * Nothing here touches a GPU: every call below returns before any kernel
 * launch. Prints one line per check and exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ep.h"

static int failures = 0;

static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok) failures++;
}

int main(void) {
    ep_shape s = {4096, 7168, 8, 256, 32, 1};
    /* record: bf16 row 14336 B + ids 32 + weights 32 + src 16 = 14416 B;
     * 31 blocks of 480 B payload -> 15872 B chunked */
    check(ep_record_bytes(&s, EP_SEG_BF16) == 14416, "record bytes, bf16 only");
    check(ep_chunked_record_bytes(&s, EP_SEG_BF16) == 15872, "chunked record bytes");
    check(ep_record_bytes(&s, EP_SEG_BF16 | EP_SEG_FP8 | EP_SEG_SCALES) == 14416 + 7168 + 224,
          "record bytes with FP8 and scales");
    check(ep_partial_row_bytes(&s) == 512 * 30, "partial row bytes");
    check(ep_workspace_bytes(&s) >= 256, "workspace bytes");

    ep_shape bad = s;
    bad.H = 7170; /* not a multiple of 8 */
    check(ep_workspace_bytes(&bad) == 0, "bad H rejected by the size query");
    bad = s;
    bad.K = 65;
    ep_layout L;
    memset(&L, 0, sizeof L);
    check(ep_get_layout(&bad, NULL, &L, NULL, 0, NULL) == EP_ERR_UNSUPPORTED, "K = 65 unsupported");
    check(ep_get_layout(&s, (const int64_t *)0x1000, &L, NULL, 1 << 20, NULL) == EP_ERR_ARG,
          "missing workspace rejected");
    check(ep_get_layout(&s, (const int64_t *)0x1000, &L, (void *)0x1010, 1 << 20, NULL) == EP_ERR_ARG,
          "misaligned workspace rejected");
    check(ep_get_layout(NULL, NULL, &L, NULL, 0, NULL) == EP_ERR_ARG, "null shape rejected");

    ep_recv rv;
    memset(&rv, 0, sizeof rv);
    ep_tokens tk;
    memset(&tk, 0, sizeof tk);
    check(ep_dispatch(&s, &L, &tk, &rv, NULL, 0, NULL) == EP_ERR_ARG, "dispatch without workspace");
    check(ep_clear_errors(NULL, NULL) == EP_ERR_ARG, "clear_errors without workspace");
    uint32_t bits = 7;
    check(ep_check_errors(NULL, NULL, &bits) == EP_ERR_ARG, "check_errors without workspace");
    check(ep_check_sticky_errors(NULL, NULL, &bits) == EP_ERR_ARG, "check_sticky_errors without workspace");
    check(bits == 7, "bits left unchanged when the word cannot be read");
    check(strstr(ep_status_string(EP_ERR_DEVICE), "device") != NULL, "status string of EP_ERR_DEVICE");

    check(strcmp(ep_status_string(EP_OK), "ok") == 0, "status string of EP_OK");
    check(strlen(ep_status_string(EP_ERR_HIP)) > 0, "status string of EP_ERR_HIP");
    check(strcmp(ep_status_string(12345), "unknown status") == 0, "status string of an unknown code");

    printf("%d failure(s)\n", failures);
    return failures ? 1 : 0;
}
