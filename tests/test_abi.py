"""CPU-side checks of the C ABI: the library loads, exports every entry point
that include/ep.h declares, and its host-only logic (sizes, argument checks)
behaves as documented. No kernel is launched here."""
import ctypes
import os
import re

import pytest

from combine_get_layout_amd import ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(ep_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ep.LIB_PATH):
        from combine_get_layout_amd import build
        build.build()
    return ep.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ep.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_sizes_match_oracle(lib, oracle_lib):
    for (T, H, K, E, R, G) in [(128, 256, 2, 16, 4, 1), (4096, 7168, 8, 256, 32, 1),
                               (16384, 7168, 8, 256, 64, 8), (5, 384, 3, 12, 6, 3)]:
        s = ep.make_shape(T, H, K, E, R, G)
        for seg, fl in [(1, (1, 0, 0)), (3, (1, 1, 0)), (7, (1, 1, 1))]:
            P = oracle_lib.record_bytes(H, K, *fl)
            assert ep.ep_record_bytes(s, seg) == P
            assert ep.ep_chunked_record_bytes(s, seg) == oracle_lib.chunked_bytes(P)
        assert ep.ep_workspace_bytes(s) >= 256


def test_bad_shapes_rejected(lib):
    bad = [(-1, 256, 2, 16, 4, 1), (8, 250, 2, 16, 4, 1), (8, 256, 0, 16, 4, 1),
           (8, 256, 2, 15, 4, 1), (8, 256, 2, 16, 4, 3)]
    for b in bad:
        assert ep.ep_workspace_bytes(ep.make_shape(*b)) == 0
    unsupported = [(8, 256, 65, 16, 4, 1), (8, 256, 2, 8192, 8, 1), (8, 256, 2, 2048, 2048, 1)]
    for u in unsupported:
        s = ep.make_shape(*u)
        assert ep.ep_workspace_bytes(s) == 0
        rc = lib.ep_get_layout(ctypes.byref(s), None, None, None, 0, None)
        assert rc == ep.EP_ERR_UNSUPPORTED
    s = ep.make_shape(8, 264, 2, 16, 4, 1)
    assert ep.ep_record_bytes(s, ep.EP_SEG_SCALES) == -1  # scales need H % 128 == 0


def test_null_and_misaligned_arguments_rejected_before_launch(lib):
    s = ep.make_shape(128, 256, 2, 16, 4, 1)
    L = ep.ep_layout()
    # no workspace
    assert lib.ep_get_layout(ctypes.byref(s), 0x1000, ctypes.byref(L), None, 1 << 20, None) == ep.EP_ERR_ARG
    # misaligned workspace
    assert lib.ep_get_layout(ctypes.byref(s), 0x1000, ctypes.byref(L), 0x1010, 1 << 20, None) == ep.EP_ERR_ARG
    # undersized workspace
    assert lib.ep_get_layout(ctypes.byref(s), 0x1000, ctypes.byref(L), 0x1000, 16, None) == ep.EP_ERR_ARG
    tk = ep.ep_tokens()
    rv = ep.ep_recv()
    ws = 0x100000
    n = ep.ep_workspace_bytes(s)
    assert lib.ep_dispatch(ctypes.byref(s), ctypes.byref(L), ctypes.byref(tk), ctypes.byref(rv),
                           ws, n, None) == ep.EP_ERR_ARG  # no slot / topk
    # epoch 0 is refused by the two-level path and by chunked combine
    assert lib.ep_hierarchical_dispatch(ctypes.byref(s), ctypes.byref(L), ctypes.byref(tk), 0, 3,
                                        None, 0, None, 0, ws, n, None) == ep.EP_ERR_ARG
    assert lib.ep_combine(ctypes.byref(s), ctypes.byref(L), 0x2000, 4, 1024, ep.EP_FMT_CHUNKED, 0,
                          0x3000, 0x4000, ws, n, None) == ep.EP_ERR_ARG
    # plain stride smaller than a row
    assert lib.ep_combine(ctypes.byref(s), ctypes.byref(L), 0x2000, 4, 256, ep.EP_FMT_PLAIN, 0,
                          0x3000, 0x4000, ws, n, None) == ep.EP_ERR_ARG
    assert lib.ep_clear_errors(None, None) == ep.EP_ERR_ARG
    assert lib.ep_check_errors(None, None, None) == ep.EP_ERR_ARG
    assert lib.ep_check_sticky_errors(None, None, None) == ep.EP_ERR_ARG
    # the allocation-free layout refuses, before any launch, a shape whose
    # count tables exceed its static scratch array
    big = ep.make_shape(1 << 20, 7168, 8, 256, 64, 1)
    assert ep.ep_workspace_bytes(big) > ep.EP_LAYOUT_SCRATCH_BYTES
    assert lib.ep_get_layout_noalloc(ctypes.byref(big), 0x1000, ctypes.byref(L), 0x2000, None) == ep.EP_ERR_SCRATCH
    assert lib.ep_get_layout_noalloc(ctypes.byref(s), 0x1000, ctypes.byref(L), None, None) == ep.EP_ERR_ARG
    assert ep.EP_ERR_DEVICE == -4 and "device" in ep.ep_status_string(ep.EP_ERR_DEVICE)
    assert ep.ep_status_string(0) == "ok"


def test_fused_options_checked_before_launch(lib):
    """The fused two-level dispatch refuses batch sizes outside 1..64, unknown
    test flags, ring sizes of 64 batches or fewer (or more than group_cap rows)
    and epoch 0 on the host; with T = 0 it enqueues nothing."""
    s = ep.make_shape(128, 256, 4, 32, 8, 4)
    n = ep.ep_workspace_bytes(s)
    ws = 0x100000
    L = ep.ep_layout(None, None, None, None, None, 0x3000, None, None, 0x4000, 0x5000, None)
    tk = ep.ep_tokens(0x6000, None, None, 0x7000, 0x8000)

    def call(opts, epoch=3):
        return lib.ep_hierarchical_dispatch_fused(ctypes.byref(s), ctypes.byref(L), ctypes.byref(tk), epoch,
                                                  0x10000, 10, 0x20000, 10, opts, ws, n, None)

    assert call(ctypes.byref(ep.ep_fused_opts(65, 0, 0, 0))) == ep.EP_ERR_ARG
    assert call(ctypes.byref(ep.ep_fused_opts(-1, 0, 0, 0))) == ep.EP_ERR_ARG
    assert call(ctypes.byref(ep.ep_fused_opts(16, 0, 2, 0))) == ep.EP_ERR_ARG  # unknown test flag
    assert call(ctypes.byref(ep.ep_fused_opts(1, 0, 0, 0, 64))) == ep.EP_ERR_ARG  # ring not above the lag
    assert call(ctypes.byref(ep.ep_fused_opts(1, 0, 0, 0, -1))) == ep.EP_ERR_ARG
    assert call(ctypes.byref(ep.ep_fused_opts(1, 0, 0, 0, 65))) == ep.EP_ERR_ARG  # 260 ring rows > group_cap 10
    big = lib.ep_hierarchical_dispatch_fused(ctypes.byref(s), ctypes.byref(L), ctypes.byref(tk), 3, 0x10000,
                                             1 << 40, 0x20000, 10, ctypes.byref(ep.ep_fused_opts(64, 0, 0, 0, 1 << 24)),
                                             ws, n, None)
    assert big == ep.EP_ERR_ARG  # 2^24 * 64 * 4 ring rows: past 32-bit row indices
    assert call(None, epoch=0) == ep.EP_ERR_ARG
    z = ep.make_shape(0, 256, 4, 32, 8, 4)
    assert lib.ep_hierarchical_dispatch_fused(ctypes.byref(z), ctypes.byref(L), ctypes.byref(tk), 3, None, 0,
                                              None, 0, None, ws, ep.ep_workspace_bytes(z), None) == ep.EP_OK


def test_zero_tokens_dispatch_and_combine_enqueue_nothing(lib):
    """With T = 0 there is nothing to read or write: both calls succeed
    without touching the device (so this runs without a GPU)."""
    s = ep.make_shape(0, 256, 2, 16, 4, 1)
    n = ep.ep_workspace_bytes(s)
    L = ep.ep_layout()
    tk = ep.ep_tokens()
    rv = ep.ep_recv(0x2000, None, None, 0x3000, None, None, 0)
    ws = 0x100000
    assert lib.ep_dispatch(ctypes.byref(s), ctypes.byref(L), ctypes.byref(tk), ctypes.byref(rv),
                           ws, n, None) == ep.EP_OK
    assert lib.ep_combine(ctypes.byref(s), ctypes.byref(L), None, 0, 512, ep.EP_FMT_PLAIN, 0,
                          None, None, ws, n, None) == ep.EP_OK


def test_source_calls_checked_before_launch(lib):
    s = ep.make_shape(4096, 7168, 8, 256, 32, 1)
    base = ep.ep_workspace_bytes(s)
    n = ep.ep_source_workspace_bytes(s, 32)
    assert n > base and n % 256 == 0
    # one tile of 128 tokens per source: [S][1][R] int32 counts after the layout workspace
    assert n - base == 32 * 1 * 32 * 4
    assert ep.ep_source_workspace_bytes(s, 0) == 0
    assert ep.ep_source_workspace_bytes(s, 2048) == 0
    ws = 0x100000

    def src(S=32, cap=128):
        return ep.ep_sources(S, cap, 0x2000, 0x3000, 0x4000)

    X = src()
    assert lib.ep_source_layout(ctypes.byref(s), 0x1000, ctypes.byref(X), ws, base, None) == ep.EP_ERR_ARG
    X = src(S=0)
    assert lib.ep_source_layout(ctypes.byref(s), 0x1000, ctypes.byref(X), ws, n, None) == ep.EP_ERR_ARG
    X = src(cap=-1)
    assert lib.ep_source_layout(ctypes.byref(s), 0x1000, ctypes.byref(X), ws, n, None) == ep.EP_ERR_ARG
    X = src(cap=1 << 22)  # R * S * capacity beyond int32 rows
    assert lib.ep_source_layout(ctypes.byref(s), 0x1000, ctypes.byref(X), ws, n, None) == ep.EP_ERR_UNSUPPORTED
    X = src()
    tk = ep.ep_tokens()
    assert lib.ep_source_dispatch(ctypes.byref(s), ctypes.byref(X), ctypes.byref(tk), 1, 0x5000,
                                  ws, n, None) == ep.EP_ERR_ARG  # no x / topk / weights
    tk = ep.ep_tokens(0x10000, None, None, 0x20000, 0x30000)
    assert lib.ep_source_dispatch(ctypes.byref(s), ctypes.byref(X), ctypes.byref(tk), 0, 0x5000,
                                  ws, n, None) == ep.EP_ERR_ARG  # epoch 0
    rv = ep.ep_recv(0x10000, 0x20000, None, None, None, None, 100)
    # fp8 receive rows asked for but not in the record
    assert lib.ep_copy_epilogue(ctypes.byref(s), ctypes.byref(X), 0x5000, 1, ep.EP_SEG_BF16,
                                ctypes.byref(rv), ws, n, None) == ep.EP_ERR_ARG
    assert lib.ep_copy_epilogue(ctypes.byref(s), ctypes.byref(X), 0x5000, 1, ep.EP_SEG_FP8,
                                ctypes.byref(rv), ws, n, None) == ep.EP_ERR_ARG  # no bf16 piece


def test_binding_rejects_host_small_and_strided_tensors():
    """The binding checks every tensor argument before the C call: on the GPU,
    contiguous and at least as long as the shape needs (no GPU required: the
    checks fire before any kernel could run)."""
    import pytest
    import torch

    from combine_get_layout_amd import ep

    shape = ep.make_shape(4, 16, 2, 8, 4, 1)
    cpu = torch.zeros(4 * 2, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU tensor"):
        ep._ptr(cpu, "topk_idx", 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        ep._layout_struct(shape, dict(slot=torch.zeros((4, 2), dtype=torch.int32)))
    assert ep._ptr(None, "x", 100) is None
    assert ep._ptr(12345, "x", 100) == 12345  # a raw device address passes through


class _FakeCuda:
    """Minimal stand-in for a GPU tensor's metadata (no device needed)."""
    def __init__(self, nbytes, contiguous=True):
        self.is_cuda = True
        self._n = nbytes
        self._c = contiguous

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def data_ptr(self):
        return 4096


def test_binding_size_and_stride_checks():
    import pytest

    from combine_get_layout_amd import ep

    assert ep._ptr(_FakeCuda(64), "topk_idx", 64) == 4096
    with pytest.raises(ValueError, match="needs 65"):
        ep._ptr(_FakeCuda(64), "topk_idx", 65)
    with pytest.raises(ValueError, match="contiguous"):
        ep._ptr(_FakeCuda(64, contiguous=False), "x", 8)
    shape = ep.make_shape(5, 256, 3, 12, 4, 2)
    # recv rows: capacity * H * 2 bytes of bf16
    with pytest.raises(ValueError, match="recv x"):
        ep._recv_struct(shape, dict(x=_FakeCuda(10 * 256 * 2 - 2)), 10)
    ep._recv_struct(shape, dict(x=_FakeCuda(10 * 256 * 2)), 10)


def test_plain_c_caller(lib, tmp_path):
    """include/ep.h is a C header: a C99 program built with gcc links libep.so
    and its host-only calls behave as documented (tests/c/abi_from_c.c)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    libdir = os.path.dirname(ep.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    src = os.path.join(ROOT, "tests", "c", "abi_from_c.c")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                        src, f"-L{libdir}", "-l:libep.so", f"-Wl,-rpath,{libdir}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
