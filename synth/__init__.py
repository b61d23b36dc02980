"""Seeded synthetic inputs for the MoE dispatch / combine path.

This module only draws inputs: it holds none of the path's arithmetic (no
layout, no routing, no record format, no combine). Both the HIP path's tests
and benchmark and the CPU oracle's tests take their inputs from here.

Workloads (shapes after the examples on the pages: E = 256 / top-8 and
E = 2048 / top-8 in the expected-distinct-ranks discussion of the DeepEP V2
deep-dive page, BF16 hidden + FP32 top-k weights on the Ascend page):

=========  =====  ====  ====  ===  ===  =  =============================
name       T      H     E     R    G    K  routing
=========  =====  ====  ====  ===  ===  =  =============================
tiny       128    256   16    4    1    2  uniform distinct
ep32       4096   7168  256   32   1    8  uniform distinct (+ FP8 option)
ep256      8192   7168  256   256  1    8  uniform distinct
zipf       16384  4096  2048  256  1    8  Zipf(1.2) without replacement
hier8x8    16384  7168  256   64   8    8  uniform distinct, two-level
many       262144 256   256   32   1    8  uniform distinct (1,024 layout
                                            workgroups; not a target config)
=========  =====  ====  ====  ===  ===  =  =============================

Recipe (numpy PCG64, seed = 20261200 + workload index unless given):
  x        ~ N(0, 1) float32, rounded to bfloat16 (nearest, ties to even)
  topk_idx uniform distinct: per token sort E iid U(0,1) keys, keep the K
           smallest in key order; Zipf: p_i ~ i^-1.2 over a seeded random
           permutation of expert ids, K draws without replacement by
           Gumbel-top-k (keys log p + Gumbel(0,1), descending)
  topk_w   float32 softmax (max subtracted) of N(0,1) float32 logits
  x_fp8    per token and 128-channel block: scale = amax / 448 (1 if amax
           is 0), q = e4m3fn(x / scale) rounded to nearest even
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

BASE_SEED = 20261200


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    R: int
    G: int
    K: int
    routing: str  # "uniform" or "zipf"
    zipf_s: float = 1.2

    @property
    def index(self) -> int:
        return [w.name for w in WORKLOADS].index(self.name)

    def scaled(self, T: int, name: str | None = None) -> "Workload":
        return Workload(name or f"{self.name}_T{T}", T, self.H, self.E, self.R, self.G, self.K,
                        self.routing, self.zipf_s)


WORKLOADS = [
    Workload("tiny", 128, 256, 16, 4, 1, 2, "uniform"),
    Workload("ep32", 4096, 7168, 256, 32, 1, 8, "uniform"),
    Workload("ep256", 8192, 7168, 256, 256, 1, 8, "uniform"),
    Workload("zipf", 16384, 4096, 2048, 256, 1, 8, "zipf"),
    Workload("hier8x8", 16384, 7168, 256, 64, 8, 8, "uniform"),
    # Beyond the five configurations: many layout workgroups (1,024 of 256
    # tokens) over a narrow hidden row, so the layout's share of a step is large.
    Workload("many", 262144, 256, 256, 32, 1, 8, "uniform"),
]


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def seed_of(w: Workload) -> int:
    names = [x.name for x in WORKLOADS]
    return BASE_SEED + (names.index(w.name) if w.name in names else 99)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (torch's cast: nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def topk_uniform(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    out = np.empty((T, K), np.int64)
    step = max(1, (1 << 24) // max(E, 1))
    for t0 in range(0, T, step):
        keys = rng.random((min(step, T - t0), E))
        out[t0:t0 + keys.shape[0]] = np.argsort(keys, axis=1, kind="stable")[:, :K]
    return out


def topk_zipf(rng: np.random.Generator, T: int, E: int, K: int, s: float) -> np.ndarray:
    perm = rng.permutation(E)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    logp -= np.log(np.exp(logp).sum())
    out = np.empty((T, K), np.int64)
    step = max(1, (1 << 23) // max(E, 1))
    for t0 in range(0, T, step):
        n = min(step, T - t0)
        u = rng.random((n, E))
        gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
        order = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :K]
        out[t0:t0 + n] = perm[order]
    return out


def softmax_weights(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    logits = rng.standard_normal((T, K), dtype=np.float32)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def fp8_quantize(x_bits: np.ndarray):
    """Per-128-channel e4m3fn codes + float32 scales of bf16 rows."""
    T, H = x_bits.shape
    assert H % 128 == 0
    xf = bf16_to_float(x_bits).reshape(T, H // 128, 128)
    amax = np.abs(xf).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(xf / scale[:, :, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q.reshape(T, H)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), scale


def make_inputs(w: Workload, seed: int | None = None, with_fp8: bool = False,
                with_x: bool = True) -> dict:
    """Seeded inputs of workload w as numpy arrays:
    x [T,H] uint16 (bf16 bits), topk_idx [T,K] int64, topk_w [T,K] float32,
    and if with_fp8: x_fp8 [T,H] uint8 (e4m3fn), x_scales [T,H/128] float32."""
    rng = np.random.Generator(np.random.PCG64(seed_of(w) if seed is None else seed))
    out = {}
    if with_x:
        out["x"] = bf16_bits(rng.standard_normal((w.T, w.H), dtype=np.float32))
    if w.routing == "uniform":
        out["topk_idx"] = topk_uniform(rng, w.T, w.E, w.K)
    elif w.routing == "zipf":
        out["topk_idx"] = topk_zipf(rng, w.T, w.E, w.K, w.zipf_s)
    else:
        raise ValueError(w.routing)
    out["topk_w"] = softmax_weights(rng, w.T, w.K)
    if with_fp8:
        assert with_x
        out["x_fp8"], out["x_scales"] = fp8_quantize(out["x"])
    return out


def random_bf16_rows(rows: int, H: int, seed: int) -> np.ndarray:
    """Stand-in expert outputs: N(0,1) rows rounded to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(rng.standard_normal((rows, H), dtype=np.float32))
