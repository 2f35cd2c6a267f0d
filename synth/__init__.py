"""Seeded synthetic inputs shaped like the ternary-g128 decode/prefill
workloads of the 27B-class model the pages describe.

This module only draws random numbers and rounds them to the storage dtypes
(binary16 scales, bfloat16 or binary32 activations, int8 ternary values and
+-1 signs).  It holds none of the method's arithmetic: no packing, no
dequantization, no matmul, no transform.  Both the oracle-side tests and the
HIP-side tests and benchmark take their inputs from here.

Every array comes from its own child stream of
``numpy.random.SeedSequence(seed)``, so adding an array never shifts the
others.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128

# child-stream indices: one per array role
_S_T, _S_SCALE, _S_X, _S_SIGNS, _S_OUTLIER = range(5)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def _ternary_from_uniform(u: np.ndarray, p_zero: float) -> np.ndarray:
    half = (1.0 - p_zero) / 2.0
    t = np.zeros(u.shape, dtype=np.int8)
    t[u < half] = -1
    t[u >= half + p_zero] = 1
    return t


def ternary(seed: int, N: int, K: int, p_zero: float = 1.0 / 3.0) -> np.ndarray:
    """int8 [N, K], i.i.d. with P(0) = p_zero and P(+1) = P(-1) = (1-p_zero)/2."""
    return np.concatenate(list(ternary_chunks(seed, N, K, p_zero)), axis=0) if N else \
        np.zeros((0, K), dtype=np.int8)


def ternary_chunks(seed: int, N: int, K: int, p_zero: float = 1.0 / 3.0,
                   max_elems: int = 1 << 23):
    """The rows of ternary(seed, N, K, p_zero), yielded in consecutive row
    chunks of at most max_elems elements (the same stream, drawn in order),
    so large matrices never exist in float64 on the host."""
    r = _rng(seed, _S_T)
    rows = max(1, max_elems // max(K, 1))
    for n0 in range(0, N, rows):
        nr = min(rows, N - n0)
        yield _ternary_from_uniform(r.random((nr, K)), p_zero)


def scales_f16(seed: int, N: int, K: int, sigma: float = 0.02, floor: float = 1e-3) -> np.ndarray:
    """binary16 bit patterns [N, K/128] of |N(0, sigma)| + floor, drawn in
    float64 and rounded to nearest-even binary16."""
    r = _rng(seed, _S_SCALE)
    v = np.abs(r.normal(0.0, sigma, size=(N, K // GROUP))) + floor
    return v.astype(np.float16).view(np.uint16)


def _f32_to_bf16_bits(v32: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, round to nearest even (the storage
    rounding of an input, done through torch's CPU conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations_f32(seed: int, M: int, K: int) -> np.ndarray:
    """float32 [M, K] ~ N(0, 1) (drawn in float64, rounded to binary32)."""
    r = _rng(seed, _S_X)
    return r.normal(0.0, 1.0, size=(M, K)).astype(np.float32)


def activations_bf16(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                     outlier_gain: float = 20.0) -> np.ndarray:
    """bfloat16 bit patterns [M, K] of N(0, 1).  With outlier_frac > 0,
    round(outlier_frac * K) distinct K-columns, drawn without replacement,
    are multiplied by outlier_gain in binary32 before the bfloat16 rounding."""
    v = activations_f32(seed, M, K)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = _rng(seed, _S_OUTLIER).choice(K, size=n_out, replace=False)
        v[:, cols] = v[:, cols] * np.float32(outlier_gain)
    return _f32_to_bf16_bits(v)


def signs(seed: int, K: int) -> np.ndarray:
    """int8 [K] Rademacher +-1."""
    r = _rng(seed, _S_SIGNS)
    return np.where(r.random(K) < 0.5, -1, 1).astype(np.int8)


def sign_bytes(seed: int, K: int) -> np.ndarray:
    """int8 [K] drawn from the whole int8 range, with 0, +-1, +-2, -128 and
    127 each drawn often: sign vectors whose entries are not all +-1."""
    r = _rng(seed, _S_SIGNS)
    special = np.array([0, 1, -1, 2, -2, -128, 127], dtype=np.int16)
    v = np.where(r.random(K) < 0.5, special[r.integers(0, len(special), K)], r.integers(-128, 128, K))
    return v.astype(np.int8)


# ---------------------------------------------------------------------------
# Named workloads (shapes of one 27B-class projection and its neighbours)
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    M: int
    K: int
    N: int
    x_dtype: str             # "f32" or "bf16"
    p_zero: float = 1.0 / 3.0
    rotate_block: int = 0     # >0: signed normalized WHT of this block first
    outlier_frac: float = 0.0
    notes: str = ""


TINY = Workload("tiny gemv M1 K1024 N1024", 1, 1024, 1024, "f32")
ROTATED = Workload("rotated decode gemv M1 K4096 N12288", 1, 4096, 12288, "bf16",
                   p_zero=0.35, rotate_block=4096)
SWEEP = [Workload(f"decode sweep M{m} K{k} N{n}", m, k, n, "bf16")
         for m in (1, 2, 4, 8, 16) for (k, n) in ((5120, 17408), (17408, 5120))]
PREFILL = [Workload(f"prefill gemm M512 K{k} N{n}", 512, k, n, "bf16", p_zero=0.35,
                    outlier_frac=0.01) for (k, n) in ((5120, 17408), (17408, 5120))]

# One decode step of a 64-block 27B-class stack: per block an attention-like
# pair (5120->12288, 6144->5120), the MLP gate and up projections (5120->17408
# each, the same input, stored as one 34816-row matrix: rows 0..17407 gate,
# 17408..34815 up) and a down projection (17408->5120); then a 5120->248320
# LM head.  (K, N) per link.
CHAIN_GATE_UP = 17408
CHAIN_BLOCK = [(5120, 12288), (6144, 5120), (5120, 2 * CHAIN_GATE_UP), (17408, 5120)]
CHAIN_BLOCKS = 64
LM_HEAD = (5120, 248320)


def chain_links(blocks: int = CHAIN_BLOCKS):
    links = [kn for _ in range(blocks) for kn in CHAIN_BLOCK]
    links.append(LM_HEAD)
    return links


@dataclass
class Problem:
    """Materialized inputs of one ternary matmul problem (host arrays)."""
    t: np.ndarray            # int8 [N, K]
    scales: np.ndarray       # uint16 binary16 bits [N, K/128]
    x: np.ndarray            # float32 [M, K] or uint16 bfloat16 bits [M, K]
    signs: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def make_problem(w: Workload, seed: int) -> Problem:
    t = ternary(seed, w.N, w.K, w.p_zero)
    s = scales_f16(seed, w.N, w.K)
    if w.x_dtype == "f32":
        x = activations_f32(seed, w.M, w.K)
    else:
        x = activations_bf16(seed, w.M, w.K, w.outlier_frac)
    d = signs(seed, w.K) if w.rotate_block else None
    return Problem(t, s, x, d, {"workload": w.name, "seed": seed})


# ---------------------------------------------------------------------------
# Device-side draws for workloads too large to generate on the host (the
# 27B-class pass: 24.4 G weights).  Same distributions; torch's seeded CUDA
# generator instead of PCG64.  Generation only: packing happens elsewhere.
# ---------------------------------------------------------------------------

def device_generator(seed: int):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def device_ternary(gen, rows: int, K: int):
    """int8 [rows, K] on the GPU, i.i.d. uniform over {-1, 0, +1}."""
    import torch
    return torch.randint(-1, 2, (rows, K), dtype=torch.int8, device="cuda", generator=gen)


def device_scales_f16(gen, N: int, K: int):
    """binary16 scales [N, K/128] on the GPU: |N(0, 0.02)| + 1e-3."""
    import torch
    return (torch.randn((N, K // 128), device="cuda", generator=gen).abs_() * 0.02 + 1e-3).half()


def device_activations_bf16(gen, M: int, K: int):
    import torch
    return torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
