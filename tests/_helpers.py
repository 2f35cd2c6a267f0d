"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the FP64 oracle."""
from __future__ import annotations

import numpy as np

import synth

# Matmul tolerance: |y - exact| <= REL_TOL * sum_k |s_g t x_k| per element.
REL_TOL = 1e-4
# FWHT tolerance: relative L2 error per row.
FWHT_TOL = 1e-5
# bfloat16 output: round to nearest even adds at most 2^-8 relative (8-bit significand).
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def torch():
    import torch as _t
    return _t


def x_to_device(x: np.ndarray):
    """float32 host array -> float32 tensor; uint16 bf16 bits -> bfloat16 tensor."""
    T = torch()
    if x.dtype == np.float32:
        return T.from_numpy(np.ascontiguousarray(x)).cuda()
    assert x.dtype == np.uint16
    return T.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(T.bfloat16)


def y_to_host(y) -> np.ndarray:
    T = torch()
    if y.dtype == T.bfloat16:
        bits = y.view(T.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def pack_to_device(tern, t: np.ndarray, s: np.ndarray):
    codes, s2 = tern.tern_pack(t, s)
    return tern.to_device(codes, s2)


def assert_matmul_close(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray,
                        bf16_out: bool = False, what: str = ""):
    allow = REL_TOL * bound
    if bf16_out:
        allow = allow * (1 + BF16_UNIT_ROUNDOFF) + BF16_UNIT_ROUNDOFF * np.abs(y_ref)
    err = np.abs(y_gpu - y_ref)
    bad = ~(err <= allow)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance; first at {tuple(i)}: "
            f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")


def assert_fwht_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    y_gpu = np.atleast_2d(y_gpu)
    y_ref = np.atleast_2d(y_ref)
    for r in range(y_ref.shape[0]):
        nref = np.linalg.norm(y_ref[r])
        nerr = np.linalg.norm(y_gpu[r] - y_ref[r])
        if nref == 0:
            assert nerr == 0, f"{what}: row {r} must be exactly zero"
        else:
            assert nerr <= FWHT_TOL * nref, f"{what}: row {r} rel L2 {nerr / nref:.3e}"


def sampled_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices: first, last, a ragged-tile row and random."""
    rng = np.random.default_rng(seed)
    picks = {0, N - 1, max(0, N - 17), N // 2}
    picks.update(rng.choice(N, size=min(count, N), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def oracle_threads(oracle_lib) -> int:
    """Host threads for the threaded oracle (bit-identical to one thread);
    at most 16, the host share of one GPU."""
    return max(1, min(16, oracle_lib.max_threads()))


def full_problem(tern, seed: int, N: int, K: int, p_zero: float):
    """A whole seeded matrix on the device and on the host (int8 t and the
    binary16 scale bits), for every-element comparisons.  The same stream
    as big_problem."""
    t = synth.ternary(seed, N, K, p_zero)
    s = synth.scales_f16(seed, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    return codes_d, scales_d, t, s


def big_problem(tern, seed: int, N: int, K: int, p_zero: float, rows: np.ndarray):
    """Pack a large seeded matrix chunk by chunk straight to device memory,
    keeping the int8 rows `rows` for the oracle.  Returns (codes_dev,
    scales_dev, t_rows, s_rows)."""
    T = torch()
    s = synth.scales_f16(seed, N, K)
    codes_dev = T.empty((N, K // 16), dtype=T.int32, device="cuda")
    keep = []
    n0 = 0
    for chunk in synth.ternary_chunks(seed, N, K, p_zero):
        nr = chunk.shape[0]
        c, _ = tern.tern_pack(chunk, s[n0:n0 + nr])
        codes_dev[n0:n0 + nr].copy_(T.from_numpy(c.view(np.int32)))
        sel = rows[(rows >= n0) & (rows < n0 + nr)]
        if len(sel):
            keep.append(chunk[sel - n0])
        n0 += nr
    t_rows = np.concatenate(keep, axis=0)
    scales_dev = T.from_numpy(s.view(np.int16)).cuda()
    return codes_dev, scales_dev, t_rows, s[rows]
