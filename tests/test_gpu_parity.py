"""GPU parity: the HIP path through the C ABI against the FP64 oracle.

Matmul: |y - exact| <= 1e-4 * sum_k |s_g t x_k| per element (bit-exact where
the arithmetic is exact).  FWHT: relative L2 error <= 1e-5 per row.  Inputs
are seeded synthetic arrays from synth; expected values come only from the
oracle.
"""
import numpy as np
import pytest

import synth
from tests._helpers import (assert_fwht_close, assert_matmul_close, big_problem, full_problem,
                            oracle_threads, pack_to_device, sampled_rows, torch, x_to_device, y_to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tern():
    T = torch()
    if not T.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_g128_amd as t
    return t


def _x(seed, M, K, xdt):
    return synth.activations_f32(seed, M, K) if xdt == "f32" else synth.activations_bf16(seed, M, K)


def _run_gemv(tern, x, codes_d, scales_d, ydt="f32"):
    T = torch()
    out_dtype = T.float32 if ydt == "f32" else T.bfloat16
    y = tern.tern_gemv(x_to_device(x), codes_d, scales_d, out_dtype=out_dtype)
    T.cuda.synchronize()
    return y_to_host(y)


# ---------------------------------------------------------------------------
# GEMV (M <= 16)
# ---------------------------------------------------------------------------

GEMV_SHAPES = [
    # (M, K, N): single group, ragged tiles, odd group counts, several tiles
    (1, 128, 1), (1, 128, 17), (1, 384, 33), (1, 1024, 1024), (2, 640, 100),
    (3, 1280, 257), (4, 2048, 31), (5, 896, 48), (8, 768, 64), (9, 384, 40),
    (16, 512, 48), (16, 2304, 300), (1, 4224, 70), (7, 6144, 129),
    # 32 or more 256-K blocks (eight K-waves), one with a one-group last block
    (1, 8192, 70), (3, 8320, 33),
]


@pytest.mark.parametrize("M,K,N", GEMV_SHAPES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_matches_oracle(tern, oracle_lib, M, K, N, xdt):
    seed = 17 * M + K + 3 * N
    print(f"gemv M={M} K={K} N={N} x={xdt} seed={seed}", flush=True)
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    x = _x(seed, M, K, xdt)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y, y_ref, bound, what=f"gemv M{M} K{K} N{N} {xdt}")


@pytest.mark.parametrize("M,K,N", [(5, 128, 3), (8, 384, 50), (9, 4224, 33), (12, 1152, 257),
                                   (16, 640, 31), (16, 8448, 100)])
def test_gemv_direct_activation_loads(tern, oracle_lib, M, K, N):
    """bfloat16 activations with five or more rows take the direct-A GEMV:
    one-group tails, odd block counts, ragged tiles."""
    seed = 77 * M + K + N
    print(f"gemv direct-A M={M} K={K} N={N} seed={seed}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y, y_ref, bound, what=f"gemv direct-A M{M} K{K} N{N}")


def test_gemv_long_k_beyond_lds(tern, oracle_lib):
    """K so long that the staged activations would not fit in LDS: the
    bfloat16 GEMV falls back to direct A loads, even for M = 1."""
    M, K, N = 2, 98304, 24
    print(f"gemv long K M={M} K={K} N={N}", flush=True)
    t = synth.ternary(98304, N, K)
    s = synth.scales_f16(98304, N, K)
    x = synth.activations_bf16(98304, M, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y, y_ref, bound, what="gemv long K")


@pytest.mark.parametrize("M,K,N,xdt", [(1, 1024, 200, "bf16"), (4, 768, 50, "f32"), (16, 256, 20, "bf16")])
def test_gemv_bf16_output(tern, oracle_lib, M, K, N, xdt):
    seed = 900 + M
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    x = _x(seed, M, K, xdt)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d, ydt="bf16")
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y, y_ref, bound, bf16_out=True, what="gemv bf16 out")


def test_gemv_zero_weights_exact(tern):
    K, N = 512, 40
    t = np.zeros((N, K), dtype=np.int8)
    s = synth.scales_f16(1, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    for xdt in ("f32", "bf16"):
        y = _run_gemv(tern, _x(1, 3, K, xdt), codes_d, scales_d)
        assert (y == 0).all()


def test_gemv_identity_exact(tern):
    K = 1024
    t = np.eye(K, dtype=np.int8)
    s = np.full((K, K // 128), 0x3C00, dtype=np.uint16)
    codes_d, scales_d = pack_to_device(tern, t, s)
    x = synth.activations_bf16(5, 4, K)
    y = _run_gemv(tern, x, codes_d, scales_d)
    assert np.array_equal(y, (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    xf = synth.activations_f32(5, 2, K)
    y = _run_gemv(tern, xf, codes_d, scales_d)
    # binary32 input is carried as two bfloat16 parts: exact to 2^-16 relative
    assert np.allclose(y, xf.astype(np.float64), rtol=2.0 ** -15, atol=0)


def test_gemv_one_hot_exact(tern):
    K, N = 768, 64
    s = synth.scales_f16(6, N, K)
    x = synth.activations_bf16(6, 2, K)
    rng = np.random.default_rng(6)
    t = np.zeros((N, K), dtype=np.int8)
    ks = rng.integers(0, K, size=N)
    sg = rng.choice([-1, 1], size=N)
    t[np.arange(N), ks] = sg
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sv = s.view(np.float16).astype(np.float64)
    expect = sg[None, :] * sv[np.arange(N), ks // 128][None, :] * xv[:, ks]
    # s * x is exact in binary32 (11 x 8 significand bits)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("M,xdt", [(1, "bf16"), (3, "f32"), (16, "bf16")])
def test_gemv_integer_inputs_bit_exact(tern, oracle_lib, M, xdt):
    # integer x in [-64, 64], scales in {0.5, 1, 2}: every partial sum is a
    # multiple of 0.5 below 2^22, so any summation order is exact
    K, N = 4096, 96
    rng = np.random.default_rng(M)
    t = synth.ternary(40 + M, N, K)
    s = rng.choice(np.array([0.5, 1.0, 2.0], dtype=np.float16), size=(N, K // 128)).view(np.uint16)
    xi = rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    x = xi if xdt == "f32" else ((xi.view(np.uint32) >> 16).astype(np.uint16))
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert np.array_equal(y, y_ref)


def test_gemv_deterministic(tern):
    T = torch()
    K, N = 17408, 640
    t = synth.ternary(8, N, K)
    s = synth.scales_f16(8, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    for M, xdt in [(1, "bf16"), (2, "f32"), (16, "bf16")]:
        xd = x_to_device(_x(8, M, K, xdt))
        y1 = tern.tern_gemv(xd, codes_d, scales_d)
        y2 = tern.tern_gemv(xd, codes_d, scales_d)
        T.cuda.synchronize()
        assert T.equal(y1, y2)


def test_gemv_k_zero_gives_zeros(tern):
    T = torch()
    x = T.empty((2, 0), dtype=T.bfloat16, device="cuda")
    codes = T.empty((5, 0), dtype=T.int32, device="cuda")
    scales = T.empty((5, 0), dtype=T.int16, device="cuda")
    y = T.full((2, 5), 7.0, device="cuda")
    tern.tern_gemv(x, codes, scales, out=y)
    T.cuda.synchronize()
    assert (y.cpu() == 0).all()


@pytest.mark.parametrize("M,K,N", [
    (5, 384, 16400),     # odd G: a one-group last block; one K-group; ragged last tile
    (8, 1280, 16384),    # five blocks over two K-groups (one has an extra step)
    (12, 2304, 16416),   # nine blocks: the unrolled loop's tail steps
    (16, 5120, 16400),   # the sweep's row count, 16 rows
    (9, 8448, 16384),    # 33 blocks: a full quad loop plus an extra step
])
def test_gemv_shared_activation_ring(tern, oracle_lib, M, K, N):
    """bfloat16 activations with 5..16 rows on wide matrices take the kernel
    whose tile-waves share an LDS ring of activation blocks; every output
    element against the oracle."""
    seed = 13 * M + K + N
    print(f"gemv ring M={M} K={K} N={N} seed={seed}", flush=True)
    codes_d, scales_d, t, s = full_problem(tern, seed, N, K, 1 / 3)
    x = synth.activations_bf16(seed, M, K)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y, y_ref, bound, what=f"gemv ring M{M} K{K} N{N}")


EVEN_SPLIT = [
    # (M, K, N)
    (1, 896, 3),       # four blocks (the fewest this kernel takes), one quad, one workgroup
    (1, 896, 1027),    # a ragged last quad
    (1, 3968, 7777),   # 31 groups: a one-group last block, unpaired scale loads, ragged quads
    (1, 2048, 1030),   # fewer quads than CUs
    (1, 5120, 5123),   # the 5120-row projection plus a ragged quad
    (1, 12288, 999),   # long rows, few quads: many steps per quad
    (2, 896, 1027), (3, 3968, 777), (4, 2048, 4099), (2, 8192, 1999), (4, 12288, 517), (3, 1024, 5),
]


@pytest.mark.parametrize("M,K,N", EVEN_SPLIT)
def test_gemv_even_split(tern, oracle_lib, M, K, N):
    """One to four rows of bfloat16 x, with a multiple of four 256-K blocks
    per row, take the kernel that splits (quad, block) pairs evenly over the
    CUs, four blocks per MFMA; every element against the oracle, fp32 and
    bf16 outputs, and a repeat is bit-identical."""
    seed = 31 * K + N + M
    print(f"gemv even split M={M} K={K} N={N} seed={seed}", flush=True)
    codes_d, scales_d, t, s = full_problem(tern, seed, N, K, 1 / 3)
    x = synth.activations_bf16(seed, M, K)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y, y_ref, bound, what=f"even split M{M} K{K} N{N}")
    assert np.array_equal(y, _run_gemv(tern, x, codes_d, scales_d)), "repeat differs"
    yb = _run_gemv(tern, x, codes_d, scales_d, ydt="bf16")
    assert_matmul_close(yb, y_ref, bound, bf16_out=True, what=f"even split bf16 M{M} K{K} N{N}")


# Full sizes of the decode workloads, in the launch configuration the
# benchmark uses: every output element against the (threaded) oracle.
FULL = [(1, 1024, 1024, "f32", 1 / 3), (1, 4096, 12288, "f32", 0.35)] + \
       [(m, k, n, "bf16", 1 / 3) for m in (1, 2, 4, 8, 16) for (k, n) in ((5120, 17408), (17408, 5120))] + \
       [(1, 5120, 12288, "bf16", 1 / 3), (1, 6144, 5120, "bf16", 1 / 3)]


@pytest.mark.parametrize("M,K,N,xdt,p0", FULL)
def test_gemv_full_size_every_element(tern, oracle_lib, M, K, N, xdt, p0):
    seed = 1000 + K + N + M
    print(f"full gemv M={M} K={K} N={N} seed={seed}", flush=True)
    codes_d, scales_d, t, s = full_problem(tern, seed, N, K, p0)
    x = _x(seed, M, K, xdt)
    y = _run_gemv(tern, x, codes_d, scales_d)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y, y_ref, bound, what=f"full M{M} K{K} N{N}")


def test_gemv_lm_head_size_sampled(tern, oracle_lib):
    # the largest single projection of the decode step: 5120 -> 248320
    K, N, seed = 5120, 248320, 77
    print("lm-head gemv", flush=True)
    rows = sampled_rows(N, 96, seed)
    codes_d, scales_d, t_rows, s_rows = big_problem(tern, seed, N, K, 1 / 3, rows)
    x = synth.activations_bf16(seed, 1, K)
    y = _run_gemv(tern, x, codes_d, scales_d, ydt="bf16")
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t_rows), s_rows, K)
    assert_matmul_close(y[:, rows], y_ref, bound, bf16_out=True, what="lm head")


# ---------------------------------------------------------------------------
# FWHT
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,block", [(1, 4096, 4096), (3, 8192, 4096), (2, 4096, 1024), (1, 512, 64),
                                       (5, 96, 32), (2, 64, 2), (1, 16, 1), (2, 3 * 256, 256)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("signed", [True, False])
def test_fwht_matches_oracle(tern, oracle_lib, M, K, block, xdt, signed):
    seed = M * 31 + K + block
    x = _x(seed, M, K, xdt)
    d = synth.signs(seed, K) if signed else None
    xd = x_to_device(x)
    dd = torch().from_numpy(d).cuda() if signed else None
    x64 = x.astype(np.float64) if xdt == "f32" else oracle_lib.bf16_bits_to_f64(x)
    y = tern.tern_fwht(xd, dd, block)
    yi = tern.tern_fwht(y, dd, block, inverse=True)
    torch().cuda.synchronize()
    assert_fwht_close(y_to_host(y), oracle_lib.fwht(x64, d, block), what="forward")
    assert_fwht_close(y_to_host(yi), oracle_lib.fwht(y_to_host(y), d, block, inverse=True), what="inverse")
    # forward then inverse returns x
    assert_fwht_close(y_to_host(yi), x64, what="round trip")


@pytest.mark.parametrize("K,block", [(4096, 4096), (64, 64), (32, 4)])
def test_fwht_rows_past_the_grid_limit(tern, oracle_lib, K, block):
    """More rows than one grid dimension holds (65,535): the workgroups loop
    over rows.  Rows on both sides of the limit, and the rows that share a
    workgroup with them, are checked against the oracle (rows are
    independent)."""
    M, seed = 65535 + 7, 71 + K
    print(f"fwht rows M={M} K={K} block={block}", flush=True)
    x = synth.activations_bf16(seed, M, K)
    d = synth.signs(seed, K)
    y = tern.tern_fwht(x_to_device(x), torch().from_numpy(d).cuda(), block)
    torch().cuda.synchronize()
    rows = np.array([0, 1, 6, 7, 65533, 65534, 65535, 65536, M - 1])
    yh = y[torch().from_numpy(rows).cuda()].cpu().numpy()
    assert_fwht_close(yh, oracle_lib.fwht(oracle_lib.bf16_bits_to_f64(x[rows]), d, block), what=f"rows K{K}")


def test_fwht_in_place(tern, oracle_lib):
    T = torch()
    x = synth.activations_f32(3, 2, 8192)
    d = synth.signs(3, 8192)
    xd = x_to_device(x)
    tern.tern_fwht(xd, T.from_numpy(d).cuda(), 4096, out=xd)
    T.cuda.synchronize()
    assert_fwht_close(y_to_host(xd), oracle_lib.fwht(x.astype(np.float64), d, 4096), what="in place")


def test_fwht_closed_forms(tern):
    T = torch()
    e0 = T.zeros((1, 4096), device="cuda")
    e0[0, 0] = 1.0
    y = tern.tern_fwht(e0, None, 4096)
    T.cuda.synchronize()
    assert (y.cpu() == 1.0 / 64).all()     # normalization 2^-6 is exact
    ones = T.ones((1, 4096), device="cuda")
    y = tern.tern_fwht(ones, None, 4096).cpu()
    assert y[0, 0] == 64.0 and (y[0, 1:] == 0).all()


# ---------------------------------------------------------------------------
# Rotated decode: sign flip + FWHT (block 4096) + GEMV at the full size
# ---------------------------------------------------------------------------

def test_rotated_decode_full_size(tern, oracle_lib):
    """Two-launch rotated decode at its full size, every output element."""
    w = synth.ROTATED
    seed = 2024
    print("rotated decode", flush=True)
    codes_d, scales_d, t, s = full_problem(tern, seed, w.N, w.K, w.p_zero)
    x = synth.activations_bf16(seed, w.M, w.K)
    d = synth.signs(seed, w.K)
    T = torch()
    xr = tern.tern_fwht(x_to_device(x), T.from_numpy(d).cuda(), w.rotate_block)
    y = tern.tern_gemv(xr, codes_d, scales_d)
    T.cuda.synchronize()
    xr_h = y_to_host(xr)
    xr_ref = oracle_lib.fwht(oracle_lib.bf16_bits_to_f64(x), d, w.rotate_block)
    assert_fwht_close(xr_h, xr_ref, what="rotation")
    # the GEMV on the rotation it was given ...
    codes_o = oracle_lib.encode(t)
    nt = oracle_threads(oracle_lib)
    y_ref, bound = oracle_lib.matmul(xr_h.astype(np.float32), codes_o, s, w.K, threads=nt)
    assert_matmul_close(y_to_host(y), y_ref, bound, what="gemv on rotated x")
    # ... and end to end against the FP64 rotation (its own error adds
    # sum |s t| * |dx| per output)
    y64, b64 = oracle_lib.matmul(xr_ref, codes_o, s, w.K, threads=nt)
    dx = np.abs(xr_h - xr_ref)
    wabs = np.abs(oracle_lib.dequant(codes_o, s, w.K))
    # allowance 1e-4 * B + sum |s t| |dx|, expressed through the bound
    assert_matmul_close(y_to_host(y), y64, b64 + 1e4 * (dx @ wabs.T), what="rotated decode end to end")


# ---------------------------------------------------------------------------
# Fused rotation + GEMV (one launch)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,block,xdt,signed", [
    (1, 4096, 300, 4096, "bf16", True), (1, 4096, 777, 4096, "f32", True), (2, 8192, 100, 4096, "bf16", True),
    (1, 1024, 64, 256, "bf16", False), (3, 2048, 50, 64, "f32", True), (4, 512, 33, 16, "bf16", True),
    (1, 384, 40, 128, "f32", False), (8, 1024, 20, 1024, "bf16", True), (16, 256, 70, 32, "bf16", True),
    # 4096-point blocks (matrix-core transform): no signs, several units per
    # wave, staged rows beyond 2M (M = 3 stages 8 rows)
    (1, 4096, 200, 4096, "bf16", False), (3, 4096, 40, 4096, "f32", False), (4, 4096, 50, 4096, "bf16", True),
])
def test_rotate_gemv_matches_oracle(tern, oracle_lib, M, K, N, block, xdt, signed):
    seed = 3 * M + K + N + block
    print(f"rotate gemv M={M} K={K} N={N} b={block} {xdt}", flush=True)
    T = torch()
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = _x(seed, M, K, xdt)
    d = synth.signs(seed, K) if signed else None
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = tern.tern_rotate_gemv(x_to_device(x), T.from_numpy(d).cuda() if signed else None, block,
                              codes_d, scales_d)
    T.cuda.synchronize()
    x64 = x.astype(np.float64) if xdt == "f32" else oracle_lib.bf16_bits_to_f64(x)
    xr = oracle_lib.fwht(x64, d, block)
    codes_o = oracle_lib.encode(t)
    y_ref, bound = oracle_lib.matmul(xr, codes_o, s, K)
    # binary32 rotation error (rel L2 <= 1e-5 per row) propagates through
    # sum |s t| |dx|; allow it on top of the matmul bound
    wabs = np.abs(oracle_lib.dequant(codes_o, s, K))
    rot_err = 1e-5 * np.linalg.norm(xr, axis=1, keepdims=True) * np.sqrt((wabs ** 2).sum(axis=1))[None, :]
    assert_matmul_close(y_to_host(y), y_ref, bound + 1e4 * rot_err, what="rotate gemv")


def test_rotate_gemv_full_size_matches_two_launch_path(tern, oracle_lib):
    """Fused rotated decode (one launch) at its full size, every output
    element, beside the two-launch path."""
    w = synth.ROTATED
    seed = 606
    print("rotated decode fused", flush=True)
    codes_d, scales_d, t, s = full_problem(tern, seed, w.N, w.K, w.p_zero)
    T = torch()
    x = synth.activations_bf16(seed, 1, w.K)
    d = synth.signs(seed, w.K)
    xd, dd = x_to_device(x), T.from_numpy(d).cuda()
    y1 = tern.tern_rotate_gemv(xd, dd, w.rotate_block, codes_d, scales_d)
    y1b = tern.tern_rotate_gemv(xd, dd, w.rotate_block, codes_d, scales_d)
    y2 = tern.tern_gemv(tern.tern_fwht(xd, dd, w.rotate_block), codes_d, scales_d)
    T.cuda.synchronize()
    assert T.equal(y1, y1b)                      # deterministic
    xr = oracle_lib.fwht(oracle_lib.bf16_bits_to_f64(x), d, w.rotate_block)
    codes_o = oracle_lib.encode(t)
    y_ref, bound = oracle_lib.matmul(xr, codes_o, s, w.K, threads=oracle_threads(oracle_lib))
    wabs = np.abs(oracle_lib.dequant(codes_o, s, w.K))
    rot_err = 1e-5 * np.linalg.norm(xr) * np.sqrt((wabs ** 2).sum(axis=1))[None, :]
    for y in (y1, y2):
        assert_matmul_close(y_to_host(y), y_ref, bound + 1e4 * rot_err, what="fused vs oracle")


# ---------------------------------------------------------------------------
# GEMM (any M)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(1, 256, 64), (17, 640, 100), (64, 1024, 128), (100, 384, 257),
                                   (130, 2048, 96), (256, 1280, 320)])
def test_gemm_matches_oracle(tern, oracle_lib, M, K, N):
    seed = 5 * M + K + N
    print(f"gemm M={M} K={K} N={N}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = tern.tern_gemm(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y_to_host(y), y_ref, bound, what=f"gemm M{M} K{K} N{N}")


@pytest.mark.parametrize("K,N", [(5120, 17408), (17408, 5120)])
def test_gemm_prefill_full_size_sampled(tern, oracle_lib, K, N):
    M, seed = 512, 4000 + K
    print(f"prefill gemm K={K} N={N}", flush=True)
    rows = sampled_rows(N, 48, seed)
    codes_d, scales_d, t_rows, s_rows = big_problem(tern, seed, N, K, 0.35, rows)
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    y = tern.tern_gemm(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t_rows), s_rows, K)
    assert_matmul_close(y_to_host(y)[:, rows], y_ref, bound, what=f"prefill K{K} N{N}")


def _gemm_sampled(tern, oracle_lib, M, K, N, seed, t, s, x, cols, what):
    """Run tern_gemm on the full problem; compare sampled output columns."""
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = tern.tern_gemm(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t[cols]), s[cols], K)
    assert_matmul_close(y_to_host(y)[:, cols], y_ref, bound, what=what)
    return y


@pytest.mark.parametrize("M,K,N", [
    (600, 4096, 700),    # ragged row and column tiles; every tile split in pieces
    (1024, 512, 1024),   # fewer tiles than workgroups, too short to split: no workspace
    (4000, 384, 3900),   # two rounds of whole tiles for some workgroups, K shorter than a piece
    (2300, 1024, 3700),  # one round of whole tiles, then the leftover tiles in K pieces (ragged)
    (300, 17408, 96),    # long K split over many workgroups
])
def test_gemm_work_split_cases(tern, oracle_lib, M, K, N):
    seed = 7 * M + 3 * K + N
    print(f"gemm split case M={M} K={K} N={N} ws={tern.tern_gemm_workspace_bytes(M, N, K)}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    cols = sampled_rows(N, 40, seed)
    _gemm_sampled(tern, oracle_lib, M, K, N, seed, t, s, x, cols, f"gemm M{M} K{K} N{N}")


def test_gemm_zero_scale_groups(tern, oracle_lib):
    """Zero scales: whole columns, the first and last group of a column, and
    random groups (the scale-rescaling path must skip them)."""
    M, K, N, seed = 300, 2048, 160, 77
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    rng = np.random.default_rng(seed)
    s[rng.random(s.shape) < 0.2] = 0
    s[3, :] = 0
    s[5, 0] = 0
    s[6, -1] = 0
    s[7, :-1] = 0
    s[8, 1:] = 0
    s[9, ::2] = 0x8000  # -0.0
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    cols = np.arange(N)
    _gemm_sampled(tern, oracle_lib, M, K, N, seed, t, s, x, cols, "gemm zero scales")


def test_gemm_wide_scale_range(tern, oracle_lib):
    """Group scales spread over 2^-24 .. 2^15 (fp16 subnormals to near max),
    negative ones too: the per-group rescaling keeps the error bound."""
    M, K, N, seed = 260, 8192, 130, 78
    t = synth.ternary(seed, N, K, 0.35)
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-24, 15, size=(N, K // 128)))
    sgn = np.where(rng.random((N, K // 128)) < 0.2, -1.0, 1.0)
    s = (sgn * mag).astype(np.float16).view(np.uint16)
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    cols = np.arange(N)
    _gemm_sampled(tern, oracle_lib, M, K, N, seed, t, s, x, cols, "gemm wide scales")


def test_gemm_integer_exact_and_deterministic(tern, oracle_lib):
    """Small-integer activations with unit scales: every partial sum is an
    integer below 2^24, so the result is exact; and repeated calls agree
    bit for bit."""
    T = torch()
    M, K, N, seed = 520, 3072, 300, 79
    t = synth.ternary(seed, N, K, 0.35)
    s = np.full((N, K // 128), 0x3C00, dtype=np.uint16)  # 1.0
    rng = np.random.default_rng(seed)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(x)
    y1 = tern.tern_gemm(xd, codes_d, scales_d)
    y2 = tern.tern_gemm(xd, codes_d, scales_d)
    T.cuda.synchronize()
    exact = xi.astype(np.float64) @ t.astype(np.float64).T
    assert np.array_equal(y_to_host(y1), exact)
    assert T.equal(y1, y2)


def test_gemm_k_zero_and_empty(tern):
    T = torch()
    x = T.zeros((300, 0), dtype=T.bfloat16, device="cuda")
    codes = T.zeros((70, 0), dtype=T.int32, device="cuda")
    scales = T.zeros((70, 0), dtype=T.int16, device="cuda")
    y = T.full((300, 70), 7.0, device="cuda")
    tern.tern_gemm(x, codes, scales, out=y)
    T.cuda.synchronize()
    assert (y == 0).all()
    y0 = T.full((0, 70), 7.0, device="cuda")
    tern.tern_gemm(T.zeros((0, 128), dtype=T.bfloat16, device="cuda"),
                   T.zeros((70, 8), dtype=T.int32, device="cuda"),
                   T.zeros((70, 1), dtype=T.int16, device="cuda"), out=y0)
    T.cuda.synchronize()


def test_gemm_at_the_k_limit(tern, oracle_lib):
    """K = 2^22 - 128, the largest K tern_gemm takes (32-bit buffer offsets
    over a 128-row tile of x): one ragged tile split along K over many
    workgroups, every element against the oracle."""
    M, K, N, seed = 3, (1 << 22) - 128, 40, 97
    print(f"gemm K limit M={M} K={K} N={N} ws={tern.tern_gemm_workspace_bytes(M, N, K)}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = tern.tern_gemm(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y_to_host(y), y_ref, bound, what=f"gemm K{K}")


@pytest.mark.parametrize("N,K", [(1, 128), (7, 256), (33, 1280), (1000, 5120)])
def test_pack_device_matches_oracle_encode(tern, oracle_lib, N, K):
    """Device packer: bit-exact against the oracle's encoder."""
    T = torch()
    t = synth.ternary(60 + N + K, N, K)
    codes = tern.tern_pack_device(T.from_numpy(t).cuda())
    T.cuda.synchronize()
    ref = oracle_lib.encode(t)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), ref)


def test_chained_block_links(tern, oracle_lib):
    """One block of the 27B-class decode pass at full size, chained the way
    the benchmark chains it (bf16 outputs feed the next link where lengths
    match); every link is checked on sampled rows against the oracle on the
    bf16 input it actually received."""
    T = torch()
    links = synth.CHAIN_BLOCK
    w = []
    for li, (K, N) in enumerate(links):
        seed = 900 + li
        rows = sampled_rows(N, 12, seed)
        codes_d, scales_d, t_rows, s_rows = big_problem(tern, seed, N, K, 1.0 / 3.0, rows)
        w.append((codes_d, scales_d, t_rows, s_rows, rows, K, N))
    x5120 = x_to_device(synth.activations_bf16(950, 1, 5120))
    x6144 = x_to_device(synth.activations_bf16(951, 1, 6144))

    def run(li, xin):
        codes_d, scales_d, t_rows, s_rows, rows, K, N = w[li]
        y = tern.tern_gemv(xin, codes_d, scales_d, out_dtype=T.bfloat16)
        T.cuda.synchronize()
        xh = xin.view(T.int16).cpu().numpy().view(np.uint16)
        y_ref, bound = oracle_lib.matmul(xh, oracle_lib.encode(t_rows), s_rows, K)
        assert_matmul_close(y_to_host(y)[:, rows], y_ref, bound, bf16_out=True,
                            what=f"chain link {li} ({K}->{N})")
        return y

    run(0, x5120)              # 5120 -> 12288
    h = run(1, x6144)          # 6144 -> 5120
    gu = run(2, h)             # 5120 -> 17408 (gate) + 17408 (up), one matrix
    up = gu[:, synth.CHAIN_GATE_UP:]
    assert up.is_contiguous()
    out = run(3, up)           # 17408 -> 5120 (down): the next block's input
    assert out.shape == (1, 5120) and T.isfinite(out.float()).all()


# ---------------------------------------------------------------------------
# HIP graph capture of the decode step: every replay equals eager execution
# ---------------------------------------------------------------------------

def test_rotated_step_graph_replays_match_eager(tern):
    T = torch()
    K, N, seed = 4096, 1000, 31
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(synth.activations_bf16(seed, 1, K))
    dd = T.from_numpy(synth.signs(seed, K)).cuda()
    xr = T.empty((1, K), dtype=T.float32, device="cuda")
    y = T.empty((1, N), dtype=T.float32, device="cuda")

    def step():
        tern.tern_fwht(xd, dd, 4096, out=xr)
        tern.tern_gemv(xr, codes_d, scales_d, out=y)

    step()
    T.cuda.synchronize()
    y_eager = y.clone()
    g = T.cuda.CUDAGraph()
    st = T.cuda.Stream()
    st.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(st):
        with T.cuda.graph(g, stream=st):
            step()
    T.cuda.current_stream().wait_stream(st)
    for r in range(4):
        y.zero_()
        xr.zero_()
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, y_eager), f"replay {r}"
        step()                      # eager work between replays
        T.cuda.synchronize()


def test_even_split_graph_replays_match_eager(tern):
    """Two chained even-split GEMV links (bf16 output feeding the next link)
    and a binary GEMV captured in one HIP graph: every replay, with eager
    work in between, equals the eager calls."""
    T = torch()
    seed, M = 43, 2
    (K1, N1), (K2, N2) = (2048, 3072), (3072, 1000)   # uneven tile splits: the even-split kernel
    c1, s1 = pack_to_device(tern, synth.ternary(seed, N1, K1), synth.scales_f16(seed, N1, K1))
    c2, s2 = pack_to_device(tern, synth.ternary(seed + 1, N2, K2), synth.scales_f16(seed + 1, N2, K2))
    bits = T.from_numpy(tern.tern_pack_b1(synth.ternary(seed + 2, N2, K2, 0.0)).view(np.int32)).cuda()
    xd = x_to_device(synth.activations_bf16(seed, M, K1))
    h = T.empty((M, N1), dtype=T.bfloat16, device="cuda")
    y = T.empty((M, N2), dtype=T.float32, device="cuda")
    yb = T.empty((M, N2), dtype=T.float32, device="cuda")

    def step():
        tern.tern_gemv(xd, c1, s1, out=h)
        tern.tern_gemv(h, c2, s2, out=y)
        tern.tern_gemv_b1(h, bits, s2, out=yb)

    step()
    T.cuda.synchronize()
    y_eager, yb_eager = y.clone(), yb.clone()
    g = T.cuda.CUDAGraph()
    st = T.cuda.Stream()
    st.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(st):
        with T.cuda.graph(g, stream=st):
            step()
    T.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        y.fill_(float("nan"))
        yb.fill_(float("nan"))
        h.zero_()
        other = T.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, y_eager) and T.equal(yb, yb_eager), f"replay {rep} differs"
        assert T.isfinite(other)


def test_gemm_graph_replays_match_eager(tern):
    """tern_gemm with split tiles (workspace + fixup pass) captured in a HIP
    graph: every replay, with eager work in between, equals the eager call."""
    T = torch()
    M, K, N, seed = 600, 4096, 700, 41
    assert tern.tern_gemm_workspace_bytes(M, N, K) > 0  # the split path
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(synth.activations_bf16(seed, M, K, outlier_frac=0.01))
    y = T.empty((M, N), dtype=T.float32, device="cuda")
    ws = T.empty(tern.tern_gemm_workspace_bytes(M, N, K), dtype=T.uint8, device="cuda")
    tern.tern_gemm(xd, codes_d, scales_d, out=y, workspace=ws)
    T.cuda.synchronize()
    y_eager = y.clone()
    g = T.cuda.CUDAGraph()
    st = T.cuda.Stream()
    st.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(st):
        with T.cuda.graph(g, stream=st):
            tern.tern_gemm(xd, codes_d, scales_d, out=y, workspace=ws)
    T.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xFF)                      # stale workspace contents must not matter
        other = T.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, y_eager), f"replay {rep} differs"
        assert T.isfinite(other)


@pytest.mark.parametrize("b", [64, 4096])
def test_rotation_fold_into_weight_rows(tern, b):
    """Folding the rotation into the weights: with W' = rows of W transformed
    forward and x' = the forward transform of x, W' x' = W x (H is symmetric,
    H H = b I, D D = I).  Dense fp32 weights, checked against fp64."""
    T = torch()
    rng = np.random.default_rng(b)
    N, K = 96, 2 * b
    W = rng.standard_normal((N, K)).astype(np.float32)
    x = rng.standard_normal((3, K)).astype(np.float32)
    d = synth.signs(b, K)
    dd = T.from_numpy(d).cuda()
    Wf = tern.tern_fwht(T.from_numpy(W).cuda(), dd, b)
    xf = tern.tern_fwht(T.from_numpy(x).cuda(), dd, b)
    T.cuda.synchronize()
    y_fold = xf.double().cpu().numpy() @ Wf.double().cpu().numpy().T
    y_ref = x.astype(np.float64) @ W.astype(np.float64).T
    scale = np.abs(x).astype(np.float64) @ np.abs(W).astype(np.float64).T
    assert np.all(np.abs(y_fold - y_ref) <= 1e-5 * scale)


# ---------------------------------------------------------------------------
# format variants: converted on the host, run through the g128 kernels, and
# checked against the oracle's dense weights of the variant itself
# ---------------------------------------------------------------------------

def _variant_problem(tern, oracle_lib, fmt, N, K, seed):
    """Returns (codes, g128 scales) for the kernels and the oracle's dense
    float64 weights of the variant as given."""
    s = synth.scales_f16(seed, N, K)
    if fmt == "b1":
        b = np.where(np.random.default_rng(seed).random((N, K)) < 0.5, 1, -1).astype(np.int8)
        bits = tern.tern_pack_b1(b)
        dense = oracle_lib.b1_decode(bits, K) * np.repeat(oracle_lib.half_bits_to_f64(s), 128, axis=1)
        return tern.tern_b1_to_codes(bits, K), s, dense
    t = synth.ternary(seed, N, K, 0.35)
    codes, _ = tern.tern_pack(t, s)
    if fmt == "g64":
        s64 = np.repeat(s, 2, axis=1)
        return codes, tern.tern_scales_from_g64(s64), oracle_lib.dequant_g64(codes, s64, K)
    sc, bi = np.ascontiguousarray(s), s | np.uint16(0x8000)      # (s, -s)
    return codes, tern.tern_mlx_import(sc, bi), oracle_lib.dequant_affine(codes, 2, 128, sc, bi, K)


@pytest.mark.parametrize("fmt", ["b1", "g64", "mlx"])
@pytest.mark.parametrize("M,K,N,op", [(1, 1024, 300, "gemv"), (5, 2304, 129, "gemv"), (96, 1280, 200, "gemm")])
def test_format_variant_through_kernels(tern, oracle_lib, fmt, M, K, N, op):
    seed = 800 + M + K + N
    print(f"variant {fmt} {op} M={M} K={K} N={N} seed={seed}", flush=True)
    codes, s, dense = _variant_problem(tern, oracle_lib, fmt, N, K, seed)
    x = synth.activations_bf16(seed, M, K)
    codes_d, scales_d = tern.to_device(codes, s)
    fn = tern.tern_gemv if op == "gemv" else tern.tern_gemm
    y = fn(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    xd = oracle_lib.bf16_bits_to_f64(x)
    y_ref = xd @ dense.T
    bound = np.abs(xd) @ np.abs(dense).T
    assert_matmul_close(y_to_host(y), y_ref, bound, what=f"{fmt} {op} M{M} K{K} N{N}")


# ---------------------------------------------------------------------------
# decode GEMV over the binary variant (one sign bit per weight)
# ---------------------------------------------------------------------------

B1_SHAPES = [
    # (M, K, N): four blocks (the fewest), ragged quads, fewer quads than CUs,
    # rows of 32 and more blocks, the decode shapes
    (1, 1024, 5), (1, 1024, 1027), (2, 2048, 4099), (3, 4096, 777), (4, 8192, 517),
    (1, 5120, 17408), (1, 17408, 5120), (4, 5120, 12288), (2, 17408, 333),
]


@pytest.mark.parametrize("M,K,N", B1_SHAPES)
def test_gemv_b1_matches_oracle(tern, oracle_lib, M, K, N):
    """tern_gemv_b1 streams the 1-bit words of tern_pack_b1 as they are; every
    element against the oracle's product of the same +-1 weights (as ternary
    values) and scales; bf16 output; a repeat is bit-identical."""
    seed = 57 * M + K + 3 * N
    print(f"gemv_b1 M={M} K={K} N={N} seed={seed}", flush=True)
    T = torch()
    b = synth.ternary(seed, N, K, 0.0)  # +-1 only
    s = synth.scales_f16(seed, N, K)
    bits = tern.tern_pack_b1(b)
    bits_d = T.from_numpy(bits.view(np.int32)).cuda()
    scales_d = T.from_numpy(s.view(np.int16)).cuda()
    x = synth.activations_bf16(seed, M, K)
    xd = x_to_device(x)
    y = tern.tern_gemv_b1(xd, bits_d, scales_d)
    T.cuda.synchronize()
    y = y_to_host(y)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(b), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y, y_ref, bound, what=f"gemv_b1 M{M} K{K} N{N}")
    y2 = tern.tern_gemv_b1(xd, bits_d, scales_d)
    T.cuda.synchronize()
    assert np.array_equal(y, y_to_host(y2)), "repeat differs"
    yb = tern.tern_gemv_b1(xd, bits_d, scales_d, out_dtype=T.bfloat16)
    T.cuda.synchronize()
    assert_matmul_close(y_to_host(yb), y_ref, bound, bf16_out=True, what=f"gemv_b1 bf16 M{M} K{K} N{N}")


def test_gemv_b1_same_as_ternary_codes(tern):
    """The binary words and their 2-bit expansion (tern_b1_to_codes) through
    tern_gemv give bit-identical results for integer-valued inputs, where
    every sum is exact."""
    T = torch()
    M, K, N, seed = 2, 3072, 700, 91
    b = synth.ternary(seed, N, K, 0.0)
    s = np.full((N, K // 128), 0x3C00, dtype=np.uint16)  # 1.0
    x32 = np.random.default_rng(seed).integers(-8, 9, size=(M, K)).astype(np.float32)
    x = (x32.view(np.uint32) >> 16).astype(np.uint16)    # exact in bfloat16
    bits = tern.tern_pack_b1(b)
    xd = x_to_device(x)
    y1 = tern.tern_gemv_b1(xd, T.from_numpy(bits.view(np.int32)).cuda(), T.from_numpy(s.view(np.int16)).cuda())
    codes_d, scales_d = tern.to_device(tern.tern_b1_to_codes(bits, K), s)
    y2 = tern.tern_gemv(xd, codes_d, scales_d)
    T.cuda.synchronize()
    assert np.array_equal(y_to_host(y1), y_to_host(y2))
    assert np.array_equal(y_to_host(y1), (x32.astype(np.float64) @ b.T.astype(np.float64)).astype(np.float32))


# ---------------------------------------------------------------------------
# decode GEMV over the base-3 layout (five ternary values per byte)
# ---------------------------------------------------------------------------

T5_SHAPES = [
    # (M, K, N): one to five groups in the last superblock, ragged tiles, M up to 16
    (1, 128, 1), (1, 256, 17), (2, 384, 33), (1, 512, 64), (3, 640, 100), (1, 768, 31),
    (4, 1280, 257), (5, 4096, 48), (8, 5120, 40), (16, 2304, 300), (1, 6144, 129),
    (7, 17408, 20), (16, 17408, 35),
]


def _run_t5(tern, x, data, s, ydt="f32"):
    """data: the base-3 bytes as the oracle's encoder writes them."""
    T = torch()
    out_dtype = T.float32 if ydt == "f32" else T.bfloat16
    y = tern.tern_gemv_t5(x_to_device(x), T.from_numpy(data).cuda(),
                          T.from_numpy(s.view(np.int16)).cuda(), out_dtype=out_dtype)
    T.cuda.synchronize()
    return y_to_host(y)


@pytest.mark.parametrize("M,K,N", T5_SHAPES)
def test_gemv_t5_matches_oracle(tern, oracle_lib, M, K, N):
    seed = 31 * M + K + 7 * N
    print(f"gemv_t5 M={M} K={K} N={N} seed={seed}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K)
    y = _run_t5(tern, x, oracle_lib.t5_encode(t), s)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y, y_ref, bound, what=f"gemv_t5 M{M} K{K} N{N}")


@pytest.mark.parametrize("M,K,N", [
    (5, 2048, 16400),    # last superblock holds one group; two tile-waves; ragged last tile
    (16, 5120, 16400),   # two tile-waves, two K-groups
    (12, 4096, 16400),   # seven superblocks over two K-groups (one has an extra one)
    (16, 17408, 700),    # one tile-wave, four K-groups
    (3, 20480, 300),     # few rows whose LDS copy of x would not fit: the ring
])
def test_gemv_t5_shared_activation_ring(tern, oracle_lib, M, K, N):
    """Base-3 GEMV with 5..16 rows (or rows too long to copy into LDS) takes
    the kernel whose tile-waves share an LDS ring of half superblocks of x;
    every output element against the oracle."""
    seed = 19 * M + K + N
    print(f"gemv t5 ring M={M} K={K} N={N} seed={seed}", flush=True)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_bf16(seed, M, K)
    y = _run_t5(tern, x, oracle_lib.t5_encode(t), s)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=oracle_threads(oracle_lib))
    assert_matmul_close(y, y_ref, bound, what=f"t5 ring M{M} K{K} N{N}")


def test_gemv_t5_integer_exact_and_bf16_out(tern, oracle_lib):
    """Integer activations and scales in {0.5, 1, 2}: every partial sum is
    exact in binary32, so the result is bit-exact; bf16 output rounds once."""
    N, K, M = 70, 3200, 3
    rng = np.random.default_rng(4242)
    t = synth.ternary(4242, N, K)
    s = rng.choice(np.array([0x3800, 0x3C00, 0x4000], dtype=np.uint16), size=(N, K // 128))
    xi = rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    data = oracle_lib.t5_encode(t)
    y = _run_t5(tern, x, data, s)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert np.array_equal(y, y_ref)
    yb = _run_t5(tern, x, data, s, "bf16")
    assert_matmul_close(yb, y_ref, bound, bf16_out=True, what="gemv_t5 bf16 out")


def test_gemv_t5_every_byte_value(tern, oracle_lib):
    """Rows whose bytes run through all 243 values (every digit pattern at
    every group position), integer activations: bit-exact."""
    K = 640 * 2 + 256                                  # two full superblocks and a two-group tail
    G = K // 128
    N = 243
    v = np.arange(243, dtype=np.int64)
    t = np.zeros((N, K), dtype=np.int8)
    for g in range(G):
        j = g % 5
        # roll the row index per position so that every byte holds many values
        idx = (v[:, None] + np.arange(128)[None, :] * 7 + g) % 243
        t[:, 128 * g:128 * (g + 1)] = ((idx // 3 ** j) % 3 - 1).astype(np.int8)
    s = np.full((N, G), 0x3C00, dtype=np.uint16)
    rng = np.random.default_rng(243)
    xi = rng.integers(-64, 65, size=(2, K)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    data = oracle_lib.t5_encode(t)
    assert len(np.unique(data[:, :256])) == 243
    y = _run_t5(tern, x, data, s)
    y_ref, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert np.array_equal(y, y_ref)


def test_gemv_t5_zero_and_empty(tern, oracle_lib):
    T = torch()
    K, N = 1280, 40
    t = np.zeros((N, K), dtype=np.int8)
    s = synth.scales_f16(5, N, K)
    x = synth.activations_bf16(5, 2, K)
    assert np.all(_run_t5(tern, x, oracle_lib.t5_encode(t), s) == 0)
    xk0 = T.zeros((2, 0), dtype=T.bfloat16, device="cuda")
    y = tern.tern_gemv_t5(xk0, T.zeros((N, 0), dtype=T.uint8, device="cuda"),
                          T.zeros((N, 0), dtype=T.int16, device="cuda"))
    T.cuda.synchronize()
    assert y.shape == (2, N) and bool((y == 0).all())


@pytest.mark.parametrize("K,N", [(5120, 17408), (17408, 5120), (4096, 12288)])
def test_gemv_t5_full_size_sampled(tern, oracle_lib, K, N):
    """Full decode shapes in the launch configuration the benchmark times;
    sampled rows checked against the oracle."""
    T = torch()
    print(f"gemv_t5 full K={K} N={N}", flush=True)
    rows = sampled_rows(N, 40, K + N)
    t = synth.ternary(K + 3 * N, N, K, 0.35)
    s = synth.scales_f16(K + 3 * N, N, K)
    x = synth.activations_bf16(K, 1, K)
    y = _run_t5(tern, x, oracle_lib.t5_encode(t), s)
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t[rows]), s[rows], K)
    assert_matmul_close(y[:, rows], y_ref, bound, what=f"gemv_t5 full K{K} N{N}")
