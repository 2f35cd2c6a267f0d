"""GPU checks of boundary contracts that are not the matmul arithmetic itself:
the reading of sign vectors whose entries are not all +-1, and binary32
activations too long to stage in LDS.

Sign vectors: only the sign bit of each int8 entry is read, d[k] = -1 where
signs[k] < 0 and +1 otherwise, on every transform path (stand-alone forward
and inverse, fused rotation).  The oracle follows the pages' definition with
an explicit +-1 vector, so it is called with that d.
"""
import numpy as np
import pytest

import synth
from tests._helpers import (assert_fwht_close, assert_matmul_close, pack_to_device, torch, x_to_device,
                            y_to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tern():
    T = torch()
    if not T.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_g128_amd as t
    return t


def _as_pm1(sb: np.ndarray) -> np.ndarray:
    """The documented reading of a sign vector: -1 where negative, else +1."""
    return np.where(sb < 0, -1, 1).astype(np.int8)


def _x(seed, M, K, xdt):
    return synth.activations_f32(seed, M, K) if xdt == "f32" else synth.activations_bf16(seed, M, K)


@pytest.mark.parametrize("M,K,block", [(2, 4096, 4096), (1, 8192, 4096), (3, 512, 64), (2, 4096, 2048),
                                       (1, 256, 16), (2, 64, 8), (1, 32, 2), (2, 16, 1)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_fwht_reads_only_the_sign_bit(tern, oracle_lib, M, K, block, xdt):
    seed = 5 * M + K + block
    print(f"fwht sign bytes M={M} K={K} b={block} {xdt}", flush=True)
    T = torch()
    sb = synth.sign_bytes(seed, K)
    assert (sb == 0).any() and (np.abs(sb.astype(np.int16)) > 1).any()
    d = _as_pm1(sb)
    x = _x(seed, M, K, xdt)
    x64 = x.astype(np.float64) if xdt == "f32" else oracle_lib.bf16_bits_to_f64(x)
    sbd = T.from_numpy(sb).cuda()
    y = tern.tern_fwht(x_to_device(x), sbd, block)
    yi = tern.tern_fwht(y, sbd, block, inverse=True)
    T.cuda.synchronize()
    assert_fwht_close(y_to_host(y), oracle_lib.fwht(x64, d, block), what="forward")
    assert_fwht_close(y_to_host(yi), oracle_lib.fwht(y_to_host(y), d, block, inverse=True), what="inverse")
    assert_fwht_close(y_to_host(yi), x64, what="round trip")
    # the same call with the +-1 vector gives the same bits
    y_pm = tern.tern_fwht(x_to_device(x), T.from_numpy(d).cuda(), block)
    T.cuda.synchronize()
    assert T.equal(y, y_pm)


@pytest.mark.parametrize("M,K,N,block,xdt", [(1, 4096, 300, 4096, "bf16"), (2, 4096, 70, 4096, "f32"),
                                             (1, 1024, 64, 64, "bf16"), (3, 512, 40, 64, "f32"),
                                             (2, 256, 33, 16, "bf16")])
def test_rotate_gemv_reads_only_the_sign_bit(tern, oracle_lib, M, K, N, block, xdt):
    seed = 11 * M + K + N + block
    print(f"rotate gemv sign bytes M={M} K={K} N={N} b={block} {xdt}", flush=True)
    T = torch()
    sb = synth.sign_bytes(seed, K)
    d = _as_pm1(sb)
    t = synth.ternary(seed, N, K, 0.35)
    s = synth.scales_f16(seed, N, K)
    x = _x(seed, M, K, xdt)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(x)
    y = tern.tern_rotate_gemv(xd, T.from_numpy(sb).cuda(), block, codes_d, scales_d)
    y_pm = tern.tern_rotate_gemv(xd, T.from_numpy(d).cuda(), block, codes_d, scales_d)
    T.cuda.synchronize()
    assert T.equal(y, y_pm)
    x64 = x.astype(np.float64) if xdt == "f32" else oracle_lib.bf16_bits_to_f64(x)
    xr = oracle_lib.fwht(x64, d, block)
    codes_o = oracle_lib.encode(t)
    y_ref, bound = oracle_lib.matmul(xr, codes_o, s, K)
    wabs = np.abs(oracle_lib.dequant(codes_o, s, K))
    rot_err = 1e-5 * np.linalg.norm(xr, axis=1, keepdims=True) * np.sqrt((wabs ** 2).sum(axis=1))[None, :]
    assert_matmul_close(y_to_host(y), y_ref, bound + 1e4 * rot_err, what="rotate gemv, sign bytes")


@pytest.mark.parametrize("M", [1, 3, 8, 9])
def test_gemv_f32_activations_beyond_lds(tern, oracle_lib, M):
    """binary32 activations whose staged image would not fit in one
    workgroup's LDS (K = 40960) take direct A loads, split into bfloat16
    parts in registers; M = 9 runs as two launches of at most eight rows."""
    K, N = 40960, 40
    seed = 4096 + M
    print(f"gemv f32 long K M={M} K={K} N={N}", flush=True)
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    x = synth.activations_f32(seed, M, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    y = tern.tern_gemv(x_to_device(x), codes_d, scales_d)
    torch().cuda.synchronize()
    y_ref, bound = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert_matmul_close(y_to_host(y), y_ref, bound, what=f"gemv f32 K{K} M{M}")


def _offset_scales(T, scales_d):
    """The same scale values at a 2-byte (not 4-byte) aligned address: the
    ABI asks scales to be 2-byte aligned only."""
    N, G = scales_d.shape
    buf = T.empty(N * G + 1, dtype=scales_d.dtype, device=scales_d.device)
    view = buf[1:].view(N, G)
    view.copy_(scales_d)
    assert view.data_ptr() % 4 == 2
    return view


def test_scales_two_byte_aligned_every_entry_point(tern):
    """Every matmul entry point gives bit-identical results when its scales
    sit at an address that is 2-byte but not 4-byte aligned (the kernels
    then build each scale pair from two 2-byte loads)."""
    T = torch()
    seed = 71
    cases = [  # (what, M, K, N, x dtype): each kernel family
        ("tiled, binary32 x", 1, 2048, 700, "f32"),
        ("tiled, two rows, three blocks", 2, 768, 300, "bf16"),
        ("even split", 1, 4096, 1000, "bf16"),
        ("activation ring", 8, 2048, 4100, "bf16"),
    ]
    for what, M, K, N, xdt in cases:
        print(f"scales offset: gemv {what} M={M} K={K} N={N}", flush=True)
        t = synth.ternary(seed, N, K)
        s = synth.scales_f16(seed, N, K)
        codes_d, scales_d = pack_to_device(tern, t, s)
        xd = x_to_device(_x(seed, M, K, xdt))
        y0 = tern.tern_gemv(xd, codes_d, scales_d)
        y1 = tern.tern_gemv(xd, codes_d, _offset_scales(T, scales_d))
        T.cuda.synchronize()
        assert T.equal(y0, y1), what
    # fused rotation
    K, N = 4096, 1000
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(synth.activations_bf16(seed, 1, K))
    dd = T.from_numpy(synth.signs(seed, K)).cuda()
    y0 = tern.tern_rotate_gemv(xd, dd, 4096, codes_d, scales_d)
    y1 = tern.tern_rotate_gemv(xd, dd, 4096, codes_d, _offset_scales(T, scales_d))
    T.cuda.synchronize()
    assert T.equal(y0, y1), "rotate_gemv"
    # binary variant
    bits = T.from_numpy(tern.tern_pack_b1(synth.ternary(seed, N, K, 0.0)).view(np.int32)).cuda()
    y0 = tern.tern_gemv_b1(xd, bits, scales_d)
    y1 = tern.tern_gemv_b1(xd, bits, _offset_scales(T, scales_d))
    T.cuda.synchronize()
    assert T.equal(y0, y1), "gemv_b1"
    # prefill GEMM
    M, K, N = 100, 1024, 300
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    codes_d, scales_d = pack_to_device(tern, t, s)
    xd = x_to_device(synth.activations_bf16(seed, M, K))
    y0 = tern.tern_gemm(xd, codes_d, scales_d)
    y1 = tern.tern_gemm(xd, codes_d, _offset_scales(T, scales_d))
    T.cuda.synchronize()
    assert T.equal(y0, y1), "gemm"
