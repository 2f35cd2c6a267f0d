"""Format variants of the library's host codec (group-64 scales, the affine
scale+bias container, binary g128 weights) against the oracle's definitions
of each format's dequantized weights.  CPU only."""
import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def tern():
    import ternary_weight_g128_amd as t
    return t


def _all_finite_halves():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return h[((h >> 10) & 0x1F) != 0x1F]


def _status(tern, exc):
    return exc.value.status


# ---------------------------------------------------------------------------
# accounting
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 128), (300, 5120), (17408, 5120)])
def test_variant_byte_counts_match_oracle_accounting(tern, oracle_lib, N, K):
    nk = N * K
    codes, s128 = tern.tern_codes_bytes(N, K), tern.tern_scales_bytes(N, K)
    s64, b1 = tern.tern_scales_g64_bytes(N, K), tern.tern_b1_bytes(N, K)
    assert 8 * (codes + s64) / nk == oracle_lib.format_bits_per_weight(oracle_lib.FMT_G64, N, K)
    assert 8 * (codes + 2 * s128) / nk == oracle_lib.format_bits_per_weight(oracle_lib.FMT_AFFINE2, N, K)
    assert 8 * (b1 + s128) / nk == oracle_lib.format_bits_per_weight(oracle_lib.FMT_B1, N, K)
    assert 8 * (b1 + 2 * s128) / nk == oracle_lib.format_bits_per_weight(oracle_lib.FMT_AFFINE1, N, K)
    assert tern.tern_scales_g64_bytes(1, 100) == 0 and tern.tern_b1_bytes(-1, 128) == 0


# ---------------------------------------------------------------------------
# group-64 scales
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 128), (19, 1024), (64, 5120)])
def test_g64_scales_same_weights(tern, oracle_lib, N, K):
    t = synth.ternary(700 + N, N, K)
    s = synth.scales_f16(701 + K, N, K)
    codes = oracle_lib.encode(t)
    s64 = tern.tern_scales_to_g64(s)
    assert s64.shape == (N, K // 64)
    assert np.array_equal(oracle_lib.dequant_g64(codes, s64, K), oracle_lib.dequant(codes, s, K))
    assert np.array_equal(tern.tern_scales_from_g64(s64), s)


def test_g64_from_rejects(tern):
    s = synth.scales_f16(710, 3, 256)
    s64 = tern.tern_scales_to_g64(s)
    bad = s64.copy()
    bad[2, 3] ^= np.uint16(1)                # halves of group (2, 1) differ
    with pytest.raises(tern.TernError) as e:
        tern.tern_scales_from_g64(bad)
    assert e.value.status == tern.TERN_ENOTTERNARY
    inf = s64.copy()
    inf[0, 0] = inf[0, 1] = 0x7C00
    with pytest.raises(tern.TernError) as e:
        tern.tern_scales_from_g64(inf)
    assert e.value.status == tern.TERN_EINVAL
    zeros = s64.copy()
    zeros[1, 0], zeros[1, 1] = 0x0000, 0x8000  # +0 and -0 are one value
    assert tern.tern_scales_from_g64(zeros)[1, 0] == 0x0000


# ---------------------------------------------------------------------------
# affine (scale, bias) container
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 128), (23, 1024), (40, 5120)])
def test_mlx_export_same_weights(tern, oracle_lib, N, K):
    t = synth.ternary(720 + N, N, K, 0.35)
    s = synth.scales_f16(721 + K, N, K)
    codes = oracle_lib.encode(t)
    sc, bi = tern.tern_mlx_export(s)
    assert np.array_equal(oracle_lib.dequant_affine(codes, 2, 128, sc, bi, K),
                          oracle_lib.dequant(codes, s, K))
    assert np.array_equal(tern.tern_mlx_import(sc, bi), s)


def test_mlx_export_every_finite_scale(tern, oracle_lib):
    h = _all_finite_halves()
    s = h.reshape(-1, 1)                       # one group per row, K = 128
    t = np.zeros((s.shape[0], 128), dtype=np.int8)
    t[:, 0], t[:, 1], t[:, 2] = -1, 0, 1
    codes = oracle_lib.encode(t)
    sc, bi = tern.tern_mlx_export(s)
    w = oracle_lib.dequant_affine(codes, 2, 128, sc, bi, 128)
    assert np.array_equal(w, oracle_lib.dequant(codes, s, 128))
    assert np.array_equal(tern.tern_mlx_import(sc, bi), s)


def test_mlx_import_rejects(tern):
    s = synth.scales_f16(730, 2, 256)
    sc, bi = tern.tern_mlx_export(s)
    bad = bi.copy()
    bad[1, 1] = sc[1, 1]                       # bias = +scale
    with pytest.raises(tern.TernError) as e:
        tern.tern_mlx_import(sc, bad)
    assert e.value.status == tern.TERN_ENOTTERNARY
    nan = sc.copy()
    nan[0, 0] = 0x7E00
    with pytest.raises(tern.TernError) as e:
        tern.tern_mlx_import(nan, bi)
    assert e.value.status == tern.TERN_EINVAL
    with pytest.raises(tern.TernError) as e:
        tern.tern_mlx_export(nan)
    assert e.value.status == tern.TERN_EINVAL
    z = np.array([[0x0000, 0x8000]], dtype=np.uint16)
    assert np.array_equal(tern.tern_mlx_import(z, z), z)   # (+0, +0) and (-0, -0)


# ---------------------------------------------------------------------------
# binary g128
# ---------------------------------------------------------------------------

def _binary(seed, N, K):
    return np.where(np.random.default_rng(seed).random((N, K)) < 0.5, 1, -1).astype(np.int8)


@pytest.mark.parametrize("N,K", [(1, 128), (31, 1024), (300, 5120)])
def test_b1_pack_matches_oracle(tern, oracle_lib, N, K):
    b = _binary(740 + N, N, K)
    bits = tern.tern_pack_b1(b)
    assert np.array_equal(bits, oracle_lib.b1_encode(b))
    assert np.array_equal(tern.tern_unpack_b1(bits, K), b)
    codes = tern.tern_b1_to_codes(bits, K)
    assert np.array_equal(oracle_lib.decode(codes, K), oracle_lib.b1_decode(bits, K))
    assert np.array_equal(tern.tern_codes_to_b1(codes, K), bits)


def test_b1_all_sixteen_bit_patterns(tern, oracle_lib):
    pats = np.arange(1 << 16, dtype=np.uint32)
    bits = np.zeros((pats.size, 4), dtype=np.uint32)   # K = 128
    bits[:, 1] = pats | (pats[::-1] << 16)
    bits[:, 3] = pats << 16
    want = oracle_lib.b1_decode(bits, 128)
    assert np.array_equal(tern.tern_unpack_b1(bits, 128), want)
    assert np.array_equal(tern.tern_pack_b1(want), bits)
    codes = tern.tern_b1_to_codes(bits, 128)
    assert np.array_equal(oracle_lib.decode(codes, 128), want)
    assert np.array_equal(tern.tern_codes_to_b1(codes, 128), bits)


def test_b1_rejects(tern):
    b = _binary(750, 2, 128)
    b[1, 5] = 0
    with pytest.raises(tern.TernError) as e:
        tern.tern_pack_b1(b)
    assert e.value.status == tern.TERN_ENOTTERNARY
    codes = tern.tern_b1_to_codes(tern.tern_pack_b1(_binary(751, 2, 128)), 128)
    z = codes.copy()
    z[1, 3] = (z[1, 3] & ~np.uint32(3 << 10)) | np.uint32(1 << 10)   # a zero weight
    with pytest.raises(tern.TernError) as e:
        tern.tern_codes_to_b1(z, 128)
    assert e.value.status == tern.TERN_ENOTTERNARY
    q3 = codes.copy()
    q3[0, 7] |= np.uint32(3 << 30)
    with pytest.raises(tern.TernError) as e:
        tern.tern_codes_to_b1(q3, 128)
    assert e.value.status == tern.TERN_EBADCODE


def test_b1_affine_export_every_scale(tern, oracle_lib):
    h = _all_finite_halves()
    ok = (h & 0x7FFF) < 0x7800                 # |s| < 32768: 2s is finite
    s = h[ok].reshape(-1, 1)
    b = np.ones((s.shape[0], 128), dtype=np.int8)
    b[:, ::3] = -1
    bits = oracle_lib.b1_encode(b)
    sc, bi = tern.tern_mlx_export_b1(s)
    w = oracle_lib.dequant_affine(bits, 1, 128, sc, bi, 128)
    assert np.array_equal(w, b * oracle_lib.half_bits_to_f64(s))
    back = tern.tern_mlx_import_b1(sc, bi)
    assert np.array_equal(oracle_lib.half_bits_to_f64(back), oracle_lib.half_bits_to_f64(s))
    assert np.array_equal(back[(s & 0x7FFF) != 0], s[(s & 0x7FFF) != 0])
    for big in h[~ok][:50]:
        with pytest.raises(tern.TernError) as e:
            tern.tern_mlx_export_b1(np.array([[big]], dtype=np.uint16))
        assert e.value.status == tern.TERN_EINVAL
    bad = sc.copy()
    bad[5, 0] = bi[5, 0] ^ np.uint16(0x8000)   # scale = s instead of 2s
    with pytest.raises(tern.TernError) as e:
        tern.tern_mlx_import_b1(bad, bi)
    assert e.value.status == tern.TERN_ENOTTERNARY


# ---------------------------------------------------------------------------
# base-3 layout (five ternary values per byte)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 128), (9, 512), (17, 640), (33, 4096), (64, 5120), (40, 17408)])
def test_t5_pack_matches_oracle(tern, oracle_lib, N, K):
    t = synth.ternary(960 + N + K, N, K, 0.35)
    codes = oracle_lib.encode(t)
    data = tern.tern_pack_t5(codes, K)
    assert np.array_equal(data, oracle_lib.t5_encode(t))
    assert np.array_equal(tern.tern_unpack_t5(data, K), codes)
    assert tern.tern_t5_bytes(N, K) == data.size
    bpw = 8 * (data.size + tern.tern_scales_bytes(N, K)) / (N * K)
    assert bpw == oracle_lib.t5_bits_per_weight(N, K)


def test_t5_every_byte_and_tail_width(tern, oracle_lib):
    for G in (1, 2, 3, 4, 5):
        K = 128 * G
        lim = 3 ** G
        d = np.zeros((lim, 128), dtype=np.uint8)
        d[:, :] = np.arange(lim, dtype=np.int64)[:, None]
        codes = tern.tern_unpack_t5(d, K)
        assert np.array_equal(tern.tern_unpack(codes, K), oracle_lib.t5_decode(d, K))
        assert np.array_equal(tern.tern_pack_t5(codes, K), d)
        if lim < 256:
            bad = d[:1].copy()
            bad[0, 100] = lim
            with pytest.raises(tern.TernError) as e:
                tern.tern_unpack_t5(bad, K)
            assert e.value.status == tern.TERN_EBADCODE


def test_t5_pack_rejects_slot_three(tern):
    codes = np.zeros((2, 640 // 16), dtype=np.uint32)
    codes[1, 9] = 3 << 6
    with pytest.raises(tern.TernError) as e:
        tern.tern_pack_t5(codes, 640)
    assert e.value.status == tern.TERN_EBADCODE
