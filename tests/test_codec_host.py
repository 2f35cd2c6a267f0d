"""The library's host codec against the oracle, bit for bit."""
import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def tern():
    import ternary_weight_g128_amd as t
    return t


@pytest.mark.parametrize("N,K,p0", [(1, 128, 1 / 3), (37, 1024, 0.35), (300, 5120, 1 / 3), (64, 17408, 0.0)])
def test_pack_matches_oracle(tern, oracle_lib, N, K, p0):
    t = synth.ternary(N * 7 + K, N, K, p0)
    s = synth.scales_f16(N + K, N, K)
    codes, s2 = tern.tern_pack(t, s)
    assert np.array_equal(codes, oracle_lib.encode(t))
    assert np.array_equal(s2, s)
    assert np.array_equal(tern.tern_unpack(codes, K), t)
    assert np.array_equal(oracle_lib.decode(codes, K), t)


def test_pack_all_word_patterns(tern, oracle_lib):
    # every one of the 3^16 ternary patterns of a 16-slot word, 8 words per
    # 128-wide row, through tern_pack / tern_unpack and the oracle encoder
    total = 3 ** 16
    rows_per_chunk = 3 ** 11 // 8 * 8
    pw = 3 ** np.arange(16, dtype=np.int64)
    start = 0
    while start < total:
        idx = np.arange(start, min(start + rows_per_chunk * 8, total), dtype=np.int64)
        pad = (-len(idx)) % 8
        idx = np.concatenate([idx, np.zeros(pad, dtype=np.int64)])
        t = ((idx[:, None] // pw[None, :]) % 3 - 1).astype(np.int8).reshape(-1, 128)
        s = np.zeros((t.shape[0], 1), dtype=np.uint16)
        codes, _ = tern.tern_pack(t, s)
        assert np.array_equal(codes, oracle_lib.encode(t))
        assert np.array_equal(tern.tern_unpack(codes, 128), t)
        start += rows_per_chunk * 8


def test_dequant_matches_oracle(tern, oracle_lib):
    N, K = 40, 640
    t = synth.ternary(3, N, K)
    s = synth.scales_f16(3, N, K)
    s[0, 0] = 0x0001  # smallest subnormal
    s[1, 1] = 0x8400  # negative normal
    codes, _ = tern.tern_pack(t, s)
    w = tern.tern_dequant_f32(codes, s, K)
    assert np.array_equal(w.astype(np.float64), oracle_lib.dequant(codes, s, K))


def test_pack_f32_matches_oracle(tern, oracle_lib):
    N, K = 12, 512
    t = synth.ternary(9, N, K)
    s = synth.scales_f16(9, N, K)
    s[2, 1] = 0x0003                     # subnormal scale
    t[3, 128:256] = 0                    # all-zero group
    w = (t.astype(np.float64) * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)).astype(np.float32)
    codes, s_out = tern.tern_pack_f32(w)
    t_o, s_o = oracle_lib.ternary_from_f32(w)
    assert np.array_equal(codes, oracle_lib.encode(t_o))
    assert np.array_equal(s_out, s_o)
    w_neg = -w
    codes_n, s_n = tern.tern_pack_f32(w_neg)
    t_n, s_on = oracle_lib.ternary_from_f32(w_neg)
    assert np.array_equal(codes_n, oracle_lib.encode(t_n)) and np.array_equal(s_n, s_on)
    w[5, 7] *= 1.5                       # breaks the one-magnitude rule
    with pytest.raises(tern.TernError) as e:
        tern.tern_pack_f32(w)
    assert e.value.status == tern.TERN_ENOTTERNARY
