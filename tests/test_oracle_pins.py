"""Pins for the FP64 oracle: each check ties an oracle function to something
other than itself -- a closed form, an invariant, a library routine, brute
force on tiny inputs, or a number the pages print.  A plausible slip in the
oracle (dropped term, wrong sign or index, transposed operand, wrong group
index, wrong slot order) fails at least one of these.

CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_half_decode_matches_numpy_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the vectorized twin used for dense dequantization agrees too
    vec = oracle_lib.half_bits_to_f64(bits)
    assert np.array_equal(vec[~nan], ref[~nan]) and np.isnan(vec[nan]).all()


def test_bf16_decode_matches_torch_all_patterns(oracle_lib):
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_lib.bf16_to_double(int(b)) for b in bits[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])
    vec = oracle_lib.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(vec[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# 2-bit slot codec: q = t + 1, 16 slots per word, slot j at bits 2j..2j+1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tval,word", [(-1, 0x00000000), (0, 0x55555555), (1, 0xAAAAAAAA)])
def test_encode_uniform_words(oracle_lib, tval, word):
    t = np.full((3, 256), tval, dtype=np.int8)
    codes = oracle_lib.encode(t)
    assert codes.shape == (3, 16)
    assert (codes == word).all()


def test_encode_single_slot_positions(oracle_lib):
    # one +1 at k in a row of -1: only slot k%16 of word k//16 is nonzero,
    # holding q = 2 at bits 2*(k%16)
    K = 64
    for k in range(K):
        t = np.full((1, K), -1, dtype=np.int8)
        t[0, k] = 1
        codes = oracle_lib.encode(t)[0]
        expect = np.zeros(K // 16, dtype=np.uint32)
        expect[k // 16] = np.uint32(2) << np.uint32(2 * (k % 16))
        assert np.array_equal(codes, expect), k
    # and a zero (q = 1) at k = 17 in a row of -1
    t = np.full((1, K), -1, dtype=np.int8)
    t[0, 17] = 0
    assert oracle_lib.encode(t)[0, 1] == 1 << 2


def test_decode_encode_roundtrip_random(oracle_lib):
    t = synth.ternary(5, 37, 1024)
    codes = oracle_lib.encode(t)
    assert np.array_equal(oracle_lib.decode(codes, 1024), t)


def test_decode_all_patterns_of_eight_slots(oracle_lib):
    # brute force: all 3^8 ternary patterns in slots 0..7 (slots 8..15 all -1)
    n = 3 ** 8
    digits = (np.arange(n)[:, None] // (3 ** np.arange(8))[None, :]) % 3
    t = np.full((n, 16), -1, dtype=np.int8)
    t[:, :8] = digits - 1
    codes = oracle_lib.encode(t)
    # the low 16 bits, read as base-4 digits, must be the pattern q = t + 1
    low = codes[:, 0] & 0xFFFF
    base4 = np.zeros(n, dtype=np.int64)
    for j in reversed(range(8)):
        base4 = base4 * 4 + (digits[:, j])
    assert np.array_equal(low.astype(np.int64), base4)
    assert (codes[:, 0] >> 16 == 0).all()
    assert np.array_equal(oracle_lib.decode(codes, 16), t)


def test_decode_rejects_slot_three(oracle_lib):
    codes = np.full((2, 8), 0x55555555, dtype=np.uint32)
    codes[1, 3] = 0x55555557  # slot 0 of word 3 holds q = 3
    with pytest.raises(ValueError):
        oracle_lib.decode(codes, 128)


def test_encode_rejects_non_ternary(oracle_lib):
    t = np.zeros((1, 16), dtype=np.int8)
    t[0, 5] = 2
    with pytest.raises(ValueError):
        oracle_lib.encode(t)


# ---------------------------------------------------------------------------
# matmul definition y = x (s_g t)^T, error scale B = sum |s_g t x|
# ---------------------------------------------------------------------------

def _dense_from_original(t, s_bits):
    """Dense weights built from the original int8 t and the binary16 scales
    by numpy's own float16 decode -- independent of the oracle's decoder."""
    s = s_bits.view(np.float16).astype(np.float64)
    return t.astype(np.float64) * np.repeat(s, 128, axis=1)


@pytest.mark.parametrize("M,K,N,xdt", [(1, 128, 1, "f32"), (3, 384, 17, "bf16"),
                                       (5, 1024, 33, "f32"), (16, 640, 40, "bf16")])
def test_matmul_matches_numpy_dense(oracle_lib, M, K, N, xdt):
    seed = 1000 + K + N
    t = synth.ternary(seed, N, K)
    s = synth.scales_f16(seed, N, K)
    if xdt == "f32":
        x = synth.activations_f32(seed, M, K)
        x64 = x.astype(np.float64)
    else:
        x = synth.activations_bf16(seed, M, K)
        x64 = oracle_lib.bf16_bits_to_f64(x)
    codes = oracle_lib.encode(t)
    y, b = oracle_lib.matmul(x, codes, s, K)
    W = _dense_from_original(t, s)
    y_np = x64 @ W.T
    b_np = np.abs(x64) @ np.abs(W).T
    assert np.allclose(y, y_np, rtol=0, atol=1e-12 * (b_np.max() + 1))
    assert np.allclose(b, b_np, rtol=1e-13, atol=0)


def test_matmul_zero_weights_exact(oracle_lib):
    K, N = 256, 5
    t = np.zeros((N, K), dtype=np.int8)
    s = synth.scales_f16(1, N, K)
    x = synth.activations_f32(1, 2, K)
    y, b = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert (y == 0).all() and (b == 0).all()


def test_matmul_all_plus_one_is_group_sums(oracle_lib):
    K, N = 512, 3
    t = np.ones((N, K), dtype=np.int8)
    s = synth.scales_f16(2, N, K)
    x = synth.activations_f32(2, 2, K).astype(np.float64)
    y, b = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    gsum = x.reshape(2, K // 128, 128).sum(axis=2)            # [M, G]
    gabs = np.abs(x).reshape(2, K // 128, 128).sum(axis=2)
    sv = s.view(np.float16).astype(np.float64)                 # [N, G]
    assert np.allclose(y, gsum @ sv.T, rtol=1e-14, atol=1e-14)
    assert np.allclose(b, gabs @ np.abs(sv).T, rtol=1e-14)


def test_matmul_one_hot_exact(oracle_lib):
    K, N = 384, 4
    x = synth.activations_f32(3, 3, K)
    s = synth.scales_f16(3, N, K)
    for n, k, sign in [(0, 0, 1), (1, 200, -1), (2, 383, 1), (3, 128, -1)]:
        t = np.zeros((N, K), dtype=np.int8)
        t[n, k] = sign
        y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
        sv = float(s.view(np.float16)[n, k // 128])
        expect = np.zeros((3, N))
        expect[:, n] = sign * sv * x[:, k].astype(np.float64)
        assert np.array_equal(y, expect)


def test_matmul_identity_exact(oracle_lib):
    K = 256
    t = np.eye(K, dtype=np.int8)
    s = np.full((K, K // 128), 0x3C00, dtype=np.uint16)  # 1.0
    x = synth.activations_bf16(4, 2, K)
    y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    assert np.array_equal(y, oracle_lib.bf16_bits_to_f64(x))


def test_matmul_integer_inputs_exact(oracle_lib):
    # integer x in [-64, 64] and scales in {0.5, 1, 2}: exact integer-like sums
    rng = np.random.default_rng(7)
    M, K, N = 4, 1024, 9
    t = synth.ternary(7, N, K)
    s = rng.choice(np.array([0.5, 1.0, 2.0], dtype=np.float16), size=(N, K // 128))
    x = rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s.view(np.uint16), K)
    W2 = t.astype(np.int64) * np.repeat((s.astype(np.float64) * 2).astype(np.int64), 128, axis=1)
    expect = (x.astype(np.int64) @ W2.T).astype(np.float64) / 2
    assert np.array_equal(y, expect)


def test_matmul_symmetries(oracle_lib):
    M, K, N = 2, 256, 6
    t = synth.ternary(8, N, K)
    s = synth.scales_f16(8, N, K)
    x = synth.activations_f32(8, M, K)
    y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s, K)
    # (s, t) -> (-s, -t): same weights
    y2, _ = oracle_lib.matmul(x, oracle_lib.encode(-t), s ^ np.uint16(0x8000), K)
    assert np.array_equal(y, y2)
    # s -> 2s: y -> 2y exactly (binary16 exponent + 1, no overflow at these sizes)
    s2 = (s.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y3, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s2, K)
    assert np.array_equal(y3, 2 * y)
    # linear in x
    x2 = synth.activations_f32(9, M, K)
    ya, _ = oracle_lib.matmul(x.astype(np.float64) + x2.astype(np.float64), oracle_lib.encode(t), s, K)
    yb, _ = oracle_lib.matmul(x2, oracle_lib.encode(t), s, K)
    assert np.allclose(ya, y + yb, rtol=0, atol=1e-12)


def test_matmul_row_group_indexing(oracle_lib):
    # a distinct power-of-two scale per (n, g) and x = 1: y[n] = sum_g 2^(n*G+g) * sum_k t
    K, N = 512, 3
    G = K // 128
    t = np.ones((N, K), dtype=np.int8)
    sv = np.array([[2.0 ** (n * G + g - 6) for g in range(G)] for n in range(N)], dtype=np.float16)
    x = np.ones((1, K), dtype=np.float32)
    y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), sv.view(np.uint16), K)
    expect = np.array([[sum(128 * 2.0 ** (n * G + g - 6) for g in range(G)) for n in range(N)]])
    assert np.array_equal(y, expect)


def test_matmul_at_matches_full(oracle_lib):
    M, K, N = 3, 384, 21
    t = synth.ternary(11, N, K)
    s = synth.scales_f16(11, N, K)
    x = synth.activations_bf16(11, M, K)
    codes = oracle_lib.encode(t)
    y, b = oracle_lib.matmul(x, codes, s, K)
    ms = np.array([0, 2, 1, 2])
    ns = np.array([0, 20, 7, 3])
    ys, bs = oracle_lib.matmul_at(x, codes, s, K, ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(bs, b[ms, ns])


# ---------------------------------------------------------------------------
# signed normalized Walsh-Hadamard transform
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_fwht_matches_scipy_hadamard(oracle_lib, b):
    rng = np.random.default_rng(b)
    x = rng.normal(size=(2, 3 * b))
    d = np.where(rng.random(3 * b) < 0.5, -1, 1).astype(np.int8)
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    y = oracle_lib.fwht(x, d, b)
    xs = (x * d).reshape(2, 3, b)
    expect = np.einsum("il,mjl->mji", H, xs).reshape(2, 3 * b)
    assert np.allclose(y, expect, rtol=0, atol=1e-12)


def test_fwht_4096_entries_match_scipy(oracle_lib):
    H = scipy.linalg.hadamard(4096, dtype=np.int8)
    rng = np.random.default_rng(0)
    ii = rng.integers(0, 4096, size=2000)
    ll = rng.integers(0, 4096, size=2000)
    got = np.array([oracle_lib.hadamard_entry(int(i), int(l)) for i, l in zip(ii, ll)])
    assert np.array_equal(got, H[ii, ll].astype(np.float64))


def test_fwht_4096_forward_matches_scipy(oracle_lib):
    b = 4096
    x = oracle_lib.bf16_bits_to_f64(synth.activations_bf16(21, 1, b))
    d = synth.signs(21, b)
    H = scipy.linalg.hadamard(b, dtype=np.int8).astype(np.float64)
    y = oracle_lib.fwht(x, d, b)
    assert np.allclose(y[0], H @ (d * x[0]) / 64.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("b", [2, 32, 512])
def test_fwht_involution_and_inverse(oracle_lib, b):
    rng = np.random.default_rng(b + 1)
    x = rng.normal(size=(3, 2 * b))
    d = np.where(rng.random(2 * b) < 0.5, -1, 1).astype(np.int8)
    # unsigned normalized H is its own inverse: H H = I
    assert np.allclose(oracle_lib.fwht(oracle_lib.fwht(x, None, b), None, b), x, atol=1e-12)
    # the signed inverse undoes the signed forward transform
    y = oracle_lib.fwht(x, d, b)
    assert np.allclose(oracle_lib.fwht(y, d, b, inverse=True), x, atol=1e-12)
    # Parseval: the normalized transform preserves the norm of each row
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_fwht_closed_forms(oracle_lib):
    b = 64
    e0 = np.zeros((1, b)); e0[0, 0] = 1.0
    assert np.allclose(oracle_lib.fwht(e0, None, b), np.full((1, b), 1 / 8.0), atol=0)
    ones = np.ones((1, b))
    expect = np.zeros((1, b)); expect[0, 0] = 8.0
    assert np.allclose(oracle_lib.fwht(ones, None, b), expect, atol=1e-15)
    # b = 1 is the identity (with signs applied); b = 2 is [[1,1],[1,-1]]/sqrt 2
    x = np.array([[3.0, -5.0, 7.0, 11.0]])
    d = np.array([1, -1, -1, 1], dtype=np.int8)
    assert np.array_equal(oracle_lib.fwht(x, d, 1), x * d)
    r2 = 1 / math.sqrt(2)
    assert np.allclose(oracle_lib.fwht(x, None, 2),
                       np.array([[-2 * r2, 8 * r2, 18 * r2, -4 * r2]]), atol=1e-15)


def test_fwht_rotation_fold_invariance(oracle_lib):
    # W x = (W D H / sqrt b)(H D x / sqrt b): folding the rotation into the
    # stored weights and applying the matching transform to activations
    # leaves the product unchanged.
    b, N = 256, 7
    rng = np.random.default_rng(3)
    W = rng.normal(size=(N, b))
    x = rng.normal(size=(1, b))
    d = np.where(rng.random(b) < 0.5, -1, 1).astype(np.int8)
    xr = oracle_lib.fwht(x, d, b)             # H D x / sqrt b
    Wr = oracle_lib.fwht(W, d, b)             # rows: H D w / sqrt b
    assert np.allclose(xr @ Wr.T, x @ W.T, atol=1e-10)


def test_fwht_rejects_ragged_block(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.fwht(np.zeros((1, 96)), None, 64)


# ---------------------------------------------------------------------------
# lossless FP32 -> ternary-g128 reading
# ---------------------------------------------------------------------------

def test_ternary_from_f32_roundtrip(oracle_lib):
    N, K = 6, 512
    t = synth.ternary(31, N, K)
    s = synth.scales_f16(31, N, K)
    w = (t.astype(np.float64) * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)).astype(np.float32)
    got = oracle_lib.ternary_from_f32(w)
    assert got is not None
    t2, s2 = got
    assert np.array_equal(t2, t) and np.array_equal(s2, s)


def test_ternary_from_f32_canonical_sign_and_zero_groups(oracle_lib):
    K = 256
    w = np.zeros((2, K), dtype=np.float32)
    w[0, :128] = -0.25          # negative scale reading -> s = +0.25, t = -1
    w[1, 128:130] = [0.5, -0.5]
    t, s = oracle_lib.ternary_from_f32(w)
    assert s[0, 0] == np.float16(0.25).view(np.uint16) and (t[0, :128] == -1).all()
    assert s[0, 1] == 0 and s[1, 0] == 0          # all-zero groups get +0
    assert s[1, 1] == np.float16(0.5).view(np.uint16)
    assert list(t[1, 128:131]) == [1, -1, 0]


def test_ternary_from_f32_rejects(oracle_lib):
    K = 128
    w = np.zeros((1, K), dtype=np.float32)
    w[0, :2] = [0.5, 0.25]                      # two magnitudes in one group
    assert oracle_lib.ternary_from_f32(w) is None
    w = np.zeros((1, K), dtype=np.float32)
    w[0, 0] = 0.1                               # not binary16-exact
    assert oracle_lib.ternary_from_f32(w) is None


# ---------------------------------------------------------------------------
# storage accounting against the pages' printed numbers
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "accounting.json")) as f:
        return {e["key"]: e["value"] for e in json.load(f)["entries"]}


def test_bits_per_weight_is_2125(oracle_lib):
    g = _golden()
    for N, K in [(1, 128), (1024, 1024), (17408, 5120), (248320, 5120)]:
        assert oracle_lib.bits_per_weight(N, K) == g["deployed_bits_per_weight"] == 2.125


def test_pages_accounting_relations():
    g = _golden()
    info = math.log2(3)
    assert round(info, 3) == g["bits_per_ternary_value"]
    eff = info + 16 / 128                       # code + scale amortised over 128
    assert round(eff, 2) == g["effective_bits_per_weight"]
    assert round(16 / eff, 1) == g["theoretical_shrink_vs_fp16"]
    p = g["ternary_language_weights_billion"]
    assert abs(p * 16 / 8 - g["fp16_size_gb"]) / g["fp16_size_gb"] < 0.02
    assert abs(p * eff / 8 - g["theoretical_size_gb"]) / g["theoretical_size_gb"] < 0.02
    assert abs(p * 2.125 / 8 - g["deployed_size_gb"]) / g["deployed_size_gb"] < 0.02
    # g128 package at 2.125 b/w and g64 repeated-scale package at 2 + 16/64
    # b/w hold the same number of weights
    n128 = g["g128_package_gb"] * 8 / g["deployed_bits_per_weight"]
    n64 = g["g64_package_gb"] * 8 / (2 + 16 / 64)
    assert abs(n128 - n64) / n128 < 0.002
    # MLX: two FP16 values per group of 128; 1-bit: 1 + 16/128
    assert 2 + 32 / 128 == g["mlx_bits_per_weight"]
    assert 1 + 16 / 128 == g["binary_bits_per_weight"]
    assert round(2.125 / 1.125, 1) == g["ternary_vs_binary_bytes_ratio"]


# ---------------------------------------------------------------------------
# format variants: group-64 scales, affine (scale, bias) container, binary g128
# ---------------------------------------------------------------------------

def _np_pack_fields(q, bits):
    """Pack unsigned fields q [N, K] (each < 2^bits) lowest-first into uint32
    words, written with numpy shifts only."""
    N, K = q.shape
    per = 32 // bits
    q = q.astype(np.uint64).reshape(N, K // per, per)
    shifts = (np.arange(per, dtype=np.uint64) * bits)[None, None, :]
    return (q << shifts).sum(axis=2).astype(np.uint32)


def test_format_bits_per_weight_pages(oracle_lib):
    g = _golden()
    for N, K in [(1, 128), (17408, 5120), (248320, 5120)]:
        assert oracle_lib.format_bits_per_weight(oracle_lib.FMT_G128, N, K) == g["deployed_bits_per_weight"]
        assert oracle_lib.format_bits_per_weight(oracle_lib.FMT_AFFINE2, N, K) == g["mlx_bits_per_weight"]
        assert oracle_lib.format_bits_per_weight(oracle_lib.FMT_B1, N, K) == g["binary_bits_per_weight"]
        assert oracle_lib.format_bits_per_weight(oracle_lib.FMT_G64, N, K) == 2.25
        assert oracle_lib.format_bits_per_weight(oracle_lib.FMT_AFFINE1, N, K) == 1.25
    # the two shipped ternary packages hold the same weights
    n128 = g["g128_package_gb"] * 8 / oracle_lib.format_bits_per_weight(oracle_lib.FMT_G128, 1, 128)
    n64 = g["g64_package_gb"] * 8 / oracle_lib.format_bits_per_weight(oracle_lib.FMT_G64, 1, 128)
    assert abs(n128 - n64) / n128 < 0.002
    b1 = oracle_lib.format_bits_per_weight(oracle_lib.FMT_B1, 1, 128)
    assert round(2.125 / b1, 1) == g["ternary_vs_binary_bytes_ratio"]
    assert oracle_lib.format_bits_per_weight(9, 1, 128) == -1.0


def test_dequant_g64_is_repeated_g128(oracle_lib):
    rng = np.random.default_rng(61)
    N, K = 5, 512
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    s128 = synth.scales_f16(611, N, K)
    codes = oracle_lib.encode(t)
    dense = t.astype(np.float64) * np.repeat(oracle_lib.half_bits_to_f64(s128), 128, axis=1)
    s64 = np.repeat(s128, 2, axis=1)
    assert np.array_equal(oracle_lib.dequant_g64(codes, s64, K), dense)
    # distinct halves: weight k takes the scale of its own 64-block
    s64b = synth.scales_f16(612, N, 2 * K)
    dense_b = t.astype(np.float64) * np.repeat(oracle_lib.half_bits_to_f64(s64b), 64, axis=1)
    assert np.array_equal(oracle_lib.dequant_g64(codes, s64b, K), dense_b)


@pytest.mark.parametrize("bits,group", [(2, 128), (2, 64), (1, 128), (1, 32)])
def test_dequant_affine_closed_form(oracle_lib, bits, group):
    rng = np.random.default_rng(62 + bits + group)
    N, K = 4, 256
    q = rng.integers(0, 1 << bits, size=(N, K))
    words = _np_pack_fields(q, bits)
    sc = synth.scales_f16(621, N, K * 128 // group)
    bi = synth.scales_f16(622, N, K * 128 // group) | np.uint16(0x8000)
    want = (q.astype(np.float64) * np.repeat(oracle_lib.half_bits_to_f64(sc), group, axis=1)
            + np.repeat(oracle_lib.half_bits_to_f64(bi), group, axis=1))
    assert np.array_equal(oracle_lib.dequant_affine(words, bits, group, sc, bi, K), want)


def test_affine_pairs_reading_of_the_mlx_packaging(oracle_lib):
    """The pair (2 s, -s) gives exactly +-s on one-bit fields, as the MLX
    packaging section says, but no zero level on 2-bit fields; the pair
    (s, -s) on the 2-bit slots q = t + 1 gives exactly s * t."""
    rng = np.random.default_rng(63)
    N, K = 3, 256
    s = synth.scales_f16(631, N, K)                      # positive FP16
    sd = oracle_lib.half_bits_to_f64(s)
    two_s = np.array([[np.float16(2.0 * v) for v in row] for row in sd], dtype=np.float16).view(np.uint16)
    neg_s = s | np.uint16(0x8000)
    b = rng.choice(np.array([-1, 1], dtype=np.int8), size=(N, K))
    bits = oracle_lib.b1_encode(b)
    w1 = oracle_lib.dequant_affine(bits, 1, 128, two_s, neg_s, K)
    assert np.array_equal(w1, b * np.repeat(sd, 128, axis=1))
    q_all = np.tile(np.arange(4), (N, K // 4))
    w2 = oracle_lib.dequant_affine(_np_pack_fields(q_all, 2), 2, 128, two_s, neg_s, K)
    levels = np.repeat(sd, 128, axis=1)
    assert np.array_equal(w2, (2 * q_all - 1) * levels)  # -s, s, 3s, 5s
    assert not np.any(w2 == 0)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    w3 = oracle_lib.dequant_affine(oracle_lib.encode(t), 2, 128, s, neg_s, K)
    assert np.array_equal(w3, t * levels)


def test_b1_decode_all_patterns_of_sixteen_bits(oracle_lib):
    pats = np.arange(1 << 16, dtype=np.uint32)
    for shift in (0, 16):
        words = np.zeros((pats.size, 4), dtype=np.uint32)      # K = 128
        words[:, 2] = pats << shift
        b = oracle_lib.b1_decode(words, 128)
        idx = np.arange(16)
        want = np.where(((pats[:, None] >> idx[None, :]) & 1) == 1, 1, -1)
        assert np.array_equal(b[:, 64 + shift: 64 + shift + 16], want)
        others = np.delete(np.arange(128), np.arange(64 + shift, 80 + shift))
        assert np.all(b[:, others] == -1)
        assert np.array_equal(oracle_lib.b1_encode(b), words)


def test_b1_encode_rejects_non_binary(oracle_lib):
    for bad in (0, 2, -2):
        b = np.ones((2, 128), dtype=np.int8)
        b[1, 77] = bad
        with pytest.raises(ValueError):
            oracle_lib.b1_encode(b)


# ---------------------------------------------------------------------------
# base-3 layout (five ternary values per byte, superblocks of five groups)
# ---------------------------------------------------------------------------

def _np_t5(t):
    """The base-3 layout built with numpy reshapes: digit j of byte i of
    superblock b is weight i of group 5b + j; missing groups are zero digits."""
    N, K = t.shape
    G = K // 128
    SB = (G + 4) // 5
    q = np.zeros((N, SB * 5, 128), dtype=np.int64)
    q[:, :G, :] = (t.astype(np.int64) + 1).reshape(N, G, 128)
    q = q.reshape(N, SB, 5, 128)
    w = (3 ** np.arange(5, dtype=np.int64))[None, None, :, None]
    return (q * w).sum(axis=2).reshape(N, SB * 128).astype(np.uint8)


def test_t5_every_byte_value(oracle_lib):
    v = np.arange(243, dtype=np.uint8)
    d = np.repeat(v[:, None], 128, axis=1)             # K = 640: one full superblock
    t = oracle_lib.t5_decode(d, 640)
    for j in range(5):
        digit = (v.astype(np.int64) // 3 ** j) % 3
        assert np.array_equal(t[:, 128 * j:128 * (j + 1)], np.repeat(digit[:, None] - 1, 128, axis=1))
    assert np.array_equal(oracle_lib.t5_encode(t), d)
    for bad in (243, 255):
        e = d[:1].copy()
        e[0, 77] = bad
        with pytest.raises(ValueError):
            oracle_lib.t5_decode(e, 640)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 7, 13, 40, 136])
def test_t5_layout_matches_numpy(oracle_lib, G):
    K = 128 * G
    t = synth.ternary(900 + G, 5, K)
    d = oracle_lib.t5_encode(t)
    assert d.shape == (5, ((G + 4) // 5) * 128)
    assert np.array_equal(d, _np_t5(t))
    assert np.array_equal(oracle_lib.t5_decode(d, K), t)
    p = G % 5
    if p:                                              # the tail superblock holds p digits
        e = d.copy()
        e[2, -1] = 3 ** p
        with pytest.raises(ValueError):
            oracle_lib.t5_decode(e, K)
        e[2, -1] = 3 ** p - 1
        assert oracle_lib.t5_decode(e, K)[2, -1] == 1


def test_t5_accounting(oracle_lib):
    g = _golden()
    for N, K in [(1, 640), (17408, 5120), (248320, 5120)]:
        assert oracle_lib.t5_bits_per_weight(N, K) == 1.6 + 16 / 128
    info = math.log2(3) + 16 / 128
    assert round(info, 2) == g["effective_bits_per_weight"]
    assert info < oracle_lib.t5_bits_per_weight(1, 640) < g["deployed_bits_per_weight"]
    # a ragged tail costs a whole superblock: K = 4096 is 7 superblocks for 32 groups
    assert oracle_lib.t5_bits_per_weight(1, 4096) == 8 * (7 * 128 + 64) / 4096


# ---------------------------------------------------------------------------
# Threaded oracle matmul: the outputs shared out over host threads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_matmul_bit_identical_to_serial(oracle_lib, threads):
    # each output is the same k-ordered double sum, whichever thread runs it
    M, K, N = 3, 1280, 97
    t = synth.ternary(41, N, K)
    s = synth.scales_f16(41, N, K)
    x = synth.activations_bf16(41, M, K)
    codes = oracle_lib.encode(t)
    y1, b1 = oracle_lib.matmul(x, codes, s, K)
    yt, bt = oracle_lib.matmul(x, codes, s, K, threads=threads)
    assert np.array_equal(y1, yt) and np.array_equal(b1, bt)


def test_threaded_matmul_integer_inputs_exact(oracle_lib):
    # the integer-exact closed form, through the threaded entry point itself
    rng = np.random.default_rng(19)
    M, K, N = 5, 2048, 33
    t = synth.ternary(19, N, K)
    s = rng.choice(np.array([0.5, 1.0, 2.0], dtype=np.float16), size=(N, K // 128))
    x = rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    y, _ = oracle_lib.matmul(x, oracle_lib.encode(t), s.view(np.uint16), K, threads=4)
    W2 = t.astype(np.int64) * np.repeat((s.astype(np.float64) * 2).astype(np.int64), 128, axis=1)
    expect = (x.astype(np.int64) @ W2.T).astype(np.float64) / 2
    assert np.array_equal(y, expect)


def test_threaded_matmul_matches_numpy_dense(oracle_lib):
    M, K, N = 2, 768, 50
    t = synth.ternary(23, N, K)
    s = synth.scales_f16(23, N, K)
    x = synth.activations_f32(23, M, K)
    y, b = oracle_lib.matmul(x, oracle_lib.encode(t), s, K, threads=5)
    W = _dense_from_original(t, s)
    x64 = x.astype(np.float64)
    assert np.allclose(y, x64 @ W.T, rtol=0, atol=1e-12 * (np.abs(x64) @ np.abs(W).T).max())
    with pytest.raises(ValueError):
        bad = oracle_lib.encode(t)
        bad[0, 0] |= 3
        oracle_lib.matmul(x, bad, s, K, threads=3)
