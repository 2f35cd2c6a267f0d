// Host codec of libtern: lossless transcode between int8 ternary values (or
// FP32 weights of ternary-g128 form) and the 2-bit-slot g128 format, plus the
// storage accounting.
//
// Format ("prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card, "Weight
// representation: ternary g128" and "Memory requirement"): t in {-1,0,+1},
// one binary16 scale per 128 consecutive K of an output row, each t in a
// 2-bit slot.  Slot code q = t + 1; slot j of word w holds k = 16 w + j at
// bits 2j..2j+1 of a little-endian uint32.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "tern_internal.h"

namespace {

constexpr int64_t kGroup = TERN_GROUP;
constexpr int64_t kSlots = TERN_SLOTS_PER_WORD;

thread_local std::string g_last_error;

bool sizes_ok(int64_t N, int64_t K) { return N >= 0 && K >= 0 && K % kGroup == 0; }

// Run fn(row_begin, row_end) over [0, N) on up to hardware_concurrency
// threads when the matrix is large; each row range is independent.
template <class Fn>
void for_rows(int64_t N, int64_t K, Fn fn)
{
    int64_t work = N * K;
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    int64_t nthreads = std::min<int64_t>({(int64_t)hw, 16, std::max<int64_t>(1, work >> 22), N});
    if (nthreads <= 1) {
        fn(0, N);
        return;
    }
    std::vector<std::thread> pool;
    for (int64_t i = 0; i < nthreads; ++i) {
        int64_t a = N * i / nthreads, b = N * (i + 1) / nthreads;
        pool.emplace_back([=] { fn(a, b); });
    }
    for (auto &th : pool) th.join();
}

// binary16 bits -> float (exact), from the format definition.
float half_bits_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t e = (h >> 10) & 0x1f, f = h & 0x3ff;
    float v;
    if (e == 0) {
        v = std::ldexp((float)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = std::ldexp(1.0f + (float)f / 1024.0f, (int)e - 15);
    }
    uint32_t u;
    std::memcpy(&u, &v, 4);
    u |= sign;
    std::memcpy(&v, &u, 4);
    return v;
}

bool half_finite(uint16_t h) { return ((h >> 10) & 0x1f) != 31; }

// Exact binary16 encoding of a positive finite float, if one exists.
bool float_to_half_exact(float a, uint16_t *out)
{
    if (!(a >= 0.0f) || !std::isfinite(a)) return false;
    if (a == 0.0f) { *out = 0; return true; }
    int e;
    float m = std::frexp(a, &e);      // a = m * 2^e, m in [0.5, 1)
    // normal binary16: a = (1 + f/1024) * 2^E, E in [-14, 15]
    int E = e - 1;
    if (E > 15) return false;
    if (E >= -14) {
        float frac = (m * 2.0f - 1.0f) * 1024.0f;
        if (frac != std::floor(frac)) return false;
        *out = (uint16_t)(((E + 15) << 10) | (int)frac);
        return true;
    }
    // subnormal: a = f * 2^-24, f in [1, 1023]
    float f = std::ldexp(a, 24);
    if (f != std::floor(f) || f < 1.0f || f > 1023.0f) return false;
    *out = (uint16_t)f;
    return true;
}

}  // namespace

namespace tern {

void set_error(const std::string &msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

}  // namespace tern

using tern::set_error;

extern "C" {

int tern_abi_version(void) { return TERN_ABI_VERSION; }

const char *tern_status_str(int status)
{
    switch (status) {
    case TERN_OK: return "TERN_OK";
    case TERN_EINVAL: return "TERN_EINVAL";
    case TERN_ENOTTERNARY: return "TERN_ENOTTERNARY";
    case TERN_EBADCODE: return "TERN_EBADCODE";
    case TERN_EUNSUPPORTED: return "TERN_EUNSUPPORTED";
    case TERN_EDEVICE: return "TERN_EDEVICE";
    default: return "unknown";
    }
}

const char *tern_last_error(void) { return g_last_error.c_str(); }

size_t tern_codes_bytes(int64_t N, int64_t K)
{
    if (!sizes_ok(N, K)) return 0;
    return (size_t)N * (size_t)(K / kSlots) * 4u;
}

size_t tern_scales_bytes(int64_t N, int64_t K)
{
    if (!sizes_ok(N, K)) return 0;
    return (size_t)N * (size_t)(K / kGroup) * 2u;
}

tern_status tern_pack(const int8_t *t, const uint16_t *s_f16, int64_t N, int64_t K,
                      uint32_t *codes, uint16_t *s_out)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_pack: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!t || !s_f16 || !codes || !s_out) {
        set_error("tern_pack: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = K / kGroup, W = K / kSlots;
    for (int64_t i = 0; i < N * G; ++i)
        if (!half_finite(s_f16[i])) {
            set_error("tern_pack: non-finite scale at index " + std::to_string(i));
            return TERN_EINVAL;
        }
    std::vector<char> bad_rows(N, 0);
    for_rows(N, K, [&](int64_t a, int64_t b) {
        for (int64_t n = a; n < b; ++n) {
            const int8_t *tr = t + n * K;
            uint32_t *cr = codes + n * W;
            for (int64_t w = 0; w < W; ++w) {
                uint32_t word = 0;
                for (int j = 0; j < kSlots; ++j) {
                    int v = tr[w * kSlots + j];
                    if (v < -1 || v > 1) { bad_rows[n] = 1; v = 0; }
                    word |= (uint32_t)(v + 1) << (2 * j);
                }
                cr[w] = word;
            }
        }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad_rows[n]) {
            set_error("tern_pack: value outside {-1,0,1} in row " + std::to_string(n));
            return TERN_ENOTTERNARY;
        }
    if (s_out != s_f16) std::memmove(s_out, s_f16, (size_t)(N * G) * 2u);
    return TERN_OK;
}

tern_status tern_pack_f32(const float *w, int64_t N, int64_t K, uint32_t *codes, uint16_t *s_out)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_pack_f32: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!w || !codes || !s_out) {
        set_error("tern_pack_f32: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = K / kGroup, W = K / kSlots;
    std::vector<int64_t> bad(N, -1);
    for_rows(N, K, [&](int64_t a, int64_t b) {
        for (int64_t n = a; n < b; ++n) {
            const float *wr = w + n * K;
            for (int64_t g = 0; g < G && bad[n] < 0; ++g) {
                float mag = 0.0f;
                bool ok = true;
                for (int64_t k = g * kGroup; k < (g + 1) * kGroup; ++k) {
                    float v = std::fabs(wr[k]);
                    if (v == 0.0f) continue;
                    if (!std::isfinite(v) || (mag != 0.0f && v != mag)) { ok = false; break; }
                    mag = v;
                }
                uint16_t h = 0;
                if (!ok || !float_to_half_exact(mag, &h)) { bad[n] = g; break; }
                s_out[n * G + g] = h;
                for (int64_t wi = g * (kGroup / kSlots); wi < (g + 1) * (kGroup / kSlots); ++wi) {
                    uint32_t word = 0;
                    for (int j = 0; j < kSlots; ++j) {
                        float v = wr[wi * kSlots + j];
                        int tv = (v > 0.0f) - (v < 0.0f);
                        word |= (uint32_t)(tv + 1) << (2 * j);
                    }
                    codes[n * W + wi] = word;
                }
            }
        }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n] >= 0) {
            set_error("tern_pack_f32: row " + std::to_string(n) + " group " + std::to_string(bad[n]) +
                      " is not s * {-1,0,1} with a binary16-exact s");
            return TERN_ENOTTERNARY;
        }
    return TERN_OK;
}

tern_status tern_unpack(const uint32_t *codes, int64_t N, int64_t K, int8_t *t)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_unpack: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!codes || !t) {
        set_error("tern_unpack: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / kSlots;
    std::vector<char> bad(N, 0);
    for_rows(N, K, [&](int64_t a, int64_t b) {
        for (int64_t n = a; n < b; ++n)
            for (int64_t w = 0; w < W; ++w) {
                uint32_t word = codes[n * W + w];
                for (int j = 0; j < kSlots; ++j) {
                    int q = (word >> (2 * j)) & 3;
                    if (q == 3) bad[n] = 1;
                    t[n * K + w * kSlots + j] = (int8_t)(q - 1);
                }
            }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n]) {
            set_error("tern_unpack: slot value 3 in row " + std::to_string(n));
            return TERN_EBADCODE;
        }
    return TERN_OK;
}

tern_status tern_dequant_f32(const uint32_t *codes, const uint16_t *s_f16, int64_t N, int64_t K,
                             float *w)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_dequant_f32: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!codes || !s_f16 || !w) {
        set_error("tern_dequant_f32: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / kSlots, G = K / kGroup;
    std::vector<char> bad(N, 0);
    for_rows(N, K, [&](int64_t a, int64_t b) {
        for (int64_t n = a; n < b; ++n)
            for (int64_t w_i = 0; w_i < W; ++w_i) {
                uint32_t word = codes[n * W + w_i];
                float s = half_bits_to_float(s_f16[n * G + (w_i * kSlots) / kGroup]);
                for (int j = 0; j < kSlots; ++j) {
                    int q = (word >> (2 * j)) & 3;
                    if (q == 3) bad[n] = 1;
                    w[n * K + w_i * kSlots + j] = s * (float)(q - 1);
                }
            }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n]) {
            set_error("tern_dequant_f32: slot value 3 in row " + std::to_string(n));
            return TERN_EBADCODE;
        }
    return TERN_OK;
}


// ---------------------------------------------------------------------------
// Format variants ("prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card,
// sections "Shipped components", "MLX packaging", and the 1-bit row of the
// variant table under "Benchmarks").
// ---------------------------------------------------------------------------

size_t tern_scales_g64_bytes(int64_t N, int64_t K)
{
    if (!sizes_ok(N, K)) return 0;
    return (size_t)N * (size_t)(K / 64) * 2u;
}

size_t tern_b1_bytes(int64_t N, int64_t K)
{
    if (!sizes_ok(N, K)) return 0;
    return (size_t)N * (size_t)(K / 32) * 4u;
}

tern_status tern_scales_to_g64(const uint16_t *s, int64_t N, int64_t K, uint16_t *s64)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_scales_to_g64: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!s || !s64) {
        set_error("tern_scales_to_g64: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    // back to front, so that s64 may start at s (in-place widening)
    for (int64_t i = G - 1; i >= 0; --i) {
        const uint16_t h = s[i];
        s64[2 * i + 1] = h;
        s64[2 * i] = h;
    }
    return TERN_OK;
}

tern_status tern_scales_from_g64(const uint16_t *s64, int64_t N, int64_t K, uint16_t *s)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_scales_from_g64: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!s64 || !s) {
        set_error("tern_scales_from_g64: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    for (int64_t i = 0; i < G; ++i) {
        const uint16_t a = s64[2 * i], b = s64[2 * i + 1];
        if (!half_finite(a) || !half_finite(b)) {
            set_error("tern_scales_from_g64: non-finite scale in group " + std::to_string(i));
            return TERN_EINVAL;
        }
        if (half_bits_to_float(a) != half_bits_to_float(b)) {
            set_error("tern_scales_from_g64: the two 64-blocks of group " + std::to_string(i) +
                      " have different scales");
            return TERN_ENOTTERNARY;
        }
    }
    for (int64_t i = 0; i < G; ++i) s[i] = s64[2 * i];  // forward: s may start at s64
    return TERN_OK;
}

tern_status tern_mlx_export(const uint16_t *s, int64_t N, int64_t K, uint16_t *mlx_scales,
                            uint16_t *mlx_biases)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_mlx_export: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!s || !mlx_scales || !mlx_biases) {
        set_error("tern_mlx_export: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    for (int64_t i = 0; i < G; ++i)
        if (!half_finite(s[i])) {
            set_error("tern_mlx_export: non-finite scale at index " + std::to_string(i));
            return TERN_EINVAL;
        }
    for (int64_t i = 0; i < G; ++i) {
        const uint16_t h = s[i];
        mlx_biases[i] = (uint16_t)(h ^ 0x8000u);  // -s: a sign flip, exact
        mlx_scales[i] = h;
    }
    return TERN_OK;
}

tern_status tern_mlx_import(const uint16_t *mlx_scales, const uint16_t *mlx_biases, int64_t N, int64_t K,
                            uint16_t *s)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_mlx_import: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!mlx_scales || !mlx_biases || !s) {
        set_error("tern_mlx_import: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    for (int64_t i = 0; i < G; ++i) {
        const uint16_t a = mlx_scales[i], b = mlx_biases[i];
        if (!half_finite(a) || !half_finite(b)) {
            set_error("tern_mlx_import: non-finite scale or bias in group " + std::to_string(i));
            return TERN_EINVAL;
        }
        if (half_bits_to_float(b) != -half_bits_to_float(a)) {
            set_error("tern_mlx_import: group " + std::to_string(i) +
                      " has bias != -scale (not a ternary group on slots q = t + 1)");
            return TERN_ENOTTERNARY;
        }
    }
    if (s != mlx_scales) std::memmove(s, mlx_scales, (size_t)G * 2u);
    return TERN_OK;
}

tern_status tern_pack_b1(const int8_t *b, int64_t N, int64_t K, uint32_t *bits)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_pack_b1: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!b || !bits) {
        set_error("tern_pack_b1: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / 32;
    std::vector<char> bad(N, 0);
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1; ++n)
            for (int64_t w = 0; w < W; ++w) {
                uint32_t word = 0;
                for (int j = 0; j < 32; ++j) {
                    const int v = b[n * K + 32 * w + j];
                    if (v != 1 && v != -1) bad[n] = 1;
                    word |= (uint32_t)(v == 1) << j;
                }
                bits[n * W + w] = word;
            }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n]) {
            set_error("tern_pack_b1: value other than -1 or +1 in row " + std::to_string(n));
            return TERN_ENOTTERNARY;
        }
    return TERN_OK;
}

tern_status tern_unpack_b1(const uint32_t *bits, int64_t N, int64_t K, int8_t *b)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_unpack_b1: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!bits || !b) {
        set_error("tern_unpack_b1: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / 32;
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t i = r0 * W; i < r1 * W; ++i)
            for (int j = 0; j < 32; ++j) b[32 * i + j] = ((bits[i] >> j) & 1u) ? (int8_t)1 : (int8_t)-1;
    });
    return TERN_OK;
}

namespace {
// Bits 0..15 of v moved to the even positions 0, 2, ..., 30.
uint32_t spread_even(uint32_t v)
{
    v &= 0xffffu;
    v = (v | (v << 8)) & 0x00ff00ffu;
    v = (v | (v << 4)) & 0x0f0f0f0fu;
    v = (v | (v << 2)) & 0x33333333u;
    v = (v | (v << 1)) & 0x55555555u;
    return v;
}
}  // namespace

tern_status tern_b1_to_codes(const uint32_t *bits, int64_t N, int64_t K, uint32_t *codes)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_b1_to_codes: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!bits || !codes) {
        set_error("tern_b1_to_codes: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / 32;
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t i = r0 * W; i < r1 * W; ++i) {
            // bit 1 (+1) -> slot 2, bit 0 (-1) -> slot 0: q = 2 * bit
            codes[2 * i] = spread_even(bits[i]) << 1;
            codes[2 * i + 1] = spread_even(bits[i] >> 16) << 1;
        }
    });
    return TERN_OK;
}

tern_status tern_codes_to_b1(const uint32_t *codes, int64_t N, int64_t K, uint32_t *bits)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_codes_to_b1: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!codes || !bits) {
        set_error("tern_codes_to_b1: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t W = K / 32;
    std::vector<char> bad(N, 0);  // 1: a zero weight, 2: slot value 3
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1; ++n)
            for (int64_t w = 0; w < W; ++w) {
                uint32_t word = 0;
                for (int j = 0; j < 32; ++j) {
                    const uint32_t c = codes[n * 2 * W + 2 * w + (j >> 4)];
                    const uint32_t q = (c >> (2 * (j & 15))) & 3u;
                    if (q == 3) bad[n] = 2;
                    else if (q == 1 && !bad[n]) bad[n] = 1;
                    word |= (uint32_t)(q == 2) << j;
                }
                bits[n * W + w] = word;
            }
    });
    for (int64_t n = 0; n < N; ++n) {
        if (bad[n] == 2) {
            set_error("tern_codes_to_b1: slot value 3 in row " + std::to_string(n));
            return TERN_EBADCODE;
        }
        if (bad[n] == 1) {
            set_error("tern_codes_to_b1: zero weight (no binary code) in row " + std::to_string(n));
            return TERN_ENOTTERNARY;
        }
    }
    return TERN_OK;
}

tern_status tern_mlx_export_b1(const uint16_t *s, int64_t N, int64_t K, uint16_t *mlx_scales,
                               uint16_t *mlx_biases)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_mlx_export_b1: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!s || !mlx_scales || !mlx_biases) {
        set_error("tern_mlx_export_b1: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    for (int64_t i = 0; i < G; ++i) {
        const uint32_t e = (s[i] >> 10) & 0x1fu;
        if (e >= 30) {  // non-finite, or 2s does not fit binary16
            set_error("tern_mlx_export_b1: scale at index " + std::to_string(i) +
                      (e == 31 ? " is not finite" : " overflows binary16 when doubled"));
            return TERN_EINVAL;
        }
    }
    for (int64_t i = 0; i < G; ++i) {
        const uint16_t h = s[i];
        const uint32_t sign = h & 0x8000u, mag = h & 0x7fffu;
        // 2s exactly: one more in the exponent for a normal number; for a
        // subnormal the fraction doubles (and may carry into the exponent)
        const uint32_t twice = ((mag >> 10) == 0) ? (mag << 1) : (mag + 0x400u);
        mlx_biases[i] = (uint16_t)(h ^ 0x8000u);
        mlx_scales[i] = (uint16_t)(sign | twice);
    }
    return TERN_OK;
}

tern_status tern_mlx_import_b1(const uint16_t *mlx_scales, const uint16_t *mlx_biases, int64_t N, int64_t K,
                               uint16_t *s)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_mlx_import_b1: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!mlx_scales || !mlx_biases || !s) {
        set_error("tern_mlx_import_b1: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = N * (K / kGroup);
    for (int64_t i = 0; i < G; ++i) {
        const uint16_t a = mlx_scales[i], b = mlx_biases[i];
        if (!half_finite(a) || !half_finite(b)) {
            set_error("tern_mlx_import_b1: non-finite scale or bias in group " + std::to_string(i));
            return TERN_EINVAL;
        }
        if (half_bits_to_float(a) != -2.0f * half_bits_to_float(b)) {
            set_error("tern_mlx_import_b1: group " + std::to_string(i) + " has scale != -2 * bias");
            return TERN_ENOTTERNARY;
        }
    }
    for (int64_t i = 0; i < G; ++i) s[i] = (uint16_t)(mlx_biases[i] ^ 0x8000u);
    return TERN_OK;
}

// ---------------------------------------------------------------------------
// Base-3 layout: five ternary values per byte (see tern.h)
// ---------------------------------------------------------------------------

size_t tern_t5_bytes(int64_t N, int64_t K)
{
    if (!sizes_ok(N, K)) return 0;
    return (size_t)N * (size_t)(((K / kGroup) + 4) / 5) * 128u;
}

tern_status tern_pack_t5(const uint32_t *codes, int64_t N, int64_t K, uint8_t *data)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_pack_t5: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!codes || !data) {
        set_error("tern_pack_t5: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = K / kGroup, SB = (G + 4) / 5, W = K / kSlots;
    std::vector<char> bad(N, 0);
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1; ++n)
            for (int64_t b = 0; b < SB; ++b) {
                const int64_t p = std::min<int64_t>(5, G - 5 * b);
                for (int i = 0; i < 128; ++i) {
                    unsigned v = 0, w3 = 1;
                    for (int64_t j = 0; j < p; ++j, w3 *= 3) {
                        const int64_t k = 128 * (5 * b + j) + i;
                        const unsigned q = (codes[n * W + k / kSlots] >> (2 * (k % kSlots))) & 3u;
                        if (q == 3) bad[n] = 1;
                        v += (q == 3 ? 0u : q) * w3;
                    }
                    data[(n * SB + b) * 128 + i] = (uint8_t)v;
                }
            }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n]) {
            set_error("tern_pack_t5: slot value 3 in row " + std::to_string(n));
            return TERN_EBADCODE;
        }
    return TERN_OK;
}

tern_status tern_unpack_t5(const uint8_t *data, int64_t N, int64_t K, uint32_t *codes)
{
    if (!sizes_ok(N, K)) {
        set_error("tern_unpack_t5: need N >= 0, K >= 0 and K % 128 == 0");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!data || !codes) {
        set_error("tern_unpack_t5: NULL pointer");
        return TERN_EINVAL;
    }
    const int64_t G = K / kGroup, SB = (G + 4) / 5, W = K / kSlots;
    std::vector<char> bad(N, 0);
    for_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1; ++n) {
            for (int64_t w = 0; w < W; ++w) codes[n * W + w] = 0;
            for (int64_t b = 0; b < SB; ++b) {
                const int64_t p = std::min<int64_t>(5, G - 5 * b);
                unsigned lim = 1;
                for (int64_t j = 0; j < p; ++j) lim *= 3;
                for (int i = 0; i < 128; ++i) {
                    unsigned v = data[(n * SB + b) * 128 + i];
                    if (v >= lim) { bad[n] = 1; v = 0; }
                    for (int64_t j = 0; j < p; ++j, v /= 3) {
                        const int64_t k = 128 * (5 * b + j) + i;
                        codes[n * W + k / kSlots] |= (v % 3) << (2 * (k % kSlots));
                    }
                }
            }
        }
    });
    for (int64_t n = 0; n < N; ++n)
        if (bad[n]) {
            set_error("tern_unpack_t5: byte outside the range of its superblock in row " + std::to_string(n));
            return TERN_EBADCODE;
        }
    return TERN_OK;
}

}  // extern "C"
