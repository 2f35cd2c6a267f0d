// The 4096-point signed Walsh-Hadamard transform on the matrix cores, shared
// by the libtern kernel sources.  Included inside an anonymous namespace,
// after tern_device.h.
#pragma once

// One 16-column slice of a 4096-point transform on the matrix cores.  A
// block viewed as a 64 x 64 matrix X[i][j] = x[64 i + j] transforms as
// H64 X H64 (the Sylvester matrix of 4096 points is the Kronecker square of
// the 64-point one).  The wave computes
//   Z  = X H64[:, 16 jt + 0..15]   (A = rows of X, B = H64)
//   X' = H64 Z                     (A = H64, B = Z as three bfloat16 parts)
// with v_mfma_f32_16x16x32_bf16 and binary32 accumulation.  The contraction
// order of the second product is the order in which the first leaves Z in
// the lanes (k-slot e of lane group g at step st is row 32 st + 16 (e >> 2)
// + 4 g + (e & 3)), so Z never leaves the registers.  +-1 is exact in
// bfloat16, and hi + mid + lo carry all 24 significand bits of Z.
// xs: row i of X at element i * (64 + pad) (bfloat16 pairs, or binary32 when
// IN_F32, which is split into two exact bfloat16 parts for the first
// product); lane (c = lane & 15, g = lane >> 4); out[ot][r] =
// X'[16 ot + 4 g + r][16 jt + c], not normalized.
template <bool IN_F32>
__device__ __forceinline__ void h64_slice(const void *xs, int jt, int c, int g, f32x4_t (&out)[4])
{
    constexpr int kPadX = IN_F32 ? 68 : 72;  // elements per staged row (conflict-free 16-byte reads)
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    auto pm1 = [](uint32_t lo_neg, uint32_t hi_neg) -> uint32_t {
        return 0x3F803F80u | ((lo_neg & 1u) << 15) | ((hi_neg & 1u) << 31);
    };
    // H64 as the A operand of the second product: row 16 ot + c, k-slot e as
    // above.  (-1)^popcount of (c & e & 3), ((c >> 2) & g), (ot & 1 & e >> 2)
    // and (ot >> 1 & st).
    const uint32_t pl = __builtin_popcount((c >> 2) & g) & 1;
    const uint32_t q1 = c & 1, q2 = (c >> 1) & 1, q3 = __builtin_popcount(c & 3) & 1;
    const uint32_t hbase0 = pm1(pl, q1 ^ pl), hbase1 = pm1(q2 ^ pl, q3 ^ pl);
    // H64 as the B operand of the first product: column 16 jt + c, k-slot e
    // -> row 32 ks + 8 g + e.  (-1)^popcount of (e & c & 7), ((g & 1) &
    // (c >> 3)), ((g >> 1) & jt & 1) and (ks & jt >> 1).
    const uint32_t pb = (g & 1) & (c >> 3);
    bf16x8_t hb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint32_t f = ((((g >> 1) & jt) ^ (ks & (jt >> 1))) & 1) ? 0x80008000u : 0u;
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = pm1((__builtin_popcount((2 * q) & c & 7) & 1) ^ pb,
                       (__builtin_popcount((2 * q + 1) & c & 7) & 1) ^ pb) ^ f;
        hb[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    // Z; lane holds Z[16 it + 4 g + r][16 jt + c].  A operand: X[16 it + c][32 ks + 8 g + 0..7]
    f32x4_t z[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        z[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int at = (16 * it + c) * kPadX + 32 * ks + 8 * g;
            if constexpr (!IN_F32) {
                const u32x4_t xa = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(xs) + at);
                z[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa), hb[ks], z[it], 0, 0, 0);
            } else {
                const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint32_t *>(xs) + at);
                const u32x4_t w0 = src[0], w1 = src[1];
                u32x4_t xh, xl;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f0 = __builtin_bit_cast(float, v < 2 ? w0[2 * v] : w1[2 * v - 4]);
                    const float f1 = __builtin_bit_cast(float, v < 2 ? w0[2 * v + 1] : w1[2 * v - 3]);
                    const bf16x2_t ph = {(__bf16)f0, (__bf16)f1};
                    const bf16x2_t plo = {(__bf16)(f0 - (float)ph[0]), (__bf16)(f1 - (float)ph[1])};
                    xh[v] = __builtin_bit_cast(uint32_t, ph);
                    xl[v] = __builtin_bit_cast(uint32_t, plo);
                }
                z[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xh), hb[ks], z[it], 0, 0, 0);
                z[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xl), hb[ks], z[it], 0, 0, 0);
            }
        }
    }
    // Z as three bfloat16 parts, in the k-slot order of the second product:
    // slots 2v, 2v + 1 of step st are tile 2 st + (v >> 1), rows 2 (v & 1), + 1
    u32x4_t zp[3][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float f0 = z[2 * st + (v >> 1)][2 * (v & 1)];
            float f1 = z[2 * st + (v >> 1)][2 * (v & 1) + 1];
#pragma unroll
            for (int pt = 0; pt < 3; ++pt) {
                const bf16x2_t b = {(__bf16)f0, (__bf16)f1};
                zp[pt][st][v] = __builtin_bit_cast(uint32_t, b);
                f0 -= (float)b[0];
                f1 -= (float)b[1];
            }
        }
    // X' = H64 Z
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
        out[ot] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const uint32_t fa = ((ot >> 1) & st) ? 0x80008000u : 0u;  // every slot
            const uint32_t fb = fa ^ ((ot & 1) ? 0x80008000u : 0u);   // slots e >= 4
            const bf16x8_t ha = __builtin_bit_cast(bf16x8_t, u32x4_t{hbase0 ^ fa, hbase1 ^ fa, hbase0 ^ fb, hbase1 ^ fb});
#pragma unroll
            for (int pt = 0; pt < 3; ++pt)
                out[ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha, __builtin_bit_cast(bf16x8_t, zp[pt][st]), out[ot], 0, 0, 0);
        }
    }
}
