// Decode GEMV (M <= 4) on the gfx950 fp8 x fp4 matrix cores.
//
// y[m][n] = sum_g s[n][g] sum_{k in g} t[n][k] x[m][k] ("prism-ml/Ternary-
// Bonsai-27B-mlx-2bit" model card, "Weight representation: ternary g128" and
// "CUDA (NVIDIA GPUs)": the 2-bit codes are unpacked and scaled inside the
// matmul), optionally on the rotated activations x' = H (d .* x) / 64 over
// blocks of 4096 ("Ternary-Bonsai-2-9B-2bit" article, section 3).
//
// Weight operands.  XOR with 0x55555555 turns slot q = t + 1 into the bit
// pair ([t = +1], [t != 0]); in the top two bits of a 4-bit e2m1 field that
// pair is the fp4 code of -2t (0b1100 = -2, 0b0100 = +2, 0 = 0).  The odd
// slots of a code word already sit at bits 4i + 2 .. 4i + 3, so
//   odd  = (w & 0xCCCCCCCC) ^ 0x44444444
//   even = ((w << 2) & 0xCCCCCCCC) ^ 0x44444444
// are the fp4 operands of the word's 16 weights (one v_bitop3 each, plus a
// shift): three VALU operations per 16 weights, exact.
//
// Activation operands.  Each activation is carried as e4m3 parts,
// x = sum_p 2^(e - 4p) c_p with c_p in e4m3, where 2^e is chosen per 32
// consecutive activations (the two code words of one B lane group, which is
// what one E8M0 scale of the instruction covers) from their largest
// magnitude and applied by that scale.  c_0 is the round-to-nearest of
// x 2^-e (in [128, 256) for the largest), and each further part rounds 16
// times the remainder, which is exact in binary32.  Parts are added until
// every remainder of the 32 is at most 2^-16 times the smallest nonzero
// magnitude among them (bfloat16 input usually stops at two or three parts,
// when the remainders are exactly zero; binary32 at about four), at most
// eight: then |x - sum| <= 2^-16 |x| for every activation, unless a block
// of 32 spans more than about 2^29 in magnitude.  Part p of x row m is A row
// 8m + p, so the parts of a row meet in the accumulators of two lanes.
//
// Instruction layout (v_mfma_scale_f32_16x16x128_f8f6f4, measured on the
// device): B lane (n, g) nibble i holds k = 32 g + i; A lane (r, g) byte i
// holds k = 16 g + i for i < 16 and k = 64 + 16 g + i - 16 for i >= 16;
// D lane (n, g) holds rows 4 g .. 4 g + 3 of column n; the E8M0 scale that
// lane group g supplies covers the k of B lane group g.  With the code words
// regrouped so that lane group g holds words 2 P(g), 2 P(g) + 1 of a group
// (P = {0, 2, 1, 3}) and the fp4 registers ordered [even(w0), odd(w0),
// even(w1), odd(w1)], A lane group g, half h takes the 16 activations of
// word 2 P(2 h + (g >> 1)) + (g & 1), slots 0, 2, .., 14, 1, 3, .., 15.
//
// One 128-K group is one MFMA per 16-row tile and 16 A rows (two for three
// or four x rows); each lane adds its four part rows and multiplies by the
// group's binary16 scale in binary32, and the two lanes of an x row are
// added at the end.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

#include "tern_internal.h"

namespace {

#include "tern_device.h"
#include "tern_h64.h"

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kParts = 8;            // e4m3 parts per activation at most (A rows per x row)
constexpr int kF4MaxM = 4;           // x rows per launch (two 16-row A tiles)
constexpr unsigned kF4Mask = 0xCCCCCCCCu, kF4Flip = 0x44444444u;
constexpr int kE8M0One = 127;        // E8M0 encoding of 2^0

struct F4Args {
    const void *x;           // [M][K] bfloat16 or binary32
    const int8_t *signs;     // rotated input: d[K] (sign bits read) or NULL
    const uint32_t *codes;   // [N][K/16]
    const uint16_t *scales;  // [N][K/128] binary16
    void *y;                 // [M][N]
    int64_t N;
    int K, M, G;             // G = K / 128
    int nblk;                // 256-K blocks (the last may hold one group)
    int wk;                  // K-waves of a workgroup
    int bq, br;              // blocks per K-wave: bq, plus one for the first br
    int y_bf16;
    float norm;              // rotated input: 1/64
};

// P = {0, 2, 1, 3}: B lane group gs holds words 2 P(gs), 2 P(gs) + 1 of a group.
__device__ __forceinline__ int f4_perm(int gs) { return (gs == 1) ? 2 : (gs == 2) ? 1 : gs; }

// fp4 operand registers of two code words (16 weights each).
__device__ __forceinline__ i32x8_t f4_weights(unsigned w0, unsigned w1)
{
    i32x8_t b;
    b[0] = (int)(((w0 << 2) & kF4Mask) ^ kF4Flip);
    b[1] = (int)((w0 & kF4Mask) ^ kF4Flip);
    b[2] = (int)(((w1 << 2) & kF4Mask) ^ kF4Flip);
    b[3] = (int)((w1 & kF4Mask) ^ kF4Flip);
    b[4] = b[5] = b[6] = b[7] = 0;
    return b;
}

// One e4m3 part of 16 scaled activations t (slot order): the 16 bytes in
// operand order (slots 0, 2, .., 14, 1, 3, .., 15), and t replaced by the
// exact remainder t - part.
__device__ __forceinline__ u32x4_t f4_part(float (&t)[16])
{
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        // dword d holds slots 2 (4 (d & 1) + i) + (d >> 1), i = 0..3
        const int s0 = 8 * (d & 1) + (d >> 1);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[s0], t[s0 + 2], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(t[s0 + 4], t[s0 + 6], w, true);
        o[d] = (unsigned)w;
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        t[s0] -= lo[0];
        t[s0 + 2] -= lo[1];
        t[s0 + 4] -= hi[0];
        t[s0 + 6] -= hi[1];
    }
    return o;
}

// LDS image of the activation operands: group G, half h, lane group ga, A row
// r (of RA = 4 M) at byte ((((G * 2 + h) * 4 + ga) * RA + r) * 16); E8M0
// scales: one dword per (256-K block, lane group, A row), byte j = group
// 2 blk + j.
struct F4Lds {
    unsigned char *aimg;
    uint32_t *simg;
    float *red;
    float *ximg;        // rotated input: binary32 x' rows, padded
    unsigned char *xs;  // rotated input: d .* x staging for the transform
};

// Padded index of activation k in a row of the rotated binary32 image:
// 16 floats of padding per 256 keep the transform's four lane groups on
// distinct banks.
__device__ __forceinline__ int f4_xpad(int k) { return k + 16 * (k >> 8); }

template <int TPW, bool XF32, bool ROT, bool SC4, int AT>
__global__ __launch_bounds__(256) void gemv_f4_kernel(const F4Args a)
{
    constexpr int PF = 4;     // ring slots (blocks)
    constexpr int kDist = 2;  // blocks of codes in flight
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int nthreads = 64 * waves;
    const int kw = wave;  // every wave splits K
    const int nn = lane & 15, g = lane >> 4;
    const int RA = kParts * a.M;  // A rows (AT tiles of 16, the last one partly used)
    const int G = a.G;

    const int b_begin = kw * a.bq + (kw < a.br ? kw : a.br);
    const int nblocks = a.bq + (kw < a.br ? 1 : 0);
    const int g_begin = 2 * b_begin;
    const int g_end = (g_begin + 2 * nblocks < G) ? g_begin + 2 * nblocks : G;

    const int rows_per_wg = kTileN * TPW;
    const int64_t n0 = (int64_t)blockIdx.x * rows_per_wg;

    // LDS carve-up (16-byte aligned pieces)
    F4Lds L;
    size_t off = 0;
    L.aimg = smem + off;
    off += (size_t)RA * a.K;
    L.simg = reinterpret_cast<uint32_t *>(smem + off);
    off += (size_t)a.nblk * 4 * RA * 4;
    L.red = reinterpret_cast<float *>(smem + off);
    off += (size_t)waves * TPW * AT * 4 * kTileN * 4;
    L.ximg = reinterpret_cast<float *>(smem + off);
    const int xrow = a.K + 16 * (a.K >> 8);  // padded binary32 row of x'
    off += ROT ? (size_t)a.M * xrow * 4 : 0;
    L.xs = smem + off;

    // 1. rotated input: d .* x for the transform, loads first
    const int wpr = a.K >> 4;  // 16-activation words per row
    const int8_t *sign_src = a.signs;
    constexpr int kPadX = XF32 ? 68 : 72;
    const int xs_row = (a.K >> 6) * kPadX;
    const int rot_units = ROT ? a.M * wpr : 0;
    // every thread stages at most a few words; the loads leave before the
    // code stream is issued
    constexpr int kRU = 2;  // staging words per thread per round (rotated)
    u32x4_t xv[kRU][XF32 ? 4 : 2];
    u32x4_t dv[kRU];
    auto load_rot = [&](int i, int u) {
        const int m = u / wpr, wi = u % wpr;
        if constexpr (XF32) {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(a.x) +
                                                                   (int64_t)m * a.K + 16 * wi);
#pragma unroll
            for (int q = 0; q < 4; ++q) xv[i][q] = src[q];
        } else {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) +
                                                                   (int64_t)m * a.K + 16 * wi);
#pragma unroll
            for (int q = 0; q < 2; ++q) xv[i][q] = src[q];
        }
        dv[i] = sign_src ? *reinterpret_cast<const u32x4_t *>(sign_src + 16 * wi)
                         : u32x4_t{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
    };
    if constexpr (ROT) {
#pragma unroll
        for (int i = 0; i < kRU; ++i) {
            int u = threadIdx.x + i * nthreads;
            u = u < rot_units ? u : rot_units - 1;
            load_rot(i, u);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. code stream: kDist blocks ahead, scale pairs with them
    const uint32_t *crow[TPW];
    const uint16_t *srow[TPW];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
        int64_t r = n0 + tp * kTileN + nn;
        if (r > a.N - 1) r = a.N - 1;  // rows past N load a valid row; results are dropped
        crow[tp] = a.codes + r * (a.K / 16);
        srow[tp] = a.scales + r * G;
    }
    u32x4_t cbuf[PF][TPW];
    uint32_t sbuf[PF][TPW];
    auto load_block = [&](int b, int p) {
        b = b < nblocks ? b : nblocks - 1;
        const int gb = g_begin + 2 * b;
        const bool two = (gb + 1) < g_end;
        const int lg = two ? g : (g & 1);
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            cbuf[p][tp] = *reinterpret_cast<const u32x4_t *>(crow[tp] + gb * kWordsPerGroup + 4 * lg);
            if constexpr (SC4)
                sbuf[p][tp] = *reinterpret_cast<const uint32_t *>(srow[tp] + gb);
            else
                sbuf[p][tp] = (uint32_t)srow[tp][gb] | ((uint32_t)srow[tp][two ? gb + 1 : gb] << 16);
        }
    };
#pragma unroll
    for (int p = 0; p < kDist; ++p) load_block(p, p);
    __builtin_amdgcn_sched_barrier(0);

    // 3. activations -> LDS operand image
    // One unit = (row m, group G, scale block gs, word j): the 16 activations
    // of word 2 P(gs) + j, which A lane group 2 (gs & 1) + j carries in half
    // gs >> 1.  Units u, u ^ 1 are the two words of one scale block; they
    // exchange their largest magnitudes so both use the same exponent.
    const int units = a.M * G * 8;
    int parts_used = 0;  // largest part count of this thread's units (wave-uniform)
    auto stage_unit = [&](int u, const float (&v)[16]) {
        const int j = u & 1, gs = (u >> 1) & 3, q = u >> 3;
        const int Gi = q % G, m = q / G;
        const int ga = 2 * (gs & 1) + j, h = gs >> 1;
        float amax = 0.0f, amin = __builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float av = __builtin_fabsf(v[e]);
            amax = __builtin_fmaxf(amax, av);
            amin = av > 0.0f ? __builtin_fminf(amin, av) : amin;
        }
        // partner lane (lane ^ 1) holds the other word of the scale block
        amax = __builtin_fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                                    __builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false)));
        amin = __builtin_fminf(amin, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                                   __builtin_bit_cast(int, amin), 0xB1, 0xF, 0xF, false)));
        // 2^e0 puts the largest magnitude in [128, 256); parts step by 2^4
        const int e0 = (int)(__builtin_bit_cast(uint32_t, amax) >> 23) - 127 - 7;
        int sp = e0 < -127 ? -127 : e0;  // exponent of the current part's scale
        float t[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = __builtin_ldexpf(v[e], -sp);
        // remainders must end at most 2^-16 of the smallest nonzero magnitude
        float thr = __builtin_ldexpf(amin, -sp - 16);
        unsigned char *dst = L.aimg + ((((size_t)Gi * 2 + h) * 4 + ga) * RA + kParts * m) * 16;
        unsigned char *sd = reinterpret_cast<unsigned char *>(L.simg) +
                            (((size_t)(Gi >> 1) * 4 + gs) * RA + kParts * m) * 4 + (Gi & 1);
        int np = 0;
        for (int p = 0; p < kParts; ++p) {
            *reinterpret_cast<u32x4_t *>(dst + 16 * p) = f4_part(t);
            if (j == 0) sd[4 * p] = (unsigned char)(kE8M0One + sp);  // read by lane group gs
            np = p + 1;
            float rmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) rmax = __builtin_fmaxf(rmax, __builtin_fabsf(t[e]));
            const bool done = rmax <= thr;
            if (__builtin_amdgcn_ballot_w64(!done) == 0) break;  // every block of the wave is done
            const int next = sp - 4 < -127 ? -127 : sp - 4;
#pragma unroll
            for (int e = 0; e < 16; ++e) t[e] = __builtin_ldexpf(t[e], sp - next);
            thr = __builtin_ldexpf(thr, sp - next);
            sp = next;
        }
        // rows of parts not produced: zero data, unit scale
        for (int p = np; p < kParts; ++p) {
            *reinterpret_cast<u32x4_t *>(dst + 16 * p) = u32x4_t{0u, 0u, 0u, 0u};
            if (j == 0) sd[4 * p] = (unsigned char)kE8M0One;
        }
        parts_used = np > parts_used ? np : parts_used;
    };
    // a unit's 16 activations: from global memory (plain input) or from the
    // rotated binary32 image in LDS
    auto unit_values = [&](int u, float (&v)[16]) {
        const int j = u & 1, gs = (u >> 1) & 3, q = u >> 3;
        const int Gi = q % G, m = q / G;
        const int k0 = 128 * Gi + 32 * f4_perm(gs) + 16 * j;
        if constexpr (ROT) {
            const float *src = L.ximg + (size_t)m * xrow + f4_xpad(k0);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const u32x4_t d = *reinterpret_cast<const u32x4_t *>(src + 4 * qd);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned de = d[e];
                    v[4 * qd + e] = __builtin_bit_cast(float, de);
                }
            }
        } else if constexpr (XF32) {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(a.x) +
                                                                   (int64_t)m * a.K + k0);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const u32x4_t d = src[qd];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned de = d[e];
                    v[4 * qd + e] = __builtin_bit_cast(float, de);
                }
            }
        } else {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) +
                                                                   (int64_t)m * a.K + k0);
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) {
                const u32x4_t d = src[qd];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned de = d[e];
                    v[8 * qd + 2 * e] = __builtin_bit_cast(float, de << 16);
                    v[8 * qd + 2 * e + 1] = __builtin_bit_cast(float, de & 0xffff0000u);
                }
            }
        }
    };

    if constexpr (ROT) {
        // d .* x into the transform's staging rows (sign bit flipped where the
        // sign byte is negative), then H64 X H64 per 4096-block on the matrix
        // cores, x' = result / 64 into the binary32 image
        auto put_rot = [&](int i, int u) {
            const int m = u / wpr, wi = u % wpr;
            const int k = 16 * wi;
            if constexpr (XF32) {
                u32x4_t q[4];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const unsigned xe = xv[i][e >> 2][e & 3];
                    const unsigned de = dv[i][e >> 2];
                    q[e >> 2][e & 3] = xe ^ (((de >> (8 * (e & 3) + 7)) & 1u) << 31);
                }
                u32x4_t *dst = reinterpret_cast<u32x4_t *>(reinterpret_cast<uint32_t *>(L.xs) +
                                                           (size_t)m * xs_row + (k >> 6) * kPadX + (k & 63));
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) dst[q4] = q[q4];
            } else {
                u32x4_t q[2];
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const uint32_t sel = (v & 1) ? 0x030C020Cu : 0x010C000Cu;  // sign bytes -> bytes 1, 3
                    const unsigned xe = xv[i][v >> 2][v & 3];
                    q[v >> 2][v & 3] = xe ^ (__builtin_amdgcn_perm(0u, dv[i][v >> 1], sel) & 0x80008000u);
                }
                u32x4_t *dst = reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(L.xs) +
                                                           (size_t)m * xs_row + (k >> 6) * kPadX + (k & 63));
                dst[0] = q[0];
                dst[1] = q[1];
            }
        };
#pragma unroll
        for (int i = 0; i < kRU; ++i) {
            int u = threadIdx.x + i * nthreads;
            u = u < rot_units ? u : rot_units - 1;
            put_rot(i, u);
        }
        for (int u0 = kRU * nthreads; u0 < rot_units; u0 += kRU * nthreads) {
#pragma unroll
            for (int i = 0; i < kRU; ++i) {
                int u = u0 + threadIdx.x + i * nthreads;
                u = u < rot_units ? u : rot_units - 1;
                load_rot(i, u);
            }
#pragma unroll
            for (int i = 0; i < kRU; ++i) {
                int u = u0 + threadIdx.x + i * nthreads;
                u = u < rot_units ? u : rot_units - 1;
                put_rot(i, u);
            }
        }
        __syncthreads();
        const int slices = a.M * (a.K >> 12) * 4;
        for (int su = wave; su < slices; su += waves) {
            const int m = su / ((a.K >> 12) * 4), rem = su % ((a.K >> 12) * 4), blk = rem >> 2, jt = rem & 3;
            const unsigned char *xsrc = L.xs + ((size_t)m * xs_row + (size_t)64 * blk * kPadX) * (XF32 ? 4 : 2);
            f32x4_t o[4];
            h64_slice<XF32>(xsrc, jt, nn, g, o);
            // lane holds X'[16 ot + 4 g + r][16 jt + nn]: activation
            // k = 4096 blk + 64 (16 ot + 4 g + r) + 16 jt + nn
            float *row = L.ximg + (size_t)m * xrow;
#pragma unroll
            for (int ot = 0; ot < 4; ++ot)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k = 4096 * blk + 64 * (16 * ot + 4 * g + r) + 16 * jt + nn;
                    row[f4_xpad(k)] = o[ot][r] * a.norm;
                }
        }
        __syncthreads();
    }
    // parts of every unit (units beyond the end repeat the last pair, so that
    // every lane has a partner in the same pair)
    for (int u0 = 0; u0 < units; u0 += nthreads) {
        int u = u0 + threadIdx.x;
        if (u >= units) u = units - 2 + (threadIdx.x & 1);
        float v[16];
        unit_values(u, v);
        stage_unit(u, v);
    }
    // the workgroup's largest part count: A rows of higher parts are zero
    // everywhere and are not read
    if (lane == 0) L.red[wave] = __builtin_bit_cast(float, parts_used);
    __syncthreads();
    int p_wg = 0;
    for (int w = 0; w < waves; ++w) {
        const int pw = __builtin_bit_cast(int, L.red[w]);
        p_wg = pw > p_wg ? pw : p_wg;
    }
    __syncthreads();  // L.red is reused by the final reduction

    // 4. stream the codes
    float yacc[TPW][AT];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int at = 0; at < AT; ++at) yacc[tp][at] = 0.0f;
    i32x8_t a0[AT], a1[AT];
    uint32_t sdw[AT];
    bool a_active[AT];
#pragma unroll
    for (int at = 0; at < AT; ++at) {
        a0[at] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        a1[at] = a0[at];
        sdw[at] = 0x7F7F7F7Fu;
        const int r = 16 * at + nn;  // A row: part (r & 7) of x row r >> 3
        a_active[at] = r < RA && (r & 7) < p_wg;
    }
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    auto process = [&](int b, int p, bool refill) {
        const int gl0 = g_begin + 2 * b;
        const bool two = gl0 + 1 < g_end;
        const int gl1 = two ? gl0 + 1 : gl0;
#pragma unroll
        for (int at = 0; at < AT; ++at) {
            if (a_active[at]) {
                const int r = 16 * at + nn;
                const unsigned char *s0 = L.aimg + (((size_t)gl0 * 8 + g) * RA + r) * 16;
                const unsigned char *s1 = L.aimg + (((size_t)gl1 * 8 + g) * RA + r) * 16;
                const size_t hstep = (size_t)4 * RA * 16;  // half 0 -> half 1
                const u32x4_t x00 = *reinterpret_cast<const u32x4_t *>(s0);
                const u32x4_t x01 = *reinterpret_cast<const u32x4_t *>(s0 + hstep);
                const u32x4_t x10 = *reinterpret_cast<const u32x4_t *>(s1);
                const u32x4_t x11 = *reinterpret_cast<const u32x4_t *>(s1 + hstep);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a0[at][e] = (int)x00[e];
                    a0[at][4 + e] = (int)x01[e];
                    a1[at][e] = (int)x10[e];
                    a1[at][4 + e] = (int)x11[e];
                }
                uint32_t sv = L.simg[((size_t)(gl0 >> 1) * 4 + g) * RA + r];
                // a one-group block reuses group gl0 (scaled by zero below);
                // its exponent byte stands in for the missing second one
                if (!two) sv = (sv & 0xffu) * 0x0101u;
                sdw[at] = sv;
            }
        }
        unsigned wq[TPW][4];
        float sc[TPW][2];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            auto s02 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][0], cbuf[p][tp][2], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][1], cbuf[p][tp][3], false, false);
            wq[tp][0] = s02[0];  // group 0, word 2 P(g)
            wq[tp][1] = s13[0];  // group 0, word 2 P(g) + 1
            wq[tp][2] = s02[1];  // group 1
            wq[tp][3] = s13[1];
            const uint32_t pair = sbuf[p][tp];
            sc[tp][0] = half_to_float((uint16_t)(pair & 0xffffu));
            sc[tp][1] = two ? half_to_float((uint16_t)(pair >> 16)) : 0.0f;
        }
        if (refill && b + kDist < nblocks) load_block(b + kDist, (p + kDist) % PF);
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const i32x8_t b0 = f4_weights(wq[tp][0], wq[tp][1]);
            const i32x8_t b1 = f4_weights(wq[tp][2], wq[tp][3]);
#pragma unroll
            for (int at = 0; at < AT; ++at) {
                const f32x4_t d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a0[at], b0, zero4, 0, 4, 0, (int)sdw[at], 0, kE8M0One);
                const f32x4_t d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a1[at], b1, zero4, 0, 4, 1, (int)sdw[at], 0, kE8M0One);
                // four parts of the lane group's x row (zero rows past M)
                const float t0 = (d0[0] + d0[1]) + (d0[2] + d0[3]);
                const float t1 = (d1[0] + d1[1]) + (d1[2] + d1[3]);
                yacc[tp][at] = __builtin_fmaf(sc[tp][0], t0, yacc[tp][at]);
                yacc[tp][at] = __builtin_fmaf(sc[tp][1], t1, yacc[tp][at]);
            }
        }
    };

    const int nfull = (nblocks / PF) * PF;
    for (int b0 = 0; b0 < nfull; b0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) process(b0 + p, p, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (nfull + p < nblocks) process(nfull + p, p, true);

    // 5. combine the K-waves' partial sums in a fixed order and store
    auto store = [&](int m, int64_t n, float sum) {
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    };
    // lane (n, g) of A tile at holds parts 4 (g & 1) .. + 3 of x row
    // 2 at + (g >> 1)
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int at = 0; at < AT; ++at) L.red[(((wave * TPW + tp) * AT + at) * 4 + g) * kTileN + nn] = yacc[tp][at];
    __syncthreads();
    const int outs = a.M * rows_per_wg;
    for (int o = threadIdx.x; o < outs; o += nthreads) {
        const int m = o / rows_per_wg, rem = o % rows_per_wg;
        const int tp = rem / kTileN, jn = rem % kTileN;
        const int64_t n = n0 + rem;
        if (n >= a.N) continue;
        const int at = m >> 1, g0 = 2 * (m & 1);
        float sum = 0.0f;
        for (int w = 0; w < waves; ++w) {
            const float *r = L.red + (((w * TPW + tp) * AT + at) * 4 + g0) * kTileN + jn;
            sum += r[0] + r[kTileN];
        }
        store(m, n, sum);
    }
}

// K = 0: zeros (an empty sum).
__global__ __launch_bounds__(256) void f4_zero_kernel(void *y, int64_t count, int y_bf16)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        if (y_bf16)
            static_cast<uint16_t *>(y)[i] = 0;
        else
            static_cast<float *>(y)[i] = 0.0f;
    }
}

struct F4Plan {
    int tpw, wk;
    int64_t wgs;
    size_t lds;
};

// LDS bytes of one workgroup.
// A tiles (16 A rows each) for M x rows of kParts parts.
inline int f4_tiles(int M) { return (kParts * M + 15) / 16; }

size_t f4_lds(int M, int64_t K, int nblk, int waves, int tpw, bool rot, bool xf32)
{
    const size_t ra = (size_t)kParts * M;
    size_t b = ra * K + (size_t)nblk * 4 * ra * 4 + (size_t)waves * tpw * f4_tiles(M) * 4 * kTileN * 4;
    if (rot) {
        b += (size_t)M * (K + 16 * (K >> 8)) * 4;
        b += (size_t)M * (K >> 6) * (xf32 ? 68 * 4 : 72 * 2);
    }
    return b;
}

// Work split: tiles per wave (tpw) and K-waves per workgroup (wk).  Every
// workgroup converts all of x once, so fewer, larger workgroups convert it
// less often; from sweeps of the decode shapes.
F4Plan plan_f4(int64_t N, int64_t K, int M, bool rot, bool xf32)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    const int cus = device_cus();
    F4Plan pl;
    int64_t t = (tiles + cus - 1) / cus;
    pl.tpw = (int)(t <= 1 ? 1 : t <= 2 ? 2 : t <= 3 ? 3 : 4);
    pl.wk = 1;
    while (pl.wk < 4 && nblk >= 2 * (pl.wk * 2)) pl.wk *= 2;
    pl.wgs = (tiles + pl.tpw - 1) / pl.tpw;
    pl.lds = f4_lds(M, K, nblk, pl.wk, pl.tpw, rot, xf32);
    return pl;
}

template <bool XF32, bool ROT, bool SC4, int AT>
void (*f4_kernel_at(int tpw))(F4Args)
{
    switch (tpw) {
    case 1: return gemv_f4_kernel<1, XF32, ROT, SC4, AT>;
    case 2: return gemv_f4_kernel<2, XF32, ROT, SC4, AT>;
    case 3: return gemv_f4_kernel<3, XF32, ROT, SC4, AT>;
    default: return gemv_f4_kernel<4, XF32, ROT, SC4, AT>;
    }
}

template <bool XF32, bool ROT, bool SC4>
void (*f4_kernel(int tpw, int M))(F4Args)
{
    return f4_tiles(M) == 1 ? f4_kernel_at<XF32, ROT, SC4, 1>(tpw) : f4_kernel_at<XF32, ROT, SC4, 2>(tpw);
}

}  // namespace

namespace tern {

bool f4_supported(int64_t M, int64_t N, int64_t K, bool rot, bool x_f32)
{
    if (M < 1 || M > kF4MaxM || K <= 0 || N <= 0) return false;
    if (rot && K % 4096 != 0) return false;
    return plan_f4(N, K, (int)M, rot, x_f32).lds <= kMaxLds;
}

int launch_gemv_f4(const void *x, bool x_f32, const int8_t *signs, bool rot, int M, int64_t K,
                   const uint32_t *codes, const uint16_t *scales, int64_t N, void *y, bool y_bf16, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t count = (int64_t)M * N;
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(f4_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, y,
                           count, y_bf16 ? 1 : 0);
        return (int)hipGetLastError();
    }
    F4Args a;
    a.x = x;
    a.signs = signs;
    a.codes = codes;
    a.scales = scales;
    a.y = y;
    a.N = N;
    a.K = (int)K;
    a.M = M;
    a.G = (int)(K / kGroup);
    a.nblk = (a.G + 1) / 2;
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.norm = 1.0f / 64.0f;
    const F4Plan pl = plan_f4(N, K, M, rot, x_f32);
    a.wk = pl.wk;
    a.bq = a.nblk / pl.wk;
    a.br = a.nblk % pl.wk;
    const bool sc4 = (a.G % 2) == 0;
    void (*kernel)(F4Args);
    if (rot)
        kernel = x_f32 ? f4_kernel<true, true, true>(pl.tpw, M) : f4_kernel<false, true, true>(pl.tpw, M);
    else if (x_f32)
        kernel = sc4 ? f4_kernel<true, false, true>(pl.tpw, M) : f4_kernel<true, false, false>(pl.tpw, M);
    else
        kernel = sc4 ? f4_kernel<false, false, true>(pl.tpw, M) : f4_kernel<false, false, false>(pl.tpw, M);
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * pl.wk), pl.lds, st, a);
    return (int)hipGetLastError();
}

}  // namespace tern
