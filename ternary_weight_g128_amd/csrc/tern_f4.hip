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
#include <type_traits>
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

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// fp4 operand registers of two code words (16 weights each); the instruction
// reads four registers for an fp4 operand, the other four are left undefined.
__device__ __forceinline__ i32x8_t f4_weights(unsigned w0, unsigned w1)
{
    const i32x4_t b = {(int)(((w0 << 2) & kF4Mask) ^ kF4Flip), (int)((w0 & kF4Mask) ^ kF4Flip),
                       (int)(((w1 << 2) & kF4Mask) ^ kF4Flip), (int)((w1 & kF4Mask) ^ kF4Flip)};
    return __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
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

// LDS image of the activation operands.  Chunk (group G, half h, lane group
// ga, A row r) -- the 16 bytes one lane reads for one operand half -- sits
// at byte (((G * 2 + h) * 4 + ga) * (RA + 1) + r) * 16 (RA = 8 M A rows;
// the extra chunk per run keeps the staging writes, 16 bytes per lane at
// a run's stride, off each other's banks).  E8M0 scales: one dword per
// (256-K block, lane group, A row), byte j = group 2 blk + j.  One zero
// chunk and one unit-scale dword serve the lanes whose rows are not in use.
struct F4Lds {
    unsigned char *aimg;
    uint32_t *simg;
    float *red;
    unsigned char *zero;  // 16 zero bytes, then the dword 0x7F7F7F7F
    float *ximg;          // rotated input: binary32 x' rows, padded
    unsigned char *xs;    // rotated input: d .* x staging for the transform
};

// Padded index of activation k in a row of the rotated binary32 image:
// 16 floats of padding per 256 keep the transform's four lane groups on
// distinct banks.
__device__ __forceinline__ int f4_xpad(int k) { return k + 16 * (k >> 8); }

constexpr unsigned kBufRaw = 0x00020000u;  // raw buffer resource, 32-bit data format

// OS ("one shot"): every wave has at most PF blocks, all loaded up front with
// no load under a branch, so that the compiler can wait for each block's
// codes alone; up to eight waves.  Otherwise a ring of PF blocks refilled as
// they are consumed; up to four waves.
template <int TPW, bool XF32, bool ROT, bool SC4, int AT, bool OS>
__global__ __launch_bounds__(OS ? 512 : 256) void gemv_f4_kernel(const F4Args a)
{
    constexpr int PF = 4;     // ring slots (blocks)
    constexpr int kDist = 4;  // blocks of codes in flight: a slot is refilled as soon as it is consumed
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int nthreads = 64 * waves;
    const int kw = wave;  // every wave splits K
    const int nn = lane & 15, g = lane >> 4;
    const int RA = kParts * a.M;  // A rows (AT tiles of 16, the last one partly used)
    const int RS = RA + 1;        // chunks per run in the operand image
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
    off += (size_t)RS * a.K;
    L.simg = reinterpret_cast<uint32_t *>(smem + off);
    off += (size_t)a.nblk * 4 * RA * 4;
    L.red = reinterpret_cast<float *>(smem + off);
    off += (size_t)waves * TPW * AT * 4 * kTileN * 4;
    L.zero = smem + off;
    off += 32;
    L.ximg = reinterpret_cast<float *>(smem + off);
    const int xrow = a.K + 16 * (a.K >> 8);  // padded binary32 row of x'
    off += ROT ? (size_t)a.M * xrow * 4 : 0;
    L.xs = smem + off;
    if (threadIdx.x == 0) {
        *reinterpret_cast<u32x4_t *>(L.zero) = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint32_t *>(L.zero + 16) = 0x7F7F7F7Fu;
    }

    // 1. rotated input: d .* x for the transform, loads first
    const int wpr = a.K >> 4;  // 16-activation words per row
    const int8_t *sign_src = a.signs;
    constexpr int kPadX = XF32 ? 68 : 72;
    const int xs_row = (a.K >> 6) * kPadX;
    const int rot_units = ROT ? a.M * wpr : 0;
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

    // plain input: the first round of staging loads leaves before the code
    // stream (each thread's first 16 activations, raw)
    const int units = a.M * G * 8;
    constexpr int kPre = 2;  // staging rounds whose loads leave up front
    u32x4_t xraw[kPre][4];
    if constexpr (!ROT) {
#pragma unroll
        for (int rd = 0; rd < kPre; ++rd) {
            int u = rd * nthreads + threadIdx.x;
            if (u >= units) u = units - 2 + (threadIdx.x & 1);
            const int j = u & 1, gs = (u >> 1) & 3, q = u >> 3;
            const int m = q / G;
            const int k0 = 128 * (q % G) + 32 * f4_perm(gs) + 16 * j;
            if constexpr (XF32) {
                const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(a.x) +
                                                                       (int64_t)m * a.K + k0);
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) xraw[rd][qd] = src[qd];
            } else {
                const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) +
                                                                       (int64_t)m * a.K + k0);
#pragma unroll
                for (int qd = 0; qd < 2; ++qd) xraw[rd][qd] = src[qd];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. code stream: raw buffer loads over this workgroup's rows (rows past
    //    N read as zero words with zero scales; their outputs are dropped),
    //    the block's offset in a scalar register
    const int64_t rows_here = a.N - n0 < rows_per_wg ? a.N - n0 : rows_per_wg;
    const int row_bytes = a.K / 4;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.codes + n0 * (a.K / 16)), (short)0, (int)(rows_here * row_bytes), (int)kBufRaw);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scales + n0 * G), (short)0, (int)(rows_here * G * 2), (int)kBufRaw);
    int cvo[TPW], svo[TPW];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
        cvo[tp] = (tp * kTileN + nn) * row_bytes + 16 * g;
        svo[tp] = (tp * kTileN + nn) * G * 2;
    }
    u32x4_t cbuf[PF][TPW];
    uint32_t sbuf[PF][TPW];
    // block b: words 4 g .. 4 g + 3 of its 256 K.  A one-group last block
    // (odd G only) has no second group: its lanes for that group and its
    // second scale take an out-of-range offset and read zero, so that no
    // load runs past the end of a row (the group's offset travels in the
    // scalar offset, which the range check may not cover)
    constexpr int kOob = 0x7FFFFFF0;
    auto load_block = [&](int b, int p) {
        const int gb = g_begin + 2 * b;
        const bool one = !SC4 && gb + 1 >= G;
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const int cv = (one && g >= 2) ? kOob : cvo[tp];
            cbuf[p][tp] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cv, gb * 32, 0));
            if constexpr (SC4)
                sbuf[p][tp] = __builtin_amdgcn_raw_buffer_load_b32(srs, svo[tp], gb * 2, 0);
            else
                sbuf[p][tp] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, svo[tp], gb * 2, 0) |
                              ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, one ? kOob : svo[tp], gb * 2 + 2, 0)
                               << 16);
        }
    };
#pragma unroll
    for (int p = 0; p < kDist; ++p) {
        if constexpr (OS)
            load_block(p < nblocks ? p : nblocks - 1, p);  // unconditional; extra slots are not used
        else if (p < nblocks)
            load_block(p, p);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. activations -> LDS operand image
    // One unit = (row m, group G, scale block gs, word j): the 16 activations
    // of word 2 P(gs) + j, which A lane group 2 (gs & 1) + j carries in half
    // gs >> 1.  Units u, u ^ 1 are the two words of one scale block; they
    // exchange their largest magnitudes so both use the same exponent.
    // Parts are produced until every remainder is at most 2^-16 of its own
    // activation: checked from the part after which bfloat16 input (8
    // significant bits) or binary32 input (16 checked bits) is normally done.
    constexpr int kFirstCheck = (XF32 || ROT) ? 4 : 2;
    int parts_used = 0;  // largest part count of this thread's units (wave-uniform)
    auto stage_unit = [&](int u, const float (&v)[16]) {
        const int j = u & 1, gs = (u >> 1) & 3, q = u >> 3;
        const int Gi = q % G, m = q / G;
        const int ga = 2 * (gs & 1) + j, h = gs >> 1;
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
        // partner lane (lane ^ 1) holds the other word of the scale block
        amax = __builtin_fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                                    __builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false)));
        // 2^e0 puts the largest magnitude in [128, 256); parts step by 2^4
        const int e0 = (int)(__builtin_bit_cast(uint32_t, amax) >> 23) - 127 - 7;
        int sp = e0 < -127 ? -127 : e0;  // exponent of the current part's scale
        float t[16], x0[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x0[e] = __builtin_ldexpf(v[e], -sp);
            t[e] = x0[e];
        }
        unsigned char *dst = L.aimg + ((((size_t)Gi * 2 + h) * 4 + ga) * RS + kParts * m) * 16;
        unsigned char *sd = reinterpret_cast<unsigned char *>(L.simg) +
                            (((size_t)(Gi >> 1) * 4 + gs) * RA + kParts * m) * 4 + (Gi & 1);
        const int sp0 = sp;
        int np = 0;
        for (int p = 0; p < kParts; ++p) {
            *reinterpret_cast<u32x4_t *>(dst + 16 * p) = f4_part(t);
            if (j == 0) sd[4 * p] = (unsigned char)(kE8M0One + sp);  // read by lane group gs
            np = p + 1;
            if (np >= kFirstCheck) {
                // remainder (in units of the part just written, 2^sp) against
                // 2^-16 of the activation (in units of 2^sp0)
                const int sh = sp0 - sp - 16;
                bool done = true;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    done = done && (__builtin_fabsf(t[e]) <= __builtin_ldexpf(__builtin_fabsf(x0[e]), sh));
                if (__builtin_amdgcn_ballot_w64(!done) == 0) break;  // every block of the wave is done
            }
            const int next = sp - 4 < -127 ? -127 : sp - 4;
#pragma unroll
            for (int e = 0; e < 16; ++e) t[e] = __builtin_ldexpf(t[e], sp - next);
            sp = next;
        }
        // rows of parts not produced: zero data, unit scale
        for (int p = np; p < kParts; ++p) {
            *reinterpret_cast<u32x4_t *>(dst + 16 * p) = u32x4_t{0u, 0u, 0u, 0u};
            if (j == 0) sd[4 * p] = (unsigned char)kE8M0One;
        }
        parts_used = np > parts_used ? np : parts_used;
    };
    // a unit's 16 activations: from global memory (plain input, loaded raw
    // first and widened when used) or from the rotated binary32 image in LDS
    auto unit_k0 = [&](int u, int &m) {
        const int j = u & 1, gs = (u >> 1) & 3, q = u >> 3;
        m = q / G;
        return 128 * (q % G) + 32 * f4_perm(gs) + 16 * j;
    };
    auto unit_raw = [&](int u, u32x4_t (&r)[4]) {
        int m;
        const int k0 = unit_k0(u, m);
        if constexpr (XF32) {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(a.x) +
                                                                   (int64_t)m * a.K + k0);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) r[qd] = src[qd];
        } else {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) +
                                                                   (int64_t)m * a.K + k0);
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) r[qd] = src[qd];
        }
    };
    auto unit_widen = [&](const u32x4_t (&r)[4], float (&v)[16]) {
        if constexpr (XF32) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned de = r[qd][e];
                    v[4 * qd + e] = __builtin_bit_cast(float, de);
                }
        } else {
#pragma unroll
            for (int qd = 0; qd < 2; ++qd)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned de = r[qd][e];
                    v[8 * qd + 2 * e] = __builtin_bit_cast(float, de << 16);
                    v[8 * qd + 2 * e + 1] = __builtin_bit_cast(float, de & 0xffff0000u);
                }
        }
    };
    auto unit_lds = [&](int u, float (&v)[16]) {
        int m;
        const int k0 = unit_k0(u, m);
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
    };
    auto unit_of = [&](int u0) {
        int u = u0 + (int)threadIdx.x;
        return u < units ? u : units - 2 + (int)(threadIdx.x & 1);
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
    // the first kPre rounds use the loads issued up front (straight-line
    // code, so the compiler waits for those loads only), then a loop
#pragma unroll
    for (int rd = 0; rd < kPre; ++rd) {
        if (rd * nthreads < units) {
            const int u = unit_of(rd * nthreads);
            float v[16];
            if constexpr (ROT)
                unit_lds(u, v);
            else
                unit_widen(xraw[rd], v);
            stage_unit(u, v);
        }
    }
    for (int u0 = kPre * nthreads; u0 < units; u0 += nthreads) {
        const int u = unit_of(u0);
        float v[16];
        if constexpr (ROT) {
            unit_lds(u, v);
        } else {
            unit_raw(u, xraw[0]);
            unit_widen(xraw[0], v);
        }
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
    // this lane's A chunks (row 16 at + nn; unused rows read the zero chunk
    // and a unit scale) as byte offsets into LDS for group 0, half 0
    // per lane: byte offsets of the A chunks of group g_begin and the E8M0
    // dword of its block, and the steps per 256-K block and per group
    // (zero for unused rows, which keep reading the zero chunk)
    int abase[AT], sbase[AT], astep[AT], gstep[AT], hstep[AT], sstep[AT];
    const int gstride = 8 * RS * 16;  // bytes per group in the operand image
#pragma unroll
    for (int at = 0; at < AT; ++at) {
        const int r = 16 * at + nn;  // A row: part (r & 7) of x row r >> 3
        const bool used = r < RA && (r & 7) < p_wg;
        abase[at] = used ? (int)(L.aimg - smem) + (g * RS + r) * 16 + g_begin * gstride : (int)(L.zero - smem);
        sbase[at] = used ? (int)((unsigned char *)L.simg - smem) + ((g_begin >> 1) * 4 * RA + g * RA + r) * 4
                         : (int)(L.zero - smem) + 16;
        astep[at] = used ? 2 * gstride : 0;
        gstep[at] = used ? gstride : 0;
        hstep[at] = used ? 4 * RS * 16 : 0;  // half 0 -> half 1
        sstep[at] = used ? 4 * RA * 4 : 0;
    }
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    // TWO: the block holds two groups (every block but a one-group last one)
    auto process = [&](int b, int p, auto two_c) {
        constexpr bool two = decltype(two_c)::value;
        // keep the blocks in order: each consumes its codes, refills the ring
        // and issues its matrix work before the next block starts
        __builtin_amdgcn_sched_barrier(0);
        i32x8_t a0[AT], a1[AT];
        uint32_t sdw[AT];
#pragma unroll
        for (int at = 0; at < AT; ++at) {
            const unsigned char *c0 = smem + abase[at] + b * astep[at];
            const unsigned char *c1 = c0 + (two ? gstep[at] : 0);
            const i32x4_t x00 = *reinterpret_cast<const i32x4_t *>(c0);
            const i32x4_t x01 = *reinterpret_cast<const i32x4_t *>(c0 + hstep[at]);
            const i32x4_t x10 = *reinterpret_cast<const i32x4_t *>(c1);
            const i32x4_t x11 = *reinterpret_cast<const i32x4_t *>(c1 + hstep[at]);
            a0[at] = __builtin_shufflevector(x00, x01, 0, 1, 2, 3, 4, 5, 6, 7);
            a1[at] = __builtin_shufflevector(x10, x11, 0, 1, 2, 3, 4, 5, 6, 7);
            uint32_t sv = *reinterpret_cast<const uint32_t *>(smem + sbase[at] + b * sstep[at]);
            // a one-group block reuses group gl0 (scaled by zero below); its
            // exponent byte stands in for the missing second one
            if (!two) sv = (sv & 0xffu) * 0x0101u;
            sdw[at] = sv;
        }
        unsigned wq[TPW][4];
        uint32_t sc[TPW];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            auto s02 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][0], cbuf[p][tp][2], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][1], cbuf[p][tp][3], false, false);
            wq[tp][0] = s02[0];  // group 0, word 2 P(g)
            wq[tp][1] = s13[0];  // group 0, word 2 P(g) + 1
            wq[tp][2] = s02[1];  // group 1
            wq[tp][3] = s13[1];
            sc[tp] = two ? sbuf[p][tp] : (sbuf[p][tp] & 0xffffu);  // binary16 pair; zero for a missing group
        }
        if constexpr (!OS)
            if (b + kDist < nblocks) load_block(b + kDist, (p + kDist) % PF);
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const i32x8_t b0 = f4_weights(wq[tp][0], wq[tp][1]);
            const i32x8_t b1 = f4_weights(wq[tp][2], wq[tp][3]);
            const float s0 = half_to_float((uint16_t)(sc[tp] & 0xffffu));
            const float s1 = half_to_float((uint16_t)(sc[tp] >> 16));
#pragma unroll
            for (int at = 0; at < AT; ++at) {
                const f32x4_t d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a0[at], b0, zero4, 0, 4, 0, (int)sdw[at], 0, kE8M0One);
                const f32x4_t d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a1[at], b1, zero4, 0, 4, 1, (int)sdw[at], 0, kE8M0One);
                // four parts of the lane group's x row (zero rows past M)
                const float t0 = (d0[0] + d0[1]) + (d0[2] + d0[3]);
                const float t1 = (d1[0] + d1[1]) + (d1[2] + d1[3]);
                yacc[tp][at] = __builtin_fmaf(s0, t0, yacc[tp][at]);
                yacc[tp][at] = __builtin_fmaf(s1, t1, yacc[tp][at]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // only the wave's last block can hold a single group (odd G)
    const int ntwo = (g_begin + 2 * nblocks > g_end) ? nblocks - 1 : nblocks;
    const int nfull = OS ? 0 : (ntwo / PF) * PF;
    for (int b0 = 0; b0 < nfull; b0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) process(b0 + p, p, std::true_type{});
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (nfull + p < ntwo) process(nfull + p, p, std::true_type{});
    if (ntwo < nblocks) {
        // ring slots are registers: the slot index must be a constant
        switch (ntwo % PF) {
        case 0: process(ntwo, 0, std::false_type{}); break;
        case 1: process(ntwo, 1, std::false_type{}); break;
        case 2: process(ntwo, 2, std::false_type{}); break;
        default: process(ntwo, 3, std::false_type{}); break;
        }
    }

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
    bool os;
    int64_t wgs;
    size_t lds;
};

// A tiles (16 A rows each) for M x rows of kParts parts.
inline int f4_tiles(int M) { return (kParts * M + 15) / 16; }

size_t f4_lds(int M, int64_t K, int nblk, int waves, int tpw, bool rot, bool xf32)
{
    const size_t ra = (size_t)kParts * M;
    size_t b = (ra + 1) * K + (size_t)nblk * 4 * ra * 4 + (size_t)waves * tpw * f4_tiles(M) * 4 * kTileN * 4 + 32;
    if (rot) {
        b += (size_t)M * (K + 16 * (K >> 8)) * 4;
        b += (size_t)M * (K >> 6) * (xf32 ? 68 * 4 : 72 * 2);
    }
    return b;
}

// Work split: tiles per wave (tpw) and K-waves per workgroup (wk).  Every
// workgroup converts all of x once, so about one workgroup per CU.  When
// every K-wave can hold all of its 256-K blocks in the four-slot ring
// (K <= 8192 with up to eight waves), the one-shot kernel loads them all up
// front; longer rows stream through the ring with four waves.
F4Plan plan_f4(int64_t N, int64_t K, int M, bool rot, bool xf32)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    const int cus = device_cus();
    F4Plan pl;
    pl.os = nblk <= 8 * 4;
    int64_t t = (tiles + cus - 1) / cus;
    pl.tpw = (int)(t <= 1 ? 1 : t <= 2 ? 2 : t <= 3 ? 3 : 4);
    if (pl.os) {
        if (pl.tpw > 3) pl.tpw = 3;  // one-shot kernels run up to three tiles per wave
        pl.wk = 1;
        while (pl.wk < 8 && (nblk + pl.wk - 1) / pl.wk > 4) pl.wk *= 2;
        while (pl.wk < 4 && nblk >= 2 * (pl.wk * 2)) pl.wk *= 2;
    } else {
        // four tiles per wave leave room for one workgroup per CU: if that
        // needs a second round, three tiles with two workgroups per CU need none
        if (pl.tpw == 4 && (tiles + 3) / 4 > cus) pl.tpw = 3;
        pl.wk = 1;
        while (pl.wk < 4 && nblk >= 2 * (pl.wk * 2)) pl.wk *= 2;
    }
    pl.wgs = (tiles + pl.tpw - 1) / pl.tpw;
    pl.lds = f4_lds(M, K, nblk, pl.wk, pl.tpw, rot, xf32);
    return pl;
}

template <bool XF32, bool ROT, bool SC4, int AT>
void (*f4_kernel_at(int tpw, bool os))(F4Args)
{
    if (os) {
        switch (tpw) {
        case 1: return gemv_f4_kernel<1, XF32, ROT, SC4, AT, true>;
        case 2: return gemv_f4_kernel<2, XF32, ROT, SC4, AT, true>;
        default: return gemv_f4_kernel<3, XF32, ROT, SC4, AT, true>;
        }
    }
    switch (tpw) {
    case 1: return gemv_f4_kernel<1, XF32, ROT, SC4, AT, false>;
    case 2: return gemv_f4_kernel<2, XF32, ROT, SC4, AT, false>;
    case 3: return gemv_f4_kernel<3, XF32, ROT, SC4, AT, false>;
    default: return gemv_f4_kernel<4, XF32, ROT, SC4, AT, false>;
    }
}

template <bool XF32, bool ROT, bool SC4>
void (*f4_kernel(int tpw, int M, bool os))(F4Args)
{
    return f4_tiles(M) == 1 ? f4_kernel_at<XF32, ROT, SC4, 1>(tpw, os) : f4_kernel_at<XF32, ROT, SC4, 2>(tpw, os);
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
    // binary16 scale pairs load as one dword: even G and a 4-byte aligned base
    const bool sc4 = (a.G % 2) == 0 && (reinterpret_cast<uintptr_t>(scales) % 4) == 0;
    void (*kernel)(F4Args);
    if (rot && sc4)
        kernel = x_f32 ? f4_kernel<true, true, true>(pl.tpw, M, pl.os) : f4_kernel<false, true, true>(pl.tpw, M, pl.os);
    else if (rot)
        kernel = x_f32 ? f4_kernel<true, true, false>(pl.tpw, M, pl.os) : f4_kernel<false, true, false>(pl.tpw, M, pl.os);
    else if (x_f32)
        kernel = sc4 ? f4_kernel<true, false, true>(pl.tpw, M, pl.os) : f4_kernel<true, false, false>(pl.tpw, M, pl.os);
    else
        kernel = sc4 ? f4_kernel<false, false, true>(pl.tpw, M, pl.os) : f4_kernel<false, false, false>(pl.tpw, M, pl.os);
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * pl.wk), pl.lds, st, a);
    return (int)hipGetLastError();
}

}  // namespace tern
