// HIP kernels of libtern for AMD MI355X (gfx950 / CDNA4).
//
// Ternary-g128 matmul ("prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card,
// "Weight representation: ternary g128", "Memory requirement", "CUDA (NVIDIA
// GPUs)"): y[m][n] = sum_g s[n][g] * sum_{k in g} t[n][k] x[m][k], with the
// 2-bit codes unpacked inside the kernel.  Signed normalized Walsh-Hadamard
// rotation ("Ternary-Bonsai-2-9B-2bit" article, section 3).
//
// Exact operand trick used by every matmul kernel here.  XOR-ing a code word
// with 0x55555555 turns each slot q = t + 1 into the bit pair
// ([t = +1], [t != 0]).  Moving a pair to bits 15..14 of a 16-bit half and
// clearing the rest gives the bfloat16 pattern 0xC000 (-2.0) for t = +1,
// 0x4000 (+2.0) for t = -1 and 0 for t = 0: the exact value -2t.  One packed
// 16-bit shift pair (v_pk_lshlrev_b16 plus v_and_b32) yields two weights, so
// the unpack costs about one VALU operation per weight, and the matrix cores
// see exact {-2, 0, +2} operands.  Products with bfloat16 activations are
// exact in the MFMA's binary32 accumulator; each 128-K group is accumulated
// from zero and then scaled by -s_g/2 in binary32, so the group scale never
// passes through a 16-bit format.
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

// Sixteen +1 signs: the sign row read when the caller passes no sign vector,
// so that the sign load is unconditional (a load under a branch makes the
// compiler wait for it, and for everything issued before it, at once).
__device__ const unsigned kOnes16[4] = {0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
typedef const u32x4_t __attribute__((address_space(1))) gu32x4_t;  // global memory
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef const u32x2_t __attribute__((address_space(1))) gu32x2_t;
typedef const uint32_t __attribute__((address_space(1))) gu32_t;

// Sign vectors: only the sign bit of each int8 entry is read, so d[k] = -1
// where signs[k] < 0 and +1 otherwise.  Every transform path applies d by
// flipping the binary32 (or bfloat16) sign bit, which is exact.
// Bit 31 set iff byte j of the four sign bytes in `w` is negative.
__device__ __forceinline__ uint32_t sign_bit(uint32_t w, int j)
{
    return ((w >> (8 * j + 7)) & 1u) << 31;
}

__device__ __forceinline__ float flip_if(float v, uint32_t bit31)
{
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) ^ bit31);
}



// Hadamard helpers (natural Sylvester order: a butterfly over every index
// bit).  See the transform section below for the data layout.
// Element index for thread t (within a block) and register index r when the
// register bits start at bit rb.
__device__ __forceinline__ int fwht_index(int t, int r, int rb)
{
    return (t & ((1 << rb) - 1)) | (r << rb) | ((t >> rb) << (rb + 4));
}

__device__ __forceinline__ int fwht_pad(int i) { return i + (i >> 4); }

__device__ __forceinline__ void butterfly_bits(float (&v)[16], int j_lo, int j_hi)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < j_lo || j >= j_hi) continue;
        const int h = 1 << j;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (r & h) continue;
            const float a = v[r], c = v[r | h];
            v[r] = a + c;
            v[r | h] = a - c;
        }
    }
}

// ---------------------------------------------------------------------------
// GEMV for M <= 16
// ---------------------------------------------------------------------------
//
// Work decomposition.  A workgroup owns TPW consecutive 16-row tiles and the
// whole K; its W waves split K into contiguous ranges of whole 256-K blocks
// (two scale groups) and the partial sums are combined in LDS in a fixed
// order at the end, so the result is deterministic.  Within a wave, lane l
// serves output row n0 + 16*tile + (l & 15) and lane group g = l >> 4 (the
// MFMA k-slot group).
//
// Codes.  Per block each lane loads one 16-byte vector per tile: words
// 4g..4g+3 of its row's 64-byte block segment, so the four lanes of a row
// read 64 contiguous bytes.  A v_permlane32_swap pair then regroups the words
// so that every lane holds two words of group 0 and two of group 1 (the MFMA
// contracts over all four lane groups, which must therefore see the same
// scale group).  After the swap, word w of a group sits in lane group
// {0, 2, 1, 3}[w >> 1] as operand half w & 1.
//
// Activations.  The MFMA A operand is x: row i = l & 15 of A is activation
// row i (bfloat16 input) or, for binary32 input, rows 2m / 2m + 1 hold the
// bfloat16 rounding of x[m] and the bfloat16 rounding of the remainder
// (x - hi is exact in binary32; the two parts carry 16 significand bits).
// The workgroup stages x for all of K in LDS once, permuted so that one
// 16-byte LDS read gives a lane its A operand for one MFMA; lanes whose A row
// does not exist never read and keep zeros (reading for them costs LDS
// bandwidth: 8x the bytes at M = 1).  LDS layout in bfloat16
// elements, for scale group G, MFMA index mu = 2 * (operand half) + h, lane
// group g, A row r and element e: ((((G * 4 + mu) * 4 + g) * MX + r) * 8 + e),
// where element e of (G, mu, g) holds k = 128 G + 16 w + 4 h + (e >> 1) +
// 8 (e & 1) for the word w = 2 {0, 2, 1, 3}[g] + (mu >> 1).

// Eight consecutive binary32 activations (one MFMA A operand's worth).
struct F32x8 {
    float e[8];
};

// Eight consecutive binary32 values from global memory (two 16-byte loads).
__device__ __forceinline__ F32x8 load_f32x8(const float *src)
{
    const u32x4_t a = reinterpret_cast<const u32x4_t *>(src)[0];
    const u32x4_t b = reinterpret_cast<const u32x4_t *>(src)[1];
    F32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // copy the element out first: bit-casting an ext_vector element
        // subscripted by a loop index reads element 0 (clang, this ROCm)
        const unsigned ai = a[i], bi = b[i];
        r.e[i] = __builtin_bit_cast(float, ai);
        r.e[4 + i] = __builtin_bit_cast(float, bi);
    }
    return r;
}

// The bfloat16 part of eight binary32 values that one A row carries: the
// rounding of each value (lo == false) or the rounding of its remainder
// (lo == true; x - hi is exact in binary32, and hi + lo carries 16
// significand bits of x).
__device__ __forceinline__ bf16x8_t split_part(const F32x8 &f, bool lo)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4_t out;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float f0 = f.e[2 * v];
        float f1 = f.e[2 * v + 1];
        // the remainder rows round x - bf16(x) instead of x (a choice per
        // value before the one pack of the pair)
        if (lo) {
            f0 -= (float)(__bf16)f0;
            f1 -= (float)(__bf16)f1;
        }
        const bf16x2_t p = {(__bf16)f0, (__bf16)f1};
        out[v] = __builtin_bit_cast(uint32_t, p);
    }
    return __builtin_bit_cast(bf16x8_t, out);
}

struct GemvArgs {
    const void *x;
    const uint32_t *codes;
    const uint16_t *scales;
    void *y;
    int64_t N;
    int K;        // multiple of 128
    int M;        // rows of x
    int nblk;     // 256-K blocks in K (the last one may hold one group)
    int wk;       // waves of a workgroup that split K (they share tiles)
    int wt;       // waves of a workgroup that split tiles (wt * wk waves)
    int bq, br;   // blocks per K-wave: bq, plus one for the first br K-waves
    int y_bf16;
    const int8_t *signs;  // rotated input: +-1 per K (or NULL)
    int log2b;            // rotated input: Hadamard block 2^log2b (>= 16)
    float norm;           // rotated input: 1/sqrt(block)
};

// One staging unit: the 16 activations of word wi (k = 16 wi .. 16 wi + 15)
// of row m, held as 32-bit words: bf16 pairs, or binary32 values.
template <bool XF32>
struct XUnit {
    uint32_t v[XF32 ? 16 : 8];
};

template <bool XF32, bool IN_F32 = XF32>
__device__ __forceinline__ void load_unit(XUnit<XF32> &u, const GemvArgs &a, int m, int wi)
{
    if constexpr (XF32 && !IN_F32) {
        // bfloat16 input, kept raw in words 0..7 here and widened to binary32
        // words by widen_unit once it is needed (no arithmetic on loaded
        // data may sit between the loads and the code stream issued next)
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
            static_cast<const uint16_t *>(a.x) + (int64_t)m * a.K + 16 * wi);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            u32x4_t d = src[q];
            u.v[4 * q + 0] = d[0]; u.v[4 * q + 1] = d[1]; u.v[4 * q + 2] = d[2]; u.v[4 * q + 3] = d[3];
        }
    } else if constexpr (XF32) {
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
            static_cast<const float *>(a.x) + (int64_t)m * a.K + 16 * wi);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x4_t d = src[q];
            u.v[4 * q + 0] = d[0]; u.v[4 * q + 1] = d[1]; u.v[4 * q + 2] = d[2]; u.v[4 * q + 3] = d[3];
        }
    } else {
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
            static_cast<const uint16_t *>(a.x) + (int64_t)m * a.K + 16 * wi);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            u32x4_t d = src[q];
            u.v[4 * q + 0] = d[0]; u.v[4 * q + 1] = d[1]; u.v[4 * q + 2] = d[2]; u.v[4 * q + 3] = d[3];
        }
    }
}

// bfloat16 pairs in words 0..7 of a binary32 unit -> binary32 words 0..15.
__device__ __forceinline__ void widen_unit(XUnit<true> &u)
{
#pragma unroll
    for (int e = 7; e >= 0; --e) {
        const uint32_t d = u.v[e];
        u.v[2 * e + 1] = d & 0xffff0000u;
        u.v[2 * e] = d << 16;
    }
}

// Write one unit into the permuted LDS image: two 16-byte chunks per A row.
template <int MX, bool XF32>
__device__ __forceinline__ void store_unit(__bf16 *lds, const XUnit<XF32> &u, int m, int wi)
{
    const int G = wi >> 3, w = wi & 7;
    const int g = ((w >> 1) == 1) ? 2 : (((w >> 1) == 2) ? 1 : (w >> 1));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int mu = 2 * (w & 1) + h;
        const int base = ((G * 4 + mu) * 4 + g) * MX;
        u32x4_t hi, lo;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // element pair (2v, 2v + 1) holds k = 4h + v and 4h + v + 8
            const int ka = 4 * h + v, kb = ka + 8;
            if constexpr (XF32) {
                const float fa = __builtin_bit_cast(float, u.v[ka]);
                const float fb = __builtin_bit_cast(float, u.v[kb]);
                typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
                const bf16x2_t ph = {(__bf16)fa, (__bf16)fb};
                const bf16x2_t pl = {(__bf16)(fa - (float)ph[0]), (__bf16)(fb - (float)ph[1])};
                hi[v] = __builtin_bit_cast(uint32_t, ph);
                lo[v] = __builtin_bit_cast(uint32_t, pl);
            } else {
                // bf16 pairs arrive as (k even, k odd) halves of 32-bit words
                const uint32_t wa = u.v[ka >> 1], wb = u.v[kb >> 1];
                const uint32_t sa = (ka & 1) ? (wa >> 16) : (wa & 0xffffu);
                const uint32_t sb = (kb & 1) ? (wb & 0xffff0000u) : (wb << 16);
                hi[v] = sa | sb;
            }
        }
        if constexpr (XF32) {
            *reinterpret_cast<u32x4_t *>(lds + (base + 2 * m) * 8) = hi;
            *reinterpret_cast<u32x4_t *>(lds + (base + 2 * m + 1) * 8) = lo;
        } else {
            *reinterpret_cast<u32x4_t *>(lds + (base + m) * 8) = hi;
        }
    }
}

// Scale of block j of a quad for lane group 0, when lane group g holds the
// scale pair of block g of the quad: v_permlane16_swap moves rows 1 -> 0 and
// 3 -> 2, v_permlane32_swap moves rows 2, 3 -> 0, 1.
__device__ __forceinline__ uint32_t quad_scale(uint32_t sq, int j)
{
    if (j == 0) return sq;
    if (j == 1) return __builtin_amdgcn_permlane16_swap(sq, sq, false, false)[1];
    const uint32_t r2 = __builtin_amdgcn_permlane32_swap(sq, sq, false, false)[1];
    if (j == 2) return r2;
    return __builtin_amdgcn_permlane16_swap(r2, r2, false, false)[1];
}

// PF == 4: the code ring holds one quad of four 256-K blocks (refilled two
// blocks ahead).  For MX <= 4
// every live output row sits in lane group 0, so the scales of a quad come
// from one load per lane (lane group g loads block g's scale pair) and are
// redistributed with cross-row swaps; for larger MX each lane loads its
// row's pair per block.
// ROT = 0: x is the activation (binary32 if XF32, else bfloat16).
// ROT = 1 / 2: x (bfloat16 / binary32) is rotated first, while the code
// stream is already in flight, and the result is staged as hi/lo bfloat16
// rows (XF32 == true).  Blocks of 4096 (ROTL == 12): d .* x goes to an LDS
// scratch as given and the transform H64 X H64 of each block runs on the
// matrix cores (see kMfmaRot).  Other blocks: d .* x in a padded binary32
// LDS scratch, the register-radix-16 butterflies of the stand-alone
// transform there, then 1/sqrt(b).
// AG: the A operand comes straight from global memory instead of an LDS
// image of x (bfloat16 input, no rotation): lane (row i, lane group g) reads
// the eight consecutive activations k = 128 G + 32 {0, 2, 1, 3}[g] + 8 mu +
// 0..7 of MFMA mu of scale group G, and the weight operand is built in the
// same consecutive order from byte planes of the raw code word.  Nothing of x
// is staged, so LDS does not limit the workgroups per CU for larger M.
template <int MX, bool XF32, int TPW, bool SC4, int ROT = 0, int ROTL = 0, bool AG = false>
__global__ __launch_bounds__(512) void gemv_kernel(const GemvArgs a)
{
    static_assert(ROT == 0 || XF32, "rotated activations are staged as hi/lo rows");
    static_assert(!AG || ROT == 0, "direct A loads take unrotated activations");
    constexpr int PF = 4;
    constexpr int kDist = 2;  // blocks of codes in flight
    constexpr bool kQuadScales = MX <= 4;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int kRowsOut = (MX < 4) ? MX : 4;  // accumulator rows per lane that can be live
    constexpr int kUB = ROT ? 1 : (XF32 ? 2 : 4);  // staging units per thread per batch
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int kw = wave % a.wk;                  // which K range
    const int tw = wave / a.wk;                  // which tiles
    const int nn = lane & 15;
    const int g = lane >> 4;
    const int arow = lane & 15;
    const int Mx = XF32 ? 2 * a.M : a.M;
    const bool a_active = arow < Mx;
    const int G = a.K / kGroup;

    const int b_begin = kw * a.bq + (kw < a.br ? kw : a.br);
    const int nblocks = a.bq + (kw < a.br ? 1 : 0);
    const int g_begin = 2 * b_begin;
    const int g_end = (g_begin + 2 * nblocks < G) ? g_begin + 2 * nblocks : G;

    const int rows_per_wg = kTileN * TPW * a.wt;
    const int64_t n_wg = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t n0 = n_wg + (int64_t)tw * (kTileN * TPW);
    if (a.K == 0) {  // empty sum: zeros (uniform branch before any load)
        for (int o = threadIdx.x; o < a.M * rows_per_wg; o += blockDim.x) {
            const int64_t n = n_wg + o % rows_per_wg;
            if (n < a.N) {
                const int m = o / rows_per_wg;
                if (a.y_bf16)
                    static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = 0;
                else
                    static_cast<float *>(a.y)[(int64_t)m * a.N + n] = 0.0f;
            }
        }
        return;
    }
    // From here on K > 0, so every wave has at least one block and every
    // thread a staging unit; the loads below are unconditional so that the
    // compiler can count outstanding loads exactly.
    __bf16 *lds_x = reinterpret_cast<__bf16 *>(smem);
    const int rowpad = ROT ? a.K + (a.K >> 4) : 0;  // padded row of the rotation scratch
    float *rot = reinterpret_cast<float *>(smem + (AG ? 0 : (size_t)a.K * MX * 2));
    float *red = rot + (ROT ? (size_t)a.M * rowpad : 0);

    // 1. activation loads for the first staging batch go out first, so that
    //    waiting for them does not wait for the code stream issued next.
    //    Unit indices past the end are clamped to the last unit: duplicate
    //    stores write the same values to the same LDS bytes.
    const int wpr = a.K / 16;  // words (units) per activation row
    const int units = AG ? 0 : a.M * wpr;
    const int nthreads = 64 * waves;
    constexpr bool kInF32 = ROT ? (ROT == 2) : XF32;
    // 4096-point blocks go through the matrix cores (rot_unit below); other
    // blocks use radix-16 butterflies in LDS.
    constexpr bool kMfmaRot = ROT != 0 && ROTL == 12;
    XUnit<XF32> xu[kUB];
    u32x4_t du[kUB];  // signs of the unit (rotation)
    const int8_t *sign_src = a.signs ? a.signs : reinterpret_cast<const int8_t *>(kOnes16);
    auto load_x = [&](int i, int u) {
        load_unit<XF32, kInF32>(xu[i], a, u / wpr, u % wpr);
        if constexpr (ROT != 0)
            du[i] = *(const gu32x4_t *)(sign_src + (a.signs ? 16 * (u % wpr) : 0));
    };
    // matrix-core rotation: d .* x staged once per workgroup in LDS (the
    // rotation scratch), rows of 64 elements padded to kPadX (conflict-free
    // 16-byte operand reads)
    const int rot_per_row = (a.K >> 12) * 4;
    const int rot_units = a.M * rot_per_row;
    constexpr int kPadX = ROT == 2 ? 68 : 72;
    const int xs_row = kMfmaRot ? (a.K >> 6) * kPadX : 0;  // elements per staged row
#pragma unroll
    for (int i = 0; i < (AG ? 0 : kUB); ++i) {
        int u = threadIdx.x + i * nthreads;
        u = u < units ? u : units - 1;
        load_x(i, u);
    }
    __builtin_amdgcn_sched_barrier(0);  // activation loads leave first

    // 2. code stream: one quad ahead
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
    uint32_t sbuf[PF][TPW];    // per-block scale pairs (MX > 4)
    uint32_t squad[TPW];       // quad scale pairs (MX <= 4)
    // For a one-group block the upper lane groups re-read the first group,
    // whose second-half contribution is multiplied by a zero scale.
    auto scale_pair = [&](int tp, int gb, bool two) -> uint32_t {
        if constexpr (SC4)
            return *reinterpret_cast<const uint32_t *>(srow[tp] + gb);
        else
            return (uint32_t)srow[tp][gb] | ((uint32_t)srow[tp][two ? gb + 1 : gb] << 16);
    };
    auto load_block = [&](int b, int p) {
        b = b < nblocks ? b : nblocks - 1;
        const int gb = g_begin + 2 * b;
        const bool two = (gb + 1) < g_end;
        const int lg = two ? g : (g & 1);
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            cbuf[p][tp] = *reinterpret_cast<const u32x4_t *>(crow[tp] + gb * kWordsPerGroup + 4 * lg);
            if constexpr (!kQuadScales) sbuf[p][tp] = scale_pair(tp, gb, two);
        }
    };
    auto load_quad_scales = [&](int b0) {
        if constexpr (kQuadScales) {
            int b = b0 + g;
            b = b < nblocks ? b : nblocks - 1;
            const int gb = g_begin + 2 * b;
            const bool two = (gb + 1) < g_end;
#pragma unroll
            for (int tp = 0; tp < TPW; ++tp) squad[tp] = scale_pair(tp, gb, two);
        }
    };
    // The ring has PF slots (one quad, the unit of the scale loads) but is
    // refilled only kDist blocks ahead: waves start computing as soon as
    // their first blocks land while the other waves keep HBM busy.
#pragma unroll
    for (int p = 0; p < kDist; ++p) load_block(p, p);
    load_quad_scales(0);
    // Keep the code stream ahead of everything that waits for the
    // activations: left to itself the scheduler moves the staging arithmetic
    // (and its wait for x) above these loads, which then leave one full
    // memory latency late.
    __builtin_amdgcn_sched_barrier(0);

    // 3. stage the activations of all of K (shared by the waves)
    auto put = [&](int i, int u) {
        XUnit<XF32> &xv = xu[i];
        const u32x4_t &dv = du[i];
        const int m = u / wpr, wi = u % wpr;
        if constexpr (kMfmaRot) {
            // d .* x for the 16 elements k = 16 wi .. 16 wi + 15 (sign bit
            // flipped where the sign byte is negative), as given: bfloat16
            // pairs or binary32 words
            const int k = 16 * wi;
            if constexpr (ROT == 1) {
                u32x4_t q[2];
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const uint32_t sel = (v & 1) ? 0x030C020Cu : 0x010C000Cu;  // sign bytes -> bytes 1, 3
                    q[v >> 2][v & 3] = xv.v[v] ^ (__builtin_amdgcn_perm(0u, dv[v >> 1], sel) & 0x80008000u);
                }
                u32x4_t *dst = reinterpret_cast<u32x4_t *>(
                    reinterpret_cast<uint16_t *>(rot) + (size_t)m * xs_row + (k >> 6) * kPadX + (k & 63));
                dst[0] = q[0];
                dst[1] = q[1];
            } else {
                u32x4_t q[4];
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    q[e >> 2][e & 3] = xv.v[e] ^ (((dv[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31);
                u32x4_t *dst = reinterpret_cast<u32x4_t *>(
                    reinterpret_cast<uint32_t *>(rot) + (size_t)m * xs_row + (k >> 6) * kPadX + (k & 63));
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) dst[q4] = q[q4];
            }
            return;
        }
        if constexpr (XF32 && !kInF32) widen_unit(xv);
        if constexpr (ROT == 0) {
            store_unit<MX, XF32>(lds_x, xv, m, wi);
        } else {
            // a unit is 16 consecutive elements: exactly one group of the
            // first butterfly pass (index bits 0..3), done here in registers
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                v[e] = __builtin_bit_cast(float, xv.v[e] ^ sign_bit(dv[e >> 2], e & 3));
            }
            butterfly_bits(v, 0, 4);
            float *row = rot + (size_t)m * rowpad + 17 * wi;  // pad(16 wi + e) = 17 wi + e
#pragma unroll
            for (int e = 0; e < 16; ++e) row[e] = v[e];
        }
    };
#pragma unroll
    for (int i = 0; i < (AG ? 0 : kUB); ++i) {
        int u = threadIdx.x + i * nthreads;
        u = u < units ? u : units - 1;
        put(i, u);
    }
    for (int u0 = kUB * nthreads; u0 < (AG ? 0 : units); u0 += kUB * nthreads) {
#pragma unroll
        for (int i = 0; i < kUB; ++i) {
            int u = u0 + threadIdx.x + i * nthreads;
            u = u < units ? u : units - 1;
            load_x(i, u);
        }
#pragma unroll
        for (int i = 0; i < kUB; ++i) {
            int u = u0 + threadIdx.x + i * nthreads;
            u = u < units ? u : units - 1;
            put(i, u);
        }
    }
    if constexpr (!AG) __syncthreads();
    if constexpr (kMfmaRot) {
        // 4096-point blocks on the matrix cores (h64_slice): a unit is one
        // 16-column slice jt of one block of one row; the result goes
        // straight into the operand image, times 1/64, as hi/lo rows 2m and
        // 2m + 1 (the image position of k is that of store_unit: group
        // k >> 7, word w = (k >> 4) & 7, slot p = k & 15)
        const int c = nn;
        auto rot_unit = [&](int u) {
            const int m = u / rot_per_row, rem = u % rot_per_row, blk = rem >> 2, jt = rem & 3;
            const size_t at = (size_t)m * xs_row + (size_t)64 * blk * kPadX;
            const void *xs = ROT == 2 ? (const void *)(reinterpret_cast<const uint32_t *>(rot) + at)
                                      : (const void *)(reinterpret_cast<const uint16_t *>(rot) + at);
            f32x4_t o[4];
            h64_slice<ROT == 2>(xs, jt, c, g, o);
            // lane holds X'[16 ot + 4 g + r][16 jt + c]: element
            // k = 4096 blk + 64 (16 ot + 4 g + r) + 16 jt + c of the row
            const int mu = 2 * (jt & 1) + ((c >> 2) & 1);
            const int e = 2 * (c & 3) + (c >> 3);
#pragma unroll
            for (int ot = 0; ot < 4; ++ot)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ip = 16 * ot + 4 * g + r;
                    const int G = 32 * blk + (ip >> 1);
                    const int g2 = 2 * (jt >> 1) + (ip & 1);
                    const float val = o[ot][r] * a.norm;
                    const __bf16 hi = (__bf16)val;
                    const __bf16 lo = (__bf16)(val - (float)hi);
                    __bf16 *dst = lds_x + ((((G * 4 + mu) * 4 + g2) * MX + 2 * m) * 8 + e);
                    dst[0] = hi;
                    dst[8] = lo;
                }
        };
        for (int u = wave; u < rot_units; u += waves) rot_unit(u);
        __syncthreads();
    } else if constexpr (ROT != 0) {
        // Hadamard butterflies over each block of 2^log2b along K, four
        // index bits per pass; a group is 16 values that differ only in the
        // pass's register bits (see fwht_index).
        const int L = ROTL ? ROTL : a.log2b;       // compile-time for 4096-point blocks
        const int tpb = 1 << (L - 4);              // groups per block per pass
        const int ngroups_all = a.M * (a.K >> 4);
        // index bits 0..3 were done at staging; the later passes
        for (int lo = 4; lo < L; lo += 4) {
            const int nrb = (lo + 4 <= L) ? lo : L - 4;
            const int j_lo = lo - nrb, j_hi = (L - nrb < 4) ? L - nrb : 4;
            // with register bits at nrb >= 4 the padded index of value r is
            // base + r * (2^nrb + 2^(nrb - 4)): the register bits carry no
            // part of the low four index bits
            const int cstride = (1 << nrb) + (1 << (nrb - 4));
            for (int q = threadIdx.x; q < ngroups_all; q += nthreads) {
                const int m = a.M == 1 ? 0 : q / wpr, rest = q - m * wpr;
                const int blk = rest >> (L - 4), t = rest & (tpb - 1);
                float *base = rot + (size_t)m * rowpad + fwht_pad((blk << L) + fwht_index(t, 0, nrb));
                float v[16];
                if (nrb >= 4) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) v[r] = base[r * cstride];
                    butterfly_bits(v, j_lo, j_hi);
#pragma unroll
                    for (int r = 0; r < 16; ++r) base[r * cstride] = v[r];
                } else {
                    float *row = rot + (size_t)m * rowpad;
                    const int kb = blk << L;
#pragma unroll
                    for (int r = 0; r < 16; ++r) v[r] = row[fwht_pad(kb + fwht_index(t, r, nrb))];
                    butterfly_bits(v, j_lo, j_hi);
#pragma unroll
                    for (int r = 0; r < 16; ++r) row[fwht_pad(kb + fwht_index(t, r, nrb))] = v[r];
                }
            }
            __syncthreads();
        }
        for (int u = threadIdx.x; u < units; u += nthreads) {
            const int m = u / wpr, wi = u % wpr;
            const float *row = rot + (size_t)m * rowpad + 17 * wi;
            XUnit<XF32> xv;
#pragma unroll
            for (int e = 0; e < 16; ++e) xv.v[e] = __builtin_bit_cast(uint32_t, row[e] * a.norm);
            store_unit<MX, XF32>(lds_x, xv, m, wi);
        }
        __syncthreads();
    }

    // 4. stream the codes
    float yacc[TPW][kRowsOut];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < kRowsOut; ++v) yacc[tp][v] = 0.0f;
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int mu = 0; mu < 4; ++mu) {
        a0[mu] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        a1[mu] = a0[mu];
    }
    const __bf16 *lds_lane = lds_x + (g * MX + arow) * 8;
    constexpr int kGroupStride = 16 * MX * 8;  // bf16 elements per staged group
    constexpr int kMuStride = 4 * MX * 8;
    // AG: A operands of the two groups of a block, loaded one block ahead
    // (binary32 input: the eight raw values, split into a bfloat16 part when
    // they are consumed: A row 2m takes the high part of x[m], row 2m + 1 the
    // remainder, as in the staged image)
    typedef typename std::conditional<XF32, F32x8, bf16x8_t>::type AgT;
    AgT ag[2][8];
    const bool lo_part = XF32 && (arow & 1);
    // lanes whose A row does not exist load the last row of x (always in
    // bounds): their output rows are never stored, and no select or branch is
    // needed per load
    const int xr = a_active ? (XF32 ? arow >> 1 : arow) : a.M - 1;
    const int xcol = 32 * (((g & 1) << 1) | (g >> 1));
    const __bf16 *xrow = static_cast<const __bf16 *>(a.x) + (int64_t)xr * a.K + xcol;
    const float *xrow_f = static_cast<const float *>(a.x) + (int64_t)xr * a.K + xcol;
    auto load_a = [&](int b, int slot) {
        if constexpr (AG) {
            b = b < nblocks ? b : nblocks - 1;
            const int gl0 = g_begin + 2 * b;
            const int gl1 = (gl0 + 1 < g_end) ? gl0 + 1 : gl0;
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                if constexpr (XF32) {
                    ag[slot][mu] = load_f32x8(xrow_f + 128 * gl0 + 8 * mu);
                    ag[slot][4 + mu] = load_f32x8(xrow_f + 128 * gl1 + 8 * mu);
                } else {
                    ag[slot][mu] = *reinterpret_cast<const bf16x8_t *>(xrow + 128 * gl0 + 8 * mu);
                    ag[slot][4 + mu] = *reinterpret_cast<const bf16x8_t *>(xrow + 128 * gl1 + 8 * mu);
                }
            }
        }
    };
    if constexpr (AG) load_a(0, 0);

    // One block: A operands from LDS, consume ring slot p (regroup and flip
    // the code words into fresh registers), refill the slot, then two
    // interleaved 4-MFMA chains per tile (one per 128-K group) and the
    // per-group scaling in binary32.
    auto process = [&](int b, int p, const uint32_t (&sq)[TPW], bool refill) {
        const int gl0 = g_begin + 2 * b;
        const bool two = gl0 + 1 < g_end;
        if constexpr (AG) {
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                if constexpr (XF32) {
                    a0[mu] = split_part(ag[p & 1][mu], lo_part);
                    a1[mu] = split_part(ag[p & 1][4 + mu], lo_part);
                } else {
                    a0[mu] = ag[p & 1][mu];
                    a1[mu] = ag[p & 1][4 + mu];
                }
            }
            load_a(b + 1, (p + 1) & 1);
        } else if (a_active) {
            const __bf16 *pa0 = lds_lane + gl0 * kGroupStride;
            const __bf16 *pa1 = pa0 + (two ? kGroupStride : 0);
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                a0[mu] = *reinterpret_cast<const bf16x8_t *>(pa0 + mu * kMuStride);
                a1[mu] = *reinterpret_cast<const bf16x8_t *>(pa1 + mu * kMuStride);
            }
        }
        unsigned wq[TPW][4];
        float sc[TPW][2];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            auto s02 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][0], cbuf[p][tp][2], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][1], cbuf[p][tp][3], false, false);
            const unsigned flip = AG ? 0u : kFlip;  // the planes apply the flip themselves
            wq[tp][0] = s02[0] ^ flip;  // group 0, operand half 0
            wq[tp][1] = s13[0] ^ flip;  // group 0, operand half 1
            wq[tp][2] = s02[1] ^ flip;  // group 1, operand half 0
            wq[tp][3] = s13[1] ^ flip;  // group 1, operand half 1
            const uint32_t pair = kQuadScales ? quad_scale(sq[tp], p) : sbuf[p][tp];
            sc[tp][0] = half_to_float((uint16_t)(pair & 0xffffu));
            sc[tp][1] = two ? half_to_float((uint16_t)(pair >> 16)) : 0.0f;
        }
        // direct A loads: no refill past the last block (M = 16, 5120 -> 17408:
        // 27.3 -> 25.7 us); the staged path keeps the unconditional clamped
        // re-load, which lets the compiler count outstanding loads exactly
        if (refill && (!AG || b + kDist < nblocks)) load_block(b + kDist, (p + kDist) % PF);
        f32x4_t acc0[TPW], acc1[TPW];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            acc0[tp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc1[tp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (AG) {
            unsigned pl[TPW][4][4];
#pragma unroll
            for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
                for (int w = 0; w < 4; ++w) code_planes(wq[tp][w], kPlaneMask, pl[tp][w]);
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
#pragma unroll
                for (int tp = 0; tp < TPW; ++tp) {
                    acc0[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a0[mu], operand_from_planes(pl[tp][mu >> 1], mu & 1), acc0[tp], 0, 0, 0);
                    acc1[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a1[mu], operand_from_planes(pl[tp][2 + (mu >> 1)], mu & 1), acc1[tp], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
#pragma unroll
                for (int tp = 0; tp < TPW; ++tp) {
                    acc0[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a0[mu], weights_operand(wq[tp][mu >> 1], mu & 1), acc0[tp], 0, 0, 0);
                    acc1[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a1[mu], weights_operand(wq[tp][2 + (mu >> 1)], mu & 1), acc1[tp], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
            for (int v = 0; v < kRowsOut; ++v) {
                yacc[tp][v] = __builtin_fmaf(sc[tp][0], acc0[tp][v], yacc[tp][v]);
                yacc[tp][v] = __builtin_fmaf(sc[tp][1], acc1[tp][v], yacc[tp][v]);
            }
    };

    const int nfull = (nblocks / PF) * PF;
    for (int b0 = 0; b0 < nfull; b0 += PF) {
        uint32_t sq[TPW];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) sq[tp] = squad[tp];
        load_quad_scales(b0 + PF);
#pragma unroll
        for (int p = 0; p < PF; ++p) process(b0 + p, p, sq, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (nfull + p < nblocks) process(nfull + p, p, squad, true);

    // 5. combine the K-waves' partial sums in a fixed order and store
    auto store = [&](int m, int64_t n, float sum) {
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    };
    if (a.wk == 1) {
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const int64_t n = n0 + tp * kTileN + nn;
#pragma unroll
            for (int v = 0; v < kRowsOut; v += (XF32 ? 2 : 1)) {
                const int i = 4 * g + v;
                const int m = XF32 ? i / 2 : i;
                if (m < a.M && n < a.N)
                    store(m, n, XF32 ? yacc[tp][v] + yacc[tp][v + 1] : yacc[tp][v]);
            }
        }
        return;
    }
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < kRowsOut; ++v) {
            const int i = 4 * g + v;
            if (i < MX) red[((wave * TPW + tp) * MX + i) * kTileN + nn] = yacc[tp][v];
        }
    __syncthreads();
    const int outs = a.M * rows_per_wg;
    for (int o = threadIdx.x; o < outs; o += blockDim.x) {
        const int m = o / rows_per_wg;
        const int rem = o - m * rows_per_wg;           // row within the workgroup
        const int twi = rem / (kTileN * TPW);          // tile-wave
        const int tp = (rem / kTileN) % TPW, j = rem % kTileN;
        const int64_t n = n_wg + rem;
        if (n >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < a.wk; ++w) {
            const float *base = red + (((twi * a.wk + w) * TPW + tp) * MX) * kTileN;
            if constexpr (XF32)
                sum += base[(2 * m) * kTileN + j] + base[(2 * m + 1) * kTileN + j];
            else
                sum += base[m * kTileN + j];
        }
        store(m, n, sum);
    }
}

// ---------------------------------------------------------------------------
// Decode GEMV with 5..16 bfloat16 rows: A operands through a shared LDS ring
// ---------------------------------------------------------------------------
//
// From five A rows on, one 256-K block of activations (MX rows x 512 bytes)
// outweighs the codes of a tile's block (1 KiB), so the number of tiles that
// share one fetch of it sets the activation traffic.  A workgroup is WT
// tile-waves x WK K-groups.  The WT waves of a K-group own different tiles
// (TPW each) over the same K range and take their A operands from one LDS
// ring of three 256-K blocks of x, which they fill together by buffer loads
// to LDS two blocks ahead.  A block holds its MX rows in x's own order,
// 32 16-byte chunks of 8 activations per row and one chunk of padding
// (row stride 528 bytes), so that each load instruction (64 lanes, 1 KiB
// of LDS) reads about two rows' contiguous 512 bytes, and the 16 rows of an
// MFMA A operand (one 16-byte LDS read per lane: chunk 16 G + 4 {0, 2, 1,
// 3}[g] + mu of its row, i.e. k = 128 G + 32 {0, 2, 1, 3}[g] + 8 mu + 0..7,
// the order the permlane-regrouped code words give the B operand) fall on
// 16 distinct bank groups.  One barrier per block publishes the block and
// frees the slot read the block before.  Codes and scales stream per wave by raw buffer
// loads, two blocks ahead (rows past N read zero; their outputs are
// dropped).
constexpr unsigned kBufRaw = 0x00020000u;  // raw buffer resource, 32-bit data format
typedef __attribute__((address_space(3))) void lds_void_t;
// s_waitcnt operand: vmcnt(n); expcnt and lgkmcnt not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// One 16-byte buffer load per lane straight into LDS (lane l writes dst +
// 16 l).  A plain device function: with the builtin written inside a kernel
// template, the host pass of this compiler drops the template's launch stub.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}

template <int MX, int TPW, int WT, bool SC4, int KD>
__global__ __launch_bounds__(512) void gemv_ring_kernel(const GemvArgs a)
{
    constexpr int NS = 3;                             // ring slots (blocks of A)
    constexpr int kRowSlots = 33;                     // 16-byte chunks per row: 32 and one of padding
    constexpr int kLoads = ((MX * kRowSlots + 63) / 64 + WT - 1) / WT;  // loads to LDS per lane per block
    constexpr int kChunk = kLoads * WT * 1024;        // LDS bytes of one block of A
    constexpr int PF = 4;                             // code ring slots
    constexpr int kDist = KD;                         // code blocks in flight (<= PF)
    static_assert(KD >= 1 && KD <= PF, "the refill reuses a consumed slot");
    constexpr int kCodeOps = TPW * (SC4 ? 2 : 3);     // loads per code refill
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = a.wk;
    const int kg = wave / WT, tw = wave - kg * WT;
    const int nn = lane & 15, g = lane >> 4;
    const int G = a.K / kGroup;

    const int b_begin = kg * a.bq + (kg < a.br ? kg : a.br);
    const int nblocks = a.bq + (kg < a.br ? 1 : 0);
    const int g_begin = 2 * b_begin;
    const int g_end = (g_begin + 2 * nblocks < G) ? g_begin + 2 * nblocks : G;

    const int rows_per_wg = kTileN * TPW * WT;
    const int64_t n_wg = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t n0 = n_wg + (int64_t)tw * (kTileN * TPW);
    unsigned char *ring = smem + (size_t)kg * NS * kChunk;
    float *red = reinterpret_cast<float *>(smem + (size_t)wk * NS * kChunk);

    // A chunks of this lane: slot p = (tw kLoads + q) 64 + lane of a block is
    // chunk p % 33 of row p / 33.  Rows past M re-read row M - 1; padding
    // slots and slots past the last row re-read a valid chunk (never read
    // back); the second group of a one-group block (odd G) re-reads the
    // first (its scale is zero).
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.x), (short)0, (int)((int64_t)a.M * a.K * 2), (int)kBufRaw);
    int voff[kLoads], voff1[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int p = (tw * kLoads + q) * 64 + lane;
        const int row = p / kRowSlots, c = p - row * kRowSlots;
        const int r = row < a.M ? row : a.M - 1;
        const int cc = c < 32 ? c : 0;
        voff[q] = (r * a.K + 8 * cc) * 2;
        voff1[q] = (r * a.K + 8 * (cc & 15)) * 2;
    }
    auto load_chunk = [&](int s, int slot) {
        const int b = b_begin + (s < nblocks ? s : nblocks - 1);
        const bool one = 2 * b + 1 >= G;
        unsigned char *dst = ring + slot * kChunk + tw * kLoads * 1024;
#pragma unroll
        for (int q = 0; q < kLoads; ++q)
            load_lds16(xrs, dst + 1024 * q, one ? voff1[q] : voff[q], 512 * b);
    };

    // code and scale streams of this wave's rows
    const int64_t left = a.N - n0;
    const int rows_here = left <= 0 ? 0 : (left < kTileN * TPW ? (int)left : kTileN * TPW);
    const int row_bytes = a.K / 4;
    const int64_t nb = rows_here > 0 ? n0 : 0;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.codes + nb * (a.K / 16)), (short)0, rows_here * row_bytes, (int)kBufRaw);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scales + nb * G), (short)0, rows_here * G * 2, (int)kBufRaw);
    u32x4_t cbuf[PF][TPW];
    uint32_t sbuf[PF][TPW];
    // block b: words 4 g .. 4 g + 3 of its 256 K; a one-group block's upper
    // lane groups re-read the first group
    auto load_block = [&](int b, int p) {
        b = b < nblocks ? b : nblocks - 1;
        const int gb = g_begin + 2 * b;
        const bool two = gb + 1 < g_end;
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const int rowoff = (tp * kTileN + nn) * row_bytes;
            cbuf[p][tp] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, rowoff + 16 * (two ? g : (g & 1)), 32 * gb, 0));
            const int so = (tp * kTileN + nn) * G * 2;
            if constexpr (SC4)
                sbuf[p][tp] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 2 * gb, 0);
            else
                sbuf[p][tp] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, so, 2 * gb, 0) |
                              ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, so, 2 * (two ? gb + 1 : gb), 0)
                               << 16);
        }
    };

    float yacc[TPW][4];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < 4; ++v) yacc[tp][v] = 0.0f;
    // this lane's A operand within a slot: chunk 4 {0, 2, 1, 3}[g] + mu of
    // group gl of its row (rows past MX read a row below MX; their outputs
    // are dropped)
    const int arow = nn & (MX - 1);
    const int a_lane = (arow * kRowSlots + 4 * (((g & 1) << 1) | (g >> 1))) * 16;

    auto process = [&](int b, int p, int slot) {
        const int gl0 = g_begin + 2 * b;
        const bool two = gl0 + 1 < g_end;
        const unsigned char *sl = ring + slot * kChunk + a_lane;
        bf16x8_t a0[4], a1[4];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
            a0[mu] = *reinterpret_cast<const bf16x8_t *>(sl + mu * 16);
            a1[mu] = *reinterpret_cast<const bf16x8_t *>(sl + (16 + mu) * 16);
        }
        unsigned wq[TPW][4];
        float sc[TPW][2];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            auto s02 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][0], cbuf[p][tp][2], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(cbuf[p][tp][1], cbuf[p][tp][3], false, false);
            wq[tp][0] = s02[0];  // group 0, operand half 0 (the planes apply the slot flip)
            wq[tp][1] = s13[0];
            wq[tp][2] = s02[1];  // group 1
            wq[tp][3] = s13[1];
            const uint32_t pair = sbuf[p][tp];
            sc[tp][0] = half_to_float((uint16_t)(pair & 0xffffu));
            sc[tp][1] = two ? half_to_float((uint16_t)(pair >> 16)) : 0.0f;
        }
        load_block(b + kDist, (p + kDist) % PF);  // unconditional (clamped): exact load counts
        f32x4_t acc0[TPW], acc1[TPW];
        unsigned pl[TPW][4][4];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            acc0[tp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc1[tp] = acc0[tp];
#pragma unroll
            for (int w = 0; w < 4; ++w) code_planes(wq[tp][w], kPlaneMask, pl[tp][w]);
        }
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int tp = 0; tp < TPW; ++tp) {
                acc0[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[mu], operand_from_planes(pl[tp][mu >> 1], mu & 1),
                                                                   acc0[tp], 0, 0, 0);
                acc1[tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a1[mu], operand_from_planes(pl[tp][2 + (mu >> 1)], mu & 1), acc1[tp], 0, 0, 0);
            }
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                yacc[tp][v] = __builtin_fmaf(sc[tp][0], acc0[tp][v], yacc[tp][v]);
                yacc[tp][v] = __builtin_fmaf(sc[tp][1], acc1[tp][v], yacc[tp][v]);
            }
    };

    // One step: wait until this wave's loads of block s have landed (issued
    // after them: two code refills and the loads of block s + 1), publish
    // it with a barrier (which also says every wave is done reading the slot
    // of block s - 1), refill that slot with block s + 2 (past the last block
    // the last one again: the loads stay unconditional, so that the counts
    // here and the compiler's own waits are exact), then compute block s.
    auto step = [&](int s, int p, bool compute) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCodeOps + kLoads));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(s + 2, (s + 2) % NS);
        __builtin_amdgcn_sched_barrier(0);
        if (compute) process(s, p, s % NS);
    };

    // prologue: blocks 0 and 1 of A, then of the codes
    load_chunk(0, 0);
    load_chunk(1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < kDist; ++p) load_block(p, p);
    __builtin_amdgcn_sched_barrier(0);

    // every K-group has at least bq blocks: those steps run unconditionally,
    // unrolled by PF so that the code ring slot is a constant; the first br
    // K-groups then have one more
    const int nfull = (a.bq / PF) * PF;
    for (int s0 = 0; s0 < nfull; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) step(s0 + p, p, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (nfull + p < a.bq) step(nfull + p, p, true);
    if (a.br > 0) {
        const bool mine = kg < a.br;
        switch (a.bq % PF) {
        case 0: step(a.bq, 0, mine); break;
        case 1: step(a.bq, 1, mine); break;
        case 2: step(a.bq, 2, mine); break;
        default: step(a.bq, 3, mine); break;
        }
    }
    // every load to LDS has landed before the workgroup's LDS is reused
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    // combine the K-groups' partial sums in a fixed order and store
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 4 * g + v;
            if (i < MX) red[(((tw * wk + kg) * TPW + tp) * MX + i) * kTileN + nn] = yacc[tp][v];
        }
    __syncthreads();
    const int outs = a.M * rows_per_wg;
    for (int o = threadIdx.x; o < outs; o += blockDim.x) {
        const int m = o / rows_per_wg, rem = o - m * rows_per_wg;
        const int twi = rem / (kTileN * TPW), tp = (rem / kTileN) % TPW, j = rem % kTileN;
        const int64_t n = n_wg + rem;
        if (n >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < wk; ++w) sum += red[(((twi * wk + w) * TPW + tp) * MX + m) * kTileN + j];
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    }
}

// ---------------------------------------------------------------------------
// Signed normalized Walsh-Hadamard transform
// ---------------------------------------------------------------------------
//
// Natural (Sylvester) order: H[i][l] = (-1)^popcount(i & l), so the
// transform is a butterfly (a, c) -> (a + c, a - c) over every index bit.
// For blocks of b = 2^L >= 16 elements a workgroup handles BPW blocks of one
// row with b/16 threads per block; each thread holds 16 values whose index
// differs in four "register bits" and applies the butterflies over those bits
// in registers.  Between passes the values go through LDS so that the next
// four index bits become register bits.  LDS index i is padded to
// i + i / 16, which keeps the strided transposes free of bank conflicts.
// binary32 throughout; the 1/sqrt(b) factor is applied once at the end (a
// power of two, so exact, when L is even).

template <bool XF32>
__global__ __launch_bounds__(256) void fwht16_kernel(
    const void *__restrict__ x, const int8_t *__restrict__ signs, int64_t M, int64_t K, int L,
    int bpw, int inverse, float *y, float norm)
{
    extern __shared__ float buf[];
    const int b = 1 << L;
    const int tpb = b >> 4;                       // threads per block
    const int jb = threadIdx.x / tpb;             // block within the workgroup
    const int t = threadIdx.x - jb * tpb;         // thread within the block
    const int64_t blocks_per_row = K >> L;
    const int64_t blk = (int64_t)blockIdx.x * bpw + jb;
    const bool live = jb < bpw && blk < blocks_per_row;
    const int64_t sbase = (blk < blocks_per_row ? blk : 0) << L;
    float *lb = buf + (size_t)jb * fwht_pad(b);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float v[16];
        const int64_t base = m * K + sbase + 16 * t;
        if (live) {
            if constexpr (XF32) {
                const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + base);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 f = src[q];
                    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
                }
            } else {
                const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(x) + base);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u32x4_t d = src[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[8 * q + 2 * e] = bf16_to_float((uint16_t)(d[e] & 0xffffu));
                        v[8 * q + 2 * e + 1] = bf16_to_float((uint16_t)(d[e] >> 16));
                    }
                }
            }
            if (!inverse && signs) {
                const u32x4_t d = *reinterpret_cast<const u32x4_t *>(signs + sbase + 16 * t);
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = flip_if(v[r], sign_bit(d[r >> 2], r & 3));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = 0.0f;
        }
        // pass 0: register bits = index bits 0..3
        butterfly_bits(v, 0, 4);
        int rb = 0;
        for (int lo = 4; lo < L; lo += 4) {
            const int nrb = (lo + 4 <= L) ? lo : L - 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) lb[fwht_pad(fwht_index(t, r, rb))] = v[r];
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = lb[fwht_pad(fwht_index(t, r, nrb))];
            __syncthreads();
            butterfly_bits(v, lo - nrb, L - nrb < 4 ? L - nrb : 4);
            rb = nrb;
        }
        if (live) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = fwht_index(t, r, rb);
                float o = v[r] * norm;
                if (inverse && signs) o = flip_if(o, sign_bit((uint32_t)(uint8_t)signs[sbase + i], 0));
                y[m * K + sbase + i] = o;
            }
        }
    }
}

// Blocks of 4096: one workgroup of four waves per block and row, the block
// staged once in LDS (d .* x forward, x inverse) and transformed on the
// matrix cores, one 16-column slice per wave (h64_slice); y = result / 64
// (times d for the inverse).  Every read of the block precedes the barrier
// and every write follows it, so y may alias binary32 x.
template <bool XF32>
__global__ __launch_bounds__(256) void fwht4096_kernel(const void *__restrict__ x, const int8_t *__restrict__ signs,
                                                       int64_t M, int64_t K, int inverse, float *y, float norm)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int kPadX = XF32 ? 68 : 72;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4, t = threadIdx.x;
    const int64_t k0 = (int64_t)blockIdx.x << 12;  // first element of this block in the row
    const bool pre = signs && !inverse;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        // thread t stages elements 16 t .. 16 t + 15: row t >> 2 of X, columns 16 (t & 3) ..
        const int64_t base = m * K + k0 + 16 * t;
        const u32x4_t dw = pre ? *reinterpret_cast<const u32x4_t *>(signs + k0 + 16 * t)
                               : u32x4_t{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
        const int at = (t >> 2) * kPadX + 16 * (t & 3);
        if constexpr (XF32) {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(x) + base);
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(reinterpret_cast<uint32_t *>(smem) + at);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4_t v = src[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] ^= ((dw[q] >> (8 * e + 7)) & 1u) << 31;
                dst[q] = v;
            }
        } else {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(x) + base);
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(smem) + at);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u32x4_t v = src[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int w = 4 * q + e;  // bfloat16 pair 2w, 2w + 1 of the 16
                    const uint32_t sel = (w & 1) ? 0x030C020Cu : 0x010C000Cu;  // sign bytes -> bytes 1, 3
                    v[e] ^= __builtin_amdgcn_perm(0u, dw[w >> 1], sel) & 0x80008000u;
                }
                dst[q] = v;
            }
        }
        __syncthreads();
        f32x4_t o[4];
        h64_slice<XF32>(smem, wave, c, g, o);
        // lane holds X'[16 ot + 4 g + r][16 wave + c]: element 64 (16 ot + 4 g + r) + 16 wave + c
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 64 * (16 * ot + 4 * g + r) + 16 * wave + c;
                float v = o[ot][r] * norm;
                if (inverse && signs) v = flip_if(v, sign_bit((uint32_t)(uint8_t)signs[k0 + i], 0));
                y[m * K + k0 + i] = v;
            }
        __syncthreads();  // the next row's staging reuses the LDS block
    }
}

// Blocks of fewer than 16 elements: one thread per block, in registers.
template <bool XF32>
__global__ __launch_bounds__(256) void fwht_small_kernel(
    const void *__restrict__ x, const int8_t *__restrict__ signs, int64_t M, int64_t K, int L,
    int inverse, float *y, float norm)
{
    const int b = 1 << L;
    const int64_t total = M * (K >> L);
    for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < total;
         blk += (int64_t)gridDim.x * blockDim.x) {
        const int64_t base = blk << L;
        const int64_t sb = base % K;
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            v[r] = 0.0f;
            if (r < b) {
                v[r] = XF32 ? static_cast<const float *>(x)[base + r]
                            : bf16_to_float(static_cast<const uint16_t *>(x)[base + r]);
                if (!inverse && signs) v[r] = flip_if(v[r], sign_bit((uint32_t)(uint8_t)signs[sb + r], 0));
            }
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (j >= L) continue;
            const int h = 1 << j;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if ((r & h) || r >= b) continue;
                const float a = v[r], c = v[r | h];
                v[r] = a + c;
                v[r | h] = a - c;
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r < b) {
                float o = v[r] * norm;
                if (inverse && signs) o = flip_if(o, sign_bit((uint32_t)(uint8_t)signs[sb + r], 0));
                y[base + r] = o;
            }
        }
    }
}

struct GemvPlan {
    int tpw, wk, wt;
    int64_t wgs;
    size_t lds;
    bool ag;  // A operand straight from global memory (no staged x)
};

// Tiles per wave and the split of a workgroup's waves between tiles (wt)
// and K (wk), from sweeps of the decode shapes on MI355X: one tile per wave,
// except two when the staged activations of a workgroup are large (then
// fewer workgroups stage them); two tile-waves x two K-waves for many tiles,
// otherwise four K-waves, or eight for long rows (each K-wave with at least
// two 256-K blocks).
inline GemvPlan plan_gemv(int64_t N, int64_t K, int mx)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    GemvPlan pl;
    pl.tpw = K * mx * 2 >= 96 * 1024 ? 2 : 1;
    const int64_t tile_groups = (tiles + pl.tpw - 1) / pl.tpw;
    pl.wt = tile_groups >= 1024 ? 2 : 1;
    pl.wk = 4 / pl.wt;
    // long rows (32 or more blocks): eight K-waves, each with half the serial
    // block chain (17408 -> 5120: 12.4 -> 11.5 us at M = 1, 14.7 -> 13.6 at M = 4)
    if (pl.wt == 1 && nblk >= 32) pl.wk = 8;
    while (pl.wk > 1 && nblk < 2 * pl.wk) pl.wk /= 2;
    pl.wgs = (tile_groups + pl.wt - 1) / pl.wt;
    const int waves = pl.wt * pl.wk;
    pl.lds = (size_t)K * mx * 2 + (size_t)waves * pl.tpw * mx * kTileN * sizeof(float);
    pl.ag = false;
    return pl;
}

// bfloat16 activations with eight or more A rows (or a staged image too large
// for LDS): direct A loads, so LDS does not cap the workgroups per CU.  Two
// tiles per wave (four spill registers) and two K-waves, four for long rows,
// from sweeps of tiles per wave x tile-waves x K-waves at M = 8 and 16.
inline GemvPlan plan_gemv_ag(int64_t N, int64_t K, int mx, bool x_f32)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    GemvPlan pl;
    pl.tpw = x_f32 ? 1 : 2;  // binary32 operands in flight take twice the registers
    const int64_t tile_groups = (tiles + pl.tpw - 1) / pl.tpw;
    pl.wt = 1;
    pl.wk = nblk >= 32 ? 4 : 2;  // 5120 -> 17408: 21.3 -> 20.5 us at M = 8
    while (pl.wk > 1 && nblk < 2 * pl.wk) pl.wk /= 2;
    pl.wgs = (tile_groups + pl.wt - 1) / pl.wt;
    pl.lds = (size_t)pl.wt * pl.wk * pl.tpw * mx * kTileN * sizeof(float);
    pl.ag = true;
    return pl;
}

// Whether the tiled kernel's workgroups (bfloat16 x, M <= 4) would leave the
// busiest CU more than 5% above the average: then the even-split kernel
// (tern_gemv1.hip) runs instead.  Measured at M = 1: 17408 -> 5120, 320
// tiles, 11.7 -> 9.7 us; 5120 -> 34816, 1088 workgroups, 15.8 -> 14.0 us;
// 4096 -> 12288, 768 workgroups (three per CU), tiled 7.0 us against 7.3.
inline bool gemv_tiles_uneven(int64_t N, int64_t K, int M)
{
    const int mx = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    const GemvPlan pl = plan_gemv(N, K, mx);
    const int64_t cus = device_cus();
    const int64_t rounds = (pl.wgs + cus - 1) / cus;
    return (double)rounds * (double)cus > 1.05 * (double)pl.wgs;
}

template <int MX, bool XF32, int TPW>
int launch_gemv_t(GemvArgs a, const GemvPlan &pl, hipStream_t stream)
{
    // scale pairs as one 4-byte load: G even and the scales 4-byte aligned
    // (the ABI asks only for 2)
    const bool sc4 = (a.K / kGroup) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.scales) % 4) == 0;
    void (*kernel)(GemvArgs) = sc4 ? gemv_kernel<MX, XF32, TPW, true> : gemv_kernel<MX, XF32, TPW, false>;
    // binary32 direct loads run one tile per wave (two would spill registers)
    if constexpr (!(XF32 && TPW > 1))
        if (pl.ag)
            kernel = sc4 ? gemv_kernel<MX, XF32, TPW, true, 0, 0, true> : gemv_kernel<MX, XF32, TPW, false, 0, 0, true>;
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    a.wk = pl.wk;
    a.wt = pl.wt;
    a.bq = a.nblk / pl.wk;
    a.br = a.nblk % pl.wk;
    if ((rc = check_block(64 * pl.wk * pl.wt, 512))) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * pl.wk * pl.wt), pl.lds, stream, a);
    return (int)hipGetLastError();
}

template <int MX, bool XF32>
int launch_gemv_mx(const GemvArgs &a, const GemvPlan &pl, hipStream_t stream)
{
    switch (pl.tpw) {
    case 1: return launch_gemv_t<MX, XF32, 1>(a, pl, stream);
    case 2: return launch_gemv_t<MX, XF32, 2>(a, pl, stream);
    default: return (int)hipErrorInvalidValue;  // plans use one or two tiles per wave
    }
}

// bfloat16 activations with 5..16 rows: the A ring (gemv_ring_kernel), two
// tiles per wave, codes two blocks ahead.  From a sweep of tile-waves (1, 2,
// 4) x K-groups (1..4) x code blocks in flight (2..4) on the decode shapes:
// one tile-wave, except two at 16 rows where that still leaves a workgroup
// per CU (5120 -> 17408: 21.5 -> 19.7 us); two K-groups, four for long rows
// (17408 -> 5120 at 16 rows: 24.4 -> 20.1 us); more code blocks in flight
// were slower.  Short rows (under 32 blocks) with two or more workgroups per
// CU run one wave per workgroup over all of K instead.  Workgroups stay
// within the kernel's 512 threads (64 wt wk).
struct RingPlan {
    int wt, wk;
    int64_t wgs;
    size_t lds;
};
constexpr int kRingTpw = 2;

inline bool plan_gemv_ring(int64_t N, int64_t K, int M, int mx, RingPlan &pl)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    if (K == 0 || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
    const int64_t wgs1 = (tiles + kRingTpw - 1) / kRingTpw;  // workgroups of one tile-wave
    if (nblk < 32 && wgs1 >= 2 * device_cus()) {
        // short rows and two or more workgroups per CU: one wave each, the
        // whole K range (5120 -> 17408: 16.2 -> 15.3 us at M = 8, 19.7 -> 18.8
        // at M = 16)
        pl.wt = 1;
        pl.wk = 1;
    } else {
        pl.wt = (mx == 16 && (tiles + 2 * kRingTpw - 1) / (2 * kRingTpw) >= device_cus()) ? 2 : 1;
        pl.wk = nblk >= 32 ? 4 : 2;
        while (pl.wk > 1 && nblk < 2 * pl.wk) pl.wk /= 2;
    }
    pl.wgs = (tiles + kRingTpw * pl.wt - 1) / (kRingTpw * pl.wt);
    const int loads = ((mx * 33 + 63) / 64 + pl.wt - 1) / pl.wt;  // as in gemv_ring_kernel
    pl.lds = (size_t)pl.wk * 3 * loads * pl.wt * 1024 + (size_t)pl.wt * pl.wk * kRingTpw * mx * kTileN * sizeof(float);
    return pl.lds <= kMaxLds;
}

template <int MX, int WT, int KD>
int launch_gemv_ring(GemvArgs a, const RingPlan &pl, hipStream_t stream)
{
    const bool sc4 = (a.K / kGroup) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.scales) % 4) == 0;
    void (*kernel)(GemvArgs) =
        sc4 ? gemv_ring_kernel<MX, kRingTpw, WT, true, KD> : gemv_ring_kernel<MX, kRingTpw, WT, false, KD>;
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    a.wk = pl.wk;
    a.wt = WT;
    a.bq = a.nblk / pl.wk;
    a.br = a.nblk % pl.wk;
    if ((rc = check_block(64 * WT * pl.wk, 512))) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * WT * pl.wk), pl.lds, stream, a);
    return (int)hipGetLastError();
}

template <bool XF32>
int launch_gemv_x(GemvArgs a, hipStream_t stream)
{
    const int Mx = XF32 ? 2 * a.M : a.M;
    const int mx = Mx <= 1 ? 1 : Mx <= 2 ? 2 : Mx <= 4 ? 4 : Mx <= 8 ? 8 : 16;
    if constexpr (!XF32) {
        RingPlan rp;
        if (mx >= 8 && plan_gemv_ring(a.N, a.K, a.M, mx, rp)) {
            if (mx == 8) return launch_gemv_ring<8, 1, 2>(a, rp, stream);
            return rp.wt == 2 ? launch_gemv_ring<16, 2, 2>(a, rp, stream) : launch_gemv_ring<16, 1, 2>(a, rp, stream);
        }
    }
    GemvPlan pl = plan_gemv(a.N, a.K, mx);
    // direct A loads: bfloat16 with eight or more A rows that the ring does
    // not take (M K at or above 2^30 elements), or any input whose staged
    // image would not fit in LDS
    if ((!XF32 && mx >= 8) || pl.lds > kMaxLds) pl = plan_gemv_ag(a.N, a.K, mx, XF32);
    switch (mx) {
    case 1: return launch_gemv_mx<1, XF32>(a, pl, stream);
    case 2: return launch_gemv_mx<2, XF32>(a, pl, stream);
    case 4: return launch_gemv_mx<4, XF32>(a, pl, stream);
    case 8: return launch_gemv_mx<8, XF32>(a, pl, stream);
    default: return launch_gemv_mx<16, XF32>(a, pl, stream);
    }
}


// Fused rotation: every workgroup transforms the activations once, so use
// about one workgroup per CU (up to four tiles per wave) and split K over
// up to four waves (all of them take part in the transform).  From a sweep
// of tiles per wave (1..4) x K-waves (1..8) on the rotated decode shape.
inline GemvPlan plan_rotate_gemv(int64_t N, int64_t K, int M, int mx)
{
    const int64_t tiles = (N + kTileN - 1) / kTileN;
    const int nblk = (int)((K / kGroup + 1) / 2);
    const int cus = device_cus();
    GemvPlan pl;
    int64_t t = (tiles + cus - 1) / cus;
    pl.tpw = (int)(t < 1 ? 1 : (t > 4 ? 4 : t));
    pl.wt = 1;
    pl.wgs = (tiles + pl.tpw - 1) / pl.tpw;
    pl.wk = 1;
    while (pl.wk < 4 && nblk >= 2 * (pl.wk * 2)) pl.wk *= 2;
    pl.lds = (size_t)K * mx * 2 + (size_t)M * (K + K / 16) * 4 +
             (size_t)pl.wk * pl.tpw * mx * kTileN * sizeof(float);
    return pl;
}

template <int MX, int ROT, int ROTL>
void (*rotate_kernel(int tpw, bool sc4))(GemvArgs)
{
    switch (tpw) {
    case 1: return sc4 ? gemv_kernel<MX, true, 1, true, ROT, ROTL> : gemv_kernel<MX, true, 1, false, ROT, ROTL>;
    case 2: return sc4 ? gemv_kernel<MX, true, 2, true, ROT, ROTL> : gemv_kernel<MX, true, 2, false, ROT, ROTL>;
    case 3: return sc4 ? gemv_kernel<MX, true, 3, true, ROT, ROTL> : gemv_kernel<MX, true, 3, false, ROT, ROTL>;
    default: return sc4 ? gemv_kernel<MX, true, 4, true, ROT, ROTL> : gemv_kernel<MX, true, 4, false, ROT, ROTL>;
    }
}

template <int MX, int ROT>
int launch_rotate_t(GemvArgs a, const GemvPlan &pl, hipStream_t stream)
{
    const bool sc4 = (a.K / kGroup) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.scales) % 4) == 0;
    void (*kernel)(GemvArgs) = a.log2b == 12 ? rotate_kernel<MX, ROT, 12>(pl.tpw, sc4)
                                             : rotate_kernel<MX, ROT, 0>(pl.tpw, sc4);
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    a.wk = pl.wk;
    a.wt = pl.wt;
    a.bq = a.nblk / pl.wk;
    a.br = a.nblk % pl.wk;
    if ((rc = check_block(64 * pl.wk, 512))) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * pl.wk), pl.lds, stream, a);
    return (int)hipGetLastError();
}

// Rows of x one launch takes: the staged activations (2 bytes per K per A
// row, two A rows per binary32 input row) must fit in LDS; larger M runs as
// several launches over the same weights.
inline int gemv_rows_per_launch(int64_t N, int64_t K, bool x_f32)
{
    if (!x_f32) return 16;  // bfloat16: direct A loads where the staged image would not fit
    const int per = 2;
    for (int rows = 16 / per; rows >= 1; rows /= 2)
        if (plan_gemv(N, K, rows * per).lds <= kMaxLds) return rows;
    return 16 / per;  // not even one row fits: direct A loads, eight rows per launch
}

// ---------------------------------------------------------------------------
// Device packer: int8 t in {-1, 0, +1} -> 2-bit slots q = t + 1
// ---------------------------------------------------------------------------
// One thread per code word: a 16-byte load of the word's 16 weights, slot j
// of the word at bits 2j..2j + 1.  Values outside {-1, 0, 1} are not checked
// (their slots are unspecified).
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ t, uint32_t *__restrict__ codes,
                                                   int64_t words)
{
    for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += (int64_t)gridDim.x * 256) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(t + 16 * w);
        uint32_t code = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tv = (int8_t)((v[j >> 2] >> (8 * (j & 3))) & 0xffu);
            code |= (uint32_t)((tv + 1) & 3) << (2 * j);
        }
        codes[w] = code;
    }
}

}  // namespace

namespace tern {

int launch_pack_device(const int8_t *t, int64_t N, int64_t K, uint32_t *codes, void *stream)
{
    const int64_t words = N * (K / 16);
    if (words == 0) return 0;
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), t, codes, words);
    return (int)hipGetLastError();
}


const char *hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

int launch_gemv(const void *x, bool x_f32, int M, int64_t K, const uint32_t *codes,
                const uint16_t *scales, int64_t N, void *y, bool y_bf16, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!x_f32 && M <= 4 && gemv_tiles_uneven(N, K, M) && tern::gemv1_applies(M, N, K))
        return tern::launch_gemv1(x, M, K, codes, scales, N, y, y_bf16, false, stream);
    const int step = gemv_rows_per_launch(N, K, x_f32);
    const size_t xsz = x_f32 ? 4 : 2, ysz = y_bf16 ? 2 : 4;
    for (int m0 = 0; m0 < M; m0 += step) {
        GemvArgs a;
        a.M = (M - m0) < step ? (M - m0) : step;
        a.x = static_cast<const char *>(x) + (size_t)m0 * K * xsz;
        a.y = static_cast<char *>(y) + (size_t)m0 * N * ysz;
        a.codes = codes;
        a.scales = scales;
        a.N = N;
        a.K = (int)K;
        a.nblk = (int)((K / kGroup + 1) / 2);
        a.bq = a.br = 0;
        a.y_bf16 = y_bf16 ? 1 : 0;
        a.signs = nullptr;
        a.log2b = 0;
        a.norm = 1.0f;
        int rc = x_f32 ? launch_gemv_x<true>(a, st) : launch_gemv_x<false>(a, st);
        if (rc) return rc;
    }
    return 0;
}

// Rotated activations are staged as hi/lo rows, two A rows per input row,
// so one launch takes at most 8 rows of x; larger M runs as several.
constexpr int kRotRowsPerLaunch = 8;

size_t rotate_gemv_lds(int64_t M, int64_t N, int64_t K)
{
    const int64_t mm = M < kRotRowsPerLaunch ? M : kRotRowsPerLaunch;
    const int mx = 2 * mm <= 2 ? 2 : 2 * mm <= 4 ? 4 : 2 * mm <= 8 ? 8 : 16;
    return plan_rotate_gemv(N, K, (int)mm, mx).lds;
}

size_t max_lds_bytes() { return kMaxLds; }

static int launch_rotate_rows(const void *x, bool x_f32, const int8_t *signs, int block, int M, int64_t K,
                              const uint32_t *codes, const uint16_t *scales, int64_t N, void *y,
                              bool y_bf16, hipStream_t st)
{
    GemvArgs a;
    a.x = x;
    a.codes = codes;
    a.scales = scales;
    a.y = y;
    a.N = N;
    a.K = (int)K;
    a.M = M;
    a.nblk = (int)((K / kGroup + 1) / 2);
    a.wk = a.wt = 1;
    a.bq = a.br = 0;
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.signs = signs;
    int L = 0;
    while ((1 << L) < block) ++L;
    a.log2b = L;
    a.norm = (float)(1.0 / __builtin_sqrt((double)block));
    const int mx = 2 * M <= 2 ? 2 : 2 * M <= 4 ? 4 : 2 * M <= 8 ? 8 : 16;
    const GemvPlan pl = plan_rotate_gemv(N, K, M, mx);
    switch (mx) {
    case 2: return x_f32 ? launch_rotate_t<2, 2>(a, pl, st) : launch_rotate_t<2, 1>(a, pl, st);
    case 4: return x_f32 ? launch_rotate_t<4, 2>(a, pl, st) : launch_rotate_t<4, 1>(a, pl, st);
    case 8: return x_f32 ? launch_rotate_t<8, 2>(a, pl, st) : launch_rotate_t<8, 1>(a, pl, st);
    default: return x_f32 ? launch_rotate_t<16, 2>(a, pl, st) : launch_rotate_t<16, 1>(a, pl, st);
    }
}

bool rotate_gemv_fits(int64_t M, int64_t N, int64_t K, int64_t block, bool x_f32)
{
    return rotate_gemv_lds(M, N, K) <= kMaxLds;
}

int launch_rotate_gemv(const void *x, bool x_f32, const int8_t *signs, int block, int M, int64_t K,
                       const uint32_t *codes, const uint16_t *scales, int64_t N, void *y, bool y_bf16,
                       void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t xsz = x_f32 ? 4 : 2, ysz = y_bf16 ? 2 : 4;
    for (int m0 = 0; m0 < M; m0 += kRotRowsPerLaunch) {
        const int mm = (M - m0) < kRotRowsPerLaunch ? (M - m0) : kRotRowsPerLaunch;
        int rc = launch_rotate_rows(static_cast<const char *>(x) + (size_t)m0 * K * xsz, x_f32, signs, block,
                                    mm, K, codes, scales, N, static_cast<char *>(y) + (size_t)m0 * N * ysz,
                                    y_bf16, st);
        if (rc) return rc;
    }
    return 0;
}

int launch_fwht(const void *x, bool x_f32, const int8_t *signs, int64_t M, int64_t K, int block,
                bool inverse, float *y, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    int L = 0;
    while ((1 << L) < block) ++L;
    const float norm = (float)(1.0 / __builtin_sqrt((double)block));
    const unsigned rows = (unsigned)(M < 65535 ? M : 65535);
    if (L == 12) {
        // one workgroup per 4096-point block and row
        const size_t lds = x_f32 ? 64 * 68 * sizeof(float) : 64 * 72 * sizeof(uint16_t);
        dim3 grid((unsigned)(K >> 12), rows);
        if (x_f32)
            hipLaunchKernelGGL(fwht4096_kernel<true>, grid, dim3(256), lds, st, x, signs, M, K, (int)inverse, y, norm);
        else
            hipLaunchKernelGGL(fwht4096_kernel<false>, grid, dim3(256), lds, st, x, signs, M, K, (int)inverse, y, norm);
        return (int)hipGetLastError();
    }
    if (L < 4) {
        const int64_t total = M * (K >> L);
        const unsigned grid = (unsigned)((total + 255) / 256 < 65535 * 16 ? (total + 255) / 256 : 65535 * 16);
        if (x_f32)
            hipLaunchKernelGGL(fwht_small_kernel<true>, dim3(grid), dim3(256), 0, st, x, signs, M, K, L,
                               (int)inverse, y, norm);
        else
            hipLaunchKernelGGL(fwht_small_kernel<false>, dim3(grid), dim3(256), 0, st, x, signs, M, K, L,
                               (int)inverse, y, norm);
        return (int)hipGetLastError();
    }
    const int tpb = block / 16;
    const int64_t blocks_per_row = K / block;
    int bpw = 256 / tpb;
    if (bpw > blocks_per_row) bpw = (int)blocks_per_row;
    if (bpw < 1) bpw = 1;
    const unsigned threads = (unsigned)(((tpb * bpw + 63) / 64) * 64);
    // every thread, including padding threads past bpw blocks, owns an LDS
    // block region (padding threads load nothing and store nothing)
    const size_t lds = (size_t)(threads / tpb) * (block + block / 16) * sizeof(float);
    dim3 grid((unsigned)((blocks_per_row + bpw - 1) / bpw), rows);
    if (x_f32)
        hipLaunchKernelGGL(fwht16_kernel<true>, grid, dim3(threads), lds, st, x, signs, M, K, L, bpw,
                           (int)inverse, y, norm);
    else
        hipLaunchKernelGGL(fwht16_kernel<false>, grid, dim3(threads), lds, st, x, signs, M, K, L, bpw,
                           (int)inverse, y, norm);
    return (int)hipGetLastError();
}

}  // namespace tern
