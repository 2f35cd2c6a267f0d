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

#include "tern_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

constexpr int kGroup = 128;          // weights per scale
constexpr int kWordsPerGroup = 8;    // 16 slots per uint32
constexpr int kTileN = 16;           // output rows per MFMA tile
constexpr unsigned kFlip = 0x55555555u;

// Packed bfloat16 pair holding -2t for slot j (low half) and slot j + 8
// (high half) of a flipped code word.
__device__ __forceinline__ unsigned neg2t_pair(unsigned flipped, int j)
{
    u16x2_t v = __builtin_bit_cast(u16x2_t, flipped);
    v = (v >> (unsigned short)(2 * j)) << (unsigned short)14;
    return __builtin_bit_cast(unsigned, v);
}

// MFMA B operand (8 bf16) from half h (slots 4h..4h+3 and 4h+8..4h+11) of a
// flipped word.  Element e corresponds to slot 4h + (e >> 1) + 8 (e & 1).
__device__ __forceinline__ bf16x8_t weights_operand(unsigned flipped, int h)
{
    u32x4_t p;
    p[0] = neg2t_pair(flipped, 4 * h + 0);
    p[1] = neg2t_pair(flipped, 4 * h + 1);
    p[2] = neg2t_pair(flipped, 4 * h + 2);
    p[3] = neg2t_pair(flipped, 4 * h + 3);
    return __builtin_bit_cast(bf16x8_t, p);
}

__device__ __forceinline__ float half_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b)
{
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// ---------------------------------------------------------------------------
// GEMV for M <= 16
// ---------------------------------------------------------------------------
//
// Work decomposition.  A workgroup owns TPW consecutive 16-row tiles and the
// whole K; its W waves split K into contiguous ranges of whole 128-K groups
// and the partial sums are combined in LDS in a fixed order at the end (so
// the result is deterministic).  Within a wave, lane l serves output row
// n0 + 16*tile + (l & 15) and lane group g = l >> 4 (the MFMA k-slot group).
//
// Codes.  Per 256-K block (two groups) each lane loads one 16-byte vector:
// words 4g..4g+3 of its row's 64-byte block segment, so the four lanes of a
// row read 64 contiguous bytes.  A v_permlane32_swap pair then regroups the
// words so that every lane holds two words of group 0 and two of group 1
// (the MFMA contracts over all four lane groups, which must therefore see
// the same scale group).  After the swap, word w of a group sits in lane
// group G(w) = {0, 2, 1, 3}[w >> 1] as operand half w & 1.
//
// Activations.  The MFMA A operand is x: row i = l & 15 of A is activation
// row i (bfloat16 input) or, for binary32 input, rows 2m / 2m + 1 hold the
// bfloat16 high part and the bfloat16 remainder of x[m] (x - hi is exact in
// binary32 and the two parts together carry 16 significand bits).  Each
// wave stages the activations of its K range in LDS, permuted so that one
// 16-byte LDS read gives a lane its A operand for one MFMA; rows that do not
// exist read nothing and stay zero.
//
// LDS layout of the staged activations, in bfloat16 elements, for local
// group gl, MFMA index mu = 2 * (operand half) + h, lane group g, A row r and
// element e:  ((((gl * 4 + mu) * 4 + g) * MX + r) * 8 + e).

template <int MX, bool XF32>
__device__ __forceinline__ void stage_activations(
    __bf16 *__restrict__ lds, const void *__restrict__ x, int M, int64_t K,
    int g_begin, int ngroups, int lane)
{
    const int nwords = ngroups * kWordsPerGroup;
    const int mrows = M;  // source rows
    for (int u = lane; u < mrows * nwords; u += 64) {
        const int m = u / nwords;
        const int wi = u - m * nwords;
        const int gl = wi >> 3, w = wi & 7;
        const int half_sel = w & 1;
        const int g = ((w >> 1) == 1) ? 2 : (((w >> 1) == 2) ? 1 : (w >> 1));
        const int64_t k0 = (int64_t)g_begin * kGroup + (int64_t)wi * 16;
        float v[16];
        if constexpr (XF32) {
            const float4 *src = reinterpret_cast<const float4 *>(
                static_cast<const float *>(x) + (int64_t)m * K + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 f = src[q];
                v[4 * q + 0] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
            }
        } else {
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
                static_cast<const uint16_t *>(x) + (int64_t)m * K + k0);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u32x4_t d = src[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[8 * q + 2 * e + 0] = bf16_to_float((uint16_t)(d[e] & 0xffffu));
                    v[8 * q + 2 * e + 1] = bf16_to_float((uint16_t)(d[e] >> 16));
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mu = 2 * half_sel + h;
            u16x8_t hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = v[4 * h + (e >> 1) + 8 * (e & 1)];
                if constexpr (XF32) {
                    const uint16_t hb = float_to_bf16_rne(f);
                    hi[e] = hb;
                    lo[e] = float_to_bf16_rne(f - bf16_to_float(hb));
                } else {
                    hi[e] = (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
                }
            }
            const int base = ((gl * 4 + mu) * 4 + g) * MX;
            if constexpr (XF32) {
                *reinterpret_cast<u16x8_t *>(lds + (base + 2 * m) * 8) = hi;
                *reinterpret_cast<u16x8_t *>(lds + (base + 2 * m + 1) * 8) = lo;
            } else {
                *reinterpret_cast<u16x8_t *>(lds + (base + m) * 8) = hi;
            }
        }
    }
}

template <int MX, bool XF32, int TPW, int PF>
__global__ __launch_bounds__(512) void gemv_kernel(
    const void *__restrict__ x, int M, int64_t K, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, int64_t N, void *__restrict__ y, int y_bf16,
    int waves, int wave_groups)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int kRowsOut = (MX < 4) ? MX : 4;  // accumulator rows per lane that can be live
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nn = lane & 15;
    const int g = lane >> 4;
    const int arow = lane & 15;
    const int Mx = XF32 ? 2 * M : M;
    const bool a_active = arow < Mx;

    const int G = (int)(K / kGroup);
    const int g_begin = (int)(((int64_t)wave * G) / waves);
    const int g_end = (int)(((int64_t)(wave + 1) * G) / waves);
    const int ngroups = g_end - g_begin;
    const int nblocks = (ngroups + 1) >> 1;

    const int64_t n0 = (int64_t)blockIdx.x * (kTileN * TPW);
    const int64_t words_per_row = K / 16;
    const int64_t groups_per_row = K / kGroup;

    // wave-private activation staging area (wave_groups = largest wave range)
    __bf16 *lds_x = reinterpret_cast<__bf16 *>(smem) +
                    (size_t)wave * wave_groups * kGroup * MX;
    float *red = reinterpret_cast<float *>(smem + (size_t)waves * wave_groups * kGroup * MX * 2);

    const uint32_t *crow[TPW];
    const uint16_t *srow[TPW];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
        int64_t r = n0 + tp * kTileN + nn;
        if (r > N - 1) r = N - 1;  // rows past N load a valid row; results are dropped
        crow[tp] = codes + r * words_per_row;
        srow[tp] = scales + r * groups_per_row;
    }

    float yacc[TPW][kRowsOut];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < kRowsOut; ++v) yacc[tp][v] = 0.0f;

    u32x4_t cbuf[PF][TPW];
    uint32_t sbuf[PF][TPW][2];

    // Block b covers local groups 2b and 2b + 1 (the second may not exist
    // at the end of an odd range).  Loads stay branch-free and in bounds: for
    // a one-group block the upper lane groups re-read the first group, whose
    // second-half contribution is multiplied by a zero scale.  Loaded values
    // are not touched until they are consumed PF blocks later.
    auto load_block = [&](int b, u32x4_t (&c)[TPW], uint32_t (&s)[TPW][2]) {
        const int gb = g_begin + 2 * b;
        const bool two = (gb + 1) < g_end;
        const int lg = two ? g : (g & 1);
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            c[tp] = *reinterpret_cast<const u32x4_t *>(crow[tp] + (int64_t)gb * kWordsPerGroup + 4 * lg);
            s[tp][0] = srow[tp][gb];
            s[tp][1] = srow[tp][two ? gb + 1 : gb];
        }
    };

    // Start the code stream, then stage this wave's activations once; the
    // loop below issues no branch that touches memory, so loads stay in
    // flight across blocks.
    if (nblocks > 0) {
#pragma unroll
        for (int p = 0; p < PF; ++p) load_block(p < nblocks ? p : nblocks - 1, cbuf[p], sbuf[p]);
    }
    stage_activations<MX, XF32>(lds_x, x, M, K, g_begin, ngroups, lane);
    __syncthreads();

    // A operands persist across blocks: lanes whose A row does not exist
    // never load and keep zeros; the rows they feed are discarded anyway.
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int mu = 0; mu < 4; ++mu) {
        a0[mu] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        a1[mu] = a0[mu];
    }
    const __bf16 *lds_lane = lds_x + (g * MX + arow) * 8;
    constexpr int kGroupStride = 16 * MX * 8;  // bf16 elements per staged group
    constexpr int kMuStride = 4 * MX * 8;

    // One block: A operands from LDS, consume ring slot p (regroup and flip
    // the code words into fresh registers), optionally refill the slot, then
    // two interleaved 4-MFMA chains (one per 128-K group) and the per-group
    // scaling in binary32.
    auto process = [&](int b, int p, bool refill) {
        const int gl0 = 2 * b;
        const bool two = gl0 + 1 < ngroups;
        if (a_active) {
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
            wq[tp][0] = s02[0] ^ kFlip;  // group 0, operand half 0
            wq[tp][1] = s13[0] ^ kFlip;  // group 0, operand half 1
            wq[tp][2] = s02[1] ^ kFlip;  // group 1, operand half 0
            wq[tp][3] = s13[1] ^ kFlip;  // group 1, operand half 1
            sc[tp][0] = half_to_float((uint16_t)sbuf[p][tp][0]);
            sc[tp][1] = two ? half_to_float((uint16_t)sbuf[p][tp][1]) : 0.0f;
        }
        if (refill) {
            const int nb = (b + PF < nblocks) ? b + PF : nblocks - 1;
            load_block(nb, cbuf[p], sbuf[p]);
        }
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[0], weights_operand(wq[tp][0], 0), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], weights_operand(wq[tp][2], 0), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[1], weights_operand(wq[tp][0], 1), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[1], weights_operand(wq[tp][2], 1), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[2], weights_operand(wq[tp][1], 0), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[2], weights_operand(wq[tp][3], 0), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[3], weights_operand(wq[tp][1], 1), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[3], weights_operand(wq[tp][3], 1), acc1, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < kRowsOut; ++v) {
                yacc[tp][v] = __builtin_fmaf(sc[tp][0], acc0[v], yacc[tp][v]);
                yacc[tp][v] = __builtin_fmaf(sc[tp][1], acc1[v], yacc[tp][v]);
            }
        }
    };

    if (nblocks > 0) {
        const int nfull = (nblocks / PF) * PF;
        for (int b0 = 0; b0 < nfull; b0 += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) process(b0 + p, p, true);
        }
#pragma unroll
        for (int p = 0; p < PF; ++p)
            if (nfull + p < nblocks) process(nfull + p, p, false);
    }

    // Cross-wave reduction in a fixed order.  red[wave][tile][A row][16]
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int v = 0; v < kRowsOut; ++v) {
            const int i = 4 * g + v;
            if (i < MX) red[((wave * TPW + tp) * MX + i) * kTileN + nn] = yacc[tp][v];
        }
    __syncthreads();
    const int outs = M * kTileN * TPW;
    for (int o = threadIdx.x; o < outs; o += blockDim.x) {
        const int m = o / (kTileN * TPW);
        const int rem = o - m * (kTileN * TPW);
        const int tp = rem / kTileN, j = rem - tp * kTileN;
        const int64_t n = n0 + tp * kTileN + j;
        if (n >= N) continue;
        float sum = 0.0f;
        for (int w = 0; w < waves; ++w) {
            const float *base = red + ((w * TPW + tp) * MX) * kTileN;
            if constexpr (XF32)
                sum += base[(2 * m) * kTileN + j] + base[(2 * m + 1) * kTileN + j];
            else
                sum += base[m * kTileN + j];
        }
        const float out = -0.5f * sum;  // operands carried -2t
        if (y_bf16)
            static_cast<uint16_t *>(y)[(int64_t)m * N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(y)[(int64_t)m * N + n] = out;
    }
}

// ---------------------------------------------------------------------------
// Signed normalized Walsh-Hadamard transform: one workgroup per (row, block)
// ---------------------------------------------------------------------------
template <bool XF32>
__global__ __launch_bounds__(256) void fwht_kernel(
    const void *__restrict__ x, const int8_t *__restrict__ signs, int64_t M, int64_t K,
    int block, int log2b, int inverse, float *y, float norm)
{
    extern __shared__ float buf[];
    const int64_t sbase = (int64_t)blockIdx.x * block;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const int64_t base = m * K + sbase;
    for (int i = threadIdx.x; i < block; i += blockDim.x) {
        float v;
        if constexpr (XF32)
            v = static_cast<const float *>(x)[base + i];
        else
            v = bf16_to_float(static_cast<const uint16_t *>(x)[base + i]);
        if (!inverse && signs) v *= (float)signs[sbase + i];
        buf[i] = v;
    }
    __syncthreads();
    for (int s = 0; s < log2b; ++s) {
        const int half = 1 << s;
        for (int p = threadIdx.x; p < (block >> 1); p += blockDim.x) {
            const int i = ((p >> s) << (s + 1)) | (p & (half - 1));
            const float a = buf[i], c = buf[i + half];
            buf[i] = a + c;
            buf[i + half] = a - c;
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < block; i += blockDim.x) {
        float v = buf[i] * norm;
        if (inverse && signs) v *= (float)signs[sbase + i];
        y[base + i] = v;
    }
    __syncthreads();  // the next row reuses buf
    }
}

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Largest LDS request made so far per (kernel, device); raising the limit
// above the 64 KiB default needs hipFuncSetAttribute once.
template <class Kernel>
int ensure_lds(Kernel kernel, size_t bytes)
{
    static std::atomic<size_t> granted[64];
    if (bytes <= 65536) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (granted[dev].load(std::memory_order_relaxed) >= bytes) return 0;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return (int)e;
    granted[dev].store(kMaxLds, std::memory_order_relaxed);
    return 0;
}

struct GemvPlan {
    int waves;
    int wave_groups;
    size_t lds;
};

// Waves per workgroup: enough waves in flight to cover HBM latency and at
// least two 256-K blocks per wave.  LDS holds every wave's staged
// activations plus the reduction area.
inline GemvPlan plan_gemv(int64_t N, int64_t K, int mx, int tpw)
{
    const int64_t tiles = (N + kTileN * tpw - 1) / (kTileN * tpw);
    const int G = (int)(K / kGroup);
    int waves = 1;
    while (waves < 8 && tiles * waves < 2048 && G >= 4 * waves) waves *= 2;
    GemvPlan pl;
    pl.waves = waves;
    pl.wave_groups = (G + waves - 1) / waves;
    pl.lds = (size_t)waves * pl.wave_groups * kGroup * mx * 2 +
             (size_t)waves * tpw * mx * kTileN * sizeof(float);
    return pl;
}

template <int MX, bool XF32, int TPW, int PF>
int launch_gemv_t(const void *x, int M, int64_t K, const uint32_t *codes, const uint16_t *scales,
                  int64_t N, void *y, bool y_bf16, hipStream_t stream)
{
    const GemvPlan pl = plan_gemv(N, K, MX, TPW);
    auto kernel = gemv_kernel<MX, XF32, TPW, PF>;
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    const int64_t tiles = (N + kTileN * TPW - 1) / (kTileN * TPW);
    hipLaunchKernelGGL(kernel, dim3((unsigned)tiles), dim3(64 * pl.waves), pl.lds, stream, x, M, K,
                       codes, scales, N, y, (int)y_bf16, pl.waves, pl.wave_groups);
    return (int)hipGetLastError();
}

template <bool XF32>
int launch_gemv_x(const void *x, int M, int64_t K, const uint32_t *codes, const uint16_t *scales,
                  int64_t N, void *y, bool y_bf16, hipStream_t stream)
{
    const int Mx = XF32 ? 2 * M : M;
    if (Mx <= 1) return launch_gemv_t<1, XF32, 1, 4>(x, M, K, codes, scales, N, y, y_bf16, stream);
    if (Mx <= 2) return launch_gemv_t<2, XF32, 1, 4>(x, M, K, codes, scales, N, y, y_bf16, stream);
    if (Mx <= 4) return launch_gemv_t<4, XF32, 1, 4>(x, M, K, codes, scales, N, y, y_bf16, stream);
    if (Mx <= 8) return launch_gemv_t<8, XF32, 2, 2>(x, M, K, codes, scales, N, y, y_bf16, stream);
    if (Mx <= 16) return launch_gemv_t<16, XF32, 4, 1>(x, M, K, codes, scales, N, y, y_bf16, stream);
    return (int)hipErrorInvalidValue;
}

// Rows of x one launch can take: every staged row costs 2 bytes per K of
// LDS (two rows for binary32 input); larger M runs as several launches.
inline int gemv_rows_per_launch(int64_t N, int64_t K, bool x_f32)
{
    const int per = x_f32 ? 2 : 1;
    for (int rows = 16 / per; rows > 1; rows /= 2) {
        int mx = rows * per;
        int tpw = mx <= 4 ? 1 : (mx <= 8 ? 2 : 4);
        if (plan_gemv(N, K, mx, tpw).lds <= kMaxLds) return rows;
    }
    return 1;
}

}  // namespace

namespace tern {

const char *hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

int launch_gemv(const void *x, bool x_f32, int M, int64_t K, const uint32_t *codes,
                const uint16_t *scales, int64_t N, void *y, bool y_bf16, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int step = gemv_rows_per_launch(N, K, x_f32);
    const size_t xsz = x_f32 ? 4 : 2, ysz = y_bf16 ? 2 : 4;
    for (int m0 = 0; m0 < M; m0 += step) {
        const int mm = (M - m0) < step ? (M - m0) : step;
        const void *xm = static_cast<const char *>(x) + (size_t)m0 * K * xsz;
        void *ym = static_cast<char *>(y) + (size_t)m0 * N * ysz;
        int rc = x_f32 ? launch_gemv_x<true>(xm, mm, K, codes, scales, N, ym, y_bf16, st)
                       : launch_gemv_x<false>(xm, mm, K, codes, scales, N, ym, y_bf16, st);
        if (rc) return rc;
    }
    return 0;
}

int launch_fwht(const void *x, bool x_f32, const int8_t *signs, int64_t M, int64_t K, int block,
                bool inverse, float *y, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    int log2b = 0;
    while ((1 << log2b) < block) ++log2b;
    const float norm = (float)(1.0 / __builtin_sqrt((double)block));
    const int threads = block >= 512 ? 256 : (block >= 128 ? block / 2 : 64);
    dim3 grid((unsigned)(K / block), (unsigned)(M < 65535 ? M : 65535));
    if (x_f32)
        hipLaunchKernelGGL(fwht_kernel<true>, grid, dim3(threads), block * sizeof(float), st, x, signs, M,
                           K, block, log2b, (int)inverse, y, norm);
    else
        hipLaunchKernelGGL(fwht_kernel<false>, grid, dim3(threads), block * sizeof(float), st, x, signs, M,
                           K, block, log2b, (int)inverse, y, norm);
    return (int)hipGetLastError();
}

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

int launch_gemm(const void *x, int64_t M, int64_t K, const uint32_t *codes, const uint16_t *scales,
                int64_t N, float *y, void *, size_t, void *stream)
{
    // First version: 16-row slices through the decode kernel.
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int mm = (int)((M - m0) < 16 ? (M - m0) : 16);
        int rc = launch_gemv(static_cast<const uint16_t *>(x) + m0 * K, false, mm, K, codes, scales, N,
                             y + m0 * N, false, stream);
        if (rc) return rc;
    }
    return 0;
}

}  // namespace tern
