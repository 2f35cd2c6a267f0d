// Decode GEMV for one to four rows of bfloat16 activations with the work
// split evenly over the CUs.
//
// y[m][n] = sum_g s[n][g] sum_{k in g} t[n][k] x[m][k] ("prism-ml/Ternary-Bonsai-
// 27B-mlx-2bit" model card, "Weight representation: ternary g128" and "CUDA
// (NVIDIA GPUs)": codes unpacked inside the kernel; the card's "Cross-platform
// throughput" puts batch-1 decode on the memory stream).
//
// Why a second small-M kernel.  The tiled GEMV hands each workgroup whole
// 16-row tiles, so a matrix of 320 or 1088 tiles on 256 CUs leaves some CUs
// 1.4-1.6x the average work, and at M <= 4 the step is bound by the slowest
// CU's unpack work.  Here the unit of work is a pair (quad, block): four
// consecutive output rows and one 256-K block (two scale groups).  Every
// workgroup takes an equal run of quads, and its waves take equal runs of
// that run's steps; a step is four pairs of one quad (blocks 4 j .. 4 j + 3
// of it: the kernel takes rows whose block count is a multiple of four), so
// every address and quad change is the same for the whole wave.
//
// Four pairs per MFMA.  v_mfma_f32_16x16x32_bf16 has 16 A rows, of which an
// M-row product uses M.  Here A row 4 i + m (i = 0..3, m < M) carries the
// activations of row m of x in block i of the step, and B column nn = 4 i + r
// carries the weights of output row r of the quad in that block, so
// D[4 i + m][4 i + r] is the block's contribution to y[m][r] and the other
// products of the instruction are discarded.  One instruction still consumes
// 16 B columns x 32 k of weights, as in the tiled kernel, and only the
// 16 M lanes of the live A rows read activations (16 bytes each) from LDS.
//
// Lanes.  A operand: lane l holds A row l & 15, k-slots 8 (l >> 4) + 0..7;
// B operand: lane l holds column l & 15, the same k-slots; result: lane l
// holds column l & 15, rows 4 (l >> 4) + 0..3, so lane (column nn, lane
// group nn >> 2) holds the useful D[4 (nn >> 2) + m][nn] in register m.
// Lane (column nn, lane group g) loads code words 4 g .. 4 g + 3 of its
// block (64 contiguous bytes per column), a v_permlane32_swap pair regroups
// them by scale group, and the weight operand of MFMA mu is built from byte
// planes in consecutive-slot order: element e of MFMA mu of group G is
// k = 128 G + 32 {0, 2, 1, 3}[g] + 8 mu + e, the 8 consecutive activations
// the A lane reads.
//
// Sums.  The result lanes keep one running sum per row of x for the current
// quad (the scaled D of each step, the scale pair being the lane's own
// block's); when the wave moves to the next quad they write them to LDS
// slots of their own (wave, block slot, quad, output row, x row) and start
// again.  The workgroup then adds
// the slots of each output row in a fixed order and stores -y/2 (operands
// carry -2t), so the result does not depend on timing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

#include "tern_internal.h"

namespace {

#include "tern_device.h"

constexpr int kSlices = 4;                      // blocks per MFMA step (A rows 0, 4, 8, 12)
constexpr int kBlockX = 256;                    // activations per block
constexpr int kXBlockBytes = 2 * kBlockX + 16;  // LDS bytes per block of x (16 of padding)
constexpr int kPF = 4;                          // code ring slots
constexpr unsigned kBufRaw1 = 0x00020000u;      // raw buffer resource, 32-bit data format
typedef unsigned u32x2v_t __attribute__((ext_vector_type(2)));

struct Gemv1Args {
    const uint16_t *x;       // bfloat16 [M][K]
    const uint32_t *codes;   // [N][K / 16] 2-bit codes, or [N][K / 32] sign bits (binary)
    const uint16_t *scales;  // [N][K / 128]
    void *y;                 // [M][N] binary32 or bfloat16
    int64_t N;
    int M;                   // rows of x, 1..MX
    int64_t quads;           // (N + 3) / 4
    int K;                   // multiple of 128
    int G;                   // K / 128
    int nblk;                // (G + 1) / 2, a multiple of kSlices
    int waves;               // per workgroup
    int qmax;                // quads of the largest workgroup
    int y_bf16;
};

// Binary weights (the 1-bit variant: bit j of word w of a row is weight
// 32 w + j, 1 for +1 and 0 for -1).  Byte plane j of a word holds, in byte
// b, 0x40 | (bit 8 b + j) << 7: the high byte of the bfloat16 -2t (0xC000
// for +1, 0x4000 for -1), so that one byte permute of two planes gives a
// bfloat16 pair of the MFMA operand, as for the 2-bit codes.
__device__ __forceinline__ void bin_planes(unsigned w, unsigned (&p)[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = ((w << (7 - j)) & 0x80808080u) | 0x40404040u;
}

// MFMA B operand of weights 8 mu + 0..7 of a binary word (element e = bit
// 8 mu + e): pair i is byte mu of planes 2 i and 2 i + 1 in bytes 1 and 3.
__device__ __forceinline__ bf16x8_t bin_operand(const unsigned (&p)[8], int mu)
{
    const unsigned sel = 0x0Cu | ((unsigned)mu << 8) | (0x0Cu << 16) | ((4u + (unsigned)mu) << 24);
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], sel);
    return __builtin_bit_cast(bf16x8_t, v);
}

// SC4: the scale pair of a block is one aligned 4-byte load (G even).
// KD: steps of codes in flight.  MX: rows of x the sums are kept for (M <= MX).
// BIN: binary weights (a block of a row is 8 words; lane group g loads words
// 2 g, 2 g + 1 and one v_permlane32_swap leaves it word {0, 2, 1, 3}[g] of
// each of the block's two groups), else 2-bit codes.
template <bool SC4, int KD, int MX, bool BIN>
__global__ __launch_bounds__(512) void gemv1_kernel(const Gemv1Args a)
{
    static_assert(KD >= 1 && KD < kPF, "the refill reuses a consumed slot");
    static_assert(MX >= 1 && MX <= 4, "four A rows per block");
    constexpr int kXBatch = MX == 4 ? 12 : 6;  // 16-byte x loads per thread per batch
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nthreads = blockDim.x;
    const int nn = lane & 15, g = lane >> 4;
    const int slice = nn >> 2, r = nn & 3;  // B column nn: row r of the quad, block `slice` of the step
    const int nblk = a.nblk, spq = nblk / kSlices;  // steps per quad

    // this workgroup's quads, and this wave's steps j (quad j / spq, blocks
    // kSlices (j % spq) + 0..3), counted from the workgroup's first quad
    const int64_t q_begin = a.quads * blockIdx.x / gridDim.x;
    const int nq = (int)(a.quads * (blockIdx.x + 1) / gridDim.x - q_begin);
    const int64_t S = (int64_t)nq * spq;
    const int j_lo = (int)(S * wave / a.waves), j_hi = (int)(S * (wave + 1) / a.waves);
    const int steps = j_hi - j_lo;

    unsigned char *xs = smem;                          // row m of x at m * xrow bytes
    const int xrow = nblk * kXBlockBytes;
    float *red = reinterpret_cast<float *>(smem + (size_t)a.M * xrow);  // [waves][kSlices][qmax][4][MX]
    const int red_count = a.waves * kSlices * a.qmax * 4 * MX;

    // 1. activation loads (first batch) go out first
    const int rchunks = a.K / 8;  // 16-byte chunks of a row of x
    const int xchunks = a.M * rchunks;
    u32x4_t xv[kXBatch];
    auto load_x = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
            int c = c0 + threadIdx.x + i * nthreads;
            c = c < xchunks ? c : xchunks - 1;  // duplicates rewrite the same bytes
            xv[i] = *reinterpret_cast<const u32x4_t *>(a.x + 8 * (int64_t)c);
        }
    };
    auto put_x = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
            int c = c0 + threadIdx.x + i * nthreads;
            c = c < xchunks ? c : xchunks - 1;
            const int m = c / rchunks, cc = c - m * rchunks;  // chunk cc of row m: block cc >> 5
            *reinterpret_cast<u32x4_t *>(xs + m * xrow + 16 * cc + 16 * (cc >> 5)) = xv[i];
        }
    };
    load_x(0);
    __builtin_amdgcn_sched_barrier(0);

    // 2. code stream.  Raw buffer loads; the offset is the wave's (quad
    //    row, block) part plus the lane's, all of it in the vector offset,
    //    which the buffer's range check covers: rows past N read zeros
    //    (their outputs are dropped), and refills past the wave's last step
    //    are never used.  The loads stay unconditional, so the waits for
    //    them are exact.
    constexpr int kWordsPerBlock = BIN ? 8 : 16;  // words of one row per 256-K block
    const int wpr = BIN ? a.K / 32 : a.K / 16;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(a.codes), (short)0, (int)(a.N * wpr * 4), (int)kBufRaw1);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.scales), (short)0, (int)(a.N * a.G * 2), (int)kBufRaw1);
    // bytes: row r, block slice, words 4 g.. (binary: 2 g..)
    const int lane_w = 4 * (r * wpr + kWordsPerBlock * slice + (BIN ? 2 : 4) * g);
    const int lane_s = 2 * (r * a.G + 2 * slice);
    int lq = j_lo / spq, lb = kSlices * (j_lo - lq * spq);   // next load: quad, first block
    u32x4_t cbuf[kPF];
    uint32_t sbuf[kPF];
    auto load_step = [&](int p) {
        const int row = ((int)q_begin + lq) * 4;
        const int uw = 4 * (row * wpr + kWordsPerBlock * lb), us = 2 * (row * a.G + 2 * lb);
        int lw = lane_w;
        bool two = true;
        if constexpr (!SC4 && !BIN) {
            // odd G: the last block holds one group; its upper lanes re-read
            // that group (its second scale is zeroed below); binary rows
            // always hold whole blocks
            two = 2 * (lb + slice) + 1 < a.G;
            lw = two ? lane_w : lane_w - 16 * (g & 2);
        }
        if constexpr (BIN) {
            const u32x2v_t w2 = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(crs, uw + lw, 0, 0));
            cbuf[p] = u32x4_t{w2[0], w2[1], 0u, 0u};
        } else {
            cbuf[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, uw + lw, 0, 0));
        }
        if constexpr (SC4) {
            sbuf[p] = __builtin_amdgcn_raw_buffer_load_b32(srs, us + lane_s, 0, 0);
        } else {
            const uint32_t s0 = __builtin_amdgcn_raw_buffer_load_b16(srs, us + lane_s, 0, 0);
            const uint32_t s1 = __builtin_amdgcn_raw_buffer_load_b16(srs, us + lane_s + (two ? 2 : 0), 0, 0);
            sbuf[p] = s0 | (two ? s1 << 16 : 0u);
        }
        lb += kSlices;
        if (lb == nblk) {
            lb = 0;
            ++lq;
        }
    };
    // unconditional (a wave without steps loads a valid row or zeros)
    for (int p = 0; p < KD; ++p) load_step(p);
    __builtin_amdgcn_sched_barrier(0);

    // 3. stage x (padded: block b at 528 b bytes) and clear the sum slots
    put_x(0);
    for (int c0 = kXBatch * nthreads; c0 < xchunks; c0 += kXBatch * nthreads) {
        load_x(c0);
        put_x(c0);
    }
    for (int i = threadIdx.x; i < red_count; i += nthreads) red[i] = 0.0f;
    __syncthreads();

    // 4. the steps
    const bool a_lane = r < a.M;       // A row 4 slice + r: row r of x in block `slice`
    const bool sum_lane = g == slice;  // holds D[4 slice + m][nn], m < M
    const unsigned a_off = 64u * (unsigned)(((g & 1) << 1) | (g >> 1)) + (unsigned)slice * kXBlockBytes +
                           (unsigned)(a_lane ? r : 0) * (unsigned)xrow;
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int mu = 0; mu < 4; ++mu) {
        a0[mu] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        a1[mu] = a0[mu];
    }
    float ysum[MX];
#pragma unroll
    for (int m = 0; m < MX; ++m) ysum[m] = 0.0f;
    int pq = j_lo / spq, pb = kSlices * (j_lo - pq * spq);  // quad and first block of the step processed next
    int qcur = pq;
    float *red_lane = red + (((wave * kSlices + slice) * a.qmax) * 4 + r) * MX;
    auto flush = [&]() {
#pragma unroll
        for (int m = 0; m < MX; ++m) red_lane[qcur * 4 * MX + m] = ysum[m];
    };

    auto process = [&](int p) {
        if (a_lane) {
            // a one-group block (odd G) re-reads its group for the second
            // (finite values; that group's scale is zero)
            const unsigned char *src = xs + (size_t)pb * kXBlockBytes + a_off;
            const unsigned second = (SC4 || 2 * (pb + slice) + 1 < a.G) ? 256u : 0u;
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                a0[mu] = *reinterpret_cast<const bf16x8_t *>(src + 16 * mu);
                a1[mu] = *reinterpret_cast<const bf16x8_t *>(src + second + 16 * mu);
            }
        }
        unsigned wq[4];
        if constexpr (BIN) {
            const auto sw = __builtin_amdgcn_permlane32_swap(cbuf[p][0], cbuf[p][1], false, false);
            wq[0] = sw[0];  // group 0 word
            wq[1] = sw[1];  // group 1 word
            wq[2] = wq[3] = 0u;
        } else {
            const auto s02 = __builtin_amdgcn_permlane32_swap(cbuf[p][0], cbuf[p][2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(cbuf[p][1], cbuf[p][3], false, false);
            wq[0] = s02[0];  // group 0 halves, group 1 halves
            wq[1] = s13[0];
            wq[2] = s02[1];
            wq[3] = s13[1];
        }
        const uint32_t sp = sbuf[p];
        const float sc0 = half_to_float((uint16_t)(sp & 0xffffu));
        const float sc1 = half_to_float((uint16_t)(sp >> 16));
        load_step((p + KD) % kPF);  // unconditional: exact load counts
        f32x4_t acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        if constexpr (BIN) {
            unsigned b0[8], b1[8];
            bin_planes(wq[0], b0);
            bin_planes(wq[1], b1);
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[mu], bin_operand(b0, mu), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[mu], bin_operand(b1, mu), acc1, 0, 0, 0);
            }
        } else {
            unsigned pl[4][4];
#pragma unroll
            for (int w = 0; w < 4; ++w) code_planes(wq[w], kPlaneMask, pl[w]);
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[mu], operand_from_planes(pl[mu >> 1], mu & 1),
                                                               acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a1[mu], operand_from_planes(pl[2 + (mu >> 1)], mu & 1), acc1, 0, 0, 0);
            }
        }
        if (pq != qcur) {  // the wave moved to the next quad (uniform)
            if (sum_lane) flush();
#pragma unroll
            for (int m = 0; m < MX; ++m) ysum[m] = 0.0f;
            qcur = pq;
        }
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            ysum[m] = __builtin_fmaf(sc0, acc0[m], ysum[m]);
            ysum[m] = __builtin_fmaf(sc1, acc1[m], ysum[m]);
        }
        pb += kSlices;
        if (pb == nblk) {
            pb = 0;
            ++pq;
        }
    };

    const int nfull = (steps / kPF) * kPF;
    for (int j0 = 0; j0 < nfull; j0 += kPF) {
#pragma unroll
        for (int p = 0; p < kPF; ++p) process(p);
    }
#pragma unroll
    for (int p = 0; p < kPF; ++p)
        if (nfull + p < steps) process(p);
    if (steps > 0 && sum_lane) flush();
    __syncthreads();

    // 5. every output: its slots in a fixed order
    for (int o = threadIdx.x; o < nq * 4 * a.M; o += nthreads) {
        const int m = o / (nq * 4), qr = o - m * (nq * 4);
        const int q = qr >> 2, rr = qr & 3;
        const int64_t n = (q_begin + q) * 4 + rr;
        if (n >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < a.waves; ++w)
#pragma unroll
            for (int s = 0; s < kSlices; ++s) sum += red[((((w * kSlices + s) * a.qmax + q) * 4 + rr) * MX) + m];
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    }
}

struct Gemv1Plan {
    int wgs, waves, qmax, mx;
    int64_t quads;
    size_t lds;
};

// From a sweep of waves per workgroup (2, 4, 8) x workgroups per CU (1-4) x
// steps in flight (2, 3) at M = 1: rows of 32 or more blocks, one workgroup
// of eight waves per CU (17408 -> 5120: 9.45 us; four waves x three
// workgroups 10.3); shorter rows, three workgroups of four waves per CU
// (5120 -> 17408: 9.12 us; eight waves x one 9.61).  Two steps in flight.
bool plan_gemv1(int M, int64_t N, int64_t K, Gemv1Plan &pl)
{
    const int G = (int)(K / kGroup);
    const int nblk = (G + 1) / 2;
    // whole steps of four blocks per quad; byte offsets of the code and
    // scale loads are 32-bit (refills past a wave's run may reach a few
    // quads past N)
    if (M < 1 || M > 4 || nblk < kSlices || nblk % kSlices != 0 || (N + 16) * (K / 4) >= ((int64_t)1 << 31))
        return false;
    pl.quads = (N + 3) / 4;
    pl.mx = M == 1 ? 1 : M == 2 ? 2 : 4;
    const int64_t cus = device_cus();
    const bool long_rows = nblk >= 32;
    const int64_t wgs = long_rows ? cus : 3 * cus;
    pl.wgs = (int)(pl.quads < wgs ? pl.quads : wgs);
    pl.waves = long_rows ? 8 : 4;
    pl.qmax = (int)((pl.quads + pl.wgs - 1) / pl.wgs);
    pl.lds = (size_t)M * nblk * kXBlockBytes + (size_t)pl.waves * kSlices * pl.qmax * 4 * pl.mx * sizeof(float);
    return pl.lds <= kMaxLds;
}

template <int MX>
void (*gemv1_pick(bool sc4, bool bin))(Gemv1Args)
{
    if (bin) return sc4 ? gemv1_kernel<true, 2, MX, true> : gemv1_kernel<false, 2, MX, true>;
    return sc4 ? gemv1_kernel<true, 2, MX, false> : gemv1_kernel<false, 2, MX, false>;
}

}  // namespace

namespace tern {

bool gemv1_applies(int M, int64_t N, int64_t K)
{
    Gemv1Plan pl;
    return N > 0 && K > 0 && plan_gemv1(M, N, K, pl);
}

int launch_gemv1(const void *x, int M, int64_t K, const uint32_t *codes, const uint16_t *scales, int64_t N,
                 void *y, bool y_bf16, bool binary, void *stream)
{
    Gemv1Plan pl;
    if (!plan_gemv1(M, N, K, pl) || (binary && (K / kGroup) % 2 != 0)) return (int)hipErrorInvalidValue;
    Gemv1Args a;
    a.x = static_cast<const uint16_t *>(x);
    a.codes = codes;
    a.scales = scales;
    a.y = y;
    a.N = N;
    a.M = M;
    a.quads = pl.quads;
    a.K = (int)K;
    a.G = (int)(K / kGroup);
    a.nblk = (a.G + 1) / 2;
    a.waves = pl.waves;
    a.qmax = pl.qmax;
    a.y_bf16 = y_bf16 ? 1 : 0;
    const bool sc4 = a.G % 2 == 0 && (reinterpret_cast<uintptr_t>(scales) % 4) == 0;
    void (*kernel)(Gemv1Args) =
        pl.mx == 1 ? gemv1_pick<1>(sc4, binary) : pl.mx == 2 ? gemv1_pick<2>(sc4, binary) : gemv1_pick<4>(sc4, binary);
    int rc = ensure_lds(kernel, pl.lds);
    if (rc) return rc;
    if ((rc = check_block(64 * pl.waves, 512))) return rc;
    hipLaunchKernelGGL(kernel, dim3((unsigned)pl.wgs), dim3(64 * pl.waves), pl.lds, static_cast<hipStream_t>(stream),
                       a);
    return (int)hipGetLastError();
}

}  // namespace tern
