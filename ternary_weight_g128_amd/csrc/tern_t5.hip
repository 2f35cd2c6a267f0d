// Decode GEMV over the base-3 layout (five ternary values per byte) for
// AMD MI355X (gfx950).
//
// Layout (a sub-2-bit native ternary packing; the "prism-ml/Ternary-Bonsai-
// 27B-mlx-2bit" model card, "Memory requirement", leaves the layout open):
// the 128-weight groups of a row are taken five at a time; superblock b is
// 128 bytes, and byte i holds sum_{j<p} q_j 3^j, q_j = t + 1 of weight
// 128 (5b + j) + i, with p = min(5, G - 5b).  1.6 bits per weight plus the
// binary16 group scales.
//
// Digits without division: for a byte value u <= 255, floor(u / 3) =
// (171 u) >> 9 exactly.  The chain alternates between plain and offset
// quotients, v_0 = u, w_1 = v_1 + 1 = (171 v_0 + 512) >> 9, v_2 = (171 w_1 -
// 171) >> 9, w_3 = v_3 + 1, v_4 (v_j = floor(u / 3^j)), so that digit q_j =
// v_j - 3 v_{j+1} satisfies q_j + 1 = (chain_j + chain_{j+1}) mod 4 (the
// offsets of neighbours sum to one).  The MFMA operand is the bfloat16 of -2t:
// ((q + 1) mod 4) << 14 is 0x4000 (+2), 0x8000 (-0) or 0xC000 (-2) for
// q = 0, 1, 2, so every digit costs one add and one shift.  Two bytes ride in
// the 16-bit halves of one register, so every step is one packed 16-bit
// instruction.
//
// Work decomposition: a workgroup owns one 16-row tile; its waves split the
// superblocks of K into contiguous ranges and combine their partial sums in
// LDS in a fixed order.  Lane l serves row n0 + (l & 15) and MFMA k-slot
// group g = l >> 4: per superblock it loads bytes 16g..16g+15 of each
// 64-byte half c of the row's 128 bytes, which hold weights i = 64c + 16g +
// 0..15 of all the superblock's groups.  The eight bytes of operand half h
// (i = 64c + 16g + 8h + 0..7) go in consecutive pairs into the 16-bit halves
// of four registers (one byte permute each), so the eight bfloat16 elements
// of one MFMA B operand are weights i = 64c + 16g + 8h + 0..7 in order, and
// the matching A operand is eight consecutive activations: a 16-byte chunk of
// x.  Up to four rows, every workgroup copies x into LDS once.  From five
// rows on (or where that copy would not fit), the tile-waves of a K-group
// share an LDS ring of half superblocks of x instead (gemv_t5_ring_kernel).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

#include "tern_internal.h"

namespace {

#include "tern_device.h"

typedef unsigned short u16x2v_t __attribute__((ext_vector_type(2)));

constexpr int kT5Bytes = 128;       // bytes per superblock row segment
constexpr int kT5Groups = 5;        // scale groups per superblock
constexpr unsigned kBufRaw = 0x00020000u;  // raw buffer resource, 32-bit data format

struct T5Args {
    const uint16_t *x;      // bfloat16 [M][K]
    const uint8_t *data;    // [N][SB * 128]
    const uint16_t *scales; // binary16 [N][G]
    void *y;
    int64_t N;
    int K, M, G, SB;
    int y_bf16;
    int wk;                 // ring kernel: K-groups of a workgroup
};

// Operand patterns of the five digits of both 16-bit halves of each u[r];
// the four chains advance in lockstep so that they hide each other's latency.
__device__ __forceinline__ void t5_patterns(const unsigned (&u)[4], unsigned (&f)[4][kT5Groups])
{
    const u16x2v_t c171 = {171, 171}, c512 = {512, 512}, c9 = {9, 9}, c14 = {14, 14}, c1 = {1, 1};
    u16x2v_t ch[kT5Groups][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ch[0][r] = __builtin_bit_cast(u16x2v_t, u[r]);
#pragma unroll
    for (int j = 1; j < kT5Groups; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ch[j][r] = (u16x2v_t)(ch[j - 1][r] * c171 + ((j & 1) ? c512 : (u16x2v_t)(-c171))) >> c9;
#pragma unroll
    for (int j = 0; j < kT5Groups; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u16x2v_t nb = (j + 1 < kT5Groups) ? ch[j + 1 < kT5Groups ? j + 1 : j][r] : c1;
            f[r][j] = __builtin_bit_cast(unsigned, (u16x2v_t)((u16x2v_t)(ch[j][r] + nb) << c14));
        }
}

// LDS index (in 16-byte segments) of activation row m for superblock sb,
// half c, group j, operand half h and k-slot group g.
__device__ __forceinline__ int t5_seg(int sb, int c, int j, int h, int g, int m, int mx)
{
    return ((((sb * 2 + c) * kT5Groups + j) * 2 + h) * 4 + g) * mx + m;
}

template <int MX>
__global__ __launch_bounds__(256) void gemv_t5_kernel(const T5Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int kRowsOut = (MX < 4) ? MX : 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int nn = lane & 15, g = lane >> 4;
    const bool a_active = nn < a.M;
    const int64_t n0 = (int64_t)blockIdx.x * kTileN;
    const int sb_begin = (int)((int64_t)wave * a.SB / waves);
    const int sb_end = (int)((int64_t)(wave + 1) * a.SB / waves);
    u32x4_t *lds_x = reinterpret_cast<u32x4_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)a.SB * 80 * MX * 16);

    // Code stream of this lane's row, one superblock ahead, by raw buffer
    // loads over the tile's rows (rows past N read zeros; their results are
    // dropped); the prefetch of the last superblock re-reads it, so that
    // every load is unconditional.  Buffer loads also keep the compiler from
    // merging the prefetch with the next iteration's use (it does so with
    // plain loads that meet in a loop phi).
    const int64_t rows_here = a.N - n0 < kTileN ? a.N - n0 : kTileN;
    const int rowb = a.SB * kT5Bytes;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.data + n0 * rowb), (short)0, (int)(rows_here * rowb), (int)kBufRaw);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scales + n0 * a.G), (short)0, (int)(rows_here * a.G * 2), (int)kBufRaw);
    const int cvo = nn * rowb + 16 * g, svo = nn * a.G * 2;
    const bool any = sb_begin < sb_end;
    u32x4_t cur0 = {0u, 0u, 0u, 0u}, cur1 = cur0;
    uint16_t csc[kT5Groups] = {0, 0, 0, 0, 0};
    auto load_sb = [&](int sb, u32x4_t &c0, u32x4_t &c1, uint16_t (&sh)[kT5Groups]) {
        c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, sb * kT5Bytes, 0));
        c1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, sb * kT5Bytes + 64, 0));
#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) {
            const int gi = kT5Groups * sb + j;
            sh[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, 2 * (gi < a.G ? gi : a.G - 1), 0);
        }
    };
    if (any) load_sb(sb_begin, cur0, cur1, csc);

    // A operands: unit = 8 consecutive k of one row (16 bytes), copied into
    // the LDS image; the groups a short last superblock lacks are staged as
    // zeros, so that their (unused) products are exact zeros.
    {
        const int upr = a.SB * 80;  // units per row, padded to whole superblocks
        const int units = a.M * upr;
        for (int u = threadIdx.x; u < units; u += blockDim.x) {
            const int m = u / upr;
            const int k = 8 * (u - m * upr);
            const bool live = k < a.K;
            u32x4_t d = *reinterpret_cast<const u32x4_t *>(a.x + (int64_t)m * a.K + (live ? k : 0));
            if (!live) d = u32x4_t{0u, 0u, 0u, 0u};
            const int sb = k / 640, rem = k - 640 * sb;
            const int j = rem >> 7, c = (rem >> 6) & 1, gg = (rem >> 4) & 3, h = (rem >> 3) & 1;
            lds_x[t5_seg(sb, c, j, h, gg, m, MX)] = d;
        }
        __syncthreads();
    }

    float yacc[kRowsOut];
#pragma unroll
    for (int v = 0; v < kRowsOut; ++v) yacc[v] = 0.0f;
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    for (int sb = sb_begin; sb < sb_end; ++sb) {
        const int p = (a.G - kT5Groups * sb) < kT5Groups ? (a.G - kT5Groups * sb) : kT5Groups;
        u32x4_t nxt0, nxt1;
        uint16_t nsc[kT5Groups];
        load_sb(sb + 1 < sb_end ? sb + 1 : sb, nxt0, nxt1, nsc);
        f32x4_t acc[kT5Groups];
#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4_t cw = c ? cur1 : cur0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t xs[kT5Groups];
#pragma unroll
                for (int j = 0; j < kT5Groups; ++j) xs[j] = a_active ? lds_x[t5_seg(sb, c, j, h, g, nn, MX)] : zero4;
                unsigned f[4][kT5Groups];
                const unsigned d0 = cw[2 * h], d1 = cw[2 * h + 1];
                // consecutive byte pairs into the 16-bit halves: bytes 0, 1 | 2, 3 | 4, 5 | 6, 7
                const unsigned pairs[4] = {__builtin_amdgcn_perm(0u, d0, 0x0c010c00u),
                                           __builtin_amdgcn_perm(0u, d0, 0x0c030c02u),
                                           __builtin_amdgcn_perm(0u, d1, 0x0c010c00u),
                                           __builtin_amdgcn_perm(0u, d1, 0x0c030c02u)};
                t5_patterns(pairs, f);
#pragma unroll
                for (int j = 0; j < kT5Groups; ++j) {
                    const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, u32x4_t{f[0][j], f[1][j], f[2][j], f[3][j]});
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xs[j]), wb,
                                                                     acc[j], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) {
            const float sj = j < p ? half_to_float(csc[j]) : 0.0f;
#pragma unroll
            for (int v = 0; v < kRowsOut; ++v) yacc[v] = __builtin_fmaf(sj, acc[j][v], yacc[v]);
        }
        cur0 = nxt0;
        cur1 = nxt1;

#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) csc[j] = nsc[j];
    }

    // combine the waves' partial sums in a fixed order and store
#pragma unroll
    for (int v = 0; v < kRowsOut; ++v) {
        const int i = 4 * g + v;
        if (i < MX) red[(wave * MX + i) * kTileN + nn] = yacc[v];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < a.M * kTileN; o += blockDim.x) {
        const int m = o / kTileN, j = o - m * kTileN;
        const int64_t n = n0 + j;
        if (n >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < waves; ++w) sum += red[(w * MX + m) * kTileN + j];
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    }
}

// ---------------------------------------------------------------------------
// Five or more rows: the A operands through a shared LDS ring
// ---------------------------------------------------------------------------
//
// A workgroup is WT tile-waves x WK K-groups; the waves of a K-group own one
// tile each over the same superblocks and take their A operands from an LDS
// ring of three half superblocks of x (half c of superblock sb: the 64
// activations k = 128 (5 sb + j) + 64 c + 0..63 of each of its five groups
// j), filled by buffer loads to LDS two halves ahead.  A half holds its MX
// rows in x's order, 40 16-byte chunks (chunk 8 j + q = k 128 (5 sb + j) +
// 64 c + 8 q .. + 7) and one of padding per row, so a load instruction reads
// contiguous 128-byte row spans and the 16 rows of an MFMA operand (chunk
// 8 j + 2 g + h of its row) fall on 16 distinct bank groups.  Codes and
// scales stream per wave one superblock ahead.  One barrier per half
// publishes it and frees the slot read the half before.
typedef __attribute__((address_space(3))) void lds_void_t;
// s_waitcnt operand: vmcnt(n); expcnt and lgkmcnt not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kT5RowSlots = 41;  // 16-byte chunks per row of a half superblock: 40 and one of padding

// One 16-byte buffer load per lane straight into LDS (lane l writes dst +
// 16 l).  A plain device function: with the builtin written inside a kernel
// template, the host pass of this compiler drops the template's launch stub.
__device__ __forceinline__ void t5_load_lds16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}

constexpr int t5_ring_loads(int mx, int wt) { return ((mx * kT5RowSlots + 63) / 64 + wt - 1) / wt; }

template <int MX, int WT>
__global__ __launch_bounds__(512) void gemv_t5_ring_kernel(const T5Args a)
{
    constexpr int NS = 3;                                // ring slots (half superblocks)
    constexpr int kLoads = t5_ring_loads(MX, WT);        // loads to LDS per lane per half
    constexpr int kChunk = kLoads * WT * 1024;           // LDS bytes of one half
    constexpr int kCodeOps = 2 + kT5Groups;              // loads of one superblock's codes and scales
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = a.wk;
    const int kg = wave / WT, tw = wave - kg * WT;
    const int nn = lane & 15, g = lane >> 4;
    const int sbq = a.SB / wk, sbr = a.SB % wk;  // every K-group has sbq (>= 1) or sbq + 1
    const int sb_begin = kg * sbq + (kg < sbr ? kg : sbr);
    const int nsb = sbq + (kg < sbr ? 1 : 0);
    const int64_t n_wg = (int64_t)blockIdx.x * (kTileN * WT);
    const int64_t n0 = n_wg + (int64_t)tw * kTileN;
    unsigned char *ring = smem + (size_t)kg * NS * kChunk;
    float *red = reinterpret_cast<float *>(smem + (size_t)wk * NS * kChunk);

    // A chunks of this lane: slot p = (tw kLoads + q) 64 + lane of a half is
    // chunk p % 41 of row p / 41.  Rows past M re-read row M - 1, padding
    // slots and slots past the last row re-read chunk 0, and groups past G
    // re-read group G - 1 (their scale is zero).
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.x, (short)0, (int)((int64_t)a.M * a.K * 2), (int)kBufRaw);
    int xoff[kLoads], xj[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int p = (tw * kLoads + q) * 64 + lane;
        const int row = p / kT5RowSlots, cs = p - row * kT5RowSlots;
        const int r = row < a.M ? row : a.M - 1;
        xj[q] = cs < 40 ? cs >> 3 : 0;
        xoff[q] = r * a.K + (cs < 40 ? 8 * (cs & 7) : 0);
    }
    auto load_half = [&](int t, int slot) {
        const int ls = t >> 1, c = t & 1;
        const int sb = sb_begin + (ls < nsb ? ls : nsb - 1);
        const int jmax = a.G - 1 - kT5Groups * sb;  // last group of the superblock (4 unless it is short)
        unsigned char *dst = ring + slot * kChunk + tw * kLoads * 1024;
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int j = xj[q] < jmax ? xj[q] : jmax;
            t5_load_lds16(xrs, dst + 1024 * q, (xoff[q] + kGroup * j) * 2, (640 * sb + 64 * c) * 2);
        }
    };

    // codes and scales of this wave's tile (rows past N read zeros; their
    // results are dropped), one superblock ahead
    const int64_t left = a.N - n0;
    const int rows_here = left <= 0 ? 0 : (left < kTileN ? (int)left : kTileN);
    const int rowb = a.SB * kT5Bytes;
    const int64_t nb = rows_here > 0 ? n0 : 0;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.data + nb * rowb), (short)0, rows_here * rowb, (int)kBufRaw);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scales + nb * a.G), (short)0, rows_here * a.G * 2, (int)kBufRaw);
    const int cvo = nn * rowb + 16 * g, svo = nn * a.G * 2;
    u32x4_t cur0, cur1, nxt0, nxt1;
    uint16_t csc[kT5Groups], nsc[kT5Groups];
    auto load_sb = [&](int ls, u32x4_t &c0, u32x4_t &c1, uint16_t (&sh)[kT5Groups]) {
        const int sb = sb_begin + (ls < nsb ? ls : nsb - 1);
        c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, sb * kT5Bytes, 0));
        c1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, sb * kT5Bytes + 64, 0));
#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) {
            const int gi = kT5Groups * sb + j;
            sh[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, 2 * (gi < a.G ? gi : a.G - 1), 0);
        }
    };

    float yacc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4_t acc[kT5Groups];
    const int arow = nn & (MX - 1);  // rows past MX read a row below MX; their outputs are dropped
    const int a_lane = (arow * kT5RowSlots + 2 * g) * 16;

    // half c of local superblock ls from ring slot `slot`
    auto half = [&](int ls, int c, int slot) {
        if (c == 0) {
#pragma unroll
            for (int j = 0; j < kT5Groups; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const unsigned char *sl = ring + slot * kChunk + a_lane;
        const u32x4_t cw = c ? cur1 : cur0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4_t xs[kT5Groups];
#pragma unroll
            for (int j = 0; j < kT5Groups; ++j) xs[j] = *reinterpret_cast<const u32x4_t *>(sl + (8 * j + h) * 16);
            unsigned f[4][kT5Groups];
            const unsigned d0 = cw[2 * h], d1 = cw[2 * h + 1];
            const unsigned pairs[4] = {__builtin_amdgcn_perm(0u, d0, 0x0c010c00u),
                                       __builtin_amdgcn_perm(0u, d0, 0x0c030c02u),
                                       __builtin_amdgcn_perm(0u, d1, 0x0c010c00u),
                                       __builtin_amdgcn_perm(0u, d1, 0x0c030c02u)};
            t5_patterns(pairs, f);
#pragma unroll
            for (int j = 0; j < kT5Groups; ++j) {
                const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, u32x4_t{f[0][j], f[1][j], f[2][j], f[3][j]});
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xs[j]), wb, acc[j], 0, 0,
                                                                 0);
            }
        }
        if (c == 1) {
            const int sb = sb_begin + ls;
            const int p = (a.G - kT5Groups * sb) < kT5Groups ? (a.G - kT5Groups * sb) : kT5Groups;
#pragma unroll
            for (int j = 0; j < kT5Groups; ++j) {
                const float sj = j < p ? half_to_float(csc[j]) : 0.0f;
#pragma unroll
                for (int v = 0; v < 4; ++v) yacc[v] = __builtin_fmaf(sj, acc[j][v], yacc[v]);
            }
        }
    };

    // One half step t: wait until this wave's loads of half t have landed
    // (issued after them: the loads of half t + 1 and one superblock of
    // codes), publish it with a barrier (which also says every wave is done
    // reading the slot of half t - 1), refill that slot with half t + 2
    // (past the end the last one again: the loads stay unconditional, so
    // the counts are exact), prefetch the next superblock's codes at the
    // first half, then compute half t.
    auto step = [&](int t, bool compute) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads + kCodeOps));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_half(t + 2, (t + 2) % NS);
        if ((t & 1) == 0) load_sb((t >> 1) + 1, nxt0, nxt1, nsc);
        __builtin_amdgcn_sched_barrier(0);
        if (compute) half(t >> 1, t & 1, t % NS);
        if (t & 1) {
            cur0 = nxt0;
            cur1 = nxt1;
#pragma unroll
            for (int j = 0; j < kT5Groups; ++j) csc[j] = nsc[j];
        }
    };

    load_half(0, 0);
    load_half(1, 1);
    load_sb(0, cur0, cur1, csc);
    __builtin_amdgcn_sched_barrier(0);
    for (int ls = 0; ls < sbq; ++ls) {
        step(2 * ls, true);
        step(2 * ls + 1, true);
    }
    if (sbr > 0) {  // the first sbr K-groups have one more superblock
        step(2 * sbq, kg < sbr);
        step(2 * sbq + 1, kg < sbr);
    }
    // every load to LDS has landed before the workgroup's LDS is reused
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    // combine the K-groups' partial sums in a fixed order and store
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int i = 4 * g + v;
        if (i < MX) red[((tw * wk + kg) * MX + i) * kTileN + nn] = yacc[v];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < a.M * kTileN * WT; o += blockDim.x) {
        const int m = o / (kTileN * WT), rem = o - m * (kTileN * WT);
        const int twi = rem / kTileN, j = rem % kTileN;
        const int64_t n = n_wg + rem;
        if (n >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < wk; ++w) sum += red[((twi * wk + w) * MX + m) * kTileN + j];
        const float out = -0.5f * sum;  // operands carried -2t
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[(int64_t)m * a.N + n] = float_to_bf16_rne(out);
        else
            static_cast<float *>(a.y)[(int64_t)m * a.N + n] = out;
    }
}

size_t t5_lds(int64_t K, int mx, int waves)
{
    const int64_t SB = (K / kGroup + kT5Groups - 1) / kT5Groups;
    return (size_t)SB * 80 * mx * 16 + (size_t)waves * mx * kTileN * sizeof(float);
}

int t5_waves(int64_t K)
{
    const int64_t SB = (K / kGroup + kT5Groups - 1) / kT5Groups;
    return SB >= 4 ? 4 : (SB >= 1 ? (int)SB : 1);
}

template <int MX>
int launch_t5_staged(const T5Args &a, hipStream_t stream)
{
    const int waves = t5_waves(a.K);
    const size_t lds = t5_lds(a.K, MX, waves);
    int rc = ensure_lds(gemv_t5_kernel<MX>, lds);
    if (rc) return rc;
    if ((rc = check_block(64 * waves, 256))) return rc;
    const unsigned wgs = (unsigned)((a.N + kTileN - 1) / kTileN);
    hipLaunchKernelGGL(gemv_t5_kernel<MX>, dim3(wgs), dim3(64 * waves), lds, stream, a);
    return (int)hipGetLastError();
}

// Ring launch: two tile-waves; two K-groups, four for long rows (at least
// one superblock each).  From a sweep of tile-waves (1, 2, 4) x K-groups
// (1, 2, 4) at 16 rows: 17408 -> 5120 went 33.4 -> 23.9 us with two
// tile-waves and four K-groups.
template <int MX>
int launch_t5_ring(T5Args a, hipStream_t stream)
{
    const int64_t tiles = (a.N + kTileN - 1) / kTileN;
    constexpr int wt = 2;
    int wk = a.SB >= 16 ? 4 : 2;
    while (wk > 1 && a.SB < wk) wk /= 2;
    a.wk = wk;
    const size_t lds = (size_t)wk * 3 * t5_ring_loads(MX, wt) * wt * 1024 + (size_t)wt * wk * MX * kTileN * sizeof(float);
    void (*kernel)(T5Args) = gemv_t5_ring_kernel<MX, wt>;
    int rc = ensure_lds(kernel, lds);
    if (rc) return rc;
    if ((rc = check_block(64 * wt * wk, 512))) return rc;
    const unsigned wgs = (unsigned)((tiles + wt - 1) / wt);
    hipLaunchKernelGGL(kernel, dim3(wgs), dim3(64 * wt * wk), lds, stream, a);
    return (int)hipGetLastError();
}

}  // namespace

namespace tern {

int64_t t5_row_bytes(int64_t K) { return ((K / kGroup + kT5Groups - 1) / kT5Groups) * kT5Bytes; }

int launch_gemv_t5(const void *x, int M, int64_t K, const uint8_t *data, const uint16_t *scales, int64_t N,
                   void *y, bool y_bf16, void *stream)
{
    // one launch for every M <= 16: the weights are read once
    hipStream_t st = static_cast<hipStream_t>(stream);
    T5Args a;
    a.M = M;
    a.x = static_cast<const uint16_t *>(x);
    a.data = data;
    a.scales = scales;
    a.y = y;
    a.N = N;
    a.K = (int)K;
    a.G = (int)(K / kGroup);
    a.SB = (int)((a.G + kT5Groups - 1) / kT5Groups);
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.wk = 1;
    const int mx = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    // up to four rows: each workgroup copies x into LDS, where that fits;
    // otherwise the shared ring (rows padded to at least four)
    if (mx <= 4 && t5_lds(K, mx, t5_waves(K)) <= kMaxLds) {
        switch (mx) {
        case 1: return launch_t5_staged<1>(a, st);
        case 2: return launch_t5_staged<2>(a, st);
        default: return launch_t5_staged<4>(a, st);
        }
    }
    switch (mx) {
    case 1:
    case 2:
    case 4: return launch_t5_ring<4>(a, st);
    case 8: return launch_t5_ring<8>(a, st);
    default: return launch_t5_ring<16>(a, st);
    }
}

}  // namespace tern
