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
// x, read from an LDS copy of x (up to four rows) or straight from memory
// (more rows, where the copy would not fit or would be made by every
// workgroup at a cost above the direct reads).
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

template <int MX, bool AG>
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
    float *red = reinterpret_cast<float *>(smem + (AG ? 0 : (size_t)a.SB * 80 * MX * 16));

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

    // A operands.  Staged: unit = 8 consecutive k of one row (16 bytes),
    // copied into the LDS image; the groups a short last superblock lacks
    // are staged as zeros, so that their (unused) products are exact zeros.
    // Direct: each lane reads its own chunks (rows past M read row M - 1,
    // whose results are dropped; a group past G re-reads group G - 1, whose
    // products meet a zero scale), one superblock ahead like the codes.
    u32x4_t xa[2][2][kT5Groups], xn[2][2][kT5Groups];
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.x, (short)0, (int)((int64_t)a.M * a.K * 2), (int)kBufRaw);
    const int xvo = ((a_active ? nn : a.M - 1) * a.K + 16 * g) * 2;
    auto load_a = [&](int sb, u32x4_t (&dst)[2][2][kT5Groups]) {
#pragma unroll
        for (int j = 0; j < kT5Groups; ++j) {
            const int gi = kT5Groups * sb + j < a.G ? kT5Groups * sb + j : a.G - 1;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    dst[c][h][j] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo, 2 * (kGroup * gi + 64 * c + 8 * h), 0));
        }
    };
    if constexpr (AG) {
        if (any) load_a(sb_begin, xa);
    } else {
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
        if constexpr (AG) load_a(sb + 1 < sb_end ? sb + 1 : sb, xn);
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
                for (int j = 0; j < kT5Groups; ++j) {
                    if constexpr (AG)
                        xs[j] = xa[c][h][j];
                    else
                        xs[j] = a_active ? lds_x[t5_seg(sb, c, j, h, g, nn, MX)] : zero4;
                }
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
        if constexpr (AG) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < kT5Groups; ++j) xa[c][h][j] = xn[c][h][j];
        }
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

size_t t5_lds(int64_t K, int mx, int waves, bool ag)
{
    const int64_t SB = (K / kGroup + kT5Groups - 1) / kT5Groups;
    return (ag ? 0 : (size_t)SB * 80 * mx * 16) + (size_t)waves * mx * kTileN * sizeof(float);
}

int t5_waves(int64_t K)
{
    const int64_t SB = (K / kGroup + kT5Groups - 1) / kT5Groups;
    return SB >= 4 ? 4 : (SB >= 1 ? (int)SB : 1);
}

// Direct A loads from five rows on (every workgroup would otherwise copy
// 5..16 rows of x into LDS), or wherever the LDS copy would not fit.
bool t5_direct(int64_t K, int mx) { return mx > 4 || t5_lds(K, mx, t5_waves(K), false) > kMaxLds; }

template <int MX>
int launch_t5_mx(const T5Args &a, hipStream_t stream)
{
    const int waves = t5_waves(a.K);
    const bool ag = t5_direct(a.K, MX);
    const size_t lds = t5_lds(a.K, MX, waves, ag);
    void (*kernel)(T5Args) = ag ? gemv_t5_kernel<MX, true> : gemv_t5_kernel<MX, false>;
    int rc = ensure_lds(kernel, lds);
    if (rc) return rc;
    const unsigned wgs = (unsigned)((a.N + kTileN - 1) / kTileN);
    hipLaunchKernelGGL(kernel, dim3(wgs), dim3(64 * waves), lds, stream, a);
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
    const int mx = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    switch (mx) {
    case 1: return launch_t5_mx<1>(a, st);
    case 2: return launch_t5_mx<2>(a, st);
    case 4: return launch_t5_mx<4>(a, st);
    case 8: return launch_t5_mx<8>(a, st);
    default: return launch_t5_mx<16>(a, st);
    }
}

}  // namespace tern
