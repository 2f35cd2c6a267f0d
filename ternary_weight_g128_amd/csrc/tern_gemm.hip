// Prefill-regime ternary-g128 matmul on gfx950 matrix cores.
//
// y[m][n] = sum_g s[n][g] sum_{k in g} t[n][k] x[m][k] ("prism-ml/Ternary-
// Bonsai-27B-mlx-2bit" model card, "Weight representation: ternary g128" and
// "CUDA (NVIDIA GPUs)": codes unpacked and scaled inside the kernel, never a
// dense FP16 weight tensor).  bfloat16 activations, binary32 result.
//
// Tiles.  A workgroup of four waves computes a 128 (m) x 128 (n) output
// tile; wave w owns columns 32w .. 32w + 31 as four 32-row sub-tiles of
// v_mfma_f32_32x32x16_bf16 (accumulators in VGPRs), so each weight operand
// it unpacks feeds four MFMAs.  Two workgroups share each CU, so every SIMD
// runs one wave of each; their barriers are independent, and one
// workgroup's barrier waits and VALU phases overlap the other's matrix
// work.  One 128-K scale group is one pipeline stage: the group's 128 x 128
// activations (32 KiB) go straight from memory into LDS with buffer loads
// to LDS (no register staging), two stages, one group ahead of the matrix
// cores; the loads are spread over the first half of the group's MFMA steps.
// The tile's code words travel two groups at a time (128 columns x 16
// words, 8 KiB, into one of two slots), so each column's load is 64
// contiguous bytes instead of 32: half the requests per code byte on the
// CU's texture path.  Rows past M read as zero through the buffer's range
// check.
//
// Operands.  For sub-tile column j, lane l holds output column l & 31 and
// lane group g = l >> 5 reads code words 4g..4g+3 of that column's group.
// Each word becomes four masked byte planes (code_planes: the flip, each
// slot moved to bits 7..6 of a byte, and the zero-scale mask, together), and
// each bfloat16 pair of the B operand is one byte permute of two planes
// (operand_from_planes).  MFMA step kappa (0..7) takes word 4g + (kappa >> 1),
// half kappa & 1, whose element e is slot 8 (kappa & 1) + e: weight
// k = 64 g + 8 kappa + e of the group -- the same 8 consecutive k as the
// 16-byte activation chunk c = 8 g + kappa.  In LDS, row r of a stage is
// 256 bytes with chunk c stored at position c ^ (r & 15), which keeps the 16
// lanes of an LDS read phase on distinct banks; a column's 64 code bytes
// hold 16-byte chunk q at position q ^ ((column >> 2) & 3), for the same
// reason.
//
// Scales (Horner form).  An accumulator holds its output in units of the
// current nonzero group scale s_c of its column: at a group boundary
// T <- T * (s_c / s_new), then the group's MFMAs add sum_k (-2t) x into T,
// and finally y = T * s_c * (-1/2).  This costs one multiply per accumulator
// per group and no second accumulator set; every product stays exact, and
// each rescale adds at most about two units of binary32 rounding to what
// was accumulated before it.  A group with a zero scale contributes nothing:
// its code words are masked to zero and s_c is kept.
//
// Work split.  P workgroups (at most two per CU) take whole tiles round
// robin for R = tiles / P rounds.  The r leftover tiles are cut along K into
// s equal pieces (s chosen on the host to balance the last round against the
// partial-sum traffic); piece j of the r * s goes to workgroup j mod P and
// into partial slot j, and a second kernel adds each leftover tile's s pieces
// in K order, so the result does not depend on timing.  Consecutive tiles
// share a column block (the same codes).

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

// Tile shape: MI 32-row and NJ 32-column sub-tiles per wave, four waves
// side by side along N, two activation stages in LDS.
template <int MI_, int NJ_>
struct GemmCfg {
    static constexpr int MI = MI_, NJ = NJ_;
    static constexpr int kWaves = 4;
    static constexpr int BM = 32 * MI, BN = 32 * NJ * kWaves;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRowBytes = kGroup * 2;                        // one group of a bf16 row
    static constexpr int kXBytes = BM * kRowBytes;                      // one group of activations
    static constexpr int kCPairBytes = BN * 2 * kWordsPerGroup * 4;     // code words of two groups
    static constexpr int kCBase = 2 * kXBytes;                          // code slots follow the stages
    static constexpr int kLdsBytes = kCBase + 2 * kCPairBytes;          // two code slots
    static constexpr int kDmaPerWave = kXBytes / (kThreads * 16);       // activation loads per group
    static constexpr int kCDmaPerWave = kCPairBytes / (kThreads * 16);  // code loads per pair
    static constexpr int kTileElems = BM * BN;
    static_assert(kLdsBytes * 2 <= 160 * 1024, "LDS for two workgroups per CU");
};
// 128 x 128 tiles: each wave 128 x 32, so one weight operand feeds four
// MFMAs
typedef GemmCfg<4, 1> GemmTile;
constexpr int kGemmWgPerCu = 2;                            // independent workgroups per CU
constexpr int kGemmThreads = GemmTile::kThreads;
constexpr int kGemmTileElems = GemmTile::kTileElems;       // outputs per tile
constexpr int kGemmMinPiece = 4;                           // groups per K piece, at least
constexpr unsigned kBufferDword3 = 0x00020000u;            // raw buffer, 32-bit data format
// s_waitcnt operand: vmcnt(n), expcnt and lgkmcnt not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct GemmArgs {
    const uint16_t *x;      // bf16 [M][K]
    const uint32_t *codes;  // [N][K/16]
    const uint16_t *scales; // [N][K/128]
    float *y;               // [M][N]
    float *partial;         // [r * s][kGemmTileElems], MFMA register order
    int64_t M, N;
    int K, G;               // G = K / 128
    int tiles_m;
    int P;                  // workgroups
    int64_t tiles;          // tiles_m * tiles_n
    int64_t full;           // R * P: tiles done whole, round robin
    int split;              // s: K pieces of each leftover tile (1: none left)
    int64_t items;          // r * s leftover pieces
    bool y_vec;             // y 16-byte aligned and N % 4 == 0
};

// One 16-byte buffer load per lane straight into LDS (lane l writes dst +
// 16 l).  A plain device function: with the builtin written inside a kernel
// template, the host pass of this compiler drops the template's launch stub.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, unsigned voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, 0, 0, 0);
}

// Position in the tile of accumulator element e in MFMA register order
// e = ((((wave * MI + i) * NJ + j) * 16 + v) * 64 + lane): lane (c, g) of
// sub-tile (i, j) holds row 32 i + 8 (v >> 2) + 4 g + (v & 3), column
// 32 (NJ wave + j) + c.
template <class C>
__device__ __forceinline__ void gemm_elem_pos(int e, int &mr, int &nc)
{
    const int lane = e & 63, v = (e >> 6) & 15, ij = e >> 10;
    const int j = ij % C::NJ, i = (ij / C::NJ) % C::MI, wave = ij / (C::NJ * C::MI);
    mr = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    nc = 32 * (C::NJ * wave + j) + (lane & 31);
}

template <class C>
__global__ __launch_bounds__(kGemmThreads, kGemmWgPerCu) void gemm_kernel(const GemmArgs a)
{
    constexpr int MI = C::MI, NJ = C::NJ;
    constexpr int kGemmBM = C::BM, kGemmBN = C::BN, kGemmRowBytes = C::kRowBytes, kGemmXBytes = C::kXBytes;
    constexpr int kGemmCPairBytes = C::kCPairBytes, kGemmCBase = C::kCBase;
    constexpr int kGemmDmaPerWave = C::kDmaPerWave, kGemmCDmaPerWave = C::kCDmaPerWave;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, lg = lane >> 5;
    const int G = a.G;
    const int64_t KW = a.K / 16;
    const unsigned row_bytes = 2u * (unsigned)a.K;

    const int w = blockIdx.x;
    // work items: whole tiles w, w + P, .. below a.full, then leftover
    // pieces j = w, w + P, .. below a.items
    const int64_t n_full = w < a.full % a.P ? a.full / a.P + 1 : a.full / a.P;
    const int64_t n_part = a.items > w ? (a.items - 1 - w) / a.P + 1 : 0;

    // Loads to LDS (D = kGemmDmaPerWave per wave): wave instruction b fills
    // 1 KiB = rows 4 (D wave + b) .. + 3 of a stage; lane l writes position
    // l & 15 of its row, i.e. chunk (l & 15) ^ (row & 15) of that row.
    unsigned voff[kGemmDmaPerWave];
#pragma unroll
    for (int b = 0; b < kGemmDmaPerWave; ++b) {
        const unsigned r = 4 * (kGemmDmaPerWave * wave + b) + (lane >> 4);
        voff[b] = r * row_bytes + 16u * ((lane & 15) ^ (r & 15));
    }
    // Code words of two groups to LDS (D' = kGemmCDmaPerWave per wave): wave
    // instruction b fills 1 KiB = columns 16 (D' wave + b) .. + 15 of the
    // tile (64 bytes each: the two
    // groups' 16 words, as four 16-byte chunks q = 2 (group in pair) +
    // half); lane l writes position l & 3 of column (l >> 2), which holds
    // chunk (l & 3) ^ ((column >> 2) & 3), so that 16 lanes reading the
    // same chunk of 16 columns hit distinct banks.
    unsigned coff[kGemmCDmaPerWave];
#pragma unroll
    for (int b = 0; b < kGemmCDmaPerWave; ++b) {
        const unsigned c = 16 * (kGemmCDmaPerWave * wave + b) + (lane >> 2);
        coff[b] = c * (unsigned)(a.K / 4) + 16u * ((lane & 3) ^ ((c >> 2) & 3));
    }
    // A operand reads: row 32 i + col, chunk 8 lg + kappa at position
    // (8 lg + kappa) ^ (col & 15)
    const unsigned a_row = col * kGemmRowBytes;
    const unsigned a_sw = (8 * lg) ^ (col & 15);

    for (int64_t it = 0; it < n_full + n_part; ++it) {
        const bool whole = it < n_full;
        const int64_t pj = (it - n_full) * a.P + w;           // leftover piece
        const int64_t tile = whole ? w + it * a.P : a.full + pj / a.split;
        const int piece = whole ? 0 : (int)(pj % a.split);
        const int ka = whole ? 0 : (int)((int64_t)piece * G / a.split);
        const int kb = whole ? G : (int)((int64_t)(piece + 1) * G / a.split);

        const int64_t tm = tile % a.tiles_m, tn = tile / a.tiles_m;
        const int64_t m0 = tm * kGemmBM, n0 = tn * kGemmBN;
        const int64_t rows = a.M - m0 < kGemmBM ? a.M - m0 : kGemmBM;
        const uint16_t *xtile = a.x + m0 * a.K;
        const unsigned tile_bytes = (unsigned)rows * row_bytes;

        // this lane's scale rows (one per sub-tile column), clamped
        const uint16_t *srow[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            int64_t n = n0 + 32 * (NJ * wave + j) + col;
            n = n < a.N ? n : a.N - 1;
            srow[j] = a.scales + n * G;
        }
        const int64_t cols = a.N - n0 < kGemmBN ? a.N - n0 : kGemmBN;
        const uint32_t *ctile = a.codes + n0 * KW;
        const unsigned ctile_bytes = (unsigned)cols * (unsigned)(a.K / 4);

        // group g of the tile's activations into stage sb, and the code
        // words of groups g0, g0 + 1 into code slot cs (columns past N read
        // as zero words, their outputs are dropped; a group past the piece
        // reads words that are never used)
        auto x_rsrc = [&](int g) {
            return __builtin_amdgcn_make_buffer_rsrc((void *)(xtile + (int64_t)g * kGroup), (short)0,
                                                     (int)(tile_bytes - 256u * (unsigned)g), (int)kBufferDword3);
        };
        auto x_dst = [&](int sb) { return smem + sb * kGemmXBytes + wave * (kGemmDmaPerWave * 1024); };
        auto stage_x = [&](int g, int sb) {
            const __amdgpu_buffer_rsrc_t rs = x_rsrc(g);
            unsigned char *dst = x_dst(sb);
#pragma unroll
            for (int b = 0; b < kGemmDmaPerWave; ++b)
                load_lds16(rs, dst + 1024 * b, voff[b]);
        };
        auto stage_c = [&](int g0, int cs) {
            __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(ctile + (int64_t)g0 * kWordsPerGroup), (short)0, (int)(ctile_bytes - 32u * (unsigned)g0),
                (int)kBufferDword3);
            unsigned char *cdst = smem + kGemmCBase + cs * kGemmCPairBytes + wave * (kGemmCDmaPerWave * 1024);
#pragma unroll
            for (int b = 0; b < kGemmCDmaPerWave; ++b)
                load_lds16(rc, cdst + 1024 * b, coff[b]);
        };
        // this lane's four code words of sub-tile column j, first group of a
        // pair, within a code slot (the second group: chunk position ^ 2)
        unsigned c_lds[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const unsigned c = 32 * (NJ * wave + j) + col;
            c_lds[j] = kGemmCBase + c * 64 + 16 * (lg ^ ((c >> 2) & 3));
        }

        f32x16_t T[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
                for (int v = 0; v < 16; ++v) T[i][jj][v] = 0.0f;
        float s_c[NJ];
        unsigned mask[NJ];
        uint32_t s1[NJ];          // scale bits of group gg + 1
        auto gcl = [&](int g) { return g < kb ? g : kb - 1; };

        // prologue: activations of group ka into stage 0, the code words of
        // groups ka and ka + 1 into slot 0; scales of groups ka and ka + 1
        stage_x(ka, 0);
        stage_c(ka, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float s0 = half_to_float(srow[j][ka]);
            s_c[j] = s0;
            mask[j] = s0 != 0.0f ? kPlaneMask : 0u;
            s1[j] = srow[j][gcl(ka + 1)];
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        int sb = 0;  // activation stage of group gg
        int cs = 0;  // code slot of the pair holding group gg
        // One group.  The first group of a pair (counted from ka) also
        // issues the code words of the next pair, into the other slot.
        auto group = [&](auto first_of_pair, int gg) {
            constexpr bool kFirst = decltype(first_of_pair)::value;
            const unsigned char *cur = smem + sb * kGemmXBytes;
            const unsigned char *ccur = smem + cs * kGemmCPairBytes;
            const bool more = gg + 1 < kb;
            const int g2 = gcl(gg + 2);

            // Scales of group gg + 2 go out first (tiny loads).  The
            // activations of gg + 1 go into the stage gg - 1 left (all its
            // reads were consumed before the last barrier), a few loads with
            // each of the first four MFMA steps, and the next pair's codes
            // mid-group: issued together, all waves' loads queue at the CU's
            // address unit and hold up the MFMAs behind them.
            uint32_t s2[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) s2[j] = srow[j][g2];
            constexpr int kXPerStep = (kGemmDmaPerWave + 3) / 4;
            const __amdgpu_buffer_rsrc_t nrs = x_rsrc(gcl(gg + 1));
            unsigned char *const ndst = x_dst(sb ^ 1);
            __builtin_amdgcn_sched_barrier(0);

            // rescale factor to group gg + 1 (its scale arrived a group ago)
            float r[NJ];
            unsigned mask_next[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float s_new = half_to_float((uint16_t)s1[j]);
                const bool nz = __builtin_unpredictable(more && s_new != 0.0f);  // selects, no branch
                const float ratio = s_c[j] * __builtin_amdgcn_rcpf(s_new);
                r[j] = nz ? ratio : 1.0f;
                mask_next[j] = __builtin_unpredictable(!more || s_new != 0.0f) ? kPlaneMask : 0u;
                s_c[j] = nz ? s_new : s_c[j];
            }

            u32x4_t cw[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                cw[j] = *reinterpret_cast<const u32x4_t *>(ccur + (c_lds[j] ^ (kFirst ? 0u : 32u)));
            const unsigned char *ap = cur + a_row;
            // activation operands one step ahead of the MFMAs that use them
            bf16x8_t aop[MI], anx[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                aop[i] = *reinterpret_cast<const bf16x8_t *>(ap + 32 * i * kGemmRowBytes + 16 * a_sw);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (kFirst && q == 2) {
                    __builtin_amdgcn_sched_barrier(0);
                    stage_c(g2, cs ^ 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                unsigned t[NJ][4];
#pragma unroll
                for (int j = 0; j < NJ; ++j) code_planes(cw[j][q], mask[j], t[j]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kappa = 2 * q + h;
                    if (kappa * kXPerStep < kGemmDmaPerWave) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int b = kappa * kXPerStep; b < (kappa + 1) * kXPerStep && b < kGemmDmaPerWave; ++b)
                            load_lds16(nrs, ndst + 1024 * b, voff[b]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (kappa < 7) {
#pragma unroll
                        for (int i = 0; i < MI; ++i)
                            anx[i] = *reinterpret_cast<const bf16x8_t *>(ap + 32 * i * kGemmRowBytes +
                                                                         16 * (a_sw ^ (kappa + 1)));
                    }
                    bf16x8_t bop[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) bop[j] = operand_from_planes(t[j], h);
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j) {
                            T[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop[j], T[i][j], 0, 0, 0);
                            // Horner step after each tile's last product of the group
                            if (kappa == 7) T[i][j] *= r[j];
                        }
                    if (kappa < 7) {
#pragma unroll
                        for (int i = 0; i < MI; ++i) aop[i] = anx[i];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                s1[j] = s2[j];
                mask[j] = mask_next[j];
            }
            // Everything but the next pair's codes (in flight after the
            // first group of a pair) has landed: the activations of group
            // gg + 1 and, after the second group of a pair, the codes of the
            // next pair.  A plain barrier (no memory fence, which would wait
            // for the codes too) publishes them to all waves.  Every LDS read
            // of this group was consumed above, so the stage and code slot
            // refilled next are free.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kFirst ? kGemmCDmaPerWave : 0));
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            sb ^= 1;
            if constexpr (!kFirst) cs ^= 1;
        };
        int gg = ka;
        for (; gg + 1 < kb; gg += 2) {
            group(std::true_type{}, gg);
            group(std::false_type{}, gg + 1);
        }
        if (gg < kb) group(std::true_type{}, gg);

        // epilogue: lane (col, lg) of sub-tile (i, j) holds rows
        // 32 i + 8 (v >> 2) + 4 lg + (v & 3), column 32 (NJ wave + j) + col
        if (whole) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int64_t n = n0 + 32 * (NJ * wave + j) + col;
                const float f = -0.5f * s_c[j];
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t m = m0 + 32 * i + 8 * (v >> 2) + 4 * lg + (v & 3);
                        if (m < a.M && n < a.N) a.y[m * a.N + n] = T[i][j][v] * f;
                    }
            }
        } else {
            float *out = a.partial + pj * kGemmTileElems + wave * (MI * NJ * 1024) + lane;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float f = -0.5f * s_c[j];
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) out[((i * NJ + j) * 16 + v) * 64] = T[i][j][v] * f;
            }
        }
        // the next item's prologue overwrites the first stages and code
        // slot 0; the last prefetches of this item may still be landing
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

// Leftover tiles: y = sum of their a.split K pieces, in K order.
// grid (leftover tiles, kGemmTileElems / 1024) x 256 threads, four outputs
// per thread: elements 4t .. 4t + 3 of the register order are four
// consecutive columns of one row, so they are one 16-byte load per piece and
// one 16-byte store.  The piece loads are issued together (up to 8 at a
// time) and added in K order.
template <class C>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(const GemmArgs a)
{
    const int64_t lt = blockIdx.x;                 // leftover tile
    const int64_t tile = a.full + lt;
    const int64_t m0 = (tile % a.tiles_m) * C::BM, n0 = (tile / a.tiles_m) * C::BN;
    const int e = 4 * (blockIdx.y * 256 + threadIdx.x);
    const f32x4_t *src = reinterpret_cast<const f32x4_t *>(a.partial + lt * a.split * kGemmTileElems + e);
    constexpr int kPieceVecs = kGemmTileElems / 4;
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < a.split; p0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = p0 + q < a.split ? src[(int64_t)(p0 + q) * kPieceVecs] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (p0 + q < a.split) s += v[q];
    }
    int mr, nc;
    gemm_elem_pos<C>(e, mr, nc);
    const int64_t m = m0 + mr, n = n0 + nc;
    if (m >= a.M) return;
    float *yp = a.y + m * a.N + n;
    if (a.y_vec && n + 3 < a.N) {
        *reinterpret_cast<f32x4_t *>(yp) = s;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (n + c < a.N) yp[c] = s[c];
    }
}

// K = 0: y = 0 (an empty sum).
__global__ __launch_bounds__(256) void fill_zero_kernel(float *y, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
        y[i] = 0.0f;
}

// Work split over C = 2 x #CUs workgroups (two per CU, which the LDS stages
// allow): R = tiles / C rounds of whole tiles, then the
// r = tiles mod C leftover tiles in s K pieces each.  s minimises the
// modelled time in units of one tile-group on one CU (~1.5 us): the busiest
// workgroup's groups plus the round trip of all partial sums through HBM
// (the whole GPU moves about 6 MiB in that time).  P workgroups run: C, or
// fewer when there are fewer work items.
template <class C>
GemmArgs plan_gemm(int64_t M, int64_t N, int64_t K)
{
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = (int)K;
    a.G = (int)(K / kGroup);
    a.tiles_m = (int)((M + C::BM - 1) / C::BM);
    a.tiles = a.tiles_m * ((N + C::BN - 1) / C::BN);
    const int64_t W = kGemmWgPerCu * (int64_t)device_cus();
    const int64_t R = a.tiles / W, r = a.tiles - R * W;
    a.split = 1;
    if (r > 0) {
        const double piece_cost = 2.0 * kGemmTileElems * 4 / (6.0 * 1024 * 1024);  // in group times
        double best = 0.0;
        const int smax = a.G / kGemmMinPiece > 1 ? a.G / kGemmMinPiece : 1;
        for (int sp = 1; sp <= smax; ++sp) {
            const int64_t per_wg = (r * sp + W - 1) / W;                // pieces on the busiest workgroup
            const int64_t longest = (a.G + sp - 1) / sp;
            const double t = (double)(R * a.G + per_wg * longest) + (sp > 1 ? piece_cost * (double)(r * sp) : 0.0);
            if (sp == 1 || t < best) {
                best = t;
                a.split = sp;
            }
        }
    }
    if (a.split == 1) {  // every tile done whole
        a.full = a.tiles;
        a.items = 0;
        a.P = (int)(a.tiles < W ? a.tiles : W);
    } else {
        a.full = R * W;
        a.items = r * a.split;
        a.P = (int)(R > 0 || a.items >= W ? W : a.items);
    }
    return a;
}

bool gemm_splits_tiles(const GemmArgs &a) { return a.items > 0; }

typedef GemmTile GemmUse;  // the tile shape every call runs

}  // namespace

// Scratch of the allocation-free entry point: the partial sums of K-split
// tiles.  Every device holds its own instance until the process ends.  In
// host code the array's name is not a device address: its address on each
// device comes from hipGetSymbolAddress (gemm_scratch below).
static __device__ __align__(256) unsigned char scratch[TERN_GEMM_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current.
int gemm_scratch(void *stream, void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return (int)e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return (int)e;
        if (p == nullptr) return (int)hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

}  // namespace

namespace tern {

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const GemmArgs a = plan_gemm<GemmUse>(M, N, K);
    return gemm_splits_tiles(a) ? (size_t)a.items * kGemmTileElems * sizeof(float) : 0;
}

int64_t gemm_max_k() { return ((int64_t)1 << 22) - kGroup; }

int launch_gemm(const void *x, int64_t M, int64_t K, const uint32_t *codes, const uint16_t *scales,
                int64_t N, float *y, void *workspace, size_t, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t count = M * N;
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                           st, y, count);
        return (int)hipGetLastError();
    }
    GemmArgs a = plan_gemm<GemmUse>(M, N, K);
    a.x = static_cast<const uint16_t *>(x);
    a.codes = codes;
    a.scales = scales;
    a.y = y;
    a.partial = static_cast<float *>(workspace);
    const size_t lds = GemmUse::kLdsBytes;
    int rc = ensure_lds(gemm_kernel<GemmUse>, lds);
    if (rc) return rc;
    hipLaunchKernelGGL(gemm_kernel<GemmUse>, dim3((unsigned)a.P), dim3(kGemmThreads), lds, st, a);
    rc = (int)hipGetLastError();
    if (rc || !gemm_splits_tiles(a)) return rc;
    a.y_vec = reinterpret_cast<uintptr_t>(y) % 16 == 0 && N % 4 == 0;
    hipLaunchKernelGGL(gemm_fixup_kernel<GemmUse>, dim3((unsigned)(a.items / a.split), kGemmTileElems / 1024), dim3(256),
                       0, st, a);
    return (int)hipGetLastError();
}

int launch_gemm_noalloc(const void *x, int64_t M, int64_t K, const uint32_t *codes, const uint16_t *scales,
                        int64_t N, float *y, void *stream)
{
    const size_t need = gemm_workspace_bytes(M, N, K);
    void *ws = nullptr;
    if (need > 0) {
        int rc = gemm_scratch(stream, &ws);
        if (rc) return rc;
    }
    return launch_gemm(x, M, K, codes, scales, N, y, ws, need, stream);
}

}  // namespace tern
