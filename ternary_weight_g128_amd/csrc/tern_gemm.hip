// Prefill-regime ternary-g128 matmul on gfx950 matrix cores.
//
// y[m][n] = sum_g s[n][g] sum_{k in g} t[n][k] x[m][k] ("prism-ml/Ternary-
// Bonsai-27B-mlx-2bit" model card, "Weight representation: ternary g128" and
// "CUDA (NVIDIA GPUs)": codes unpacked and scaled inside the kernel, never a
// dense FP16 weight tensor).  bfloat16 activations, binary32 result.
//
// Tiles.  A workgroup of four waves (2 x 2) computes a 256 (m) x 128 (n)
// output tile; a wave owns 128 x 64 as 4 x 2 sub-tiles of
// v_mfma_f32_32x32x16_bf16.  One 128-K scale group is one pipeline stage:
// the group's 256 x 128 activations (64 KiB) go straight from memory into
// LDS with buffer loads to LDS (no register staging), double buffered, while
// the matrix cores work on the previous group.  Rows past M read as zero
// through the buffer's range check.
//
// Operands.  For sub-tile column j, lane l holds output column l & 31 and
// lane group g = l >> 5 loads code words 4g..4g+3 of that column's group.
// Each word is first unshuffled (slots 0, 2, .., 14 to the low half, 1, 3,
// .., 15 to the high half), so that the packed 16-bit shift of neg2t_pair
// yields consecutive slot pairs: MFMA step kappa (0..7) then takes word
// 4g + (kappa >> 1), half kappa & 1, and its B element e is weight
// k = 64 g + 8 kappa + e of the group -- the same 8 consecutive k as the
// 16-byte activation chunk c = 8 g + kappa.  In LDS, row r of a stage is
// 256 bytes with chunk c stored at position c ^ (r & 15), which keeps the 16
// lanes of an LDS read phase on distinct banks.
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
// Work split (balanced K ranges).  The (tile, group) pairs are numbered
// unit = tile * G + group and cut into P equal contiguous ranges, one per
// workgroup and at most one workgroup per CU, so no CU idles through a
// short last round.  A workgroup walks its range tile by tile: a tile it
// covers from the first to the last group goes straight to y; a piece of a
// tile goes to a partial-sum slot (slot 0 for the first piece of the range,
// slot 1 for the last) and a second kernel adds each tile's pieces in K
// order, so the result does not depend on timing.  Consecutive tiles share a
// column block (the same codes), and consecutive ranges run on one XCD, so
// that XCD's L2 serves the codes to both row tiles.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

#include "tern_internal.h"

namespace {

#include "tern_device.h"

constexpr int kGemmBM = 128, kGemmBN = 512;
constexpr int kGemmWaves = 8;                              // one per 64 output columns
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmStages = 3;                             // x prefetched two groups ahead
constexpr int kGemmRowBytes = kGroup * 2;                  // one group of a bf16 row
constexpr int kGemmStageBytes = kGemmBM * kGemmRowBytes;   // 32 KiB
constexpr int kGemmDmaPerWave = kGemmStageBytes / (kGemmThreads * 16);  // 4
constexpr int kGemmTileElems = kGemmBM * kGemmBN;          // outputs per tile
constexpr int kGemmMinUnits = 4;                           // groups per range, at least
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
    float *partial;         // [P][2][kGemmTileElems], MFMA register order
    int64_t M, N;
    int K, G;               // G = K / 128
    int tiles_m;
    int P;                  // workgroups (ranges)
    int64_t units;          // tiles * G
};

// Weight operands without per-pair shifts.  For a code word w, plane s
// (s = 0..3) is ((w ^ 0x55555555) << (6 - 2 s)) & m: byte b of it holds the
// flipped slot 4 b + s at bits 7..6 and zeros elsewhere (m = 0xC0C0C0C0, or
// 0 for a zero-scale group).  A bfloat16 pair of the MFMA operand -- slots
// 2p and 2p + 1 at bits 15..14 and 31..30 -- is then one byte permute of
// two planes: byte p >> 1 of plane 2 (p & 1) into byte 1, the same byte of
// plane 2 (p & 1) + 1 into byte 3, zeros elsewhere.
constexpr unsigned kPlaneMask = 0xC0C0C0C0u;

__device__ __forceinline__ void code_planes(unsigned w, unsigned m, unsigned (&t)[4])
{
    t[0] = ((w << 6) ^ (kFlip << 6)) & m;
    t[1] = ((w << 4) ^ (kFlip << 4)) & m;
    t[2] = ((w << 2) ^ (kFlip << 2)) & m;
    t[3] = (w ^ kFlip) & m;
}

// MFMA B operand for slots 8h .. 8h + 7 of a word (element e = slot 8h + e).
__device__ __forceinline__ bf16x8_t operand_from_planes(const unsigned (&t)[4], int h)
{
    u32x4_t p;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int pair = 4 * h + v, b = pair >> 1;
        const unsigned sel = 0x0Cu | ((unsigned)b << 8) | (0x0Cu << 16) | ((4u + b) << 24);
        p[v] = (pair & 1) ? __builtin_amdgcn_perm(t[3], t[2], sel) : __builtin_amdgcn_perm(t[1], t[0], sel);
    }
    return __builtin_bit_cast(bf16x8_t, p);
}

// Range of logical workgroup w: units [w U / P, (w + 1) U / P).
__device__ __forceinline__ int64_t gemm_range_start(int64_t w, const GemmArgs &a)
{
    return w * a.units / a.P;
}

// Workgroups are dispatched round-robin over the 8 XCDs; number them so that
// each XCD gets a contiguous block of ranges.
__device__ __forceinline__ int gemm_logical_wg(int raw, int P)
{
    const int q = P >> 3, r = P & 7;
    const int xcd = raw & 7, k = raw >> 3;
    return xcd * q + (xcd < r ? xcd : r) + k;
}

// Position in the tile of accumulator element e in MFMA register order
// e = ((((wave * 4 + i) * 2 + j) * 16 + v) * 64 + lane): lane (c, g) of
// sub-tile (i, j) holds row 32 i + 8 (v >> 2) + 4 g + (v & 3), column
// 64 wave + 32 j + c.
__device__ __forceinline__ void gemm_elem_pos(int e, int &mr, int &nc)
{
    const int lane = e & 63, v = (e >> 6) & 15, j = (e >> 10) & 1, i = (e >> 11) & 3, wave = e >> 13;
    mr = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    nc = 64 * wave + 32 * j + (lane & 31);
}

__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const GemmArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, lg = lane >> 5;
    const int G = a.G;
    const int64_t KW = a.K / 16;
    const unsigned row_bytes = 2u * (unsigned)a.K;

    const int w = __builtin_amdgcn_readfirstlane(gemm_logical_wg(blockIdx.x, a.P));
    const int64_t u0 = gemm_range_start(w, a), u1 = gemm_range_start(w + 1, a);

    // Loads to LDS: wave instruction b fills 1 KiB = rows 16 wave + 4 b ..
    // + 3 of a stage; lane l writes position l & 15 of row 16 wave + 4 b +
    // (l >> 4), i.e. chunk (l & 15) ^ (row & 15) of that row.
    unsigned voff[kGemmDmaPerWave];
#pragma unroll
    for (int b = 0; b < kGemmDmaPerWave; ++b) {
        const unsigned r = 16 * wave + 4 * b + (lane >> 4);
        voff[b] = r * row_bytes + 16u * ((lane & 15) ^ (r & 15));
    }
    // A operand reads: row 32 i + col, chunk 8 lg + kappa at position
    // (8 lg + kappa) ^ (col & 15)
    const unsigned a_row = col * kGemmRowBytes;
    const unsigned a_sw = (8 * lg) ^ (col & 15);

    for (int64_t u = u0; u < u1;) {
        const int64_t tile = u / G;
        const int ka = (int)(u - tile * G);
        const int kb = (int)(u1 - tile * G < G ? u1 - tile * G : G);
        const int slot = u == u0 ? 0 : 1;
        u = tile * G + kb;

        const int64_t tm = tile % a.tiles_m, tn = tile / a.tiles_m;
        const int64_t m0 = tm * kGemmBM, n0 = tn * kGemmBN;
        const int64_t rows = a.M - m0 < kGemmBM ? a.M - m0 : kGemmBM;
        const uint16_t *xtile = a.x + m0 * a.K;
        const unsigned tile_bytes = (unsigned)rows * row_bytes;

        // this lane's code and scale rows (two sub-tile columns), clamped
        const uint32_t *crow[2];
        const uint16_t *srow[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int64_t n = n0 + 64 * wave + 32 * j + col;
            n = n < a.N ? n : a.N - 1;
            crow[j] = a.codes + n * KW + 4 * lg;
            srow[j] = a.scales + n * G;
        }

        // group g of the tile's rows into stage buffer sb
        auto stage = [&](int g, int sb) {
            __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(xtile + (int64_t)g * kGroup), (short)0, (int)(tile_bytes - 256u * (unsigned)g),
                (int)kBufferDword3);
            unsigned char *dst = smem + sb * kGemmStageBytes + wave * (kGemmDmaPerWave * 1024);
#pragma unroll
            for (int b = 0; b < kGemmDmaPerWave; ++b)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + 1024 * b), 16, voff[b], 0, 0, 0);
        };

        f32x16_t T[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) T[i][j][v] = 0.0f;
        float s_c[2];
        unsigned mask[2];
        u32x4_t cb[2];
        uint32_t s1[2];

        // prologue: activations of groups ka and ka + 1 (clamped) into
        // stages 0 and 1, codes and scale of group ka, scale of ka + 1
        stage(ka, 0);
        stage(ka + 1 < kb ? ka + 1 : ka, 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            cb[j] = *reinterpret_cast<const u32x4_t *>(crow[j] + (int64_t)ka * kWordsPerGroup);
            const float s0 = half_to_float(srow[j][ka]);
            s_c[j] = s0;
            mask[j] = s0 != 0.0f ? kPlaneMask : 0u;
            s1[j] = srow[j][ka + 1 < kb ? ka + 1 : ka];
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        int sb = 0;
        for (int gg = ka; gg < kb; ++gg) {
            const unsigned char *cur = smem + sb * kGemmStageBytes;
            const bool more = gg + 1 < kb;
            const int g1 = more ? gg + 1 : gg;               // codes: one group ahead
            const int g2 = gg + 2 < kb ? gg + 2 : kb - 1;    // scales, activations: two ahead
            const int sb2 = sb == 0 ? 2 : sb - 1;            // (sb + 2) % 3

            // issue order matters for the counted wait below: scales of g2,
            // codes of g1, then the activations of g2
            uint32_t s2[2];
            u32x4_t cbn[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) s2[j] = srow[j][g2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                cbn[j] = *reinterpret_cast<const u32x4_t *>(crow[j] + (int64_t)g1 * kWordsPerGroup);
            stage(g2, sb2);
            __builtin_amdgcn_sched_barrier(0);

            // rescale factor to group gg + 1 (its scale arrived a group ago)
            float r[2];
            unsigned mask_next[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float s_new = half_to_float((uint16_t)s1[j]);
                const bool nz = __builtin_unpredictable(more && s_new != 0.0f);  // selects, no branch
                const float ratio = s_c[j] * __builtin_amdgcn_rcpf(s_new);
                r[j] = nz ? ratio : 1.0f;
                mask_next[j] = __builtin_unpredictable(!more || s_new != 0.0f) ? kPlaneMask : 0u;
                s_c[j] = nz ? s_new : s_c[j];
            }

            const unsigned char *ap = cur + a_row;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned t[2][4];
#pragma unroll
                for (int j = 0; j < 2; ++j) code_planes(cb[j][q], mask[j], t[j]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kappa = 2 * q + h;
                    bf16x8_t aop[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        aop[i] = *reinterpret_cast<const bf16x8_t *>(ap + 32 * i * kGemmRowBytes +
                                                                     16 * (a_sw ^ kappa));
                    bf16x8_t bop[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) bop[j] = operand_from_planes(t[j], h);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            T[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop[j], T[i][j], 0, 0, 0);
                            // Horner step after each tile's last product of the group
                            if (kappa == 7) T[i][j] *= r[j];
                        }
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                cb[j] = cbn[j];
                s1[j] = s2[j];
                mask[j] = mask_next[j];
            }
            // everything but this group's activation prefetch has landed,
            // in particular the stage of group gg + 1; a plain barrier (no
            // memory fence, which would wait for the prefetch too) then
            // publishes it to all waves.  Every LDS read of this group was
            // consumed by an MFMA above, so the stage refilled next is free.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kGemmDmaPerWave));
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            sb = sb == 2 ? 0 : sb + 1;
        }

        // epilogue: lane (col, lg) of sub-tile (i, j) holds rows
        // 32 i + 8 (v >> 2) + 4 lg + (v & 3), column 64 wave + 32 j + col
        if (ka == 0 && kb == G) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t n = n0 + 64 * wave + 32 * j + col;
                const float f = -0.5f * s_c[j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t m = m0 + 32 * i + 8 * (v >> 2) + 4 * lg + (v & 3);
                        if (m < a.M && n < a.N) a.y[m * a.N + n] = T[i][j][v] * f;
                    }
            }
        } else {
            float *out = a.partial + ((int64_t)w * 2 + slot) * kGemmTileElems + wave * 8192 + lane;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float f = -0.5f * s_c[j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) out[((i * 2 + j) * 16 + v) * 64] = T[i][j][v] * f;
            }
        }
        // the next segment's prologue overwrites stages 0 and 1; the last
        // prefetch of this segment may still be landing in one of them
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

// Tiles split between workgroups: y = sum of the pieces in K order.
// grid (tiles, kGemmTileElems / 2048) x 256 threads, 8 outputs per thread.
__global__ __launch_bounds__(256) void gemm_fixup_kernel(const GemmArgs a)
{
    const int64_t tile = blockIdx.x;
    const int64_t first = tile * a.G, last = first + a.G - 1;
    // logical workgroup holding unit u: the largest w with w U / P <= u
    const int64_t wa = ((first + 1) * a.P - 1) / a.units;
    const int64_t wb = ((last + 1) * a.P - 1) / a.units;
    if (wa == wb) return;  // written directly
    const int64_t m0 = (tile % a.tiles_m) * kGemmBM, n0 = (tile / a.tiles_m) * kGemmBN;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = (blockIdx.y * 8 + k) * 256 + threadIdx.x;
        float s = 0.0f;
        for (int64_t w = wa; w <= wb; ++w) {
            const int slot = w * a.units / a.P >= first ? 0 : 1;
            s += a.partial[(w * 2 + slot) * kGemmTileElems + e];
        }
        int mr, nc;
        gemm_elem_pos(e, mr, nc);
        const int64_t m = m0 + mr, n = n0 + nc;
        if (m < a.M && n < a.N) a.y[m * a.N + n] = s;
    }
}

// K = 0: y = 0 (an empty sum).
__global__ __launch_bounds__(256) void fill_zero_kernel(float *y, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
        y[i] = 0.0f;
}

// P ranges of at least kGemmMinUnits groups, at most one per CU (the
// kernel's LDS, three 32 KiB stages, allows one workgroup per CU).
GemmArgs plan_gemm(int64_t M, int64_t N, int64_t K)
{
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = (int)K;
    a.G = (int)(K / kGroup);
    a.tiles_m = (int)((M + kGemmBM - 1) / kGemmBM);
    const int64_t tiles = a.tiles_m * ((N + kGemmBN - 1) / kGemmBN);
    a.units = tiles * a.G;
    int64_t P = a.units / kGemmMinUnits;
    const int cus = device_cus();
    P = P < cus ? P : cus;
    a.P = (int)(P < 1 ? 1 : P);
    return a;
}

bool gemm_splits_tiles(const GemmArgs &a)
{
    return a.units > 0 && !(a.units % a.P == 0 && (a.units / a.P) % a.G == 0);
}

}  // namespace

namespace tern {

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const GemmArgs a = plan_gemm(M, N, K);
    return gemm_splits_tiles(a) ? (size_t)a.P * 2 * kGemmTileElems * sizeof(float) : 0;
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
    GemmArgs a = plan_gemm(M, N, K);
    a.x = static_cast<const uint16_t *>(x);
    a.codes = codes;
    a.scales = scales;
    a.y = y;
    a.partial = static_cast<float *>(workspace);
    const size_t lds = kGemmStages * (size_t)kGemmStageBytes;
    int rc = ensure_lds(gemm_kernel, lds);
    if (rc) return rc;
    hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)a.P), dim3(kGemmThreads), lds, st, a);
    rc = (int)hipGetLastError();
    if (rc || !gemm_splits_tiles(a)) return rc;
    const int64_t tiles = a.units / a.G;
    hipLaunchKernelGGL(gemm_fixup_kernel, dim3((unsigned)tiles, kGemmTileElems / 2048), dim3(256), 0, st,
                       a);
    return (int)hipGetLastError();
}

}  // namespace tern
