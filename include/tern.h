/*
 * tern.h -- C ABI of libtern: ternary-g128 weights on AMD MI355X (gfx950).
 *
 * The weight format ("prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card,
 * sections "Weight representation: ternary g128" and "Memory requirement"):
 * every weight is t in {-1, 0, +1}; each run of 128 consecutive weights along
 * K in one output row shares one IEEE binary16 scale s_g, so the weight value
 * is w = s_g * t; each t is stored in a 2-bit slot, 2.125 bits per weight.
 *
 * The matmul ("CUDA (NVIDIA GPUs)" section of the same card) unpacks the
 * codes and applies the group scales inside the kernel; the weights are never
 * expanded to a dense FP16 tensor in memory.
 *
 * The optional activation rotation ("Ternary-Bonsai-2-9B-2bit" article,
 * section 3, "Ternary weights and Hadamard rotation") is a normalized
 * Sylvester-Walsh-Hadamard transform with an explicit +-1 sign pattern over
 * blocks of the last dimension (block 4096 in that model); the rotation is
 * folded into the stored weights and the matching transform is applied to
 * activations at run time, forward and inverse.
 *
 * Layouts (all row-major, K contiguous):
 *   x      [M][K]      activations, binary32 or bfloat16
 *   codes  [N][K/16]   uint32; slot j of word w of row n holds
 *                      q = t[n][16w + j] + 1 at bits 2j..2j+1 (q = 3 unused)
 *   scales [N][K/128]  binary16 bit patterns
 *   y      [M][N]      binary32 (or bfloat16 where stated)
 *
 * Conventions for every call:
 *   - The caller owns and allocates every buffer; the library allocates
 *     nothing.  Host-codec calls take host pointers and are synchronous.
 *     Device calls take device pointers on the current HIP device and are
 *     enqueued on `stream` (a hipStream_t; NULL is the null stream); they
 *     return once the work is enqueued.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a status and launches nothing.  tern_last_error()
 *     then holds a one-line reason (thread-local).  No exception crosses the
 *     ABI.  A HIP launch failure returns TERN_EDEVICE with the HIP message.
 *   - M, N, K are >= 0; a zero M or N writes nothing; K = 0 writes zeros
 *     (an empty sum).  K must be a multiple of 128 (whole scale groups).
 *   - Device kernels do not check code values: a slot holding 3 gives an
 *     unspecified result (it is never produced by the packer).
 *   - Results are bitwise reproducible run to run for the same arguments.
 *   - Calls are stateless and may be made from several host threads.
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tern_status {
    TERN_OK = 0,
    TERN_EINVAL = 1,        /* bad size, pointer, alignment or non-finite scale */
    TERN_ENOTTERNARY = 2,   /* input values are not ternary-g128 */
    TERN_EBADCODE = 3,      /* a 2-bit slot holds the unused value 3 */
    TERN_EUNSUPPORTED = 4,  /* valid request that the library does not implement */
    TERN_EDEVICE = 5        /* HIP runtime error */
} tern_status;

typedef enum tern_dtype {
    TERN_F32 = 0,           /* IEEE binary32 */
    TERN_BF16 = 1,          /* bfloat16 (upper half of binary32) */
    TERN_F16 = 2            /* IEEE binary16: named for completeness; no device
                               call takes it (TERN_EUNSUPPORTED).  The scales
                               are binary16 bit patterns, passed as uint16. */
} tern_dtype;

#define TERN_GROUP 128            /* weights per FP16 scale */
#define TERN_SLOTS_PER_WORD 16    /* 2-bit slots per uint32 code word */
#define TERN_GEMV_MAX_M 16        /* rows of x one tern_gemv call takes */
#define TERN_FWHT_MAX_BLOCK 4096  /* largest Hadamard block tern_fwht takes */
#define TERN_MAX_K 2147483520     /* INT32_MAX - 127: largest K of a device matmul */
#define TERN_ABI_VERSION 1

/* ABI version of the loaded library (TERN_ABI_VERSION it was built with). */
int tern_abi_version(void);

/* Static name of a status code ("TERN_OK", ...); "unknown" otherwise. */
const char *tern_status_str(int status);

/* Reason for the last non-OK status returned on this host thread, or "". */
const char *tern_last_error(void);

/* ---------------------------------------------------------------------------
 * Storage accounting ("Memory requirement": 2-bit slots + one FP16 scale per
 * 128 weights = 2.125 bits/weight).  Pure functions; 0 for invalid sizes
 * (negative, or K not a multiple of 128).
 * ------------------------------------------------------------------------ */
size_t tern_codes_bytes(int64_t N, int64_t K);   /* N*K/4  */
size_t tern_scales_bytes(int64_t N, int64_t K);  /* 2*N*K/128 */

/* ---------------------------------------------------------------------------
 * Host codec (lossless transcode into the 2-bit g128 slot format; the
 * "Ternary-Bonsai-2-9B-2bit" article, section 3, describes the transcode as
 * lossless).  Host pointers, caller-owned, synchronous.
 * ------------------------------------------------------------------------ */

/* Pack t[N][K] (int8, each -1, 0 or +1) into codes[N][K/16] and copy the
 * binary16 scales s_f16[N][K/128] to s_out (s_out may equal s_f16).
 * Errors: TERN_EINVAL (sizes, NULL, K % 128, a non-finite scale),
 * TERN_ENOTTERNARY (some t outside {-1,0,1}; codes then undefined). */
tern_status tern_pack(const int8_t *t, const uint16_t *s_f16, int64_t N, int64_t K,
                      uint32_t *codes, uint16_t *s_out);

/* Lossless reading of FP32 weights w[N][K] as ternary-g128: a group is
 * accepted iff all its nonzero |w| equal one value a that binary16
 * represents exactly; then s = a (+0 for an all-zero group) and t = sign(w).
 * This is not a quantizer: any other group gives TERN_ENOTTERNARY.
 * Outputs codes[N][K/16] and s_out[N][K/128]. */
tern_status tern_pack_f32(const float *w, int64_t N, int64_t K,
                          uint32_t *codes, uint16_t *s_out);

/* Decode codes[N][K/16] into t[N][K] (int8).  TERN_EBADCODE if a slot holds 3. */
tern_status tern_unpack(const uint32_t *codes, int64_t N, int64_t K, int8_t *t);

/* Dense w[N][K] = s_g * t in binary32 (exact).  TERN_EBADCODE on slot 3. */
tern_status tern_dequant_f32(const uint32_t *codes, const uint16_t *s_f16,
                             int64_t N, int64_t K, float *w);

/* ---------------------------------------------------------------------------
 * Format variants ("prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card).
 * Host pointers, caller-owned, synchronous; K a multiple of 128 throughout.
 * Each variant converts to and from the g128 slot format exactly, so the
 * device kernels above serve all of them.
 * ------------------------------------------------------------------------ */

/* Group-size-64 variant ("Shipped components"): the same codes, with each
 * g128 scale repeated for both 64-value halves of its group; 2.25 bits per
 * weight.  Scale array [N][K/64]. */
size_t tern_scales_g64_bytes(int64_t N, int64_t K);  /* 2*N*K/64 */

/* s[N][K/128] -> s64[N][K/64], s64[n][2g] = s64[n][2g+1] = s[n][g].  s64 may
 * start at s (in-place widening; the buffer must hold N*K/64 values).
 * Errors: TERN_EINVAL (sizes, NULL). */
tern_status tern_scales_to_g64(const uint16_t *s, int64_t N, int64_t K, uint16_t *s64);

/* s64[N][K/64] -> s[N][K/128] (s may start at s64).  Every pair of halves must
 * hold equal values (the first of the pair is kept): TERN_ENOTTERNARY if
 * not, since such a matrix has no g128 form; TERN_EINVAL for a non-finite
 * scale, bad sizes or NULL.  Nothing is written on error. */
tern_status tern_scales_from_g64(const uint16_t *s64, int64_t N, int64_t K, uint16_t *s);

/* Affine scale+bias container ("MLX packaging": a binary16 scale and bias per
 * group of 128, weight = scale * q + bias, 2.25 bits per weight).  The 2-bit
 * fields are the slot codes unchanged (q = t + 1, lowest field first), and a
 * ternary group exports as (scale, bias) = (s, -s), so scale * q + bias =
 * s * t exactly.  (The pair (2s, -s) that section prints has no zero level on
 * 2-bit fields; it is the pair of the binary variant, tern_mlx_export_b1.)
 * Outputs mlx_scales, mlx_biases [N][K/128].  Errors: TERN_EINVAL (sizes,
 * NULL, a non-finite scale). */
tern_status tern_mlx_export(const uint16_t *s, int64_t N, int64_t K,
                            uint16_t *mlx_scales, uint16_t *mlx_biases);

/* Inverse of tern_mlx_export: s = mlx_scales (s may equal mlx_scales).
 * TERN_ENOTTERNARY if some group has bias != -scale (by value); TERN_EINVAL
 * for non-finite values, bad sizes or NULL.  Nothing is written on error. */
tern_status tern_mlx_import(const uint16_t *mlx_scales, const uint16_t *mlx_biases,
                            int64_t N, int64_t K, uint16_t *s);

/* Binary g128 variant (the 1-bit model of the "Benchmarks" variant table,
 * 1.125 bits per weight): b in {-1, +1}, one bit per weight, bit j of word w
 * of row n holds k = 32w + j (1 for +1, 0 for -1, lowest bit first), and the
 * same binary16 scale per 128 as the ternary format.  Bit words [N][K/32]. */
#define TERN_B1_PER_WORD 32
size_t tern_b1_bytes(int64_t N, int64_t K);  /* N*K/8 */

/* b[N][K] int8 (each -1 or +1) -> bits[N][K/32].
 * Errors: TERN_EINVAL (sizes, NULL), TERN_ENOTTERNARY (a value not +-1;
 * bits then undefined). */
tern_status tern_pack_b1(const int8_t *b, int64_t N, int64_t K, uint32_t *bits);

/* bits[N][K/32] -> b[N][K] in {-1, +1}.  Errors: TERN_EINVAL. */
tern_status tern_unpack_b1(const uint32_t *bits, int64_t N, int64_t K, int8_t *b);

/* Binary weights as ternary slot codes (t = b, so q = 2 * bit), for the
 * g128 kernels: bits[N][K/32] -> codes[N][K/16]; the scales carry over
 * unchanged.  Errors: TERN_EINVAL. */
tern_status tern_b1_to_codes(const uint32_t *bits, int64_t N, int64_t K, uint32_t *codes);

/* Ternary slot codes with no zero weight -> bits.  TERN_ENOTTERNARY if some
 * t = 0 (no binary code), TERN_EBADCODE for slot value 3; bits then
 * undefined.  Errors also TERN_EINVAL. */
tern_status tern_codes_to_b1(const uint32_t *codes, int64_t N, int64_t K, uint32_t *bits);

/* Affine container of the binary variant with 1-bit fields ("MLX packaging"
 * pair): (scale, bias) = (2s, -s), so scale * bit + bias = +-s exactly; the
 * bit words are used unchanged (1.25 bits per weight).  TERN_EINVAL if some
 * |s| >= 32768 (2s overflows binary16) or is not finite. */
tern_status tern_mlx_export_b1(const uint16_t *s, int64_t N, int64_t K,
                               uint16_t *mlx_scales, uint16_t *mlx_biases);

/* Inverse: s = -bias.  TERN_ENOTTERNARY if some group has scale != -2 * bias
 * (by value); TERN_EINVAL for non-finite values, bad sizes or NULL. */
tern_status tern_mlx_import_b1(const uint16_t *mlx_scales, const uint16_t *mlx_biases,
                               int64_t N, int64_t K, uint16_t *s);

/* ---------------------------------------------------------------------------
 * Base-3 layout below two bits per weight.  "Memory requirement" notes that
 * 2-bit slots cost 2.125 bits/weight against about 1.71 for the information
 * content, to be closed by native ternary kernels; the layout is not given,
 * and this one is ours: five ternary values per byte (3^5 = 243 <= 256).
 * The groups of 128 of a row are taken five at a time; superblock b (128
 * bytes) holds groups 5b .. 5b + p - 1, p = min(5, K/128 - 5b), and its byte i
 * holds sum_{j<p} (t + 1) 3^j over weights k = 128 (5b + j) + i.  A row is
 * ceil(K/640) * 128 bytes (1.6 bits/weight when K is a multiple of 640); the
 * binary16 scales [N][K/128] are unchanged.  data: uint8 [N][ceil(K/640)*128].
 * ------------------------------------------------------------------------ */
size_t tern_t5_bytes(int64_t N, int64_t K);

/* 2-bit slot codes [N][K/16] -> base-3 data.  TERN_EBADCODE for slot value 3
 * (data then undefined); TERN_EINVAL for sizes or NULL.  Host pointers. */
tern_status tern_pack_t5(const uint32_t *codes, int64_t N, int64_t K, uint8_t *data);

/* Base-3 data -> 2-bit slot codes.  TERN_EBADCODE if a byte is not below
 * 3^p for its superblock (codes then undefined); TERN_EINVAL.  Host pointers. */
tern_status tern_unpack_t5(const uint8_t *data, int64_t N, int64_t K, uint32_t *codes);

/* ---------------------------------------------------------------------------
 * Device operations.  Device pointers; enqueued on `stream`.
 * ------------------------------------------------------------------------ */

/* Device-side packer (same slot format as tern_pack, "Memory requirement"):
 * t[N][K] int8 on the device, each -1, 0 or +1, into codes[N][K/16].  Values
 * are not checked: anything outside {-1, 0, 1} gives unspecified slots (use
 * tern_pack on the host for validated packing).  Scales need no packing.
 * t 16-byte aligned, codes 4-byte aligned, K a multiple of 128.
 * Errors: TERN_EINVAL, TERN_EDEVICE. */
tern_status tern_pack_device(const int8_t *t, int64_t N, int64_t K, uint32_t *codes, void *stream);

/* Signed normalized Walsh-Hadamard transform along the last dimension, over
 * contiguous blocks of `block` elements ("Ternary-Bonsai-2-9B-2bit",
 * section 3), in natural Sylvester order H[i][l] = (-1)^popcount(i & l):
 *   inverse == 0:  y[m, jb+i] = b^-1/2 sum_l H[i][l] d[jb+l] x[m, jb+l]
 *   inverse != 0:  y[m, jb+i] = d[jb+i] b^-1/2 sum_l H[i][l] x[m, jb+l]
 * x: [M][K] TERN_F32 or TERN_BF16; signs: int8 [K] (16-byte aligned), or NULL for all +1.
 * Only the sign bit of each entry is read: d[k] = -1 where signs[k] < 0 and
 * d[k] = +1 otherwise (so +1 and -1 mean what they say, 0 counts as +1, and
 * the transform stays exactly orthonormal); y: float [M][K], which may be
 * the same buffer as x when xdt == TERN_F32.  block: a power of two in
 * [1, 4096]; K % block == 0.  x and y 16-byte aligned.
 * Accuracy: within 1e-5 relative L2 error per row of the exact transform.
 * Errors: TERN_EINVAL, TERN_EUNSUPPORTED (dtype), TERN_EDEVICE. */
tern_status tern_fwht(const void *x, int xdt, const int8_t *signs, int64_t M, int64_t K,
                      int64_t block, int inverse, float *y, void *stream);

/* Decode-regime matmul y[m][n] = sum_k s_g t[n][k] x[m][k] for M <= 16
 * ("CUDA (NVIDIA GPUs)": fused unpack + group scale).  The codes are streamed
 * once from HBM; products are formed exactly and accumulated in binary32
 * per 128-K group, then scaled.
 * x: [M][K], xdt TERN_F32 or TERN_BF16, 16-byte aligned; codes [N][K/16]
 * 16-byte aligned; scales [N][K/128] 2-byte aligned; y [M][N] written as
 * ydt (TERN_F32, or TERN_BF16 rounded to nearest even), aligned to its dtype.
 * Accuracy: |y - exact| <= 1e-4 * sum_k |s_g t x_k| per element (binary32
 * output; a bfloat16 output adds its own rounding).
 * K <= TERN_MAX_K.
 * Errors: TERN_EINVAL (M > 16, K > TERN_MAX_K, sizes, alignment, NULL),
 * TERN_EUNSUPPORTED (dtype), TERN_EDEVICE. */
tern_status tern_gemv(const void *x, int xdt, int64_t M, int64_t K,
                      const uint32_t *codes, const uint16_t *scales, int64_t N,
                      void *y, int ydt, void *stream);

/* tern_gemv over the base-3 layout: the same product and accuracy, with the
 * weights streamed at 1.6 bits/weight (plus scales) and their digits decoded
 * in the kernel.  x: [M][K] TERN_BF16 only, 16-byte aligned; data as above,
 * 16-byte aligned; scales [N][K/128]; y [M][N] as ydt.  Bytes out of range for
 * their superblock give unspecified results (tern_unpack_t5 checks them).
 * Errors: TERN_EINVAL (M > 16, sizes, alignment, NULL), TERN_EUNSUPPORTED
 * (TERN_F32 activations, dtype), TERN_EDEVICE. */
tern_status tern_gemv_t5(const void *x, int xdt, int64_t M, int64_t K, const uint8_t *data,
                         const uint16_t *scales, int64_t N, void *y, int ydt, void *stream);

/* Decode-regime matmul over the binary variant ("prism-ml/Ternary-Bonsai-
 * 27B-mlx-2bit" model card, "Benchmarks", the 1-bit row: one sign bit per
 * weight plus the binary16 scale of each 128 weights, 1.125 bits/weight):
 * y[m][n] = sum_g s[n][g] sum_{k in g} b[n][k] x[m][k], with b = +1 for a
 * set bit and -1 for a clear one, in the word layout of tern_pack_b1.  The
 * words are streamed as they are (no 2-bit expansion) and turned into
 * operands in the kernel; the same accuracy as tern_gemv.
 * x: [M][K] TERN_BF16, 16-byte aligned, M <= 4; bits [N][K/32] 16-byte
 * aligned; scales [N][K/128] 2-byte aligned; K a multiple of 1024; y [M][N]
 * written as ydt (TERN_F32, or TERN_BF16 rounded to nearest even).
 * Errors: TERN_EINVAL (sizes, alignment, NULL), TERN_EUNSUPPORTED (M > 4,
 * TERN_F32 activations, K not a multiple of 1024, an output dtype other
 * than TERN_F32 / TERN_BF16, or a shape whose LDS image of x and per-
 * workgroup sums exceed one workgroup's LDS: K beyond about 38000 at M = 4,
 * or, for rows of 8192 or more, N beyond about 250000), TERN_EDEVICE. */
tern_status tern_gemv_b1(const void *x, int xdt, int64_t M, int64_t K, const uint32_t *bits,
                         const uint16_t *scales, int64_t N, void *y, int ydt, void *stream);

/* Rotated decode in one launch: y = (H_b D x / sqrt(b)) (s_g t)^T, i.e. the
 * signed normalized Walsh-Hadamard transform of tern_fwht (forward, blocks
 * of b along K) followed by the tern_gemv matmul on the rotated binary32
 * activations.  The rotation is the run-time half of the one the
 * "Ternary-Bonsai-2-9B-2bit" article (section 3) folds into the stored
 * weights; every workgroup applies it to x in LDS while the code stream is
 * already in flight, so the rotated activations never go to memory.
 * x: [M][K] TERN_F32 or TERN_BF16, 16-byte aligned; signs: int8 [K]
 * (16-byte aligned) or NULL, read as in tern_fwht (d[k] = -1 where
 * signs[k] < 0, else +1); block: a power of two in [16, 4096] with
 * K % block == 0; M <= 16; codes, scales, y, ydt as tern_gemv.
 * Accuracy: within tern_gemv's bound for the exact rotation plus
 * sum_k |s_g t| |x'_k - exact x'_k| (the rotation is computed to binary32
 * accuracy: radix-16 butterflies in binary32, or for b = 4096 two bf16
 * matrix-core products with binary32 accumulation whose binary32 operand is
 * split exactly into three bfloat16 parts).
 * Errors: as tern_gemv; TERN_EUNSUPPORTED when the staged activations of
 * one workgroup (about 8.25 * M * K bytes) exceed LDS -- use tern_fwht then
 * tern_gemv instead. */
tern_status tern_rotate_gemv(const void *x, int xdt, const int8_t *signs, int64_t block, int64_t M,
                             int64_t K, const uint32_t *codes, const uint16_t *scales, int64_t N,
                             void *y, int ydt, void *stream);

/* Bytes of device workspace tern_gemm needs for these sizes (may be 0). */
size_t tern_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Prefill-regime matmul, same definition as tern_gemv, any M >= 0 (tuned for
 * M in the hundreds and up): unpacked codes feed bf16 matrix-core (MFMA)
 * tiles as exact -2t operands; each accumulator is kept in units of its
 * column's current group scale and rescaled in binary32 at every group
 * boundary (one multiply per group), then multiplied by the last scale.
 * x: [M][K] TERN_BF16 only, 16-byte aligned; codes 16-byte aligned;
 * K <= 4194176 (2^22 - 128); y: float [M][N]; workspace: device memory of
 * at least tern_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned (NULL
 * allowed when that is 0); it holds partial sums of output tiles that are
 * split along K, and its contents on entry do not matter.
 * Accuracy as tern_gemv.  Errors: TERN_EINVAL, TERN_EUNSUPPORTED,
 * TERN_EDEVICE. */
tern_status tern_gemm(const void *x, int xdt, int64_t M, int64_t K,
                      const uint32_t *codes, const uint16_t *scales, int64_t N,
                      float *y, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device scratch that tern_gemm_noalloc holds per device. */
#define TERN_GEMM_SCRATCH_BYTES ((size_t)32 << 20)

/* tern_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * kernels and result as tern_gemm (bit for bit), with the partial sums of
 * K-split tiles in a static device array of the library instead of a
 * workspace argument: TERN_GEMM_SCRATCH_BYTES per device, held from the first
 * call on that device until the process ends.  The call allocates nothing.
 * The array's contents on entry do not matter (every partial sum is written
 * before it is read).  All calls on one device share the array: calls that
 * may overlap on one device (different streams, or host threads without an
 * order between them) race and give wrong results; calls ordered on one
 * stream are safe.  Arguments as tern_gemm, without the workspace.
 * Errors: as tern_gemm; TERN_EUNSUPPORTED when tern_gemm_workspace_bytes(M,
 * N, K) exceeds TERN_GEMM_SCRATCH_BYTES (use tern_gemm with a workspace). */
tern_status tern_gemm_noalloc(const void *x, int xdt, int64_t M, int64_t K,
                              const uint32_t *codes, const uint16_t *scales, int64_t N,
                              float *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
