// C ABI of libtern: argument validation on the host, then kernel launch on
// the caller's stream.  Nothing here allocates device memory.
#include <cstdint>
#include <string>

#include "tern_internal.h"

using tern::set_error;

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tern_status device_status(int err, const char *what)
{
    if (err == 0) return TERN_OK;
    set_error(std::string(what) + ": HIP error " + std::to_string(err) + " (" +
              tern::hip_error_string(err) + ")");
    return TERN_EDEVICE;
}

tern_status check_matmul_args(const char *fn, const void *x, int xdt, int64_t M, int64_t K,
                              const uint32_t *codes, const uint16_t *scales, int64_t N,
                              const void *y)
{
    if (M < 0 || N < 0 || K < 0) {
        set_error(std::string(fn) + ": negative size");
        return TERN_EINVAL;
    }
    if (K % TERN_GROUP != 0) {
        set_error(std::string(fn) + ": K must be a multiple of 128 (whole scale groups)");
        return TERN_EINVAL;
    }
    if (K > TERN_MAX_K) {
        // the kernels index K and the groups of a row in 32-bit integers
        set_error(std::string(fn) + ": K above TERN_MAX_K (" + std::to_string(TERN_MAX_K) + ")");
        return TERN_EINVAL;
    }
    if (xdt != TERN_F32 && xdt != TERN_BF16) {
        set_error(std::string(fn) + ": activation dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (!y || (K > 0 && (!x || !codes || !scales))) {
        set_error(std::string(fn) + ": NULL pointer");
        return TERN_EINVAL;
    }
    if (K > 0 && (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2))) {
        set_error(std::string(fn) + ": x and codes must be 16-byte aligned, scales 2-byte aligned");
        return TERN_EINVAL;
    }
    if ((int64_t)N * (K / 16) >= ((int64_t)1 << 40)) {
        set_error(std::string(fn) + ": matrix too large");
        return TERN_EINVAL;
    }
    return TERN_OK;
}

}  // namespace

extern "C" {

tern_status tern_gemv(const void *x, int xdt, int64_t M, int64_t K, const uint32_t *codes,
                      const uint16_t *scales, int64_t N, void *y, int ydt, void *stream)
{
    tern_status st = check_matmul_args("tern_gemv", x, xdt, M, K, codes, scales, N, y);
    if (st != TERN_OK) return st;
    if (M > TERN_GEMV_MAX_M) {
        set_error("tern_gemv: M must be at most 16 (use tern_gemm for larger M)");
        return TERN_EINVAL;
    }
    if (ydt != TERN_F32 && ydt != TERN_BF16) {
        set_error("tern_gemv: output dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (!aligned(y, ydt == TERN_F32 ? 4 : 2)) {
        set_error("tern_gemv: y not aligned to its dtype");
        return TERN_EINVAL;
    }
    if (N > ((int64_t)1 << 31) - 64) {
        set_error("tern_gemv: N too large");
        return TERN_EINVAL;
    }
    return device_status(tern::launch_gemv(x, xdt == TERN_F32, (int)M, K, codes, scales, N, y,
                                           ydt == TERN_BF16, stream),
                         "tern_gemv");
}

tern_status tern_rotate_gemv(const void *x, int xdt, const int8_t *signs, int64_t block, int64_t M,
                             int64_t K, const uint32_t *codes, const uint16_t *scales, int64_t N,
                             void *y, int ydt, void *stream)
{
    tern_status st = check_matmul_args("tern_rotate_gemv", x, xdt, M, K, codes, scales, N, y);
    if (st != TERN_OK) return st;
    if (M > TERN_GEMV_MAX_M) {
        set_error("tern_rotate_gemv: M must be at most 16");
        return TERN_EINVAL;
    }
    if (block < 16 || block > TERN_FWHT_MAX_BLOCK || (block & (block - 1)) != 0) {
        set_error("tern_rotate_gemv: block must be a power of two in [16, 4096]");
        return TERN_EINVAL;
    }
    if (K % block != 0) {
        set_error("tern_rotate_gemv: K must be a multiple of block");
        return TERN_EINVAL;
    }
    if (ydt != TERN_F32 && ydt != TERN_BF16) {
        set_error("tern_rotate_gemv: output dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (K == 0) {
        set_error("tern_rotate_gemv: K must be positive");
        return TERN_EINVAL;
    }
    if (signs && !aligned(signs, 16)) {
        set_error("tern_rotate_gemv: signs must be 16-byte aligned");
        return TERN_EINVAL;
    }
    if (!aligned(y, ydt == TERN_F32 ? 4 : 2)) {
        set_error("tern_rotate_gemv: y not aligned to its dtype");
        return TERN_EINVAL;
    }
    if (N > ((int64_t)1 << 31) - 64) {
        set_error("tern_rotate_gemv: N too large");
        return TERN_EINVAL;
    }
    if (!tern::rotate_gemv_fits(M, N, K, block, xdt == TERN_F32)) {
        set_error("tern_rotate_gemv: M * K too large for one workgroup's LDS; use tern_fwht then "
                  "tern_gemv");
        return TERN_EUNSUPPORTED;
    }
    return device_status(tern::launch_rotate_gemv(x, xdt == TERN_F32, signs, (int)block, (int)M, K,
                                                  codes, scales, N, y, ydt == TERN_BF16, stream),
                         "tern_rotate_gemv");
}

size_t tern_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % TERN_GROUP) return 0;
    return tern::gemm_workspace_bytes(M, N, K);
}

namespace {

// Checks shared by tern_gemm and tern_gemm_noalloc (all but the workspace).
tern_status check_gemm_args(const char *fn, const void *x, int xdt, int64_t M, int64_t K,
                            const uint32_t *codes, const uint16_t *scales, int64_t N, const float *y)
{
    tern_status st = check_matmul_args(fn, x, xdt, M, K, codes, scales, N, y);
    if (st != TERN_OK) return st;
    if (xdt != TERN_BF16) {
        set_error(std::string(fn) + ": activations must be TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (K > tern::gemm_max_k()) {
        set_error(std::string(fn) + ": K above " + std::to_string(tern::gemm_max_k()));
        return TERN_EINVAL;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (!aligned(y, 4)) {
        set_error(std::string(fn) + ": y must be 4-byte aligned");
        return TERN_EINVAL;
    }
    if (M > ((int64_t)1 << 31) - 256 || N > ((int64_t)1 << 31) - 256) {
        set_error(std::string(fn) + ": M or N too large");
        return TERN_EINVAL;
    }
    return TERN_OK;
}

}  // namespace

tern_status tern_gemm(const void *x, int xdt, int64_t M, int64_t K, const uint32_t *codes,
                      const uint16_t *scales, int64_t N, float *y, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    tern_status st = check_gemm_args("tern_gemm", x, xdt, M, K, codes, scales, N, y);
    if (st != TERN_OK || M == 0 || N == 0) return st;
    const size_t need = tern::gemm_workspace_bytes(M, N, K);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))) {
        set_error("tern_gemm: workspace missing, misaligned or smaller than "
                  "tern_gemm_workspace_bytes() = " + std::to_string(need));
        return TERN_EINVAL;
    }
    return device_status(
        tern::launch_gemm(x, M, K, codes, scales, N, y, workspace, workspace_bytes, stream),
        "tern_gemm");
}

tern_status tern_gemm_noalloc(const void *x, int xdt, int64_t M, int64_t K, const uint32_t *codes,
                              const uint16_t *scales, int64_t N, float *y, void *stream)
{
    tern_status st = check_gemm_args("tern_gemm_noalloc", x, xdt, M, K, codes, scales, N, y);
    if (st != TERN_OK || M == 0 || N == 0) return st;
    const size_t need = tern::gemm_workspace_bytes(M, N, K);
    if (need > TERN_GEMM_SCRATCH_BYTES) {
        set_error("tern_gemm_noalloc: these sizes need " + std::to_string(need) +
                  " bytes of scratch, above TERN_GEMM_SCRATCH_BYTES = " +
                  std::to_string((size_t)TERN_GEMM_SCRATCH_BYTES) + "; use tern_gemm with a workspace");
        return TERN_EUNSUPPORTED;
    }
    return device_status(tern::launch_gemm_noalloc(x, M, K, codes, scales, N, y, stream), "tern_gemm_noalloc");
}

tern_status tern_gemv_b1(const void *x, int xdt, int64_t M, int64_t K, const uint32_t *bits,
                         const uint16_t *scales, int64_t N, void *y, int ydt, void *stream)
{
    if (M < 0 || N < 0 || K < 0) {
        set_error("tern_gemv_b1: negative size");
        return TERN_EINVAL;
    }
    if (K % TERN_GROUP != 0) {
        set_error("tern_gemv_b1: K must be a multiple of 128 (whole scale groups)");
        return TERN_EINVAL;
    }
    if (M > 4) {
        set_error("tern_gemv_b1: M must be at most 4");
        return TERN_EUNSUPPORTED;
    }
    if (xdt != TERN_BF16) {
        set_error("tern_gemv_b1: activations must be TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (ydt != TERN_F32 && ydt != TERN_BF16) {
        set_error("tern_gemv_b1: output dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (K % 1024 != 0) {
        set_error("tern_gemv_b1: K must be a multiple of 1024 (four 256-K blocks per step)");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (K == 0) {
        set_error("tern_gemv_b1: K must be positive");
        return TERN_EUNSUPPORTED;
    }
    if (!x || !bits || !scales || !y) {
        set_error("tern_gemv_b1: NULL pointer");
        return TERN_EINVAL;
    }
    if (!aligned(x, 16) || !aligned(bits, 16) || !aligned(scales, 2) || !aligned(y, ydt == TERN_F32 ? 4 : 2)) {
        set_error("tern_gemv_b1: x and bits must be 16-byte aligned, scales 2-byte, y to its dtype");
        return TERN_EINVAL;
    }
    if (N > ((int64_t)1 << 31) - 64 || K > TERN_MAX_K) {
        set_error("tern_gemv_b1: matrix too large");
        return TERN_EINVAL;
    }
    if (!tern::gemv1_applies((int)M, N, K)) {
        set_error("tern_gemv_b1: shape not supported (activation image beyond LDS, or offsets beyond 32 bits)");
        return TERN_EUNSUPPORTED;
    }
    return device_status(tern::launch_gemv1(x, (int)M, K, bits, scales, N, y, ydt == TERN_BF16, true, stream),
                         "tern_gemv_b1");
}

tern_status tern_gemv_t5(const void *x, int xdt, int64_t M, int64_t K, const uint8_t *data,
                         const uint16_t *scales, int64_t N, void *y, int ydt, void *stream)
{
    if (M < 0 || N < 0 || K < 0) {
        set_error("tern_gemv_t5: negative size");
        return TERN_EINVAL;
    }
    if (K % TERN_GROUP != 0) {
        set_error("tern_gemv_t5: K must be a multiple of 128 (whole scale groups)");
        return TERN_EINVAL;
    }
    if (M > TERN_GEMV_MAX_M) {
        set_error("tern_gemv_t5: M must be at most 16");
        return TERN_EINVAL;
    }
    if (xdt != TERN_BF16) {
        set_error("tern_gemv_t5: activations must be TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (ydt != TERN_F32 && ydt != TERN_BF16) {
        set_error("tern_gemv_t5: output dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || N == 0) return TERN_OK;
    if (!y || (K > 0 && (!x || !data || !scales))) {
        set_error("tern_gemv_t5: NULL pointer");
        return TERN_EINVAL;
    }
    if (!aligned(y, ydt == TERN_F32 ? 4 : 2) ||
        (K > 0 && (!aligned(x, 16) || !aligned(data, 16) || !aligned(scales, 2)))) {
        set_error("tern_gemv_t5: x and data must be 16-byte aligned, scales 2-byte, y to its dtype");
        return TERN_EINVAL;
    }
    if (N > ((int64_t)1 << 31) - 64 || K > ((int64_t)1 << 24) ||
        N * tern::t5_row_bytes(K) >= ((int64_t)1 << 40)) {
        set_error("tern_gemv_t5: matrix too large");
        return TERN_EINVAL;
    }
    return device_status(tern::launch_gemv_t5(x, (int)M, K, data, scales, N, y, ydt == TERN_BF16, stream),
                         "tern_gemv_t5");
}

tern_status tern_pack_device(const int8_t *t, int64_t N, int64_t K, uint32_t *codes, void *stream)
{
    if (N < 0 || K < 0) {
        set_error("tern_pack_device: negative size");
        return TERN_EINVAL;
    }
    if (K % TERN_GROUP != 0) {
        set_error("tern_pack_device: K must be a multiple of 128");
        return TERN_EINVAL;
    }
    if (N == 0 || K == 0) return TERN_OK;
    if (!t || !codes) {
        set_error("tern_pack_device: NULL pointer");
        return TERN_EINVAL;
    }
    if (!aligned(t, 16) || !aligned(codes, 4)) {
        set_error("tern_pack_device: t must be 16-byte aligned, codes 4-byte aligned");
        return TERN_EINVAL;
    }
    if (N * (K / 16) >= ((int64_t)1 << 40)) {
        set_error("tern_pack_device: matrix too large");
        return TERN_EINVAL;
    }
    return device_status(tern::launch_pack_device(t, N, K, codes, stream), "tern_pack_device");
}

tern_status tern_fwht(const void *x, int xdt, const int8_t *signs, int64_t M, int64_t K,
                      int64_t block, int inverse, float *y, void *stream)
{
    if (M < 0 || K < 0) {
        set_error("tern_fwht: negative size");
        return TERN_EINVAL;
    }
    if (block < 1 || block > TERN_FWHT_MAX_BLOCK || (block & (block - 1)) != 0) {
        set_error("tern_fwht: block must be a power of two in [1, 4096]");
        return TERN_EINVAL;
    }
    if (K % block != 0) {
        set_error("tern_fwht: K must be a multiple of block");
        return TERN_EINVAL;
    }
    if (xdt != TERN_F32 && xdt != TERN_BF16) {
        set_error("tern_fwht: activation dtype must be TERN_F32 or TERN_BF16");
        return TERN_EUNSUPPORTED;
    }
    if (M == 0 || K == 0) return TERN_OK;
    if (!x || !y) {
        set_error("tern_fwht: NULL pointer");
        return TERN_EINVAL;
    }
    if (!aligned(x, 16) || !aligned(y, 16) || (signs && !aligned(signs, 16))) {
        set_error("tern_fwht: x, y and signs must be 16-byte aligned");
        return TERN_EINVAL;
    }
    if (xdt == TERN_BF16 && static_cast<const void *>(y) == x) {
        set_error("tern_fwht: in-place operation needs TERN_F32 activations");
        return TERN_EINVAL;
    }
    if (K / block > ((int64_t)1 << 31) - 1) {
        set_error("tern_fwht: too many blocks for one launch");
        return TERN_EINVAL;
    }
    return device_status(tern::launch_fwht(x, xdt == TERN_F32, signs, M, K, (int)block,
                                           inverse != 0, y, stream),
                         "tern_fwht");
}

}  // extern "C"
