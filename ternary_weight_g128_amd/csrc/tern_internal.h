// Internal declarations shared by the libtern translation units.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "tern.h"

namespace tern {

// Thread-local reason for the last failing call.
void set_error(const std::string &msg);
void clear_error();

// Kernel launchers (tern_kernels.hip).  Arguments are already validated.
// They return hipSuccess or the launch error code (as int, to keep HIP types
// out of this header).
int launch_gemv(const void *x, bool x_f32, int M, int64_t K, const uint32_t *codes,
                const uint16_t *scales, int64_t N, void *y, bool y_bf16, void *stream);
int launch_rotate_gemv(const void *x, bool x_f32, const int8_t *signs, int block, int M, int64_t K,
                       const uint32_t *codes, const uint16_t *scales, int64_t N, void *y, bool y_bf16,
                       void *stream);
size_t rotate_gemv_lds(int64_t M, int64_t N, int64_t K);
// GEMV of one to four rows of bfloat16 x with the work split evenly over
// the CUs (tern_gemv1.hip): whether it takes this shape, and the launch;
// `binary`: the weights are the 1-bit variant's sign words (K / 128 even).
bool gemv1_applies(int M, int64_t N, int64_t K);
int launch_gemv1(const void *x, int M, int64_t K, const uint32_t *codes, const uint16_t *scales, int64_t N,
                 void *y, bool y_bf16, bool binary, void *stream);
size_t max_lds_bytes();
int launch_fwht(const void *x, bool x_f32, const int8_t *signs, int64_t M, int64_t K,
                int block, bool inverse, float *y, void *stream);
int launch_gemm(const void *x, int64_t M, int64_t K, const uint32_t *codes,
                const uint16_t *scales, int64_t N, float *y, void *workspace,
                size_t workspace_bytes, void *stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
// tern_gemm with its K-split partial sums in the library's static device
// scratch (tern_gemm.hip); the caller has checked that they fit.
int launch_gemm_noalloc(const void *x, int64_t M, int64_t K, const uint32_t *codes,
                        const uint16_t *scales, int64_t N, float *y, void *stream);
int launch_pack_device(const int8_t *t, int64_t N, int64_t K, uint32_t *codes, void *stream);
int64_t gemm_max_k();
int launch_gemv_t5(const void *x, int M, int64_t K, const uint8_t *data, const uint16_t *scales, int64_t N,
                   void *y, bool y_bf16, void *stream);
int64_t t5_row_bytes(int64_t K);
// whether tern_rotate_gemv can run this shape in one pass over the weights
bool rotate_gemv_fits(int64_t M, int64_t N, int64_t K, int64_t block, bool x_f32);

const char *hip_error_string(int err);

}  // namespace tern
