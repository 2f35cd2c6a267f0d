// Measurement helper for the benchmark (not part of the matmul path): a
// kernel that only reads a buffer, to measure what streaming a given number
// of bytes costs in one launch on this GPU.  It gives the floor that any
// decode GEMV over the same bytes, launched the same way, sits above.
//
// Built as its own library (libtern_bench.so) with a C entry point; nothing
// in libtern calls it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Workgroup w reads the contiguous 16-byte units [w * per_wg, (w + 1) *
// per_wg) of the buffer (the last one fewer), DEPTH loads per thread in
// flight, and writes the XOR of everything it read to sink[w] so that the
// loads are kept.
template <int DEPTH>
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t *__restrict__ p, int64_t units, int64_t per_wg,
                                                   unsigned *__restrict__ sink)
{
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    int64_t end = begin + per_wg;
    if (end > units) end = units;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t u0 = begin + threadIdx.x; u0 < end; u0 += 256 * DEPTH) {
        u32x4_t v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t u = u0 + 256 * d;
            v[d] = u < end ? p[u] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
    }
    __shared__ unsigned red[256];
    red[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned r = 0;
        for (int i = 0; i < 256; ++i) r ^= red[i];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from device buffer p with `wgs` workgroups
// of 256 threads, `depth` (1, 2, 4 or 8) 16-byte loads per thread in flight;
// sink: device memory for wgs unsigned values.  Returns a hipError_t.
int tern_bench_read(const void *p, int64_t bytes, int wgs, int depth, unsigned *sink, void *stream)
{
    if (!p || !sink || bytes <= 0 || bytes % 16 || wgs <= 0) return (int)hipErrorInvalidValue;
    const int64_t units = bytes / 16;
    const int64_t per_wg = (units + wgs - 1) / wgs;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4_t *src = static_cast<const u32x4_t *>(p);
    switch (depth) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(wgs), dim3(256), 0, st, src, units, per_wg, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, dim3(wgs), dim3(256), 0, st, src, units, per_wg, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(wgs), dim3(256), 0, st, src, units, per_wg, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(wgs), dim3(256), 0, st, src, units, per_wg, sink); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
