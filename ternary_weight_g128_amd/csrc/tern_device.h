// Device helpers shared by the libtern kernel sources: operand types, the
// exact -2t weight operand, scalar conversions, LDS limit and CU count.
// Included inside an anonymous namespace by each .hip file.
#pragma once

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


constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Raising a kernel's dynamic LDS limit above the 64 KiB default needs
// hipFuncSetAttribute once per (kernel, device).
template <class Kernel>
int ensure_lds(Kernel kernel, size_t bytes)
{
    if (bytes > kMaxLds) return (int)hipErrorInvalidValue;  // more than one workgroup's LDS
    if (bytes <= 65536) return 0;
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> granted;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const void *k = reinterpret_cast<const void *>(kernel);
    std::lock_guard<std::mutex> lock(mu);
    if (granted.count({k, dev})) return 0;
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return (int)e;
    granted.insert({k, dev});
    return 0;
}

// A workgroup wider than the kernel's __launch_bounds__ does not fit the
// registers and barrier the kernel was built for: refused on the host.
inline int check_block(unsigned threads, unsigned bound)
{
    return threads == 0 || threads > bound ? (int)hipErrorInvalidConfiguration : 0;
}

inline int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}
