/*
 * tern_oracle.c -- plain, slow, FP64 reference for the ternary-g128 matmul
 * and the signed normalized Walsh-Hadamard rotation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or constant with the HIP library and includes nothing
 * from it.  Every function is the definition written out, in the order the
 * sources state it, with no blocking, fusion or reordering.
 *
 * Sources (web pages; cited by title and section):
 *  [MC]  "prism-ml/Ternary-Bonsai-27B-mlx-2bit" model card,
 *        sections "Weight representation: ternary g128", "Memory requirement",
 *        "CUDA (NVIDIA GPUs)".
 *  [9B]  "Ternary-Bonsai-2-9B-2bit" article, section 3
 *        "Ternary weights and Hadamard rotation".
 *
 * Readings where the sources are silent (each is listed in the design notes):
 *  - slot code q = t + 1 in {0,1,2}; 16 slots per little-endian uint32,
 *    K-major, slot j of word w holds k = 16 w + j at bits 2j..2j+1;
 *  - scales are IEEE binary16, one per 128 consecutive K of one output row;
 *  - the Hadamard matrix is in natural (Sylvester) order,
 *    H[i][l] = (-1)^popcount(i & l), normalized by 1/sqrt(b), applied to
 *    contiguous blocks of b along the last dimension, signs first.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (closed forms, invariants, library routines, brute force); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 128   /* [MC] Weight representation: 128 weights per FP16 scale */
#define ORACLE_SLOTS 16    /* 2-bit slots per 32-bit word ([MC] Memory requirement) */

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)            /* zero or subnormal: f * 2^-24 */
        v = ldexp((double)f, -24);
    else if (e == 31)      /* infinity or NaN */
        v = (f == 0) ? INFINITY : NAN;
    else                   /* normal: (1 + f/1024) * 2^(e-15) */
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* bfloat16 -> double: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    union { uint32_t u; float f; } cvt;
    cvt.u = (uint32_t)b << 16;
    return (double)cvt.f;
}

/* Activation element (m, k) as a double; xdt 0 = binary32, 1 = bfloat16,
 * 2 = binary64. */
static double x_at(const void *x, int xdt, int64_t K, int64_t m, int64_t k)
{
    int64_t i = m * K + k;
    if (xdt == 0) return (double)((const float *)x)[i];
    if (xdt == 1) return oracle_bf16_to_double(((const uint16_t *)x)[i]);
    return ((const double *)x)[i];
}

/* Ternary value of weight (n, k) from its 2-bit slot: t = q - 1.
 * Returns 2 for the unused slot value q = 3 (not a ternary code). */
static int slot_t(const uint32_t *codes, int64_t K, int64_t n, int64_t k, int *t)
{
    int64_t words_per_row = K / ORACLE_SLOTS;
    uint32_t w = codes[n * words_per_row + k / ORACLE_SLOTS];
    int q = (int)((w >> (2 * (k % ORACLE_SLOTS))) & 3u);
    if (q == 3) return 2;
    *t = q - 1;
    return 0;
}

/* Decode every slot into t in {-1,0,+1}.  Returns 0, or 3 if a slot holds 3. */
int oracle_decode(const uint32_t *codes, int64_t N, int64_t K, int8_t *t)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v;
            if (slot_t(codes, K, n, k, &v)) return 3;
            t[n * K + k] = (int8_t)v;
        }
    return 0;
}

/* Encode t in {-1,0,+1} into 2-bit slots q = t + 1.  Returns 0, or 2 if some
 * t is not ternary.  codes must hold N*K/16 words. */
int oracle_encode(const int8_t *t, int64_t N, int64_t K, uint32_t *codes)
{
    int64_t words = N * (K / ORACLE_SLOTS);
    for (int64_t i = 0; i < words; ++i) codes[i] = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v = t[n * K + k];
            if (v < -1 || v > 1) return 2;
            uint32_t q = (uint32_t)(v + 1);
            codes[n * (K / ORACLE_SLOTS) + k / ORACLE_SLOTS] |= q << (2 * (k % ORACLE_SLOTS));
        }
    return 0;
}

/* Dequantized weight w = s_g * t, with s_g the scale of the group of 128
 * consecutive K that k falls in ([MC] Weight representation).  Exact in
 * double: a binary16 times -1, 0 or +1. */
static double weight(const uint32_t *codes, const uint16_t *scales, int64_t K,
                     int64_t n, int64_t k, int *bad)
{
    int t;
    if (slot_t(codes, K, n, k, &t)) { *bad = 1; return 0.0; }
    double s = oracle_half_to_double(scales[n * (K / ORACLE_GROUP) + k / ORACLE_GROUP]);
    return s * (double)t;
}

/* One output: y = sum_k w[n][k] * x[m][k] and the error scale
 * B = sum_k |w[n][k] * x[m][k]|, summed in k order in double. */
static int one_output(const void *x, int xdt, int64_t K, const uint32_t *codes,
                      const uint16_t *scales, int64_t m, int64_t n,
                      double *y, double *bound)
{
    double acc = 0.0, b = 0.0;
    int bad = 0;
    for (int64_t k = 0; k < K; ++k) {
        double p = weight(codes, scales, K, n, k, &bad) * x_at(x, xdt, K, m, k);
        acc += p;
        b += fabs(p);
    }
    *y = acc;
    *bound = b;
    return bad ? 3 : 0;
}

/* y[m][n] = sum_k (s_g t)[n][k] x[m][k] for all m < M, n < N, i.e. x times
 * the transposed dequantized weight matrix ([MC] CUDA: the matmul consumes
 * packed codes plus group scales).  Naive loops over m, n, then k. */
int oracle_matmul(const void *x, int xdt, int64_t M, int64_t K,
                  const uint32_t *codes, const uint16_t *scales, int64_t N,
                  double *y, double *bound)
{
    int rc = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            rc |= one_output(x, xdt, K, codes, scales, m, n,
                             &y[m * N + n], &bound[m * N + n]);
    return rc;
}

/* oracle_matmul with its (m, n) outputs shared out over `threads` host
 * threads (OpenMP, static partition).  Each output is still one_output: the
 * same k loop in the same order, so the result is bit-identical to
 * oracle_matmul for any thread count; only which thread computes an output
 * changes. */
int oracle_matmul_threaded(const void *x, int xdt, int64_t M, int64_t K,
                           const uint32_t *codes, const uint16_t *scales, int64_t N,
                           double *y, double *bound, int threads)
{
    int rc = 0;
    const int64_t total = M * N;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) reduction(| : rc)
    for (int64_t i = 0; i < total; ++i) {
        const int64_t m = i / N, n = i % N;
        rc |= one_output(x, xdt, K, codes, scales, m, n, &y[m * N + n], &bound[m * N + n]);
    }
    return rc;
}

/* The number of host threads an OpenMP region may use here. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The same definition at a list of (m, n) output positions only. */
int oracle_matmul_at(const void *x, int xdt, int64_t K,
                     const uint32_t *codes, const uint16_t *scales,
                     const int64_t *ms, const int64_t *ns, int64_t count,
                     double *y, double *bound)
{
    int rc = 0;
    for (int64_t i = 0; i < count; ++i)
        rc |= one_output(x, xdt, K, codes, scales, ms[i], ns[i], &y[i], &bound[i]);
    return rc;
}

/* popcount of a 64-bit value, bit by bit. */
static int popcount64(uint64_t v)
{
    int c = 0;
    while (v) { c += (int)(v & 1u); v >>= 1; }
    return c;
}

/* Entry (i, l) of the b x b Sylvester Hadamard matrix: (-1)^popcount(i & l). */
double oracle_hadamard_entry(int64_t i, int64_t l)
{
    return (popcount64((uint64_t)(i & l)) & 1) ? -1.0 : 1.0;
}

/* Signed normalized Walsh-Hadamard transform along the last dimension, in
 * contiguous blocks of b ([9B] section 3: normalized Sylvester-Walsh-Hadamard,
 * block 4096, last dimension, explicit sign pattern).
 *   forward:  y = (1/sqrt(b)) H_b (d .* x)     (per block)
 *   inverse:  y = d .* ((1/sqrt(b)) H_b x)     (per block)
 * d is the +-1 sign vector of length K (NULL means all +1).  The matrix is
 * applied entry by entry, O(b^2) per block.  Returns 1 if K % b != 0. */
int oracle_fwht(const double *x, const int8_t *signs, int64_t M, int64_t K,
                int64_t b, int inverse, double *y)
{
    if (b <= 0 || K % b != 0) return 1;
    double norm = 1.0 / sqrt((double)b);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; j += b)
            for (int64_t i = 0; i < b; ++i) {
                double acc = 0.0;
                for (int64_t l = 0; l < b; ++l) {
                    double v = x[m * K + j + l];
                    if (!inverse && signs) v *= (double)signs[j + l];
                    acc += oracle_hadamard_entry(i, l) * v;
                }
                acc *= norm;
                if (inverse && signs) acc *= (double)signs[j + i];
                y[m * K + j + i] = acc;
            }
    return 0;
}

/* Lossless reading of an FP32 matrix as ternary-g128 ([9B] section 3: the
 * transcode to 2-bit groups of 128 is lossless).  A group is ternary iff all
 * its nonzero |w| equal one value a that binary16 represents exactly; then
 * s = a (s = +0 for an all-zero group) and t = sign(w).  Returns 0, or 2 at
 * the first group that is not of that form.  scale_bits receives the
 * binary16 bit pattern of s. */
int oracle_ternary_from_f32(const float *w, int64_t N, int64_t K,
                            int8_t *t, uint16_t *scale_bits)
{
    int64_t G = K / ORACLE_GROUP;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            double a = 0.0;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k) {
                double v = fabs((double)w[n * K + k]);
                if (v == 0.0) continue;
                if (!isfinite(v)) return 2;
                if (a == 0.0) a = v;
                else if (v != a) return 2;
            }
            /* find the binary16 pattern whose value is exactly a */
            uint16_t bits = 0;
            int found = (a == 0.0);
            for (uint32_t h = 0; h < 0x7c00u && !found; ++h)
                if (oracle_half_to_double((uint16_t)h) == a) { bits = (uint16_t)h; found = 1; }
            if (!found) return 2;
            scale_bits[n * G + g] = bits;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k) {
                float v = w[n * K + k];
                t[n * K + k] = (int8_t)((v > 0.0f) - (v < 0.0f));
            }
        }
    return 0;
}

/* Storage accounting of the 2-bit-slot format ([MC] Memory requirement):
 * N*K/4 bytes of codes plus 2 bytes of FP16 scale per 128 weights. */
double oracle_bits_per_weight(int64_t N, int64_t K)
{
    double code_bytes = (double)N * (double)K / 4.0;
    double scale_bytes = 2.0 * (double)N * (double)K / ORACLE_GROUP;
    return 8.0 * (code_bytes + scale_bytes) / ((double)N * (double)K);
}

/* ------------------------------------------------------------------------
 * Format variants ([MC] "Shipped components", "MLX packaging", and the
 * 1-bit row of the variant table under "Benchmarks").  Each is written as
 * its dequantized value, so that a transcode can be checked by comparing
 * dense weights.
 * --------------------------------------------------------------------- */

/* Group-size-64 variant ([MC] Shipped components): the same 2-bit slot codes;
 * the FP16 scale of weight k of row n is s64[n][k/64].  Dense w[N][K] in
 * double.  Returns 0, or 3 if a slot holds 3. */
int oracle_dequant_g64(const uint32_t *codes, const uint16_t *s64, int64_t N, int64_t K, double *w)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int t;
            if (slot_t(codes, K, n, k, &t)) return 3;
            w[n * K + k] = oracle_half_to_double(s64[n * (K / 64) + k / 64]) * (double)t;
        }
    return 0;
}

/* Affine group format with a scale and a bias per group ([MC] MLX packaging):
 * unsigned fields of `bits` bits (1 or 2), 32/bits of them per little-endian
 * uint32 word, lowest field first, K-major per row; one FP16 (scale, bias)
 * pair per `group` consecutive K; the weight is scale * q + bias, evaluated in
 * double.  Returns 0, or 1 for unsupported bits/group. */
int oracle_dequant_affine(const uint32_t *words, int bits, int group, const uint16_t *scales,
                          const uint16_t *biases, int64_t N, int64_t K, double *w)
{
    if ((bits != 1 && bits != 2) || group <= 0 || K % group != 0 || (K * bits) % 32 != 0) return 1;
    const int64_t per_word = 32 / bits, wpr = K / per_word, gpr = K / group;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint32_t word = words[n * wpr + k / per_word];
            double q = (double)((word >> (bits * (k % per_word))) & mask);
            double scale = oracle_half_to_double(scales[n * gpr + k / group]);
            double bias = oracle_half_to_double(biases[n * gpr + k / group]);
            w[n * K + k] = scale * q + bias;
        }
    return 0;
}

/* Binary g128 variant ([MC] Benchmarks: the 1-bit model, 1.125 bits/weight =
 * one bit plus an FP16 scale per 128): bit j of word w of row n holds weight
 * k = 32 w + j, 1 for +1 and 0 for -1 (little-endian uint32, lowest bit
 * first).  Decode into b in {-1, +1}. */
void oracle_b1_decode(const uint32_t *bits, int64_t N, int64_t K, int8_t *b)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint32_t bit = (bits[n * (K / 32) + k / 32] >> (k % 32)) & 1u;
            b[n * K + k] = bit ? (int8_t)1 : (int8_t)-1;
        }
}

/* Encode b in {-1, +1} as above.  Returns 0, or 2 if some b is not +-1. */
int oracle_b1_encode(const int8_t *b, int64_t N, int64_t K, uint32_t *bits)
{
    for (int64_t i = 0; i < N * (K / 32); ++i) bits[i] = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v = b[n * K + k];
            if (v != 1 && v != -1) return 2;
            if (v == 1) bits[n * (K / 32) + k / 32] |= 1u << (k % 32);
        }
    return 0;
}

/* Storage of each format in bits per weight, from its byte counts:
 *   0  ternary g128, 2-bit slots + FP16 scale per 128   ([MC] Memory requirement)
 *   1  ternary, 2-bit slots + FP16 scale per 64          ([MC] Shipped components)
 *   2  2-bit fields + FP16 scale and FP16 bias per 128   ([MC] MLX packaging)
 *   3  binary g128, 1 bit + FP16 scale per 128           ([MC] Benchmarks, 1-bit row)
 *   4  1-bit fields + FP16 scale and FP16 bias per 128   (affine container of format 3)
 * Returns -1 for an unknown format. */
double oracle_format_bits_per_weight(int format, int64_t N, int64_t K)
{
    double nk = (double)N * (double)K, field_bytes, side_bytes;
    switch (format) {
    case 0: field_bytes = nk / 4.0; side_bytes = 2.0 * nk / 128.0; break;
    case 1: field_bytes = nk / 4.0; side_bytes = 2.0 * nk / 64.0; break;
    case 2: field_bytes = nk / 4.0; side_bytes = 4.0 * nk / 128.0; break;
    case 3: field_bytes = nk / 8.0; side_bytes = 2.0 * nk / 128.0; break;
    case 4: field_bytes = nk / 8.0; side_bytes = 4.0 * nk / 128.0; break;
    default: return -1.0;
    }
    return 8.0 * (field_bytes + side_bytes) / nk;
}

/* ------------------------------------------------------------------------
 * Base-3 layout below two bits per weight.  The card ("Memory requirement")
 * notes that 2-bit slots cost 2.125 bits/weight against about 1.71 for the
 * information content, and that native ternary kernels would close the gap;
 * it does not give a layout.  This one packs five ternary values into a byte
 * (3^5 = 243 <= 256), 1.6 bits per weight:
 *   - the groups of 128 of a row are taken five at a time ("superblocks");
 *     superblock b holds groups 5b .. 5b + p - 1, p = min(5, G - 5b);
 *   - superblock b is 128 bytes; byte i holds sum_{j<p} q_j 3^j with q_j = t + 1
 *     of weight k = 128 (5b + j) + i, i.e. digit j of byte i is weight i of
 *     the superblock's group j;
 *   - a row is ceil(G/5) * 128 bytes; scales stay one FP16 per group.
 * --------------------------------------------------------------------- */

static int64_t t5_row_bytes(int64_t K)
{
    int64_t G = K / ORACLE_GROUP;
    return ((G + 4) / 5) * 128;
}

/* Decode into t.  Returns 0, or 3 if a byte is not below 3^p. */
int oracle_t5_decode(const uint8_t *d, int64_t N, int64_t K, int8_t *t)
{
    const int64_t G = K / ORACLE_GROUP, rb = t5_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t g = k / ORACLE_GROUP, b = g / 5, j = g % 5;
            int64_t p = (G - 5 * b) < 5 ? (G - 5 * b) : 5;
            int v = d[n * rb + 128 * b + k % ORACLE_GROUP];
            int lim = 1;
            for (int e = 0; e < p; ++e) lim *= 3;
            if (v >= lim) return 3;
            for (int e = 0; e < j; ++e) v /= 3;
            t[n * K + k] = (int8_t)(v % 3 - 1);
        }
    return 0;
}

/* Encode t in {-1,0,+1}.  Returns 0, or 2 if some t is not ternary.  d must
 * hold N * ceil(K/640) * 128 bytes. */
int oracle_t5_encode(const int8_t *t, int64_t N, int64_t K, uint8_t *d)
{
    const int64_t rb = t5_row_bytes(K);
    for (int64_t i = 0; i < N * rb; ++i) d[i] = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v = t[n * K + k];
            if (v < -1 || v > 1) return 2;
            int64_t g = k / ORACLE_GROUP, b = g / 5, j = g % 5;
            int w = 1;
            for (int e = 0; e < j; ++e) w *= 3;
            d[n * rb + 128 * b + k % ORACLE_GROUP] += (uint8_t)((v + 1) * w);
        }
    return 0;
}

/* Bits per weight of the base-3 layout with its FP16 group scales. */
double oracle_t5_bits_per_weight(int64_t N, int64_t K)
{
    double bytes = (double)N * (double)t5_row_bytes(K) + 2.0 * (double)N * (double)(K / ORACLE_GROUP);
    return 8.0 * bytes / ((double)N * (double)K);
}
