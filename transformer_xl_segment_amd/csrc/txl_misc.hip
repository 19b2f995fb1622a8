// txl_misc.hip -- memory ring update, LayerNorm and the distance table.
//
// These are bandwidth kernels: every byte is read once and written once, with
// consecutive lanes on consecutive addresses (16-byte accesses where the
// operands allow) so each wave moves whole cache lines.
#include <math.h>

#include <type_traits>

#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

// Memory update (segment-recurrence simulator: mem = last M rows of [mem; h]).
// For one batch row the n source rows are contiguous, and so are their ring
// slots up to the wrap: the copy is two contiguous runs, slots pos0 .. M-1 and
// then 0 onwards. Grid (blocks, B): each workgroup moves kRingUnroll runs of
// 256 words (16 bytes, or 4 when a row or a base is not 16-byte aligned) of
// one batch row, all loads issued before the stores, with no division.
constexpr int kRingUnroll = 4;

template <bool VEC>
__global__ void __launch_bounds__(256) ring_write_kernel(char *ring, int M, int row_words, int pos0,
                                                         const char *src, long long src_bstride_bytes,
                                                         int src_row0, int n) {
    typedef typename std::conditional<VEC, u32x4, uint32_t>::type Word;
    constexpr int WB = (int)sizeof(Word);
    const int b = blockIdx.y;
    const int total = n * row_words;                             // words of this batch row
    const int split = min(n, M - pos0) * row_words;              // words before the wrap
    const Word *s0 = reinterpret_cast<const Word *>(src + (long long)b * src_bstride_bytes) + (long long)src_row0 * row_words;
    Word *d0 = reinterpret_cast<Word *>(ring) + (long long)b * M * row_words;
    const int base = blockIdx.x * 256 * kRingUnroll + threadIdx.x;
    Word v[kRingUnroll];
#pragma unroll
    for (int u = 0; u < kRingUnroll; ++u) {
        const int w = base + 256 * u;
        if (w < total) v[u] = s0[w];
    }
#pragma unroll
    for (int u = 0; u < kRingUnroll; ++u) {
        const int w = base + 256 * u;
        if (w < total) d0[w < split ? (long long)pos0 * row_words + w : w - split] = v[u];
    }
    (void)WB;
}

// LayerNorm of the NumPy layer on "Implementing Transformer-XL":
// gamma * (x - mean) / (std + 1e-6) + beta with the population std. One wave
// per row; statistics in fp32 from an fp32 input row.
template <typename T>
__global__ void layer_norm_kernel(const float *x, const T *g, const T *bt, T *y, long long y_bstride,
                                  int rows, int W, int D) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *xr = x + (long long)row * D;
    constexpr int MAXE = 16;                 // D <= 1024
    float v[MAXE];
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int c = lane + 64 * e;
        v[e] = c < D ? xr[c] : 0.f;
        s += v[e];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float mean = s / (float)D;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int c = lane + 64 * e;
        const float d = c < D ? v[e] - mean : 0.f;
        q += d * d;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off);
    const float inv = 1.f / (sqrtf(q / (float)D) + 1e-6f);
    const int b = row / W, t = row - b * W;
    T *yr = y + (long long)b * y_bstride + (long long)t * D;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int c = lane + 64 * e;
        if (c < D) yr[c] = from_f32<T>(to_f32(g[c]) * (v[e] - mean) * inv + to_f32(bt[c]));
    }
}

// Distance table: R[d][k] = sin(d w_k), R[d][D/2 + k] = cos(d w_k),
// w_k = 10000^(-2k/D), evaluated in double precision.
template <typename T>
__global__ void sinusoid_kernel(T *R, int R_len, int D) {
    const int half = D / 2;
    const long long n = (long long)R_len * half;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const int d = (int)(idx / half), k = (int)(idx - (long long)d * half);
        const double w = pow(10000.0, -2.0 * (double)k / (double)D);
        const double a = (double)d * w;
        R[(long long)d * D + k] = from_f32<T>((float)sin(a));
        R[(long long)d * D + half + k] = from_f32<T>((float)cos(a));
    }
}

}  // namespace

hipError_t launch_ring_write(bool is_bf16, void *ring, int M, int D, int pos0, const void *src,
                             long long src_bstride, int src_row0, int n, int B, hipStream_t s) {
    if (n <= 0 || B <= 0) return hipSuccess;
    const long long es = is_bf16 ? 2 : 4;
    const long long row_bytes = D * es;
    const bool vec = (row_bytes % 16 == 0) && (((uintptr_t)ring | (uintptr_t)src) % 16 == 0) &&
                     ((src_bstride * es) % 16 == 0);
    const long long per_block = 256LL * kRingUnroll;
    const long long row_words_ll = row_bytes / (vec ? 16 : 4);
    const long long words = (long long)n * row_words_ll;         // per batch row
    // 32-bit word indices within a batch row, one grid row per batch row
    if (words > 0x7fffffffLL - per_block || (long long)M * row_words_ll > 0x7fffffffLL || B > 65535)
        return hipErrorInvalidValue;
    const int row_words = (int)row_words_ll;
    dim3 grid((unsigned)((words + per_block - 1) / per_block), (unsigned)B), block(256);
    if (grid.x == 0) return hipSuccess;
    if (vec)
        hipLaunchKernelGGL(ring_write_kernel<true>, grid, block, 0, s, (char *)ring, M, row_words, pos0,
                           (const char *)src, src_bstride * es, src_row0, n);
    else
        hipLaunchKernelGGL(ring_write_kernel<false>, grid, block, 0, s, (char *)ring, M, row_words, pos0,
                           (const char *)src, src_bstride * es, src_row0, n);
    return hipGetLastError();
}

hipError_t launch_layer_norm(bool is_bf16, const float *x, const void *g, const void *b, void *y,
                             long long y_bstride, int B, int W, int D, hipStream_t s) {
    const int rows = B * W;
    dim3 grid((rows + 3) / 4), block(256);
    if (is_bf16)
        hipLaunchKernelGGL(layer_norm_kernel<bf16>, grid, block, 0, s, x, (const bf16 *)g, (const bf16 *)b,
                           (bf16 *)y, y_bstride, rows, W, D);
    else
        hipLaunchKernelGGL(layer_norm_kernel<float>, grid, block, 0, s, x, (const float *)g,
                           (const float *)b, (float *)y, y_bstride, rows, W, D);
    return hipGetLastError();
}

hipError_t launch_sinusoid(bool is_bf16, void *R, int R_len, int D, hipStream_t s) {
    const long long n = (long long)R_len * (D / 2);
    if (n <= 0) return hipSuccess;
    int blocks = (int)((n + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (is_bf16) hipLaunchKernelGGL(sinusoid_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16 *)R, R_len, D);
    else hipLaunchKernelGGL(sinusoid_kernel<float>, dim3(blocks), dim3(256), 0, s, (float *)R, R_len, D);
    return hipGetLastError();
}

}  // namespace txl
