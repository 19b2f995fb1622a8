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

// Memory update (segment-recurrence simulator: mem = last M rows of [mem; h]),
// as its own launch: one workgroup per ring_copy_block (txl_internal.hpp).
__global__ void __launch_bounds__(256) ring_write_kernel(const RingCopy rc) { ring_copy_block(rc, blockIdx.x); }

// LayerNorm of the NumPy layer on "Implementing Transformer-XL":
// gamma * (x - mean) / (std + 1e-6) + beta with the population std. One wave
// per row; statistics in fp32 from an fp32 input row, which is x, or x + x2
// when the producing GEMM split its reduction in two. With VEC (rows of x and
// y, gamma and beta aligned to four elements) each lane holds groups of four
// consecutive columns (4 lane + 256 e), one 16-byte load of x and one store of
// y per group; otherwise single columns lane + 64 e.
template <typename T, bool VEC>
__global__ void layer_norm_kernel(const float *x, const float *x2, long long x_ld, const T *g, const T *bt, T *y,
                                  long long y_bstride, long long y_ld, int rows, int W, int D) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *xr = x + (long long)row * x_ld;
    const float *x2r = x2 ? x2 + (long long)row * x_ld : nullptr;
    constexpr int G = VEC ? 4 : 1;           // consecutive columns per group
    constexpr int NG = 16 / G;               // groups per lane (D <= 1024)
    constexpr int STRIDE = 64 * G;           // columns between a lane's groups
    auto col = [&](int e) { return G * lane + STRIDE * e; };
    float v[NG][G];
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < NG; ++e) {
        const int c = col(e);
        if constexpr (VEC) {
            if (c < D) {
                // x_ld is a multiple of 4 and D <= x_ld: the whole group lies in the row
                f32x4 a = *reinterpret_cast<const f32x4 *>(xr + c);
                if (x2r) {
                    const f32x4 a2 = *reinterpret_cast<const f32x4 *>(x2r + c);
                    a += a2;
                }
#pragma unroll
                for (int i = 0; i < G; ++i) v[e][i] = c + i < D ? a[i] : 0.f;
            } else {
#pragma unroll
                for (int i = 0; i < G; ++i) v[e][i] = 0.f;
            }
        } else {
            v[e][0] = c < D ? xr[c] : 0.f;
            if (x2r && c < D) v[e][0] += x2r[c];
        }
#pragma unroll
        for (int i = 0; i < G; ++i) s += v[e][i];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float mean = s / (float)D;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < NG; ++e)
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float d = col(e) + i < D ? v[e][i] - mean : 0.f;
            q += d * d;
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off);
    const float inv = 1.f / (sqrtf(q / (float)D) + 1e-6f);
    const int b = row / W, t = row - b * W;
    T *yr = y + (long long)b * y_bstride + (long long)t * y_ld;
#pragma unroll
    for (int e = 0; e < NG; ++e) {
        const int c = col(e);
        if (c >= D) continue;
        if (VEC && c + 4 <= D) {
            float gg[4], bb[4], o[4];
            if constexpr (sizeof(T) == 2) {
                const bf16x4 g4 = *reinterpret_cast<const bf16x4 *>(g + c);
                const bf16x4 b4 = *reinterpret_cast<const bf16x4 *>(bt + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) { gg[i] = (float)g4[i]; bb[i] = (float)b4[i]; }
            } else {
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(g + c);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bt + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) { gg[i] = g4[i]; bb[i] = b4[i]; }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = gg[i] * (v[e][i] - mean) * inv + bb[i];
            if constexpr (sizeof(T) == 2)
                *reinterpret_cast<bf16x4 *>(yr + c) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
            else
                *reinterpret_cast<f32x4 *>(yr + c) = f32x4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
            for (int i = 0; i < G; ++i)
                if (c + i < D) yr[c + i] = from_f32<T>(to_f32(g[c + i]) * (v[e][i] - mean) * inv + to_f32(bt[c + i]));
        }
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

int plan_ring_copy(bool is_bf16, RingCopy &rc, void *ring, int M, int D, int pos0, const void *src,
                   long long src_bstride, long long src_ld, int src_row0, int n, int B) {
    if (n <= 0 || B <= 0) return 0;
    const long long es = is_bf16 ? 2 : 4;
    const long long row_bytes = D * es;
    const bool pitched = src_ld != D;
    const bool vec = !pitched && (row_bytes % 16 == 0) && (((uintptr_t)ring | (uintptr_t)src) % 16 == 0) &&
                     ((src_bstride * es) % 16 == 0);
    const long long per_block = 256LL * kRingCopyUnroll;
    const long long row_words = row_bytes / (vec ? 16 : 4);
    const long long words = (long long)n * row_words;            // per batch row
    if (words > 0x7fffffffLL - per_block || (long long)M * row_words > 0x7fffffffLL) return -1;
    if (pitched && (src_ld * es) % 4) return -1;
    const long long bx = pitched ? (n + kRingCopyRows - 1) / kRingCopyRows : (words + per_block - 1) / per_block;
    if (bx * B > 0x7fffffffLL) return -1;
    rc.ring = (char *)ring;
    rc.src = (const char *)src;
    rc.src_bstride_bytes = src_bstride * es;
    rc.M = M;
    rc.row_words = (int)row_words;
    rc.pos0 = pos0;
    rc.src_row0 = src_row0;
    rc.n = n;
    rc.blocks_x = (int)bx;
    rc.vec = vec;
    rc.src_pitch_words = pitched ? (int)(src_ld * es / 4) : (int)row_words;
    return (int)(bx * B);
}

hipError_t launch_ring_copy(const RingCopy &rc, int blocks, hipStream_t s) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(ring_write_kernel, dim3(blocks), dim3(256), 0, s, rc);
    return hipGetLastError();
}

hipError_t launch_layer_norm(bool is_bf16, const float *x, const float *x2, long long x_ld, const void *g,
                             const void *b, void *y, long long y_bstride, long long y_ld, int B, int W, int D,
                             hipStream_t s) {
    const int rows = B * W;
    dim3 grid((rows + 3) / 4), block(256);
    // groups of four: x rows 16-byte aligned, y rows, gamma and beta aligned to
    // four elements
    const uintptr_t es = is_bf16 ? 2 : 4;
    const bool vec = ((uintptr_t)x % 16) == 0 && (!x2 || ((uintptr_t)x2 % 16) == 0) && x_ld % 4 == 0 &&
                     ((uintptr_t)y % (4 * es)) == 0 && y_ld % 4 == 0 && y_bstride % 4 == 0 &&
                     ((uintptr_t)g % (4 * es)) == 0 && ((uintptr_t)b % (4 * es)) == 0;
    if (is_bf16) {
        if (vec)
            hipLaunchKernelGGL((layer_norm_kernel<bf16, true>), grid, block, 0, s, x, x2, x_ld, (const bf16 *)g,
                               (const bf16 *)b, (bf16 *)y, y_bstride, y_ld, rows, W, D);
        else
            hipLaunchKernelGGL((layer_norm_kernel<bf16, false>), grid, block, 0, s, x, x2, x_ld, (const bf16 *)g,
                               (const bf16 *)b, (bf16 *)y, y_bstride, y_ld, rows, W, D);
    } else {
        if (vec)
            hipLaunchKernelGGL((layer_norm_kernel<float, true>), grid, block, 0, s, x, x2, x_ld, (const float *)g,
                               (const float *)b, (float *)y, y_bstride, y_ld, rows, W, D);
        else
            hipLaunchKernelGGL((layer_norm_kernel<float, false>), grid, block, 0, s, x, x2, x_ld, (const float *)g,
                               (const float *)b, (float *)y, y_bstride, y_ld, rows, W, D);
    }
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
