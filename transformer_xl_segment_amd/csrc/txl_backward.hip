// txl_backward.hip -- layout, softmax-gradient and reduction kernels of the
// relative-attention backward pass.
//
// Training stops the gradient at the memory ("Transformer-XL, explained.",
// method step 2 and the SG(.) legend entry): the cached rows are a fixed
// input, so the backward of one segment needs only the gradients of its
// projected operands. With c = 1/sqrt(dh), score s_ij = c((q_i+u).k_j +
// (q_i+v).r_{m+i-j}), p = softmax, o_i = sum_j p_ij val_j and the incoming dO:
//   D_i = sum_j p_ij dP_ij with dP_ij = dO_i.val_j,   dS_ij = c p_ij (dP_ij - D_i)
//   dq_i = sum_j dS_ij (k_j + r_{m+i-j}),   dk_j = sum_i dS_ij (q_i + u)
//   dval_j = sum_i p_ij dO_i,   dr_d = sum_{m+i-j=d} dS_ij (q_i + v)
//   du = sum_ij dS_ij k_j,   dv = sum_ij dS_ij r_{m+i-j}.
// The products run as batched GEMMs on the matrix cores (txl_gemm.hip) over
// per-(batch, head) matrices kept in HBM: the score terms (q+u)K^T, (q+v)R^T
// and dO V^T; then dS K, dS_d R (dS re-indexed by distance), dS^T (q+u),
// P^T dO and, summed over the batch in the reduction axis, dS_d^T (q+v). The
// kernels here build the head-major operands and their transposes, turn the
// score terms into P and dS row by row, and unpack and reduce the results.
#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

// dst[(b*H + h)][t][c] = src[b][t][h*dh + c] (+ bias[h*dh + c]) for t < nrows, c < dh; zero elsewhere.
template <typename T>
__global__ void heads_kernel(const T *src, long long src_bs, int B, int nrows, int nrows_p, int D, int H, int dh,
                             int dp, const T *bias, T *dst) {
    const long long n = (long long)B * H * nrows_p * dp;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const int c = (int)(idx % dp);
        const long long rt = idx / dp;
        const int t = (int)(rt % nrows_p);
        const int g = (int)(rt / nrows_p);
        const int b = g / H, h = g - b * H;
        float x = 0.f;
        if (t < nrows && c < dh) {
            x = to_f32(src[(long long)b * src_bs + (long long)t * D + h * dh + c]);
            if (bias) x += to_f32(bias[h * dh + c]);
        }
        dst[idx] = from_f32<T>(x);
    }
}

// 64 x 64 tiles through LDS: element (g, row, col) of src [G][nrow][src_ld] goes to
// dst + h*dst_hs + col*dst_cs + b*dst_bs + row with g = b*H + h.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T *src, int H, int nrow, int ncol, long long src_ld,
                                                        T *dst, long long dst_hs, long long dst_cs,
                                                        long long dst_bs) {
    __shared__ T tile[64][65];
    const int g = blockIdx.z, b = g / H, h = g - b * H;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const T *s = src + ((long long)g * nrow) * src_ld;
    for (int rr = ty; rr < 64; rr += 4) {
        const int r = r0 + rr, c = c0 + tx;
        tile[rr][tx] = (r < nrow && c < ncol) ? s[(long long)r * src_ld + c] : from_f32<T>(0.f);
    }
    __syncthreads();
    T *d = dst + (long long)h * dst_hs + (long long)b * dst_bs;
    for (int cc = ty; cc < 64; cc += 4) {
        const int c = c0 + cc, r = r0 + tx;
        if (c < ncol && r < nrow) d[(long long)c * dst_cs + r] = tile[tx][cc];
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One wave per query row (g, i), i < Wp; rows i >= W and columns past the
// visible keys are written as zeros (they are GEMM operands).
template <typename T>
__global__ void __launch_bounds__(256) bwd_scores_kernel(const float *ac, const float *bd, const float *dpm, T *p,
                                                         T *ds, T *dsd, int G, int W, int Wp, int m, int K, int Kp,
                                                         float c) {
    extern __shared__ float rowbuf[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * 4 + w;          // g * Wp + i
    if (row >= (long long)G * Wp) return;                          // wave-uniform
    float *buf = rowbuf + w * Kp;
    const int i = (int)(row % Wp);
    const long long off = row * Kp;
    const int last = i < W ? min(m + i, K - 1) : -1;               // visible keys 0 .. last
    float mx = -INFINITY;
    for (int j = lane; j < Kp; j += 64) {
        const float sc = j <= last ? c * (ac[off + j] + bd[off + (m + i - j)]) : -INFINITY;
        buf[j] = sc;
        mx = fmaxf(mx, sc);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < Kp; j += 64) {
        const float e = j <= last ? __expf(buf[j] - mx) : 0.f;
        buf[j] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    const float inv = last >= 0 ? 1.f / sum : 0.f;
    float dsum = 0.f;
    for (int j = lane; j < Kp; j += 64) {
        const float pj = buf[j] * inv;
        buf[j] = pj;
        p[off + j] = from_f32<T>(pj);
        if (j <= last) dsum += pj * dpm[off + j];
    }
    const float Di = wave_sum(dsum);
    for (int j = lane; j < Kp; j += 64) {
        const float dsj = j <= last ? c * buf[j] * (dpm[off + j] - Di) : 0.f;
        buf[j] = dsj;
        ds[off + j] = from_f32<T>(dsj);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // re-indexed by distance: dsd[i][d] = ds[i][m + i - d]
    for (int d = lane; d < Kp; d += 64) {
        const int j = m + i - d;
        dsd[off + d] = from_f32<T>(j >= 0 && j <= last ? buf[j] : 0.f);
    }
}

// dq = dq1 + dq2 and the unpacking of dk, dval, dr into row layouts.
__global__ void bwd_unpack_kernel(BwdDims d, const float *dq1, const float *dq2, const float *dkh,
                                  const float *dvh, const float *drh, float *dq, float *dk, float *dval,
                                  float *dr) {
    const long long nq = (long long)d.B * d.W * d.D, nk = (long long)d.B * d.K * d.D, nr = (long long)d.K * d.D;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < nq + 2 * nk + nr;
         idx += (long long)gridDim.x * blockDim.x) {
        if (idx < nq) {
            const int col = (int)(idx % d.D);
            const long long bt = idx / d.D;
            const int t = (int)(bt % d.W), b = (int)(bt / d.W);
            const int h = col / d.dh, c = col - h * d.dh;
            const long long src = (((long long)b * d.H + h) * d.Wp + t) * d.dp + c;
            dq[idx] = dq1[src] + dq2[src];
        } else if (idx < nq + 2 * nk) {
            const bool isv = idx >= nq + nk;
            const long long e = idx - nq - (isv ? nk : 0);
            const int col = (int)(e % d.D);
            const long long bj = e / d.D;
            const int j = (int)(bj % d.K), b = (int)(bj / d.K);
            const int h = col / d.dh, c = col - h * d.dh;
            const long long src = (((long long)b * d.H + h) * d.Kp + j) * d.dp + c;
            if (isv) dval[e] = dvh[src];
            else dk[e] = dkh[src];
        } else {
            const long long e = idx - nq - 2 * nk;
            const int col = (int)(e % d.D), j = (int)(e / d.D);
            const int h = col / d.dh, c = col - h * d.dh;
            dr[e] = drh[((long long)h * d.Kp + j) * d.dp + c];
        }
    }
}

// du, dv: per head, column sums of dq1 (resp. dq2) over every (b, t < W) row,
// in two stages: workgroup (h, which, chunk) sums one chunk of kBiasChunk rows
// into part[which][h][chunk][c]; then one thread per (which, h, c) adds the chunks.
constexpr int kBiasChunk = 64;

__global__ void __launch_bounds__(256) bwd_bias_partial_kernel(BwdDims d, const float *dq1, const float *dq2,
                                                               float *part, int nchunk) {
    __shared__ float red[4][64];
    const int chunk = blockIdx.x % nchunk;
    const int hw = blockIdx.x / nchunk;                  // h * 2 + which
    const int h = hw >> 1;
    const float *src = (hw & 1) ? dq2 : dq1;
    const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
    float acc = 0.f;
    if (c < d.dh) {
        const int r1 = min((chunk + 1) * kBiasChunk, d.B * d.W);
        for (int row = chunk * kBiasChunk + grp; row < r1; row += 4) {   // row = b * W + t
            const int b = row / d.W, t = row - b * d.W;
            acc += src[(((long long)b * d.H + h) * d.Wp + t) * d.dp + c];
        }
    }
    red[grp][c] = acc;
    __syncthreads();
    if (grp == 0 && c < d.dh)
        part[((long long)hw * nchunk + chunk) * 64 + c] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
}

__global__ void bwd_bias_final_kernel(BwdDims d, const float *part, int nchunk, float *du, float *dv) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;      // (h * 2 + which) * 64 + c
    if (idx >= d.H * 2 * 64) return;
    const int c = idx & 63, hw = idx >> 6, h = hw >> 1;
    if (c >= d.dh) return;
    float s = 0.f;
    for (int k = 0; k < nchunk; ++k) s += part[((long long)hw * nchunk + k) * 64 + c];
    ((hw & 1) ? dv : du)[h * d.dh + c] = s;
}

int grid_for(long long n) {
    long long blocks = (n + 255) / 256;
    return (int)(blocks > 8192 ? 8192 : (blocks < 1 ? 1 : blocks));
}

template <typename T>
void heads(const BwdDims &d, const void *src, long long src_bs, int nrows, int nrows_p, const void *bias, void *dst,
           hipStream_t s) {
    const long long n = (long long)d.B * d.H * nrows_p * d.dp;
    hipLaunchKernelGGL(heads_kernel<T>, dim3(grid_for(n)), dim3(256), 0, s, (const T *)src, src_bs, d.B, nrows,
                       nrows_p, d.D, d.H, d.dh, d.dp, (const T *)bias, (T *)dst);
}

}  // namespace

hipError_t launch_bwd_pack(bool is_bf16, const BwdDims &d, const void *q, const void *k, const void *val,
                           const void *r, const void *u, const void *v, const void *dO, void *qu, void *qv,
                           void *dOh, void *ke, void *vk, void *rk, hipStream_t s) {
    const long long qbs = (long long)d.W * d.D, kbs = (long long)d.K * d.D;
    if (is_bf16) {
        heads<bf16>(d, q, qbs, d.W, d.Wp, u, qu, s);
        heads<bf16>(d, q, qbs, d.W, d.Wp, v, qv, s);
        heads<bf16>(d, dO, qbs, d.W, d.Wp, nullptr, dOh, s);
        heads<bf16>(d, k, kbs, d.K, d.Kp, nullptr, ke, s);
        heads<bf16>(d, val, kbs, d.K, d.Kp, nullptr, vk, s);
        heads<bf16>(d, r, 0, d.K, d.Kp, nullptr, rk, s);
    } else {
        heads<float>(d, q, qbs, d.W, d.Wp, u, qu, s);
        heads<float>(d, q, qbs, d.W, d.Wp, v, qv, s);
        heads<float>(d, dO, qbs, d.W, d.Wp, nullptr, dOh, s);
        heads<float>(d, k, kbs, d.K, d.Kp, nullptr, ke, s);
        heads<float>(d, val, kbs, d.K, d.Kp, nullptr, vk, s);
        heads<float>(d, r, 0, d.K, d.Kp, nullptr, rk, s);
    }
    return hipGetLastError();
}

hipError_t launch_transpose(bool is_bf16, const void *src, int G, int H, int nrow, int ncol, long long src_ld,
                            void *dst, long long dst_hs, long long dst_cs, long long dst_bs, hipStream_t s) {
    const dim3 grid((ncol + 63) / 64, (nrow + 63) / 64, G), block(256);
    if (is_bf16)
        hipLaunchKernelGGL(transpose_kernel<bf16>, grid, block, 0, s, (const bf16 *)src, H, nrow, ncol, src_ld,
                           (bf16 *)dst, dst_hs, dst_cs, dst_bs);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float *)src, H, nrow, ncol, src_ld,
                           (float *)dst, dst_hs, dst_cs, dst_bs);
    return hipGetLastError();
}

hipError_t launch_bwd_scores(bool is_bf16, const BwdDims &d, const float *ac, const float *bd, const float *dp,
                             void *p, void *ds, void *dsd, hipStream_t s) {
    const int G = d.B * d.H;
    const long long rows = (long long)G * d.Wp;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const size_t lds = (size_t)4 * d.Kp * sizeof(float);
    const float c = (float)(1.0 / sqrt((double)d.dh));
    if (is_bf16)
        hipLaunchKernelGGL(bwd_scores_kernel<bf16>, grid, block, lds, s, ac, bd, dp, (bf16 *)p, (bf16 *)ds,
                           (bf16 *)dsd, G, d.W, d.Wp, d.m, d.K, d.Kp, c);
    else
        hipLaunchKernelGGL(bwd_scores_kernel<float>, grid, block, lds, s, ac, bd, dp, (float *)p, (float *)ds,
                           (float *)dsd, G, d.W, d.Wp, d.m, d.K, d.Kp, c);
    return hipGetLastError();
}

int bwd_bias_chunks(const BwdDims &d) { return (d.B * d.W + kBiasChunk - 1) / kBiasChunk; }

hipError_t launch_bwd_unpack(const BwdDims &d, const float *dq1, const float *dq2, const float *dkh,
                             const float *dvh, const float *drh, float *dq, float *dk, float *dval, float *dr,
                             float *du, float *dv, float *part, hipStream_t s) {
    const long long n = (long long)d.B * d.W * d.D + 2LL * d.B * d.K * d.D + (long long)d.K * d.D;
    hipLaunchKernelGGL(bwd_unpack_kernel, dim3(grid_for(n)), dim3(256), 0, s, d, dq1, dq2, dkh, dvh, drh, dq, dk,
                       dval, dr);
    const int nchunk = bwd_bias_chunks(d);
    hipLaunchKernelGGL(bwd_bias_partial_kernel, dim3(2 * d.H * nchunk), dim3(256), 0, s, d, dq1, dq2, part, nchunk);
    hipLaunchKernelGGL(bwd_bias_final_kernel, dim3((d.H * 2 * 64 + 255) / 256), dim3(256), 0, s, d, part, nchunk,
                       du, dv);
    return hipGetLastError();
}

}  // namespace txl
