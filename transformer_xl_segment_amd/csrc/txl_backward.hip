// txl_backward.hip -- operand packing and reductions around the fused
// relative-attention backward (txl_attn_bwd.hip).
//
// The packing builds the head-major operands the attention kernels read (the
// pre-scaled (q + u) and (q + v), dO, keys, values, the two distance-key
// tables) and the transposed ones the batched GEMMs of dval, dk and dr take;
// the unpacking turns the head-major fp32 gradients back into row layouts and
// sums du, dv (the column sums of dq's two parts, "Transformer-XL,
// explained.", the u and v legend entries: one vector per model, shared by
// every query).
#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

// dst[(b*H + h)][t][c] = (src[b][t][h*dh + c] (+ bias[h*dh + c])) * scale for t < nrows, c < dh;
// zero elsewhere (t < nrows_p, c < dp). One thread per eight consecutive columns: one or two
// 16-byte stores (dp is a multiple of 16).
template <typename T>
__global__ void heads_kernel(const T *src, long long src_bs, int B, int nrows, int nrows_p, int D, int H, int dh,
                             int dp, const T *bias, float scale, T *dst) {
    const int c8n = dp >> 3;
    const int n = B * H * nrows_p * c8n;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
        const int c0 = (idx % c8n) * 8;
        const int rt = idx / c8n;
        const int t = rt % nrows_p, g = rt / nrows_p;
        const int b = g / H, h = g - b * H;
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = 0.f;
        if (t < nrows) {
            const T *row = src + (long long)b * src_bs + (long long)t * D + h * dh;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = c0 + k;
                if (c < dh) x[k] = (to_f32(row[c]) + (bias ? to_f32(bias[h * dh + c]) : 0.f)) * scale;
            }
        }
        T *out = dst + (long long)idx * 8;
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x8 *>(out) = bf16x8{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3],
                                                      (bf16)x[4], (bf16)x[5], (bf16)x[6], (bf16)x[7]};
        } else {
            *reinterpret_cast<f32x4 *>(out) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4 *>(out + 4) = f32x4{x[4], x[5], x[6], x[7]};
        }
    }
}

// 64 x 64 tiles through LDS: element (g, row, col) of src (entry g at g*src_gs, rows
// src_ld apart) goes to dst + h*dst_hs + col*dst_cs + b*dst_bs + row with g = b*H + h.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T *src, long long src_gs, int H, int nrow, int ncol,
                                                        long long src_ld, T *dst, long long dst_hs,
                                                        long long dst_cs, long long dst_bs) {
    __shared__ T tile[64][65];
    const int g = blockIdx.z, b = g / H, h = g - b * H;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const T *s = src + (long long)g * src_gs;
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

// Distance-key table of every head in the rk_elem layout (row offset off):
// table row ATTN_RPAD + d holds r[d][h*dh + c] for 0 <= d < K, c < dh; zeros elsewhere.
template <typename T>
__global__ void rk_table_kernel(const T *r, int K, int D, int H, int dh, int dp, int Kp, int off, T *tab) {
    const long long per_head = (long long)rk_table_rows(Kp) * dp, n = per_head * H;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const int h = (int)(idx / per_head);
        const int e = (int)(idx - h * per_head);
        const int t = e / (32 * dp), rem = e - t * 32 * dp;        // 32-row block, offset within it
        const int cg = rem >> 8, rr = (rem & 255) >> 3;            // column group of 8, row in block
        const int c = 8 * cg + (rem & 7);
        const int d = 32 * t + off - 32 + rr - ATTN_RPAD;
        tab[idx] = (d >= 0 && d < K && c < dh) ? r[(long long)d * D + h * dh + c] : from_f32<T>(0.f);
    }
}

// Transposed distance keys: tab[h][c][t] = r[t - toff][h*dh + c] where that is a
// distance in [0, K) and c < dh; zeros elsewhere (ld columns per row).
template <typename T>
__global__ void rt_table_kernel(const T *r, int K, int D, int H, int dh, int dp, int ld, int toff, T *tab) {
    const long long n = (long long)H * dp * ld;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const int t = (int)(idx % ld);
        const int hc = (int)(idx / ld);
        const int h = hc / dp, c = hc - h * dp;
        const int d = t - toff;
        tab[idx] = (d >= 0 && d < K && c < dh) ? r[(long long)d * D + h * dh + c] : from_f32<T>(0.f);
    }
}

// dq = dq1 + dq2 and the unpacking of dk, dval and (summed over the batch) dr into row layouts;
// one thread per output element (every count here is below 2^30).
__global__ void bwd_unpack_kernel(BwdDims d, const float *dq1, const float *dq2, const float *dkh,
                                  const float *dvh, const float *drh, float *dq, float *dk, float *dval,
                                  float *dr) {
    const int nq = d.B * d.W * d.D, nk = d.B * d.K * d.D, nr = d.K * d.D;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < nq + 2 * nk + nr; idx += gridDim.x * blockDim.x) {
        if (idx < nq) {
            const int col = idx % d.D, bt = idx / d.D;
            const int t = bt % d.W, b = bt / d.W;
            const int h = col / d.dh, c = col - h * d.dh;
            const long long src = (((long long)b * d.H + h) * d.Wp + t) * d.dp + c;
            dq[idx] = dq1[src] + dq2[src];
        } else if (idx < nq + 2 * nk) {
            const bool isv = idx >= nq + nk;
            const int e = idx - nq - (isv ? nk : 0);
            const int col = e % d.D, bj = e / d.D;
            const int j = bj % d.K, b = bj / d.K;
            const int h = col / d.dh, c = col - h * d.dh;
            const long long src = (((long long)b * d.H + h) * d.Kp + j) * d.dp + c;
            if (isv) dval[e] = dvh[src];
            else dk[e] = dkh[src];
        } else {
            const int e = idx - nq - 2 * nk;
            const int col = e % d.D, j = e / d.D;
            const int h = col / d.dh, c = col - h * d.dh;
            const long long gs = (long long)d.H * d.Kp * d.dp;         // between batch rows
            const float *p = drh + ((long long)h * d.Kp + j) * d.dp + c;
            float s = 0.f;
            for (int b = 0; b < d.B; ++b) s += p[b * gs];
            dr[e] = s;
        }
    }
}

// du, dv: per head, column sums of dq1 (resp. dq2) over every (b, t < W) row,
// in two stages: workgroup (h, which, chunk) sums one chunk of kBiasChunk rows
// into part[which][h][chunk][c]; then workgroup (h, which) adds the chunks.
constexpr int kBiasChunk = 256;

__global__ void __launch_bounds__(256) bwd_bias_partial_kernel(BwdDims d, const float *dq1, const float *dq2,
                                                               float *part, int nchunk) {
    __shared__ float red[4][64];
    const int chunk = blockIdx.x % nchunk;
    const int hw = blockIdx.x / nchunk;                  // h * 2 + which
    const int h = hw >> 1;
    const float *src = (hw & 1) ? dq2 : dq1;
    const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < d.dh) {
        const int r1 = min((chunk + 1) * kBiasChunk, d.B * d.W);
        int k = 0;
        for (int row = chunk * kBiasChunk + grp; row < r1; row += 4, k = (k + 1) & 3) {   // row = b * W + t
            const int b = row / d.W, t = row - b * d.W;
            acc[k] += src[(((long long)b * d.H + h) * d.Wp + t) * d.dp + c];
        }
    }
    red[grp][c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (grp == 0 && c < d.dh)
        part[((long long)hw * nchunk + chunk) * 64 + c] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
}

__global__ void __launch_bounds__(256) bwd_bias_final_kernel(BwdDims d, const float *part, int nchunk, float *du,
                                                             float *dv) {
    __shared__ float red[4][64];
    const int hw = blockIdx.x, h = hw >> 1;
    const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
    float s = 0.f;
    for (int k = grp; k < nchunk; k += 4) s += part[((long long)hw * nchunk + k) * 64 + c];
    red[grp][c] = s;
    __syncthreads();
    if (grp == 0 && c < d.dh) ((hw & 1) ? dv : du)[h * d.dh + c] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
}

int grid_for(long long n) {
    long long blocks = (n + 255) / 256;
    return (int)(blocks > 8192 ? 8192 : (blocks < 1 ? 1 : blocks));
}

template <typename T>
void heads(const BwdDims &d, const void *src, long long src_bs, int nrows, int nrows_p, const void *bias, float scale,
           void *dst, hipStream_t s) {
    const long long n = (long long)d.B * d.H * nrows_p * (d.dp / 8);
    hipLaunchKernelGGL(heads_kernel<T>, dim3(grid_for(n)), dim3(256), 0, s, (const T *)src, src_bs, d.B, nrows,
                       nrows_p, d.D, d.H, d.dh, d.dp, (const T *)bias, scale, (T *)dst);
}

template <typename T>
void pack(const BwdDims &d, const void *q, const void *k, const void *val, const void *r, const void *u,
          const void *v, const void *dO, float qscale, void *qu, void *qv, void *dOh, void *ke, void *vk, void *rk,
          void *rt, hipStream_t s) {
    const long long qbs = (long long)d.W * d.D, kbs = (long long)d.K * d.D;
    heads<T>(d, q, qbs, d.W, d.Wp, u, qscale, qu, s);
    heads<T>(d, q, qbs, d.W, d.Wp, v, qscale, qv, s);
    heads<T>(d, dO, qbs, d.W, d.Wp, nullptr, 1.f, dOh, s);
    heads<T>(d, k, kbs, d.K, d.Kp, nullptr, 1.f, ke, s);
    heads<T>(d, val, kbs, d.K, d.Kp, nullptr, 1.f, vk, s);
    const long long nrk = (long long)d.H * rk_table_rows(d.Kp) * d.dp;
    hipLaunchKernelGGL(rk_table_kernel<T>, dim3(grid_for(nrk)), dim3(256), 0, s, (const T *)r, d.K, d.D, d.H, d.dh,
                       d.dp, d.Kp, rk_frag_off(d.m), (T *)rk);
    const int ld = attn_bwd_rt_ld(d.Kp);
    const long long nrt = (long long)d.H * d.dp * ld;
    hipLaunchKernelGGL(rt_table_kernel<T>, dim3(grid_for(nrt)), dim3(256), 0, s, (const T *)r, d.K, d.D, d.H, d.dh,
                       d.dp, ld, attn_bwd_rt_off(d.m), (T *)rt);
}

}  // namespace

hipError_t launch_bwd_pack(bool is_bf16, const BwdDims &d, const void *q, const void *k, const void *val,
                           const void *r, const void *u, const void *v, const void *dO, float qscale, void *qu,
                           void *qv, void *dOh, void *ke, void *vk, void *rk, void *rt, hipStream_t s) {
    if (is_bf16) pack<bf16>(d, q, k, val, r, u, v, dO, qscale, qu, qv, dOh, ke, vk, rk, rt, s);
    else pack<float>(d, q, k, val, r, u, v, dO, qscale, qu, qv, dOh, ke, vk, rk, rt, s);
    return hipGetLastError();
}

hipError_t launch_heads(bool is_bf16, const BwdDims &d, const void *src, long long src_bs, int nrows, int nrows_p,
                        const void *bias, float scale, void *dst, hipStream_t s) {
    if (is_bf16) heads<bf16>(d, src, src_bs, nrows, nrows_p, bias, scale, dst, s);
    else heads<float>(d, src, src_bs, nrows, nrows_p, bias, scale, dst, s);
    return hipGetLastError();
}

hipError_t launch_transpose(bool is_bf16, const void *src, long long src_gs, int G, int H, int nrow, int ncol,
                            long long src_ld, void *dst, long long dst_hs, long long dst_cs, long long dst_bs,
                            hipStream_t s) {
    const dim3 grid((ncol + 63) / 64, (nrow + 63) / 64, G), block(256);
    if (is_bf16)
        hipLaunchKernelGGL(transpose_kernel<bf16>, grid, block, 0, s, (const bf16 *)src, src_gs, H, nrow, ncol, src_ld,
                           (bf16 *)dst, dst_hs, dst_cs, dst_bs);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float *)src, src_gs, H, nrow, ncol, src_ld,
                           (float *)dst, dst_hs, dst_cs, dst_bs);
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
    hipLaunchKernelGGL(bwd_bias_final_kernel, dim3(d.H * 2), dim3(256), 0, s, d, part, nchunk, du, dv);
    return hipGetLastError();
}

}  // namespace txl
