// txl_backward.hip -- operand packing and reductions around the fused
// relative-attention backward (txl_attn_bwd.hip).
//
// The packing builds the head-major operands the attention kernels read (the
// pre-scaled (q + u) and (q + v), dO, keys, values, the two distance-key
// tables) and the transposed ones the batched GEMMs of dval, dk and dr take.
// The reductions sum dr's per-(batch, head) parts over the batch and du, dv
// from the fused kernel's per-wave partials (the column sums of dq's two
// parts; "Transformer-XL, explained.", the u and v legend entries: one vector
// per model, shared by every query). dq, dk and dval are written in their row
// layouts by the fused kernel and the GEMM epilogue.
#include <cstring>

#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

// One pass over the rows of a [B][nrows][D] operand, per head h of entry g = b*H + h and
// k = 0, 1 (bias0 / bias1, either may be null; out*1 null: k = 0 only), x = src[b][t][h*dh + c]:
//   hm_k[g][t][c] = (x + bias_k[h*dh + c]) * hm_scale      t < nrows_p, c < dp   (head-major)
//   tr_k[g][c][t] = x + bias_k[h*dh + c]                   c < dp, t < nrows_p   (transposed)
// zero for t >= nrows or c >= dh. A workgroup owns 64 rows of one entry: loads and head-major
// stores along c, transposed stores along t through an LDS tile. VEC (16-byte aligned rows,
// dh % 8 == 0): a thread moves eight consecutive elements per access.
// One operand to pack (rows of src, its row counts, biases, scale, outputs).
struct PackJob {
    const void *src;
    long long src_bs;
    int nrows, nrows_p;
    const void *bias0, *bias1;
    float hm_scale;
    void *hm0, *hm1, *tr0, *tr1;
    int block_begin;             // first workgroup of this job in the launch; it has nrows_p / 64 x B H
};
// The four operands of a backward call in one launch.
struct PackLaunch {
    PackJob j[4];
    int count, D, H, dh, dp;
};

template <typename T, bool VEC>
__device__ __forceinline__ void pack_tile(float (&tile)[64][65], const T *src, long long src_bs, int nrows,
                                          int nrows_p, int D, int H, int dh, int dp, const T *bias0, const T *bias1,
                                          float hm_scale, T *hm0, T *hm1, T *tr0, T *tr1, int bx, int g) {
    const int b = g / H, h = g - b * H;
    const int t0 = bx * 64;
    const int tid = threadIdx.x;
    const bool two = hm1 || tr1;
    const T *s = src + (long long)b * src_bs + h * dh;
    constexpr int E = VEC ? 8 : 1;                       // elements per access
    constexpr int TPR = 64 / E;                          // threads per row of 64 columns
    constexpr int RPI = 256 / TPR;                       // rows per iteration
    const int c0 = (tid % TPR) * E;
    float bb0[E], bb1[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        bb0[e] = (bias0 && c0 + e < dh) ? to_f32(bias0[h * dh + c0 + e]) : 0.f;
        bb1[e] = (bias1 && c0 + e < dh) ? to_f32(bias1[h * dh + c0 + e]) : 0.f;
    }
    for (int rr = tid / TPR; rr < 64; rr += RPI) {
        const int t = t0 + rr;
        float x[E];
        if constexpr (VEC) {
            if (t < nrows && c0 < dh) {
                if constexpr (sizeof(T) == 2) {
                    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(s + (long long)t * D + c0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
                } else {
                    const f32x4 lo = *reinterpret_cast<const f32x4 *>(s + (long long)t * D + c0);
                    const f32x4 hi = *reinterpret_cast<const f32x4 *>(s + (long long)t * D + c0 + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { x[e] = lo[e]; x[4 + e] = hi[e]; }
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = 0.f;
            }
        } else {
            x[0] = (t < nrows && c0 < dh) ? to_f32(s[(long long)t * D + c0]) : 0.f;
        }
        const bool rin = t < nrows;
#pragma unroll
        for (int e = 0; e < E; ++e) tile[rr][c0 + e] = x[e];
        if (c0 < dp && t < nrows_p) {
            T *o0 = hm0 + ((long long)g * nrows_p + t) * dp + c0;
            T *o1 = two && hm1 ? hm1 + ((long long)g * nrows_p + t) * dp + c0 : nullptr;
            float y0[E], y1[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool in = rin && c0 + e < dh;
                y0[e] = in ? (x[e] + bb0[e]) * hm_scale : 0.f;
                y1[e] = in ? (x[e] + bb1[e]) * hm_scale : 0.f;
            }
            if constexpr (VEC && sizeof(T) == 2) {
                if (hm0) *reinterpret_cast<bf16x8 *>(o0) = bf16x8{(bf16)y0[0], (bf16)y0[1], (bf16)y0[2], (bf16)y0[3],
                                                                  (bf16)y0[4], (bf16)y0[5], (bf16)y0[6], (bf16)y0[7]};
                if (o1) *reinterpret_cast<bf16x8 *>(o1) = bf16x8{(bf16)y1[0], (bf16)y1[1], (bf16)y1[2], (bf16)y1[3],
                                                                 (bf16)y1[4], (bf16)y1[5], (bf16)y1[6], (bf16)y1[7]};
            } else if constexpr (VEC) {
                if (hm0) {
                    *reinterpret_cast<f32x4 *>(o0) = f32x4{y0[0], y0[1], y0[2], y0[3]};
                    *reinterpret_cast<f32x4 *>(o0 + 4) = f32x4{y0[4], y0[5], y0[6], y0[7]};
                }
                if (o1) {
                    *reinterpret_cast<f32x4 *>(o1) = f32x4{y1[0], y1[1], y1[2], y1[3]};
                    *reinterpret_cast<f32x4 *>(o1 + 4) = f32x4{y1[4], y1[5], y1[6], y1[7]};
                }
            } else {
                if (hm0) o0[0] = from_f32<T>(y0[0]);
                if (o1) o1[0] = from_f32<T>(y1[0]);
            }
        }
    }
    if (!tr0 && !tr1) return;                           // uniform over the workgroup
    __syncthreads();
    // transposed: thread (c, group of E rows); column c of rows t0 + tt .. + E
    for (int idx = tid; idx < dp * TPR; idx += 256) {
        const int c = idx / TPR, tt = (idx % TPR) * E;
        const bool cin = c < dh;
        const float b0 = (bias0 && cin) ? to_f32(bias0[h * dh + c]) : 0.f;
        const float b1 = (bias1 && cin) ? to_f32(bias1[h * dh + c]) : 0.f;
        float y0[E], y1[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool in = cin && t0 + tt + e < nrows;
            const float x = tile[tt + e][c];
            y0[e] = in ? x + b0 : 0.f;
            y1[e] = in ? x + b1 : 0.f;
        }
        const long long o = ((long long)g * dp + c) * nrows_p + t0 + tt;
        if constexpr (VEC && sizeof(T) == 2) {
            if (tr0) *reinterpret_cast<bf16x8 *>(tr0 + o) = bf16x8{(bf16)y0[0], (bf16)y0[1], (bf16)y0[2], (bf16)y0[3],
                                                                   (bf16)y0[4], (bf16)y0[5], (bf16)y0[6], (bf16)y0[7]};
            if (two && tr1) *reinterpret_cast<bf16x8 *>(tr1 + o) = bf16x8{(bf16)y1[0], (bf16)y1[1], (bf16)y1[2], (bf16)y1[3],
                                                                          (bf16)y1[4], (bf16)y1[5], (bf16)y1[6], (bf16)y1[7]};
        } else if constexpr (VEC) {
            if (tr0) {
                *reinterpret_cast<f32x4 *>(tr0 + o) = f32x4{y0[0], y0[1], y0[2], y0[3]};
                *reinterpret_cast<f32x4 *>(tr0 + o + 4) = f32x4{y0[4], y0[5], y0[6], y0[7]};
            }
            if (two && tr1) {
                *reinterpret_cast<f32x4 *>(tr1 + o) = f32x4{y1[0], y1[1], y1[2], y1[3]};
                *reinterpret_cast<f32x4 *>(tr1 + o + 4) = f32x4{y1[4], y1[5], y1[6], y1[7]};
            }
        } else {
            if (tr0) tr0[o] = from_f32<T>(y0[0]);
            if (two && tr1) tr1[o] = from_f32<T>(y1[0]);
        }
    }
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(256) pack_kernel(const PackLaunch L) {
    __shared__ float tile[64][65];
    // the job of this workgroup, by uniform branches (a dynamic index into the
    // kernel-argument struct would copy it to private memory)
    const int blk = blockIdx.x;
    PackJob J;
    if (L.count > 3 && blk >= L.j[3].block_begin) J = L.j[3];
    else if (L.count > 2 && blk >= L.j[2].block_begin) J = L.j[2];
    else if (L.count > 1 && blk >= L.j[1].block_begin) J = L.j[1];
    else J = L.j[0];
    const int local = blk - J.block_begin, bxn = J.nrows_p / 64;
    const int g = local / bxn, bx = local - g * bxn;
    pack_tile<T, VEC>(tile, (const T *)J.src, J.src_bs, J.nrows, J.nrows_p, L.D, L.H, L.dh, L.dp, (const T *)J.bias0,
                      (const T *)J.bias1, J.hm_scale, (T *)J.hm0, (T *)J.hm1, (T *)J.tr0, (T *)J.tr1, bx, g);
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

// dr[j][h*dh + c] = sum over batch rows b of drh[b*H + h][j][c]; one thread per element.
__global__ void bwd_dr_kernel(BwdDims d, const float *drh, float *dr) {
    const int n = d.K * d.D;
    const long long gs = (long long)d.H * d.Kp * d.dp;          // between batch rows
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
        const int col = e % d.D, j = e / d.D;
        const int h = col / d.dh, c = col - h * d.dh;
        const float *p = drh + ((long long)h * d.Kp + j) * d.dp + c;
        float s = 0.f;
        for (int b = 0; b < d.B; ++b) s += p[b * gs];
        dr[e] = s;
    }
}

// du, dv: workgroup (which, h) adds that head's nparts per-wave column sums in a fixed order.
__global__ void __launch_bounds__(256) bwd_bias_kernel(BwdDims d, const float *part, int nparts, float *du,
                                                       float *dv) {
    __shared__ float red[4][64];
    const int which = blockIdx.x / d.H, h = blockIdx.x - which * d.H;
    const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
    const float *p = part + ((long long)which * d.H + h) * nparts * 64 + c;
    // eight independent chains (the loads of one round are all in flight together)
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int k = grp;
    for (; k + 28 < nparts; k += 32)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += p[(long long)(k + 4 * u) * 64];
    for (int u = 0; k < nparts; k += 4, ++u) acc[u] += p[(long long)k * 64];
    red[grp][c] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    if (grp == 0 && c < d.dh) (which ? dv : du)[h * d.dh + c] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
}

int grid_for(long long n) {
    long long blocks = (n + 255) / 256;
    return (int)(blocks > 8192 ? 8192 : (blocks < 1 ? 1 : blocks));
}

template <typename T>
void pack(const BwdDims &d, const BwdPack &o, const void *q, const void *k, const void *val, const void *r,
          const void *u, const void *v, const void *dO, float qscale, hipStream_t s) {
    const long long qbs = (long long)d.W * d.D, kbs = (long long)d.K * d.D;
    PackLaunch L;
    memset(&L, 0, sizeof(L));
    L.D = d.D; L.H = d.H; L.dh = d.dh; L.dp = d.dp;
    auto job = [&](const void *src, long long src_bs, int nrows, int nrows_p, const void *bias0, const void *bias1,
                   float scale, void *hm0, void *hm1, void *tr0, void *tr1) {
        PackJob &J = L.j[L.count++];
        J.src = src; J.src_bs = src_bs; J.nrows = nrows; J.nrows_p = nrows_p;
        J.bias0 = bias0; J.bias1 = bias1; J.hm_scale = scale;
        J.hm0 = hm0; J.hm1 = hm1; J.tr0 = tr0; J.tr1 = tr1;
    };
    job(q, qbs, d.W, d.Wp, u, v, qscale, o.qu, o.qv, o.qut, o.qvt);
    job(dO, qbs, d.W, d.Wp, nullptr, nullptr, 1.f, o.dOh, nullptr, o.dOt, nullptr);
    job(k, kbs, d.K, d.Kp, nullptr, nullptr, 1.f, o.ke, nullptr, o.ket, nullptr);
    job(val, kbs, d.K, d.Kp, nullptr, nullptr, 1.f, o.vk, nullptr, o.vt, nullptr);
    int blocks = 0;
    bool vec = d.dh % 8 == 0 && (d.D * sizeof(T)) % 16 == 0;
    for (int i = 0; i < L.count; ++i) {
        PackJob &J = L.j[i];
        J.block_begin = blocks;
        blocks += (J.nrows_p / 64) * d.B * d.H;
        vec = vec && (J.src_bs * sizeof(T)) % 16 == 0 && (uintptr_t)J.src % 16 == 0 &&
              (!J.bias0 || (uintptr_t)J.bias0 % 16 == 0) && (!J.bias1 || (uintptr_t)J.bias1 % 16 == 0);
    }
    if (vec) hipLaunchKernelGGL((pack_kernel<T, true>), dim3(blocks), dim3(256), 0, s, L);
    else hipLaunchKernelGGL((pack_kernel<T, false>), dim3(blocks), dim3(256), 0, s, L);
    const long long nrk = (long long)d.H * rk_table_rows(d.Kp) * d.dp;
    hipLaunchKernelGGL(rk_table_kernel<T>, dim3(grid_for(nrk)), dim3(256), 0, s, (const T *)r, d.K, d.D, d.H, d.dh,
                       d.dp, d.Kp, rk_frag_off(d.m), (T *)o.rk);
    const int ld = attn_bwd_rt_ld(d.Kp);
    const long long nrt = (long long)d.H * d.dp * ld;
    hipLaunchKernelGGL(rt_table_kernel<T>, dim3(grid_for(nrt)), dim3(256), 0, s, (const T *)r, d.K, d.D, d.H, d.dh,
                       d.dp, ld, attn_bwd_rt_off(d.m), (T *)o.rt);
}

}  // namespace

hipError_t launch_bwd_pack(bool is_bf16, const BwdDims &d, const BwdPack &o, const void *q, const void *k,
                           const void *val, const void *r, const void *u, const void *v, const void *dO,
                           float qscale, hipStream_t s) {
    if (is_bf16) pack<bf16>(d, o, q, k, val, r, u, v, dO, qscale, s);
    else pack<float>(d, o, q, k, val, r, u, v, dO, qscale, s);
    return hipGetLastError();
}

int bwd_parts(const BwdDims &d) { return d.B * ((d.W + ATTN_QBLOCK - 1) / ATTN_QBLOCK) * 4; }

hipError_t launch_bwd_finish(const BwdDims &d, const float *drh, const float *part, float *dr, float *du, float *dv,
                             hipStream_t s) {
    hipLaunchKernelGGL(bwd_dr_kernel, dim3(grid_for((long long)d.K * d.D)), dim3(256), 0, s, d, drh, dr);
    hipLaunchKernelGGL(bwd_bias_kernel, dim3(2 * d.H), dim3(256), 0, s, d, part, bwd_parts(d), du, dv);
    return hipGetLastError();
}

}  // namespace txl
