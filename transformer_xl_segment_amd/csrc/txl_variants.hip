// txl_variants.hip -- the position encodings Transformer-XL is compared against.
//
// "Transformer-XL, explained." ("What it adds to earlier relative positions";
// the ablations in its results) sets the paper's encoding against two others:
//  - Shaw, Uszkoreit and Vaswani: learned embeddings of the clipped distance,
//    used in the first two score terms only (no u, v) and also added to the
//    values: o_i = sum_j p_ij (val_j + aV[min(delta, clip)]);
//  - absolute sinusoid positions added to the rows, with content-only attention.
// The attention kernel serves both: with a one-table distance buffer built from
// aK for Shaw (the band machinery needs no change), without its distance term
// for absolute positions. The kernels below build that buffer, add Shaw's value
// term after the fact, and add absolute positions to rows.
#include <math.h>

#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

// Distance keys of Shaw's encoding in the attention kernel's table layout
// (rk_elem with row offset off): one table shared by all heads; row
// ATTN_RPAD + d is aK[min(d, clip)] for 0 <= d < K, zeros elsewhere and in
// columns >= dh.
template <typename T>
__global__ void shaw_rows_kernel(T *rk, const T *aK, int clip, int K, int rows, int dh, int dp, int off) {
    const long long n = (long long)rows * dp;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const int r = (int)(idx / dp), c = (int)(idx - (long long)r * dp);
        const int d = r - ATTN_RPAD;
        T v = from_f32<T>(0.f);
        if (d >= 0 && d < K && c < dh) v = aK[(long long)(d < clip ? d : clip) * dh + c];
        rk[rk_elem(r, c, off, dp)] = v;
    }
}

// Shaw's value term, added to the attention output o [B][W][D] (head slices of
// width dh). Because aV is constant for distances >= clip and the weights of a
// query sum to one,
//   sum_j p_ij aV[min(delta, clip)] = aV[clip] + sum_{delta < min(clip, m+i+1)} p_i(delta) (aV[delta] - aV[clip]).
// A workgroup takes 16 consecutive queries of one (b, h). It stages in LDS,
// once, the key rows the 16 bands touch, the distance rows aK[d] for d < clip
// and the differences aV[d] - aV[clip] (global reads coalesced, rows padded to
// an odd number of dwords so lanes reading different rows hit distinct banks).
// Each wave then takes four queries in turn: lanes score the band's keys (the
// same pre-scaled operands as the attention kernel, fp32 sums), p = exp2(s -
// lse) with the kernel's log-sum-exp, and lanes own output columns to sum over
// the band.
constexpr int kShawMaxClip = 128;
constexpr int kShawQueries = 16;

template <typename T, int DP>
struct ShawSmem {
    static constexpr int kRowDw = DP * (int)sizeof(T) / 4;        // dwords of one operand row
    static constexpr int kPitchDw = kRowDw + 1;                     // odd: conflict-free row-wise reads
    uint32_t k[(kShawMaxClip + kShawQueries) * kPitchDw];
    uint32_t ak[kShawMaxClip * kPitchDw];
    float dv[kShawMaxClip * DP];
    float p[4][kShawMaxClip];
    float q[4][2][DP];
};

// Adds the products of one operand dword (one fp32 or two bf16 columns) with
// the query columns it belongs to.
template <typename T> __device__ __forceinline__ float dot_dw(uint32_t x, const float *q, float s);
template <> __device__ __forceinline__ float dot_dw<float>(uint32_t x, const float *q, float s) {
    return fmaf(q[0], __uint_as_float(x), s);
}
template <> __device__ __forceinline__ float dot_dw<bf16>(uint32_t x, const float *q, float s) {
    s = fmaf(q[0], __uint_as_float(x << 16), s);
    return fmaf(q[1], __uint_as_float(x & 0xffff0000u), s);
}

template <typename T, int DP>
__global__ void __launch_bounds__(256) shaw_values_kernel(const T *qu, const T *qv, const T *ke, const T *aK,
                                                          const float *lse, const T *aV, T *o, int H, int W,
                                                          int Wp, int m, int Kp, int dh, int D, int clip) {
    typedef ShawSmem<T, DP> SM;
    constexpr int RD = SM::kRowDw, PD = SM::kPitchDw, EPD = 4 / (int)sizeof(T);   // columns per dword
    __shared__ SM sm;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nqb = (W + kShawQueries - 1) / kShawQueries;
    const int bh = blockIdx.x / nqb;
    const int i0 = (blockIdx.x - bh * nqb) * kShawQueries;
    const int iend = min(i0 + kShawQueries, W);
    const int b = bh / H, h = bh - b * H;
    // keys of the 16 bands: jlo .. m + iend - 1
    const int jlo = max(0, m + i0 - clip + 1);
    const int nk = m + iend - jlo;
    // (independent loads, unrolled so that several are in flight at once)
    const uint32_t *kg = reinterpret_cast<const uint32_t *>(ke + ((long long)bh * Kp + jlo) * DP);
#pragma unroll 8
    for (int idx = threadIdx.x; idx < nk * RD; idx += 256) {
        const int r = idx / RD, u = idx - r * RD;
        sm.k[r * PD + u] = kg[idx];
    }
    // aK rows 0 .. clip-1, zero past column dh
    T *akl = reinterpret_cast<T *>(sm.ak);
#pragma unroll 8
    for (int idx = threadIdx.x; idx < clip * DP; idx += 256) {
        const int r = idx / DP, c = idx - r * DP;
        akl[r * PD * EPD + c] = c < dh ? aK[(long long)r * dh + c] : from_f32<T>(0.f);
    }
    // rows d = w, w + 4, ... of the value differences (columns >= dh are never read)
    const float tail = lane < dh ? to_f32(aV[(long long)clip * dh + lane]) : 0.f;
    if (lane < dh) {
#pragma unroll 8
        for (int d = w; d < clip; d += 4) sm.dv[d * DP + lane] = to_f32(aV[(long long)d * dh + lane]) - tail;
    }
    __syncthreads();
    for (int qq = 0; qq < kShawQueries / 4; ++qq) {
        const int i = i0 + 4 * qq + w;
        if (i >= W) break;                                        // wave-uniform
        const int nb = min(clip, m + i + 1);                      // band distances 0 .. nb-1
        if (lane < DP) {
            sm.q[w][0][lane] = to_f32(qu[((long long)bh * Wp + i) * DP + lane]);
            sm.q[w][1][lane] = to_f32(qv[((long long)bh * Wp + i) * DP + lane]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float l = lse[(long long)bh * Wp + i];
        for (int d = lane; d < nb; d += 64) {
            const uint32_t *kr = sm.k + (m + i - d - jlo) * PD;
            const uint32_t *ar = sm.ak + d * PD;
            float s[4] = {0.f, 0.f, 0.f, 0.f};       // four independent chains
#pragma unroll
            for (int u = 0; u < RD; ++u) {
                s[u & 3] = dot_dw<T>(kr[u], &sm.q[w][0][EPD * u], s[u & 3]);
                s[u & 3] = dot_dw<T>(ar[u], &sm.q[w][1][EPD * u], s[u & 3]);
            }
            sm.p[w][d] = exp2f(((s[0] + s[1]) + (s[2] + s[3])) - l);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < dh) {
            float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
            int d = 0;
            for (; d + 4 <= nb; d += 4) {
                acc0 = fmaf(sm.p[w][d], sm.dv[d * DP + lane], acc0);
                acc1 = fmaf(sm.p[w][d + 1], sm.dv[(d + 1) * DP + lane], acc1);
                acc2 = fmaf(sm.p[w][d + 2], sm.dv[(d + 2) * DP + lane], acc2);
                acc3 = fmaf(sm.p[w][d + 3], sm.dv[(d + 3) * DP + lane], acc3);
            }
            for (; d < nb; ++d) acc0 = fmaf(sm.p[w][d], sm.dv[d * DP + lane], acc0);
            T *dst = o + ((long long)b * W + i) * D + (long long)h * dh + lane;
            *dst = from_f32<T>(to_f32(*dst) + (tail + ((acc0 + acc1) + (acc2 + acc3))));
        }
        // the next query reuses q and p of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// y[b][t] = x[b][t] + U[pos0 + t], U the [sin | cos] sinusoid of the absolute
// position (the distance table's formula with a position in place of a
// distance): the angle and its sine and cosine in double precision (the
// frequencies computed once per workgroup), the sum in fp32.
template <typename T>
__global__ void add_positions_kernel(const T *x, long long x_bstride, T *y, long long y_bstride, int B, int W,
                                     int D, int pos0) {
    __shared__ double freq[512];
    const int half = D / 2;
    for (int k = threadIdx.x; k < half; k += blockDim.x) freq[k] = pow(10000.0, -2.0 * (double)k / (double)D);
    __syncthreads();
    const long long n = (long long)B * W * half;
    for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
         idx += (long long)gridDim.x * blockDim.x) {
        const long long bt = idx / half;
        const int k = (int)(idx - bt * half);
        const int b = (int)(bt / W), t = (int)(bt - (long long)b * W);
        double sn, cs;
        sincos((double)(pos0 + t) * freq[k], &sn, &cs);
        const T *xr = x + (long long)b * x_bstride + (long long)t * D;
        T *yr = y + (long long)b * y_bstride + (long long)t * D;
        yr[k] = from_f32<T>(to_f32(xr[k]) + (float)sn);
        yr[half + k] = from_f32<T>(to_f32(xr[half + k]) + (float)cs);
    }
}

int grid_for(long long n) {
    long long blocks = (n + 255) / 256;
    return (int)(blocks > 4096 ? 4096 : (blocks < 1 ? 1 : blocks));
}

}  // namespace

int shaw_max_clip() { return kShawMaxClip; }

hipError_t launch_shaw_rows(bool is_bf16, void *rk, const void *aK, int clip, int K, int Kp, int dh, int dp,
                            int off, hipStream_t s) {
    const int rows = Kp + 2 * ATTN_RPAD;
    const int g = grid_for((long long)rows * dp);
    if (is_bf16)
        hipLaunchKernelGGL(shaw_rows_kernel<bf16>, dim3(g), dim3(256), 0, s, (bf16 *)rk, (const bf16 *)aK, clip, K,
                           rows, dh, dp, off);
    else
        hipLaunchKernelGGL(shaw_rows_kernel<float>, dim3(g), dim3(256), 0, s, (float *)rk, (const float *)aK, clip,
                           K, rows, dh, dp, off);
    return hipGetLastError();
}

template <typename T, int DP>
void launch_shaw_values_t(const AttnArgs &a, const void *aK, const void *aV, int clip, hipStream_t s) {
    const int nqb = (a.W + kShawQueries - 1) / kShawQueries;
    hipLaunchKernelGGL((shaw_values_kernel<T, DP>), dim3(a.B * a.H * nqb), dim3(256), 0, s, (const T *)a.qu,
                       (const T *)a.qv, (const T *)a.ke, (const T *)aK, (const float *)a.lse, (const T *)aV,
                       (T *)a.o, a.H, a.W, a.Wp, a.m, a.Kp, a.dh, a.D, clip);
}

template <typename T>
hipError_t launch_shaw_values_dp(const AttnArgs &a, const void *aK, const void *aV, int clip, hipStream_t s) {
    switch (a.dp) {
        case 16: launch_shaw_values_t<T, 16>(a, aK, aV, clip, s); break;
        case 32: launch_shaw_values_t<T, 32>(a, aK, aV, clip, s); break;
        case 48: launch_shaw_values_t<T, 48>(a, aK, aV, clip, s); break;
        case 64: launch_shaw_values_t<T, 64>(a, aK, aV, clip, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shaw_values(bool is_bf16, const AttnArgs &a, const void *aK, const void *aV, int clip,
                              hipStream_t s) {
    return is_bf16 ? launch_shaw_values_dp<bf16>(a, aK, aV, clip, s) : launch_shaw_values_dp<float>(a, aK, aV, clip, s);
}

hipError_t launch_add_positions(bool is_bf16, const void *x, long long x_bstride, void *y, long long y_bstride,
                                int B, int W, int D, int pos0, hipStream_t s) {
    const int g = grid_for((long long)B * W * (D / 2));
    if (is_bf16)
        hipLaunchKernelGGL(add_positions_kernel<bf16>, dim3(g), dim3(256), 0, s, (const bf16 *)x, x_bstride,
                           (bf16 *)y, y_bstride, B, W, D, pos0);
    else
        hipLaunchKernelGGL(add_positions_kernel<float>, dim3(g), dim3(256), 0, s, (const float *)x, x_bstride,
                           (float *)y, y_bstride, B, W, D, pos0);
    return hipGetLastError();
}

}  // namespace txl
