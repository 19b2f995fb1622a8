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

#include "txl_attn_tile.hpp"
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
//   sum_j p_ij aV[min(delta, clip)] = aV[clip] + sum_{delta < min(clip, m+i+1)} p_i(delta) (aV[delta] - aV[clip]),
// a product over at most 128 distances per query, which runs on the matrix
// cores. A workgroup takes 128 queries of one (b, h), 32 per wave, as the
// attention kernel does, and stages (aV[d] - aV[clip])^T once. Per wave and
// chunk of 64 distances (at most two):
//   - content scores K (q+u)^T of the 95 keys the chunk reaches (key
//     m + i_wave + a - d for query a), written per query in key order to the
//     wave's band buffer;
//   - distance scores G = aK (q+v)^T in distance order, aK read from the
//     attention kernel's distance table (row ATTN_RPAD + d holds aK[min(d, clip)]);
//   - the content score of distance d read back at band position a - d' + 63
//     (d' = d - 64 chunk), p = exp2(s - lse) with the attention kernel's
//     log-sum-exp, masked to d < min(clip, m + i + 1);
//   - O^T += (aV - aV[clip])^T P^T; finally o += O + aV[clip].
// 68 KB of LDS for bf16: two workgroups per CU.
constexpr int kShawMaxClip = 128;

template <typename T, int DP>
struct ShawSmem {
    static constexpr int NO = (DP + 31) / 32;
    static constexpr int kPitchDV = kShawMaxClip * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);   // dV^T row, bytes
    float g[4][32 * kGPitch];
    char dvt[NO * 32 * kPitchDV];
};

template <typename T, int DP>
__global__ void __launch_bounds__(256, (sizeof(T) == 2 ? 2 : 1)) shaw_values_kernel(const AttnArgs A, const T *aV,
                                                                                     int clip) {
    typedef ShawSmem<T, DP> SM;
    constexpr int NS = DP / 16, NO = SM::NO;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int fr = lane & 31, hf = lane >> 5;
    const int nqb = (A.W + 127) / 128;
    const int bh = blockIdx.x / nqb;
    const int i0 = (blockIdx.x - bh * nqb) * 128;
    const int b = bh / A.H, h = bh - b * A.H;
    const int m = A.m, dh = A.dh;

    // dV^T[c][d] = aV[d][c] - aV[clip][c] for the distances the products read,
    // d < clip rounded up to 32 (zero for d >= clip or c >= dh); reads along c
    const int dlim = min(kShawMaxClip, (clip + 31) / 32 * 32);
    for (int idx = tid; idx < dlim * NO * 32; idx += 256) {
        const int d = idx / (NO * 32), c = idx - d * (NO * 32);
        const float x = (d < clip && c < dh) ? to_f32(aV[(long long)d * dh + c]) - to_f32(aV[(long long)clip * dh + c])
                                             : 0.f;
        reinterpret_cast<T *>(sm.dvt + c * SM::kPitchDV)[d] = from_f32<T>(x);
    }
    __syncthreads();

    const int iw = i0 + 32 * w;
    if (iw >= A.W) return;                               // no barrier follows
    const int qi = iw + fr;
    const bool q_ok = qi < A.W;
    const int qc = min(qi, A.Wp - 1);
    const T *qu = (const T *)A.qu + ((long long)bh * A.Wp + qc) * DP;
    const T *qv = (const T *)A.qv + ((long long)bh * A.Wp + qc) * DP;
    Frag<T> fqu[NS], fqv[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        load8(fqu[s], qu + 16 * s + 8 * hf);
        load8(fqv[s], qv + 16 * s + 8 * hf);
    }
    const float lse = q_ok ? A.lse[(long long)bh * A.Wp + qi] : 0.f;
    const T *ke = (const T *)A.ke + (long long)bh * A.C * DP;
    const T *rtab = (const T *)A.rk;                     // one table for every head
    const int roff = rk_frag_off(m);
    float *grow = sm.g[w] + fr * kGPitch;

    f32x16 oacc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) oacc[o] = zero16();
    for (int dc = 0; 64 * dc < clip; ++dc) {
        // ---- content scores of keys jbase .. jbase + 95, key order
        const int jbase = m + iw - 64 * dc - 63;
        wave_lds_sync();                                 // the previous chunk's reads are done
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) {
            int j = min(max(jbase + 32 * kb + fr, 0), A.K - 1);    // out-of-range keys are masked below
            j += A.khead;
            if (j >= A.C) j -= A.C;
            f32x16 sc = zero16();
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Frag<T> fk;
                load8(fk, ke + (long long)j * DP + 16 * s + 8 * hf);
                mma16(sc, fk, fqu[s]);
            }
            write_gblock(grow, sc, 32 * kb, hf);
        }
        wave_lds_sync();
        // ---- distance scores, p and the value product, 32 distances at a time
        const float *rb = grow + fr - 4 * hf;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const int d0 = 64 * dc + 32 * db;
            if (d0 < clip) {
                f32x16 g = zero16();
                const int row = ATTN_RPAD + d0 + fr;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    Frag<T> fa;
                    load8(fa, rtab + rk_elem(row, 16 * s + 8 * hf, roff, DP));
                    mma16(g, fa, fqv[s]);
                }
                // register i: distance d0 + crow(i) of query qi, band position fr - (32 db + crow(i)) + 63
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int d = d0 + crow(i, lane);
                    const bool ok = q_ok && d < clip && d <= m + qi;
                    const float c = rb[63 - 32 * db - 8 * (i >> 2) - (i & 3)];
                    g[i] = ok ? __builtin_amdgcn_exp2f(c + g[i] - lse) : 0.f;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Frag<T> fp;
                    p_frag(fp, g, 8 * half);
#pragma unroll
                    for (int o = 0; o < NO; ++o) {
                        Frag<T> fv;
                        load_vt(fv, sm.dvt + (32 * o + fr) * SM::kPitchDV, d0 + 16 * half + 4 * hf);
                        mma16(oacc[o], fv, fp);
                    }
                }
            }
        }
    }
    if (!q_ok) return;
    T *orow = (T *)A.o + (long long)b * A.o_bstride + (long long)qi * (A.o_ld > 0 ? A.o_ld : A.D) + h * dh;
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = 32 * o + crow(i, lane);
            if (c < dh) orow[c] = from_f32<T>(to_f32(orow[c]) + oacc[o][i] + to_f32(aV[(long long)clip * dh + c]));
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
void launch_shaw_values_t(const AttnArgs &a, const void *aV, int clip, hipStream_t s) {
    const int nqb = (a.W + 127) / 128;
    hipLaunchKernelGGL((shaw_values_kernel<T, DP>), dim3(a.B * a.H * nqb), dim3(256), 0, s, a, (const T *)aV, clip);
}

template <typename T>
hipError_t launch_shaw_values_dp(const AttnArgs &a, const void *aV, int clip, hipStream_t s) {
    switch (a.dp) {
        case 16: launch_shaw_values_t<T, 16>(a, aV, clip, s); break;
        case 32: launch_shaw_values_t<T, 32>(a, aV, clip, s); break;
        case 48: launch_shaw_values_t<T, 48>(a, aV, clip, s); break;
        case 64: launch_shaw_values_t<T, 64>(a, aV, clip, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shaw_values(bool is_bf16, const AttnArgs &a, const void *aV, int clip, hipStream_t s) {
    return is_bf16 ? launch_shaw_values_dp<bf16>(a, aV, clip, s) : launch_shaw_values_dp<float>(a, aV, clip, s);
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
