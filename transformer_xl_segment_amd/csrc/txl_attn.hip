// txl_attn.hip -- fused relative-position attention over [mem; segment].
//
// Per (batch b, head h) the kernel computes, for queries i < W and keys j < K,
//   s_ij = (q_i + u).k_j + (q_i + v).r_{m+i-j}     (visible iff j <= m + i)
//   o_i  = sum_j softmax_j(s_ij) val_j
// ("Transformer-XL, explained.", method steps 3-5 and the score legend). The
// projected operands arrive head-major; (q + u) and (q + v) are pre-scaled by
// log2(e)/sqrt(dh) so the softmax runs on exp2.
//
// Work split. A 256-thread workgroup owns 128 consecutive queries of one
// (b, h); each wave owns 32 of them and walks the visible keys in blocks of 64.
// All products use the 32x32 MFMA block with the scores held TRANSPOSED
// (S^T = K Q^T): lane a%32 of a wave holds the column of query a, and the keys
// sit in its registers, so row max and row sum over keys are register
// reductions plus one exchange with the other half of the wave, and the
// probabilities feed the P.V product (O^T = V^T P^T) straight from registers.
//
// Distance term without re-scoring every pair. For one key block the wave needs
// (q_a + v).r_delta for delta = c + a - b, c = m + i_wave - j0, a 95-wide band of
// distances. The band moves by exactly 64 per key block, so each block costs one
// new 64-distance chunk G = R_chunk (q+v)^T (the same MFMA work as the content
// term): the distance term is evaluated once per (query, distance) as the
// explainer's step 5 says, never per pair. The shift of that step becomes index
// arithmetic in LDS: each wave writes its chunk (plus the first 32 distances of
// the previous chunk, kept in registers) into a per-query row at position
// 95 - e_rel, where e_rel = a - b + 63 is the distance's offset in the band; then
// the value for key b sits at position 32 - a + b, which a lane reads with a
// per-lane base and a compile-time offset per register. Those values seed the
// accumulators of the content-term MFMAs, so the two terms add for free.
//
// The row pitch of that buffer (100 floats) keeps both the 16-byte writes of
// 16 consecutive lanes and the 4-byte skewed reads of 32 lanes on distinct
// banks. K and V^T tiles are staged in LDS with 16 bytes of row padding.
// Softmax uses a lazy maximum: the running maximum only moves (and the output
// accumulators are only rescaled) when a block's maximum exceeds it by more
// than 8 in log2 units, which keeps every exp2 below 2^8.
#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

constexpr int kWaves = 4;
constexpr int kQB = 128;          // queries per workgroup (32 per wave)
constexpr int kKB = 64;           // keys per block
constexpr int kGPitch = 100;      // floats per query row of the distance buffer
constexpr int kGX = kKB + 31;     // position of band offset 0

template <typename T, int DP>
struct AttnSmem {
    static constexpr int NO = (DP + 31) / 32;                  // 32-row blocks of O^T
    static constexpr int kPitchK = DP * (int)sizeof(T) + 16;   // bytes per key row
    static constexpr int kPitchV = kKB * (int)sizeof(T) + 16;  // bytes per value row (V^T)
    float g[kWaves][32 * kGPitch];
    char k[kKB * kPitchK];
    char v[NO * 32 * kPitchV];
};

// Two groups of four consecutive keys of one V^T row: keys [k0, k0+4) and [k0+8, k0+12).
__device__ __forceinline__ void load_vt(Frag<bf16> &f, const char *row, int k0) {
    bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + k0 * 2);
    bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + (k0 + 8) * 2);
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void load_vt(Frag<float> &f, const char *row, int k0) {
    f.lo = *reinterpret_cast<const f32x4 *>(row + k0 * 4);
    f.hi = *reinterpret_cast<const f32x4 *>(row + (k0 + 8) * 4);
}

// Registers [r0, r0+8) of an S^T block as the B operand of P.V.
__device__ __forceinline__ void p_frag(Frag<bf16> &f, const f32x16 &s, int r0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) f.v[q] = (bf16)s[r0 + q];
}
__device__ __forceinline__ void p_frag(Frag<float> &f, const f32x16 &s, int r0) {
    f.lo = f32x4{s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3]};
    f.hi = f32x4{s[r0 + 4], s[r0 + 5], s[r0 + 6], s[r0 + 7]};
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Write the 16 values of one 32-distance block of G (register i holds band
// offset e0 + crow(i)) at positions X - e for every band offset e.
__device__ __forceinline__ void write_gblock(float *grow, const f32x16 &g, int x_minus_e0, int hf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int pos = x_minus_e0 - 8 * q - 4 * hf - 3;   // lowest position of the group
        *reinterpret_cast<f32x4 *>(grow + pos) = f32x4{g[4 * q + 3], g[4 * q + 2], g[4 * q + 1], g[4 * q]};
    }
}

template <typename T, int DP>
__global__ void __launch_bounds__(256, 2) rel_attn_kernel(const AttnArgs A) {
    typedef AttnSmem<T, DP> SM;
    constexpr int NS = DP / 16;
    constexpr int NO = SM::NO;
    __shared__ SM sm;

    const int BH = A.B * A.H;
    const int nqb = (A.W + kQB - 1) / kQB;
    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x - rank * BH;
    const int qblk = nqb - 1 - rank;                 // longest query blocks first
    const int b = bh / A.H, h = bh - b * A.H;
    const int i0 = qblk * kQB;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int fr = lane & 31, hf = lane >> 5;
    const int m = A.m;
    const int iw = i0 + 32 * w;                      // first query of this wave
    const bool wave_has_queries = iw < A.W;
    const int jend = min(A.K, m + i0 + kQB);         // keys any query here can see
    const int nkb = (jend + kKB - 1) / kKB;
    const int last_key_wave = m + iw + 31;           // last key any query of the wave sees

    const T *qu = (const T *)A.qu + ((long long)bh * A.Wp) * DP;
    const T *qv = (const T *)A.qv + ((long long)bh * A.Wp) * DP;
    const T *ke = (const T *)A.ke + ((long long)bh * A.Kp) * DP;
    const T *vt = (const T *)A.vt + ((long long)bh * DP) * A.Kp;
    const T *rk = (const T *)A.rk + ((long long)h * A.Kp) * DP;

    // zero the V^T rows past DP once (they pad the last 32-row block of O^T)
    for (int idx = tid; idx < (NO * 32 - DP) * (SM::kPitchV / 4); idx += 256)
        reinterpret_cast<uint32_t *>(sm.v + DP * SM::kPitchV)[idx] = 0u;

    Frag<T> fqu[NS], fqv[NS];
    {
        const int qi = min(iw + fr, A.Wp - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            load8(fqu[s], qu + (long long)qi * DP + 16 * s + 8 * hf);
            load8(fqv[s], qv + (long long)qi * DP + 16 * s + 8 * hf);
        }
    }

    auto r_frag = [&](Frag<T> &f, int delta, int s) {
        if (delta >= 0 && delta < A.Kp) load8(f, rk + (long long)delta * DP + 16 * s + 8 * hf);
        else zero8(f);
    };

    float *grow = sm.g[w] + fr * kGPitch;
    f32x16 oacc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) oacc[o] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    // Distances [c0 + 1, c0 + 32] with c0 = m + iw: the part of the band below
    // the first key block that no chunk of the loop covers.
    f32x16 gprev = zero16();
    if (wave_has_queries) {
        const int d0 = m + iw + 1 + fr;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            Frag<T> fr_;
            r_frag(fr_, d0, s);
            mma16(gprev, fr_, fqv[s]);
        }
    }

    // cooperative K / V^T staging
    constexpr int KCH = kKB * DP * (int)sizeof(T) / 16;    // 16-byte chunks per K tile
    constexpr int VCH = DP * kKB * (int)sizeof(T) / 16;    // ... per V^T tile
    constexpr int KPT = (KCH + 255) / 256, VPT = (VCH + 255) / 256;
    constexpr int KCPR = DP * (int)sizeof(T) / 16;         // chunks per key row
    constexpr int VCPR = kKB * (int)sizeof(T) / 16;        // chunks per V^T row
    u32x4 rkt[KPT], rvt[VPT];
    auto gload = [&](int kb) {
        const int j0 = kb * kKB;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const int idx = tid + 256 * c;
            if (idx < KCH) {
                const int r = idx / KCPR, q = idx - r * KCPR;
                rkt[c] = *reinterpret_cast<const u32x4 *>((const char *)(ke + (long long)(j0 + r) * DP) + q * 16);
            }
        }
#pragma unroll
        for (int c = 0; c < VPT; ++c) {
            const int idx = tid + 256 * c;
            if (idx < VCH) {
                const int r = idx / VCPR, q = idx - r * VCPR;
                rvt[c] = *reinterpret_cast<const u32x4 *>((const char *)(vt + (long long)r * A.Kp + j0) + q * 16);
            }
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const int idx = tid + 256 * c;
            if (idx < KCH) {
                const int r = idx / KCPR, q = idx - r * KCPR;
                *reinterpret_cast<u32x4 *>(sm.k + r * SM::kPitchK + q * 16) = rkt[c];
            }
        }
#pragma unroll
        for (int c = 0; c < VPT; ++c) {
            const int idx = tid + 256 * c;
            if (idx < VCH) {
                const int r = idx / VCPR, q = idx - r * VCPR;
                *reinterpret_cast<u32x4 *>(sm.v + r * SM::kPitchV + q * 16) = rvt[c];
            }
        }
    };

    gload(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (kb + 1 < nkb) gload(kb + 1);
        const int j0 = kb * kKB;
        if (!wave_has_queries || j0 > last_key_wave) continue;

        // ---- new distance chunk: band offsets 0..63 = distances cw-63 .. cw
        const int cw = m + iw - j0;
        f32x16 gcur[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            gcur[bb] = zero16();
            const int d = cw - 63 + 32 * bb + fr;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Frag<T> f;
                r_frag(f, d, s);
                mma16(gcur[bb], f, fqv[s]);
            }
        }
        // ---- shift into place through LDS
        write_gblock(grow, gcur[0], kGX - 0, hf);
        write_gblock(grow, gcur[1], kGX - 32, hf);
        write_gblock(grow, gprev, kGX - 64, hf);
        wave_lds_sync();
        f32x16 sacc[2];
        {
            const float *rb = grow + 32 - fr + 4 * hf;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[sb][i] = rb[32 * sb + 8 * (i >> 2) + (i & 3)];
        }
        gprev = gcur[0];
        // ---- content term on top: S^T += K (q+u)^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Frag<T> f;
                load8(f, reinterpret_cast<const T *>(sm.k + (32 * sb + fr) * SM::kPitchK + (16 * s + 8 * hf) * (int)sizeof(T)));
                mma16(sacc[sb], f, fqu[s]);
            }
        // ---- causal mask on blocks that reach past the wave's first query
        if (j0 + kKB - 1 > m + iw) {
            const int lim = m + iw + fr - j0;            // last visible key offset for this lane
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * sb + crow(i, lane) > lim) sacc[sb][i] = -INFINITY;
        }
        // ---- online softmax (log2 domain)
        float mx = sacc[0][0];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[sb][i]);
        mx = fmaxf(mx, swap_half(mx));
        const float m_new = fmaxf(m_run, mx);
        if (__builtin_amdgcn_read_exec() && __any(m_new > m_run + 8.f)) {
            const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int o = 0; o < NO; ++o)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[o][i] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        float lsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(sacc[sb][i] - m_run);
                sacc[sb][i] = p;
                lsum += p;
            }
        l_run += lsum;
        // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            Frag<T> fp;
            p_frag(fp, sacc[p >> 1], 8 * (p & 1));
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                Frag<T> fv;
                load_vt(fv, sm.v + (32 * o + fr) * SM::kPitchV, 16 * p + 4 * hf);
                mma16(oacc[o], fv, fp);
            }
        }
    }

    if (!wave_has_queries) return;
    const float l_tot = l_run + swap_half(l_run);
    const float inv = 1.f / l_tot;
    const int qi = iw + fr;
    if (qi >= A.W) return;
    T *orow = (T *)A.o + (long long)b * A.o_bstride + (long long)qi * A.D + h * A.dh;
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d = 32 * o + crow(i, lane);
            if (d < A.dh) orow[d] = from_f32<T>(oacc[o][i] * inv);
        }
}

template <typename T, int DP>
hipError_t launch_dp(const AttnArgs &a, hipStream_t s) {
    const int nqb = (a.W + kQB - 1) / kQB;
    dim3 grid(a.B * a.H * nqb), block(256);
    hipLaunchKernelGGL((rel_attn_kernel<T, DP>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    switch (a.dp) {
        case 16: return launch_dp<T, 16>(a, s);
        case 32: return launch_dp<T, 32>(a, s);
        case 48: return launch_dp<T, 48>(a, s);
        case 64: return launch_dp<T, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attn_dp(int dh) { return (dh + 15) / 16 * 16; }
bool rel_attn_supported(int dh) { return dh >= 1 && dh <= 64; }

hipError_t launch_rel_attn(bool is_bf16, const AttnArgs &a, hipStream_t s) {
    return is_bf16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace txl
