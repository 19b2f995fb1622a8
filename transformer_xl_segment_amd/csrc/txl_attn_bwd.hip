// txl_attn_bwd.hip -- fused query side of the relative-attention backward.
//
// Training stops the gradient at the memory ("Transformer-XL, explained.",
// method step 2 and the SG(.) legend entry), so the backward of one segment is
// the gradient of the attention w.r.t. its projected operands. With
// c = 1/sqrt(dh), p the softmax of the scores and dO the incoming gradient:
//   dP_ij = dO_i.val_j,  D_i = sum_j p_ij dP_ij = dO_i.o_i,  dS_ij = c p_ij (dP_ij - D_i)
//   dq_i  = sum_j dS_ij k_j + sum_j dS_ij r_{m+i-j}
//   dk_j  = sum_i dS_ij (q_i + u),  dval_j = sum_i p_ij dO_i,
//   dr_d  = sum_{m+i-j=d} dS_ij (q_i + v).
//
// This kernel walks the keys of each query exactly like the forward kernel
// (txl_attn.hip): a workgroup owns 128 queries of one (b, h), each wave 32,
// the scores are held transposed (lane = query, keys in registers) and the
// distance term arrives through the same LDS band of G = R (q+v)^T chunks. It
// recomputes p from the forward's log-sum-exp (no running maximum), forms dP
// on the matrix cores (V dO^T) and dS, and then
//   - accumulates dq's content part K^T dS^T in registers (K^T staged in LDS
//     like V^T in the forward);
//   - scatters dS by distance into a per-query ring of 128 LDS slots: key b of
//     query a lands at distance cw + a - b, cw = m + i_wave - j0. The band of a
//     key block spans 95 distances and moves by 64 per block, so after block
//     kb the 64 distances [cw-32, cw+31] are complete: they are read back as
//     the B operand of dq's distance part R^T dS_d^T (R^T fragments from a
//     transposed table in L2) and written out, distance-major, for dr;
//   - writes p and dS themselves, key-major, for dval and dk.
// dval = P^T dO, dk = dS^T (q+u) and, per batch row, dr = dS_d^T (q+v) are
// then plain batched GEMMs over those matrices (dr summed over the batch after). Every matrix entry is
// written once (zeros where no key is visible), so no clearing pass is needed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "txl_attn_tile.hpp"
#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

constexpr int kWaves = 4;
constexpr int kQB = 128;          // queries per workgroup (32 per wave)
constexpr int kKB = 64;           // keys per block
constexpr int kRing = 128;        // distance slots per query row of the dS ring

template <typename T, int DP>
struct BwdSmem {
    // bf16 stages V in LDS; fp32 reads its V fragments from L2 (the fp32 tiles
    // would not fit next to the band and the ring)
    static constexpr bool VLDS = sizeof(T) == 2;
    static constexpr int NO = (DP + 31) / 32;
    static constexpr int kPitchK = DP * (int)sizeof(T) + 16;                        // K / V row, bytes
    static constexpr int kPitchT = kKB * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16); // K^T row, bytes
    static constexpr int kPitchR = kRing + 16 / (int)sizeof(T);                      // ring row, elements
    float g[kWaves][32 * kGPitch];
    T ring[kWaves][32 * kPitchR];
    char k[kKB * kPitchK];
    char v[VLDS ? kKB * kPitchK : 16];
    char kt[NO * 32 * kPitchT];
};

__device__ __forceinline__ float frag_at(const Frag<bf16> &f, int t) { return (float)f.v[t]; }
__device__ __forceinline__ bf16 frag_elem(const Frag<bf16> &f, int t) { return f.v[t]; }
__device__ __forceinline__ float frag_elem(const Frag<float> &f, int t) { return t < 4 ? f.lo[t] : f.hi[t - 4]; }
__device__ __forceinline__ float frag_at(const Frag<float> &f, int t) { return t < 4 ? f.lo[t] : f.hi[t - 4]; }
__device__ __forceinline__ void frag_set(Frag<bf16> &f, int t, float x) { f.v[t] = (bf16)x; }
__device__ __forceinline__ void frag_set(Frag<float> &f, int t, float x) {
    if (t < 4) f.lo[t] = x;
    else f.hi[t - 4] = x;
}

template <typename T, int DP>
__global__ void __launch_bounds__(256, 1) rel_attn_bwd_kernel(const AttnBwdArgs A) {
    typedef BwdSmem<T, DP> SM;
    constexpr int NS = DP / 16;
    constexpr int NO = SM::NO;
    constexpr int RP = SM::kPitchR;
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
    const int qi = iw + fr;                          // this lane's query
    const bool q_ok = qi < A.W;
    const int jend = min(A.K, m + i0 + kQB);         // keys any query here can see
    const int nkb = (jend + kKB - 1) / kKB;
    const int last_key_wave = m + iw + 31;           // last key any query of the wave sees
    const int kb_last = min(last_key_wave / kKB, nkb - 1);

    const T *qu = (const T *)A.qu + ((long long)bh * A.Wp) * DP;
    const T *qv = (const T *)A.qv + ((long long)bh * A.Wp) * DP;
    const T *dO = (const T *)A.dO + ((long long)bh * A.Wp) * DP;
    const T *ke = (const T *)A.ke + ((long long)bh * A.Kp) * DP;
    const T *vk = (const T *)A.vk + ((long long)bh * A.Kp) * DP;
    const T *kt = (const T *)A.kt + ((long long)bh * DP) * A.Kp;
    const T *rtab = (const T *)A.rk + (long long)h * A.rk_hstride;
    const T *rt = (const T *)A.rt + (long long)h * DP * A.rt_ld + A.rt_off;
    T *pt = (T *)A.pt + (long long)bh * A.Kp * A.Wp;
    T *dst = (T *)A.dst + (long long)bh * A.Kp * A.Wp;
    T *dsd = (T *)A.dsd + (long long)bh * A.Kp * A.Wp;
    const int roff = rk_frag_off(m);
    const int dlow = -94 + ((roff - (ATTN_RPAD - 94)) & 31);

    // zero the K^T rows past DP once (they pad the last 32-row block of dq^T)
    for (int idx = tid; idx < (NO * 32 - DP) * (SM::kPitchT / 4); idx += 256)
        reinterpret_cast<uint32_t *>(sm.kt + DP * SM::kPitchT)[idx] = 0u;

    Frag<T> fqu[NS], fqv[NS], fdo[NS];
    {
        const int qc = min(qi, A.Wp - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            load8(fqu[s], qu + (long long)qc * DP + 16 * s + 8 * hf);
            load8(fqv[s], qv + (long long)qc * DP + 16 * s + 8 * hf);
            load8(fdo[s], dO + (long long)qc * DP + 16 * s + 8 * hf);
        }
    }
    // per query: log-sum-exp of the forward (log2 units) and D = dO . o
    const float lse_q = q_ok ? A.lse[(long long)bh * A.Wp + qi] : 0.f;
    float dpart = 0.f;
    if (q_ok) {
        const T *orow = (const T *)A.o + ((long long)b * A.W + qi) * A.D + h * A.dh;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int c = 16 * s + 8 * hf + t;
                if (c < A.dh) dpart += frag_at(fdo[s], t) * to_f32(orow[c]);
            }
    }
    const float Dq = half_sum(dpart);

    auto r_frag = [&](Frag<T> &f, int d0, int s) {
        const long long blk = (d0 + ATTN_RPAD - roff) / 32 + 1;
        load8(f, rtab + blk * 32 * DP + (2 * s + hf) * 256 + fr * 8);
    };
    auto r_chunk = [&](Frag<T> (&f)[2][NS], int d0) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int s = 0; s < NS; ++s) r_frag(f[bb][s], d0 + 32 * bb, s);
    };
    auto g_chunk = [&](f32x16 (&g)[2], const Frag<T> (&f)[2][NS]) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            g[bb] = zero16();
#pragma unroll
            for (int s = 0; s < NS; ++s) mma16(g[bb], f[bb][s], fqv[s]);
        }
    };

    // cooperative staging of the K, V (bf16) and K^T tiles of a key block
    constexpr int KCH = kKB * DP * (int)sizeof(T) / 16;    // 16-byte chunks per K tile
    constexpr int TCH = DP * kKB * (int)sizeof(T) / 16;    // ... per K^T tile
    constexpr int KPT = (KCH + 255) / 256, TPT = (TCH + 255) / 256;
    constexpr int VPT = SM::VLDS ? KPT : 1;
    constexpr int KCPR = DP * (int)sizeof(T) / 16;         // chunks per key row
    constexpr int TCPR = kKB * (int)sizeof(T) / 16;        // chunks per K^T row
    u32x4 sk[KPT], sv[VPT], st[TPT];
    auto gload = [&](int kb) {
        const int j0 = kb * kKB;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const int idx = tid + 256 * c;
            if (KCH % 256 == 0 || idx < KCH) {
                const int r = idx / KCPR, q = idx - r * KCPR;
                sk[c] = *reinterpret_cast<const u32x4 *>((const char *)(ke + (long long)(j0 + r) * DP) + q * 16);
                if constexpr (SM::VLDS)
                    sv[c] = *reinterpret_cast<const u32x4 *>((const char *)(vk + (long long)(j0 + r) * DP) + q * 16);
            }
        }
#pragma unroll
        for (int c = 0; c < TPT; ++c) {
            const int idx = tid + 256 * c;
            if (TCH % 256 == 0 || idx < TCH) {
                const int r = idx / TCPR, q = idx - r * TCPR;
                st[c] = *reinterpret_cast<const u32x4 *>(kt + (long long)r * A.Kp + j0 + q * (16 / (int)sizeof(T)));
            }
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const int idx = tid + 256 * c;
            if (KCH % 256 == 0 || idx < KCH) {
                const int r = idx / KCPR, q = idx - r * KCPR;
                *reinterpret_cast<u32x4 *>(sm.k + r * SM::kPitchK + q * 16) = sk[c];
                if constexpr (SM::VLDS) *reinterpret_cast<u32x4 *>(sm.v + r * SM::kPitchK + q * 16) = sv[c];
            }
        }
#pragma unroll
        for (int c = 0; c < TPT; ++c) {
            const int idx = tid + 256 * c;
            if (TCH % 256 == 0 || idx < TCH) {
                const int r = idx / TCPR, q = idx - r * TCPR;
                u32x2 *d = reinterpret_cast<u32x2 *>(sm.kt + r * SM::kPitchT + q * 16);
                d[0] = u32x2{st[c][0], st[c][1]};
                d[1] = u32x2{st[c][2], st[c][3]};
            }
        }
    };
    if (nkb > 0) gload(0);

    float *grow = sm.g[w] + fr * kGPitch;
    // byte offsets of this lane's stores, fixed for the kernel: rows 4*hf + r of a group
    // of four keys (p, dS) and row 8*hf of a group of eight distances, column qi
    uint32_t poff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) poff[r] = (uint32_t)(((4 * hf + r) * A.Wp + qi) * (int)sizeof(T));
    const uint32_t doff = (uint32_t)((8 * hf * A.Wp + qi) * (int)sizeof(T));
    T *ring = sm.ring[w] + fr * RP;
    f32x16 dqu[NO], dqv[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) dqu[o] = dqv[o] = zero16();

    // distance band, as in the forward kernel: gb[kb & 1] holds the chunk
    // cw-63 .. cw of block kb, rnext the r fragments of the next chunk
    f32x16 gtop = zero16(), gb[2][2];
    Frag<T> rnext[2][NS];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s = 0; s < NS; ++s) rnext[bb][s] = Frag<T>{};
    if (wave_has_queries && nkb > 0) {
        const int c0 = m + iw;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            Frag<T> f;
            r_frag(f, c0 + 1, s);
            mma16(gtop, f, fqv[s]);
        }
        r_chunk(rnext, c0 - 63);
        g_chunk(gb[0], rnext);
        if (kKB <= last_key_wave) r_chunk(rnext, c0 - 127);
        write_gblock(grow, gb[0][0], 0, hf);
        write_gblock(grow, gb[0][1], 32, hf);
        write_gblock(grow, gtop, 64, hf);
    }

    // Distances [base, base + 64) of the ring, which start at slot p0: masked to
    // the keys seen so far (0 <= j <= jmax, d >= 0), written out for dr and
    // multiplied into dq's distance part.
    // Only the first block's window (keys below 0, never written) and the last one (keys past
    // the wave's last block, stale) need the mask; every other entry was written by this
    // block or the one before it, zero where the key is not visible.
    auto flush = [&](int base, int p0, int jmax, bool masked) __attribute__((always_inline)) {
        wave_lds_sync();
        const bool rows_in = base >= 0 && base + 63 < A.Kp;     // every row of the window exists
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int d0 = base + 16 * s4 + 8 * hf;
            Frag<T> fb;
            load8(fb, ring + p0 + 16 * s4 + 8 * hf);
            if (masked) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int d = d0 + t, j = m + qi - d;
                    if (d < 0 || j < 0 || j > jmax) frag_set(fb, t, 0.f);
                }
            }
            if (rows_in) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    char *rowp = (char *)dsd + (long long)(base + 16 * s4 + t) * A.Wp * (long long)sizeof(T);
                    *reinterpret_cast<T *>(rowp + doff) = frag_elem(fb, t);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int d = d0 + t;
                    if (d >= 0 && d < A.Kp) dsd[(long long)d * A.Wp + qi] = frag_elem(fb, t);
                }
            }
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                Frag<T> fa;
                load8(fa, rt + (long long)min(32 * o + fr, DP - 1) * A.rt_ld + d0);
                mma16(dqv[o], fa, fb);
            }
        }
    };

    auto step = [&](auto parity, int kb) __attribute__((always_inline)) {
        constexpr int P = decltype(parity)::value, Q = 1 - P;
        __syncthreads();
        sstore();
        __syncthreads();
        if (kb + 1 < nkb) gload(kb + 1);
        const int j0 = kb * kKB;
        if (!wave_has_queries || j0 > last_key_wave) return;

        // ---- distance term from the band, relative to the log-sum-exp
        wave_lds_sync();
        f32x16 sacc[2];
        {
            const float *rb = grow + fr - 4 * hf;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[sb][i] = rb[63 - 32 * sb - 8 * (i >> 2) - (i & 3)] - lse_q;
        }
        // ---- content term: S^T += K (q+u)^T; dP^T = V dO^T
        f32x16 dpa[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            dpa[sb] = zero16();
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Frag<T> f, fv;
                const int off = (32 * sb + fr) * SM::kPitchK + (16 * s + 8 * hf) * (int)sizeof(T);
                load8(f, reinterpret_cast<const T *>(sm.k + off));
                mma16(sacc[sb], f, fqu[s]);
                if constexpr (SM::VLDS) load8(fv, reinterpret_cast<const T *>(sm.v + off));
                else load8(fv, vk + (long long)(j0 + 32 * sb + fr) * DP + 16 * s + 8 * hf);
                mma16(dpa[sb], fv, fdo[s]);
            }
        }
        // ---- causal mask (and queries past W)
        if (j0 + kKB - 1 > m + iw || iw + 31 >= A.W) {
            const int lim = q_ok ? m + qi - j0 : -1;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * sb + crow(i, lane) > lim) sacc[sb][i] = -INFINITY;
        }
        // ---- next distance chunk, then p = exp2(s - lse)
        g_chunk(gb[Q], rnext);
        r_chunk(rnext, max(m + iw - j0 - kKB - 127, dlow));
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[sb][i] = __builtin_amdgcn_exp2f(sacc[sb][i]);
        // band of block kb+1 (this block's band reads are complete)
        write_gblock(grow, gb[Q][0], 0, hf);
        write_gblock(grow, gb[Q][1], 32, hf);
        write_gblock(grow, gb[P][0], 64, hf);
        // ---- dS = c p (dP - D)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) dpa[sb][i] = A.c * sacc[sb][i] * (dpa[sb][i] - Dq);
        // ---- p and dS, key-major (row j0 + b, column qi): a uniform row base per group of
        // four keys plus the lane's fixed offset
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const long long ro = (long long)(j0 + 32 * sb + 8 * q) * A.Wp * (long long)sizeof(T);
                char *pb = (char *)pt + ro;
                char *db = (char *)dst + ro;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *reinterpret_cast<T *>(pb + poff[r]) = from_f32<T>(sacc[sb][4 * q + r]);
                    *reinterpret_cast<T *>(db + poff[r]) = from_f32<T>(dpa[sb][4 * q + r]);
                }
            }
        // ---- dq^T (content) += K^T dS^T, 16 keys per MFMA
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            Frag<T> fd;
            p_frag(fd, dpa[p >> 1], 8 * (p & 1));
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                Frag<T> fk;
                load_vt(fk, sm.kt + (32 * o + fr) * SM::kPitchT, 16 * p + 4 * hf);
                mma16(dqu[o], fk, fd);
            }
        }
        // ---- dS into the ring: key b of query a at distance cw + a - b, slot
        // (d - (m + iw) + 160) mod 128
        {
            const int L = fr - 4 * hf + 160 - kKB * kb;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    ring[(L - (32 * sb + 8 * (i >> 2) + (i & 3))) & (kRing - 1)] = from_f32<T>(dpa[sb][i]);
        }
        // distances [cw - 32, cw + 31] are complete
        flush(m + iw - j0 - 32, (kRing - kKB * kb) & (kRing - 1), j0 + kKB - 1, kb == 0);
    };

    for (int kb = 0; kb < nkb; kb += 2) {
        step(std::integral_constant<int, 0>(), kb);
        if (kb + 1 < nkb) step(std::integral_constant<int, 1>(), kb + 1);
    }

    // du, dv partials: slot (b, query block, wave) of each head holds the column sums of
    // dq's two parts over the wave's queries (lanes past W hold exact zeros)
    const int nparts = A.B * nqb * kWaves;
    float *pu = A.part + ((long long)h * nparts + (b * nqb + qblk) * kWaves + w) * 64;
    float *pv = pu + (long long)A.H * nparts * 64;
    if (!wave_has_queries) {
        pu[lane] = 0.f;
        pv[lane] = 0.f;
        return;
    }
    // the distances the last block left open
    flush(m + iw - kb_last * kKB - 96, (kKB - kKB * kb_last) & (kRing - 1), kb_last * kKB + kKB - 1, true);
    // zeros where no key of the wave is visible: key rows past its last block,
    // distances past its last query's
    for (int j = (kb_last + 1) * kKB + hf; j < A.Kp; j += 2) {
        pt[(long long)j * A.Wp + qi] = from_f32<T>(0.f);
        dst[(long long)j * A.Wp + qi] = from_f32<T>(0.f);
    }
    for (int d = m + iw + 32 + hf; d < A.Kp; d += 2) dsd[(long long)d * A.Wp + qi] = from_f32<T>(0.f);
    // column sums through the wave's band buffer (free now): row a = query, column c
    {
        constexpr int CP = 68;                           // 32 x 68 floats fit the 32 x kGPitch buffer
        float *buf = sm.g[w];
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            wave_lds_sync();
#pragma unroll
            for (int o = 0; o < NO; ++o)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 32 * o + crow(4 * q, lane);
                    const f32x16 &acc = pass ? dqv[o] : dqu[o];
                    if (c < DP)
                        *reinterpret_cast<f32x4 *>(buf + fr * CP + c) =
                            f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
                }
            wave_lds_sync();
            float sum = 0.f;
            if (lane < DP)
#pragma unroll 8
                for (int a = 0; a < 32; ++a) sum += buf[a * CP + lane];
            (pass ? pv : pu)[lane] = sum;
        }
    }
    if (!q_ok) return;
    // dq = content part + distance part, row layout [B][W][D]
    float *dqrow = A.dq + ((long long)b * A.W + qi) * A.D + h * A.dh;
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = 32 * o + crow(i, lane);
            if (c < A.dh) dqrow[c] = dqu[o][i] + dqv[o][i];
        }
}

template <typename T, int DP>
hipError_t launch_bwd_dp(const AttnBwdArgs &a, hipStream_t s) {
    const int nqb = (a.W + kQB - 1) / kQB;
    hipLaunchKernelGGL((rel_attn_bwd_kernel<T, DP>), dim3(a.B * a.H * nqb), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_t(const AttnBwdArgs &a, hipStream_t s) {
    switch (a.dp) {
        case 16: return launch_bwd_dp<T, 16>(a, s);
        case 32: return launch_bwd_dp<T, 32>(a, s);
        case 48: return launch_bwd_dp<T, 48>(a, s);
        case 64: return launch_bwd_dp<T, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attn_bwd_rt_off(int m) { return ATTN_RPAD + ((-m) & 7); }
int attn_bwd_rt_ld(int Kp) { return Kp + 2 * ATTN_RPAD + 16; }

hipError_t launch_rel_attn_bwd(bool is_bf16, const AttnBwdArgs &a, hipStream_t s) {
    return is_bf16 ? launch_bwd_t<bf16>(a, s) : launch_bwd_t<float>(a, s);
}

}  // namespace txl
