// txl_attn.hip -- fused relative-position attention over [mem; segment].
//
// Per (batch b, head h) the kernel computes, for queries i < W and keys j < K,
//   s_ij = (q_i + u).k_j + (q_i + v).r_{m+i-j}     (visible iff j <= m + i)
//   o_i  = sum_j softmax_j(s_ij) val_j
// ("Transformer-XL, explained.", method steps 3-5 and the score legend). The
// projected operands arrive head-major; (q + u) and (q + v) are pre-scaled by
// log2(e)/sqrt(dh) so the softmax runs on exp2.
//
// Work split. A workgroup of NW waves (four, or three when that does not add
// query blocks, e.g. 150 queries: two blocks of 96 rather than of 128; or two
// when that takes fewer rounds of the chip) owns 32 NW consecutive queries of
// one (b, h); each wave owns 32 of them and walks the visible keys in blocks of
// 64.
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
// e_rel, the distance's offset in the band (four accumulator registers per
// aligned 16-byte store); the value for key b of query a sits at position
// a - b + 63, which a lane reads with a per-lane base and a compile-time offset
// per register. Those values seed the accumulators of the content-term MFMAs,
// so the two terms add for free.
//
// The row pitch of that buffer (100 floats) keeps both the 16-byte writes and
// the 4-byte skewed reads on distinct banks. K and V^T tiles are staged in LDS
// with row padding chosen for their 16- and 8-byte fragment reads. The row sum
// of the probabilities is taken with packed bf16 dot products over the very
// values the P.V product consumes.
//
// Softmax uses a lazy maximum: the scores are taken relative to a running base
// m_run (subtracted as the band values are read, so the exponentials need no
// subtraction of their own); the base only moves (and the output accumulators
// are only rescaled) when a block's maximum exceeds it by more than 8 in log2
// units (which keeps every exp2 below 2^8); it starts at the first block's
// maximum.
//
// Key split. When the query blocks alone give too few workgroups to fill the
// chip (a short segment over a long memory), each query block is run by
// nsplit workgroups over disjoint ranges of its key blocks. Each writes its
// unnormalised output with its running base and sum; a second kernel rescales
// the parts to their common maximum and divides by the total sum (the online
// softmax's own merge rule, applied once across the parts).
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "txl_attn_tile.hpp"
#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

constexpr int kKB = 64;           // keys per block
constexpr int kMaxSplit = 8;      // most key parts per query block

template <typename T, int DP, bool DIST, int NW>
struct AttnSmem {
    static constexpr int NO = (DP + 31) / 32;                  // 32-row blocks of O^T
    // bf16: key and value rows of 128 bytes whose 16-byte chunks are
    // XOR-swizzled by the row (chunk q of row r at position q ^ (r % 8)), so the
    // 16-byte fragment reads of 8 consecutive rows hit 8 distinct bank groups.
    // fp32: padded rows, 16 bytes past the data.
    static constexpr bool SWZ = sizeof(T) == 2;
    static constexpr int kPitchK = SWZ ? 128 : DP * (int)sizeof(T) + 16;   // bytes per key row
    static constexpr int kPitchV = SWZ ? 128 : kKB * (int)sizeof(T) + 16;  // bytes per value row (V^T)
    // V^T rows past DP: stored as zero rows (fp32) or not stored, their
    // fragments then taken as zero (bf16)
    static constexpr int kRowsV = SWZ ? DP : NO * 32;
    float g[DIST ? NW : 1][DIST ? 32 * kGPitch : 4];
    alignas(16) char k[kKB * kPitchK];
    alignas(16) char v[kRowsV * kPitchV];
};

// bf16 key tiles hold their rows permuted inside each group of 16: row r
// holds key perm_key(r) of the block. Score register i of half hf in 32-key
// block sb (C row 32 sb + crow(i, hf)) then holds key reg_key(sb, i, hf), and
// the eight keys of each P.V fragment (registers 8 p' .. 8 p' + 7 of one half)
// are consecutive, so the matching V^T fragment is one 16-byte read.
__device__ __forceinline__ int perm_key(int r) {
    return (r & ~15) | (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 3);
}
__device__ __forceinline__ constexpr int reg_key_perm(int sb, int i, int hf) {
    return 32 * sb + 16 * (i >> 3) + 8 * hf + (i & 7);
}

// Row sum of eight probabilities already packed as the bf16 B operand.
__device__ __forceinline__ float psum(const Frag<bf16> &f, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f.v[2 * q], f.v[2 * q + 1]}, one, acc, false);
    return acc;
}
__device__ __forceinline__ float psum(const Frag<float> &f, float acc) {
    return acc + ((f.lo[0] + f.lo[1]) + (f.lo[2] + f.lo[3])) + ((f.hi[0] + f.hi[1]) + (f.hi[2] + f.hi[3]));
}

// As many workgroups per CU as its 160 KB of LDS holds, up to two waves per
// SIMD in bf16 (two waves hide each other's latency; a third would leave too
// few registers): two four- or three-wave workgroups, up to four two-wave ones.
// fp32 operands double the fragment registers, so fp32 runs one wave per SIMD
// with the full register file: one four-wave workgroup per CU, or two
// two-wave ones.
template <typename T, int DP, bool DIST, int NW>
constexpr int attn_wgs_per_cu() {
    const int by_lds = (int)((160 * 1024) / sizeof(AttnSmem<T, DP, DIST, NW>));
    const int by_regs = (sizeof(T) == 2 ? 8 : 4) / NW;   // two waves per SIMD (bf16), one (fp32)
    return by_lds < 1 ? 1 : by_lds < by_regs ? by_lds : by_regs;
}
// the same as waves per SIMD, the unit of the launch bound
template <typename T, int DP, bool DIST, int NW>
constexpr int attn_waves_per_simd() { return (attn_wgs_per_cu<T, DP, DIST, NW>() * NW + 3) / 4; }

// MODE 0: the full score; 1: also writes the log-sum-exp of every query (for
// a correction applied afterwards); 2: no distance term (content attention).
template <typename T, int DP, int MODE, int NW>
__global__ void __launch_bounds__(64 * NW, (attn_waves_per_simd<T, DP, MODE != 2, NW>())) rel_attn_kernel(const AttnArgs A) {
    constexpr bool DIST = MODE != 2;
    constexpr int NT = 64 * NW;                        // threads
    constexpr int kQB = 32 * NW;                       // queries per workgroup
    typedef AttnSmem<T, DP, DIST, NW> SM;
    constexpr int NS = DP / 16;
    constexpr int NO = SM::NO;
    __shared__ SM sm;

    const int BH = A.B * A.H;
    const int nqb = (A.W + kQB - 1) / kQB;
    const int ns = A.nsplit;
    const int rank = blockIdx.x / (BH * ns);
    const int rem = blockIdx.x - rank * (BH * ns);
    const int split = rem / BH;
    const int bh = rem - split * BH;
    // the first half of the ranks takes the query blocks longest first, the
    // second half shortest first: workgroup g and g + (grid / 2), which the
    // dispatcher tends to place on the same CU, then carry complementary key
    // ranges (the first and last query blocks, the second and second-to-last)
    const int hq = (nqb + 1) / 2;
    const int qblk = rank < hq ? nqb - 1 - rank : rank - hq;
    const int b = bh / A.H, h = bh - b * A.H;
    const int i0 = qblk * kQB;

    // the wave index is uniform across the wave: held in a scalar register, so
    // the per-wave conditions below are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 31, hf = lane >> 5;
    const int m = A.m;
    const int iw = i0 + 32 * w;                      // first query of this wave
    const bool wave_has_queries = iw < A.W;
    const int jend = min(A.K, m + i0 + kQB);         // keys any query here can see
    const int nkb_all = (jend + kKB - 1) / kKB;
    // this workgroup's key blocks [kb_lo, nkb)
    const int kb_lo = (int)((long long)split * nkb_all / ns);
    const int nkb = (int)((long long)(split + 1) * nkb_all / ns);
    const int last_key_wave = m + iw + 31;           // last key any query of the wave sees

    const T *qu = (const T *)A.qu + ((long long)bh * A.Wp) * DP;
    const T *qv = (const T *)A.qv + ((long long)bh * A.Wp) * DP;
    const T *ke = (const T *)A.ke + ((long long)bh * A.C) * DP;
    const T *vt = (const T *)A.vt + ((long long)bh * DP) * A.C;
    // this head's distance-key table (rk_elem layout): ATTN_RPAD zero rows on
    // either side of distances 0 .. K-1, in 32-row blocks starting at rows
    // congruent to roff = (m + 1) mod 32, the residue of every distance window
    // loaded below, so that each fragment load is one contiguous 1 KB
    const T *rtab = (const T *)A.rk + (long long)h * A.rk_hstride;
    const int roff = rk_frag_off(m);
    // lowest window start congruent to m + 1 at or above distance -94
    const int dlow = -94 + ((roff - (ATTN_RPAD - 94)) & 31);

    // zero the V^T rows past DP once (they pad the last 32-row block of O^T)
    for (int idx = tid; idx < (SM::kRowsV - DP) * (SM::kPitchV / 4); idx += NT)
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

    // r fragments of 32 distances d0 + fr (d0 congruent to m + 1 mod 32): the
    // block of table row d0 + ATTN_RPAD, column group 2s + hf, row fr.
    // Every distance a wave touches lies in [-ATTN_RPAD, Kp + ATTN_RPAD).
    auto r_frag = [&](Frag<T> &f, int d0, int s) {
        const long long blk = (d0 + ATTN_RPAD - roff) / 32 + 1;
        load8(f, rtab + blk * 32 * DP + (2 * s + hf) * 256 + fr * 8);
    };
    // r fragments of one 64-distance chunk: distances d0 + 32*bb + fr.
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

    // cooperative K / V^T staging; key j lives in slot (khead + j) mod C, and a
    // 16-byte V^T chunk (8 bf16 or 4 fp32 keys) never straddles the wrap
    // because khead and C are multiples of 8
    auto key_slot = [&](int j) { const int s = A.khead + j; return s >= A.C ? s - A.C : s; };
    constexpr int KCH = kKB * DP * (int)sizeof(T) / 16;    // 16-byte chunks per K tile
    constexpr int VCH = DP * kKB * (int)sizeof(T) / 16;    // ... per V^T tile
    constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT;
    constexpr int KCPR = DP * (int)sizeof(T) / 16;         // chunks per key row
    constexpr int VCPR = kKB * (int)sizeof(T) / 16;        // chunks per V^T row
    constexpr bool SWZ = SM::SWZ;
    u32x4 rkt[KPT], rvt[VPT];
#define TXL_KV_GLOAD(kb_)                                                                          \
    do {                                                                                           \
        const int j0_ = (kb_) * kKB;                                                               \
        _Pragma("unroll") for (int c = 0; c < KPT; ++c) {                                          \
            const int idx = tid + NT * c;                                                          \
            if (KCH % NT == 0 || idx < KCH) {                                                      \
                const int r_ = idx / KCPR, q_ = idx - r_ * KCPR;                                   \
                const int s_ = key_slot(j0_ + (SWZ ? perm_key(r_) : r_));                          \
                rkt[c] = *reinterpret_cast<const u32x4 *>((const char *)(ke + (long long)s_ * DP) + q_ * 16); \
            }                                                                                      \
        }                                                                                          \
        _Pragma("unroll") for (int c = 0; c < VPT; ++c) {                                          \
            const int idx = tid + NT * c;                                                          \
            if (VCH % NT == 0 || idx < VCH) {                                                      \
                const int r_ = idx / VCPR, q_ = idx - r_ * VCPR;                                   \
                const int s_ = key_slot(j0_ + q_ * (16 / (int)sizeof(T)));                         \
                rvt[c] = *reinterpret_cast<const u32x4 *>(vt + (long long)r_ * A.C + s_);           \
            }                                                                                      \
        }                                                                                          \
    } while (0)
#define TXL_KV_SSTORE()                                                                            \
    do {                                                                                           \
        _Pragma("unroll") for (int c = 0; c < KPT; ++c) {                                          \
            const int idx = tid + NT * c;                                                          \
            if (KCH % NT == 0 || idx < KCH) {                                                      \
                const int r_ = idx / KCPR, q_ = idx - r_ * KCPR;                                   \
                *reinterpret_cast<u32x4 *>(sm.k + r_ * SM::kPitchK + ((SWZ ? q_ ^ (r_ & 7) : q_) << 4)) = rkt[c]; \
            }                                                                                      \
        }                                                                                          \
        _Pragma("unroll") for (int c = 0; c < VPT; ++c) {                                          \
            const int idx = tid + NT * c;                                                          \
            if (VCH % NT == 0 || idx < VCH) {                                                      \
                const int r_ = idx / VCPR, q_ = idx - r_ * VCPR;                                   \
                *reinterpret_cast<u32x4 *>(sm.v + r_ * SM::kPitchV + ((SWZ ? q_ ^ (r_ & 7) : q_) << 4)) = rvt[c]; \
            }                                                                                      \
        }                                                                                          \
    } while (0)
    // the first K / V tile is requested before the distance prologue, whose
    // loads and products then cover its latency
    if (kb_lo < nkb) TXL_KV_GLOAD(kb_lo);

    float *grow = sm.g[DIST ? w : 0] + (DIST ? fr * kGPitch : 0);
    f32x16 oacc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) oacc[o] = zero16();
    // running maximum (the base the scores are taken relative to) and sum;
    // `started` turns true at the first block in which the query sees a key.
    // It follows the block maximum mx, which both lanes of a query share, so
    // the two halves of the wave always re-base together (l_run is only this
    // half's partial sum and may stay zero while the other half's is not).
    float m_run = 0.f, l_run = 0.f;
    bool started = false;

    // Band of key block kb: distances cw-63 .. cw+31 with cw = m + iw - 64*kb.
    // gb[kb & 1] holds the chunk cw-63 .. cw (two 32-distance blocks); the band's
    // top part cw+1 .. cw+31 is block 0 of the previous chunk, gb[(kb+1) & 1][0],
    // or for kb = 0 the block gtop computed here (written to LDS before the
    // loop). rnext holds r of the next chunk.
    // The two chunk buffers alternate with the parity of kb (the loop is unrolled
    // by two), so no register tile is copied from one step to the next.
    f32x16 gtop = zero16(), gb[2][2];
    Frag<T> rnext[2][NS];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s = 0; s < NS; ++s) rnext[bb][s] = Frag<T>{};
    if (DIST && wave_has_queries && kb_lo < nkb && kb_lo * kKB <= last_key_wave) {
        const int c0 = m + iw - kb_lo * kKB;         // >= -31: block kb_lo is visible
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            Frag<T> f;
            r_frag(f, c0 + 1, s);
            mma16(gtop, f, fqv[s]);
        }
        r_chunk(rnext, c0 - 63);
        g_chunk(gb[0], rnext);
        // the next chunk only while its block is visible (keeps the reads >= -94)
        if ((kb_lo + 1) * kKB <= last_key_wave) r_chunk(rnext, c0 - 127);
        // the band of block 0; every later band is written at the end of the
        // block before it, where it overlaps that block's P.V products
        write_gblock(grow, gb[0][0], 0, hf);
        write_gblock(grow, gb[0][1], 32, hf);
        write_gblock(grow, gtop, 64, hf);
    }


    // One key block; P is the parity of kb (compile time), so gb[P] / gb[Q] are
    // fixed register tiles.
    auto step = [&](auto parity, int kb) {
        constexpr int P = decltype(parity)::value, Q = 1 - P;
        __syncthreads();
        TXL_KV_SSTORE();
        __syncthreads();
        if (kb + 1 < nkb) TXL_KV_GLOAD(kb + 1);
        const int j0 = kb * kKB;
        if (!wave_has_queries || j0 > last_key_wave) return;

        // ---- shift the distance term into place through LDS
        f32x16 sacc[2];
        if constexpr (!DIST) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[0][i] = sacc[1][i] = -m_run;
        } else {
        wave_lds_sync();
        // key b of query a needs band offset a - b + 63 (b = 32 sb + crow(i) for
        // fp32 tiles, reg_key_perm(sb, i, hf) for the permuted bf16 ones)
        {
            if constexpr (SWZ) {
                const float *rb = grow + fr - 8 * hf + 63;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[sb][i] = rb[-(32 * sb + 16 * (i >> 3) + (i & 7))] - m_run;
            } else {
                const float *rb = grow + fr - 4 * hf;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[sb][i] = rb[63 - 32 * sb - 8 * (i >> 2) - (i & 3)] - m_run;
            }
        }
        }
        // ---- content term on top: S^T += K (q+u)^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Frag<T> f;
                if constexpr (SWZ)
                    f.v = *reinterpret_cast<const bf16x8 *>(__builtin_assume_aligned(
                        sm.k + (32 * sb + fr) * SM::kPitchK + (((2 * s + hf) ^ (fr & 7)) << 4), 16));
                else
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
                    if ((SWZ ? reg_key_perm(sb, i, hf) : 32 * sb + crow(i, lane)) > lim) sacc[sb][i] = -INFINITY;
        }
        // ---- online softmax (log2 domain; the scores are held relative to m_run)
        float mx = sacc[0][0];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[sb][i]);
        mx = half_max(mx);
        // lazy re-base: to the first block's maximum, then whenever a block
        // maximum exceeds the base by more than 8
        const bool first = !started && mx > -INFINITY;
        const bool rebase = mx > 8.f || first;
        started = started || mx > -INFINITY;
        if (__any(rebase)) {
            const float shift = rebase ? mx : 0.f;
            // before its first visible key a query's output and sum are exactly
            // zero and stay so: the first re-base scales nothing (its shift, the
            // first maximum, may be far below zero, where exp2(-shift) overflows)
            const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-shift);
#pragma unroll
            for (int o = 0; o < NO; ++o)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[o][i] *= alpha;
            l_run *= alpha;
            m_run += shift;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[sb][i] -= shift;
        }
        // ---- next distance chunk (MFMA) interleaved with exp / pack / row sum (VALU)
        if constexpr (DIST) {
            g_chunk(gb[Q], rnext);
            // prefetch for block kb+2; once that block is past the wave's keys the
            // window is clamped into the zero padding (to dlow >= -94, keeping its
            // residue mod 32). Unconditional,
            // so that the chunk's MFMAs share one basic block with the
            // exponentials below and the scheduler can interleave them.
            r_chunk(rnext, max(m + iw - j0 - kKB - 127, dlow));
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[sb][i] = __builtin_amdgcn_exp2f(sacc[sb][i]);
        // ---- band of block kb+1: its chunk (computed above) and, on top, the
        // low half of this block's chunk. This block's band reads are complete
        // (the content-term MFMAs consumed them); written here, the stores
        // drain while the P.V products run.
        if constexpr (DIST) {
            write_gblock(grow, gb[Q][0], 0, hf);
            write_gblock(grow, gb[Q][1], 32, hf);
            write_gblock(grow, gb[P][0], 64, hf);
        }
        Frag<T> fp4[4];
        float lsum[2] = {0.f, 0.f};          // two independent chains
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            p_frag(fp4[p], sacc[p >> 1], 8 * (p & 1));
            lsum[p & 1] = psum(fp4[p], lsum[p & 1]);   // sums exactly the values P.V uses
        }
        l_run += lsum[0] + lsum[1];
        // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                Frag<T> fv;
                if constexpr (SWZ) {    // keys 16 p + 8 hf .. + 7: one swizzled chunk
                    // rows past DP are not stored: read a stored row, use zeros
                    const int vr = 32 * o + fr;
                    const bool in = DP % 32 == 0 || o + 1 < NO || vr < DP;
                    const int rr = in ? vr : DP - 1;
                    fv.v = *reinterpret_cast<const bf16x8 *>(__builtin_assume_aligned(
                        sm.v + rr * SM::kPitchV + (((2 * p + hf) ^ (rr & 7)) << 4), 16));
                    if (!in) fv.v = bf16x8{};
                } else
                    load_vt(fv, sm.v + (32 * o + fr) * SM::kPitchV, 16 * p + 4 * hf);
                mma16(oacc[o], fv, fp4[p]);
            }
        }
    };

    for (int kb = kb_lo; kb < nkb; kb += 2) {
        step(std::integral_constant<int, 0>(), kb);
        if (kb + 1 < nkb) step(std::integral_constant<int, 1>(), kb + 1);
    }
#undef TXL_KV_GLOAD
#undef TXL_KV_SSTORE

    if (!wave_has_queries) return;
    const float l_tot = half_sum(l_run);
    const int qi = iw + fr;
    if (qi >= A.W) return;
    if (ns > 1) {
        // one part of a split query block: unnormalised output, base and sum
        // (a zero sum marks a part in which this query sees no key)
        const long long row = ((long long)split * BH + bh) * A.Wp + qi;
        float *po = A.part_o + row * DP;
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * o + crow(4 * q, lane);
                if (d < DP)
                    *reinterpret_cast<f32x4 *>(po + d) =
                        f32x4{oacc[o][4 * q], oacc[o][4 * q + 1], oacc[o][4 * q + 2], oacc[o][4 * q + 3]};
            }
        if (hf == 0)
            *reinterpret_cast<float2 *>(A.part_ml + 2 * row) = float2{l_tot > 0.f ? m_run : -INFINITY, l_tot};
        return;
    }
    const float inv = 1.f / l_tot;
    // log2 of the softmax denominator in the pre-scaled score units
    if (MODE == 1 && hf == 0) A.lse[(long long)bh * A.Wp + qi] = m_run + log2f(l_tot);
    T *orow = (T *)A.o + (long long)b * A.o_bstride + (long long)qi * A.o_ld + h * A.dh;
    // each group of four registers holds four consecutive columns: one store
    // per group when the row offsets keep those stores aligned
    const bool vec4 = A.dh % 4 == 0 && A.o_ld % 4 == 0 && A.o_bstride % 4 == 0 &&
                      ((uintptr_t)A.o % (4 * sizeof(T))) == 0;
    if (vec4) {
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * o + crow(4 * q, lane);
                if (d < A.dh) {
                    const float x0 = oacc[o][4 * q] * inv, x1 = oacc[o][4 * q + 1] * inv;
                    const float x2 = oacc[o][4 * q + 2] * inv, x3 = oacc[o][4 * q + 3] * inv;
                    if constexpr (sizeof(T) == 2)
                        *reinterpret_cast<bf16x4 *>(orow + d) = bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
                    else
                        *reinterpret_cast<f32x4 *>(orow + d) = f32x4{x0, x1, x2, x3};
                }
            }
    } else {
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d = 32 * o + crow(i, lane);
                if (d < A.dh) orow[d] = from_f32<T>(oacc[o][i] * inv);
            }
    }
}

// Merge of the key-split parts: one thread per (batch-head, query, group of 8
// output columns). With bases m_s and sums l_s, the output is
// sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s for M = max_s m_s, and the
// log-sum-exp (log2 units) M + log2 of the denominator.
template <typename T, int DP>
__global__ void __launch_bounds__(256) attn_merge_kernel(const AttnArgs A) {
    constexpr int G = DP / 8;
    const int BH = A.B * A.H;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)BH * A.W * G) return;
    const int g = (int)(idx % G);
    const long long r = idx / G;
    const int qi = (int)(r % A.W);
    const int bh = (int)(r / A.W);
    const long long stride = (long long)BH * A.Wp;          // rows per part
    const long long row0 = (long long)bh * A.Wp + qi;
    // every part's (base, sum) and output columns in one round of loads
    float2 ml[kMaxSplit];
    f32x4 lo[kMaxSplit], hi[kMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) {
        if (sp < A.nsplit) {
            const long long row = row0 + sp * stride;
            ml[sp] = *reinterpret_cast<const float2 *>(A.part_ml + 2 * row);
            lo[sp] = *reinterpret_cast<const f32x4 *>(A.part_o + row * DP + 8 * g);
            hi[sp] = *reinterpret_cast<const f32x4 *>(A.part_o + row * DP + 8 * g + 4);
        } else {
            ml[sp] = float2{-INFINITY, 0.f};
            lo[sp] = hi[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) M = fmaxf(M, ml[sp].x);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) {
        // a part with a zero sum (no visible key) has base -inf and weight 0
        const float wgt = ml[sp].y > 0.f ? __builtin_amdgcn_exp2f(ml[sp].x - M) : 0.f;
        L += wgt * ml[sp].y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i] += wgt * lo[sp][i];
            acc[4 + i] += wgt * hi[sp][i];
        }
    }
    const float inv = 1.f / L;
    const int b = bh / A.H, h = bh - b * A.H;
    T *orow = (T *)A.o + (long long)b * A.o_bstride + (long long)qi * A.o_ld + h * A.dh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int d = 8 * g + i;
        if (d < A.dh) orow[d] = from_f32<T>(acc[i] * inv);
    }
    if (A.lse && g == 0) A.lse[row0] = M + log2f(L);
}

// start/stop (may be null) are stamped by the kernels' own dispatches, so they
// bracket exactly this launch (attention, and the merge of a key split) on its
// stream.
// Three waves (96 queries) per bf16 workgroup when that takes no more query
// blocks than four would: fewer idle waves in the last block and the active
// queries spread more evenly over the blocks (150 queries: 96 + 54 instead of
// 128 + 22). The number of query blocks, and so the key split, is the same
// either way.
int attn_waves(bool is_bf16, int W) { return is_bf16 && (W + 95) / 96 <= (W + 127) / 128 ? 3 : 4; }

// Compute units of the current device (queried once per device).
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Two-wave workgroups (64 queries) when they take fewer rounds of the chip
// than the three- or four-wave choice above. The 16-layer workload's 320 (b, h)
// of 150 queries: in bf16 640 three-wave blocks on 512 slots, or 960 two-wave
// blocks on 1024 (one round); in fp32 640 four-wave blocks on 256 slots, or
// 960 two-wave blocks on 512 (two rounds instead of three).
template <typename T, int DP>
int pick_waves(const AttnArgs &a) {
    const int nw = attn_waves(sizeof(T) == 2, a.W);
    const long long bh = (long long)a.B * a.H * a.nsplit;
    const long long cus = device_cus();
    auto rounds = [&](int w, int per_cu) {
        const long long wgs = bh * ((a.W + 32 * w - 1) / (32 * w));
        return (wgs + per_cu * cus - 1) / (per_cu * cus);
    };
    const int per_nw = a.dist ? (nw == 3 ? attn_wgs_per_cu<T, DP, true, 3>() : attn_wgs_per_cu<T, DP, true, 4>())
                              : (nw == 3 ? attn_wgs_per_cu<T, DP, false, 3>() : attn_wgs_per_cu<T, DP, false, 4>());
    const int per_2 = a.dist ? attn_wgs_per_cu<T, DP, true, 2>() : attn_wgs_per_cu<T, DP, false, 2>();
    return rounds(2, per_2) < rounds(nw, per_nw) ? 2 : nw;
}

template <typename T, int DP, int NW>
void launch_modes(const AttnArgs &a, dim3 grid, hipStream_t s, hipEvent_t start, hipEvent_t stop1) {
    dim3 block(64 * NW);
    if (!a.dist)
        hipExtLaunchKernelGGL((rel_attn_kernel<T, DP, 2, NW>), grid, block, 0, s, start, stop1, 0, a);
    else if (a.lse)
        hipExtLaunchKernelGGL((rel_attn_kernel<T, DP, 1, NW>), grid, block, 0, s, start, stop1, 0, a);
    else
        hipExtLaunchKernelGGL((rel_attn_kernel<T, DP, 0, NW>), grid, block, 0, s, start, stop1, 0, a);
}

template <typename T, int DP>
hipError_t launch_dp(const AttnArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const int nw = pick_waves<T, DP>(a);
    const int nqb = (a.W + 32 * nw - 1) / (32 * nw);
    dim3 grid(a.B * a.H * nqb * a.nsplit), block(256);
    const bool merge = a.nsplit > 1;
    hipEvent_t stop1 = merge ? nullptr : stop;
    if constexpr (sizeof(T) == 2) {
        if (nw == 2) launch_modes<T, DP, 2>(a, grid, s, start, stop1);
        else if (nw == 3) launch_modes<T, DP, 3>(a, grid, s, start, stop1);
        else launch_modes<T, DP, 4>(a, grid, s, start, stop1);
    } else {
        if (nw == 2) launch_modes<T, DP, 2>(a, grid, s, start, stop1);
        else launch_modes<T, DP, 4>(a, grid, s, start, stop1);
    }
    if (merge) {
        const long long threads = (long long)a.B * a.H * a.W * (DP / 8);
        dim3 mgrid((unsigned)((threads + 255) / 256));
        hipExtLaunchKernelGGL((attn_merge_kernel<T, DP>), mgrid, block, 0, s, nullptr, stop, 0, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    switch (a.dp) {
        case 16: return launch_dp<T, 16>(a, s, start, stop);
        case 32: return launch_dp<T, 32>(a, s, start, stop);
        case 48: return launch_dp<T, 48>(a, s, start, stop);
        case 64: return launch_dp<T, 64>(a, s, start, stop);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attn_dp(int dh) { return (dh + 15) / 16 * 16; }

int attn_splits(int B, int H, int W, int K) {
    const long long wgs = (long long)B * H * ((W + 127) / 128);     // query blocks (of 128 or of 96)
    if (wgs >= 512) return 1;                     // two workgroups per CU already
    const int nkb = (K + kKB - 1) / kKB;          // key blocks of the last query block
    const int want = (int)((512 + wgs - 1) / wgs);
    return std::max(1, std::min(want, std::min(kMaxSplit, nkb / 4)));   // parts of >= 4 key blocks
}
bool rel_attn_supported(int dh) { return dh >= 1 && dh <= 64; }

hipError_t launch_rel_attn(bool is_bf16, const AttnArgs &args, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    AttnArgs a = args;
    if (a.nsplit < 1 || !a.part_o || !a.part_ml) a.nsplit = 1;
    if (a.o_ld <= 0) a.o_ld = a.D;
    return is_bf16 ? launch_t<bf16>(a, s, start, stop) : launch_t<float>(a, s, start, stop);
}

}  // namespace txl
