// txl_gemm.hip -- grouped GEMM on the gfx950 matrix cores.
//
// Computes C = A B^T for up to three independent problems per launch, where B
// is a weight stored out-major ([n][k], the layout every projection of the
// layer uses: y = x W^T). Both operands are therefore contiguous along the
// reduction axis and load straight into MFMA fragments without a transpose.
//
// Work split: a 256-thread workgroup computes a BM x 128 tile of C (BM = 128,
// or 64 when 128-row tiles would leave fewer than two workgroups per CU); each
// of its four waves owns a (BM/2) x 64 part as (BM/64) x 2 blocks of 32 x 32
// MFMA output. The reduction runs in k-tiles of 128 bytes per row (64 bf16 or 32
// fp32 values), double-buffered in LDS with 16 bytes of padding per row so
// that the fragment reads of 32 rows hit distinct banks. Global loads of the
// next k-tile are issued before the MFMAs of the current one.
//
// Tiles are numbered so that tiles sharing rows of A are consecutive, and the
// workgroup index is remapped so that consecutive tiles land on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs, each with its own L2).
#include <string.h>

#include <type_traits>

#include "txl_device.hpp"
#include "txl_internal.hpp"

namespace txl {

namespace {

constexpr int kBN = 128, kThreads = 256;
constexpr int kRowBytes = 128;                       // bytes per row of one k-tile
constexpr int kPitch = kRowBytes + 16;               // LDS bytes per row
constexpr int kPrefetch = 2;                         // k-tiles of global loads in flight

template <int BM>
struct GemmSmem {
    char a[2][BM * kPitch];
    char b[2][kBN * kPitch];
};
static_assert(sizeof(GemmSmem<128>) >= 128 * 132 * 4, "C tile staging must fit in the operand buffers");
static_assert(sizeof(GemmSmem<64>) >= 64 * 132 * 4, "C tile staging must fit in the operand buffers");

// Fast floor(x / d) for 0 <= x < 2^22 with a float reciprocal and one fix-up.
__device__ __forceinline__ int fdiv(int x, int d, float inv) {
    int q = (int)((float)x * inv);
    int r = x - q * d;
    if (r < 0) q -= 1;
    else if (r >= d) q += 1;
    return q;
}

template <typename T>
__device__ __forceinline__ const char *a_row_ptr(const GemmProblem &P, int row, float inv_seg) {
    if (row >= P.rows) return nullptr;
    int b = fdiv(row, P.seg_rows, inv_seg);
    int t = row - b * P.seg_rows;
    if (P.a_mode == A_CONTEXT) {
        if (t < P.mem_len) {
            int pr = P.ring_head + t;
            if (pr >= P.ring_M) pr -= P.ring_M;
            return (const char *)P.ring + ((long long)b * P.ring_bstride + (long long)pr * P.ring_ld) * (long long)sizeof(T);
        }
        t -= P.mem_len;
    }
    t -= P.a_first;
    if (t < 0 || t >= P.valid_rows) return nullptr;
    return (const char *)P.a + ((long long)b * P.a_bstride + (long long)t * P.a_ld) * (long long)sizeof(T);
}

template <typename T>
__device__ __forceinline__ const char *b_row_ptr(const GemmProblem &P, int n, int bidx) {
    if (n >= P.cols) return nullptr;
    const void *w = (const char *)P.b0 + (long long)bidx * P.b_bstride * (long long)sizeof(T);
    if (n >= P.b_split) { n -= P.b_split; w = P.b1; }
    int wrow = n;
    if (P.b_mode == B_HEADS) {
        int hh = n / P.dhp, c = n - hh * P.dhp;
        if (c >= P.dh) return nullptr;
        wrow = hh * P.dh + c;
    }
    return (const char *)w + (long long)wrow * P.b_ld * (long long)sizeof(T);
}

// Load one 16-byte chunk (elements [k, k + 16/sizeof(T))) of a row, zero past kdim.
// Without VEC the rows are only 4-byte aligned (d_model 410): a chunk wholly
// inside kdim is still one 16-byte load (dword alignment suffices for global
// memory), the tail chunk goes by dwords.
template <typename T, bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const char *row, int k, int kdim) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (!row) return z;
    if (VEC) {
        if (k < kdim) z = *reinterpret_cast<const u32x4 *>(row + (long long)k * sizeof(T));
    } else {
        constexpr int per = 4 / sizeof(T);   // elements per dword
        if (k + 4 * per <= kdim) {
            __builtin_memcpy(&z, __builtin_assume_aligned(row + (long long)k * sizeof(T), 4), 16);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int kk = k + q * per;
                if (kk < kdim) z[q] = *reinterpret_cast<const uint32_t *>(row + (long long)kk * sizeof(T));
            }
        }
    }
    return z;
}

constexpr int kCPitch = 132;   // floats per row of the staged C tile (16-byte aligned rows)

// Eight consecutive output elements as one store (16 bytes for bf16, 32 for fp32).
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { bf16x8 v; };
template <> struct Vec8<float> { f32x4 lo, hi; };

template <typename T, bool VEC>
__device__ __forceinline__ void store8(T *dst, const float (&x)[8]) {
    if (VEC) {
        if constexpr (sizeof(T) == 2) {
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
            *reinterpret_cast<bf16x8 *>(dst) = v;
        } else {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
        }
    } else {
        // dword-aligned destination: one wide store of the packed values
        if constexpr (sizeof(T) == 2) {
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
            __builtin_memcpy(__builtin_assume_aligned(dst, 4), &v, 16);
        } else {
            const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
            __builtin_memcpy(__builtin_assume_aligned(dst, 4), &lo, 16);
            __builtin_memcpy(__builtin_assume_aligned((T *)dst + 4, 4), &hi, 16);
        }
    }
}

template <typename T, bool VEC>
__device__ __forceinline__ void load8f(float (&x)[8], const T *src) {
    if (VEC && sizeof(T) == 2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(src);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(((const T *)&v)[i]);
    } else if constexpr (sizeof(T) == 2) {
        bf16x8 v;
        __builtin_memcpy(&v, __builtin_assume_aligned(src, 4), 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(((const T *)&v)[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(src[i]);
    }
}

// Write the BM x 128 C tile staged in LDS (cs). Row-major destinations: a
// thread owns eight consecutive columns and walks every 32nd row of the tile
// (rows advance incrementally, no division). The transposed value output: a
// wave covers 64 consecutive columns of one 8-row group, each lane writing
// eight consecutive rows of its column as one store.
// Key slot of segment row t for EPI_KV outputs.
__device__ __forceinline__ int kv_slot(const GemmProblem &P, int t) {
    const int s = P.kv_base + t;
    return s >= P.kv_slots ? s - P.kv_slots : s;
}

template <typename T, bool VEC, int BM, int BN = 128>
__device__ __forceinline__ void epilogue(const GemmProblem &P, const float *cs, int m0, int n0, int tid,
                                         float inv_seg) {
    const bool trans = P.epi == EPI_KV && n0 >= P.b_split;
    if (!trans) {
        const int cg = tid & 15;                       // column group: columns n0 + 8*cg .. +7
        const int n = n0 + 8 * cg;
        if (8 * cg >= BN || n >= P.cols) return;
        const bool full = n + 8 <= P.cols;
        float bias[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float uu[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float vv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int hh = 0, c = 0;
        bool second = false;
        if (P.epi == EPI_ROWS) {
            if (P.bias)
#pragma unroll
                for (int i = 0; i < 8; ++i) bias[i] = n + i < P.cols ? to_f32(((const T *)P.bias)[n + i]) : 0.f;
        } else {
            int nn = n;
            if (P.epi == EPI_KV && n >= P.b_split) { nn = n - P.b_split; second = true; }
            hh = nn / P.dhp;                           // the 8 columns share one head (dhp % 16 == 0)
            c = nn - hh * P.dhp;
            if (P.epi == EPI_QUV && P.u)      // u, v null: both biases zero
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (c + i < P.dh) {
                        uu[i] = to_f32(((const T *)P.u)[hh * P.dh + c + i]);
                        vv[i] = to_f32(((const T *)P.v)[hh * P.dh + c + i]);
                    }
        }
        int rl = tid >> 4;                              // 0..15, then +16 per iteration
        int row = m0 + rl;
        int b = fdiv(row, P.seg_rows, inv_seg);
        int t = row - b * P.seg_rows;
        for (; rl < BM; rl += 16) {
            if (row >= P.rows) break;
            float x[8];
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(cs + rl * kCPitch + 8 * cg);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(cs + rl * kCPitch + 8 * cg + 4);
            x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
            x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
            if (P.epi == EPI_ROWS) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] += bias[i];
                    if (P.relu) x[i] = fmaxf(x[i], 0.f);
                }
                const long long ridx = (long long)b * P.res_bstride + (long long)t * P.res_ld + n;
                const long long idx = (long long)b * P.c_bstride + (long long)t * P.c_ld + n;
                if (full) {
                    if (P.res) {
                        float r[8];
                        load8f<T, VEC>(r, (const T *)P.res + ridx);
#pragma unroll
                        for (int i = 0; i < 8; ++i) x[i] += r[i];
                    }
                    if (P.out_f32) store8<float, VEC>((float *)P.c0 + idx, x);
                    else store8<T, VEC>((T *)P.c0 + idx, x);
                } else {
                    for (int i = 0; i < 8 && n + i < P.cols; ++i) {
                        float y = x[i];
                        if (P.res) y += to_f32(((const T *)P.res)[ridx + i]);
                        if (P.out_f32) ((float *)P.c0)[idx + i] = y;
                        else ((T *)P.c0)[idx + i] = from_f32<T>(y);
                    }
                }
            } else {
                const long long bh = (long long)b * P.heads + hh;
                if (P.epi == EPI_QUV) {
                    const long long idx = (bh * P.seg_rows + t) * P.dhp + c;
                    float xu[8], xv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        xu[i] = (x[i] + uu[i]) * P.qscale;
                        xv[i] = (x[i] + vv[i]) * P.qscale;
                    }
                    store8<T, true>((T *)P.c0 + idx, xu);
                    store8<T, true>((T *)P.c1 + idx, xv);
                } else if (second) {
                    // a tile that straddles the K_E / V split writes its V columns here
                    const int slot = kv_slot(P, t);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        ((T *)P.c1)[(bh * P.dhp + c + i) * P.kv_slots + slot] = from_f32<T>(x[i]);
                } else if (P.epi == EPI_KV) {
                    store8<T, true>((T *)P.c0 + (bh * P.kv_slots + kv_slot(P, t)) * P.dhp + c, x);
                } else if (P.epi == EPI_GROWS) {
                    if (t < P.c_rows) {
                        const int bb = b / P.heads, gh = b - bb * P.heads;
                        float *dst = (float *)P.c0 + (long long)bb * P.c_bstride + (long long)t * P.c_ld + gh * P.dh + c;
                        if (c + 8 <= P.dh && ((uintptr_t)dst & 15) == 0) {
                            *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
                            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
                        } else {
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                if (c + i < P.dh) dst[i] = x[i];
                        }
                    }
                } else if (P.epi == EPI_RFRAG) {
                    // eight consecutive columns of a row stay contiguous (c % 8 == 0)
                    store8<T, true>((T *)P.c0 + hh * P.frag_hstride + rk_elem(t, c, P.frag_off, P.dhp), x);
                } else {
                    store8<T, true>((T *)P.c0 + (bh * P.seg_rows + t) * P.dhp + c, x);
                }
            }
            row += 16;
            t += 16;
            while (t >= P.seg_rows) { t -= P.seg_rows; ++b; }
        }
    } else {
        // V^T [b][hh][c][slot]: rows of the tile are consecutive t (seg_rows % 8 == 0)
        const int lane = tid & 63, wv = tid >> 6;
        for (int task = wv; task < BM / 4; task += 4) {  // task = (row group rg, column half ch)
            const int rg = task >> 1, ch = task & 1;
            if (64 * ch >= BN) continue;
            const int nl = 64 * ch + lane;
            const int n = n0 + nl;
            const int row = m0 + 8 * rg;
            if (n >= P.cols || row >= P.rows) continue;
            const int b = fdiv(row, P.seg_rows, inv_seg);
            const int t = row - b * P.seg_rows;
            const int nn = n - P.b_split;
            const int hh = nn / P.dhp, c = nn - hh * P.dhp;
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = cs[(8 * rg + i) * kCPitch + nl];
            // t, kv_base and kv_slots are multiples of 8: the eight slots are consecutive
            store8<T, true>((T *)P.c1 + (((long long)b * P.heads + hh) * P.dhp + c) * P.kv_slots + kv_slot(P, t), x);
        }
    }
}

template <typename T, bool VEC, int BM>
__global__ void __launch_bounds__(kThreads, 2) gemm_kernel(const GemmLaunch g) {
    constexpr int MI = BM / 64;                                     // 32-row blocks per wave
    constexpr int kChA = BM * (kRowBytes / 16) / kThreads;          // 16-byte chunks per thread, A
    constexpr int kChB = kBN * (kRowBytes / 16) / kThreads;         // ... B
    __shared__ GemmSmem<BM> sm;
    if ((int)blockIdx.x >= g.total_tiles) {                         // a copy workgroup
        extra_block(g, blockIdx.x - g.total_tiles);
        return;
    }
    // XCD-aware remap: deal consecutive tiles to the same XCD.
    const int tile = deal_tile(blockIdx.x, g.total_tiles, lead_tiles(g));
    // select the problem with uniform branches (a dynamic index into the
    // kernel-argument struct would copy it to private memory)
    GemmProblem P;
    if (g.count > 2 && tile >= g.p[2].tile_begin) P = g.p[2];
    else if (g.count > 1 && tile >= g.p[1].tile_begin) P = g.p[1];
    else P = g.p[0];
    const int lt = tile - P.tile_begin;
    const int tm = lt / P.tiles_n, tn = lt - tm * P.tiles_n;
    const int m0 = tm * BM, n0 = tn * kBN;
    const float inv_seg = 1.0f / (float)P.seg_rows;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
    constexpr int BK = kRowBytes / sizeof(T);    // elements per k-tile

    // Rows and chunk column this thread stages: rows tid/8 + 32c, chunk tid%8.
    const int ccol = tid & 7;
    const int bidx = P.b_bstride ? m0 / P.seg_rows : 0;    // batch entry of every row of this tile
    const char *arow[kChA], *brow[kChB];
#pragma unroll
    for (int c = 0; c < kChA; ++c) arow[c] = a_row_ptr<T>(P, m0 + (tid >> 3) + 32 * c, inv_seg);
#pragma unroll
    for (int c = 0; c < kChB; ++c) brow[c] = b_row_ptr<T>(P, n0 + (tid >> 3) + 32 * c, bidx);
    const int nk = (P.kdim + BK - 1) / BK;

    // Global loads run kPre k-tiles ahead of the MFMAs (a ring of register
    // sets): a k-tile's MFMAs take far less time than an L2 round trip.
    constexpr int kPre = kPrefetch;
    static_assert(kPre == 2 || kPre == 3, "the ring needs two or three register sets");
    u32x4 ra[kPre][kChA], rb[kPre][kChB];
#define TXL_GLOAD(set_, kt_)                                              \
    do {                                                                  \
        const int k_ = (kt_) * BK + ccol * EPC;                           \
        _Pragma("unroll") for (int c = 0; c < kChB; ++c) {                \
            if (c < kChA) ra[set_][c] = load_chunk<T, VEC>(arow[c], k_, P.kdim); \
            rb[set_][c] = load_chunk<T, VEC>(brow[c], k_, P.kdim);        \
        }                                                                 \
    } while (0)
#define TXL_SSTORE(set_, buf_)                                            \
    do {                                                                  \
        _Pragma("unroll") for (int c = 0; c < kChB; ++c) {                \
            const int r_ = (tid >> 3) + 32 * c;                           \
            if (c < kChA) *reinterpret_cast<u32x4 *>(&sm.a[buf_][r_ * kPitch + ccol * 16]) = ra[set_][c]; \
            *reinterpret_cast<u32x4 *>(&sm.b[buf_][r_ * kPitch + ccol * 16]) = rb[set_][c]; \
        }                                                                 \
    } while (0)

    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

    const int fr = lane & 31, fh = lane >> 5;
    auto mma_tile = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            Frag<T> fa[MI], fb[2];
            const int koff = (ks * 16 + fh * 8) * (int)sizeof(T);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                load8(fa[i], reinterpret_cast<const T *>(&sm.a[buf][(wm * (BM / 2) + i * 32 + fr) * kPitch + koff]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                load8(fb[j], reinterpret_cast<const T *>(&sm.b[buf][(wn * 64 + j * 32 + fr) * kPitch + koff]));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma16(acc[i][j], fb[j], fa[i]);   // C^T block: lane = row of C
        }
    };
    // k-tile kt lives in register set kt % kPre and LDS buffer kt & 1; the loop
    // is unrolled by kPre so every set index is a compile-time constant, and
    // each unrolled step issues the same loads in the same order
    auto step = [&](auto phase, int kt) {
        constexpr int S = decltype(phase)::value;
        constexpr int S1 = (S + 1) % kPre;
        mma_tile(kt & 1);
        if (kt + 1 < nk) TXL_SSTORE(S1, (kt + 1) & 1);
        if (kt + kPre < nk) TXL_GLOAD(S, kt + kPre);
        __syncthreads();
    };

    TXL_GLOAD(0, 0);
    if (1 < nk) TXL_GLOAD(1, 1);
    if constexpr (kPre > 2) {
        if (2 < nk) TXL_GLOAD(2, 2);
    }
    TXL_SSTORE(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += kPre) {
        step(std::integral_constant<int, 0>(), kt);
        if (kt + 1 < nk) step(std::integral_constant<int, 1>(), kt + 1);
        if constexpr (kPre > 2) {
            if (kt + 2 < nk) step(std::integral_constant<int, 2>(), kt + 2);
        }
    }

    // stage the C tile in LDS (the k-loop ended with a barrier), then write it out.
    // The blocks were computed transposed, so lane fr holds row fr of the block and
    // each group of four registers four consecutive columns: one 16-byte store each.
    float *cs = reinterpret_cast<float *>(&sm);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4 *>(&cs[(wm * (BM / 2) + i * 32 + fr) * kCPitch + wn * 64 + j * 32 + crow(4 * q, lane)]) =
                    f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __syncthreads();
    epilogue<T, VEC, BM>(P, cs, m0, n0, tid, inv_seg);
#undef TXL_GLOAD
#undef TXL_SSTORE
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for 16-byte aligned operands. k-tiles are 64 bytes
// per row (A rows, then B rows, four 16-byte chunks each) and travel from
// global memory to LDS with global_load_lds (no register round trip and no
// LDS store instructions): each wave instruction fills 1 KB of LDS, 16 rows,
// lane l at byte 16 l, so each lane fetches the global chunk that belongs at
// its position. Chunk c of row r sits at position c ^ ((r >> 2) & 3) of the
// row: the 16-byte fragment reads of 16 consecutive rows then hit 16 distinct
// bank groups. Three LDS buffers: the loads of k-tile kt+2 go into the buffer
// of k-tile kt-1, so one barrier per k-tile orders them after every wave's
// reads of that buffer.
// ---------------------------------------------------------------------------
constexpr int kLRow = 64;                                 // bytes per row of one k-tile

template <int BM, int BN>
struct GemmLdsSmem {
    char buf[3][(BM + BN) * kLRow];
};
static_assert(sizeof(GemmLdsSmem<64, 128>) >= 64 * 132 * 4, "C staging must fit in the operand buffers");
static_assert(sizeof(GemmLdsSmem<128, 64>) >= 64 * 132 * 4, "C staging must fit in the operand buffers");
static_assert(sizeof(GemmLdsSmem<128, 128>) >= 128 * 136 * 2, "bf16 staging must fit in the operand buffers");

// Source of lanes whose chunk lies past kdim or in a row without data.
__device__ __align__(16) unsigned int g_zero_chunk[4];

typedef __attribute__((address_space(3))) void *lds_ptr;

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4
// and lgkmcnt 11:8 left at their maxima): this wave's direct-to-LDS loads have
// written LDS.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// BN = 64 (problems of at most 64 columns): 36 KB of LDS, four workgroups per CU.
template <typename T, int BM, int BN>
__global__ void __launch_bounds__(kThreads, BN == 64 ? 4 : 3) gemm_lds_kernel(const GemmLaunch g) {
    constexpr int MI = BM / 64;                          // 32-row blocks per wave
    constexpr int NJ = BN / 64;                          // 32-column blocks per wave
    constexpr int ROWS = BM + BN;                        // rows per k-tile (A, then B)
    constexpr int NI = ROWS / 16 / 4;                    // load instructions per wave per k-tile
    constexpr int BK = kLRow / (int)sizeof(T);           // elements per row of a k-tile
    constexpr int EPC = 16 / (int)sizeof(T);             // elements per chunk
    static_assert(ROWS % 64 == 0, "whole load instructions per wave");
    __shared__ GemmLdsSmem<BM, BN> sm;
    if ((int)blockIdx.x >= g.total_tiles) {                         // a copy workgroup
        extra_block(g, blockIdx.x - g.total_tiles);
        return;
    }

    const int tile = deal_tile(blockIdx.x, g.total_tiles, lead_tiles(g));
    GemmProblem P;
    if (g.count > 2 && tile >= g.p[2].tile_begin) P = g.p[2];
    else if (g.count > 1 && tile >= g.p[1].tile_begin) P = g.p[1];
    else P = g.p[0];
    const int lt = tile - P.tile_begin;
    const int tm = lt / P.tiles_n, tn = lt - tm * P.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const float inv_seg = 1.0f / (float)P.seg_rows;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int bidx = P.b_bstride ? m0 / P.seg_rows : 0;

    // instruction j of this wave fills rows 16 (wave + 4 j) .. +16 of a k-tile;
    // this lane's row and the global chunk it fetches
    const char *src[NI];
    int cel[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int row = 16 * (wave + 4 * j) + (lane >> 2);
        cel[j] = ((lane & 3) ^ ((row >> 2) & 3)) * EPC;
        src[j] = row < BM ? a_row_ptr<T>(P, m0 + row, inv_seg) : b_row_ptr<T>(P, n0 + row - BM, bidx);
    }
    const int nk = (P.kdim + BK - 1) / BK;
    const char *zero = reinterpret_cast<const char *>(g_zero_chunk);
    // k-tiles whose chunk at element offset cel[j] is still inside kdim (kdim is a
    // multiple of the chunk width on this path)
    int kin[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        kin[j] = src[j] ? (P.kdim - cel[j] + BK - 1) / BK : 0;
        if (!src[j]) src[j] = zero;
    }
    auto issue = [&](int kt, int b) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const char *p = kt < kin[j] ? src[j] + ((long long)kt * BK + cel[j]) * (long long)sizeof(T) : zero;
            __builtin_amdgcn_global_load_lds(p, (lds_ptr)(sm.buf[b] + 1024 * (wave + 4 * j)), 16, 0, 0);
        }
    };

    const int fr = lane & 31, fh = lane >> 5;
    const int sw = (fr >> 2) & 3;                        // this lane's row swizzle
    auto frag = [&](Frag<T> &f, const char *bufp, int row, int e0) {
        // elements e0 .. e0+7 of a k-tile row (one chunk for bf16, two for fp32)
        const char *r = bufp + row * kLRow;
        if constexpr (sizeof(T) == 2) {
            f.v = *reinterpret_cast<const bf16x8 *>(r + (((e0 / EPC) ^ sw) << 4));
        } else {
            f.lo = *reinterpret_cast<const f32x4 *>(r + (((e0 / EPC) ^ sw) << 4));
            f.hi = *reinterpret_cast<const f32x4 *>(r + (((e0 / EPC + 1) ^ sw) << 4));
        }
    };

    // bf16 key / value tiles wholly on one side of the split write their output
    // through a bf16 staging tile in one round; the value tiles compute C blocks
    // (operands swapped: lane = column, registers = four consecutive rows) so
    // that the staging holds the transposed output row by row
    const bool kvtile = sizeof(T) == 2 && BM == 128 && BN == 128 && P.epi == EPI_KV &&
                        (n0 + BN <= P.b_split || n0 >= P.b_split);
    const bool vtile = kvtile && n0 >= P.b_split;

    auto run = [&](auto swap) {
        constexpr bool SWAP = decltype(swap)::value;
        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = zero16();
        auto mma_tile = [&](const char *bufp) {
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                Frag<T> fa[MI], fb[NJ];
                const int e0 = ks * 16 + fh * 8;
#pragma unroll
                for (int i = 0; i < MI; ++i) frag(fa[i], bufp, wm * (BM / 2) + i * 32 + fr, e0);
#pragma unroll
                for (int j = 0; j < NJ; ++j) frag(fb[j], bufp, BM + wn * (BN / 2) + j * 32 + fr, e0);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        if constexpr (SWAP) mma16(acc[i][j], fa[i], fb[j]);   // C block: lane = column of C
                        else mma16(acc[i][j], fb[j], fa[i]);                  // C^T block: lane = row of C
                    }
            }
        };

        // Each wave completes all of its loads in flight before the barrier of a
        // k-tile (the compiler cannot tell the three buffers apart and would wait
        // for them before the fragment reads anyway): k-tile kt+2 is requested
        // right after the barrier of k-tile kt and complete at the barrier of
        // k-tile kt+1, one k-tile of products later.
        // a causal band of zeros in A: this tile's rows are zero before k-tile kt0
        int kt0 = 0;
        if (P.kz_on) kt0 = min(max(0, m0 - bidx * P.seg_rows - P.kz_lag) / BK, nk - 1);   // >= 1 k-tile runs
        issue(kt0, 0);
        if (kt0 + 1 < nk) issue(kt0 + 1, 1);
        int b = 0;                                           // buffer of k-tile kt
        for (int kt = kt0; kt < nk; ++kt) {
            // every wave's chunks of k-tile kt are in LDS, and every wave is done
            // reading the buffer of k-tile kt-1, which k-tile kt+2 now fills
            wait_loads();
            __syncthreads();
            if (kt + 2 < nk) issue(kt + 2, b == 0 ? 2 : b - 1);
            mma_tile(sm.buf[b]);
            b = b == 2 ? 0 : b + 1;
        }
        __syncthreads();                                     // all reads done before C staging

        if (SWAP || kvtile) {
            // bf16 staging, 136 elements (272 bytes) per row: rows of the tile for
            // key tiles, columns of the tile for value tiles
            constexpr int SP = 136;
            bf16 *st = reinterpret_cast<bf16 *>(&sm);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16x4 v4 = {(bf16)acc[i][j][4 * q], (bf16)acc[i][j][4 * q + 1],
                                           (bf16)acc[i][j][4 * q + 2], (bf16)acc[i][j][4 * q + 3]};
                        // C^T: lane row wm*64 + 32i + fr, columns wn*64 + 32j + crow(4q);
                        // C: lane column wn*64 + 32j + fr, rows wm*64 + 32i + crow(4q)
                        const int lr = SWAP ? wn * (BN / 2) + 32 * j + fr : wm * (BM / 2) + 32 * i + fr;
                        const int lc = SWAP ? wm * (BM / 2) + 32 * i + crow(4 * q, lane)
                                            : wn * (BN / 2) + 32 * j + crow(4 * q, lane);
                        *reinterpret_cast<bf16x4 *>(__builtin_assume_aligned(st + lr * SP + lc, 8)) = v4;
                    }
            __syncthreads();
            // 16-byte chunks: 128 staging rows x 16 chunks of 8 elements
#pragma unroll 2
            for (int ch = tid; ch < 128 * 16; ch += kThreads) {
                const int sr = ch >> 4, cc = ch & 15;
                const bf16x8 v8 = *reinterpret_cast<const bf16x8 *>(
                    __builtin_assume_aligned(st + sr * SP + 8 * cc, 16));
                if constexpr (SWAP) {
                    // staging row = value column n, chunk = 8 consecutive rows (key slots)
                    const int n = n0 + sr, row = m0 + 8 * cc;
                    if (n < P.cols && row < P.rows) {
                        const int bb = fdiv(row, P.seg_rows, inv_seg);
                        const int t = row - bb * P.seg_rows;
                        const int nn = n - P.b_split;
                        const int hh = nn / P.dhp, c = nn - hh * P.dhp;
                        *reinterpret_cast<bf16x8 *>((bf16 *)P.c1 + (((long long)bb * P.heads + hh) * P.dhp + c) *
                                                                       P.kv_slots + kv_slot(P, t)) = v8;
                    }
                } else {
                    // staging row = tile row, chunk = 8 consecutive key columns of one head
                    const int row = m0 + sr, n = n0 + 8 * cc;
                    if (n < P.cols && row < P.rows) {
                        const int bb = fdiv(row, P.seg_rows, inv_seg);
                        const int t = row - bb * P.seg_rows;
                        const int hh = n / P.dhp, c = n - hh * P.dhp;
                        *reinterpret_cast<bf16x8 *>((bf16 *)P.c0 + (((long long)bb * P.heads + hh) * P.kv_slots +
                                                                    kv_slot(P, t)) * P.dhp + c) = v8;
                    }
                }
            }
            return;
        }

        // C staged 64 rows at a time (the waves whose rows fall in that half)
        float *cs = reinterpret_cast<float *>(&sm);
#pragma unroll
        for (int half = 0; half < BM / 64; ++half) {
            if ((wm * (BM / 2)) / 64 == half) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<f32x4 *>(&cs[(wm * (BM / 2) + i * 32 + fr - 64 * half) * kCPitch +
                                                           wn * (BN / 2) + j * 32 + crow(4 * q, lane)]) =
                                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                      acc[i][j][4 * q + 3]};
            }
            __syncthreads();
            epilogue<T, true, 64, BN>(P, cs, m0 + 64 * half, n0, tid, inv_seg);
            if (half + 1 < BM / 64) __syncthreads();
        }
    };
    if (vtile) run(std::true_type());
    else run(std::false_type());
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool gemm_vec_ok(bool is_bf16, const GemmProblem &p) {
    const long long es = is_bf16 ? 2 : 4;
    const long long epc = 16 / es;
    if (p.kdim % epc) return false;
    if ((p.a_ld * es) % 16 || (p.a_bstride * es) % 16 || !aligned16(p.a)) return false;
    if (p.a_mode == A_CONTEXT && (!aligned16(p.ring) || (p.ring_bstride * es) % 16 || (p.ring_ld * es) % 16))
        return false;
    if ((p.b_ld * es) % 16 || (p.b_bstride * es) % 16 || !aligned16(p.b0) || (p.b1 && !aligned16(p.b1))) return false;
    if (p.epi == EPI_ROWS) {
        // eight-column vector stores of the output (and loads of the residual)
        const long long oes = p.out_f32 ? 4 : es;
        if (!aligned16(p.c0) || (p.c_ld * oes) % 16 || (p.c_bstride * oes) % 16) return false;
        if (p.res && (!aligned16(p.res) || (p.res_ld * es) % 16 || (p.res_bstride * es) % 16)) return false;
    }
    return true;
}

template <int BM>
void launch_bm(bool is_bf16, bool vec, const GemmLaunch &g, hipStream_t s) {
    dim3 grid(g.total_tiles + extra_blocks(g)), block(kThreads);
    if (is_bf16) {
        if (vec) hipLaunchKernelGGL((gemm_lds_kernel<bf16, BM, kBN>), grid, block, 0, s, g);
        else hipLaunchKernelGGL((gemm_kernel<bf16, false, BM>), grid, block, 0, s, g);
    } else {
        if (vec) hipLaunchKernelGGL((gemm_lds_kernel<float, BM, kBN>), grid, block, 0, s, g);
        else hipLaunchKernelGGL((gemm_kernel<float, false, BM>), grid, block, 0, s, g);
    }
}

// Launches with fewer 128-row tiles than two per CU (one wave per SIMD) take
// 64-row tiles instead: twice the workgroups, each half the work.
constexpr int kSmallGrid = 512;

hipError_t launch_gemm(bool is_bf16, const GemmLaunch &g, hipStream_t s) {
    if (g.total_tiles <= 0 && extra_blocks(g) <= 0) return hipSuccess;
    if (g.total_tiles <= 0) {                     // copies alone
        hipLaunchKernelGGL((gemm_kernel<bf16, false, 64>), dim3(extra_blocks(g)), dim3(kThreads), 0, s, g);
        return hipGetLastError();
    }
    bool vec = true, narrow = true;
    for (int i = 0; i < g.count; ++i) {
        vec = vec && gemm_vec_ok(is_bf16, g.p[i]);
        narrow = narrow && g.p[i].cols <= 64 && g.p[i].epi != EPI_KV;
    }
    if (vec && narrow && g.total_tiles >= kSmallGrid) {
        // every problem fits one 64-column tile: 128 x 64 tiles, none of the MFMA
        // work and LDS rows spent on columns past the problem
        GemmLaunch gn = g;
        int t = 0;
        for (int i = 0; i < gn.count; ++i) {
            GemmProblem &P = gn.p[i];
            P.tiles_n = 1;
            P.tile_begin = t;
            P.tile_count = (P.rows + 127) / 128;
            t += P.tile_count;
        }
        gn.total_tiles = t;
        dim3 grid(gn.total_tiles + extra_blocks(gn)), block(kThreads);
        if (is_bf16) hipLaunchKernelGGL((gemm_lds_kernel<bf16, 128, 64>), grid, block, 0, s, gn);
        else hipLaunchKernelGGL((gemm_lds_kernel<float, 128, 64>), grid, block, 0, s, gn);
        return hipGetLastError();
    }
    if (g.total_tiles >= kSmallGrid) {
        launch_bm<128>(is_bf16, vec, g, s);
    } else {
        GemmLaunch g64 = g;
        int t = 0;
        for (int i = 0; i < g64.count; ++i) {
            GemmProblem &P = g64.p[i];
            P.tile_begin = t;
            P.tile_count = ((P.rows + 63) / 64) * P.tiles_n;
            t += P.tile_count;
        }
        g64.total_tiles = t;
        launch_bm<64>(is_bf16, vec, g64, s);
    }
    return hipGetLastError();
}

}  // namespace txl

namespace txl {

hipError_t launch_pitch_copies(const PitchCopy *pc, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (n > kMaxPitchCopies) return hipErrorInvalidValue;
    GemmLaunch g;
    memset(&g, 0, sizeof(g));
    for (int i = 0; i < n; ++i) g.pc[i] = pc[i];
    g.pc_count = n;
    return launch_gemm(true, g, s);
}

}  // namespace txl
