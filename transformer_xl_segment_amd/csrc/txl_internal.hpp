// txl_internal.hpp -- launchers behind the C ABI and the descriptors they take.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace txl {

// ---------------------------------------------------------------------------
// Grouped GEMM: C = A B^T with B out-major [n][k] (a weight), up to 3
// independent problems in one launch. Rows of A and C are addressed as
// (batch b, row t) with t < seg_rows; columns of C may live in a padded
// per-head space (head hh, column c < dhp; columns c >= dh of every head are
// exact zeros because the matching weight rows read as zero).
// ---------------------------------------------------------------------------
enum ARowMode {
    A_ROWS = 0,      // row (b, t): a_first <= t < a_first + valid_rows -> a + b*a_bstride + (t - a_first)*a_ld,
                     //             else zero
    A_CONTEXT = 1,   // row (b, j): j < mem_len -> ring row (head + j) % ring_M of batch b,
                     //             j < mem_len + valid_rows -> a row j - mem_len, else zero
};
enum BColMode {
    B_ROWS = 0,      // column n < cols reads weight row n
    B_HEADS = 1,     // column n -> (hh, c) = (n / dhp, n % dhp); c < dh -> weight row hh*dh + c
};
enum EpiMode {
    EPI_ROWS = 0,    // dst = c0 + b*c_bstride + t*c_ld + n (+bias[n], relu, +residual), T or fp32
    EPI_QUV = 1,     // c0 = (acc + u) * qscale, c1 = (acc + v) * qscale, head-major [b][hh][t][c]
                     // (u and v both null: no biases)
    EPI_KV = 2,      // n < b_split: c0 head-major [b][hh][slot][c]; else c1 transposed [b][hh][c][slot],
                     // slot = (kv_base + t) mod kv_slots
    EPI_HEADS = 3,   // c0 head-major [b][hh][t][c]
    EPI_RFRAG = 4,   // c0 distance-key table of head hh (hh * frag_hstride), row t, column c in the
                     // fragment-major order of rk_elem (rows offset by frag_off)
    EPI_GROWS = 5,   // batch entry b = (bb, hh) = (b / heads, b % heads): fp32 c0 + bb*c_bstride + t*c_ld +
                     // hh*dh + c for t < c_rows and c < dh (column c of dhp = the entry's only head)
};

struct GemmProblem {
    int rows, cols, kdim;        // C is rows x cols; reduction over kdim
    int tiles_n, tile_begin, tile_count;
    int seg_rows;                // rows per batch entry (row = b*seg_rows + t)
    int valid_rows;              // rows per batch entry that hold data (A side)
    int a_first;                 // A_ROWS: first output row that holds data
    // A operand
    int a_mode;
    const void *a;
    long long a_ld, a_bstride;
    const void *ring;
    long long ring_bstride;      // elements between batch entries of the ring (M*ld)
    long long ring_ld;           // elements between rows of the ring
    int ring_M, ring_head, mem_len;
    // B operand
    int b_mode;
    const void *b0, *b1;
    int b_split;                 // columns >= b_split read b1 at column n - b_split
    long long b_ld;
    int dh, dhp, heads;
    // epilogue
    int epi;
    void *c0, *c1;
    long long c_ld, c_bstride;
    const void *bias;
    const void *res;
    long long res_ld, res_bstride;
    const void *u, *v;
    float qscale;
    int relu, out_f32;
    int kv_slots, kv_base;       // EPI_KV: slots per (b, hh) and slot of row t = 0 (multiples of 8)
    int frag_off;                // EPI_RFRAG: row offset of the 32-row blocks
    long long frag_hstride;      // EPI_RFRAG: elements per head
    long long b_bstride;         // B_ROWS: elements between the B operands of batch entries (0: one B;
                                 // nonzero requires seg_rows % 128 == 0 so no tile straddles entries)
    int c_rows;                  // EPI_GROWS: rows of each entry that are written
    int kz_on, kz_lag;           // kz_on: row t of every entry of A is zero for k < t - kz_lag (a causal
                                 // band), so a tile may start its reduction there
};

// Memory update riding along a GEMM launch (segment-recurrence simulator: mem =
// last M rows of [mem; h]): the workgroups after the launch's tiles copy, for
// every batch row b, the n source rows src_row0 .. src_row0+n-1 of b into ring
// slots pos0, pos0+1, ... (mod M). With contiguous source rows one batch row's
// copy is two contiguous runs (before and after the wrap), moved in words of
// 16 bytes (vec) or 4 bytes, kRingCopyUnroll x 256 words per workgroup; with a
// source row pitch other than the row length (a padded activation) each
// workgroup copies kRingCopyRows rows word by word. Word indices within a
// batch row fit 32 bits. blocks_x workgroups per batch row.
struct RingCopy {
    char *ring;
    const char *src;
    long long src_bstride_bytes;
    int M, row_words, pos0, src_row0, n, blocks_x, vec;
    int src_pitch_words;         // words between source rows
};
constexpr int kRingCopyUnroll = 4;
constexpr int kRingCopyRows = 8;

// A strided copy with zero fill riding along a launch the same way: for rows
// r < rows (batch entry r / seg_rows, row r % seg_rows), dst words [w0, w1) take
// src word c - w0 while c - w0 < copy_w and zero after it (src null: zeros
// only). Used to lay rows out at a 16-byte aligned pitch.
struct PitchCopy {
    const uint32_t *src;
    uint32_t *dst;
    long long src_pitch, dst_pitch;   // words between rows of one batch entry
    long long src_bstride, dst_bstride;  // words between batch entries
    int seg_rows;                     // rows per batch entry (row r = (r / seg_rows, r % seg_rows))
    int rows, w0, w1, copy_w, blocks;
    int rb;                           // rows per workgroup (about kPitchWords words)
};
constexpr int kPitchWords = 2048;     // words a pitched-copy workgroup moves (8 per thread)
constexpr int kMaxPitchCopies = 6;

struct GemmLaunch {
    GemmProblem p[3];
    int count;
    int total_tiles;
    int lead;                    // 1 or 2: the tiles of p[0 .. lead-1] are dealt out before the others
    RingCopy rc;
    int copy_blocks;             // workgroups after the tiles that run rc (0: none)
    PitchCopy pc[kMaxPitchCopies];
    int pc_count;                // pitched copies run by the workgroups after those
};

// Tile of workgroup gid. Workgroups are dispatched in order, round-robin over
// the 8 XCDs (gid % 8), so each XCD is dealt a contiguous run of tiles
// (consecutive tiles share A rows in its L2). With `first` > 0 the first
// first & ~7 tiles are dealt that way before the rest: they all start in the
// first round of a launch with more tiles than slots.
__device__ __forceinline__ int deal_tile(int gid, int total, int first) {
    const int p8 = first & ~7;
    const int base = gid < p8 ? 0 : p8;
    const int n = gid < p8 ? p8 : total - p8;
    const int g = gid - base;
    const int full = n - (n & 7);
    return base + (g < full ? (g & 7) * (full >> 3) + (g >> 3) : g);
}
__device__ __forceinline__ int lead_tiles(const GemmLaunch &g) {
    return g.lead == 1 && g.count > 1 ? g.p[1].tile_begin : g.lead == 2 && g.count > 2 ? g.p[2].tile_begin : 0;
}

// Workgroups a launch adds after its tiles.
inline int extra_blocks(const GemmLaunch &g) {
    int n = g.copy_blocks;
    for (int i = 0; i < g.pc_count; ++i) n += g.pc[i].blocks;
    return n;
}

// Workgroup `blk` (0 <= blk < blocks_x * B) of a ring copy, 256 threads.
__device__ __forceinline__ void ring_copy_block(const RingCopy &rc, int blk) {
    const int b = blk / rc.blocks_x, bx = blk - b * rc.blocks_x;
    const char *s0 = rc.src + (long long)b * rc.src_bstride_bytes;
    char *d0 = rc.ring + (long long)b * rc.M * rc.row_words * (rc.vec ? 16 : 4);
    if (rc.src_pitch_words != rc.row_words) {
        // pitched source rows (4-byte words): kRingCopyRows rows per workgroup
        const uint32_t *s = reinterpret_cast<const uint32_t *>(s0);
        uint32_t *d = reinterpret_cast<uint32_t *>(d0);
        const int r1 = min(rc.n, (bx + 1) * kRingCopyRows);
        for (int r = bx * kRingCopyRows; r < r1; ++r) {
            int slot = rc.pos0 + r;
            if (slot >= rc.M) slot -= rc.M;
            const uint32_t *sr = s + (long long)(rc.src_row0 + r) * rc.src_pitch_words;
            uint32_t *dr = d + (long long)slot * rc.row_words;
            for (int c = (int)threadIdx.x; c < rc.row_words; c += 256) dr[c] = sr[c];
        }
        return;
    }
    const int total = rc.n * rc.row_words;                       // words of this batch row
    const int split = min(rc.n, rc.M - rc.pos0) * rc.row_words;  // words before the wrap
    const int base = bx * 256 * kRingCopyUnroll + (int)threadIdx.x;
    auto run = [&](auto word) {
        typedef decltype(word) Word;
        const Word *s = reinterpret_cast<const Word *>(s0) + (long long)rc.src_row0 * rc.row_words;
        Word *d = reinterpret_cast<Word *>(d0);
        Word v[kRingCopyUnroll];
#pragma unroll
        for (int u = 0; u < kRingCopyUnroll; ++u) {
            const int w = base + 256 * u;
            if (w < total) v[u] = s[w];
        }
#pragma unroll
        for (int u = 0; u < kRingCopyUnroll; ++u) {
            const int w = base + 256 * u;
            if (w < total) d[w < split ? (long long)rc.pos0 * rc.row_words + w : w - split] = v[u];
        }
    };
    typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
    if (rc.vec) run(u32x4_());
    else run(uint32_t());
}

// floor(x / d) for 0 <= x < 2^22 (a float reciprocal and one fix-up)
__device__ __forceinline__ int small_div(int x, int d, float inv) {
    int q = (int)((float)x * inv);
    const int r = x - q * d;
    if (r < 0) q -= 1;
    else if (r >= d) q += 1;
    return q;
}

// Workgroup `blk` of a pitched copy: rows blk rb .. +rb, flat over those rows'
// words (columns w0 .. w1 of the destination), eight words per thread with
// all eight loads in flight before the stores.
__device__ __forceinline__ void pitch_copy_block(const PitchCopy &pc, int blk) {
    const int width = pc.w1 - pc.w0;
    const int r0 = blk * pc.rb;
    const int nr = min(pc.rb, pc.rows - r0);
    if (nr <= 0 || width <= 0) return;
    const int total = nr * width;                     // < 2^22: rb width is about kPitchWords
    const float inv_w = 1.f / (float)width, inv_s = 1.f / (float)pc.seg_rows;
    constexpr int U = kPitchWords / 256;
    for (int base = (int)threadIdx.x; base < total; base += 256 * U) {
        uint32_t v[U];
        long long at[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + 256 * u;
            v[u] = 0u;
            at[u] = -1;
            if (idx < total) {
                const int rl = small_div(idx, width, inv_w);
                const int k = idx - rl * width;
                const int r = r0 + rl;
                const int b = small_div(r, pc.seg_rows, inv_s), t = r - b * pc.seg_rows;
                if (pc.src && pc.w0 + k < pc.copy_w)
                    v[u] = pc.src[(long long)b * pc.src_bstride + (long long)t * pc.src_pitch + pc.w0 + k];
                at[u] = (long long)b * pc.dst_bstride + (long long)t * pc.dst_pitch + pc.w0 + k;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (at[u] >= 0) pc.dst[at[u]] = v[u];
    }
}

// The work of workgroup `blk` counted from the first one after a launch's tiles.
__device__ __forceinline__ void extra_block(const GemmLaunch &g, int blk) {
    if (blk < g.copy_blocks) {
        ring_copy_block(g.rc, blk);
        return;
    }
    blk -= g.copy_blocks;
#pragma unroll
    for (int i = 0; i < kMaxPitchCopies; ++i) {
        if (i < g.pc_count) {
            if (blk < g.pc[i].blocks) {
                pitch_copy_block(g.pc[i], blk);
                return;
            }
            blk -= g.pc[i].blocks;
        }
    }
}

// Plans the copy "ring rows (pos0 + t) % M of every batch entry <- src rows
// src_row0 + t, t < n" (source rows src_ld elements apart) into rc; returns the
// number of workgroups (B * blocks_x, 0 for nothing to copy) or -1 if the sizes
// exceed the 32-bit word indexing.
int plan_ring_copy(bool is_bf16, RingCopy &rc, void *ring, int M, int D, int pos0, const void *src,
                   long long src_bstride, long long src_ld, int src_row0, int n, int B);

// Returns a hipError_t from the launch.
hipError_t launch_gemm(bool is_bf16, const GemmLaunch &g, hipStream_t s);

// Is every operand row of the problem 16-byte aligned (vectorised loads)?
bool gemm_vec_ok(bool is_bf16, const GemmProblem &p);

// ---------------------------------------------------------------------------
// Relative attention over projected, head-major operands.
//   qu, qv  [B][H][Wp][dp]  (q + u) and (q + v), pre-scaled by log2(e)/sqrt(dh)
//   ke      [B][H][C][dp]   content keys; key j lives in slot (khead + j) mod C
//   vt      [B][H][dp][C]   values, transposed, same slots (khead and C multiples
//                           of 8, C >= Kp)
//   rk      [H][ATTN_RPAD + Kp + ATTN_RPAD][dp]  distance keys, head stride rk_hstride
//           elements (0: one table shared by every head); row ATTN_RPAD + d holds
//           distance d for 0 <= d < K and zeros elsewhere, so reads of distances in
//           [-ATTN_RPAD, Kp + ATTN_RPAD) need no bounds checks
//   dist    0: no distance term (content attention; rk unused)
//   lse     optional [B][H][Wp] fp32: per query, log2 of the softmax denominator
//           in the pre-scaled score units (max + log2(sum))
//   o       [B][W][D]       output rows (heads concatenated), batch stride o_bstride
// Rows past W (queries) hold zeros; key slots past K hold finite values (they
// are masked).
// ---------------------------------------------------------------------------
struct AttnArgs {
    const void *qu, *qv, *ke, *vt, *rk;
    void *o;
    long long o_bstride;
    long long o_ld;              // elements between rows of o (0: D)
    int B, H, W, Wp, m, K, Kp, dh, dp, D;
    int C, khead;
    long long rk_hstride;
    int dist;
    float *lse;
    // key split: nsplit > 1 runs nsplit workgroups per query block over disjoint
    // key ranges; each writes its unnormalised output (part_o, [split][bh][Wp][dp]
    // fp32) and (running base, sum) pair (part_ml, [split][bh][Wp][2]), and a
    // second kernel merges them
    int nsplit;
    float *part_o, *part_ml;
};
// start / stop: optional events stamped at this kernel's own start and end.
hipError_t launch_rel_attn(bool is_bf16, const AttnArgs &a, hipStream_t s, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr);
bool rel_attn_supported(int dh);
// key splits for a launch over K keys: more than one only when the query blocks
// alone cannot fill the chip; non-decreasing in K
int attn_splits(int B, int H, int W, int K);
int attn_dp(int dh);          // padded head width used by the attention kernel
const int ATTN_QBLOCK = 128;  // queries per workgroup
const int ATTN_KBLOCK = 64;   // keys per step
const int ATTN_RPAD = 128;    // zero rows before and after the distance keys

// Distance-key table of one head, [ATTN_RPAD + Kp + ATTN_RPAD] rows of dp columns
// (row ATTN_RPAD + d holds distance d), stored in the order the attention
// kernel's MFMA fragments read it: 32-row blocks whose first row is congruent
// to off (mod 32), each block as dp/8 column groups of 32 rows x 8 columns, so
// that one 16-byte fragment load of a wave (32 rows, 8 columns each, for both
// halves of a column group of 16) is 1 KB contiguous. The table takes
// rk_table_rows(Kp) rows' worth of elements (one more block than the rows).
__host__ __device__ inline int rk_table_rows(int Kp) { return Kp + 2 * ATTN_RPAD + 32; }
__host__ __device__ inline long long rk_elem(int row, int col, int off, int dp) {
    const int t = (row - off + 32) >> 5;            // block of this row (row >= 0, 0 <= off < 32)
    const int r = row - (32 * t + off - 32);        // row within the block
    return (long long)t * 32 * dp + (col >> 3) * 256 + r * 8 + (col & 7);
}
// the row offset a launch with m memory keys uses: every window of distances
// the attention kernel loads starts at a distance congruent to m + 1 (mod 32)
__host__ __device__ inline int rk_frag_off(int m) { return (m + 1) & 31; }

// Encoding variants (txl_variants.hip).
int shaw_max_clip();
// Shaw's distance keys: one table in the rk_elem layout (row offset off), row ATTN_RPAD + d = aK[min(d, clip)]
hipError_t launch_shaw_rows(bool is_bf16, void *rk, const void *aK, int clip, int K, int Kp, int dh, int dp,
                            int off, hipStream_t s);
// Shaw's value term added to a.o, from a.qu, a.qv, a.ke, a.lse and the distance table a.rk (the aK rows)
// of a finished attention launch
hipError_t launch_shaw_values(bool is_bf16, const AttnArgs &a, const void *aV, int clip, hipStream_t s);
hipError_t launch_add_positions(bool is_bf16, const void *x, long long x_bstride, void *y, long long y_bstride,
                                int B, int W, int D, int pos0, hipStream_t s);

// Backward of the relative attention: fused query side (txl_attn_bwd.hip).
//   qu, qv, dO [B][H][Wp][dp]  (q + u), (q + v) pre-scaled as for the forward; dO unscaled
//   ke, vk     [B][H][Kp][dp]  content keys and values;  kt [B][H][dp][Kp]  keys transposed
//   rk         distance-key table in the rk_elem layout (row offset rk_frag_off(m)), head stride rk_hstride
//   rt         [H][dp][rt_ld]  distance keys transposed: distance d at column d + rt_off
//              (attn_bwd_rt_off(m), attn_bwd_rt_ld(Kp)), zero outside 0 <= d < K
//   o          [B][W][D]  forward output;  lse [B][H][Wp]  its log-sum-exp (log2 units)
// Writes dq [B][W][D] fp32; part [2][H][B * ceil(W / ATTN_QBLOCK) * 4][64] fp32, per wave
// of 32 queries the column sums of dq's content (du) and distance (dv) parts; pt, dst [B][H][Kp][Wp] (p and c p (dP - D), key-major) and dsd [B][H][Kp][Wp] (the
// latter re-indexed by distance d = m + i - j); columns < W8 (W rounded up to 8) hold
// data, zero where no key is visible (in particular past W); c = 1/sqrt(dh).
struct AttnBwdArgs {
    const void *qu, *qv, *dO, *ke, *vk, *kt, *rk, *rt, *o;
    const float *lse;
    float *dq, *part;
    void *pt, *dst, *dsd;
    int B, H, W, Wp, m, K, Kp, dh, dp, D;
    long long rk_hstride;
    int rt_ld, rt_off;
    float c;
};
hipError_t launch_rel_attn_bwd(bool is_bf16, const AttnBwdArgs &a, hipStream_t s);
int attn_bwd_rt_off(int m);
int attn_bwd_rt_ld(int Kp);

// Operand packing and reductions of the backward (txl_backward.hip).
struct BwdDims {
    int B, H, W, Wp, W8, m, K, Kp, dh, dp, D;
};
// Packed operands of the backward (G = B*H entries, zero padding past the data):
//   qu, qv = (q + u) * qscale, (q + v) * qscale and dOh  [G][Wp][dp];  qut, qvt = (q + u), (q + v)
//   and dOt transposed [G][dp][Wp];  ke, vk [G][Kp][dp] and ket, vt [G][dp][Kp] (keys, values);
//   rk: the attention kernels' distance-key table (rk_elem layout, row offset rk_frag_off(m),
//   rk_table_rows(Kp)*dp per head); rt [H][dp][attn_bwd_rt_ld(Kp)], distance d at column
//   d + attn_bwd_rt_off(m)
struct BwdPack {
    void *qu, *qv, *dOh, *qut, *qvt, *dOt, *ke, *vk, *ket, *vt, *rk, *rt;
};
hipError_t launch_bwd_pack(bool is_bf16, const BwdDims &d, const BwdPack &o, const void *q, const void *k,
                           const void *val, const void *r, const void *u, const void *v, const void *dO,
                           float qscale, hipStream_t s);
// per-wave partial sums of du, dv written by the attention backward
int bwd_parts(const BwdDims &d);
// dr [K][D] = drh [G][Kp][dp] summed over the batch; du, dv [D] from part
// ([2][H][bwd_parts(d)][64] fp32, fixed summation order)
hipError_t launch_bwd_finish(const BwdDims &d, const float *drh, const float *part, float *dr, float *du, float *dv,
                             hipStream_t s);

// ---------------------------------------------------------------------------
// Small kernels.
// ---------------------------------------------------------------------------
// A planned ring copy (plan_ring_copy) as its own launch of `blocks` workgroups.
hipError_t launch_ring_copy(const RingCopy &rc, int blocks, hipStream_t s);
// Pitched copies (at most kMaxPitchCopies) as a launch of their own.
hipError_t launch_pitch_copies(const PitchCopy *pc, int n, hipStream_t s);
// y[b][t] = LN(x[b][t] (+ x2[b][t])) with fp32 input(s) (rows x_ld apart, row b*W + t), T output (batch
// stride y_bstride, rows y_ld apart); x2 may be null
hipError_t launch_layer_norm(bool is_bf16, const float *x, const float *x2, long long x_ld, const void *g,
                             const void *b, void *y, long long y_bstride, long long y_ld, int B, int W, int D,
                             hipStream_t s);
hipError_t launch_sinusoid(bool is_bf16, void *R, int R_len, int D, hipStream_t s);

}  // namespace txl
