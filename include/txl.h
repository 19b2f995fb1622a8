/*
 * txl.h -- C ABI of libtxl: Transformer-XL relative-position attention over a
 * cached segment memory, on MI355X (gfx950).
 *
 * Method (web pages on Transformer-XL):
 *  - "Transformer-XL, explained." (vibeengines.com), the numbered method steps:
 *    keys and values span the cached states of the previous segment followed by
 *    the current segment, queries come from the current segment only, under a
 *    causal mask (step 3); the score of query i and key j adds a content term and
 *    a term in a sinusoidal encoding of the distance i - j, with separate key
 *    projections for content and distance and two learned global biases u and v
 *    (step 4, and the legend of the score equation); the distance term is
 *    computed once against all distances and shifted into place (step 5); the
 *    memory may be longer at evaluation than in training (step 7).
 *  - the segment-recurrence simulator (mysimulator.uk): h~ = [SG(mem); h],
 *    K,V = h~ W, Q = h W, mem = last M rows of h~, softmax(Q K^T / sqrt(d)) V.
 *  - "Implementing Transformer-XL" (mbrenndoerfer.com), the NumPy layer: the
 *    output projection W_o, post-LN residual blocks with LayerNorm
 *    gamma * (x - mean) / (std + 1e-6) + beta (population std) and a ReLU FFN.
 *
 * What one call computes, per batch row b and head hd (columns
 * [hd*dh, (hd+1)*dh) of every D-wide tensor, dh = D / H), with m = mem->len
 * cached rows (oldest first) and K = m + W keys:
 *    ctx = [mem rows; h rows]                       (K x D)
 *    q = h Wq^T,  k = ctx WkE^T,  val = ctx Wv^T,  r = R[0:K] WkR^T
 *    s_ij = ((q_i + u).k_j + (q_i + v).r_{m+i-j}) / sqrt(dh)   for j <= m + i
 *    p_ij = softmax_j(s_ij),  o_i = sum_j p_ij val_j,  out = o Wo^T
 *
 * Conventions:
 *  - Every weight matrix is stored out-major, W[d_out][d_in], row-major, and
 *    a projection computes y = x W^T (the torch.nn.Linear layout).
 *  - All tensors of one call share one storage dtype (txl_dtype). Products
 *    and sums accumulate in fp32; softmax statistics, LayerNorm statistics and
 *    pre-LayerNorm residual sums are kept in fp32.
 *  - All pointers are device pointers unless stated otherwise; every buffer
 *    belongs to the caller. The library never allocates device memory: scratch
 *    space is the caller's workspace, sized by txl_workspace_bytes() (the one
 *    exception, txl_rel_attn_fwd_noalloc, uses a fixed array in the library).
 *  - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and
 *    nothing waits for it: results are ready when the stream reaches them.
 *  - Strides are in elements. `*_bstride` is the distance between batch rows;
 *    rows within a batch row are D elements apart.
 *  - Pointers must be aligned to 4 bytes; 16-byte aligned pointers with D a
 *    multiple of 8 take the vectorised load path.
 *
 * Errors: a call returns a txl_status. Arguments are checked before anything is
 * enqueued; a call that returns anything but TXL_OK has enqueued no work, except
 * TXL_ERR_HIP, which reports a launch failure after earlier launches of the same
 * call may have been enqueued. txl_last_error() gives a message for the calling
 * thread's last failure.
 */
#ifndef TXL_H
#define TXL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TXL_OK = 0,
    TXL_ERR_ARG = 1,          /* bad size, null or misaligned pointer, inconsistent memory */
    TXL_ERR_UNSUPPORTED = 2,  /* a head width or dtype this build has no kernel for */
    TXL_ERR_WORKSPACE = 3,    /* workspace missing or smaller than txl_workspace_bytes() */
    TXL_ERR_HIP = 4           /* a HIP runtime call failed */
} txl_status;

typedef enum { TXL_FP32 = 0, TXL_BF16 = 1 } txl_dtype;

typedef enum {
    TXL_OP_REL_ATTN = 0,      /* txl_rel_attn_fwd, txl_rel_attn_fwd_update */
    TXL_OP_LAYER = 1,         /* txl_layer_fwd */
    TXL_OP_STACK = 2,         /* txl_stack_fwd_segments */
    TXL_OP_REL_ATTN_CACHED = 3, /* txl_rel_attn_fwd_cached */
    TXL_OP_ATTN_VARIANT = 4,  /* txl_attn_fwd_variant */
    TXL_OP_REL_ATTN_BWD = 5   /* txl_rel_attn_bwd (M = the memory length m) */
} txl_op;

/* Position encodings Transformer-XL is compared against ("Transformer-XL,
 * explained.", "What it adds to earlier relative positions" and the ablations
 * among its results). */
typedef enum {
    TXL_POS_SHAW = 1,         /* Shaw et al.: learned clipped-distance embeddings on keys and values */
    TXL_POS_ABSOLUTE = 2      /* absolute positions in the rows, content-only attention */
} txl_pos_variant;

/* One layer's parameters, all device pointers of the call's dtype.
 * Attention (pages: W_q, W_k,E, W_k,R, W_v, W_o and the global biases u, v):
 *   Wq, WkE, WkR, Wv, Wo  [D][D] out-major;  u, v  [D].
 * Post-LN block (only read by txl_layer_fwd / txl_stack_fwd_segments):
 *   ln1_g, ln1_b  [D];  W1 [F][D], b1 [F];  W2 [D][F], b2 [D];  ln2_g, ln2_b [D]. */
typedef struct {
    const void *Wq, *WkE, *WkR, *Wv, *Wo;
    const void *u, *v;
    const void *ln1_g, *ln1_b;
    const void *W1, *b1;
    const void *W2, *b2;
    const void *ln2_g, *ln2_b;
} txl_layer_params;

/* Segment memory of one layer: a ring of M rows per batch row.
 *   data  device, [B][M][D] of the call's dtype, owned by the caller;
 *   M     capacity in rows (>= 1);
 *   len   valid rows m, 0 <= len <= M (0 = empty memory);
 *   head  physical row of the oldest valid row, 0 <= head < M.
 * Logical row l (0 = oldest) of batch row b is data[b][(head + l) % M][:].
 * Attention calls only read the ring; txl_mem_update advances it. */
typedef struct {
    void *data;
    int M;
    int len;
    int head;
} txl_mem;

/* Projected key/value cache of one attention layer: the memory kept as the
 * keys k = x WkE^T and values val = x Wv^T of its rows instead of the rows x
 * themselves, so a segment projects only its own W rows ("Transformer-XL,
 * explained.", closing assessment: computed keys and values are cached rather
 * than recomputed; Ultralytics glossary, comparison with related models, the
 * key/value cache). A ring of C slots per (batch row, head), head-major:
 *   k   device [B][H][C][dp]   keys, dp = D/H rounded up to a multiple of 16
 *   vt  device [B][H][dp][C]   values transposed (one row per head column)
 * Slot s of (b, hh) is k[b][hh][s][:] and vt[b][hh][:][s]; padding columns
 * (dh <= c < dp) hold zeros.
 *   M     memory length in rows, a positive multiple of 8;
 *   C     slots, txl_kv_cache_capacity(M, W) for the largest W used;
 *   len   cached rows (0 = empty), a multiple of 8, len <= M;
 *   head  slot of the oldest cached row, a multiple of 8, head < C.
 * Both buffers belong to the caller and must be zero-filled before first use
 * (slots outside the window are read for masked keys and must be finite).
 * The calls below advance len and head on the host. */
typedef struct {
    void *k;
    void *vt;
    int C;
    int M;
    int len;
    int head;
} txl_kv_cache;

/* Workspace bytes that `op` needs for these sizes (M = memory capacity; F is
 * ignored for TXL_OP_REL_ATTN and TXL_OP_REL_ATTN_CACHED). Returns 0 for invalid sizes. The same value
 * serves every call of that op with sizes no larger than these. */
size_t txl_workspace_bytes(txl_op op, txl_dtype dtype, int B, int W, int M, int D, int H, int F);

/* Relative-encoding table R [R_len][D] (explainer, step 4). R is a fixed
 * function of the distance, not a learned table. Row d holds
 *   R[d][k] = sin(d * 10000^(-2k/D)),  R[d][D/2 + k] = cos(d * 10000^(-2k/D)),
 * for k < D/2, evaluated in double precision and rounded to `dtype`.
 * D must be even. */
txl_status txl_sinusoid_table(txl_dtype dtype, int R_len, int D, void *R, void *stream);

/* Relative multi-head attention of one segment over [mem; h], then the output
 * projection (explainer steps 3-5; simulator equations; NumPy layer's
 * relative_attention without its attention-weight output).
 *   h    [B][W][D], batch stride h_bstride (>= W*D);
 *   mem  NULL or a ring with len == 0 for an empty memory; read only;
 *   p    reads Wq, WkE, WkR, Wv, Wo, u, v;
 *   R    [R_len][D] distance table, R_len >= mem->len + W;
 *   out  [B][W][D], batch stride out_bstride; must not overlap h or mem.
 * D % H == 0 and D / H <= 64 (dh of 8, 32, 41 and 64 are the tested widths). */
txl_status txl_rel_attn_fwd(txl_dtype dtype, int B, int W, int D, int H,
                            const void *h, long long h_bstride,
                            const txl_mem *mem, const txl_layer_params *p,
                            const void *R, int R_len,
                            void *out, long long out_bstride,
                            void *ws, size_t ws_bytes, void *stream);

/* txl_rel_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, launches and results as
 * txl_rel_attn_fwd; the scratch space is a fixed device array of
 * TXL_NOALLOC_SCRATCH_BYTES inside the library instead of the caller's
 * workspace. The call itself allocates nothing; each GPU the library is loaded
 * on holds its own copy of the array until the process ends.
 *  - A call whose workspace (txl_workspace_bytes(TXL_OP_REL_ATTN, dtype, B, W,
 *    mem->len, D, H, 0)) exceeds TXL_NOALLOC_SCRATCH_BYTES returns
 *    TXL_ERR_WORKSPACE before touching the device (64 MiB covers B = 16,
 *    W = M = 512, D = 512 in bf16).
 *  - Every call on one GPU shares that GPU's array and leaves its contents
 *    behind; nothing in it needs to start zeroed (every scratch element is
 *    written before it is read). Calls that overlap on one GPU (two streams,
 *    or two threads) race on the array: serialize them.
 *  - The calling thread's current device must be the device of `stream`. */
#define TXL_NOALLOC_SCRATCH_BYTES (64u << 20)
txl_status txl_rel_attn_fwd_noalloc(txl_dtype dtype, int B, int W, int D, int H,
                                    const void *h, long long h_bstride,
                                    const txl_mem *mem, const txl_layer_params *p,
                                    const void *R, int R_len,
                                    void *out, long long out_bstride, void *stream);

/* txl_rel_attn_fwd followed by the memory update of the same segment
 * (txl_mem_update with the same h and W), in one call: out and the ring hold
 * exactly what those two calls would leave, and mem->len / mem->head advance
 * on the host as txl_mem_update advances them. The copy into the ring runs
 * inside the output projection's launch, after every launch that reads the
 * old rows, so the step needs no launch of its own for it. mem must not be
 * NULL (an empty ring has len == 0); out must not overlap h or the ring. On
 * any error nothing is launched and mem is unchanged. Same workspace as
 * txl_rel_attn_fwd. */
txl_status txl_rel_attn_fwd_update(txl_dtype dtype, int B, int W, int D, int H,
                                   const void *h, long long h_bstride,
                                   txl_mem *mem, const txl_layer_params *p,
                                   const void *R, int R_len,
                                   void *out, long long out_bstride,
                                   void *ws, size_t ws_bytes, void *stream);

/* Memory update (simulator: mem = last M rows of h~ = [mem; h]). Appends the
 * last min(W, M) rows of h [B][W][D] (batch stride h_bstride) to the ring,
 * dropping the oldest rows beyond M, and advances mem->len and mem->head on the
 * host. The copy is exact. Enqueue it after every attention call that reads the
 * old memory: the new rows overwrite the oldest ones. */
txl_status txl_mem_update(txl_dtype dtype, int B, int D, txl_mem *mem,
                          const void *h, long long h_bstride, int W, void *stream);

/* One post-LN Transformer-XL block (NumPy layer's forward):
 *   a = rel_attn(h, mem);  h1 = LN1(h + a);
 *   y = LN2(h1 + ReLU(h1 W1^T + b1) W2^T + b2).
 * y [B][W][D] with batch stride y_bstride must not overlap h or mem. The memory
 * is not updated (call txl_mem_update with the same h afterwards). */
txl_status txl_layer_fwd(txl_dtype dtype, int B, int W, int D, int H, int F,
                         const void *h, long long h_bstride,
                         const txl_mem *mem, const txl_layer_params *p,
                         const void *R, int R_len,
                         void *y, long long y_bstride,
                         void *ws, size_t ws_bytes, void *stream);

/* Segment-by-segment forward of a stack of n_layers blocks over a stream
 * (explainer steps 1-3 and 6): x [B][n_seg*W][D] is split into n_seg segments;
 * for each segment in order and each layer n in order, layer n runs on its
 * input h_n with memory mems[n], then mems[n] receives h_n (the layer's input
 * rows) and h_{n+1} is the layer's output. y [B][n_seg*W][D] receives the last
 * layer's output of every segment. mems[n] may start non-empty (resuming a
 * stream); every ring must have the same M. R_len >= M + W. */
txl_status txl_stack_fwd_segments(txl_dtype dtype, int B, int W, int D, int H, int F,
                                  int n_layers, int n_seg, const void *x,
                                  txl_mem *mems, const txl_layer_params *params,
                                  const void *R, int R_len, void *y,
                                  void *ws, size_t ws_bytes, void *stream);

/* Vanilla (no-memory) evaluation of a stack over one window: the model the
 * pages compare Transformer-XL against re-encodes a window of the last W tokens
 * from scratch for every new token, with no state carried between windows
 * ("Transformer-XL, explained.", the evaluation-speed result; Ultralytics
 * glossary, comparison with the vanilla Transformer). Runs n_layers blocks over
 * x [B][W][D] (batch stride x_bstride, e.g. a window of a longer stream) with no
 * memory, each layer attending within the window only, and writes the last
 * layer's output to y [B][W][D] (batch stride y_bstride, must not overlap x).
 * R_len >= W. Workspace: txl_workspace_bytes(TXL_OP_STACK, dtype, B, W, 0, D, H, F). */
txl_status txl_stack_fwd_window(txl_dtype dtype, int B, int W, int D, int H, int F, int n_layers,
                                const void *x, long long x_bstride,
                                const txl_layer_params *params, const void *R, int R_len,
                                void *y, long long y_bstride,
                                void *ws, size_t ws_bytes, void *stream);

/* Attention + output projection of one segment over [mem; h] with an encoding
 * other than Transformer-XL's (txl_pos_variant), for comparison. Reads Wq, WkE,
 * Wv and Wo of p only (no u, v, WkR, R). Causal over [mem; h] as in
 * txl_rel_attn_fwd; the memory is not updated (txl_mem_update).
 *   TXL_POS_SHAW: score_ij = (q_i.k_j + q_i.aK[min(delta, clip)]) / sqrt(dh) and
 *     o_i = sum_j p_ij (val_j + aV[min(delta, clip)]), delta = m + i - j: the
 *     first two score terms only, with learned embeddings of the clipped
 *     distance (the NumPy layer's clip to max_rel_dist) also on the values.
 *     aK, aV device [clip+1][dh] of the call's dtype, the same for every head;
 *     0 <= clip <= 128.
 *   TXL_POS_ABSOLUTE: score_ij = q_i.k_j / sqrt(dh), o_i = sum_j p_ij val_j; the
 *     positions are part of the rows (txl_add_positions on the model's input, so
 *     that cached rows keep the positions of their own segment). aK, aV unused.
 * Workspace: txl_workspace_bytes(TXL_OP_ATTN_VARIANT, ...). */
txl_status txl_attn_fwd_variant(txl_dtype dtype, txl_pos_variant variant, int B, int W, int D, int H,
                                const void *h, long long h_bstride,
                                const txl_mem *mem, const txl_layer_params *p,
                                const void *aK, const void *aV, int clip,
                                void *out, long long out_bstride,
                                void *ws, size_t ws_bytes, void *stream);

/* Backward pass of the relative attention with the memory behind a
 * stop-gradient ("Transformer-XL, explained.", method step 2 and the SG(.)
 * legend entry). The memory rows receive no gradient; their projected keys
 * and values do, as part of this segment's graph. Inputs are the projected
 * operands of one segment, in the call's dtype, rows contiguous:
 *   q, dO  [B][W][D]   queries h W_q^T; gradient of the loss w.r.t. the attention
 *                      output o (heads concatenated, before W_o)
 *   k, val [B][K][D]   content keys and values of [mem; h], K = m + W, memory first
 *   r      [K][D]      distance keys R W_kR^T for distances 0 .. K-1
 *   u, v   [D]
 * with score_ij = ((q_i+u).k_j + (q_i+v).r_{m+i-j}) / sqrt(dh), causal, and
 * o_i = sum_j softmax_j(score_ij) val_j. Outputs, fp32, rows contiguous: dq
 * [B][W][D], dk and dval [B][K][D], dr [K][D], du and dv [D], the gradients
 * w.r.t. these operands. Rows j < m of dk and dval belong to the memory's
 * projections (they reach W_kE and W_v); nothing is propagated into the memory
 * rows themselves. m + W <= 4096, D/H <= 64. Workspace:
 * txl_workspace_bytes(TXL_OP_REL_ATTN_BWD, dtype, B, W, m, D, H, 0). */
txl_status txl_rel_attn_bwd(txl_dtype dtype, int B, int W, int D, int H, int m,
                            const void *q, const void *k, const void *val, const void *r,
                            const void *u, const void *v, const void *dO,
                            float *dq, float *dk, float *dval, float *dr, float *du, float *dv,
                            void *ws, size_t ws_bytes, void *stream);

/* Absolute positions for the comparison model: y[b][t] = x[b][t] + U[pos0 + t]
 * for t < W, U[p][k] = sin(p * 10000^(-2k/D)) and U[p][D/2 + k] = cos(...), the
 * distance table's sinusoid at a position (the absolute model gives every
 * segment positions 0 .. W-1, so pos0 = 0). x and y [B][W][D] with batch strides;
 * y may equal x. D even, at most 1024. */
txl_status txl_add_positions(txl_dtype dtype, int B, int W, int D, const void *x, long long x_bstride,
                             int pos0, void *y, long long y_bstride, void *stream);

/* Slots a key/value cache needs for memory length M and segments of up to W
 * rows: M + W rounded up to a multiple of 64. Returns 0 for M < 0 or W < 1. */
int txl_kv_cache_capacity(int M, int W);

/* Projects rows x [B][n][D] (batch stride x_bstride) with WkE and Wv and
 * appends the last min(n, M) of them to the cache, dropping the oldest rows
 * beyond M (filling a cache from known rows, e.g. a warm start). Reads p->WkE
 * and p->Wv; min(n, M) must be a multiple of 8. No workspace. */
txl_status txl_kv_cache_append(txl_dtype dtype, int B, int D, int H, txl_kv_cache *cache,
                               const txl_layer_params *p, const void *x, long long x_bstride, int n,
                               void *stream);

/* txl_rel_attn_fwd over a key/value cache instead of a row memory: projects
 * the W segment rows into the cache, attends over the cached rows followed by
 * the segment (keys and values of the cached rows are reused, not recomputed),
 * applies Wo, then advances the cache window by W rows as txl_mem_update does.
 * The result equals txl_rel_attn_fwd followed by txl_mem_update on a row memory
 * that holds the same rows, bit for bit. W must be a multiple of 8 and
 * cache->C >= cache->M + W. Workspace: txl_workspace_bytes(TXL_OP_REL_ATTN_CACHED, ...). */
txl_status txl_rel_attn_fwd_cached(txl_dtype dtype, int B, int W, int D, int H,
                                   const void *h, long long h_bstride, txl_kv_cache *cache,
                                   const txl_layer_params *p, const void *R, int R_len,
                                   void *out, long long out_bstride,
                                   void *ws, size_t ws_bytes, void *stream);

/* Event timing of the relative-attention kernel. Between txl_profile_begin and
 * txl_profile_end, every attention-kernel launch (from any entry point, on its
 * own stream) gets a pair of HIP events stamped by the kernel's own dispatch
 * at its start and end, up to max_launches launches. txl_profile_end waits for
 * those events and returns the summed kernel time in milliseconds and the
 * number of timed launches. Not thread-safe; meant for benchmarks. */
txl_status txl_profile_begin(int max_launches);
txl_status txl_profile_end(double *total_ms, int *launches);
/* Per-launch kernel times, in milliseconds and launch order, of the window the
 * last txl_profile_end closed: copies min(capacity, launches) values into ms
 * (host memory owned by the caller) and their count into *n. Fails while a
 * window is open or if ms is NULL with capacity > 0. */
txl_status txl_profile_times(double *ms, int capacity, int *n);

/* Static description of a status code, and the calling thread's last error. */
const char *txl_status_string(txl_status s);
const char *txl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TXL_H */
