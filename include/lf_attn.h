/*
 * lf_attn.h - C ABI of the Longformer window + global sparse self-attention
 * forward for AMD MI355X (gfx950).  Library: liblfattn.so.
 *
 * The operation (one softmax per query over the union of its keys):
 *
 *   O[b,h,i,:] = sum_j P[i,j] V[b,h,j,:],
 *   P[i,:]     = softmax_j( Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_h) )  over j in keys(i),
 *
 *   keys(i) = all positions                        if i is global,
 *           = { i + m*dil[h] : m = -w..w } ∩ [0,L) ∪ globals   otherwise,
 *   minus every padded key; a query with no key gets an all-zero row.
 *
 * Sources: page "基于自注意力机制的长文本建模算法：Longformer详解" (Longformer
 * explained) §2 (sliding window with w keys on each side, dilated window
 * i-d*w .. i+d*w, global tokens that see every position) and §4 (the patterns
 * combined into one attention, linear cost, banded matrix products); page
 * "基于Block-Sparse Attention的Longformer" §2 and §4 (global tokens attend to
 * all tokens and all tokens attend to them); page "Reformer哈希" §"core
 * principle" (softmax(QK^T/sqrt(d))V).  Key padding and the per-head dilation
 * are conventions of this library.
 *
 * All entry points return an lf_status and never throw.  Validation is done on
 * the host before anything is enqueued, so on any error no kernel runs and
 * `out` is untouched.  Errors raised while kernels execute surface at the
 * caller's next synchronisation of `stream`.
 */
#ifndef LF_ATTN_H
#define LF_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lf_status {
    LF_OK = 0,
    LF_ERR_INVALID_ARG = 1, /* null pointer, bad size, index out of range, misaligned, aliasing */
    LF_ERR_UNSUPPORTED = 2, /* d_h != 64, too many heads or globals, unknown dtype */
    LF_ERR_HIP = 3,         /* a HIP runtime call failed (message in lf_attn_last_error) */
    LF_ERR_OOM = 4          /* device workspace allocation failed */
} lf_status;

typedef enum lf_dtype {
    LF_F32 = 0,  /* float32 inputs and output */
    LF_BF16 = 1  /* bfloat16 inputs and output; fp32 accumulation and softmax */
} lf_dtype;

#define LF_MAX_HEADS 64
#define LF_MAX_GLOBALS 256
#define LF_HEAD_DIM 64
#define LF_MAX_BIAS_W 1024 /* widest window with a relative position bias */
#define LF_RANDOM_BLOCK 64 /* keys per random block (and queries per query block) */
#define LF_MAX_RANDOM_DRAWS 16 /* random key blocks per query block */
#define LF_STATIC_SCRATCH_BYTES (16 << 20) /* device scratch of lf_attn_forward_static */

/* Kernel launches timed by lf_attn_stage_times. */
#define LF_N_STAGES 10
#define LF_STAGE_BAND 0      /* window band, global-column fold, global-row partials */
#define LF_STAGE_MERGE 1     /* log-sum-exp merge of the partials (only with globals) */
#define LF_STAGE_BWD_PREP 2  /* backward: D = rowsum(dO * O), base-2 log-sum-exp */
#define LF_STAGE_BWD_DQ 3    /* backward: dQ (row-owned), global-row partials */
#define LF_STAGE_BWD_DKV 4   /* backward: dK, dV (key-owned), global-key partials */
#define LF_STAGE_BWD_MERGE 5 /* backward: sums of the global partials (only with globals) */
#define LF_STAGE_LAYER_GEMM 6      /* layer: the four projection / feed-forward GEMMs (hipBLASLt) */
#define LF_STAGE_LAYER_POINTWISE 7 /* layer: bias + residual + LayerNorm, bias + GELU */
#define LF_STAGE_BWD_DKV_GLOBAL 8  /* backward, separate global projections: dK_g, dV_g */
#define LF_STAGE_BWD_DBIAS 9       /* backward: sums of the position-bias table gradient */

/* Pattern variants (lf_attn_set_window_mode). */
#define LF_WINDOW_SYMMETRIC 0 /* keys i + m*dil, m = -w..w (default) */
#define LF_WINDOW_CAUSAL 1    /* one-sided: every pair with its key after its query removed */

/* Global sets (lf_attn_set_global_mode). */
#define LF_GLOBALS_SHARED 0       /* global_idx[n_global]: one set for every sequence (default) */
#define LF_GLOBALS_PER_SEQUENCE 1 /* global_idx[B][n_global]: one row per sequence, entries < 0 unused */

typedef struct lf_attn_s* lf_attn_t;

/*
 * Create a handle for one element type.  Allocates only host memory; device
 * workspace is allocated on first use, on the device current at that call.
 * Errors: LF_ERR_INVALID_ARG (out == NULL), LF_ERR_UNSUPPORTED (unknown dtype).
 *
 * Failure injection for tests: if the environment variable LF_ATTN_FAULT is "alloc"
 * when the handle is created, its next device-workspace allocation fails as if
 * hipMalloc had (LF_ERR_OOM, the handle keeps its previous workspace); if it is
 * "launch", its next kernel launch fails before anything is enqueued (LF_ERR_HIP).
 * Each fires once; afterwards the handle works normally.
 */
lf_status lf_attn_create(lf_attn_t* out, lf_dtype dtype);

/*
 * Enqueue one forward pass on `stream`.
 *
 * q, k, v, out : DEVICE pointers to contiguous [B][H][L][d_h] tensors of the
 *                handle's dtype, 16-byte aligned, caller-owned; `out` must not
 *                overlap q, k or v.  They must stay valid until `stream` has
 *                finished the work.
 * B, H, L      : batch, heads, sequence length; each >= 1, H <= LF_MAX_HEADS.
 * d_h          : head dimension; must be 64 (else LF_ERR_UNSUPPORTED).
 * w            : window half-width (keys on each side); >= 0.  w*dil may exceed L.
 * dil_per_head : HOST array [H], dilation of each head, each >= 1.  Read during
 *                the call only.
 * global_idx   : HOST array [n_global] of positions in [0, L), shared by every
 *                sequence and head; duplicates are allowed and ignored; NULL iff
 *                n_global == 0.  Read during the call only.
 * n_global     : 0 .. LF_MAX_GLOBALS.
 * key_pad_mask : DEVICE array uint8 [B][L], nonzero = padded key, or NULL for
 *                no padding.  Padded keys are never attended to (their K and V
 *                contents never reach the output); padded query rows are
 *                computed by the same rule as any other row.
 * stream       : a hipStream_t (NULL = the null stream).  All kernels are
 *                enqueued on it; the call does not wait for them.
 *
 * The handle may grow its device workspace (hipMalloc) inside this call when
 * global positions are given.  Calls on one
 * handle must not overlap in time (one thread, and one stream at a time, or the
 * caller orders the streams): they share that workspace.
 */
lf_status lf_attn_forward(lf_attn_t h, const void* q, const void* k, const void* v, void* out,
                          int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                          const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                          void* stream);

/*
 * lf_attn_forward that allocates nothing, for callers that cannot allocate device
 * memory during the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * lf_attn_forward.  The global-row partials go to a static device array of
 * LF_STATIC_SCRATCH_BYTES (16 MiB) that each GPU the library runs on holds until the
 * process ends, instead of the handle's workspace; the call makes no hipMalloc,
 * hipFree or other allocating call (the array's device address is looked up once per
 * device, on the first call there).
 *
 * Limits and errors, all checked before anything is enqueued:
 *   LF_ERR_UNSUPPORTED if the partials need more than LF_STATIC_SCRATCH_BYTES
 *   (B * H * row tiles per head * 32 * ceil(n_global / 32) * 264 bytes, where a head of
 *   dilation d has d * ceil(ceil(L / d) / 128) row tiles; e.g. B = 2, H = 12, L = 4096,
 *   up to 32 globals: 6.5 MB), or if random blocks are set on the handle but their
 *   tables were not yet uploaded to this device by another entry point (this one
 *   uploads nothing); otherwise the errors of lf_attn_forward.
 * Per-launch timing (lf_attn_set_stage_timing) does not record these launches.
 * Every call on one GPU shares that GPU's array, whichever handle it comes from:
 * calls that overlap in time on one GPU (other streams, other threads) race.
 */
lf_status lf_attn_forward_static(lf_attn_t h, const void* q, const void* k, const void* v, void* out,
                                 int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                                 const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                                 void* stream);

/*
 * lf_attn_forward that also writes each row's log-sum-exp, for the backward.
 *
 * lse : DEVICE float32 [B][H][L], 4-byte aligned, not overlapping q, k, v or out:
 *       lse[b,h,i] = log sum_{j in keys(i)} exp(Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_h))
 *       (natural log), -inf for a row with no key.  It is the normaliser of the
 *       row's softmax (page "Reformer哈希" §"core principle" formula).
 * Everything else: as lf_attn_forward.  LF_ERR_INVALID_ARG if lse is NULL.
 */
lf_status lf_attn_forward_lse(lf_attn_t h, const void* q, const void* k, const void* v, void* out,
                              float* lse, int B, int H, int L, int d_h, int w,
                              const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                              const uint8_t* key_pad_mask, void* stream);

/*
 * Gradients of the forward: given dout = dL/dO, write dq, dk, dv = dL/dQ, dL/dK,
 * dL/dV for the same pattern (window, globals, padding), from the textbook
 * derivatives of O = softmax(S) V, S = Q K^T / sqrt(d_h) restricted to the key
 * sets (page "Reformer哈希" §"core principle"; the pattern as above):
 *
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . V_j - dO_i . O_i),
 *   dQ_i = sum_j dS_ij K_j / sqrt(d_h),   dK_j = sum_i dS_ij Q_i / sqrt(d_h).
 *
 * q, k, v, out, dout : DEVICE [B][H][L][d_h] of the handle's dtype (bf16 or fp32),
 *                      16-byte aligned; out and lse as written by
 *                      lf_attn_forward_lse for the same q, k, v and pattern (P is
 *                      recomputed from them).
 * lse                : DEVICE float32 [B][H][L], 4-byte aligned.
 * dq, dk, dv         : DEVICE [B][H][L][d_h] outputs of the handle's dtype, 16-byte
 *                      aligned, not overlapping any input or each other.  Padded keys
 *                      get dk = dv = 0; rows with no key get dq = 0.
 * Other arguments: as lf_attn_forward.  Both dtypes run the same kernels (bf16: bf16
 * MFMA products with fp32 accumulation; fp32: fp32 MFMA products).  The handle grows a
 * second device workspace (hipMalloc) for row statistics and the partial sums of
 * global rows and keys; calls on one handle must not overlap.  The result is
 * deterministic (fixed summation order, no atomics).
 */
lf_status lf_attn_backward(lf_attn_t h, const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                           const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                           void* stream);

/*
 * lf_attn_backward that also writes the gradient of the relative position bias table
 * set on the handle (lf_attn_set_position_bias), so that the table can be learned
 * (page "基于自注意力机制的长文本建模算法：Longformer详解" §5 names the relative
 * position bias, §6 the pretraining).  With the table added to the scaled score of
 * each window pair j = i + m*dil of a non-global row i,
 *
 *   dbias[h][m + w] = sum over b and those pairs of dS_ij      (m = -w .. w),
 *
 * dS as in lf_attn_backward.  Pairs that enter through the global pattern or a random
 * block carry no bias and add nothing.
 *
 * dbias : DEVICE float32 [H][2w + 1], 4-byte aligned, fully overwritten, not
 *         overlapping any other argument.  With w >= L the entries of offsets no pair
 *         reaches are 0.
 * Other arguments, outputs and errors: as lf_attn_backward, whose dq, dk and dv it
 * writes bit for bit; LF_ERR_INVALID_ARG if no table is set on the handle or dbias is
 * NULL.  Each dQ work-group keeps per-wave offset sums in 4 * (2w' + 193) * 4 bytes of
 * LDS (w' = min(w, L)) and writes them to the backward workspace (which grows by
 * B * H * tiles * (2w' + 1) floats); a last kernel adds them up per head in a fixed
 * order, so repeated calls give the same table bit for bit.
 */
lf_status lf_attn_backward_bias(lf_attn_t h, const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dbias,
                                int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                                const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                                void* stream);

/*
 * The same forward with separate projections for the global rows.
 *
 * Page "基于Block-Sparse Attention的Longformer" §4 gives global attention its
 * own query, key and value projections.  Here a global query row i attends
 * every unpadded key with them,
 *
 *   O[b,h,i,:] = softmax_j( Q_g[b,h,i,:] . K_g[b,h,j,:] / sqrt(d_h) ) V_g[b,h,j,:],
 *
 * and every other row is computed exactly as by lf_attn_forward from q, k, v
 * (its global keys included).
 *
 * q_g, k_g, v_g : DEVICE pointers to contiguous [B][H][L][d_h] tensors of the
 *                 handle's dtype, 16-byte aligned, caller-owned, none of them
 *                 overlapping `out` (they may alias q, k, v or each other).
 *                 Only the global rows of q_g are read, and only when
 *                 n_global > 0; all three must be non-null regardless.
 * All other arguments, ownership, workspace and error behaviour: as for
 * lf_attn_forward.  With q_g = q, k_g = k, v_g = v the result equals
 * lf_attn_forward's up to rounding.
 */
lf_status lf_attn_forward_global_proj(lf_attn_t h, const void* q, const void* k, const void* v,
                                      const void* q_g, const void* k_g, const void* v_g, void* out,
                                      int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                                      const int32_t* global_idx, int n_global,
                                      const uint8_t* key_pad_mask, void* stream);

/*
 * lf_attn_forward_global_proj that also writes each row's log-sum-exp, as
 * lf_attn_forward_lse does: lse[b,h,i] = log sum_j exp(score_ij) over the row's own
 * key set and scores, which for a global row are Q_g . K_g / sqrt(d_h) over every
 * unpadded key (up to i in the causal mode).  lse: DEVICE float32 [B][H][L], 4-byte
 * aligned, overlapping no input and not `out`; -inf for rows without keys.  The
 * statistics lf_attn_backward_global_proj needs.
 */
lf_status lf_attn_forward_global_proj_lse(lf_attn_t h, const void* q, const void* k, const void* v,
                                          const void* q_g, const void* k_g, const void* v_g, void* out,
                                          float* lse, int B, int H, int L, int d_h, int w,
                                          const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                                          const uint8_t* key_pad_mask, void* stream);

/*
 * Backward of lf_attn_forward_global_proj: the gradients of both projections.
 *
 * A row outside the global set attends with q, k, v (its key set as in
 * lf_attn_forward), which gives dq of that row and dk, dv of its keys (global keys
 * included); a global row attends every unpadded key (only the keys up to itself in
 * the causal mode) with q_g, k_g, v_g (page "基于Block-Sparse Attention的Longformer"
 * §4: global attention has its own projections), which gives dq_g of that row and
 * dk_g, dv_g of every key.  dq of a global row and dq_g of any other row are written
 * as zero; dk_g, dv_g of padded keys are zero.
 *
 * q_g, k_g, v_g : DEVICE [B][H][L][d_h] of the handle's dtype, as passed to the forward.
 * dq_g, dk_g, dv_g : DEVICE [B][H][L][d_h] outputs of the handle's dtype, 16-byte aligned, overlapping
 *                    no input and no other gradient.
 * out and lse: as returned by lf_attn_forward_global_proj_lse for the same inputs
 * (not lse from lf_attn_forward_lse: the global rows' normaliser differs).
 * Everything else, including the handle's settings (window mode, global mode,
 * position bias and random blocks, which reach only the other rows), as
 * lf_attn_backward.  One more launch than lf_attn_backward (dk_g, dv_g).
 */
lf_status lf_attn_backward_global_proj(lf_attn_t h, const void* q, const void* k, const void* v,
                                       const void* q_g, const void* k_g, const void* v_g, const void* out,
                                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                       void* dq_g, void* dk_g, void* dv_g, int B, int H, int L, int d_h, int w,
                                       const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                                       const uint8_t* key_pad_mask, void* stream);

/*
 * Pattern variant of every later call on `h` (forward, forward_lse,
 * forward_global_proj, forward_global_proj_lse, backward, backward_global_proj).
 *
 * LF_WINDOW_SYMMETRIC (default): the pattern above.
 * LF_WINDOW_CAUSAL: the same key sets intersected with {j <= i}: window keys
 *   i - m*dil for m = 0..w, global keys g <= i, and a global row sees the keys
 *   j <= g.  This is the pattern of autoregressive language modelling, which page
 *   "基于自注意力机制的长文本建模算法：Longformer详解" §6 lists among the
 *   pretraining tasks; the pages give no rule of their own for it.
 * Errors: LF_ERR_INVALID_ARG (h == NULL or unknown mode); the mode is unchanged.
 */
lf_status lf_attn_set_window_mode(lf_attn_t h, int mode);

/*
 * Relative position bias on the window scores of every later call on `h`
 * (forward, forward_lse, forward_global_proj, forward_global_proj_lse, backward,
 * backward_global_proj, layer).
 *
 * Page "基于自注意力机制的长文本建模算法：Longformer详解" §5 adds a relative
 * position bias to strengthen the local attention.  Read as a learned scalar per
 * head and window offset: a pair (i, j = i + m*dil_h) that row i attends through
 * its window (i not global, |m| <= w; m <= 0 in the causal mode) scores
 *     S_ij = q_i . k_j / sqrt(d_h) + table[h][m + w];
 * pairs that enter through the global pattern (global rows; global keys outside
 * the row's window) get no bias.  A global key inside the window is a window pair.
 *
 * table   : DEVICE fp32 [n_heads][2*w + 1], 4-byte aligned, caller-owned; it is
 *           borrowed, not copied: it must stay valid and unchanged while calls on
 *           `h` that use it are in flight.  NULL removes the bias (n_heads and w
 *           are then ignored).
 * n_heads : 1 .. LF_MAX_HEADS; every later call must pass H == n_heads.
 * w       : 0 .. LF_MAX_BIAS_W; every later call must pass the same w.
 * The backward returns dQ, dK and dV with the bias held fixed (no gradient of
 * the table).  Errors: LF_ERR_INVALID_ARG (h == NULL, n_heads out of range,
 * misaligned table), LF_ERR_UNSUPPORTED (w > LF_MAX_BIAS_W); the setting is then
 * unchanged.  A later call with another H or w fails with LF_ERR_INVALID_ARG.
 */
lf_status lf_attn_set_position_bias(lf_attn_t h, const float* table, int n_heads, int w);

/*
 * Random key blocks (BigBird-style random attention) for every later call on `h`
 * (forward, forward_lse, forward_global_proj, forward_global_proj_lse, backward,
 * backward_global_proj, layer).
 *
 * The survey page (commentary on "Efficient Transformers: A Survey", §3.1-§3.2)
 * describes BigBird as window + global + random attention and recommends fixed
 * draws for repeatable inference; the draws are therefore inputs.  Positions are
 * grouped in blocks of LF_RANDOM_BLOCK: a non-global row i also attends every key of
 * the key blocks [64*kb, 64*kb + 64) that its query block i / 64 drew, in the union
 * with its window and the global keys (a key reached several ways counts once);
 * padded keys stay masked, and in the causal mode keys after the row are dropped.
 *
 * blocks    : HOST int32 [n_heads][n_qblocks][r], copied during the call (the
 *             caller may free it on return); entry kb < 0 is unused, duplicates
 *             count once, 0 <= kb < n_qblocks otherwise.  NULL removes the draws.
 * n_heads   : 1 .. LF_MAX_HEADS; later calls must pass H == n_heads.
 * n_qblocks : ceil(L / LF_RANDOM_BLOCK) of the later calls (they must match).
 * r         : 0 .. LF_MAX_RANDOM_DRAWS draws per query block.
 * Later calls must have every head undilated (LF_ERR_UNSUPPORTED otherwise).  The
 * library keeps a device copy of the tables, uploaded (synchronously, after a
 * device-wide synchronisation) by the first call after this one on each device, so
 * that first call cannot be captured in a graph.  Do not call this while calls on
 * `h` are in flight.  Errors: LF_ERR_INVALID_ARG (h == NULL, sizes out of range,
 * an entry >= n_qblocks), LF_ERR_UNSUPPORTED (r > LF_MAX_RANDOM_DRAWS); the setting
 * is then unchanged.
 */
lf_status lf_attn_set_random_blocks(lf_attn_t h, const int32_t* blocks, int n_heads, int n_qblocks, int r);

/*
 * One Longformer layer around the attention (bf16 handles only):
 *
 *   q, k, v = split_heads(x W_qkv^T + b_qkv)     (rows of W_qkv: q, then k, then v;
 *                                                 head h = features 64h .. 64h+63)
 *   a       = merge_heads(attention(q, k, v))    (this library's forward, with the
 *                                                 handle's window mode and
 *                                                 position bias)
 *   x1      = LayerNorm1(x + a W_o^T + b_o)
 *   out     = LayerNorm2(x1 + GELU(x1 W_1^T + b_1) W_2^T + b_2)
 *
 * LayerNorm over the features with the biased variance and eps = ln_eps;
 * GELU(t) = 0.5 t (1 + erf(t / sqrt(2))).  The order of the steps is the layer of
 * page "基于Block-Sparse Attention的Longformer" §6 (attention, residual, LayerNorm,
 * feed-forward, residual, LayerNorm); the projections and the GELU feed-forward are
 * RoBERTa's, whose weights page "基于自注意力机制的长文本建模算法：Longformer详解"
 * §6 says Longformer starts from.
 *
 * x, out : DEVICE bf16 [B][L][hidden], 16-byte aligned, not overlapping.
 * wts    : HOST struct of DEVICE bf16 pointers (16-byte aligned), nn.Linear layout
 *          (weight [out][in]): w_qkv [3*hidden][hidden], b_qkv [3*hidden],
 *          w_o [hidden][hidden], b_o, ln1_g, ln1_b [hidden], w_1 [ffn][hidden],
 *          b_1 [ffn], w_2 [hidden][ffn], b_2, ln2_g, ln2_b [hidden].
 * hidden : 64 * heads, heads <= LF_MAX_HEADS, hidden <= 2048.
 * ffn    : feed-forward width, a positive multiple of 8.
 * w, dil_per_head (one per head), global_idx, n_global, key_pad_mask [B][L]: as
 * lf_attn_forward.
 * GEMMs run in hipBLASLt (bf16 inputs, fp32 accumulation; the QKV and first
 * feed-forward outputs in bf16, the two outputs that feed a LayerNorm in fp32;
 * b_qkv is added in the QKV GEMM's epilogue, the other biases in fp32 by the
 * pointwise passes; the algorithm is hipBLASLt's first heuristic choice, fixed per
 * shape at its first call on the handle).  The attention reads q, k, v where the QKV
 * GEMM leaves them (row stride 3 * hidden) and writes its output with the heads
 * merged (row stride hidden), so no pass splits or merges heads.  The handle owns a
 * hipBLASLt handle, a 32 MiB GEMM workspace and a device workspace for the
 * intermediates (max(6 * hidden, 2 * ffn) + 2 * hidden + 2 * ffn bytes per token).  Errors: as lf_attn_forward; LF_ERR_UNSUPPORTED for fp32 handles or
 * unsupported sizes.
 */
typedef struct lf_layer_weights {
    const void* w_qkv;
    const void* b_qkv;
    const void* w_o;
    const void* b_o;
    const void* ln1_g;
    const void* ln1_b;
    const void* w_1;
    const void* b_1;
    const void* w_2;
    const void* b_2;
    const void* ln2_g;
    const void* ln2_b;
} lf_layer_weights;

lf_status lf_layer_forward(lf_attn_t h, const void* x, const lf_layer_weights* wts, void* out, int B, int L,
                           int hidden, int ffn, float ln_eps, int w, const int32_t* dil_per_head,
                           const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                           void* stream);

/*
 * How every later call on `h` reads `global_idx`.
 *
 * LF_GLOBALS_SHARED (default): global_idx[n_global], one set for every sequence
 *   and head; every entry must lie in [0, L).
 * LF_GLOBALS_PER_SEQUENCE: global_idx[B][n_global] (HOST, row-major): row b is
 *   the set of sequence b; negative entries are unused; other entries must lie in
 *   [0, L); duplicates are ignored.  B * n_global <= LF_MAX_GLOBALS
 *   (LF_ERR_UNSUPPORTED otherwise).  Different documents mark different tokens
 *   global (a question of its own length in each, page
 *   "基于自注意力机制的长文本建模算法：Longformer详解" §7), which one shared set
 *   cannot express.
 * Errors: LF_ERR_INVALID_ARG (h == NULL or unknown mode); the mode is unchanged.
 */
lf_status lf_attn_set_global_mode(lf_attn_t h, int mode);

/*
 * Query rows per work-group of the forward kernels (a tuning setting; results agree
 * within rounding either way).  rows = 128: four waves of 32 rows each.  rows = 64:
 * two 32-row blocks, each computed by two waves that take alternate 32-key sub-tiles
 * of every staged tile of keys and merge their partial softmax states (each part's
 * largest score, weight sum and weighted values rescaled to the larger of the two),
 * i.e. twice the waves for the same rows.  rows = 0
 * (the default): 64 when the 128-row grid (B * H * tiles) would fill at most half of
 * the device's work-group slots (three bf16 or one fp32 work-group per compute unit),
 * else 128.  The 64-row form has no variant with a position bias, random blocks or
 * strided tensors (the layer's in-place attention); those always use 128.  The
 * backward keeps its own 128-row tiling.
 * Errors: LF_ERR_INVALID_ARG (h == NULL, or rows not 0, 64 or 128); the setting is
 * unchanged.
 */
lf_status lf_attn_set_tile_rows(lf_attn_t h, int rows);

/* Free the handle and its device workspace.  NULL is a no-op.  Waits for the
 * device before freeing (hipFree semantics). */
lf_status lf_attn_destroy(lf_attn_t h);

/* Static description of a status code. */
const char* lf_attn_status_string(lf_status s);

/* Message of the last failed call on `h` ("" if none); valid until the next call on h. */
const char* lf_attn_last_error(lf_attn_t h);

/*
 * Per-stage kernel timing with HIP events on the launch stream: each kernel of this
 * library is launched with hipExtLaunchKernel and a pair of events that it stamps with
 * the kernel's own start and end; the layer's library GEMMs are bracketed by two
 * recorded events.  enable != 0 starts recording (clearing earlier totals), 0 stops.
 * Errors: LF_ERR_INVALID_ARG (h == NULL), LF_ERR_HIP.
 */
lf_status lf_attn_set_stage_timing(lf_attn_t h, int enable);

/*
 * Wait for every recorded event, then write the summed milliseconds and the
 * number of timed launches per stage (arrays of LF_N_STAGES entries; either may
 * be NULL) and clear the totals.
 */
lf_status lf_attn_stage_times(lf_attn_t h, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LF_ATTN_H */
