/*
 * monarch_attn.h -- C ABI of the MonarchAttention forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * MonarchAttention replaces softmax attention softmax(scale * Q K^T) V by a
 * Monarch matrix M = P^T L P R (L, R block diagonal; in block form every
 * block of M is rank one) fitted by alternating maximisation of the softmax
 * variational objective f(M) = sum over rows of <M_row, S_row> + H(M_row),
 * S = scale * Q K^T, for `steps` steps, without forming the N x N matrix;
 * then Y = M V is applied as two batched block contractions, at
 * Theta(N sqrt(N) d) compute and Theta(N d) IO.
 *   Sources: "MonarchAttention: Zero-Shot Conversion to Fast, Hardware-Aware
 *   Structured Attention" (abstract; scime atlas summary "Proposal" and
 *   "Approach"; OpenReview reviews and author responses on the objective,
 *   its concavity, the positivity constraints, T and the block sizes).
 * The tiled variant splits every Monarch block into c1 x c2 independently
 * rank-one sub-tiles, and the video layouts choose the block grid so that
 * each of the f, h, w axes of a video latent lies in one factor.
 *   Source: "MonarchRT: Efficient Attention for Real-Time Video Generation",
 *   summary page, "Key claims" (section 4.1, Theorem 4.1) and "Method".
 *
 * Grid and factors (per (batch, head) slice).  Token n sits at grid position
 * (l, i), l in [b1] (block), i in [b2] (position in block); for the flat
 * layout n = l*b2 + i.  With t(l) = floor(l*c1/b1), s(j) = floor(j*c2/b2):
 *     M[(l,i),(k,j)] = L[i,l,k,s(j)] * R[k,i,t(l),j]
 * Rows of R sum to one over each segment s, rows of L over (k, s).
 * Updates (exact block-wise maximisers of f):
 *     R[k,i,t,j in s] = softmax_j( scale * qt[k,i,t,s] . k[k,j] )
 *     L[i,l,k,s]      = softmax_(k,s)( scale * q[l,i] . c[k,i,t(l),s] + H_R[k,i,t(l),s] )
 *     c = sum_j R k,  u = sum_j R v,  H_R = entropy of the R segment,
 *     qt = sum_(l in t) L q / sum_(l in t) L     (steps 2..T),
 *     y[l,i] = sum_(k,s) L[i,l,k,s] u[k,i,t(l),s].
 * Initialisation: L0 = block identity, so qt[k,i,t(k),s] = q[k,i]; sub-rows
 * with t != t(k) (zero weight) use the mean of q[l,i] over the rows l of
 * tile t.
 *
 * Conventions
 * -----------
 * All tensor arguments are DEVICE pointers on the current HIP device.
 * Q, K, V, Y: [batch, heads, seq_len, head_dim], contiguous, element type
 * `dtype`; accumulation is always fp32.  The caller owns every buffer; the
 * library never allocates, frees or synchronises (except the diagnostic
 * helpers marked so), keeps no pointer after return and holds no mutable
 * global state.  Work is enqueued asynchronously on `stream` (a hipStream_t;
 * NULL = the default stream).  Calls on one stream are ordered; calls that
 * share a workspace must not overlap.
 *
 * Errors: every argument check runs on the host before any HIP call and
 * returns a status with nothing launched.  A launch failure returns
 * MA_ERR_DEVICE.  No exceptions cross the ABI.  NaN/Inf in the inputs
 * propagate to the outputs (not checked).
 */
#ifndef MONARCH_ATTN_H
#define MONARCH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MA_OK = 0,
  MA_ERR_INVALID_ARGUMENT = 1,   /* shapes inconsistent, null or misaligned pointer, aliasing */
  MA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (head_dim, dtype, segment width) */
  MA_ERR_WORKSPACE_TOO_SMALL = 3,
  MA_ERR_DEVICE = 4              /* a HIP call or kernel launch failed */
} ma_status;

typedef enum { MA_F32 = 0, MA_BF16 = 1 } ma_dtype;

/* Token order -> (b1, b2) grid.  FLAT: n = l*b2 + i.  The video layouts take
 * a row-major f x h x w latent; the name lists the axes of b1 then of b2, in
 * major-to-minor order within each factor (MonarchRT summary page, "Key
 * claims": the six aligned block-size choices). */
typedef enum {
  MA_LAYOUT_FLAT = 0,
  MA_LAYOUT_FH_W = 1,   /* b1 = f*h, b2 = w */
  MA_LAYOUT_W_FH = 2,   /* b1 = w,   b2 = f*h */
  MA_LAYOUT_F_HW = 3,   /* b1 = f,   b2 = h*w */
  MA_LAYOUT_HW_F = 4,   /* b1 = h*w, b2 = f */
  MA_LAYOUT_FW_H = 5,   /* b1 = f*w, b2 = h */
  MA_LAYOUT_H_FW = 6    /* b1 = h,   b2 = f*w */
} ma_layout;

/* Execution-path flags (ma_problem.flags). */
/* T = 1 runs either as separate stage launches or as one cooperative launch
 * (grid-wide barriers between the phases).  The library picks the staged
 * sequence unless MA_FLAG_FORCE_FUSED is set; FORCE_STAGED wins over it. */
#define MA_FLAG_FORCE_STAGED 1u
#define MA_FLAG_FORCE_FUSED 4u
/* Precision of the aggregate c = R K (bf16 only).  Split: R enters R K as
 * bf16 hi + lo parts, c is exchanged as two bf16 planes hi + lo and the
 * next-step queries stay fp32 (about 16 significant bits on that path).
 * Plain: bf16 R and a bf16 c (fewer MFMAs, half the bytes for c).  Errors
 * on the c path grow with the number of steps (c feeds the next queries), so
 * the default is plain for T = 1 and split for T > 1; the flags force one or
 * the other (PRECISE wins over FAST). */
#define MA_FLAG_FAST_AGGREGATE 2u
#define MA_FLAG_PRECISE_AGGREGATE 8u
/* Padding of a flat sequence with seq_len < b1*b2 (MonarchAttention,
 * OpenReview author response on block sizes: b is chosen, m = ceil(N/b), and
 * the sequence is padded before -- as for ViT's leading class token -- or
 * after its tokens).  Default: after; this flag: before.  The P = b1*b2 -
 * seq_len padding positions are not tokens: the method fits the attention
 * among the real tokens only (R rows are softmaxes over real keys, padding
 * rows carry no L row and no output, the column sums for the next queries
 * and the tile means run over real rows; a padding position takes the tile
 * mean as its first-step query).  Requires P < b2 / c2, so that every key
 * segment holds a real key. */
#define MA_FLAG_PAD_FRONT 16u
/* Backward only, steps = 1: the workspace already holds the forward state of
 * these inputs (c, u, entropies and both normalisers), left there by a
 * monarch_attn_forward call of the same problem and inputs that was given
 * this workspace (at least monarch_attn_backward_workspace_size bytes); the
 * backward then skips rebuilding it, as a training step that keeps its
 * forward's state would.  The flag does not change the forward.  Returns
 * MA_ERR_UNSUPPORTED where the forward's state layout is not the backward's
 * (steps > 1, or a bf16 aggregate path other than the plain one). */
#define MA_FLAG_REUSE_FORWARD_STATE 32u

typedef struct {
  int64_t batch, heads, seq_len, head_dim;  /* Q, Y: [batch, heads, seq_len, head_dim];
                                               K, V: [batch, kv_heads, seq_len, head_dim] */
  int32_t b1, b2;      /* seq_len == b1*b2, or for FLAT b1*b2 - b2/c2 < seq_len <=
                          b1*b2 (padded, see MA_FLAG_PAD_FRONT); b1 = number of
                          blocks (the pages' m), b2 = block length (the pages' b) */
  int32_t c1, c2;      /* sub-tiles per block; 1,1 = untiled Monarch; c1 | b1, c2 | b2 */
  int32_t steps;       /* alternating-maximisation steps T >= 1 */
  float scale;         /* multiplies Q.K^T; 0 means 1/sqrt(head_dim) */
  int32_t dtype;       /* ma_dtype of Q, K, V, Y */
  int32_t layout;      /* ma_layout */
  int32_t f, h, w;     /* video latent (layout != FLAT): f*h*w == seq_len */
  uint32_t flags;      /* MA_FLAG_* */
  int32_t kv_heads;    /* heads of K and V; 0 means heads.  Grouped-query
                          attention: heads % kv_heads == 0 and query head h
                          uses K/V head h / (heads / kv_heads) (MonarchAttention
                          OpenReview author response on GQA/MLA: the method
                          applies per query head, stage 1 reading the shared
                          K/V of its group) */
  int32_t causal;      /* 0: bidirectional.  g >= 1: block-causal use, query
                          block l (grid row) attends to key block k iff
                          floor(k/g) <= floor(l/g), i.e. causally across
                          units of g consecutive grid blocks and fully inside
                          one.  On a flat sequence g = 1 is the usual
                          block-causal mask with blocks of b2 tokens; on the
                          (fh, w) video layout g = h (times frames per chunk)
                          is frame-causal.  The pages note that token-level
                          causal masking does not fit the method
                          (MonarchAttention, scime summary "Limitations") and
                          target autoregressive video models (MonarchRT,
                          summary page); a mask over whole blocks keeps every
                          block rank one: M and L are zero on masked blocks,
                          the objective runs over the allowed entries, the
                          L-update is a softmax over the allowed keys and the
                          R-update keeps its form.  g >= b1 masks nothing.
                          The backward differentiates the masked method
                          (masked L entries carry no gradient). */
} ma_problem;

/* Optional exports (device pointers, each may be NULL), always fp32/fp64.
 * L:   [batch, heads, b2, b1, b1*c2]    L[i][l][k*c2 + s] after the last step
 *                                       (grid positions; zero rows at padding,
 *                                       zero at blocks a causal mask removes)
 * R:   [batch, heads, b1, b2, c1, b2]   R[k][i][t][j]     after the last step
 * lse: [batch, heads, seq_len]          token order; logsumexp (natural log)
 *      of the last L-update's scores for each query row
 * objective: [batch*heads] fp64         f(L_T, R_T) = sum of lse over the slice */
typedef struct {
  float* L;
  float* R;
  float* lse;
  double* objective;
} ma_exports;

/* Current limits: head_dim in {64, 128}; segment width b2/c2 <= 128, except
 * <= 64 for fp32 with head_dim 128; any b1; batch*heads <= 2^24, b1*b2 <=
 * 2^26 and batch*heads*b1*b2*c1*c2 < 2^31.  Other shapes return
 * MA_ERR_UNSUPPORTED. */

/* Bytes of device workspace monarch_attn_forward needs for problem *p
 * (256-byte aligned start required).  Pure host function. */
ma_status monarch_attn_workspace_size(const ma_problem* p, size_t* bytes);

/* Y = MonarchAttention(Q, K, V).  exports may be NULL.  workspace must be at
 * least monarch_attn_workspace_size bytes, 256-byte aligned, and not overlap
 * any other argument.  Y must not overlap Q, K or V.  Q, K, V, Y must be
 * 16-byte aligned. */
ma_status monarch_attn_forward(const ma_problem* p, const void* q, const void* k,
                               const void* v, void* y, const ma_exports* exports,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Size of the library-owned device workspace of monarch_attn_forward_noalloc
 * (one array per GPU the library runs on, held until the process ends). */
#define MONARCH_ATTN_SCRATCH_BYTES (64u << 20)

/* monarch_attn_forward without a workspace argument and without allocating,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It runs
 * the same kernels as monarch_attn_forward, with the workspace taken from a
 * fixed device array of MONARCH_ATTN_SCRATCH_BYTES that the library holds
 * on every GPU it runs on (looked up on the first call on each device); it
 * calls no hipMalloc, hipFree or other allocating routine.  The caller still
 * passes Q, K, V, Y and the optional exports, with the same rules as
 * monarch_attn_forward.
 * Returns MA_ERR_WORKSPACE_TOO_SMALL, with nothing launched, for a problem
 * whose workspace (monarch_attn_workspace_size) exceeds
 * MONARCH_ATTN_SCRATCH_BYTES (the 12-head, 16384-token, head_dim 64 bf16
 * problem needs 53 MB and fits), and MA_ERR_UNSUPPORTED with
 * MA_FLAG_FORCE_FUSED (the cooperative launch's grid barrier keeps state of
 * the runtime's own).  The array keeps what the last call left; nothing in
 * it has to start at zero.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one device (other streams, other host threads)
 * race, and the caller must order them. */
ma_status monarch_attn_forward_noalloc(const ma_problem* p, const void* q, const void* k,
                                       const void* v, void* y, const ma_exports* exports,
                                       void* stream);

/* Number of kernel launches monarch_attn_forward makes for *p (host only),
 * or -1 for an invalid problem. */
int32_t monarch_attn_num_launches(const ma_problem* p);

/* Name of the j-th kernel launch for *p (static string) or NULL. */
const char* monarch_attn_launch_name(const ma_problem* p, int32_t j);

/* Diagnostic variant of monarch_attn_forward: events[2j] and events[2j+1]
 * take the start and end time stamps of kernel launch j, for 2j + 1 <
 * n_events (hipEvent_t created by the caller, e.g. with
 * monarch_attn_event_create).  They are recorded with the launch itself
 * (hipExtLaunchKernel), so nothing is queued between two launches; the
 * single-launch cooperative path records them just before and after its
 * launch.  Never synchronises. */
ma_status monarch_attn_forward_timed(const ma_problem* p, const void* q, const void* k,
                                     const void* v, void* y, const ma_exports* exports,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events, int32_t n_events);

/* Backward pass: dQ, dK, dV of <dY, Y> for Y = MonarchAttention(Q, K, V)
 * (Q, dY, dQ: [batch, heads, seq_len, head_dim] in the problem's dtype).
 * The pages train through the method (MonarchRT "Method" part (3): one-step
 * fine-tuning) without stating a backward; this is the exact gradient of
 * the forward's steps, computed by recomputing the forward's block softmaxes
 * from its normalisers (the forward state is rebuilt inside the call unless
 * MA_FLAG_REUSE_FORWARD_STATE says the workspace holds it).
 * dK, dV have K's shape [batch, kv_heads, seq_len, head_dim]; with grouped
 * K/V they sum over the query heads of each group.  A padded sequence
 * (MA_FLAG_PAD_FRONT or post-padding) routes the query gradient of a padding
 * position through the tile mean it used.  Covers b2 <= 128 (<= 64 for
 * fp32 with head_dim 128) with: steps = 1, with padding and with row tiles
 * and key segments c1, c2 (whose other-tile queries route their gradient
 * through the tile means of the real rows), also together; steps > 1 (the
 * gradient through every unrolled step, each step's L feeding the next
 * step's queries) with padding and with row tiles and key segments (also
 * together), and for bf16 at head_dim 128 b2 <= 64.  Block-causal use
 * (causal) at any of these.
 * Any b1: stage-2 columns longer than one key chunk are walked chunk by
 * chunk.  Other problems return MA_ERR_UNSUPPORTED.
 * With MA_FLAG_REUSE_FORWARD_STATE the forward state is read from the
 * workspace instead of rebuilt.  For bf16 the recomputed forward takes
 * the c path the forward defaults to (plain for steps = 1, split for
 * steps > 1), so these are its gradients.  A column whose next-step weights
 * all underflow to zero (the forward then takes the tile mean as the next
 * query) passes no gradient back through that query.
 * y: null, or the forward's output Y for these inputs (shaped like Q).  The
 * softmax gradient of every stage-2 row needs D = sum over keys of P dP,
 * which equals dY . y (at the last step when steps > 1); a column of more
 * than one key chunk (more than 128 keys; 64 for fp32 with head_dim 128 and
 * for bf16 with head_dim 128 and steps > 1) then takes D from y instead of
 * a separate pass over all its keys (as FlashAttention-2 does); elsewhere y
 * is not read.
 * With y the result is that of the given output; for bf16 it may differ from
 * the call without y by the rounding of y.
 * workspace: at least monarch_attn_backward_workspace_size bytes, 256-byte
 * aligned, overlapping no other argument; dQ, dK, dV must not overlap each
 * other or the inputs (y included); every tensor 16-byte aligned.  The
 * outputs are written, not accumulated. */
ma_status monarch_attn_backward_workspace_size(const ma_problem* p, size_t* bytes);
ma_status monarch_attn_backward(const ma_problem* p, const void* q, const void* k,
                                const void* v, const void* y, const void* dy, void* dq, void* dk,
                                void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic helpers around hipEvent_t (thin wrappers of the HIP runtime),
 * for timing only: the events are created with hipEventDisableSystemFence,
 * so recording one adds no system-scope cache writeback and invalidation
 * between the launches it separates (such a fence would be timed as part of
 * the next launch), and waiting on one does not make the device's writes
 * visible to the host (synchronise the stream for that).
 * monarch_attn_event_record records the event on a hipStream_t (null: the
 * default stream) and does not wait; monarch_attn_event_elapsed_ms waits
 * for event b. */
ma_status monarch_attn_event_create(void** event);
ma_status monarch_attn_event_destroy(void* event);
ma_status monarch_attn_event_record(void* event, void* stream);
ma_status monarch_attn_event_elapsed_ms(void* a, void* b, float* ms);

/* Static description of a status code. */
const char* monarch_attn_status_string(ma_status s);

/* Library version, e.g. "0.1.0". */
const char* monarch_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MONARCH_ATTN_H */
