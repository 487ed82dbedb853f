/*
 * lighthouse.h -- C ABI of the MI355X (gfx950) Lighthouse attention library.
 *
 * Lighthouse attention replaces causal scaled-dot-product attention on one
 * head-batch by four stages ("Long Context Pre-Training with Lighthouse
 * Attention", Sec. 3.2):
 *   (i)   mean-pool Q, K and V alike into an L-level pyramid with factor p
 *         (Sec. 3.3: window W_i^(l) = [i p^l, (i+1) p^l - 1], p^(L-1) | N);
 *   (ii)  score every entry with per-head l2 norms (QK: ||Q||, KQ: ||K||), coarser
 *         levels max-pooling the level-0 scores, and select jointly over both
 *         streams and all levels (Sec. 3.4); the coarsest level is always kept;
 *   (iii) gather the selected (Q, K, V) triples, sorted topologically by window
 *         end, into a contiguous sub-sequence of length S and run plain causal
 *         softmax attention over it (Sec. 3.5, Eq. 8 and Eq. 9);
 *   (iv)  scatter each entry's output to the p^l base positions of its window
 *         shifted by p^l - 1, summing the levels (Sec. 3.6), in deterministic
 *         int64 fixed point (32 fractional bits, round-to-nearest-even).
 * Selection budget: B = min((L-1) p k, |E|) distinct entries of the non-coarsest
 * levels E, ranked by max(QK, KQ) with ties to the lowest stream index (QK score
 * of flat entry f has stream index f, its KQ score |P| + f; flat index runs
 * level-major, finest first).  S = N / p^(L-1) + B.
 *
 * Conventions for every entry point:
 *  - Tensors are [B, H, N, d] contiguous (d fastest), heads independent.  All
 *    pointers are DEVICE pointers unless stated otherwise, 16-byte aligned.
 *  - The caller owns and allocates every buffer; the library allocates, frees
 *    and synchronises nothing.  Calls only enqueue work on `stream` (0 = the
 *    null stream) and return; results are ready when the stream reaches them.
 *  - Arguments are validated on the host before anything is enqueued: a call
 *    that returns an error status has no side effects.  lh_last_error() then
 *    gives a thread-local description.
 *  - Inputs must be finite (NaN or Inf give undefined selections).
 *  - Supported: d in {64, 128}; io dtype LH_F32 or LH_BF16 (bf16 storage, fp32
 *    arithmetic, bf16 MFMA for the attention); L >= 1; p >= 2; topk >= 0.
 *    topk larger than the candidates selects everything (S = |P|).
 *  - No global mutable state except the thread-local error text, the
 *    thread-local stage timing switch (lh_timing_begin), and the fixed scratch
 *    array of lh_attention_backward_noalloc (with its per-GPU address, looked up
 *    once): calls are re-entrant; concurrent calls on different streams must use
 *    distinct buffers (and lh_attention_backward_noalloc calls on one GPU must
 *    not overlap).
 */
#ifndef LIGHTHOUSE_H
#define LIGHTHOUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  The two range enumerators are not dtypes: they make every
 * 32-bit int a value of lh_dtype, so that an invalid dtype argument from a C
 * caller is an ordinary value that validation rejects with LH_EINVAL rather than
 * undefined behaviour in the C++ implementation. */
typedef enum {
  LH_F32 = 0,
  LH_BF16 = 1,
  LH_DTYPE_RANGE_MIN = -2147483647 - 1,
  LH_DTYPE_RANGE_MAX = 2147483647
} lh_dtype;

typedef enum {
  LH_OK = 0,
  LH_EINVAL = 1,        /* null / misaligned pointer, non-positive size, bad enum */
  LH_EDIVIS = 2,        /* p^(L-1) does not divide N */
  LH_EUNSUPPORTED = 3,  /* d not in {64, 128}, or sizes beyond int32 indexing */
  LH_EWORKSPACE = 4,    /* saved or workspace buffer smaller than lh_query says */
  LH_EHIP = 5           /* a HIP launch failed; see lh_last_error() */
} lh_status;

/* Byte offsets of the arrays inside the `saved` buffer that lh_forward fills
 * and lh_backward reads.  "BH" = B*H heads; P = pyramid entries per head;
 * S = gathered length per head.  Exposed so tests can read intermediates. */
typedef struct lh_saved_layout_t {
  size_t scores;   /* fp32  [BH][2][P]  QK stream, then KQ stream (Sec. 3.4) */
  size_t flags;    /* uint8 [BH][P]     1 = entry is in the index set I */
  size_t slot;     /* int32 [BH][P]     position in the sub-sequence, -1 if not selected */
  size_t coords;   /* int32 [BH][S]     flat pyramid index of the entry at each slot */
  size_t qt;       /* io    [BH][Sv][d] gathered Q~ (topological order); head stride Sv = S
                            rounded up to a multiple of 64, rows S..Sv-1 zero */
  size_t kt;       /* io    [BH][Sv][d] gathered K~; rows S..Sv-1 zero */
  size_t vt;       /* io    [BH][Sv][d] gathered V~; rows S..Sv-1 zero */
  size_t ot;       /* fp32  [BH][S][d]  sub-sequence attention output O~ */
  size_t lse;      /* fp32  [BH][S]     natural-log log-sum-exp of each O~ row's logits */
  size_t total;    /* bytes needed */
  int64_t P;       /* pyramid entries per head */
  int64_t E;       /* candidate (non-coarsest) entries per head */
  int64_t Bsel;    /* selected candidates per head */
  int64_t S;       /* gathered length per head */
  int64_t Sv;      /* rows per head of qt, kt, vt: S rounded up to a multiple of 64 */
} lh_saved_layout_t;

/* Host-only.  Validates the shape and returns S and the byte sizes the caller
 * must allocate: `saved` (forward -> backward state), and the forward and
 * backward workspaces.  Any output pointer may be NULL.  (Sec. 3.3, 3.5.) */
lh_status lh_query(int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io,
                   int64_t *S, size_t *saved_bytes, size_t *fwd_ws_bytes, size_t *bwd_ws_bytes);

/* Host-only.  Offsets of the arrays inside `saved` for this shape. */
lh_status lh_saved_layout(int B, int H, int64_t N, int d, int L, int p, int64_t topk,
                          lh_dtype io, lh_saved_layout_t *out);

/* Forward of the Lighthouse layer (Sec. 3.2, stages i-iv).
 *   q, k, v : [B,H,N,d] in dtype `io` (read only).
 *   o       : [B,H,N,d] output in dtype `o_dtype` (LH_F32 or LH_BF16); positions
 *             with no selected contributor (t < p^(L-1) - 1 not covered by a
 *             selected finer entry) are written as 0.
 *   saved   : >= saved_bytes from lh_query; filled for lh_backward (layout above).
 *   ws      : >= fwd_ws_bytes from lh_query; scratch, contents undefined after.
 * Deterministic: equal inputs give bit-equal outputs. */
lh_status lh_forward(const void *q, const void *k, const void *v, void *o, lh_dtype o_dtype,
                     int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io,
                     void *saved, size_t saved_bytes, void *ws, size_t ws_bytes, void *stream);

/* Backward of the Lighthouse layer with the forward's selection frozen: the
 * indices carry no gradient and nothing flows into the scores (Sec. 3.2).
 *   dout       : [B,H,N,d] upstream gradient in dtype `dout_dtype`.
 *   saved      : the buffer filled by lh_forward for the same q, k, v and shape.
 *   dq, dk, dv : [B,H,N,d] gradients in dtype `grad_dtype` (overwritten).
 *   ws         : >= bwd_ws_bytes from lh_query.
 * Deterministic (no floating-point atomics). */
lh_status lh_backward(const void *q, const void *k, const void *v, const void *dout,
                      lh_dtype dout_dtype, const void *saved, size_t saved_bytes,
                      void *dq, void *dk, void *dv, lh_dtype grad_dtype,
                      int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io,
                      void *ws, size_t ws_bytes, void *stream);

/* Dense causal softmax attention, softmax(Q K^T / sqrt(d) + causal) V, on given
 * [BH,S,d] tensors (Sec. 3.1, Eq. 1): the kernel of stage (iii), exposed for the
 * dense baseline at S = N.
 *   q, k, v : [BH][S][d] dtype `io` (read only).
 *   o       : [BH][S][d] fp32.   lse: [BH][S] fp32 (may be NULL).  */
lh_status lh_attention_forward(const void *q, const void *k, const void *v, float *o, float *lse,
                               int BH, int64_t S, int d, lh_dtype io, void *stream);

/* Backward of lh_attention_forward (Sec. 3.1 Eq. 1; Sec. 3.2): with P
 * recomputed from the forward's LSE, delta = rowsum(dO o O),
 *   dV = P^T dO,  dS = P o (dO V^T - delta),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
 *   q, k, v : [BH][S][d] dtype `io`, as given to lh_attention_forward.
 *   o, lse  : its outputs, [BH][S][d] and [BH][S] fp32 (lse non-NULL).
 *   dout    : [BH][S][d] dtype `io`.
 *   dq, dk, dv : [BH][S][d] fp32 (overwritten).
 *   ws      : >= 8*BH*S bytes (LH_BF16) or 4*BH*S bytes (LH_F32); contents undefined after.
 * LH_BF16 needs S to be a multiple of 64 (whole 64-row tiles), else LH_EUNSUPPORTED.
 * Deterministic (no floating-point atomics). */
lh_status lh_attention_backward(const void *q, const void *k, const void *v, const float *o, const float *lse,
                                const void *dout, float *dq, float *dk, float *dv, int BH, int64_t S, int d,
                                lh_dtype io, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * computation and kernels as lh_attention_backward (bit-identical results), but
 * with no workspace argument.  Its per-row scratch lives in a fixed array inside
 * the library (32 MiB per GPU, held from when the library is loaded until the
 * process ends), which bounds the rows: BH * S <= 4,194,304 in LH_BF16 (8 bytes
 * per row) or 8,388,608 in LH_F32 (4 bytes per row); larger shapes return
 * LH_EWORKSPACE before anything is enqueued.  The call allocates and frees
 * nothing; on its first use on a GPU it looks up that GPU's copy of the array
 * (hipGetSymbolAddress) and keeps the address.  Nothing in the array needs to
 * start at zero: the call writes every row it reads.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  Stage timing
 * records nothing for this call.  Other arguments and errors as
 * lh_attention_backward. */
lh_status lh_attention_backward_noalloc(const void *q, const void *k, const void *v, const float *o,
                                        const float *lse, const void *dout, float *dq, float *dk, float *dv, int BH,
                                        int64_t S, int d, lh_dtype io, void *stream);

/* ---- Projection-inclusive layer ----
 * The attention layer of the decoder the pages train, around the Lighthouse
 * attention (Sec. 3.1: Q, K, V in R^{N x d} are the per-head projections
 * X W_Q, X W_K, X W_V of the layer input X in R^{N x d_model}; Sec. 3.2: the
 * gradient reaches W_Q, W_K, W_V through the scatter, the sub-sequence attention
 * and the gather; the selection stays frozen).  The output projection W_O is that
 * of the Llama-3-style attention block (experiments: d_model = 1024, 8 heads,
 * head dimension 128):
 *   Q_h = X W_Q[:, h d:(h+1) d]  (likewise K_h, V_h),   O_h = Lighthouse(Q_h, K_h, V_h),
 *   Y = [O_0 | ... | O_{H-1}] W_O.
 * Layouts: x, y, dy, dx [B][N][d_model]; wq, wk, wv [d_model][H d] (head h =
 * columns h d .. h d + d - 1); wo [H d][d_model]; all row-major.  x, the weights
 * and dy are in the io dtype.  The products run on bf16 MFMA with fp32
 * accumulation (LH_BF16) or in fp32 on the vector ALUs (LH_F32).  d_model must be
 * a multiple of 64.  Conventions as above (caller-owned buffers, validation
 * first, only enqueues on `stream`).  The backward's weight gradients sum over
 * every token of the batch with a fixed split and a fixed summation order:
 * deterministic. */
typedef struct lh_layer_layout_t {
  size_t q, k, v;     /* io [B][H][N][d] projected Q, K, V (the Lighthouse inputs)        */
  size_t o;           /* io [B][H][N][d] Lighthouse output O (the input of W_O)           */
  size_t inner;       /* the lh_forward `saved` buffer of the attention (lh_saved_layout) */
  size_t inner_bytes; /* its size                                                         */
  size_t total;       /* bytes needed                                                     */
} lh_layer_layout_t;

/* Host-only.  Validates the layer shape; returns S and the byte sizes of the
 * layer's `saved` buffer and of its forward and backward workspaces. */
lh_status lh_layer_query(int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk, lh_dtype io,
                         int64_t *S, size_t *saved_bytes, size_t *fwd_ws_bytes, size_t *bwd_ws_bytes);

/* Host-only.  Offsets inside the layer's `saved` buffer. */
lh_status lh_layer_saved_layout(int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk,
                                lh_dtype io, lh_layer_layout_t *out);

/* Forward of the layer: projections, Lighthouse attention of every head, output
 * projection.  y in dtype y_dtype (LH_F32 or LH_BF16).  saved: >= saved_bytes of
 * lh_layer_query, filled for lh_layer_backward.  ws: >= fwd_ws_bytes. */
lh_status lh_layer_forward(const void *x, const void *wq, const void *wk, const void *wv, const void *wo, void *y,
                           lh_dtype y_dtype, int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk,
                           lh_dtype io, void *saved, size_t saved_bytes, void *ws, size_t ws_bytes, void *stream);

/* Backward of the layer for upstream gradient dy (io dtype): dx in dx_dtype
 * (LH_F32 or LH_BF16); dwq, dwk, dwv [d_model][H d] and dwo [H d][d_model] in
 * fp32 (overwritten).  saved: the buffer lh_layer_forward filled for the same
 * x and weights.  ws: >= bwd_ws_bytes of lh_layer_query. */
lh_status lh_layer_backward(const void *x, const void *wq, const void *wk, const void *wv, const void *wo,
                            const void *dy, const void *saved, size_t saved_bytes, void *dx, lh_dtype dx_dtype,
                            float *dwq, float *dwk, float *dwv, float *dwo, int B, int H, int64_t N, int d_model,
                            int d, int L, int p, int64_t topk, lh_dtype io, void *ws, size_t ws_bytes, void *stream);

/* Stages of lh_forward / lh_backward (and of the layer entry points), for stage timing. */
typedef enum {
  LH_STAGE_POOL_SCORE = 0,   /* (i)+(ii): pyramid and scores, one pass over Q, K, V          */
  LH_STAGE_TOPK = 1,         /* (ii): joint top-B selection (histogram, filter, refine passes) */
  LH_STAGE_GATHER = 2,       /* (iii): topological compaction and gather                      */
  LH_STAGE_ATTN_FWD = 3,     /* (iii): causal attention over the sub-sequence (Eq. 9)         */
  LH_STAGE_SCATTER = 4,      /* (iv): scatter to the base positions                           */
  LH_STAGE_SCATTER_BWD = 5,  /* adjoint of (iv): dO~ and the softmax row terms               */
  LH_STAGE_ATTN_BWD_DQ = 6,  /* adjoint of Eq. 9: dQ~                                         */
  LH_STAGE_ATTN_BWD_DKDV = 7,/* adjoint of Eq. 9: dK~, dV~                                    */
  LH_STAGE_POOL_BWD = 8,     /* adjoint of the gather and of the pooling: dQ, dK, dV          */
  LH_STAGE_PROJ = 9,         /* layer: Q, K, V = X W_Q, X W_K, X W_V                           */
  LH_STAGE_OUT_PROJ = 10,    /* layer: Y = O W_O                                               */
  LH_STAGE_OUT_PROJ_BWD = 11,/* layer: dO = dY W_O^T and dW_O = O^T dY                         */
  LH_STAGE_PROJ_BWD = 12,    /* layer: dX = dQ W_Q^T + dK W_K^T + dV W_V^T and dW_Q, dW_K, dW_V */
  LH_STAGE_COUNT = 13
} lh_stage;

/* Host-only.  Short name of a stage ("attn_bwd_dkdv", ...; static storage). */
const char *lh_stage_name(int stage);

/* Host-only.  Stage timing, for benchmarks (not part of the compute path).
 * lh_timing_begin switches timing on for the calling host thread and drops
 * any earlier records.  While it is on, lh_forward, lh_backward and the layer
 * entry points bracket the
 * kernel launches of each stage with a pair of HIP events recorded on the
 * call's stream -- the only time the library creates anything.
 * lh_timing_end switches it off, waits for the recorded events, and writes for
 * each stage s < n the summed elapsed milliseconds ms[s] and the number of
 * bracketed spans spans[s]; stages >= n are dropped.  It releases the events.
 * Returns LH_EHIP (after filling what it could) if an event fails. */
lh_status lh_timing_begin(void);
lh_status lh_timing_end(double *ms, int *spans, int n);

/* Text of a status code (static storage). */
const char *lh_status_string(lh_status s);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *lh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTHOUSE_H */
