/*
 * relpos.h -- C ABI of the MI355X (gfx950) exact relative-position attention
 * library.
 *
 * Method: "Fast and Exact Relative-Position Attention via Structure-Aware
 * Kernels" (arXiv 2611.01182), cited as [RPA].  The library computes, for
 * every (batch, head) slice, the score of [RPA] §3.2 Eq. (4),
 *
 *   S_ij = tau * ( (q_i + u) . k_j
 *                 + (q_i + v) . A^Q[phi_Q(i,j)] + k_j . A^K[phi_K(i,j)]
 *                 + b[phi_b(i,j)] ) + M_ij ,
 *
 * with u, v the two Transformer-XL query biases (zero when absent) and
 * M_ij = -inf for j > i under the causal mask, then P = softmax(S), O = P V
 * ([RPA] §3.1 Eq. (1)), and in backward every gradient of [RPA] App. B.1.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] with d = 64;
 *    device pointers, 16-byte aligned.
 *  - The relation offset is delta = i - j ([RPA] §4.1).  Table X in
 *    {A^Q, A^K, b} reads its map at sign_X * delta; sign -1 expresses the maps
 *    written in j - i (Shaw, T5, DeBERTa's position-to-content term).
 *  - The library never allocates or frees device memory and never
 *    synchronises: all work is enqueued on the HIP stream passed as `stream`
 *    (a hipStream_t; NULL is the default stream).  The caller owns every
 *    buffer and must keep them alive until that stream's work has finished.
 *  - Buffers `z` (retained projections) and `ws` (workspace) are opaque;
 *    their byte sizes come from relpos_plan_sizes().  256-byte alignment.
 *  - Return value: RELPOS_OK (0) or a negative RELPOS_E_* code.  No C++
 *    exception crosses the ABI.  relpos_last_error() gives a per-thread
 *    detail string for the last failing call on this thread.
 *  - Host arrays referenced by the descriptor are read during the call only.
 */
#ifndef RELPOS_H
#define RELPOS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RELPOS_ABI_VERSION 4

/* ---- return codes ---------------------------------------------------- */
#define RELPOS_OK 0
#define RELPOS_E_INVALID_ARG (-1)        /* null/inconsistent argument      */
#define RELPOS_E_UNSUPPORTED (-2)        /* e.g. head dim != 64             */
#define RELPOS_E_UNSUPPORTED_MAP (-3)    /* map rows outside the table      */
#define RELPOS_E_MISALIGNED (-4)         /* pointer / stride not 16-byte    */
#define RELPOS_E_WORKSPACE_TOO_SMALL (-5)
#define RELPOS_E_HIP (-6)                /* a HIP launch or copy failed     */
#define RELPOS_E_ABI (-7)                /* abi_version mismatch            */

/* ---- relation maps ([RPA] §3.2 "identity, clipped, bucketed") --------- */
#define RELPOS_MAP_IDENTITY 0   /* row = x + identity_offset                */
#define RELPOS_MAP_CLIPPED 1    /* row = clip(x, -clip, clip) + clip         */
#define RELPOS_MAP_T5_BUCKET 2  /* T5 buckets (num_buckets, max_distance,    */
                                /* bidirectional); x is T5's argument        */
#define RELPOS_MAP_LOG_BUCKET 3 /* DeBERTa-v3 log buckets (bucket_size,     */
                                /* max_position); row = clip(bkt(x)+bs,0,2bs-1) */
#define RELPOS_MAP_EXPLICIT 4   /* row = explicit_rows[clip(x,-clip,clip)+clip] */
/* Any map of the offset alone is accepted, including maps whose rows are not
   one interval of offsets (e.g. x and -x sharing a row, [RPA] "Atomic
   fallback"): the bucket copy gives every offset its own expanded row, and a
   table row's gradient is the fixed-order sum over its copies, so no atomics
   are needed for them either. */

/* ---- dtypes ------------------------------------------------------------ */
#define RELPOS_DTYPE_F32 0
#define RELPOS_DTYPE_BF16 1

/* ---- active terms of Eq. (4) ------------------------------------------- */
#define RELPOS_TERM_AQ 1    /* q_i . A^Q[phi_Q]   (content-to-position)      */
#define RELPOS_TERM_AK 2    /* k_j . A^K[phi_K]   (position-to-content)      */
#define RELPOS_TERM_BIAS 4  /* b[phi_b, h]        (scalar bias)              */
#define RELPOS_TERM_U 8     /* u_h . k_j          (Transformer-XL content bias) */
#define RELPOS_TERM_V 16    /* v_h . A^Q[phi_Q]   (Transformer-XL position bias; needs AQ) */

typedef struct relpos_map {
  int32_t kind;            /* RELPOS_MAP_*                                   */
  int32_t clip;            /* CLIPPED: clip; EXPLICIT: half width c          */
  int32_t identity_offset; /* IDENTITY                                       */
  int32_t num_buckets;     /* T5_BUCKET                                      */
  int32_t max_distance;    /* T5_BUCKET                                      */
  int32_t bidirectional;   /* T5_BUCKET (0/1)                                */
  int32_t bucket_size;     /* LOG_BUCKET                                     */
  int32_t max_position;    /* LOG_BUCKET                                     */
  const int32_t *explicit_rows; /* EXPLICIT: host array of 2c+1 rows         */
} relpos_map;

typedef struct relpos_desc {
  int32_t abi_version;     /* = RELPOS_ABI_VERSION                           */
  int32_t terms;           /* OR of RELPOS_TERM_*; at least one              */
  int32_t causal;          /* 0/1: mask j > i                                */
  float scale;             /* tau                                            */
  int32_t dtype;           /* inputs Q,K,V,dO, tables, u, v                  */
  int32_t out_dtype;       /* O, dQ, dK, dV                                  */
  int32_t num_rows;        /* R: rows of every relation table                */
  int32_t sign_q, sign_k, sign_b; /* +1 or -1 (see conventions)              */
  /* Precision of the probability and score-gradient operands of the MFMA
     products O = P V, dV = P^T dO, dQ = G K and dK = G^T Q (G = tau dS;
     bf16 inputs only, ignored for fp32): 0 = rounded once to bf16 (8
     significant bits, [RPA] "Half-precision numerics"); 1 = a bf16 pair
     hi + lo (about 16 significant bits; one more MFMA product each), for a
     strongly peaked softmax such as tau = 1 with unit-variance inputs, where
     an 8-bit P moves O, hence D = rowdot(dO, O), by more than 2^-9.
     The T5 mechanism at tau = 1 (bias as the only term, no 1/sqrt(d)) with
     unit-variance inputs needs 1 to stay within max-abs 2e-2 on O and every
     gradient; Shaw, DeBERTa and Transformer-XL meet it with 0. */
  int32_t split_operands;
  relpos_map map;
  /* Table layouts, in elements.  A^Q, A^K: element (r, h, e) at
     r*row_stride + h*head_stride + e (e < 64 contiguous).  head_stride 0
     shares one table across heads (A^Q only).  bias: element (r, h) at
     r*row_stride + h*head_stride.  The fp32 table gradients use the same
     strides. */
  int64_t aq_row_stride, aq_head_stride;
  int64_t ak_row_stride, ak_head_stride;
  int64_t bias_row_stride, bias_head_stride;
  /* Segment mask ([RPA] appendix "Masks, packing, and dropout": padding
     masks and packed variable-length sequences).  1: relpos_tensors.seg
     holds, for every token t of batch row b, the bounds [start, end) of
     its segment (int32 [B, N, 2], device memory, 8-byte aligned); a pair
     (i, j) is visible iff j lies in i's segment.  Every token of a segment
     must carry that segment's bounds; a padding token carries an empty
     segment (start = end).  One segment [0, L) per row is a padding mask of
     length L, several are packed sequences (offsets stay i - j).  A query
     with no visible key gets O = 0, L = -inf and zero gradients. */
  int32_t segmented;
  /* Attention dropout: a pair is dropped with probability dropout_p8 / 256
     (0..255; 0 = none) and kept probabilities are scaled by
     256 / (256 - dropout_p8).  The mask comes from Philox4x32-10 (Salmon
     et al., SC 2011) keyed by dropout_seed: counter (j >> 2, i >> 2,
     b H + h, 0), byte (j & 3) of word (i & 3), kept iff >= dropout_p8.  The
     backward regenerates the forward's mask from the same seed, so pass the
     same descriptor to both.  The seed is not part of the cached plan. */
  int32_t dropout_p8;
  uint64_t dropout_seed;
  /* In-tile relation products ([RPA] §6 "Limitations" and Table 7, row
     "Projections": the tiles compute their own relation products instead of
     reading stored projections).  1: no projection Z^Q is stored; every
     attention pass computes the products q_i . A~^Q[s] for the rows s its
     tile reaches on MFMA, from the expanded table, and the backward takes
     the table and bias gradients from an offset-parallel pass (one
     workgroup per block of 64 offsets sums its diagonals in a fixed order:
     deterministic, no atomics) instead of a stored offset-gradient buffer.
     Projection memory and workspace become O(N) per (batch, head) slice
     (identity maps such as Transformer-XL's otherwise store O(N^2)), at the
     cost of the per-tile products.  Requires bf16 inputs and the A^Q term;
     u, v, a scalar bias, segment masks and dropout may be present; the A^K
     term, and split_operands together with segment masks or dropout, are
     not supported with it (RELPOS_E_UNSUPPORTED).  relpos_project then
     stores only the per-token entries, the expanded bias and the expanded
     table (with its transpose), and the relpos_sizes figures shrink
     accordingly. */
  int32_t in_tile;
  int32_t reserved0;       /* must be 0                                      */
} relpos_desc;

/* Problem shape: B, H >= 1, 1 <= N <= 2^22, d = 64.  An empty problem (any
   of B, H, N zero) is refused with RELPOS_E_INVALID_ARG rather than treated
   as a no-op; N > 2^22 and d != 64 are RELPOS_E_UNSUPPORTED. */
typedef struct relpos_shape {
  int32_t B, H, N, d;
} relpos_shape;

/* Device pointers; unused terms may be NULL.  u and v are [H, 64].  seg:
   int32 [B, N, 2] segment bounds, read when desc->segmented (else NULL). */
typedef struct relpos_tensors {
  const void *q, *k, *v;
  const void *aq, *ak, *bias;
  const void *u, *vbias;
  const int32_t *seg;
} relpos_tensors;

/* Device pointers.  dq/dk/dv in out_dtype; table gradients fp32 with the
   tables' strides; du/dvbias fp32 [H, 64].  Every present gradient is
   overwritten (not accumulated). */
typedef struct relpos_grads {
  void *dq, *dk, *dv;
  float *daq, *dak, *dbias, *du, *dvbias;
} relpos_grads;

typedef struct relpos_sizes {
  size_t z_bytes;          /* retained projection buffer                     */
  size_t fwd_ws_bytes;     /* relpos_project workspace (relpos_attn_fwd with
                              retained z needs none: ws may be NULL)         */
  size_t fwd_ws_bytes_noz; /* relpos_attn_fwd workspace when z == NULL       */
  size_t bwd_ws_bytes;     /* relpos_attn_bwd workspace                      */
  size_t bwd_ws_bytes_noz; /* relpos_attn_bwd workspace when z == NULL       */
  int32_t delta;           /* saturation radius D: rows constant for |delta|>=D */
  int32_t expanded_rows;   /* 2D+1 rows after the bucket copy              */
  int32_t group_size;      /* queries per projection group (G)             */
  int32_t num_groups;
} relpos_sizes;

/*
 * relpos_plan_sizes -- host only (no GPU call).
 * Validates the descriptor and shape and returns buffer sizes and the plan's
 * saturation radius.  [RPA] §4.1 "Reachable Projection Ranges" and
 * "Constant-Range Reuse" define the per-group reachable rows and D; App. B.2
 * (reachable-range lemma) gives the per-group ranges.
 * Errors: INVALID_ARG, UNSUPPORTED, UNSUPPORTED_MAP, ABI.
 */
int relpos_plan_sizes(const relpos_desc *desc, const relpos_shape *shape,
                      relpos_sizes *out);

/*
 * relpos_plan_rows -- host only.  Writes the expanded row map beta of table
 * `which` (0 = A^Q, 1 = A^K, 2 = b) over s = 0 .. 2D (s = clip(delta,-D,D)+D),
 * i.e. the bucket copy of [RPA] App. B.1 (bucket-copy lemma): row s of the
 * expanded table is row beta(s) of the original.  Entries for offsets no pair
 * can reach are -1.  `cap` is the capacity of `rows_out`; returns the number
 * of entries (2D+1) or a negative error code.
 */
int relpos_plan_rows(const relpos_desc *desc, const relpos_shape *shape,
                     int32_t which, int32_t *rows_out, int32_t cap);

/*
 * relpos_project -- [RPA] Table 9 "Projection" (the projection step of Algorithm 1):
 * bucket copies of the tables, then Z^Q = Q (A^Q over each group's reachable
 * rows)^T (+ b folded in, [RPA] "Kernel structure") and Z^K likewise, stored
 * fp16 (fp32 for fp32 inputs) in `z`, plus per-token boundary entries.
 * Writes z (z_bytes >= relpos_sizes.z_bytes); uses ws (>= fwd_ws_bytes).
 */
int relpos_project(const relpos_desc *desc, const relpos_shape *shape,
                   const relpos_tensors *in, void *z, size_t z_bytes,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * relpos_project_noalloc -- relpos_project without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It runs the same
 * kernels as relpos_project; their workspace (row maps and expanded tables,
 * relpos_sizes.fwd_ws_bytes) is a static device array of 64 MiB inside the
 * library, one per GPU, held until the process ends.  The caller still owns
 * the inputs and z; with z retained, relpos_attn_fwd needs no workspace, so
 * the forward runs allocation-free.  Call it with the stream's device
 * current.  Calls on one GPU share its array: calls that overlap on one GPU
 * (several streams or threads) race and must be serialised by the caller.
 * Nothing in the array needs clearing between calls (every entry read is
 * written first by the same call).  Allocates nothing (no hipMalloc, hipFree
 * or allocating library routine).
 * Errors: as relpos_project; WORKSPACE_TOO_SMALL when fwd_ws_bytes exceeds
 * 64 MiB (e.g. an identity map over 2N - 1 offsets with many heads) or when
 * z_bytes is too small; UNSUPPORTED for a device index above 63.
 */
int relpos_project_noalloc(const relpos_desc *desc, const relpos_shape *shape,
                           const relpos_tensors *in, void *z, size_t z_bytes, void *stream);

/*
 * relpos_attn_fwd -- [RPA] Table 9 "Attention" (the tiled loop of Algorithm 1):
 * the tiled online-softmax forward with offset-aware tiles (three key ranges
 * per query tile: saturated-high, band, saturated-low).  Writes
 * O [B,H,N,64] (out_dtype) and L [B,H,N] fp32, L_i = ln sum_j exp(S_ij).
 * `z` holds relpos_project's output for these inputs; if z is NULL the
 * projection runs into ws first (ws >= fwd_ws_bytes_noz).
 */
int relpos_attn_fwd(const relpos_desc *desc, const relpos_shape *shape,
                    const relpos_tensors *in, const void *z, size_t z_bytes,
                    void *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * relpos_attn_bwd -- [RPA] Table 9 backward kernels (Algorithm 2):
 * preprocessing D = rowdot(dO, O); query-parallel pass (dQ and offset
 * gradients of the queries, single writer per entry, [RPA] §4.2); query
 * reduction (bucket fold, dA^Q, db, deterministic two-phase sums, [RPA]
 * "Deterministic table gradients"); key-parallel pass (dK, dV, key offset
 * gradients); key reduction (dA^K).  No atomics: results are bitwise
 * reproducible.  `z` as for relpos_attn_fwd (NULL: recomputed into ws,
 * ws >= bwd_ws_bytes_noz).  O and L are the forward's outputs.
 */
int relpos_attn_bwd(const relpos_desc *desc, const relpos_shape *shape,
                    const relpos_tensors *in, const void *z, size_t z_bytes,
                    const void *o, const float *lse, const void *dout,
                    relpos_grads *grads, void *ws, size_t ws_bytes, void *stream);

/*
 * relpos_set_stage_events -- instrumentation, host only (not a step of the
 * method).  Registers up to 8 hipEvent_t handles, passed as void*, for the
 * calling thread; the entry points called afterwards on this thread record
 * them on their stream: relpos_attn_fwd records [0] before and [1] after its
 * attention kernel; relpos_attn_bwd records [0] before preprocessing, [1]
 * after it, [2] after the query-parallel pass, [3] before the key-parallel
 * pass, [4] after it and [5] at its end.  Handles beyond `count` are not
 * recorded; count = 0 clears the registration.  The events stay owned by the
 * caller and must outlive the calls that record them.
 * Errors: INVALID_ARG (count outside [0, 8], or events NULL with count > 0).
 */
int relpos_set_stage_events(void *const *events, int32_t count);

/* Static description of a return code. */
const char *relpos_strerror(int code);

/* Detail of the last failing call on the calling thread ("" if none). */
const char *relpos_last_error(void);

/* Library ABI version (RELPOS_ABI_VERSION it was built with). */
int relpos_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELPOS_H */
