/*
 * tpslice.h - C ABI of the sliced tensor-parallel layer shard for MI355X (gfx950).
 *
 * One GPU's tensor-parallel share of a transformer layer's dense GEMM chain: a column-parallel
 * projection, a fused GeLU/SwiGLU epilogue and a row-parallel projection whose output is this rank's
 * partial sum (the Megatron-LM layer that Domino speeds up: Domino page, Abstract; builds-on list:
 * "Megatron-LM", "GLU Variants Improve Transformer"). The batch is cut into independent pieces -
 * contiguous token-row slices, and column slices of the partial-sum output - and each finished piece
 * is handed off (here: copied by a DMA engine on a side stream, in place of the group's reduction)
 * while later pieces compute (Domino page, Abstract: break one batch's dependency into independent
 * pieces and overlap their communication with later computation; FiCCO page, Abstract: overlap below
 * shard granularity, communication offloaded to GPU DMA engines). Slicing and overlap change no value
 * (DHelix review, "If this is right": reordering/overlap leaves training semantics unchanged).
 *
 * Conventions for every entry point
 *   - Device pointers are plain `void*` into GPU memory owned by the caller; the library never frees
 *     or keeps them beyond the call's stream work. 16-byte alignment is required. Tensors with a
 *     token dimension may be NULL when the plan's token count is 0 (an empty batch); the weight
 *     gradients are then set to zero (accumulate = 0) or left as they are (accumulate = 1).
 *   - bf16 tensors are row-major and contiguous. Weights use the [out_features][in_features] layout
 *     of a linear layer:  W1 [N1][h] (N1 = F' for GeLU, 2F' for SwiGLU with rows [gate | up]),
 *     W2 [h][F'], Wqkv [(q+2kv)d][h] with rows [Q | K | V], Wo [h][q d].
 *     Activations: X, Z, dY, dX [M][h]; U [M][N1]; C, dC [M][q d]; QKV, dQKV [M][(q+2kv)d].
 *     Weight and bias gradients are fp32 in the weight's own layout.
 *   - Streams belong to the caller (tpslice_streams_t below): the library creates and destroys no
 *     stream. Calls are asynchronous and stream-ordered: they start after work already queued on
 *     the caller's stream, fork onto the caller's worker and copy streams, and join back, so every
 *     output (the hand-off copy included) is complete when the caller's stream reaches the point
 *     after the call (TPSLICE_F_PIPELINE relaxes this for the hand-off copies only).
 *   - The calls of a joined plan (no TPSLICE_F_PIPELINE) with one worker stream may be captured into
 *     a HIP graph on the caller's stream: they allocate nothing, synchronize nothing and clear no
 *     memory, and the hand-off copies become graph copy nodes; each replay gives the bits of the
 *     same calls run eagerly. A pipelined plan, or one with more worker streams, returns
 *     TPSLICE_ERR_UNSUPPORTED when the caller's stream is capturing, before queueing anything.
 *   - Outputs must not alias inputs or each other. Results are deterministic: the same plan and
 *     inputs give bitwise identical outputs, whatever the slice timing.
 *   - Errors are reported by status code only; argument, shape and workspace errors are detected
 *     before any GPU work is queued. tpslice_last_error() gives the text of the calling thread's last
 *     failure. A plan must not be used from two host threads at once.
 */
#ifndef TPSLICE_H
#define TPSLICE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define TPSLICE_API __attribute__((visibility("default")))
#else
#define TPSLICE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TPSLICE_OK = 0,
  TPSLICE_ERR_INVALID = 1,     /* null required pointer, bad enum value, bad or destroyed plan      */
  TPSLICE_ERR_SHAPE = 2,       /* sizes the slicing or the kernels cannot take                       */
  TPSLICE_ERR_UNSUPPORTED = 3, /* valid request outside what the plan describes (e.g. no heads)      */
  TPSLICE_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned                         */
  TPSLICE_ERR_HIP = 5          /* a HIP runtime call failed; see tpslice_last_error()                */
} tpslice_status_t;

typedef enum {
  TPSLICE_ACT_GELU = 1,   /* H = U * Phi(U), exact erf form                                   */
  TPSLICE_ACT_SWIGLU = 2  /* U = [G | V]; H = silu(G) * V, silu(g) = g / (1 + e^-g)          */
} tpslice_act_t;

/* tpslice_desc_t.flags */
#define TPSLICE_F_SERIALIZE 0x1u /* every product and copy in order on the caller stream (ablation)  */
#define TPSLICE_F_COPY_BLIT 0x2u /* hand-off copies by the runtime's copy kernel instead of the DMA
                                    engines (uses compute units; for comparison)                       */
#define TPSLICE_F_PIPELINE 0x4u  /* pipelined hand-off: the caller's stream waits for the products
                                    only; a later call's row slice i waits for this call's hand-off
                                    copies of row slice i (a product over all tokens that no row
                                    slice of its call precedes: for all of them). It may wait for
                                    more: after a call that queued products over all tokens behind
                                    its last copies, the next call's first row slice waits for all
                                    of that call's copies, which ran under those products. Chained
                                    calls (a layer reading the previous layer's hand-off) then
                                    overlap the last pieces' copies with the next call's first
                                    pieces (Domino page,
                                    Abstract: independent pieces pipelined across the batch's work).
                                    Use tpslice_handoff_wait() before reading a hand-off buffer on
                                    another stream, or before freeing buffers the copies touch.    */
#define TPSLICE_F_HANDOFF_ROWS 0x8u /* with column slices (c > 1): hand off each row slice as one
                                    contiguous copy on the DMA engines once the row slice is done,
                                    instead of each (row, column) piece on its own. A piece is a
                                    strided 2D region, which the HIP runtime copies with a kernel on
                                    the compute units (taking them from the products); a whole row
                                    slice is contiguous. Since the copy then waits for every column
                                    of the row slice, the row slice's product runs as one launch over
                                    all h columns (c times the blocks of a piece: the GPU's compute
                                    units filled by one product; same k order, same bits).        */
#define TPSLICE_F_CALLER_WORKER 0x40u /* worker stream 0 is the caller's stream (no stream of its own):
                                    one fork and join fewer per call, and one hardware queue fewer
                                    (a process has four by default), so that two plans with their
                                    own copy streams can run side by side, e.g. the forward of one
                                    micro-batch beside the backward of another. A call from a
                                    different stream than the previous call waits for it first.
                                    A plan with one worker stream (not serialized) always works
                                    this way.                                                      */
/* Block tile of every product (ablation, testing): flags |= TPSLICE_F_TILE(id). By default (id 0)
   each product takes the tile with the smallest estimated time on the 256 CUs. The tile never
   changes a result bit. Ids: 1 = 256 x 256, 2 = 128 x 128 (4 waves, two blocks per CU),
   3 = 256 x 320, 4 = 128 x 320, 5 = 128 x 256, 6 = 128 x 128 (8 waves, one block per CU),
   7 = 256 x 256, 8 = 256 x 160, 9 = 256 x 320 and 10 = 256 x 224 (4 waves, software-pipelined).
   The 320-wide tiles serve only forward products without the SwiGLU pairing, id 8 those and
   activation gradients with a bf16 or GeLU-gradient epilogue, id 10 only forward SwiGLU products
   (112 gate and 112 up columns per block), ids 7-10 only products whose k is a multiple of 64 and
   that do not add to an fp32 output (accumulate = 1); other products then take the automatic
   choice.                                                                                        */
#define TPSLICE_F_TILE_SHIFT 8
#define TPSLICE_F_TILE_MASK (0xFu << TPSLICE_F_TILE_SHIFT)
#define TPSLICE_F_TILE(id) (((uint32_t)(id) << TPSLICE_F_TILE_SHIFT) & TPSLICE_F_TILE_MASK)
#define TPSLICE_TILE_COUNT 11

typedef struct {
  int64_t tokens;         /* M: token rows in the batch (micro-batch x sequence, batch-major)         */
  int64_t hidden;         /* h: model width; multiple of 8                                            */
  int64_t ffn;            /* F: full FFN width; this rank holds F' = ffn / tp_size (multiple of 8)    */
  int32_t tp_size;        /* simulated tensor-parallel group size (>= 1); no communication happens   */
  int32_t n_row_slices;   /* r: equal contiguous token-row slices; must divide tokens (0: automatic) */
  int32_t n_col_slices;   /* c: equal column slices of each hand-off output (width h); h/c % 8 == 0
                             (0: automatic)                                                         */
  int32_t n_heads;        /* full-model query heads; 0 = no attention projections in this plan       */
  int32_t n_kv_heads;     /* full-model key/value heads (GQA); this rank holds max(1, n_kv/tp_size)   */
  int32_t head_dim;       /* d; multiple of 8                                                          */
  int32_t act;            /* tpslice_act_t                                                              */
  int32_t n_streams;      /* worker streams for the slices (0 = default: 1 for one row slice, for a
                             layer shard (n_heads > 0) and when the up-projection runs over groups
                             of row slices; otherwise 2 when the per-slice forward products, each
                             alone with its tile, leave more than 5% of their flop-weighted block
                             rounds empty on the 256 CUs, else 1); slice i runs on stream
                             i mod n_streams and starts once slice i-1's first product is done     */
  int32_t n_copy_streams; /* side streams for hand-off copies (0 = default: 1)                        */
  uint32_t flags;         /* TPSLICE_F_*                                                                */
  float handoff_gbps;     /* hand-off rate in GB/s that the automatic slice counts assume (0: the
                             local DMA copy of this GPU, about 600 GB/s); ignored for given counts */
  int32_t dh_group;       /* row slices per dH product of the MLP backward (0: automatic, see
                             tpslice_plan_info_t.dh_group_slices); else a power of two dividing
                             the row slice count                                                  */
  int32_t up_group;       /* row slices per up-projection of the MLP forward, likewise            */
} tpslice_desc_t;

/* Automatic slice counts (Design Space Exploration of DMA based Finer-Grain Compute Communication
 * Overlap page, Abstract: decomposition and contention slow finer pieces down, and schedules are
 * picked by heuristics on the operators' static sizes). An r or c of 0 is chosen from r in
 * {1, 2, 4, 8, 16} dividing tokens and c in {1, 2, 4} keeping h/c a multiple of 8, for the smallest
 * predicted time of one call of the forward products: the per-slice products' estimated times
 * (tile, split and launch costs of this GPU) plus the hand-off's exposed time at `handoff_gbps`
 * (with TPSLICE_F_PIPELINE: the larger of compute and copies per call, plus the part of the first
 * row slice's copy that the rest of the call does not cover, since the next call's first row slice
 * waits for it; without: the copies of the last row slice, or of all slices when copying is the
 * slower side). Within 2%, fewer pieces win.
 * tpslice_plan_info reports the counts taken.                                                    */

typedef struct tpslice_plan_s* tpslice_plan_t;

/* The streams of one call (all hipStream_t, passed as void*). The caller owns them; the library only
 * queues work on them and records and waits on events of its own plan. With TPSLICE_F_CALLER_WORKER
 * (always set for a plan with one worker stream) worker 0 is `caller` and `workers` holds the other
 * n_streams - 1, else all n_streams (tpslice_plan_info reports n_streams and n_copy_streams; extra
 * entries are ignored). A call that hands off (a non-NULL hand-off buffer, tpslice_handoff_copy)
 * also takes n_copy_streams copy streams. The streams one call uses must all differ. A serialized
 * plan (TPSLICE_F_SERIALIZE) uses `caller` only. A NULL tpslice_streams_t* means the null stream
 * as caller and no other streams. Different calls of one plan may use different streams.          */
typedef struct {
  void* caller;            /* the stream the call is ordered on (NULL: the null stream)               */
  void* const* workers;    /* worker streams for the row slices                                        */
  int32_t n_workers;
  void* const* copiers;    /* side streams for the hand-off copies                                     */
  int32_t n_copiers;
} tpslice_streams_t;


typedef struct {
  int64_t tokens, hidden, ffn_shard, n1, qkv_width, ctx_width;
  int64_t rows_per_slice;       /* M / r                                                             */
  int64_t handoff_cols;         /* h / c                                                             */
  int32_t n_row_slices, n_col_slices, n_streams, n_copy_streams;
  int32_t q_heads, kv_heads;    /* this rank's head counts                                           */
  /* k splits (1 = none) the plan takes for, in order: the up-projection of each group of row
     slices, the QKV projection over all tokens, dH of each group of row slices, then dW1, dW2, dC,
     dWo, dWqkv over all tokens. A split product sums its k runs' fp32 partials in order before the
     epilogue: the same bits for every slicing of the same batch, other rounding than an unsplit
     product. k_split_rows says which rows a split covers.                                       */
  int32_t k_splits[8];
  /* the slice-count model's predicted time (us) of one call of the forward products with this
     plan's r and c (see the automatic slice counts above); a comparison figure, not a timing */
  double predicted_forward_us;
  /* row slices per dH product of the MLP backward (dH is not handed off: it runs over groups of
     consecutive row slices large enough to fill the GPU, each row slice's dX product and hand-off
     after it)                                                                                  */
  int32_t dh_group_slices;
  /* row slices per up-projection of the MLP forward (likewise: only the down-projection after it is
     handed off, each row slice's after its group's up-projection)                              */
  int32_t up_group_slices;
  /* rows of each product in k_splits (same order) that its split covers: 0 when it is not split,
     the product's rows when the whole product is split, fewer for a weight gradient whose last
     rows alone are split (a "tail split": its other rows, a whole number of rounds of 256 x 256
     tiles on the 256 CUs, run unsplit, and the tail's split fills the last round instead of
     leaving it part empty; each output element still has one fixed summation order)           */
  int32_t k_split_rows[8];
} tpslice_plan_info_t;

typedef enum {
  TPSLICE_OP_MLP_FWD = 0,
  TPSLICE_OP_ATTNPROJ_FWD = 1,
  TPSLICE_OP_MLP_BWD = 2,
  TPSLICE_OP_ATTNPROJ_BWD = 3,
  TPSLICE_OP_ATTN_CORE_BWD = 4
} tpslice_op_t;

/* Validate `desc` and build a plan (host memory only; no GPU call is made). The slice geometry is
 * r equal contiguous token-row ranges, each cut into c equal column ranges of the hand-off output,
 * finished in order row slice major (Domino page, Abstract: independent pieces of one batch).
 * Returns TPSLICE_ERR_INVALID for a null argument or bad enum, TPSLICE_ERR_SHAPE for sizes that do
 * not divide or are not multiples of 8, or whose operands exceed 4 GiB. On error *out is NULL.     */
TPSLICE_API tpslice_status_t tpslice_plan(const tpslice_desc_t* desc, tpslice_plan_t* out);

/* Release the plan and its events. NULL is a no-op. Blocks until the plan's queued work (products,
 * hand-off copies) has finished, so it may be called with work in flight; no stream is touched.   */
TPSLICE_API tpslice_status_t tpslice_plan_destroy(tpslice_plan_t plan);

/* Sizes the plan derived from its descriptor.                                                     */
TPSLICE_API tpslice_status_t tpslice_plan_info(tpslice_plan_t plan, tpslice_plan_info_t* info);

/* The index-th hand-off piece in finish order (0 <= index < r*c): out[0..3] = row begin, row end,
 * column begin, column end (end exclusive) of the [M][h] hand-off tensor.                         */
TPSLICE_API tpslice_status_t tpslice_plan_piece(tpslice_plan_t plan, int32_t index, int64_t out[4]);

/* Bytes of device workspace that `op` needs (may be 0). Workspace must be 256-byte aligned.       */
TPSLICE_API tpslice_status_t tpslice_workspace_size(tpslice_plan_t plan, int32_t op, size_t* bytes);

/* MLP forward (one rank's share). Defined by: the Megatron-LM layer that Domino starts from (Domino
 * page, Abstract, and its builds-on list: "Megatron-LM", "GLU Variants Improve Transformer" for
 * SwiGLU), cut into the independent pieces whose hand-off overlaps later pieces' computation (Domino
 * page, Abstract) with communication offloaded to DMA engines (FiCCO page, Abstract).
 *   U = X W1^T + b1;  H = act(U);  Z = H W2^T   (Z: this rank's partial sum, no row-parallel bias)
 * Inputs : X [M][h], W1 [N1][h], b1 [N1] bf16 or NULL, W2 [h][F'].
 * Outputs: Z [M][h] bf16; U_save [M][N1] bf16 or NULL (pre-activation kept for the backward pass);
 *          Z_handoff [M][h] bf16 or NULL: when given, each finished piece of Z is copied into it on
 *          a side stream while later pieces compute (Z_handoff == Z bitwise when the call is done).
 * Workspace: tpslice_workspace_size(TPSLICE_OP_MLP_FWD) bytes (holds H).                          */
TPSLICE_API tpslice_status_t tpslice_mlp_fwd(tpslice_plan_t plan, const void* X, const void* W1, const void* b1,
                                 const void* W2, void* Z, void* U_save, void* Z_handoff,
                                 void* workspace, size_t workspace_bytes, const tpslice_streams_t* streams);

/* Attention input/output projections, forward (one rank's heads). Defined by: the same Megatron-LM
 * split applied to the attention block's projections, sliced and handed off as the MLP's (Domino
 * page, Abstract).
 *   QKV = X Wqkv^T (+ bqkv)   column-parallel;   Z = C Wo^T   row-parallel partial sum
 * C is the attention context of this rank's heads (an input here; tpslice_attn_core_fwd computes it
 * from QKV). Z_handoff as in tpslice_mlp_fwd. Z runs by row slices (its pieces are the hand-off);
 * QKV, which nothing hands off, runs after them as one product over all tokens, under the last
 * pieces' copies. Needs n_heads > 0 in the plan. Either projection may
 * be left out: Wqkv = NULL skips QKV (X, bqkv, QKV unused), Wo = NULL skips Z (C, Z, Z_handoff
 * unused), so that a layer can run QKV, then tpslice_attn_core_fwd, then the output projection;
 * both NULL is TPSLICE_ERR_INVALID.                                                              */
TPSLICE_API tpslice_status_t tpslice_attnproj_fwd(tpslice_plan_t plan, const void* X, const void* Wqkv,
                                      const void* bqkv, void* QKV, const void* C, const void* Wo,
                                      void* Z, void* Z_handoff, void* workspace,
                                      size_t workspace_bytes, const tpslice_streams_t* streams);

/* MLP backward. Defined by: the gradient of tpslice_mlp_fwd (chain rule), the backward pass whose
 * tensor-parallel communication the pages hide the same way as the forward's (Domino page, Abstract;
 * the micro-batch co-execution review, "What carries the argument": forward of one micro-batch beside
 * the backward of another). Given the saved pre-activation U [M][N1] and upstream gradient dY [M][h]:
 *   dH = dY W2;  dU = dH * act'(U) (SwiGLU: [dH V silu'(G) | dH silu(G)]);  dX = dU W1
 *   dW1 (+)= dU^T X;  db1 (+)= column sums of dU;  dW2 (+)= dY^T act(U)
 * dX [M][h] bf16 is this rank's partial sum and the hand-off tensor (dX_handoff as Z_handoff above).
 * dW1 [N1][h], dW2 [h][F'] and db1 [N1] (or NULL) are fp32; accumulate = 0 overwrites them,
 * 1 adds to their contents. Workspace: tpslice_workspace_size(TPSLICE_OP_MLP_BWD).
 * dH, which is not handed off, runs over groups of consecutive row slices (plan info
 * dh_group_slices); each row slice's dX product and hand-off follow its group's dH.               */
TPSLICE_API tpslice_status_t tpslice_mlp_bwd(tpslice_plan_t plan, const void* X, const void* W1, const void* W2,
                                 const void* U_saved, const void* dY, void* dX, void* dX_handoff,
                                 float* dW1, float* db1, float* dW2, int32_t accumulate,
                                 void* workspace, size_t workspace_bytes, const tpslice_streams_t* streams);

/* Attention projections backward. Defined by: the gradient of tpslice_attnproj_fwd (chain rule),
 * sliced and handed off as tpslice_mlp_bwd. Given dQKV [M][(q+2kv)d] (from the attention core) and
 * dY [M][h] (into the output projection):
 *   dC = dY Wo;  dWo (+)= dY^T C;  dX = dQKV Wqkv (partial sum, hand-off);  dWqkv (+)= dQKV^T X;
 *   dbqkv (+)= column sums of dQKV (or NULL).  dC bf16; weight/bias gradients fp32.
 * Either half may be left out: Wo = NULL skips dC and dWo (C, dY, dC, dWo unused), Wqkv = NULL skips
 * dX, dWqkv and dbqkv (X, dQKV, dX, dX_handoff, dWqkv, dbqkv unused), so that a layer can take dC to
 * tpslice_attn_core_bwd and its dQKV back here; both NULL is TPSLICE_ERR_INVALID.                */
TPSLICE_API tpslice_status_t tpslice_attnproj_bwd(tpslice_plan_t plan, const void* X, const void* Wqkv,
                                      const void* dQKV, const void* C, const void* Wo,
                                      const void* dY, void* dX, void* dX_handoff, void* dC,
                                      float* dWqkv, float* dbqkv, float* dWo, int32_t accumulate,
                                      void* workspace, size_t workspace_bytes,
                                      const tpslice_streams_t* streams);

/* Causal attention core between the two projections, forward (the tiled softmax attention of the
 * FlashAttention titles on the Domino page's builds-on list, computed exactly up to rounding):
 *   C[t, h] = sum over s <= t of softmax_s(Q[t, h] . K[s, g] / sqrt(head_dim)) V[s, g],
 *   g = h / (q_heads / kv_heads), t and s positions in the same sequence.
 * Inputs : QKV [M][(q + 2 kv) head_dim] bf16 as tpslice_attnproj_fwd writes it (Q heads, K heads,
 *          V heads); the sequences are consecutive runs of `seq_len` token rows.
 * Outputs: C [M][q head_dim] bf16, the context the output projection reads; lse [M][q] fp32 or
 *          NULL: each row's log-sum-exp of its scaled scores (natural log), which
 *          tpslice_attn_core_bwd takes.
 * Requires the plan's head_dim = 128 (else TPSLICE_ERR_UNSUPPORTED), seq_len a multiple of 128
 * that divides the token count (else TPSLICE_ERR_SHAPE). Softmax in fp32; the probabilities are
 * rounded to bf16 for the product with V. Runs on streams->caller (no slicing, no hand-off).      */
TPSLICE_API tpslice_status_t tpslice_attn_core_fwd(tpslice_plan_t plan, const void* QKV, void* C, float* lse,
                                                   int64_t seq_len, const tpslice_streams_t* streams);

/* Causal attention core, backward: the gradient of tpslice_attn_core_fwd by the chain rule through
 * the softmax, computed in tiles from the forward's inputs, output and row log-sum-exp (the
 * FlashAttention titles on the Domino page's builds-on list):
 *   dV[s, g] = sum over the group's heads h, t >= s of P[t, s] dC[t, h]
 *   dA[t, s] = P[t, s] (dC[t, h] . V[s, g] - dC[t, h] . C[t, h])
 *   dQ[t, h] = sum over s <= t of dA[t, s] K[s, g] / sqrt(head_dim)
 *   dK[s, g] = sum over the group's heads h, t >= s of dA[t, s] Q[t, h] / sqrt(head_dim)
 * Inputs : QKV, C and lse as the forward took and wrote them; dC [M][q head_dim] bf16, the gradient
 *          of C (tpslice_attnproj_bwd's dC).
 * Outputs: dQKV [M][(q + 2 kv) head_dim] bf16 in QKV's column layout (the dQKV that
 *          tpslice_attnproj_bwd takes). Grouped key/value heads sum their query heads' shares in
 *          head order (deterministic).
 * Workspace: tpslice_workspace_size(TPSLICE_OP_ATTN_CORE_BWD) bytes. Same requirements as the
 * forward. Runs on streams->caller.                                                              */
TPSLICE_API tpslice_status_t tpslice_attn_core_bwd(tpslice_plan_t plan, const void* QKV, const void* C,
                                                   const float* lse, const void* dC, void* dQKV, int64_t seq_len,
                                                   void* workspace, size_t workspace_bytes,
                                                   const tpslice_streams_t* streams);

/* Allocation-free MLP forward, for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): tpslice_mlp_fwd with its
 * workspace in a fixed device array of the library (TPSLICE_STATIC_SCRATCH_BYTES per GPU, held from
 * the library's first use on that GPU until the process ends) instead of a caller buffer. Same
 * arguments, semantics and results as tpslice_mlp_fwd; a plan whose MLP forward workspace
 * (tpslice_workspace_size, TPSLICE_OP_MLP_FWD) exceeds the array gets TPSLICE_ERR_WORKSPACE before
 * anything is queued. It calls no device allocation (the array's address is looked up on the first
 * call on each GPU, and a plan creates its events on its first call of any entry point). Every call
 * on one GPU uses the same array: calls that overlap in time on one GPU race on it.               */
#define TPSLICE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
TPSLICE_API tpslice_status_t tpslice_mlp_fwd_static(tpslice_plan_t plan, const void* X, const void* W1,
                                                    const void* b1, const void* W2, void* Z, void* U_save,
                                                    void* Z_handoff, const tpslice_streams_t* streams);

/* Tracing. When enabled, every product and every hand-off copy is bracketed by timing events on
 * the stream it runs on. Records accumulate over calls until they are read; times are milliseconds
 * from the start (on the caller stream) of the first call traced since the last read, and `call`
 * numbers the calls from 0 in that window. Tracing adds event records to the streams; it changes
 * no result.                                                                                      */
typedef enum {
  TPSLICE_TRACE_GEMM = 0,      /* a product's GEMM kernel (for a product split along k: its partial products) */
  TPSLICE_TRACE_COPY = 1,      /* a hand-off copy                                                       */
  TPSLICE_TRACE_COLSUM = 2,    /* the bias gradient's column sums                                       */
  TPSLICE_TRACE_SPLIT_SUM = 3  /* a split product's ordered reduction of its partials, with the epilogue */
} tpslice_trace_kind_t;
typedef enum {
  TPSLICE_STEP_MLP_UP = 0,     /* X W1^T + activation                 */
  TPSLICE_STEP_MLP_DOWN = 1,   /* H W2^T (partial sum piece)          */
  TPSLICE_STEP_QKV = 2,        /* X Wqkv^T                            */
  TPSLICE_STEP_OUT = 3,        /* C Wo^T (partial sum piece)          */
  TPSLICE_STEP_MLP_DH = 4,     /* dY W2 with the activation derivative */
  TPSLICE_STEP_MLP_DX = 5,     /* dU W1 (partial sum piece)           */
  TPSLICE_STEP_MLP_DW1 = 6,    /* dU^T X                              */
  TPSLICE_STEP_MLP_DW2 = 7,    /* dY^T H                              */
  TPSLICE_STEP_ATTN_DX = 8,    /* dQKV Wqkv (partial sum piece)       */
  TPSLICE_STEP_ATTN_DC = 9,    /* dY Wo                               */
  TPSLICE_STEP_ATTN_DWQKV = 10,/* dQKV^T X                            */
  TPSLICE_STEP_ATTN_DWO = 11,  /* dY^T C                              */
  TPSLICE_STEP_BIAS_GRAD = 12, /* column sums                         */
  TPSLICE_STEP_HANDOFF = 13    /* hand-off copy                       */
} tpslice_step_t;
typedef struct {
  int32_t kind;     /* tpslice_trace_kind_t                                           */
  int32_t step;     /* tpslice_step_t                                                 */
  int32_t slice;    /* row slice (-1: all tokens)                                    */
  int32_t piece;    /* column piece (-1: none)                                        */
  int32_t stream;   /* 0..S-1 worker, S..S+E-1 copy stream, -1 caller stream         */
  int32_t call;     /* index of the call in the current trace window                 */
  double flops;     /* algorithmic flops, 2*M*N*K (0 for copies)                      */
  double bytes;     /* bytes copied (copies), 0 otherwise                             */
  float start_ms, end_ms;
  /* the GEMM kernel of a TPSLICE_TRACE_GEMM record (zeros otherwise): its block tile
     tile_m x tile_n, waves_m x waves_n waves, blocks_per_cu resident blocks per CU, layout
     (0 forward, 1 activation gradient, 2 weight gradient), epilogue, and its grid of `blocks`
     workgroups of `threads` work-items - the identity a kernel profiler reports for the launch */
  int32_t tile_m, tile_n, waves_m, waves_n, blocks_per_cu, layout, epilogue, blocks, threads;
} tpslice_trace_rec_t;

/* enable: 0 off; bit 0 traces products (GEMMs, column sums); bit 1 traces hand-off copies (each
 * traced copy is closed by a one-wave fence kernel so that its end event covers the DMA engine).   */
TPSLICE_API tpslice_status_t tpslice_trace_enable(tpslice_plan_t plan, int32_t enable);
/* Sets *count to the number of records in the window. With cap >= *count it also copies them into
 * `recs` (blocking until their events have completed) and starts a new window; with a smaller cap
 * (e.g. 0) it only reports the count. TPSLICE_ERR_INVALID if tracing is off.                      */
TPSLICE_API tpslice_status_t tpslice_trace_read(tpslice_plan_t plan, tpslice_trace_rec_t* recs, int32_t cap,
                                                int32_t* count);

/* Only the hand-off: copy every piece of the [M][h] bf16 tensor `src` into `dst` exactly as a call
 * hands off its partial sums (same pieces, copy streams and engines), with no products. This is the
 * communication-only run that the overlap measurement compares against.                         */
TPSLICE_API tpslice_status_t tpslice_handoff_copy(tpslice_plan_t plan, const void* src, void* dst,
                                                  const tpslice_streams_t* streams);

/* Make `stream` wait until every hand-off copy the plan has queued so far is complete (needed only
 * with TPSLICE_F_PIPELINE; a no-op before the plan's first call).                                */
TPSLICE_API tpslice_status_t tpslice_handoff_wait(tpslice_plan_t plan, void* stream);

/* Two-strand pairing (host only; no GPU work). The forward segments 1..nf of one micro-batch and
 * the backward segments 1..nb of another run in order within each strand; each step of a pairing
 * runs one forward segment alone, one backward segment alone, or one of each side by side (the
 * strand interleaving of the micro-batch co-execution review, "What carries the argument"). With
 * P the measured times - P[i (nb + 1) + j] for forward segment i beside backward segment j,
 * P[i (nb + 1)] for forward segment i alone, P[j] for backward segment j alone (P[0] unused) - the
 * pairing of least total time follows the review's recurrence
 *   T(i, j) = min{ T(i-1, j) + P(i, none), T(i, j-1) + P(none, j), T(i-1, j-1) + P(i, j) }.
 * Outputs: steps [2 (nf + nb)] int32 (capacity), filled with *n_steps (forward, backward) pairs of
 * segment numbers in execution order, 0 meaning none; *makespan = T(nf, nb). Ties take the pair,
 * then the forward segment alone. TPSLICE_ERR_INVALID for a NULL pointer or a negative or
 * non-finite time, TPSLICE_ERR_SHAPE for counts outside [0, 4096].                              */
TPSLICE_API tpslice_status_t tpslice_strand_schedule(const double* P, int32_t nf, int32_t nb, int32_t* steps,
                                                     int32_t* n_steps, double* makespan);

/* Static text for a status code.                                                                   */
TPSLICE_API const char* tpslice_error_string(tpslice_status_t status);

/* Text of the calling thread's most recent failure ("" if none).                                   */
TPSLICE_API const char* tpslice_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSLICE_H */
