/*
 * kda_tree.h -- C-ABI of the tree-packed chunkwise KDA library (libkda_tree.so)
 *
 * What the library computes follows the HARTS pages (arXiv 2608.28158):
 *   - devfeed.tech abstract: prefix sharing over rollout trees; differentiable
 *     boundary-state handoff and bounded replay keep each trajectory's
 *     chunkwise numerical path; a linear-time planner reaches the minimum
 *     number of sequential linear-attention calls under the packed
 *     chunkwise-call model; log-probs are recovered per original position.
 *   - thelatestinai.com Figure 1 (compact layout, call example), Figure 2
 *     (continuations, replay-started side branches, rounds = packed calls),
 *     Figure C.1(b) (replay inside the core writes no outputs) and C.1(d)
 *     (mapped log-probs without expanded logits).
 *   - zot.news summary: the interfaces keep gradient flow and RL objectives.
 *
 * The KDA recurrence (the pages name it but do not print it) is the gated
 * delta rule, per head, with state S (dk x dv, fp32):
 *     Sbar = diag(exp(g_t)) S;  u = beta_t (v_t - Sbar^T k_t);
 *     S = Sbar + k_t u^T;       o_t = scale * S^T q_t.
 *
 * Conventions for every call:
 *   - All device memory is owned by the caller.  Tensors are contiguous,
 *     row-major, with the row (token) dimension first: q,k [rows,H,dk];
 *     v [rows,H,dv]; g [rows,H,dk] fp32; beta [rows,H] fp32; o [rows,H,dv]
 *     fp32; states [*,H,dk,dv] fp32.  Every device pointer (tensors,
 *     `saved`, `ws`) is 16-byte aligned, beta and dbeta 4-byte aligned
 *     (KDA_ERR_ARG otherwise): rows move in 16-byte vectors.
 *   - The library never allocates device memory and never synchronises the
 *     device.  Work is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream) in stream order.  kda_tree_fwd and kda_tree_bwd run part of
 *     their kernels on a second stream of the current device (created on
 *     the first such call, default priority, kept until the process ends),
 *     forked from `stream` and joined back into it with events: all of
 *     their work still follows earlier work on `stream` and precedes later
 *     work on it, and the pattern is valid under stream capture
 *     (kda_set_overlap(0) keeps all work on `stream`).
 *   - Results are deterministic: bitwise identical from run to run (no
 *     floating-point atomics; every reduction has a fixed order).
 *   - Status codes: KDA_OK (0) or a negative KDA_ERR_*; on error nothing is
 *     enqueued and kda_last_error() holds a message (thread-local).
 */
#ifndef KDA_TREE_H
#define KDA_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KDA_OK = 0,
  KDA_ERR_TREE = -1,      /* malformed tree: bad parent, cycle, zero length, overlapping rows */
  KDA_ERR_SHAPE = -2,     /* unsupported head dims / chunk size / dtype */
  KDA_ERR_WORKSPACE = -3, /* a workspace or buffer is smaller than required */
  KDA_ERR_ARG = -4,       /* null pointer or inconsistent argument */
  KDA_ERR_HIP = -5        /* a HIP runtime call or kernel launch failed */
};

enum {
  KDA_MODE_MINCALL = 0,
  KDA_MODE_EXPANDED = 1,
  KDA_MODE_NOREPLAY = 2,
  KDA_MODE_NODEWISE = 3,
  KDA_MODE_MINCALL_SHORT = 4
};
enum { KDA_DTYPE_FP32 = 0, KDA_DTYPE_BF16 = 1 };

typedef struct kda_plan kda_plan;

typedef struct {
  int32_t n_seg, n_rounds, n_seq, n_chunks, n_buf, n_leaf, n_root, chunk, mode;
  int32_t max_seq_per_round;
  int64_t n_rows;      /* compact (unique) rows N */
  int64_t n_packed;    /* packed rows over all rounds (N + R in MINCALL mode) */
  int64_t n_out_rows;  /* rows of o / dO / input gradients (N, or n_packed in EXPANDED) */
  int64_t R;           /* total replay rows */
  int64_t n_pos;       /* trajectory positions with a next-token target */
  int64_t n_expanded;  /* sum of trajectory lengths */
  size_t device_bytes; /* size of the device copy made by kda_plan_upload */
  int32_t n_att_tiles; /* 64-row tiles of all segments (tree attention query / key tiles) */
  int32_t n_att_items; /* dk / dv work items of the tree attention backward */
  int32_t n_att_slots; /* partial dk / dv slots (per head) of split key tiles */
  int32_t n_att_split; /* key tiles whose work is split over several items */
} kda_plan_info_t;

/*
 * kda_tree_plan -- validate a rollout tree and build its min-call plan (host only).
 *
 * Follows the Figure 2 call model (thelatestinai.com) and the abstract's
 * linear-time planner: every fork-free segment runs once; each internal
 * segment continues one child directly (same sequence, same round); every
 * other child is side-started from the boundary state at b = B*floor(p/B)
 * (p = the fork position) and replays r = p - b < B parent rows without
 * writing outputs.  It starts in the round of its parent's sequence when b is
 * where that sequence started, otherwise in the next round.  A two-mode
 * dynamic program picks the continuations that minimise the number of rounds
 * (ties: larger side cost, larger subtree token count, smaller segment id).
 * Sequences of a round are ordered by head segment id.
 *
 *   n_seg    number of segments (> 0)
 *   parent   [n_seg] parent segment id, -1 for a root (a forest is allowed;
 *            roots are indexed by ascending id for h0 / dh0)
 *   seg_len  [n_seg] tokens per segment (> 0)
 *   seg_row  [n_seg] first compact row of each segment, or NULL for segments
 *            packed in id order; the ranges must tile [0, N) exactly
 *   chunk    chunk size B (>= 1; the kernels accept 16 and 64)
 *   mode     KDA_MODE_MINCALL, or KDA_MODE_EXPANDED: one sequence per
 *            trajectory (leaf ascending), all in one round, no sharing; rows
 *            of o / dO / gradients are then the packed (expanded) rows.
 *            Two ablations of the replay rule (thelatestinai.com Figure 5,
 *            the no-replay variant; Figure 4, node-wise linear attention),
 *            both on compact rows like MINCALL and with R = 0:
 *            KDA_MODE_NOREPLAY: continuations as above, but every side child
 *            starts at its own first position from the exact state there,
 *            one round after its parent's sequence; the parent's chunk grid
 *            is cut at that position (a short chunk) and the child's grid
 *            starts there.  Continuations minimise rounds under that rule
 *            (each side start costs one round).
 *            KDA_MODE_NODEWISE: one sequence per segment, started from its
 *            parent's end state, round = depth; a sequence ending at an
 *            inner segment has no leaf (KDA_F_SEQ_LEAF = -1).
 *            KDA_MODE_MINCALL_SHORT (not the pages' planner; a variant for
 *            the GPU): the same minimum number of rounds and the same replay
 *            rule, but a segment whose children can all be side-started
 *            without adding a round continues none of them, so sequences end
 *            sooner and the longest sequence of a round (what its call waits
 *            for) shrinks, at the price of more replay rows.
 *   out      receives the plan (immutable; free with kda_plan_destroy)
 * Host pointers.  Errors: KDA_ERR_TREE, KDA_ERR_ARG.
 */
int kda_tree_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len,
                  const int64_t* seg_row, int32_t chunk, int32_t mode, kda_plan** out);

void kda_plan_destroy(kda_plan* plan);

/*
 * kda_l1_plan -- compression-oriented microbatches of whole trajectories
 * (HARTS abstract and Figure 1(c): the first planner level builds
 * compression-oriented microbatches; Table 4 measures compression and
 * balance).  A microbatch's load is its unique token count (the union of
 * its trajectories' rows) and stays within `budget` (a trajectory longer
 * than the budget goes alone).  Trees that fit stay whole; larger trees are
 * cut into groups of leaves in depth-first order; the items are packed
 * first-fit decreasing, then placed on the least-loaded microbatch (kept
 * when all fit).  Host only; deterministic.
 *
 *   parent, seg_len  as for kda_tree_plan (n_seg entries)
 *   leaf_mb          [n_leaf] out: microbatch of each trajectory, leaves by
 *                    ascending segment id
 *   n_mb             out: number of microbatches (<= n_leaf)
 *   mb_unique, mb_expanded  [n_leaf] out: per microbatch (first *n_mb used)
 *                    its unique tokens and the summed lengths of its
 *                    trajectories; compression = sum expanded / sum unique,
 *                    balance = mean unique / max unique
 * Errors: KDA_ERR_ARG, KDA_ERR_TREE (malformed tree, budget <= 0).
 */
int kda_l1_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len, int64_t budget,
                int32_t* leaf_mb, int32_t* n_mb, int64_t* mb_unique, int64_t* mb_expanded);

/* Sizes and counts of a plan.  Host pointers. */
int kda_plan_info(const kda_plan* plan, kda_plan_info_t* info);

/*
 * kda_plan_export -- copy one canonical plan array to host memory as int64.
 * Returns the array length (>= 0) when dst is NULL or n >= length, else a
 * KDA_ERR_*.  Arrays:
 *   SEG_*      per segment: round, sequence, 1 if a direct continuation,
 *              start b of a side/root sequence (-1 for continuations), replay r
 *   ROUND_SEQ_PTR  [n_rounds+1] sequences of each round (sequence order)
 *   SEQ_*      per sequence: round, head segment, leaf index, start position
 *              b_head, replay rows, packed-row and chunk ranges ([n_seq+1]),
 *              init kind (0 root h0, 1 handoff buffer) and index
 *   CHUNK_*    per chunk: sequence, first packed row, rows (<= B), handoff
 *              buffer saved at its end (-1 none)
 *   ROW_INDEX  per packed row: compact row read;  OUT_ROW: row written (-1 replay)
 *   BUF_*      per handoff buffer: producer sequence, trajectory position,
 *              chunk whose end it is, consumer sequences (CSR)
 *   POS_ROW, POS_NEXT_ROW  gather map (trajectories by leaf id, positions
 *              0..L-2): row of the position and row of its next token;
 *   ROW_POS_PTR/IDX  positions of every compact row (CSR, ascending)
 *   LEAF_SEG, ROOT_SEG  leaf and root segment ids, ascending
 *   ROW_MULT   per compact row: its occurrence count, the number of
 *              root-to-leaf trajectories through it
 *   SEQ_LPT    per round (indexed like the sequences): the round's sequence
 *              ids in the order the round kernels launch them, most chunks
 *              first, ties by id (a scheduling order only; results do not
 *              depend on it)
 */
enum {
  KDA_F_SEG_ROUND = 0, KDA_F_SEG_SEQ, KDA_F_SEG_IS_CONT, KDA_F_SEG_B, KDA_F_SEG_REPLAY,
  KDA_F_ROUND_SEQ_PTR, KDA_F_SEQ_ROUND, KDA_F_SEQ_HEAD, KDA_F_SEQ_LEAF, KDA_F_SEQ_B_HEAD,
  KDA_F_SEQ_REPLAY, KDA_F_SEQ_ROW_PTR, KDA_F_SEQ_CHUNK_PTR, KDA_F_SEQ_INIT_KIND,
  KDA_F_SEQ_INIT_IDX, KDA_F_CHUNK_SEQ, KDA_F_CHUNK_ROW0, KDA_F_CHUNK_LEN, KDA_F_CHUNK_SAVE,
  KDA_F_ROW_INDEX, KDA_F_OUT_ROW, KDA_F_BUF_SEQ, KDA_F_BUF_POS, KDA_F_BUF_CHUNK,
  KDA_F_BUF_CONS_PTR, KDA_F_BUF_CONS, KDA_F_POS_ROW, KDA_F_POS_NEXT_ROW, KDA_F_ROW_POS_PTR,
  KDA_F_ROW_POS_IDX, KDA_F_LEAF_SEG, KDA_F_ROOT_SEG,
  KDA_F_ATT_ANC_PTR, KDA_F_ATT_ANC, KDA_F_ATT_SEG_TILE0, KDA_F_ATT_TILE_SEG, KDA_F_ATT_TILE_OFF,
  KDA_F_ATT_QORDER, KDA_F_ATT_KQ_PTR, KDA_F_ATT_KQ, KDA_F_ATT_KW_TILE, KDA_F_ATT_KW_Q0,
  KDA_F_ATT_KW_NQ, KDA_F_ATT_KW_SLOT, KDA_F_ROW_MULT, KDA_F_SEQ_LPT,
  KDA_F_COUNT
};
int64_t kda_plan_export(const kda_plan* plan, int32_t field, int64_t* dst, int64_t n);

/*
 * kda_plan_upload -- copy the plan's int32 device tables into a caller-owned
 * device buffer of at least info.device_bytes bytes (256-byte aligned), with
 * an asynchronous host-to-device copy on `stream`.  The host staging memory
 * stays owned by the plan, so the plan must outlive the copy.  This is the
 * only host-to-device transfer of the library.
 */
int kda_plan_upload(const kda_plan* plan, void* dev, size_t bytes, void* stream);

/* Byte offset of an int32 table (KDA_F_POS_ROW, KDA_F_POS_NEXT_ROW,
 * KDA_F_ROW_POS_PTR, KDA_F_ROW_POS_IDX, KDA_F_ROW_INDEX, KDA_F_OUT_ROW,
 * KDA_F_ROW_MULT) inside the uploaded device copy, or a negative KDA_ERR_*. */
int64_t kda_plan_device_offset(const kda_plan* plan, int32_t field);

/*
 * Buffer sizes for kda_tree_fwd / kda_tree_bwd at head count H and head dims
 * dk, dv.  `saved` is written by the forward and read by the backward (an
 * fp16 copy of every chunk's start state, every handoff state in fp32, and
 * each chunk's state-independent operands); `ws` is scratch (any content on
 * entry).  Both are in bytes; 0 for an unsupported shape.
 */
size_t kda_saved_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv);
size_t kda_fwd_workspace_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv);
size_t kda_bwd_workspace_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv);

/*
 * kda_tree_fwd -- forward pass of tree-packed chunkwise KDA.
 *
 * Runs every packed round (one launch group per round, in stream order): each
 * sequence starts from its root's h0 or from a handoff state saved by an
 * earlier round, replays its leading rows without writing outputs, and
 * emits per-token outputs and its leaf's final state (Figure 1(b): linear
 * attention consumes a state and produces a branch-specific next state).
 *
 *   plan, dev_plan  the plan and its uploaded device copy
 *   H, dk, dv       heads and head dims; supported: dk = dv in {64, 128}
 *   in_dtype        dtype of q, k, v: KDA_DTYPE_BF16 or KDA_DTYPE_FP32
 *   scale           output scale (usually 1/sqrt(dk))
 *   q, k, v         [N,H,dk], [N,H,dk], [N,H,dv] compact rows (device)
 *   g               [N,H,dk] fp32 log-decay per channel (<= 0 expected)
 *   beta            [N,H] fp32 write strength
 *   h0              [n_root,H,dk,dv] fp32 initial states, or NULL for zeros
 *   o               [n_out_rows,H,dv] fp32 outputs (replay rows write nothing)
 *   h_leaf          [n_leaf,H,dk,dv] fp32 final state per leaf (leaves ascending)
 *   saved, saved_bytes  at least kda_saved_bytes(...) bytes, kept for kda_tree_bwd
 *   ws, ws_bytes    scratch of kda_fwd_workspace_bytes(...) bytes
 * Precision: the state products run on fp16 matrix-core operands with fp32
 * accumulation (the state itself stays fp32); the chunk start states kept in
 * `saved` are fp16.  Values v and start states h0 of magnitude 2^-12 .. 2^12
 * times unit scale keep the 2e-3 accuracy (the states then stay far inside
 * fp16 range); far larger values overflow fp16 and far smaller ones lose
 * precision.
 * Gates: any finite g <= 0.  The chunk math factors per-pair decays through
 * the first row of each 16-row block; rows whose decay from that row exceeds
 * 64 (from the first such row of a chunk on) take exact per-pair
 * exponentials instead, chosen from the rows up to them, so replayed chunks
 * still give the trajectory-expanded bits.
 * Errors: KDA_ERR_SHAPE, KDA_ERR_WORKSPACE, KDA_ERR_ARG, KDA_ERR_HIP.
 */
int kda_tree_fwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t dk, int32_t dv,
                 int32_t in_dtype, float scale, const void* q, const void* k, const void* v,
                 const float* g, const float* beta, const float* h0, float* o, float* h_leaf,
                 void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * kda_set_overlap -- process-wide launch policy of kda_tree_fwd / kda_tree_bwd.
 *
 * With enable != 0 (the default) the chunk-parallel passes of a call run on a
 * second stream of the device beside the sequential per-round passes (the
 * rounds of Figure 2(c) form a chain; the chunk passes do not), forked from
 * and joined back into the caller's stream.  With enable == 0 every kernel of
 * a call runs on the caller's stream in order.  Results are bitwise the same
 * either way.  Takes effect for calls made after it returns.  Returns KDA_OK.
 */
int kda_set_overlap(int32_t enable);

/*
 * kda_tree_bwd -- reverse mode of kda_tree_fwd (rounds in reverse order).
 *
 * Gradients flow back through every handoff (abstract: differentiable
 * boundary-state handoff): a handoff state's gradient is the sum of its own
 * sequence's continuation gradient and the start gradients of every
 * sequence that started from it, added in a fixed order.  Gradients of
 * replayed rows are added into the compact rows they were read from, in a
 * fixed order.
 *
 *   q..h0      the forward's inputs (same pointers or equal contents)
 *   saved, saved_bytes  as written by kda_tree_fwd with the same inputs (size
 *              at least kda_saved_bytes(...))
 *   dO         [n_out_rows,H,dv] output gradients, dtype in_dtype
 *   dh_leaf    [n_leaf,H,dk,dv] fp32 gradient of each leaf state, or NULL for zeros
 *   dq, dk     [n_out_rows,H,dk] fp32;  dv [n_out_rows,H,dv] fp32
 *   dg         [n_out_rows,H,dk] fp32;  dbeta [n_out_rows,H] fp32
 *   dh0        [n_root,H,dk,dv] fp32 gradient of each root state
 *   dh_boundary [n_buf,H,dk,dv] fp32 total gradient of each handoff state, or NULL
 *   ws, ws_bytes scratch of kda_bwd_workspace_bytes(...) bytes
 * Range: the state gradients, the per-chunk dO and dy are fp16 matrix-core
 * operands; the call first finds the largest |dO| * scale and |dh_leaf| and
 * runs in units of a power of two that brings it to [8, 16), dividing every
 * gradient by that power of two on output (exact).  Upstream gradients of
 * any magnitude (a loss averaged over many positions, a scaled loss) give
 * the same relative accuracy, and a call with dO and dh_leaf times 2^e
 * returns exactly 2^e times the gradients.
 * Errors: as kda_tree_fwd.
 */
int kda_tree_bwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t dk, int32_t dv,
                 int32_t in_dtype, float scale, const void* q, const void* k, const void* v,
                 const float* g, const float* beta, const float* h0, const void* saved,
                 size_t saved_bytes, const void* dO, const float* dh_leaf, float* dq, float* dk_,
                 float* dv_, float* dg, float* dbeta, float* dh0, float* dh_boundary, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * gather_logprobs -- per-original-position log-probs from compact logit rows
 * (abstract: recovering log-probabilities for each original trajectory
 * position; Figure 1: one logit row serves several trajectories' targets;
 * Figure C.1(d): no expanded vocabulary-sized logits).
 *
 *   logits      [n_rows, vocab] (dtype KDA_DTYPE_BF16 or KDA_DTYPE_FP32), device
 *   pos_row     [n_pos] int32 compact row of each position (device)
 *   pos_target  [n_pos] int32 target token id of each position, in [0, vocab)
 *   logp        [n_pos] fp32 out: logits[row, tgt] - logsumexp(logits[row, :])
 *   lse         [n_rows] fp32 out: logsumexp of every row
 * Errors: KDA_ERR_ARG, KDA_ERR_SHAPE, KDA_ERR_HIP.
 */
int gather_logprobs(const void* logits, int32_t dtype, int64_t n_rows, int32_t vocab,
                    const int32_t* pos_row, const int32_t* pos_target, int64_t n_pos,
                    float* logp, float* lse, void* stream);

/*
 * gather_logprobs_bwd -- gradient of the logits for gather_logprobs:
 *   dlogits[r, :] = sum over positions p of row r, in CSR order, of
 *                   dlogp[p] * (onehot(pos_target[p]) - softmax(logits[r, :])).
 *   row_pos_ptr [n_rows+1], row_pos_idx [n_pos] int32: positions of each row
 *   (the plan exports them in ascending position order).
 *   lse         [n_rows] from gather_logprobs;  dlogp [n_pos] fp32
 *   dlogits     [n_rows, vocab], same dtype as logits; every element is written.
 */
int gather_logprobs_bwd(const void* logits, int32_t dtype, int64_t n_rows, int32_t vocab,
                        const float* lse, const int32_t* row_pos_ptr,
                        const int32_t* row_pos_idx, const int32_t* pos_target,
                        const float* dlogp, void* dlogits, void* stream);

/*
 * moe_router_stats -- router statistics of the trajectory-expanded batch from
 * compact rows weighted by their occurrence counts (HARTS abstract: with
 * deterministic top-k routing and no token dropping, occurrence counts
 * restore MoE objective weights and expert-load statistics; Figure 1
 * caption, q_B = 2 for a row shared by two trajectories; Figure C.1(d)).
 * A row read by q trajectory positions counts q times:
 *   load[e]  = sum_r q_r [e in topk(x_r)]     (int64, exact)
 *   psum[e]  = sum_r q_r softmax(x_r)[e]       (fp32)
 *   zsum[0]  = sum_r q_r logsumexp(x_r)^2      (fp32)
 *   n_tok[0] = sum_r q_r                       (int64: expanded positions)
 * from which a load-balancing loss E sum_e load[e]/(k n_tok) psum[e]/n_tok
 * and a z-loss zsum/n_tok follow.  topk(x): the top_k largest logits, equal
 * logits by the lower expert index.  Every sum has a fixed order: the results
 * are bitwise reproducible.
 *
 *   logits      [n_rows, n_experts] bf16 or fp32 (dtype), device
 *   n_experts   64, 128, 256 or 512;  top_k in [1, min(32, n_experts)]
 *   row_mult    [n_rows] int32 occurrence counts (device; the plan's
 *               KDA_F_ROW_MULT table, see kda_plan_device_offset)
 *   topk_idx    [n_rows, top_k] int32 out, or NULL: chosen experts, in order
 *   topk_prob   [n_rows, top_k] fp32 out, or NULL: their softmax probabilities
 *   load, psum  [n_experts] int64 / fp32 out (device);  zsum [1] fp32,
 *               n_tok [1] int64 out (device)
 *   ws          moe_router_workspace_bytes(n_rows, n_experts) bytes of scratch
 * Errors: KDA_ERR_ARG, KDA_ERR_SHAPE, KDA_ERR_WORKSPACE, KDA_ERR_HIP.
 */
size_t moe_router_workspace_bytes(int64_t n_rows, int32_t n_experts);
int moe_router_stats(const void* logits, int32_t dtype, int64_t n_rows, int32_t n_experts,
                     int32_t top_k, const int32_t* row_mult, int32_t* topk_idx, float* topk_prob,
                     int64_t* load, float* psum, float* zsum, int64_t* n_tok, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * moe_router_stats_noalloc -- moe_router_stats without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and errors as moe_router_stats, bitwise the same
 * results; the block partials go to a scratch array built into the library
 * (8,404,992 bytes per device, the most any call needs: at most 2048 blocks
 * of n_experts + 1 partials), held by each device the library runs on until
 * the process ends; its device address is looked up on the first call on
 * each device.  The call allocates nothing.  Every call on one device uses
 * the same scratch (each call writes every partial before it reads it), so
 * calls that overlap on one device -- on different streams, or from
 * different threads without ordering -- race and must not be made.  Errors:
 * as moe_router_stats; KDA_ERR_WORKSPACE if a call would need more scratch
 * than the array holds, KDA_ERR_HIP if the scratch lookup fails.
 */
int moe_router_stats_noalloc(const void* logits, int32_t dtype, int64_t n_rows,
                             int32_t n_experts, int32_t top_k, const int32_t* row_mult,
                             int32_t* topk_idx, float* topk_prob, int64_t* load, float* psum,
                             float* zsum, int64_t* n_tok, void* stream);

/*
 * moe_router_stats_bwd -- gradient of L = <g_psum, psum> + g_z * zsum with
 * respect to the logits (top-k membership carries none):
 *   dlogits[r, :] = q_r * p_r * (g_psum - <p_r, g_psum> + 2 g_z lse_r),
 *   p_r = softmax(x_r), lse_r = logsumexp(x_r).
 *   g_psum [n_experts] fp32 (device);  dlogits [n_rows, n_experts] fp32 out.
 * Errors: KDA_ERR_ARG, KDA_ERR_SHAPE, KDA_ERR_HIP.
 */
int moe_router_stats_bwd(const void* logits, int32_t dtype, int64_t n_rows, int32_t n_experts,
                         const int32_t* row_mult, const float* g_psum, float g_z, float* dlogits,
                         void* stream);

/*
 * Tree-ancestor softmax attention over the plan's compact rows (the full
 * attention layers of the hybrid model: thelatestinai.com Figure 1(b), full
 * attention reads ancestor keys and values; Figure C.1(c)).  The query of the
 * row at offset i of segment v sees every row of every ancestor segment of v
 * and the rows of v at offsets <= i -- its root path up to itself -- so one
 * compact row serves every trajectory through it:
 *     o_r = sum_j softmax_j(scale q_r . k_j) v_j,   lse_r = logsumexp_j(scale q_r . k_j)
 * Multi-head, H heads of dimension d in {64, 128}.
 *   q, k, v  [n_rows, H, d] bf16 (compact rows, as the plan's tree)
 *   o        [n_rows, H, d] fp32;  lse [n_rows, H] fp32
 * tree_attn_bwd: gradients of sum(dO * o): dO [n_rows, H, d] bf16, o and lse
 *   from tree_attn_fwd; dq, dk, dv [n_rows, H, d] fp32, every element written;
 *   ws of tree_attn_workspace_bytes(plan, H, d) bytes (row deltas and partial
 *   sums of key tiles whose queries are split over several blocks; summed in
 *   a fixed order, so results are deterministic).
 * scale must be positive and finite (the kernels take each query's running
 * maximum over unscaled scores).
 * Tensors, o and ws are 16-byte aligned, lse 4-byte aligned (rows move in
 * 16-byte vectors).
 * Errors: KDA_ERR_SHAPE for other head dims, KDA_ERR_ARG for null or
 * misaligned pointers or a scale that is not positive and finite,
 * KDA_ERR_WORKSPACE for a small workspace, KDA_ERR_HIP for launch failures.
 */
size_t tree_attn_workspace_bytes(const kda_plan* plan, int32_t H, int32_t d);
int tree_attn_fwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t d, float scale,
                  const void* q, const void* k, const void* v, float* o, float* lse, void* stream);
int tree_attn_bwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t d, float scale,
                  const void* q, const void* k, const void* v, const float* o, const float* lse,
                  const void* dO, float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * Launch timing for benchmarks and profilers (not needed for computing).
 * kda_timing_enable(1) clears the counters and makes every later kernel launch
 * of the library record a pair of hipEvents around it on its launch stream
 * (the events are created by the library and reused); kda_timing_enable(0)
 * stops recording.  kda_timing_read(idx, ...) synchronises the recorded events
 * and returns, for kernel class idx, its name, the number of timed launches
 * and their summed duration in milliseconds; it returns the number of kernel
 * classes (call with idx < 0 to get the count only), or KDA_ERR_ARG.
 * kda_timing_filter(name) limits the recording to launches of that kernel
 * class (NULL or "" : every class), so that a timed region carries only the
 * events it needs; it applies from the next launch on.
 */
int kda_timing_enable(int32_t on);
int kda_timing_filter(const char* name);
int kda_timing_read(int32_t idx, char* name, int32_t name_len, int64_t* launches,
                    double* total_ms);

/* Message of the last failed call on this thread ("" if none). */
const char* kda_last_error(void);

/*
 * Sharing windows (thelatestinai.com Figure 3; HARTS abstract): a producer
 * call computes a shared prefix once and consumer microbatches start from its
 * end states; within the window the gradients of the consumers' start states
 * accumulate into the producer's end-state gradients before the one producer
 * backward.  The calls are kda_tree_fwd / kda_tree_bwd on separate plans
 * (consumer roots take their h0 from the producer's h_leaf); these two calls
 * move and sum the states between them.  A state is `elems` floats (H*dk*dv,
 * a multiple of 4); src and dst are device pointers, 16-byte aligned; index
 * arrays are device int32 arrays.  Stream-ordered; no allocation.
 *
 * kda_state_copy: dst[dst_idx[i]] = src[src_idx[i]] for i < n (a NULL index
 *   array is the identity).  Used to hand producer end states to consumer
 *   roots and to scatter leaf states into a whole-tree array.
 * kda_state_sum: dst[d] = (accumulate ? dst[d] : 0) + sum of src[idx[j]] over
 *   j in [ptr[d], ptr[d+1]) in ascending j, for d < n_dst (an empty range
 *   gives dst[d] or 0).  Fixed order: bitwise deterministic.  Used to
 *   accumulate consumer start-state gradients into the producer's end-state
 *   gradients, one microbatch after another.
 * Errors: KDA_ERR_ARG (bad sizes, null or misaligned pointers), KDA_ERR_HIP.
 */
int kda_state_copy(const float* src, const int32_t* src_idx, float* dst, const int32_t* dst_idx,
                   int32_t n, int64_t elems, void* stream);
int kda_state_sum(const float* src, const int32_t* ptr, const int32_t* idx, int32_t n_dst,
                  int64_t elems, int32_t accumulate, float* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_TREE_H */
