/*
 * gdn.h -- C ABI of the Gated DeltaNet recurrent-state library for MI355X
 * (gfx950): speculative-draft verify over a chain or a tree, commit of the
 * accepted node, and chunked prefill.
 *
 * The recurrence, per (sequence, value head), with S the d_v x d_k state:
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t                     (read after the update)
 * This is the gated delta rule of a Gated DeltaNet layer, the layer of the
 * page "LightSeek's TokenSpeed Hits 580 Tokens per Second on Qwen3.5's 400B
 * Model", section "Why Qwen3.5 is hard to serve fast": a fixed state of
 * head-dimension-squared size per layer, updated per token, with the output
 * read from the current state.  The page states it in words; the formula
 * above is this library's definition of it.
 *
 * Conventions for every entry point
 *  - All tensors are dense, C-contiguous, in device memory, with these
 *    layouts (B = shape.batch, N = shape.n_nodes):
 *        q, k         [B][N][h_qk][d_k]      qkv_dtype (F32 or BF16)
 *        v            [B][N][h_v][d_v]       qkv_dtype
 *        alpha, beta  [B][N][h_v]            fp32
 *        state        [n_slots][h_v][d_v][d_k] fp32   (row j = value channel j)
 *        state_slot   [B] int32, nullable: sequence b uses state[state_slot[b]];
 *                     NULL means sequence b uses state[b]
 *        out          [B][N][h_v][d_v]       out_dtype (F32, F16 or BF16)
 *        persist      [B][N][h_v][d_v][d_k]  persist_dtype (F16 or F32)
 *        final_state  [B][h_v][d_v][d_k]     fp32
 *    Value head h reads q/k head h / (h_v / h_qk).
 *  - q, k, v, state, persist and final_state must be 16-byte aligned; the
 *    other pointers 4-byte aligned.
 *  - The caller owns every buffer.  The library allocates no memory and is
 *    safe to call from several host threads.  Its only host-side state is
 *    set once per device and never changes afterwards: the compute-unit count
 *    it reads, and the attribute that lets a kernel use all of a compute
 *    unit's LDS (both behind atomics).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return; they never synchronise the host.
 *  - Errors found on the host (null or misaligned pointers, bad shapes or
 *    dtypes, bad parent arrays, small workspace) return a negative
 *    gdn_status before anything is enqueued; no buffer is touched.
 *    Errors only the device can see (an out-of-range accepted node or state
 *    slot) skip that sequence, leave its buffers untouched and store the
 *    code into *status when `status` is not NULL.  The caller zeroes
 *    *status beforehand; concurrent errors leave one of their codes.
 *  - A failed kernel launch returns GDN_ERR_HIP.
 *  - The library built with -DGDN_DEBUG (libgdn_debug.so) checks the indices
 *    its kernels form into the caller's arrays and the workspace: one past
 *    its array's end stores GDN_ERR_INTERNAL into *status and is clamped into
 *    the array.  The release build carries no such checks.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_MAX_NODES 32      /* draft nodes per verify call (a 22-node tree plus margin) */
#define GDN_MAX_TREE_DEPTH 16 /* nodes on a root-to-leaf path, root included */
#define GDN_PREFILL_CHUNK 64  /* tokens per chunk of gdn_prefill_chunked */
#define GDN_MAX_CONV_WIDTH 8  /* taps of the causal convolution whose history gdn_conv_commit keeps */

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    GDN_ERR_DTYPE = -3,       /* a dtype code is not allowed where it was given */
    GDN_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
    GDN_ERR_PARENT = -5,      /* the parent array is not a valid tree */
    GDN_ERR_NODE = -6,        /* device: accepted node outside [0, N) */
    GDN_ERR_WORKSPACE = -7,   /* workspace missing or too small */
    GDN_ERR_UNSUPPORTED = -8, /* valid request this library does not implement */
    GDN_ERR_HIP = -9,         /* the HIP runtime refused the launch */
    GDN_ERR_SLOT = -10,       /* device: state slot outside [0, n_slots) */
    GDN_ERR_RANGE = -11,      /* device: a prefill value left the f16 range of the matrix-core operands */
    GDN_ERR_INTERNAL = -12    /* device, debug build only: an index check inside a kernel failed */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype;

typedef struct gdn_shape {
    int32_t batch;         /* independent sequences (or sequence x layer units), >= 0 */
    int32_t n_nodes;       /* draft nodes per sequence; tokens per sequence for prefill */
    int32_t h_qk;          /* q/k heads, >= 1 */
    int32_t h_v;           /* value heads, a multiple of h_qk; verify and commit by replay need
                              h_v * d_v * d_k * GDN_MAX_NODES < 2^32 */
    int32_t d_k;           /* key channels: 32, 64 or 128 */
    int32_t d_v;           /* value channels: a multiple of 16, at most 256 */
    int32_t n_slots;       /* rows of `state` when state_slot is given (ignored otherwise) */
    int32_t qkv_dtype;     /* GDN_F32 or GDN_BF16 */
    int32_t out_dtype;     /* GDN_F32, GDN_F16 or GDN_BF16 */
    int32_t persist_dtype; /* GDN_F16 or GDN_F32 */
    float scale;           /* output scale; 1 for the plain rule */
} gdn_shape;

/*
 * Verify a causal chain of N draft nodes per sequence.
 * Page "400 tok/s with Qwen3.5", sections "Speculative verification in a
 * megakernel" and "Handling recurrent state": the target checks a block of
 * draft tokens in one causal pass, keeping the recurrent working state on
 * chip across the block.
 *
 * Node n of sequence b starts from node n-1 (node 0 from the cached state
 * state[slot(b)], which is only read).  For every node the output goes to
 * out (nullable) and the state after the node to persist (nullable), stored
 * in persist_dtype with round-to-nearest-even: page "We got 207 tok/s with
 * Qwen3.5-27B on an RTX 3090", section "Key wins" (an f16 per-node cache,
 * written by the recurrence kernel itself).  The fp32 state after node N-1
 * goes to final_state (nullable), exactly as computed.  final_state may be
 * `state` itself (in-place advance) when state_slot is NULL.
 */
int gdn_verify_chain(const gdn_shape* shape, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* state,
                     const int32_t* state_slot, void* out, void* persist, float* final_state,
                     int32_t* status, void* stream);

/*
 * One launch for a decode step: commit the previous step's accepted node, then
 * verify the next chain from the committed state.  Equivalent to
 *     gdn_commit(shape, accepted_prev, persist_prev, final_prev, state, state_slot, status)
 *     gdn_verify_chain(shape, q, k, v, alpha, beta, state, state_slot, out, persist,
 *                      final_state, status)
 * with the commit fused into the verify's state load, so the committed state is
 * read once (as the f16 node copy, or final_prev on full acceptance), written to
 * state[slot(b)] and used directly.  Page "400 tok/s with Qwen3.5", section
 * "Handling recurrent state" (state set to the accepted boundary before the next
 * verification).
 *
 * persist_prev and final_prev (nullable) are the previous step's persist and
 * final_state: same layout, n_nodes and persist_dtype as this call's outputs.
 * They may be the very buffers this call writes (each value is read before it
 * is overwritten).  accepted_prev is a device array [B]; a node outside [0, N)
 * skips the sequence entirely (state and outputs untouched) and sets *status to
 * GDN_ERR_NODE.  Other arguments and errors as gdn_verify_chain; final_state
 * may not be `state` here.
 */
int gdn_commit_verify_chain(const gdn_shape* shape, const int32_t* accepted_prev, const void* persist_prev,
                            const float* final_prev, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                            void* out, void* persist, float* final_state, int32_t* status, void* stream);

/*
 * Verify a tree of N draft nodes per sequence.
 * Page "Qwen3.6 27B: From 20 t/s to 184 t/s", section "Diffusion applied to
 * text": a best-first tree of up to 22 nodes is verified in one target pass.
 *
 * `parent` is a HOST array of n_trees x N int32, n_trees = 1 (one tree for
 * every sequence) or batch (one per sequence).  parent[0] = -1 (node 0, the
 * root, starts from the cached state); for n >= 1, 0 <= parent[n] < n; no
 * root-to-leaf path holds more than GDN_MAX_TREE_DEPTH nodes.  Node n starts
 * from the exact fp32 state of node parent[n]; outputs and persisted states
 * are indexed by node.  The array is read during the call only.
 */
int gdn_verify_tree(const gdn_shape* shape, const int32_t* parent, int32_t n_trees, const void* q,
                    const void* k, const void* v, const float* alpha, const float* beta,
                    const float* state, const int32_t* state_slot, void* out, void* persist,
                    int32_t* status, void* stream);

/*
 * One launch for a tree decode step: commit the previous step's accepted node,
 * then verify the next tree from the committed state.  Equivalent to
 *     gdn_commit(shape, accepted_prev, persist_prev, NULL, state, state_slot, status)
 *     gdn_verify_tree(shape, parent, n_trees, q, k, v, alpha, beta, state, state_slot,
 *                     out, persist, status)
 * with the commit fused into the verify's state load: the accepted node's
 * persisted copy is read once, widened to fp32, written to state[slot(b)] and
 * used directly as the root's starting state.  Page "400 tok/s with Qwen3.5",
 * section "Handling recurrent state" (state set to the accepted boundary before
 * the next verification); page "Qwen3.6 27B: From 20 t/s to 184 t/s", section
 * "Diffusion applied to text" (the tree verified in one pass).
 *
 * persist_prev is the previous step's persist: same layout, n_nodes and
 * persist_dtype as this call's; it may be the very buffer this call writes
 * (each value is read before it is overwritten).  accepted_prev is a device
 * array [B] of node indices of the previous step (the last node of its accepted
 * path); a node outside [0, N) skips the sequence entirely (state and outputs
 * untouched) and sets *status to GDN_ERR_NODE.  parent, n_trees and the other
 * arguments and errors as gdn_verify_tree.
 */
int gdn_commit_verify_tree(const gdn_shape* shape, const int32_t* accepted_prev, const void* persist_prev,
                           const int32_t* parent, int32_t n_trees, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                           void* out, void* persist, int32_t* status, void* stream);

/*
 * Commit the accepted node of every sequence into the state cache.
 * Page "400 tok/s with Qwen3.5", section "Handling recurrent state": after a
 * rejection the state is set to the accepted boundary; a fully accepted
 * block uses the verified state directly.
 *
 * accepted_node is a DEVICE array [B] of node indices (node L-1 for an
 * accepted chain prefix of length L; the last node of the accepted path in a
 * tree).  state[slot(b)] <- persist[b][a] widened to fp32, or final_state[b]
 * when final_state is not NULL and a = N-1.  Only shape.batch, n_nodes, h_v,
 * d_k, d_v, n_slots and persist_dtype are read.  An accepted node outside
 * [0, N) or a slot outside [0, n_slots) skips the sequence and sets *status.
 */
int gdn_commit(const gdn_shape* shape, const int32_t* accepted_node, const void* persist,
               const float* final_state, float* state, const int32_t* state_slot,
               int32_t* status, void* stream);

/*
 * Commit by replay: set the cached state to the accepted node's state by
 * running the recurrence again over the accepted nodes, from the state the
 * block was verified from, with the block's retained inputs.  Page "400 tok/s
 * with Qwen3.5", section "Handling recurrent state" (checkpoint-and-replay: the
 * state from before the draft block is kept with the projected inputs, and a
 * replay kernel advances it through the accepted positions only).  With this
 * commit a verify needs to persist no node states (persist = NULL).
 *
 * On entry state[slot(b)] is the state the block was verified from (the
 * checkpoint); on return it is the fp32 state after node accepted_node[b]
 * (device array [B]).  The nodes replayed are the node's root path: nodes
 * 0 .. a of a chain (parent == NULL), or the ancestors of a, root first, of a
 * tree (parent: HOST array as in gdn_verify_tree, n_trees x N with n_trees = 1
 * or batch).  The arithmetic per node is the verify's, so the result equals
 * bit for bit the fp32 node state that gdn_verify_chain / gdn_verify_tree
 * persist with persist_dtype F32 for the same inputs.  q, k, v, alpha, beta are
 * the block's inputs, laid out as for verify.  No outputs are written;
 * shape.out_dtype, persist_dtype and scale are not used.  A node outside
 * [0, N) or a slot outside [0, n_slots) skips the sequence (its state is left
 * as it was) and sets *status.
 */
int gdn_commit_replay(const gdn_shape* shape, const int32_t* parent, int32_t n_trees,
                      const int32_t* accepted_node, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                      int32_t* status, void* stream);

/*
 * One launch for a decode step with commit by replay: replay the previous chain
 * block's accepted nodes (as gdn_commit_replay with parent = NULL, inputs
 * q_prev .. beta_prev and accepted_prev), write the result to state[slot(b)],
 * then verify the next chain (q .. beta) from it, as gdn_verify_chain would
 * from the updated cache.  Page "400 tok/s with Qwen3.5", section "Handling
 * recurrent state".  The replayed state never leaves registers between the
 * two.  persist is usually NULL in this scheme (nothing to persist: the next
 * step replays); out and final_state are as in gdn_verify_chain, and
 * final_state may not be `state`.  The previous block has this call's shape.
 * An accepted node outside [0, N) skips the sequence entirely (state and
 * outputs untouched) and sets *status to GDN_ERR_NODE.
 */
int gdn_replay_verify_chain(const gdn_shape* shape, const int32_t* accepted_prev, const void* q_prev,
                            const void* k_prev, const void* v_prev, const float* alpha_prev,
                            const float* beta_prev, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                            void* out, void* persist, float* final_state, int32_t* status, void* stream);

/*
 * Index-table commit: commit the accepted node by pointing the sequence's
 * index-table entry at the row that already holds its state, instead of
 * copying the state.  Page "LightSeek's TokenSpeed Hits 580 Tokens per Second
 * on Qwen3.5's 400B Model", section "How they actually got there" (move
 * pointers, not data: the state buffer gains a draft region, and an index
 * table records which row holds each sequence's state).
 *
 * Protocol.  `state` is a pool [n_slots][h_v][d_v][d_k] fp32 whose rows
 * draft_row0 .. draft_row0 + B N - 1 form the draft region; state_slot [B] is
 * the index table.  gdn_verify_chain / gdn_verify_tree are called with this
 * state_slot and with persist = the pool's row draft_row0 (persist_dtype F32),
 * so node n of sequence b is persisted, exactly, in row draft_row0 + b N + n.
 * A verify may persist over the row it reads its state from: every element is
 * read before it is written.  gdn_commit_index then sets, on the device,
 *     state_slot[b] <- draft_row0 + b N + accepted_node[b]
 * and the next verify reads the accepted node's exact fp32 state from there.
 * accepted_node and state_slot are DEVICE arrays [B]; draft_row0 + B N must
 * not exceed n_slots.  An accepted node outside [0, n_nodes) leaves the entry
 * as it was and sets *status to GDN_ERR_NODE.
 */
int gdn_commit_index(const int32_t* accepted_node, int32_t* state_slot, int32_t batch, int32_t n_nodes,
                     int32_t draft_row0, int32_t n_slots, int32_t* status, void* stream);

/* Shape of a causal-convolution history commit. */
typedef struct gdn_conv_shape {
    int32_t batch;    /* sequences, >= 0 */
    int32_t n_nodes;  /* draft nodes per sequence, 1 .. GDN_MAX_NODES */
    int32_t channels; /* C, input channels of the convolution; C * element size a multiple of 16 bytes */
    int32_t width;    /* W, taps of the convolution, 2 .. GDN_MAX_CONV_WIDTH; the history keeps W - 1 rows */
    int32_t n_slots;  /* rows of conv_state when state_slot is given (ignored otherwise) */
    int32_t dtype;    /* element type of x and conv_state: GDN_F32, GDN_BF16 or GDN_F16 (bytes are copied) */
} gdn_conv_shape;

/*
 * Commit the causal-convolution input history to the accepted boundary.
 * Page "400 tok/s with Qwen3.5", section "Handling recurrent state": the
 * convolution history is committed to the same boundary as the recurrent
 * state.  A causal convolution of width W reads the current input row and the
 * W - 1 before it, so each sequence keeps its last W - 1 input rows:
 *     conv_state [n_slots][W-1][C]   oldest row first (16-byte aligned)
 *     x          [B][N][C]           the draft block's convolution inputs
 * On return conv_state[slot(b)] holds the last W - 1 rows of the accepted
 * stream: the previous history rows followed by the inputs of the nodes on
 * accepted_node[b]'s root path, root first (nodes 0 .. a of a chain when
 * parent == NULL; parent as in gdn_verify_tree otherwise, n_trees = 1 or
 * batch).  Rows are copied bit for bit.  accepted_node is a DEVICE array [B];
 * a node outside [0, N) or a slot outside [0, n_slots) skips the sequence and
 * sets *status.
 */
int gdn_conv_commit(const gdn_conv_shape* shape, const int32_t* parent, int32_t n_trees,
                    const int32_t* accepted_node, const void* x, void* conv_state,
                    const int32_t* state_slot, int32_t* status, void* stream);

/*
 * Chunked prefill of a prompt: the same recurrence over shape.n_nodes = T
 * tokens per sequence, evaluated GDN_PREFILL_CHUNK tokens at a time in the
 * WY / UT form.  Page "We got 207 tok/s with Qwen3.5-27B on an RTX 3090",
 * section "Prefill" (prompts are processed in micro-batches of tokens); the
 * chunk algebra is derived from the rule (see the kernel source).
 *
 * q, k [B][T][h_qk][d_k], v [B][T][h_v][d_v] (qkv_dtype F32 or BF16; values
 * are converted to f16 for the matrix cores, so they must lie inside the f16
 * range, |x| <= 65504, and magnitudes below 2^-14 keep an absolute precision
 * of 2^-25).  A q or k element outside that range, or a value of the
 * recurrence that leaves it on the way (from v, the state or the initial
 * state, which then leaves the final state non-finite), sets *status to
 * GDN_ERR_RANGE when status is not NULL; the outputs and the state of that
 * call are then not meaningful;
 * alpha, beta [B][T][h_v] fp32; out [B][T][h_v][d_v] in out_dtype (F32, F16
 * or BF16), 16-byte aligned.  state[slot(b)] holds the initial state on entry and the state
 * after token T-1 on return (updated in place).  A zero alpha resets the state
 * up to a factor e^-80 (the log-gate is clamped at -80).  d_k must be 32, 64 or
 * 128, d_v a multiple of 32 and h_v / h_qk at most 128 (else GDN_ERR_UNSUPPORTED).
 * persist_dtype is ignored.  T = 0 or batch = 0
 * is a no-op.
 *
 * `workspace` is caller-owned device memory of at least
 * gdn_prefill_workspace_bytes(shape) bytes (16-byte aligned), used during the
 * call for the per-chunk operands that do not depend on the state (the UT
 * transform and masked Q K^T per chunk and value head in f16, the gate factors,
 * K and Q in f16 per chunk and q/k head); about 1.3 MB per 64 tokens at 48 value
 * heads, 16 q/k heads and d_k = 128.  Its contents on entry are ignored.  A missing or short workspace
 * returns GDN_ERR_WORKSPACE.  Calls sharing one workspace must be ordered on
 * one stream.
 */
size_t gdn_prefill_workspace_bytes(const gdn_shape* shape);
int gdn_prefill_chunked(const gdn_shape* shape, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, float* state,
                        const int32_t* state_slot, void* out, void* workspace,
                        size_t workspace_bytes, int32_t* status, void* stream);

/*
 * gdn_prefill_chunked for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument.  The per-chunk operands go to a static
 * array of this library, GDN_PREFILL_SCRATCH_BYTES per GPU, which each GPU the
 * library runs on holds until the process ends.  A prompt whose workspace
 * (gdn_prefill_workspace_bytes) exceeds the array is processed in segments of
 * whole 64-token chunks, each a launch pair that reuses it; the results are
 * bit for bit those of gdn_prefill_chunked.  Heads so large that one 64-token
 * chunk does not fit return GDN_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU uses the same array: calls that may overlap on one GPU
 * (on different streams, or from several host threads without ordering) race
 * and must not be issued.  The call allocates nothing: no hipMalloc, hipFree
 * or allocating library routine.  Other arguments, limits and errors as
 * gdn_prefill_chunked.
 */
#define GDN_PREFILL_SCRATCH_BYTES (32u << 20)
int gdn_prefill_chunked_noalloc(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                                void* out, int32_t* status, void* stream);

/*
 * Varlen batched prefill with chunk-boundary states.  The same recurrence
 * and chunked evaluation as gdn_prefill_chunked, for `batch` sequences of
 * different lengths packed one after another along the token dimension, in
 * one call.  Page "LightSeek's TokenSpeed Hits 580 Tokens per Second on
 * Qwen3.5's 400B Model", section "How they actually got there" (hybrid prefix
 * caching needs the recurrent state at the exact prefix boundary): the call
 * can also emit the state at every state_interval-th chunk boundary.
 *
 * cu_seqlens is a HOST array [batch + 1]: 0 = cu[0] <= cu[1] <= ... <=
 * cu[batch] = shape.n_nodes (the total token count); sequence b holds tokens
 * cu[b] .. cu[b+1]-1 of
 *     q, k [total][h_qk][d_k],  v [total][h_v][d_v],  alpha, beta [total][h_v],
 *     out [total][h_v][d_v] (out_dtype, 16-byte aligned),
 * and state[slot(b)] (initial state in, final state out, in place; an empty
 * sequence keeps its state).  chunk_states (nullable, fp32, [n][h_v][d_v][d_k])
 * receives, sequence after sequence, the state after token
 * 64 state_interval m - 1 of the sequence for m = 1, 2, ... while that token
 * exists: n = gdn_prefill_boundary_states(cu_seqlens, batch, state_interval)
 * states in all.  state_interval >= 1 when chunk_states is set.  Sequences
 * are processed in launches of up to 64; the workspace (at least
 * gdn_prefill_varlen_workspace_bytes(shape, cu_seqlens) bytes) is reused by
 * each.  Other arguments, limits and errors as gdn_prefill_chunked; an
 * invalid cu_seqlens returns GDN_ERR_SHAPE (GDN_ERR_NULL if missing).
 */
size_t gdn_prefill_varlen_workspace_bytes(const gdn_shape* shape, const int32_t* cu_seqlens);
int64_t gdn_prefill_boundary_states(const int32_t* cu_seqlens, int32_t batch, int32_t state_interval);
int gdn_prefill_varlen(const gdn_shape* shape, const int32_t* cu_seqlens, const void* q, const void* k,
                       const void* v, const float* alpha, const float* beta, float* state,
                       const int32_t* state_slot, void* out, float* chunk_states, int32_t state_interval,
                       void* workspace, size_t workspace_bytes, int32_t* status, void* stream);

/*
 * Plan (and validate) the walk gdn_verify_tree takes through one tree.
 * Host-only; enqueues nothing.  Writes n_nodes steps to `walk` (host,
 * uint16 each): bits 0-4 the node, bit 5 "restore the parent's state from
 * fork slot bits 6-9 first", bit 10 "save the state to fork slot bits 11-14
 * after the node".  Nodes are visited depth first, children in index order;
 * a step without bit 5 continues from the previous step's state (node 0 from
 * the cached state).  *fork_slots receives the number of slots the walk
 * needs (at most GDN_MAX_TREE_DEPTH - 1).  Returns GDN_ERR_PARENT for an
 * invalid tree, with the rules of gdn_verify_tree.
 */
int gdn_tree_walk(const int32_t* parent, int32_t n_nodes, uint16_t* walk, int32_t* fork_slots);

/* Human-readable name of a gdn_status code (static storage). */
const char* gdn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
