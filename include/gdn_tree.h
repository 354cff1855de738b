/*
 * gdn_tree.h -- C ABI of libgdntree: verification of speculative draft trees
 * through Gated DeltaNet (GDN) layers on AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A batch holds B independent sequences. Sequence b carries a draft tree of
 * N_b nodes (1 <= N_b <= 64), flattened into one node order with the root
 * first and a parent index per node (-1 for the root, otherwise smaller than
 * the node's own index). The flattening with a parent index per node is the
 * input the GDN layers receive in the fork page's verify flow
 * (rainlin-top.pages.dev "Qwen3.5 tree spec", section 7 step 2); the -1 root
 * convention and the root-first order are the handbook's
 * (anrans.github.io ai-infra-handbooks "speculative", implementation section).
 *
 * Every node t of every head h gets the output the gated delta rule gives
 * when run from the sequence's initial state S0 along t's own root-to-node
 * path, and nothing else (siblings never see each other):
 *     S_t = alpha_t S_parent (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,       S_parent = S0 for the root.
 * (The state update formula is stripped from the fork page's section 3; this
 * is the gated delta rule the TreeWY abstract, arxivdaily 2608.20961, builds
 * on.) Commit then writes the state S_a of the one accepted node a per
 * sequence (fork page section 5, rollback to the last accepted token).
 *
 * Two modes compute the same results:
 *  - GDN_MODE_WY: tree-structured WY form. One unit-lower-triangular solve per
 *    (tree, head) yields pseudo-values u_t with
 *        S_t = G_t S0 + sum_{i in path(t)} (G_t/G_i) u_i k_i^T,
 *        G_t = product of alpha over path(t);
 *    verify stores only U and the gate prefixes; commit rebuilds S_a alone
 *    (TreeWY abstract: single triangular solve, pseudo-value matrix instead
 *    of per-node states, only the accepted state reconstructed).
 *  - GDN_MODE_FORK: the fork/checkpoint baseline. Depth-by-depth, every node
 *    starts from its parent's checkpoint and stores its own full state
 *    (fork page section 4, depth-by-depth subsection); commit copies the
 *    accepted node's checkpoint (section 5).
 *  - GDN_MODE_FORK_DELTA: the same depth-by-depth fork with delta-compressed
 *    checkpoints (fork page section 8, checkpoint compression): a node keeps
 *    only what its update adds to its parent's state, the rank-one term
 *    u_t k_t^T with u_t = beta_t (v_t - alpha_t S_parent k_t), and its gate.
 *    These u_t are exactly the WY pseudo-values, so the kept part of the
 *    workspace has the WY layout and commit is the WY commit; full states are
 *    kept only for nodes with children, while verify runs.
 *
 * Conventions (all entry points)
 * ------------------------------
 *  - Every pointer except `desc` is a DEVICE pointer owned by the caller. The
 *    library never allocates or frees memory and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream) and completes in stream order.
 *  - Dense row-major layouts, T = total nodes = offsets[B]:
 *      offsets [B+1] int32   node range of sequence b is [offsets[b], offsets[b+1])
 *      parents [T]   int32   local parent index within the sequence, root -1
 *      q, k    [T,H,dk]      io dtype (fp32 or bf16)
 *      v, o    [T,H,dv]      io dtype
 *      alpha, beta [T,H]     fp32; alpha in (0,1] (values below 2^-64 act as
 *                            2^-64), beta in [0,1]
 *      S0, S_out [B,H,dv,dk] fp32; S[r][c] multiplies k[c]
 *      tree_status [B] int32 per-sequence result code (GDN_TREE_*)
 *  - The gdn_status return value reports only host-side checks made before
 *    anything is enqueued (null pointers, shapes, dtype, workspace size) and
 *    launch failures. Data-dependent problems are reported per sequence in
 *    tree_status on the device; such a sequence's output rows are zero and
 *    its commit writes nothing.
 *  - Calls are re-entrant; nothing is kept between calls except what the
 *    caller's workspace holds. q, k, v, alpha, beta need no normalisation by
 *    the library (the GDN convention of L2-normalised q, k is the caller's).
 *  - Empty batches (num_seqs == 0) are valid and enqueue nothing.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_TREE_MAX_NODES 64

/* Host-side result of every entry point. */
typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL_PTR = 1,       /* a required pointer is NULL                         */
  GDN_ERR_BAD_SHAPE = 2,      /* negative/zero sizes, max_nodes outside [1,64], ... */
  GDN_ERR_UNSUPPORTED = 3,    /* dk/dv/io dtype/mode combination not built          */
  GDN_ERR_WORKSPACE = 4,      /* workspace smaller than gdn_tree_workspace_bytes()  */
  GDN_ERR_LAUNCH = 5,         /* the HIP runtime refused a launch                   */
  GDN_ERR_GRAPH = 6,          /* the HIP runtime refused graph capture or launch    */
  GDN_ERR_SCRATCH = 7         /* the call needs more than the fixed scratch holds   */
} gdn_status;

/* Element type of q, k, v and o. State, gates and accumulation are fp32. */
typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;

typedef enum { GDN_MODE_WY = 0, GDN_MODE_FORK = 1, GDN_MODE_FORK_DELTA = 2 } gdn_mode;

/* Per-sequence codes written to tree_status (checked in this order). */
enum {
  GDN_TREE_OK = 0,
  GDN_TREE_BAD_ROOT = 1,      /* parents[first node] != -1                          */
  GDN_TREE_BAD_PARENT = 2,    /* a non-root node's parent is < 0 or >= its index    */
  GDN_TREE_BAD_SIZE = 3,      /* N_b outside [1, max_nodes] or range outside [0,T]  */
  GDN_TREE_BAD_ACCEPTED = 4,  /* commit: accepted[b] outside [-1, N_b)              */
  GDN_TREE_TOO_DEEP = 5,      /* FORK modes: a node deeper than desc.max_depth      */
  GDN_TREE_CACHE_FULL = 6,    /* attention commit: the path would overflow the cache */
  GDN_TREE_BAD_TOKEN = 7,     /* sampling acceptance: a draft token outside [0, V)  */
  GDN_TREE_TOO_MANY_KEPT = 8  /* selective fork: more saved nodes than max_kept      */
};
/* Precedence: BAD_SIZE, then BAD_ROOT, then BAD_PARENT, then TOO_DEEP (FORK
 * modes), then TOO_MANY_KEPT (selective fork), then BAD_ACCEPTED (commit). */

/* The fused round-boundary calls (gdn_tree_commit_verify, gdn_tree_replay_verify
 * and their layer-batched forms) report two outcomes per sequence in one code:
 *   tree_status & 0xF                    this round's tree (OK, BAD_SIZE,
 *                                        BAD_ROOT, BAD_PARENT);
 *   tree_status >> GDN_TREE_PREV_SHIFT   the previous round's commit (OK when
 *                                        it was applied, else BAD_SIZE /
 *                                        BAD_ROOT / BAD_PARENT of the previous
 *                                        tree or BAD_ACCEPTED).
 * GDN_TREE_PREV(code) forms the second part. */
#define GDN_TREE_PREV_SHIFT 4
#define GDN_TREE_PREV(code) ((code) << GDN_TREE_PREV_SHIFT)

typedef struct {
  int32_t num_seqs;     /* B >= 0                                                   */
  int32_t num_heads;    /* H >= 1                                                   */
  int32_t dk, dv;       /* supported: dk == dv in {32, 64, 128}                     */
  int32_t total_nodes;  /* T = offsets[B] (host copy; sizes outputs and workspace)  */
  int32_t max_nodes;    /* upper bound on every N_b, in [1, 64]; sizes on-chip tiles */
  int32_t max_depth;    /* FORK modes: number of levels - 1 to run (root = depth 0);
                           0 or negative means max_nodes - 1. Ignored in WY mode.    */
  int32_t io_dtype;     /* gdn_dtype                                                */
  int32_t mode;         /* gdn_mode                                                 */
} gdn_tree_desc;

/* Bytes of speculative state a verify call leaves for its commit, i.e. the
 * workspace size:
 *   WY:   T*H*(dv + 1)*4 bytes -- pseudo-values U [T,H,dv] fp32, then the
 *         base-2 gate prefixes g [T,H] fp32 (each part 256-byte aligned);
 *   FORK: T*H*dv*dk*4 bytes    -- one fp32 checkpoint [T,H,dv,dk] per node-head;
 *   FORK_DELTA: the WY part (U, then g), then T*H*dv*dk*4 bytes of node
 *         states [T,H,dv,dk] (256-byte aligned). Commit reads only the WY
 *         part: the states are verify's working memory (only nodes with
 *         children are written) and may be reused once verify has run.
 * Returns 0 for an invalid descriptor. */
size_t gdn_tree_workspace_bytes(const gdn_tree_desc* desc);

/* Ancestor masks and depths of every node (handbook implementation section:
 * tree_mask and depths; fork page section 2 mask table).
 *   depth    [T] int32  : 0 for the root, parent's depth + 1 otherwise
 *   anc_mask [T] uint64 : bit j set iff local node j is the node or one of its
 *                         ancestors (row of the tree attention mask)
 *   tree_status [B]     : GDN_TREE_OK / BAD_SIZE / BAD_ROOT / BAD_PARENT
 * Outputs of a sequence with a nonzero status are not written (when its node
 * range is valid they are set to depth -1 and mask 0). Mode and io dtype are
 * ignored. */
gdn_status gdn_tree_build(const gdn_tree_desc* desc, const int32_t* offsets,
                          const int32_t* parents, int32_t* depth, uint64_t* anc_mask,
                          int32_t* tree_status, void* stream);

/* Verify: o [T,H,dv] for every node, and the speculative state in `workspace`
 * (layout per gdn_tree_workspace_bytes) for the matching commit.
 * `workspace_bytes` is the size of the caller's buffer. o must not alias any
 * input. tree_status receives the GDN_TREE_* code of every sequence. */
gdn_status gdn_tree_verify(const gdn_tree_desc* desc, const int32_t* offsets,
                           const int32_t* parents, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta,
                           const float* S0, void* o, void* workspace, size_t workspace_bytes,
                           int32_t* tree_status, void* stream);

/* Commit: for every sequence b, S_out[b] = state of local node accepted[b]
 * (the last node of the accepted root-to-node path), or S0[b] when
 * accepted[b] == -1. S_out may equal S0 (in place); partial overlap is not
 * allowed. `workspace` is the one written by gdn_tree_verify with the same
 * descriptor, inputs and mode, and its U and g parts must not have been
 * modified since. WY and FORK_DELTA modes also read k and the same
 * offsets/parents (k may be NULL in FORK mode); FORK mode ignores k. tree_status receives the GDN_TREE_* code of every
 * sequence; sequences with a nonzero code are left unwritten. */
gdn_status gdn_tree_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                           const int32_t* parents, const int32_t* accepted, const void* k,
                           const float* S0, float* S_out, const void* workspace,
                           size_t workspace_bytes, int32_t* tree_status, void* stream);

/* One layer's buffers for the layer-batched calls below: the per-layer
 * arguments of gdn_tree_verify / gdn_tree_commit (device pointers, same
 * layouts). Verify reads q, k, v, alpha, beta, S0 and writes o and workspace;
 * commit reads k, S0 and workspace and writes S_out (fields a call does not
 * use are ignored). */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  void* o;
  float* S_out;
  void* workspace;
} gdn_layer_io;

/* Layer-batched verify and commit: the same work as n_layers calls of
 * gdn_tree_verify / gdn_tree_commit on layers that share one draft tree
 * (offsets, parents, accepted, tree_status), issued as a few launches instead
 * of one per layer (the round runs every GDN layer of the model on the same
 * tree: fork page section 7, steps 2 and 4). `layers` is a HOST array of
 * n_layers entries; every layer's workspace holds workspace_bytes bytes.
 * Results are identical to the per-layer calls. FORK mode runs the per-layer
 * calls. n_layers <= 0 is a no-op. */
gdn_status gdn_tree_verify_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                  const int32_t* offsets, const int32_t* parents,
                                  const gdn_layer_io* layers, size_t workspace_bytes,
                                  int32_t* tree_status, void* stream);
gdn_status gdn_tree_commit_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                  const int32_t* offsets, const int32_t* parents,
                                  const int32_t* accepted, const gdn_layer_io* layers,
                                  size_t workspace_bytes, int32_t* tree_status, void* stream);

/* Fused round boundary: the previous round's commit followed by this round's
 * verify, in one pass over the state.
 *
 * A serving loop runs, per GDN layer, gdn_tree_commit for round r (the
 * accepted path of r's tree, fork page section 5; TreeWY abstract: only the
 * accepted state is rebuilt) and later gdn_tree_verify for round r+1 on the
 * committed state (fork page section 7, steps 4 then 2 of the next round).
 * Both read the (B,H,dv,dk) state; this call reads it once: every
 * workgroup applies the previous commit's update
 *     S = G_a S0 + sum_{i in path(a)} (G_a/G_i) u_i k_i^T
 * to its slice of S0 in registers, writes S to S_out and verifies this
 * round's tree against S. The results are those of
 *     gdn_tree_commit(prev_desc, prev_offsets, prev_parents, accepted,
 *                     prev_k, S0, S_out, prev_workspace, ...)
 *     gdn_tree_verify(desc, offsets, parents, q, k, v, alpha, beta,
 *                     S_out, o, workspace, ...)
 * up to fp32 rounding order, with these differences:
 *  - prev_desc describes the previous round (its own total_nodes and
 *    max_nodes); num_seqs, num_heads, dk, dv and io_dtype must equal desc's,
 *    and both modes must be GDN_MODE_WY (else GDN_ERR_BAD_SHAPE /
 *    GDN_ERR_UNSUPPORTED). prev_desc->total_nodes must be >= 1 when
 *    num_seqs > 0.
 *  - prev_workspace is the previous verify's workspace (U and g unchanged
 *    since), prev_k its k rows [T',H,dk]. The two workspaces must not overlap
 *    (checked: GDN_ERR_BAD_SHAPE); callers alternate two buffers.
 *  - S_out may equal S0 (in place) or must not overlap it; S_out must not
 *    overlap any other argument.
 *  - tree_status [B] receives two codes per sequence (GDN_TREE_PREV_SHIFT):
 *    this round's tree checks (BAD_SIZE, BAD_ROOT, BAD_PARENT) in the low
 *    bits, and GDN_TREE_PREV() of the previous round's (its tree's BAD_SIZE,
 *    BAD_ROOT, BAD_PARENT, then BAD_ACCEPTED for accepted[b] outside
 *    [-1, N'_b)). The previous tree is checked only when accepted[b] != -1.
 *  - The previous commit is applied (S_out written) whenever its own part is
 *    OK, also when this round's tree is rejected, so one malformed draft tree
 *    never loses the accepted tokens' update. A sequence with any nonzero
 *    part gets zero o rows and a zero workspace (none are written when this
 *    round's part is BAD_SIZE); when the previous part is nonzero its S_out
 *    is not written.
 *  - accepted[b] == -1 keeps S0 (S_out = S0; nothing is written in place).
 * The layer-batched form takes HOST arrays of n_layers entries: prev_layers
 * (fields k and workspace used) and layers (q, k, v, alpha, beta, S0, o,
 * S_out, workspace). All layers share both trees and accepted. */
gdn_status gdn_tree_commit_verify(const gdn_tree_desc* prev_desc, const int32_t* prev_offsets,
                                  const int32_t* prev_parents, const int32_t* accepted,
                                  const void* prev_k, const void* prev_workspace,
                                  size_t prev_workspace_bytes, const gdn_tree_desc* desc,
                                  const int32_t* offsets, const int32_t* parents, const void* q,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* S0, float* S_out, void* o,
                                  void* workspace, size_t workspace_bytes, int32_t* tree_status,
                                  void* stream);
gdn_status gdn_tree_commit_verify_layers(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    size_t prev_workspace_bytes, const gdn_layer_io* layers, size_t workspace_bytes,
    int32_t* tree_status, void* stream);

/* Fused round boundary by replay: the same round boundary as
 * gdn_tree_commit_verify, but the previous round's accepted path is committed
 * by running the gated delta rule along it (root first) on each workgroup's
 * slice of S0,
 *     w = S k_j,   S <- alpha_j S + beta_j (v_j - alpha_j w) k_j^T,
 * from that path's own k, v, alpha, beta (fork page section 5: the kept state
 * is the last accepted token's; the update is the one every node's output is
 * defined by), and this round's verify writes no workspace: the next round
 * replays from this round's inputs. The results are those of
 *     gdn_tree_commit(...) of the previous round, then
 *     gdn_tree_verify(desc, ..., S_out, o, ...)
 * up to fp32 rounding order (the path is applied as a recurrence instead of
 * through pseudo-values), without the workspace. Arguments, checks and status
 * codes as for gdn_tree_commit_verify, except:
 *  - prev_k, prev_v [T',H,dk|dv] (io dtype) and prev_alpha, prev_beta [T',H]
 *    are the previous round's verify inputs, unchanged since;
 *  - there is no workspace argument; desc's workspace size is not used.
 * The layer-batched form takes HOST arrays of n_layers entries: prev_layers
 * (fields k, v, alpha, beta used) and layers (q, k, v, alpha, beta, S0, o,
 * S_out used). All layers share both trees and accepted. */
gdn_status gdn_tree_replay_verify(const gdn_tree_desc* prev_desc, const int32_t* prev_offsets,
                                  const int32_t* prev_parents, const int32_t* accepted,
                                  const void* prev_k, const void* prev_v,
                                  const float* prev_alpha, const float* prev_beta,
                                  const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const float* S0, float* S_out, void* o, int32_t* tree_status,
                                  void* stream);
gdn_status gdn_tree_replay_verify_layers(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    const gdn_layer_io* layers, int32_t* tree_status, void* stream);

/* Commit by replay, with no workspace: for every sequence b, S_out[b] = the
 * state of local node accepted[b] (or S0[b] when accepted[b] == -1), formed
 * by running the gated delta rule along the accepted path, root first, on S0:
 *     w = S k_j,   S <- alpha_j S + beta_j (v_j - alpha_j w) k_j^T
 * (fork page section 5: the kept state is the last accepted token's; the
 * update is the one every node's output is defined by). It is the commit of
 * a round verified by gdn_tree_replay_verify, whose verify kept no
 * pseudo-values: a sequence that leaves the batch, or the last round before
 * a pause, is committed with it instead of with the next round's fused call.
 *   k, v [T,H,dk|dv] (io dtype), alpha, beta [T,H] fp32: the round's verify
 *     inputs, unchanged since; only the accepted path's rows are read.
 * desc as for gdn_tree_commit (mode and max_depth are ignored). S_out may
 * equal S0 (in place) or must not overlap it. tree_status receives BAD_SIZE,
 * BAD_ROOT, BAD_PARENT or BAD_ACCEPTED (accepted[b] outside [-1, N_b));
 * such a sequence is left unwritten. The layer-batched form takes a HOST array
 * of n_layers entries (fields k, v, alpha, beta, S0, S_out used) sharing
 * offsets, parents, accepted and tree_status; n_layers <= 0 is a no-op. */
gdn_status gdn_tree_replay_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const int32_t* accepted,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* S0, float* S_out,
                                  int32_t* tree_status, void* stream);
gdn_status gdn_tree_replay_commit_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                         const int32_t* offsets, const int32_t* parents,
                                         const int32_t* accepted, const gdn_layer_io* layers,
                                         int32_t* tree_status, void* stream);

/* Selective fork: the fork/checkpoint baseline (GDN_MODE_FORK's depth-by-
 * depth scheme) keeping a rollback point only for nodes the draft is unsure
 * of (fork page section 8, "selective fork": a branch whose draft confidence
 * is above 0.95 is processed directly, without saving a checkpoint, because
 * it is almost certainly accepted). Node t saves its state iff
 * confidence[t] <= threshold (the page's 0.95 is the caller's threshold; a
 * confidence exactly equal to it saves). A node whose state was not saved is
 * rebuilt wherever it is needed: a node starts from its nearest saved proper
 * ancestor (S0 when there is none) and applies the gated delta rule of every
 * path node below it, its own last; the commit does the same for the accepted
 * node (or copies its own saved state). Results are those of GDN_MODE_FORK.
 *   confidence [T] fp32   the draft's confidence in each node's token
 *   max_kept              saved nodes each sequence may hold, in [0, max_nodes]
 *                         (GDN_ERR_BAD_SHAPE otherwise); a sequence that would
 *                         save more gets GDN_TREE_TOO_MANY_KEPT
 *   workspace             gdn_tree_fork_selective_workspace_bytes(desc,
 *                         max_kept) bytes: checkpoints [B*max_kept, H, dv, dk]
 *                         fp32, sequence b's saved nodes in node order from
 *                         slot b*max_kept (may be NULL when the size is 0)
 * desc as for GDN_MODE_FORK (desc.mode is ignored; desc.max_depth bounds the
 * levels run, deeper trees get GDN_TREE_TOO_DEEP). Verify writes o and the
 * saved states; commit reads them, the same confidence, threshold and
 * max_kept, and the path's k, v, alpha, beta, and writes S_out (may equal
 * S0). Status codes and zeroed rows as gdn_tree_verify / gdn_tree_commit.
 * The workspace size function returns 0 for an invalid descriptor or
 * max_kept. */
size_t gdn_tree_fork_selective_workspace_bytes(const gdn_tree_desc* desc, int32_t max_kept);
gdn_status gdn_tree_fork_selective_verify(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const float* confidence,
                                          float threshold, int32_t max_kept, const void* q,
                                          const void* k, const void* v, const float* alpha,
                                          const float* beta, const float* S0, void* o,
                                          void* workspace, size_t workspace_bytes,
                                          int32_t* tree_status, void* stream);
gdn_status gdn_tree_fork_selective_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const float* confidence,
                                          float threshold, int32_t max_kept,
                                          const int32_t* accepted, const void* k, const void* v,
                                          const float* alpha, const float* beta,
                                          const float* S0, float* S_out, const void* workspace,
                                          size_t workspace_bytes, int32_t* tree_status,
                                          void* stream);

/* Static text for a gdn_status value. */
const char* gdn_tree_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
