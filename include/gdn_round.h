/*
 * gdn_round.h -- C ABI of libgdntree, one speculative round across the layers
 * of a hybrid model: acceptance of the verified draft tree, one arena for the
 * round's speculative state, tree sizing under a memory budget, and the whole
 * round (verify -> accept -> commit) captured once as a HIP graph.
 *
 * A round of tree speculation runs every layer of the model on the same draft
 * tree, picks the accepted path, and keeps the state of that path only
 * (rainlin-top.pages.dev "Qwen3.5 tree spec", section 7: GDN layers verify the
 * flattened tree, attention layers verify it under the tree mask, then the
 * accepted path's state is restored in the GDN layers and its K/V rows are
 * kept in the attention layers). The per-layer calls are in gdn_tree.h and
 * gdn_tree_attn.h; this header composes them.
 *
 * Conventions follow gdn_tree.h: device pointers owned by the caller, no
 * device allocation and no synchronisation, host-side checks reported by the
 * gdn_status return value, data-dependent problems per sequence in
 * tree_status (GDN_TREE_* codes).
 */
#ifndef GDN_ROUND_H
#define GDN_ROUND_H

#include <stddef.h>
#include <stdint.h>

#include "gdn_tree.h"
#include "gdn_tree_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ acceptance */

/* Greedy acceptance of a verified draft tree, per sequence (handbook
 * anrans.github.io ai-infra-handbooks "speculative", implementation section,
 * the generation loop): the walk starts at the root, which is always
 * accepted; at the current node it takes the target model's prediction for
 * the next token, looks for a child of the node whose draft token equals it,
 * taking the first such child in node order, and moves there; it stops at the
 * first node with no such child.
 *   draft_tokens  [T] int32  token of every node (the root's is not read)
 *   target_tokens [T] int32  the target model's predicted next token at every
 *                            node (the argmax of its logits at that node)
 *   accepted      [B] int32  out: last node of the accepted path (local
 *                            index), the input of the commits
 *   accept_len    [B] int32  out: nodes on the accepted path, root included
 *   next_token    [B] int32  out: target_tokens at the last accepted node (the
 *                            target's own next token, the next round's root)
 *   tree_status   [B] int32  out: GDN_TREE_OK / BAD_SIZE / BAD_ROOT /
 *                            BAD_PARENT; a rejected sequence gets accepted -1,
 *                            accept_len 0 and next_token -1 (so every commit
 *                            leaves it unchanged)
 * Only num_seqs, total_nodes and max_nodes of `desc` are used. Integer work:
 * results are exact. */
gdn_status gdn_tree_accept_greedy(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const int32_t* draft_tokens,
                                  const int32_t* target_tokens, int32_t* accepted,
                                  int32_t* accept_len, int32_t* next_token,
                                  int32_t* tree_status, void* stream);

/* Sampling-mode acceptance: multi-candidate rejection sampling down the tree
 * (handbook, same chapter, exercise on sampling with a tree). The walk starts
 * at the root. At the current node, with the target's distribution p and the
 * draft's distribution q from which the node's children were drawn (without
 * replacement, in node order), each child's token x is tried in node order:
 * it is accepted iff u * q(x) < p(x), u being the child's first uniform; the
 * walk then moves to it and starts afresh with its rows. After a rejection p
 * becomes max(0, p - q) normalised (left unchanged if that has no mass) and
 * q loses the rejected token and is renormalised. When no child is accepted
 * (or the node has none), one token is drawn from the current p by inverse
 * CDF with the node's second uniform (the first token whose cumulative mass
 * exceeds u times the total) and the walk ends. The emitted tokens then have
 * the target's distribution.
 *   draft_tokens  [T] int32   token of every node (the root's is not read)
 *   target_probs  [T, vocab]  fp32, row t: the target's distribution of the
 *                             token after node t (softmax already applied)
 *   draft_probs   [T, vocab]  fp32, row t: the draft's distribution t's
 *                             children were drawn from (rows of leaves unread)
 *   uniforms      [T, 2]      fp32 in [0, 1): node t's draw as a candidate,
 *                             and its draw for the final token
 *   accepted, accept_len, next_token, tree_status: as for the greedy walk;
 *                             next_token is the drawn token; status adds
 *                             GDN_TREE_BAD_TOKEN for a draft token outside
 *                             [0, vocab)
 * vocab must be a multiple of 4 in [4, 2^20] (GDN_ERR_UNSUPPORTED otherwise).
 * Decisions are taken in fp32. */
gdn_status gdn_tree_accept_sampling(const gdn_tree_desc* desc, const int32_t* offsets,
                                    const int32_t* parents, const int32_t* draft_tokens,
                                    const float* target_probs, const float* draft_probs,
                                    int32_t vocab, const float* uniforms, int32_t* accepted,
                                    int32_t* accept_len, int32_t* next_token,
                                    int32_t* tree_status, void* stream);

/* The same acceptance with every pass over a node's rows spread over `splits`
 * workgroups per sequence, for batches too small to fill the device with one
 * workgroup per sequence. The decisions are the same, bit for bit, as
 * gdn_tree_accept_sampling's: both calls cut a row's 256-token tiles into
 * GDN_SAMPLING_MAX_SPLITS fixed groups and take every total over the group
 * sums in group order, each group sum over its tiles in a fixed order, so no
 * sum depends on how the groups are divided. After each pass the workgroups
 * of a sequence trade their group sums through `workspace`; a workgroup that
 * waits too long for the others (none is ever required to be resident at the
 * same time) sums the whole row itself, with the same result, so the call
 * always completes.
 *   splits     workgroups per sequence: 1, 2, 4, 8 or 16 (each takes whole
 *              groups; GDN_ERR_UNSUPPORTED otherwise), or 0 for
 *              gdn_tree_accept_sampling_splits(desc) (the most whose grid
 *              the device holds at once; a larger grid is correct but slower)
 *   workspace  device memory of at least
 *              gdn_tree_accept_sampling_split_workspace_bytes(desc, vocab) bytes
 *              (520 per sequence), 256-byte aligned, owned by the caller, all
 *              zero before its first use (hipMemset once); every call that
 *              runs leaves the part it used zero again (the last workgroup of
 *              each sequence to finish clears it), so the workspace is reused
 *              with no preparation and no clearing launch. Two calls in flight
 *              at once must not share it, and a workspace with other contents
 *              may give wrong results
 * Other arguments, checks and status codes as for gdn_tree_accept_sampling.
 * splits = 1 is that call (the workspace is not used and may be NULL). */
#define GDN_SAMPLING_MAX_SPLITS 16
size_t gdn_tree_accept_sampling_split_workspace_bytes(const gdn_tree_desc* desc, int32_t vocab);
/* The splits that `splits = 0` picks on the current device: the largest power
 * of two up to GDN_SAMPLING_MAX_SPLITS whose grid is resident at once, at
 * least 1. */
int32_t gdn_tree_accept_sampling_splits(const gdn_tree_desc* desc);
gdn_status gdn_tree_accept_sampling_split(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const int32_t* draft_tokens,
                                          const float* target_probs, const float* draft_probs,
                                          int32_t vocab, const float* uniforms, int32_t splits,
                                          void* workspace, size_t workspace_bytes,
                                          int32_t* accepted, int32_t* accept_len,
                                          int32_t* next_token, int32_t* tree_status,
                                          void* stream);

/* ------------------------------------------------------------------ round shape and arena */

/* The layers of one round. Every GDN layer has the shape `gdn` (WY or FORK
 * mode) and every full-attention layer the shape `attn`; both describe the
 * same batch of trees (num_seqs, total_nodes and max_nodes agree when both
 * kinds are present). */
typedef struct {
  gdn_tree_desc gdn;
  int32_t n_gdn_layers;     /* >= 0                                            */
  gdn_attn_desc attn;       /* ignored when n_attn_layers == 0                 */
  int32_t n_attn_layers;    /* >= 0                                            */
} gdn_round_desc;

/* Where each layer's scratch lives in one caller-owned arena (byte offsets;
 * every slice 256-byte aligned). GDN layer l's workspace (gdn_ws_bytes, the
 * speculative state its verify leaves for its commit) starts at
 * l * gdn_ws_stride, attention layer l's at attn_ws_offset + l *
 * attn_ws_stride. In GDN_MODE_FORK_DELTA the stride covers only the part
 * commit reads (U and g); a layer's workspace runs on over the slices of the
 * layers after it, whose verify-time states share that memory. This is
 * valid when the GDN layers verify in increasing order, as a round does:
 * every later layer writes its states past the kept part of every earlier
 * one. */
typedef struct {
  size_t total_bytes;       /* arena size for the whole round                  */
  size_t gdn_ws_bytes;      /* gdn_tree_workspace_bytes(&desc.gdn)             */
  size_t gdn_ws_stride;
  size_t attn_ws_bytes;     /* gdn_tree_attn_workspace_bytes(&desc.attn)       */
  size_t attn_ws_offset;
  size_t attn_ws_stride;
} gdn_round_layout;

/* Arena layout of a round. GDN_ERR_BAD_SHAPE when the two shapes disagree on
 * the batch, or a layer count is negative; otherwise the per-layer
 * descriptor checks of the per-layer calls. */
gdn_status gdn_round_plan(const gdn_round_desc* desc, gdn_round_layout* layout);

/* Tree sizing under a memory budget (fork page, section 8: the draft tree's
 * width and depth are limited so that the speculative state fits the memory
 * at hand). Among complete trees with branching factor k in [1, 8] and depth
 * d in [1, max_depth] (1 + k + ... + k^d nodes, at most GDN_TREE_MAX_NODES),
 * picks the one with the most nodes whose speculative state -- num_seqs
 * sequences, n_gdn_layers layers: the GDN part of the round's arena
 * (gdn_round_plan) in desc.gdn's mode -- fits budget_bytes; ties go to the
 * wider tree. total_nodes and max_nodes of
 * desc.gdn are ignored. When no tree with a draft node fits, the result is
 * the root alone (branching 0, depth 0, nodes 1). state_bytes receives the
 * chosen tree's bytes as the arena holds them (may be NULL). */
gdn_status gdn_round_tree_for_budget(const gdn_round_desc* desc, size_t budget_bytes,
                                     int32_t max_depth, int32_t* branching, int32_t* depth,
                                     int32_t* nodes, size_t* state_bytes);

/* ------------------------------------------------------------------ captured round */

/* Everything one round reads and writes. Host arrays: gdn_layers
 * [n_gdn_layers] (their workspace fields are ignored: the arena supplies
 * them), attn_layers [n_attn_layers], layer_kinds [n_gdn_layers +
 * n_attn_layers] (0 = the next GDN layer, 1 = the next attention layer, in
 * model order; NULL = the GDN layers, then the attention layers). All other
 * pointers are device pointers. cache_len is shared by the attention layers
 * (one committed length per sequence); commit advances it once. */
typedef struct {
  const int32_t* offsets;
  const int32_t* parents;
  const gdn_layer_io* gdn_layers;
  const gdn_attn_layer_io* attn_layers;
  const int32_t* layer_kinds;
  int32_t* cache_len;
  float attn_scale;
  void* arena;
  size_t arena_bytes;
  const int32_t* draft_tokens;
  const int32_t* target_tokens;
  int32_t* accepted;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* tree_status;
} gdn_round_io;

typedef struct gdn_round_graph_s* gdn_round_graph;

/* Record one round on `stream` (a non-null hipStream_t that is not already
 * capturing) as a HIP graph: every layer's verify in model order, the greedy
 * acceptance, the GDN commits of all layers, and the attention layers' KV
 * append. Nothing runs during capture. The graph keeps the pointers of `io`:
 * every buffer must stay allocated, at the same address, while the graph is
 * used; their contents are read when the graph runs. GDN_ERR_GRAPH when the
 * HIP runtime refuses capture or instantiation (the stream is left out of
 * capture). *out is set only on success. */
gdn_status gdn_round_capture(const gdn_round_desc* desc, const gdn_round_io* io, void* stream,
                             gdn_round_graph* out);

/* The previous round, for a round whose GDN layers commit it inside their
 * verify by replay (gdn_tree_replay_verify, gdn_tree.h): its GDN shape
 * (num_seqs, num_heads, dk, dv and io_dtype as the round's; its own
 * total_nodes and max_nodes), its tree, its accepted nodes, and per GDN
 * layer its k, v, alpha and beta (gdn_layers: HOST array of the round's
 * n_gdn_layers entries, fields k, v, alpha, beta used). Device pointers
 * otherwise. */
typedef struct {
  gdn_tree_desc gdn;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
  const gdn_layer_io* gdn_layers;
} gdn_round_prev;

/* gdn_round_capture for a round that also commits the previous one: every
 * GDN layer's verify is gdn_tree_replay_verify (the previous round's accepted
 * path replayed on the layer's state, S0 -> S_out, then this round's tree
 * verified against it, fork page section 7 step 4 of one round joined to step
 * 2 of the next), and the round ends after the attention layers' KV append:
 * its own GDN commit is left to the next round's graph. The GDN layers' S0
 * and S_out are used, their workspace fields are ignored and the arena's GDN
 * part is not written. The buffers of the previous round must be other than
 * this round's (callers alternate two sets and capture one graph each way). */
gdn_status gdn_round_capture_replay(const gdn_round_desc* desc, const gdn_round_io* io,
                                    const gdn_round_prev* prev, void* stream,
                                    gdn_round_graph* out);

/* Run a captured round on `stream` (any stream of the same device). Runs of
 * one graph must not overlap. */
gdn_status gdn_round_launch(gdn_round_graph graph, void* stream);

/* Free a captured round (host-side objects only). NULL is a no-op. */
void gdn_round_destroy(gdn_round_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ROUND_H */
