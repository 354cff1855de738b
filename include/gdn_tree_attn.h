/*
 * gdn_tree_attn.h -- C ABI of libgdntree, full-attention layers of a hybrid
 * model: tree-masked attention verify and the accepted-path KV-cache commit
 * on AMD Instinct MI355X (gfx950).
 *
 * In a hybrid model the Gated DeltaNet layers (gdn_tree.h) alternate with
 * full-attention layers. Under a speculative draft tree the attention layers
 * verify every node in one pass: node t of sequence b attends to the whole
 * committed KV cache of b and, among the tree nodes, to itself and its
 * ancestors only (anrans.github.io ai-infra-handbooks "speculative",
 * implementation section: every new token sees the cached prefix, the tree
 * mask decides visibility among the new tokens, query heads share K/V heads
 * in groups). After acceptance only the K/V rows of the accepted path are
 * kept, appended to the cache in path order; they were computed at the right
 * positions during verification and are not recomputed (same section, last
 * step; rainlin-top.pages.dev "Qwen3.5 tree spec", section 7 step 4: the
 * attention layers keep the accepted tokens' KV cache and drop the rest).
 *
 * Positions (rotary embeddings) are applied by the caller to q and k before
 * verification (a tree node's position is the committed length plus its
 * depth, as in the handbook); this library takes q and k as they are.
 *
 * Conventions follow gdn_tree.h: device pointers owned by the caller, no
 * allocation or synchronisation, work enqueued on `stream`, host-side checks
 * reported by the gdn_status return value, data-dependent problems per
 * sequence in tree_status (GDN_TREE_* codes; a rejected sequence whose
 * node range is well formed gets zero output rows, rows of a malformed node
 * range are not written, and a rejected commit writes nothing). All tensors are dense and
 * row-major; q, k, v, the caches and o are bf16 (as raw 16-bit patterns);
 * arithmetic is fp32.
 *   offsets      [B+1] int32       node range of sequence b: [offsets[b], offsets[b+1])
 *   parents      [T]   int32       local parent, -1 for the root (root first)
 *   q            [T,Hq,d]          queries of the tree nodes
 *   k, v         [T,Hkv,d]         keys / values of the tree nodes
 *   k_cache, v_cache [B,Hkv,cap,d] committed keys / values; row p < cache_len[b] valid
 *   cache_len    [B]   int32       committed length per sequence (updated by commit)
 *   o            [T,Hq,d]          outputs
 * Query head h reads K/V head h / (Hq / Hkv).
 */
#ifndef GDN_TREE_ATTN_H
#define GDN_TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "gdn_tree.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_seqs;       /* B >= 0                                                  */
  int32_t num_q_heads;    /* Hq >= 1                                                 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0                                  */
  int32_t head_dim;       /* d: supported 64, 128                                    */
  int32_t total_nodes;    /* T = offsets[B]                                          */
  int32_t max_nodes;      /* bound on every N_b, in [1, 64]; (Hq/Hkv) * max_nodes <= 256 */
  int32_t cache_capacity; /* cap: cache rows per (sequence, KV head)                 */
  int32_t max_cache_len;  /* bound on every cache_len[b] at verify, in [0, cap];
                             sizes the split of the cache over workgroups           */
} gdn_attn_desc;

/* Bytes of scratch gdn_tree_attn_verify needs (partial results when the cache
 * is split over several workgroups per (sequence, KV head); 0 when it is not).
 * Returns 0 for an invalid descriptor as well. */
size_t gdn_tree_attn_workspace_bytes(const gdn_attn_desc* desc);

/* Tree-masked attention for every node: o[t,h] = softmax over the visible keys
 * of scale * <q[t,h], key> applied to the values, where the visible keys are
 * cache rows 0 .. cache_len[b]-1 and the tree nodes on t's root path
 * (t included). `scale` is usually 1/sqrt(d). `workspace` (may be NULL when
 * the size above is 0) must hold workspace_bytes. tree_status receives
 * GDN_TREE_OK / BAD_SIZE (range, or cache_len outside [0, max_cache_len]) /
 * BAD_ROOT / BAD_PARENT per sequence. o must not alias an input. */
gdn_status gdn_tree_attn_verify(const gdn_attn_desc* desc, const int32_t* offsets,
                                const int32_t* parents, const void* q, const void* k,
                                const void* v, const void* k_cache, const void* v_cache,
                                const int32_t* cache_len, float scale, void* o,
                                void* workspace, size_t workspace_bytes, int32_t* tree_status,
                                void* stream);

/* gdn_tree_attn_verify without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The split-cache partials go to a scratch
 * buffer of 32 MiB per GPU that the library holds in its code object until
 * the process ends; its address is taken on the first call on each device.
 * The call allocates nothing. A descriptor whose partials would exceed 32 MiB
 * (gdn_tree_attn_workspace_bytes > 32 MiB) gets GDN_ERR_SCRATCH and nothing
 * is enqueued. Every call on one GPU shares that GPU's scratch: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller. Results are identical to gdn_tree_attn_verify. */
gdn_status gdn_tree_attn_verify_noalloc(const gdn_attn_desc* desc, const int32_t* offsets,
                                        const int32_t* parents, const void* q, const void* k,
                                        const void* v, const void* k_cache, const void* v_cache,
                                        const int32_t* cache_len, float scale, void* o,
                                        int32_t* tree_status, void* stream);

/* Commit: for every sequence b with accepted[b] = a >= 0, append the K/V rows
 * of the path root .. a (root first) at cache rows cache_len[b] .. and advance
 * cache_len[b] by the path length; accepted[b] = -1 leaves b unchanged.
 * k and v are the same tree rows that were verified. tree_status receives
 * BAD_SIZE / BAD_ROOT / BAD_PARENT / BAD_ACCEPTED (outside [-1, N_b)) /
 * CACHE_FULL (path longer than cap - cache_len[b]); such a sequence is left
 * unchanged. */
gdn_status gdn_tree_attn_commit(const gdn_attn_desc* desc, const int32_t* offsets,
                                const int32_t* parents, const int32_t* accepted, const void* k,
                                const void* v, void* k_cache, void* v_cache, int32_t* cache_len,
                                int32_t* tree_status, void* stream);

/* One attention layer's buffers for the layer-batched commit below and for a
 * captured round (gdn_round.h); layouts as above. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  void* o;
} gdn_attn_layer_io;

/* Layer-batched commit: the accepted-path K/V append of n_layers attention
 * layers of one model, which share the trees, the accepted nodes and the
 * committed length of every sequence (all layers of a model hold the same
 * prefix). Every layer's path rows go to cache rows cache_len[b] .. of its
 * own caches, then cache_len[b] advances once by the path length. `layers` is
 * a HOST array (q and o are not read). Per-sequence status and the
 * unchanged-on-error rule are those of gdn_tree_attn_commit; the rows written
 * are identical to n_layers single-layer commits that each start from the
 * same length. n_layers <= 0 is a no-op. */
gdn_status gdn_tree_attn_commit_layers(const gdn_attn_desc* desc, int32_t n_layers,
                                       const int32_t* offsets, const int32_t* parents,
                                       const int32_t* accepted, const gdn_attn_layer_io* layers,
                                       int32_t* cache_len, int32_t* tree_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_ATTN_H */
