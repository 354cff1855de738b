// tree_attn_api.cpp -- the C ABI of the attention half of libgdntree
// (gdn_tree_attn.h): descriptor checks, the split of the cache over
// workgroups, workspace sizing and dispatch. Never allocates, never
// synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "gdn_tree_attn.h"
#include "api_internal.h"
#include "launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kKeyBlock = 64;          // keys per staged block in the verify kernel
constexpr int kMaxQueryRows = 256;     // query rows per (sequence, KV head) workgroup
constexpr long long kTargetGroups = 256;  // one verify workgroup per CU (a CU holds one)

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

namespace gdn {

gdn_status check_attn_desc(const gdn_attn_desc* d) {
  if (d == nullptr) return GDN_ERR_NULL_PTR;
  if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->total_nodes < 0 ||
      d->max_nodes < 1 || d->max_nodes > GDN_TREE_MAX_NODES || d->cache_capacity < 0 ||
      d->max_cache_len < 0 || d->max_cache_len > d->cache_capacity)
    return GDN_ERR_BAD_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return GDN_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return GDN_ERR_UNSUPPORTED;
  if ((long long)(d->num_q_heads / d->num_kv_heads) * d->max_nodes > kMaxQueryRows)
    return GDN_ERR_UNSUPPORTED;
  // row indices (node * Hq) and the grid must fit int
  if ((long long)d->total_nodes * d->num_q_heads > INT_MAX / 2 ||
      (long long)d->num_seqs * d->num_kv_heads * 64 > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

}  // namespace gdn

namespace {

gdn_status check_desc(const gdn_attn_desc* d) { return gdn::check_attn_desc(d); }

// Split of each (sequence, KV head)'s cache rows over NS workgroups of CL
// rows (CL a multiple of the key block), so that about kTargetGroups
// workgroups run when B * Hkv alone is too few.
void cache_split(const gdn_attn_desc* d, int* ns, int* cl) {
  const long long pairs = (long long)d->num_seqs * d->num_kv_heads;
  const int blocks = (d->max_cache_len + kKeyBlock - 1) / kKeyBlock;
  long long want = pairs > 0 ? (kTargetGroups + pairs - 1) / pairs : 1;
  if (want > blocks) want = blocks;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  const int per = (blocks + (int)want - 1) / (int)want;          // blocks per split
  *cl = (per > 0 ? per : 1) * kKeyBlock;
  *ns = blocks > 0 ? (blocks + per - 1) / per : 1;
}

size_t workspace_bytes(const gdn_attn_desc* d) {
  int ns, cl;
  cache_split(d, &ns, &cl);
  if (ns == 1) return 0;
  const size_t rows = (size_t)d->total_nodes * d->num_q_heads * ns;
  return round_up(rows * d->head_dim * sizeof(float)) + round_up(rows * 2 * sizeof(float));
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

gdn::AttnCommitArgs commit_base(const gdn_attn_desc* d, const int32_t* offsets,
                                const int32_t* parents, const int32_t* accepted,
                                int32_t* cache_len, int32_t* tree_status) {
  gdn::AttnCommitArgs a{};
  a.B = d->num_seqs;
  a.Hkv = d->num_kv_heads;
  a.T = d->total_nodes;
  a.max_nodes = d->max_nodes;
  a.cap = d->cache_capacity;
  a.offsets = offsets;
  a.parents = parents;
  a.accepted = accepted;
  a.cache_len = cache_len;
  a.status = tree_status;
  return a;
}

}  // namespace

extern "C" {

size_t gdn_tree_attn_workspace_bytes(const gdn_attn_desc* desc) {
  if (check_desc(desc) != GDN_OK) return 0;
  return workspace_bytes(desc);
}

}  // extern "C"

namespace gdn {

gdn_status attn_verify_impl(const gdn_attn_desc* desc, const int32_t* offsets,
                            const int32_t* parents, const void* q, const void* k, const void* v,
                            const void* k_cache, const void* v_cache, const int32_t* cache_len,
                            float scale, void* o, void* workspace, size_t ws_bytes,
                            int32_t* tree_status, void* stream, int merge) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !cache_len || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !q || !k || !v || !o)) return GDN_ERR_NULL_PTR;
  if (desc->max_cache_len > 0 && (!k_cache || !v_cache)) return GDN_ERR_NULL_PTR;
  const size_t need = workspace_bytes(desc);
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (need > 0 && !workspace) return GDN_ERR_NULL_PTR;
  int ns, cl;
  cache_split(desc, &ns, &cl);
  const size_t rows = (size_t)desc->total_nodes * desc->num_q_heads * ns;
  float* part_o = ns > 1 ? static_cast<float*>(workspace) : nullptr;
  float* part_ml =
      ns > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        round_up(rows * desc->head_dim * sizeof(float)))
             : nullptr;
  gdn::AttnArgs a{};
  a.B = desc->num_seqs;
  a.Hq = desc->num_q_heads;
  a.Hkv = desc->num_kv_heads;
  a.T = desc->total_nodes;
  a.max_nodes = desc->max_nodes;
  a.cap = desc->cache_capacity;
  a.max_len = desc->max_cache_len;
  a.NS = ns;
  a.CL = cl;
  a.scale_log2 = scale * 1.44269504088896340736f;   // scores in the base-2 domain
  a.offsets = offsets;
  a.parents = parents;
  a.cache_len = cache_len;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.o = static_cast<uint16_t*>(o);
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.status = tree_status;
  a.merge = merge;
  return launched(gdn::launch_tree_attn(desc->head_dim, a, static_cast<hipStream_t>(stream)));
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_attn_verify(const gdn_attn_desc* desc, const int32_t* offsets,
                                const int32_t* parents, const void* q, const void* k,
                                const void* v, const void* k_cache, const void* v_cache,
                                const int32_t* cache_len, float scale, void* o,
                                void* workspace, size_t ws_bytes, int32_t* tree_status,
                                void* stream) {
  return gdn::attn_verify_impl(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                               scale, o, workspace, ws_bytes, tree_status, stream, 0);
}

gdn_status gdn_tree_attn_verify_noalloc(const gdn_attn_desc* desc, const int32_t* offsets,
                                        const int32_t* parents, const void* q, const void* k,
                                        const void* v, const void* k_cache, const void* v_cache,
                                        const int32_t* cache_len, float scale, void* o,
                                        int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  const size_t need = workspace_bytes(desc);
  if (need > gdn::kAttnScratchBytes) return GDN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (need > 0 && gdn::attn_scratch(&scratch) != hipSuccess) return GDN_ERR_LAUNCH;
  return gdn::attn_verify_impl(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                               scale, o, scratch, need, tree_status, stream, 0);
}

gdn_status gdn_tree_attn_commit(const gdn_attn_desc* desc, const int32_t* offsets,
                                const int32_t* parents, const int32_t* accepted, const void* k,
                                const void* v, void* k_cache, void* v_cache, int32_t* cache_len,
                                int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !accepted || !cache_len || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !k || !v)) return GDN_ERR_NULL_PTR;
  if (desc->cache_capacity > 0 && (!k_cache || !v_cache)) return GDN_ERR_NULL_PTR;
  gdn::AttnCommitArgs a = commit_base(desc, offsets, parents, accepted, cache_len, tree_status);
  a.layers = 1;
  a.advance = 1;
  a.L[0] = {static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
            static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache)};
  return launched(
      gdn::launch_tree_attn_commit(desc->head_dim, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace gdn {

gdn_status attn_commit_layers_impl(const gdn_attn_desc* desc, int32_t n_layers,
                                   const int32_t* offsets, const int32_t* parents,
                                   const int32_t* accepted, const gdn_attn_layer_io* layers,
                                   int32_t* cache_len, int32_t* tree_status, void* stream,
                                   int merge) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0 || n_layers <= 0) return GDN_OK;
  if (!offsets || !accepted || !cache_len || !tree_status || !layers) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  for (int l = 0; l < n_layers; ++l) {
    if (desc->total_nodes > 0 && (!layers[l].k || !layers[l].v)) return GDN_ERR_NULL_PTR;
    if (desc->cache_capacity > 0 && (!layers[l].k_cache || !layers[l].v_cache))
      return GDN_ERR_NULL_PTR;
  }
  // every launch reads the same committed length; only the last advances it
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxLayersPerLaunch) {
    const int nl = n_layers - l0 < gdn::kMaxLayersPerLaunch ? n_layers - l0
                                                            : gdn::kMaxLayersPerLaunch;
    gdn::AttnCommitArgs a =
        commit_base(desc, offsets, parents, accepted, cache_len, tree_status);
    a.layers = nl;
    a.advance = l0 + nl == n_layers;
    a.merge = merge;
    for (int i = 0; i < nl; ++i) {
      const gdn_attn_layer_io& ly = layers[l0 + i];
      a.L[i] = {static_cast<const uint16_t*>(ly.k), static_cast<const uint16_t*>(ly.v),
                static_cast<uint16_t*>(ly.k_cache), static_cast<uint16_t*>(ly.v_cache)};
    }
    st = launched(
        gdn::launch_tree_attn_commit(desc->head_dim, a, static_cast<hipStream_t>(stream)));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_attn_commit_layers(const gdn_attn_desc* desc, int32_t n_layers,
                                       const int32_t* offsets, const int32_t* parents,
                                       const int32_t* accepted, const gdn_attn_layer_io* layers,
                                       int32_t* cache_len, int32_t* tree_status, void* stream) {
  return gdn::attn_commit_layers_impl(desc, n_layers, offsets, parents, accepted, layers,
                                      cache_len, tree_status, stream, 0);
}

}  // extern "C"
