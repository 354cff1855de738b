// round_api.cpp -- the C ABI of gdn_round.h: greedy acceptance, the arena
// layout of a round, tree sizing under a memory budget, and one round
// (every layer's verify, acceptance, every layer's commit) recorded as a HIP
// graph. Never allocates device memory, never synchronises.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include <new>
#include <vector>

#include "api_internal.h"
#include "gdn_round.h"
#include "launch.h"

struct gdn_round_graph_s {
  hipGraphExec_t exec;
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxBranching = 8;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

gdn_status check_round(const gdn_round_desc* d) {
  if (d == nullptr) return GDN_ERR_NULL_PTR;
  if (d->n_gdn_layers < 0 || d->n_attn_layers < 0) return GDN_ERR_BAD_SHAPE;
  gdn_status st = GDN_OK;
  if (d->n_gdn_layers > 0 && (st = gdn::check_tree_desc(&d->gdn)) != GDN_OK) return st;
  if (d->n_attn_layers > 0 && (st = gdn::check_attn_desc(&d->attn)) != GDN_OK) return st;
  if (d->n_gdn_layers > 0 && d->n_attn_layers > 0 &&
      (d->gdn.num_seqs != d->attn.num_seqs || d->gdn.total_nodes != d->attn.total_nodes ||
       d->gdn.max_nodes != d->attn.max_nodes))
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

// Bytes of the part of a FORK_DELTA workspace that commit reads (U, then g).
size_t kept_bytes(const gdn_tree_desc* g) {
  const size_t th = (size_t)g->total_nodes * g->num_heads;
  return round_up(th * g->dv * sizeof(float)) + round_up(th * sizeof(float));
}

void plan(const gdn_round_desc* d, gdn_round_layout* out) {
  gdn_round_layout L{};
  size_t gdn_end = 0;
  if (d->n_gdn_layers > 0) {
    L.gdn_ws_bytes = gdn_tree_workspace_bytes(&d->gdn);
    if (d->gdn.mode == GDN_MODE_FORK_DELTA) {
      // slices of the kept parts only; each layer's verify-time states lie
      // past every slice of the layers before it, so layers verified in
      // order share one state region
      L.gdn_ws_stride = kept_bytes(&d->gdn);
      gdn_end = L.gdn_ws_stride * (size_t)(d->n_gdn_layers - 1) + round_up(L.gdn_ws_bytes);
    } else {
      L.gdn_ws_stride = round_up(L.gdn_ws_bytes);
      gdn_end = L.gdn_ws_stride * (size_t)d->n_gdn_layers;
    }
  }
  L.attn_ws_offset = gdn_end;
  if (d->n_attn_layers > 0) {
    L.attn_ws_bytes = gdn_tree_attn_workspace_bytes(&d->attn);
    L.attn_ws_stride = round_up(L.attn_ws_bytes);
  }
  L.total_bytes = L.attn_ws_offset + L.attn_ws_stride * (size_t)d->n_attn_layers;
  *out = L;
}

// The tree shape the acceptance reads: the GDN descriptor, or one built from
// the attention descriptor's batch when the round has no GDN layer.
gdn_tree_desc tree_shape(const gdn_round_desc* d) {
  if (d->n_gdn_layers > 0) return d->gdn;
  gdn_tree_desc t{};
  t.num_seqs = d->attn.num_seqs;
  t.num_heads = 1;
  t.dk = t.dv = 128;
  t.total_nodes = d->attn.total_nodes;
  t.max_nodes = d->attn.max_nodes;
  t.io_dtype = GDN_DTYPE_BF16;
  t.mode = GDN_MODE_WY;
  return t;
}

// Greedy acceptance; merge != 0 inside a captured round (see enqueue_round).
gdn_status accept_greedy_impl(const gdn_tree_desc* desc, const int32_t* offsets,
                              const int32_t* parents, const int32_t* draft_tokens,
                              const int32_t* target_tokens, int32_t* accepted,
                              int32_t* accept_len, int32_t* next_token, int32_t* tree_status,
                              void* stream, int merge) {
  if (desc == nullptr) return GDN_ERR_NULL_PTR;
  if (desc->num_seqs < 0 || desc->total_nodes < 0 || desc->max_nodes < 1 ||
      desc->max_nodes > GDN_TREE_MAX_NODES || desc->num_seqs > INT_MAX - 3)
    return GDN_ERR_BAD_SHAPE;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !accepted || !accept_len || !next_token || !tree_status)
    return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !draft_tokens || !target_tokens))
    return GDN_ERR_NULL_PTR;
  gdn::AcceptArgs a{desc->num_seqs, desc->total_nodes, desc->max_nodes, offsets, parents,
                    draft_tokens, target_tokens, accepted, accept_len, next_token,
                    tree_status};
  a.merge = merge;
  return gdn::launch_accept_greedy(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? GDN_OK
             : GDN_ERR_LAUNCH;
}

// Every call of one round, in order, on `stream`. The round's first step
// writes tree_status; every later step keeps a code an earlier one set (a
// verify that rejected the sequence in one layer, or the previous round's
// commit that could not be applied), and the acceptance then accepts nothing
// for such a sequence, so no commit changes its state.
gdn_status enqueue_round(const gdn_round_desc* d, const gdn_round_io* io,
                         const gdn_round_layout& L, const gdn_round_prev* prev, void* stream) {
  const int ng = d->n_gdn_layers, na = d->n_attn_layers;
  char* base = static_cast<char*>(io->arena);
  int gi = 0, ai = 0;
  gdn_status st = GDN_OK;
  for (int pos = 0; pos < ng + na; ++pos) {
    const int kind = io->layer_kinds ? io->layer_kinds[pos] : (pos < ng ? 0 : 1);
    const int merge = pos > 0;
    if (kind == 0) {
      const gdn_layer_io& ly = io->gdn_layers[gi];
      if (prev) {
        st = gdn::replay_verify_layers_impl(&prev->gdn, &d->gdn, 1, prev->offsets,
                                            prev->parents, prev->accepted, io->offsets,
                                            io->parents, &prev->gdn_layers[gi], &ly,
                                            io->tree_status, stream, merge);
      } else {
        void* ws = L.gdn_ws_bytes ? base + (size_t)gi * L.gdn_ws_stride : nullptr;
        st = gdn::verify_impl(&d->gdn, io->offsets, io->parents, ly.q, ly.k, ly.v, ly.alpha,
                              ly.beta, ly.S0, ly.o, ws, L.gdn_ws_bytes, io->tree_status, stream,
                              merge);
      }
      ++gi;
    } else {
      const gdn_attn_layer_io& ly = io->attn_layers[ai];
      void* ws = L.attn_ws_bytes ? base + L.attn_ws_offset + (size_t)ai * L.attn_ws_stride
                                 : nullptr;
      st = gdn::attn_verify_impl(&d->attn, io->offsets, io->parents, ly.q, ly.k, ly.v,
                                 ly.k_cache, ly.v_cache, io->cache_len, io->attn_scale, ly.o, ws,
                                 L.attn_ws_bytes, io->tree_status, stream, merge);
      ++ai;
    }
    if (st != GDN_OK) return st;
  }
  const gdn_tree_desc ts = tree_shape(d);
  st = accept_greedy_impl(&ts, io->offsets, io->parents, io->draft_tokens, io->target_tokens,
                          io->accepted, io->accept_len, io->next_token, io->tree_status, stream,
                          ng + na > 0);
  if (st != GDN_OK) return st;
  if (ng > 0 && !prev) {
    std::vector<gdn_layer_io> layers(io->gdn_layers, io->gdn_layers + ng);
    for (int l = 0; l < ng; ++l)
      layers[l].workspace = L.gdn_ws_bytes ? base + (size_t)l * L.gdn_ws_stride : nullptr;
    st = gdn::commit_layers_impl(&d->gdn, ng, io->offsets, io->parents, io->accepted,
                                 layers.data(), L.gdn_ws_bytes, io->tree_status, stream, 1);
    if (st != GDN_OK) return st;
  }
  if (na > 0)
    st = gdn::attn_commit_layers_impl(&d->attn, na, io->offsets, io->parents, io->accepted,
                                      io->attn_layers, io->cache_len, io->tree_status, stream,
                                      1);
  return st;
}

}  // namespace

extern "C" {

gdn_status gdn_tree_accept_greedy(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const int32_t* draft_tokens,
                                  const int32_t* target_tokens, int32_t* accepted,
                                  int32_t* accept_len, int32_t* next_token,
                                  int32_t* tree_status, void* stream) {
  return accept_greedy_impl(desc, offsets, parents, draft_tokens, target_tokens, accepted,
                            accept_len, next_token, tree_status, stream, 0);
}

namespace {

// Checks shared by the sampling calls (before anything is enqueued).
gdn_status check_sampling(const gdn_tree_desc* desc, const int32_t* offsets,
                          const int32_t* parents, const int32_t* draft_tokens,
                          const float* target_probs, const float* draft_probs, int32_t vocab,
                          const float* uniforms, const int32_t* accepted,
                          const int32_t* accept_len, const int32_t* next_token,
                          const int32_t* tree_status) {
  if (desc == nullptr) return GDN_ERR_NULL_PTR;
  if (desc->num_seqs < 0 || desc->total_nodes < 0 || desc->max_nodes < 1 ||
      desc->max_nodes > GDN_TREE_MAX_NODES)
    return GDN_ERR_BAD_SHAPE;
  if (vocab < 4 || vocab > (1 << 20) || vocab % 4 != 0) return GDN_ERR_UNSUPPORTED;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !accepted || !accept_len || !next_token || !tree_status)
    return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 &&
      (!parents || !draft_tokens || !target_probs || !draft_probs || !uniforms))
    return GDN_ERR_NULL_PTR;
  return GDN_OK;
}

static_assert(gdn::kSamplingGroups == GDN_SAMPLING_MAX_SPLITS,
              "every workgroup of the split form takes whole groups of tiles");

// A split count the group layout supports: a power of two dividing the group
// count.
bool valid_splits(int32_t splits) {
  return splits >= 1 && splits <= gdn::kSamplingGroups && (splits & (splits - 1)) == 0;
}


}  // namespace

gdn_status gdn_tree_accept_sampling(const gdn_tree_desc* desc, const int32_t* offsets,
                                    const int32_t* parents, const int32_t* draft_tokens,
                                    const float* target_probs, const float* draft_probs,
                                    int32_t vocab, const float* uniforms, int32_t* accepted,
                                    int32_t* accept_len, int32_t* next_token,
                                    int32_t* tree_status, void* stream) {
  const gdn_status st = check_sampling(desc, offsets, parents, draft_tokens, target_probs,
                                       draft_probs, vocab, uniforms, accepted, accept_len,
                                       next_token, tree_status);
  if (st != GDN_OK || desc->num_seqs == 0) return st;
  gdn::AcceptSampleArgs a{desc->num_seqs, desc->total_nodes, desc->max_nodes, vocab, offsets,
                          parents, draft_tokens, target_probs, draft_probs, uniforms,
                          accepted, accept_len, next_token, tree_status};
  return gdn::launch_accept_sampling(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? GDN_OK
             : GDN_ERR_LAUNCH;
}

size_t gdn_tree_accept_sampling_split_workspace_bytes(const gdn_tree_desc* desc, int32_t vocab) {
  if (desc == nullptr || desc->num_seqs <= 0 || vocab < 4 || vocab > (1 << 20)) return 0;
  // per sequence two sets of [group sums | q group sums], one 64-bit word
  // each, and an arrival count
  return round_up((size_t)desc->num_seqs * (4 * gdn::kSamplingGroups + 1) * 8);
}

int32_t gdn_tree_accept_sampling_splits(const gdn_tree_desc* desc) {
  if (desc == nullptr || desc->num_seqs <= 0) return 1;
  const int cap = gdn::accept_sampling_split_capacity();
  // the largest power of two up to GDN_SAMPLING_MAX_SPLITS within cap / B
  const int fit = cap / desc->num_seqs;
  int splits = 1;
  while (splits * 2 <= fit && splits * 2 <= GDN_SAMPLING_MAX_SPLITS) splits *= 2;
  return splits;
}

gdn_status gdn_tree_accept_sampling_split(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const int32_t* draft_tokens,
                                          const float* target_probs, const float* draft_probs,
                                          int32_t vocab, const float* uniforms, int32_t splits,
                                          void* workspace, size_t workspace_bytes,
                                          int32_t* accepted, int32_t* accept_len,
                                          int32_t* next_token, int32_t* tree_status,
                                          void* stream) {
  const gdn_status st = check_sampling(desc, offsets, parents, draft_tokens, target_probs,
                                       draft_probs, vocab, uniforms, accepted, accept_len,
                                       next_token, tree_status);
  if (st != GDN_OK || desc->num_seqs == 0) return st;
  if (splits != 0 && !valid_splits(splits)) return GDN_ERR_UNSUPPORTED;
  if (splits == 0) splits = gdn_tree_accept_sampling_splits(desc);
  if (splits == 1)
    return gdn_tree_accept_sampling(desc, offsets, parents, draft_tokens, target_probs,
                                    draft_probs, vocab, uniforms, accepted, accept_len,
                                    next_token, tree_status, stream);
  if (workspace == nullptr) return GDN_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return GDN_ERR_BAD_SHAPE;
  if (workspace_bytes < gdn_tree_accept_sampling_split_workspace_bytes(desc, vocab))
    return GDN_ERR_WORKSPACE;
  gdn::AcceptSampleArgs a{desc->num_seqs, desc->total_nodes, desc->max_nodes, vocab, offsets,
                          parents, draft_tokens, target_probs, draft_probs, uniforms,
                          accepted, accept_len, next_token, tree_status};
  a.splits = splits;
  a.xch = static_cast<unsigned long long*>(workspace);
  return gdn::launch_accept_sampling_split(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? GDN_OK
             : GDN_ERR_LAUNCH;
}

gdn_status gdn_round_plan(const gdn_round_desc* desc, gdn_round_layout* layout) {
  if (layout == nullptr) return GDN_ERR_NULL_PTR;
  const gdn_status st = check_round(desc);
  if (st != GDN_OK) return st;
  plan(desc, layout);
  return GDN_OK;
}

gdn_status gdn_round_tree_for_budget(const gdn_round_desc* desc, size_t budget_bytes,
                                     int32_t max_depth, int32_t* branching, int32_t* depth,
                                     int32_t* nodes, size_t* state_bytes) {
  if (desc == nullptr || branching == nullptr || depth == nullptr || nodes == nullptr)
    return GDN_ERR_NULL_PTR;
  if (desc->n_gdn_layers < 0 || max_depth < 0) return GDN_ERR_BAD_SHAPE;
  gdn_tree_desc g = desc->gdn;
  g.max_nodes = GDN_TREE_MAX_NODES;
  g.total_nodes = 0;
  gdn_status st = gdn::check_tree_desc(&g);
  if (st != GDN_OK) return st;
  if ((long long)g.num_seqs * GDN_TREE_MAX_NODES * g.num_heads > INT_MAX) return GDN_ERR_BAD_SHAPE;
  // the GDN part of the round's arena for trees of N nodes
  auto bytes_for = [&](int N) {
    gdn_round_desc r = *desc;
    r.gdn = g;
    r.gdn.total_nodes = g.num_seqs * N;
    r.n_attn_layers = 0;
    gdn_round_layout L;
    plan(&r, &L);
    return L.total_bytes;
  };
  int best_k = 0, best_d = 0, best_n = 1;
  size_t best_bytes = bytes_for(1);
  for (int d = 1; d <= max_depth && d < GDN_TREE_MAX_NODES; ++d) {
    for (int k = 1; k <= kMaxBranching; ++k) {
      long long n = 1, level = 1;
      for (int i = 1; i <= d && n <= GDN_TREE_MAX_NODES; ++i) {
        level *= k;
        n += level;
      }
      if (n > GDN_TREE_MAX_NODES) break;  // wider trees of this depth are larger still
      const size_t bytes = bytes_for((int)n);
      if (bytes <= budget_bytes && (n > best_n || (n == best_n && k > best_k))) {
        best_k = k;
        best_d = d;
        best_n = (int)n;
        best_bytes = bytes;
      }
    }
  }
  *branching = best_k;
  *depth = best_d;
  *nodes = best_n;
  if (state_bytes) *state_bytes = best_bytes;
  return GDN_OK;
}

}  // extern "C"

namespace {

gdn_status capture_round(const gdn_round_desc* desc, const gdn_round_io* io,
                         const gdn_round_prev* prev, void* stream, gdn_round_graph* out) {
  if (desc == nullptr || io == nullptr || out == nullptr) return GDN_ERR_NULL_PTR;
  gdn_status st = check_round(desc);
  if (st != GDN_OK) return st;
  const int ng = desc->n_gdn_layers, na = desc->n_attn_layers;
  if ((ng > 0 && !io->gdn_layers) || (na > 0 && !io->attn_layers)) return GDN_ERR_NULL_PTR;
  if (io->layer_kinds) {
    int zeros = 0, ones = 0;
    for (int i = 0; i < ng + na; ++i) {
      if (io->layer_kinds[i] == 0) ++zeros;
      else if (io->layer_kinds[i] == 1) ++ones;
      else return GDN_ERR_BAD_SHAPE;
    }
    if (zeros != ng || ones != na) return GDN_ERR_BAD_SHAPE;
  }
  gdn_round_layout L;
  plan(desc, &L);
  if (io->arena_bytes < L.total_bytes) return GDN_ERR_WORKSPACE;
  if (L.total_bytes > 0 && io->arena == nullptr) return GDN_ERR_NULL_PTR;
  if (prev && ng > 0) {
    // the replay's host checks, before capture starts (enqueueing repeats them)
    if (!prev->gdn_layers) return GDN_ERR_NULL_PTR;
    for (int l = 0; l < ng; ++l) {
      const gdn_layer_io& y = io->gdn_layers[l];
      st = gdn_tree_replay_verify_layers(&prev->gdn, &desc->gdn, 0, prev->offsets,
                                         prev->parents, prev->accepted, io->offsets,
                                         io->parents, &prev->gdn_layers[l], &y,
                                         io->tree_status, nullptr);
      if (st != GDN_OK) return st;
      const gdn_layer_io& p = prev->gdn_layers[l];
      if (!y.S0 || !y.S_out || !p.k || !p.v || !p.alpha || !p.beta || !prev->offsets ||
          !prev->parents || !prev->accepted)
        return GDN_ERR_NULL_PTR;
      if (desc->gdn.num_seqs > 0 && prev->gdn.total_nodes < 1) return GDN_ERR_BAD_SHAPE;
    }
  }
  if (stream == nullptr) return GDN_ERR_GRAPH;  // the null stream cannot be captured
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return GDN_ERR_GRAPH;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return GDN_ERR_GRAPH;
  st = enqueue_round(desc, io, L, prev, stream);
  hipGraph_t graph = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &graph);
  if (st != GDN_OK || e != hipSuccess) {
    if (graph) hipGraphDestroy(graph);
    return st != GDN_OK ? st : GDN_ERR_GRAPH;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  hipGraphDestroy(graph);
  if (ei != hipSuccess) return GDN_ERR_GRAPH;
  gdn_round_graph g = new (std::nothrow) gdn_round_graph_s{exec};
  if (g == nullptr) {
    hipGraphExecDestroy(exec);
    return GDN_ERR_GRAPH;
  }
  *out = g;
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_round_capture(const gdn_round_desc* desc, const gdn_round_io* io, void* stream,
                             gdn_round_graph* out) {
  return capture_round(desc, io, nullptr, stream, out);
}

gdn_status gdn_round_capture_replay(const gdn_round_desc* desc, const gdn_round_io* io,
                                    const gdn_round_prev* prev, void* stream,
                                    gdn_round_graph* out) {
  if (prev == nullptr) return GDN_ERR_NULL_PTR;
  return capture_round(desc, io, prev, stream, out);
}

gdn_status gdn_round_launch(gdn_round_graph graph, void* stream) {
  if (graph == nullptr) return GDN_ERR_NULL_PTR;
  return hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) == hipSuccess
             ? GDN_OK
             : GDN_ERR_GRAPH;
}

void gdn_round_destroy(gdn_round_graph graph) {
  if (graph == nullptr) return;
  hipGraphExecDestroy(graph->exec);
  delete graph;
}

}  // extern "C"
