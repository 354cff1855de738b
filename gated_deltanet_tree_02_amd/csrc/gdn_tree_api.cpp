// gdn_tree_api.cpp -- the C ABI of libgdntree: host-side checks, workspace
// sizing and kernel dispatch. Never allocates, never synchronises; every
// launch goes to the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstddef>
#include <cstdint>

#include "gdn_tree.h"
#include "api_internal.h"
#include "launch.h"

namespace gdn {

gdn_status check_tree_desc(const gdn_tree_desc* d) {
  if (d == nullptr) return GDN_ERR_NULL_PTR;
  if (d->num_seqs < 0 || d->num_heads < 1 || d->total_nodes < 0 || d->max_nodes < 1 ||
      d->max_nodes > GDN_TREE_MAX_NODES)
    return GDN_ERR_BAD_SHAPE;
  if (d->dk != d->dv || (d->dk != 32 && d->dk != 64 && d->dk != 128)) return GDN_ERR_UNSUPPORTED;
  if (d->io_dtype != GDN_DTYPE_F32 && d->io_dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (d->mode != GDN_MODE_WY && d->mode != GDN_MODE_FORK && d->mode != GDN_MODE_FORK_DELTA)
    return GDN_ERR_UNSUPPORTED;
  // grids are B*H*(chunks <= 4) workgroups; node indices (T*H) must fit int
  const long long bh = (long long)d->num_seqs * d->num_heads;
  if (bh * 4 > INT_MAX || (long long)d->total_nodes * d->num_heads > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

}  // namespace gdn

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

gdn_status check_desc(const gdn_tree_desc* d) { return gdn::check_tree_desc(d); }

int levels(const gdn_tree_desc* d) {
  const int md = d->max_depth > 0 ? d->max_depth : d->max_nodes - 1;
  return (md < d->max_nodes - 1 ? md : d->max_nodes - 1) + 1;
}

size_t wy_u_bytes(const gdn_tree_desc* d) {
  return round_up((size_t)d->total_nodes * d->num_heads * d->dv * sizeof(float));
}

// U and g2: the part of the workspace that commit reads (WY and FORK_DELTA)
size_t wy_bytes(const gdn_tree_desc* d) {
  const size_t th = (size_t)d->total_nodes * d->num_heads;
  return wy_u_bytes(d) + round_up(th * sizeof(float));
}

size_t state_bytes(const gdn_tree_desc* d) {
  return round_up((size_t)d->total_nodes * d->num_heads * d->dv * d->dk * sizeof(float));
}

size_t workspace_bytes(const gdn_tree_desc* d) {
  if (d->mode == GDN_MODE_FORK) return state_bytes(d);
  if (d->mode == GDN_MODE_FORK_DELTA) return wy_bytes(d) + state_bytes(d);
  return wy_bytes(d);
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// FORK_DELTA verify runs a fixed number of levels; its commit rejects deeper
// trees as FORK's does. WY has no depth limit.
int commit_depth_limit(const gdn_tree_desc* d) {
  return d->mode == GDN_MODE_FORK_DELTA ? levels(d) - 1 : -1;
}

}  // namespace

extern "C" {

size_t gdn_tree_workspace_bytes(const gdn_tree_desc* desc) {
  if (check_desc(desc) != GDN_OK) return 0;
  return workspace_bytes(desc);
}

gdn_status gdn_tree_build(const gdn_tree_desc* desc, const int32_t* offsets,
                          const int32_t* parents, int32_t* depth, uint64_t* anc_mask,
                          int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !depth || !anc_mask)) return GDN_ERR_NULL_PTR;
  gdn::TreeArgs a{desc->num_seqs, desc->total_nodes, desc->max_nodes, offsets, parents,
                  depth, anc_mask, tree_status};
  return launched(gdn::launch_tree_build(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace gdn {

gdn_status verify_impl(const gdn_tree_desc* desc, const int32_t* offsets,
                       const int32_t* parents, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const float* S0, void* o,
                       void* workspace, size_t ws_bytes, int32_t* tree_status, void* stream,
                       int merge) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !tree_status || !S0) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 &&
      (!parents || !q || !k || !v || !alpha || !beta || !o || !workspace))
    return GDN_ERR_NULL_PTR;
  if (ws_bytes < workspace_bytes(desc)) return GDN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = desc->dk;
  if (desc->mode == GDN_MODE_WY) {
    float* U = static_cast<float*>(workspace);
    float* g2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + wy_u_bytes(desc));
    gdn::VerifyArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                      offsets, parents, q, k, v, alpha, beta, S0, o, U, g2, tree_status};
    a.merge = merge;
    const int mt = (desc->max_nodes + 15) / 16;
    return launched(gdn::launch_wy_verify(desc->io_dtype, d, mt, a, s));
  }
  const int L = levels(desc);
  const bool delta = desc->mode == GDN_MODE_FORK_DELTA;
  char* ws = static_cast<char*>(workspace);
  float* ckpt = reinterpret_cast<float*>(delta ? ws + wy_bytes(desc) : ws);
  float* U = delta ? reinterpret_cast<float*>(ws) : nullptr;
  float* g2 = delta ? reinterpret_cast<float*>(ws + wy_u_bytes(desc)) : nullptr;
  for (int level = 0; level < L; ++level) {
    gdn::ForkArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                    L - 1, level, offsets, parents, q, k, v, alpha, beta, S0, o,
                    ckpt, tree_status, U, g2};
    a.merge = merge;
    st = launched(gdn::launch_fork_level(desc->io_dtype, d, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_verify(const gdn_tree_desc* desc, const int32_t* offsets,
                           const int32_t* parents, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta,
                           const float* S0, void* o, void* workspace, size_t ws_bytes,
                           int32_t* tree_status, void* stream) {
  return gdn::verify_impl(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace,
                          ws_bytes, tree_status, stream, 0);
}

}  // extern "C"

namespace gdn {

gdn_status commit_impl(const gdn_tree_desc* desc, const int32_t* offsets,
                       const int32_t* parents, const int32_t* accepted, const void* k,
                       const float* S0, float* S_out, const void* workspace, size_t ws_bytes,
                       int32_t* tree_status, void* stream, int merge) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !accepted || !S0 || !S_out || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !workspace)) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && desc->mode != GDN_MODE_FORK && !k) return GDN_ERR_NULL_PTR;
  if (ws_bytes < workspace_bytes(desc)) return GDN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = desc->dk;
  if (desc->mode != GDN_MODE_FORK) {
    // WY, and FORK_DELTA, whose deltas are the same pseudo-values
    const float* U = static_cast<const float*>(workspace);
    const float* g2 =
        reinterpret_cast<const float*>(static_cast<const char*>(workspace) + wy_u_bytes(desc));
    gdn::CommitArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                      offsets, parents, accepted, k, S0, S_out, U, g2, tree_status,
                      commit_depth_limit(desc)};
    a.merge = merge;
    return launched(gdn::launch_wy_commit(desc->io_dtype, d, a, s));
  }
  gdn::ForkCommitArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                        levels(desc) - 1, offsets, parents, accepted, S0, S_out,
                        static_cast<const float*>(workspace), tree_status};
  a.merge = merge;
  return launched(gdn::launch_fork_commit(d, a, s));
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                           const int32_t* parents, const int32_t* accepted, const void* k,
                           const float* S0, float* S_out, const void* workspace,
                           size_t ws_bytes, int32_t* tree_status, void* stream) {
  return gdn::commit_impl(desc, offsets, parents, accepted, k, S0, S_out, workspace, ws_bytes,
                          tree_status, stream, 0);
}

gdn_status gdn_tree_verify_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                  const int32_t* offsets, const int32_t* parents,
                                  const gdn_layer_io* layers, size_t ws_bytes,
                                  int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (n_layers <= 0 || desc->num_seqs == 0) return GDN_OK;
  if (!layers) return GDN_ERR_NULL_PTR;
  if (desc->mode != GDN_MODE_WY) {
    for (int l = 0; l < n_layers; ++l) {
      const gdn_layer_io& y = layers[l];
      st = gdn_tree_verify(desc, offsets, parents, y.q, y.k, y.v, y.alpha, y.beta, y.S0, y.o,
                           y.workspace, ws_bytes, tree_status, stream);
      if (st != GDN_OK) return st;
    }
    return GDN_OK;
  }
  if (!offsets || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  for (int l = 0; l < n_layers; ++l) {
    const gdn_layer_io& y = layers[l];
    if (!y.S0) return GDN_ERR_NULL_PTR;
    if (desc->total_nodes > 0 && (!y.q || !y.k || !y.v || !y.alpha || !y.beta || !y.o ||
                                  !y.workspace))
      return GDN_ERR_NULL_PTR;
  }
  if (ws_bytes < workspace_bytes(desc)) return GDN_ERR_WORKSPACE;
  if ((long long)desc->num_seqs * desc->num_heads * gdn::kMaxLayersPerLaunch > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mt = (desc->max_nodes + 15) / 16;
  gdn::VerifyLayersArgs a{};
  a.base = gdn::VerifyArgs{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                           offsets, parents, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, tree_status};
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxLayersPerLaunch) {
    a.layers = std::min(n_layers - l0, gdn::kMaxLayersPerLaunch);
    for (int i = 0; i < a.layers; ++i) {
      const gdn_layer_io& y = layers[l0 + i];
      float* U = static_cast<float*>(y.workspace);
      float* g2 = reinterpret_cast<float*>(static_cast<char*>(y.workspace) + wy_u_bytes(desc));
      a.L[i] = gdn::VerifyLayer{y.q, y.k, y.v, y.alpha, y.beta, y.S0, y.o, U, g2};
    }
    st = launched(gdn::launch_wy_verify_layers(desc->io_dtype, desc->dk, mt, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

}  // extern "C"

namespace gdn {

gdn_status commit_layers_impl(const gdn_tree_desc* desc, int32_t n_layers,
                              const int32_t* offsets, const int32_t* parents,
                              const int32_t* accepted, const gdn_layer_io* layers,
                              size_t ws_bytes, int32_t* tree_status, void* stream, int merge) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (n_layers <= 0 || desc->num_seqs == 0) return GDN_OK;
  if (!layers) return GDN_ERR_NULL_PTR;
  if (desc->mode == GDN_MODE_FORK) {
    for (int l = 0; l < n_layers; ++l) {
      const gdn_layer_io& y = layers[l];
      st = commit_impl(desc, offsets, parents, accepted, y.k, y.S0, y.S_out, y.workspace,
                       ws_bytes, tree_status, stream, merge);
      if (st != GDN_OK) return st;
    }
    return GDN_OK;
  }
  if (!offsets || !accepted || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  for (int l = 0; l < n_layers; ++l) {
    const gdn_layer_io& y = layers[l];
    if (!y.S0 || !y.S_out) return GDN_ERR_NULL_PTR;
    if (desc->total_nodes > 0 && (!y.workspace || !y.k)) return GDN_ERR_NULL_PTR;
  }
  if (ws_bytes < workspace_bytes(desc)) return GDN_ERR_WORKSPACE;
  if ((long long)desc->num_seqs * desc->num_heads * gdn::kMaxLayersPerLaunch > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  gdn::CommitLayersArgs a{};
  a.base = gdn::CommitArgs{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                           offsets, parents, accepted, nullptr, nullptr, nullptr, nullptr,
                           nullptr, tree_status, commit_depth_limit(desc)};
  a.base.merge = merge;
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxLayersPerLaunch) {
    a.layers = std::min(n_layers - l0, gdn::kMaxLayersPerLaunch);
    for (int i = 0; i < a.layers; ++i) {
      const gdn_layer_io& y = layers[l0 + i];
      const float* U = static_cast<const float*>(y.workspace);
      const float* g2 = reinterpret_cast<const float*>(static_cast<const char*>(y.workspace) +
                                                       wy_u_bytes(desc));
      a.L[i] = gdn::CommitLayer{y.k, y.S0, y.S_out, U, g2};
    }
    st = launched(gdn::launch_wy_commit_layers(desc->io_dtype, desc->dk, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_commit_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                  const int32_t* offsets, const int32_t* parents,
                                  const int32_t* accepted, const gdn_layer_io* layers,
                                  size_t ws_bytes, int32_t* tree_status, void* stream) {
  return gdn::commit_layers_impl(desc, n_layers, offsets, parents, accepted, layers, ws_bytes,
                                 tree_status, stream, 0);
}

gdn_status gdn_tree_commit_verify_layers(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    size_t prev_ws_bytes, const gdn_layer_io* layers, size_t ws_bytes, int32_t* tree_status,
    void* stream) {
  gdn_status st = check_desc(prev_desc);
  if (st != GDN_OK) return st;
  st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (prev_desc->mode != GDN_MODE_WY || desc->mode != GDN_MODE_WY) return GDN_ERR_UNSUPPORTED;
  if (prev_desc->num_seqs != desc->num_seqs || prev_desc->num_heads != desc->num_heads ||
      prev_desc->dk != desc->dk || prev_desc->dv != desc->dv ||
      prev_desc->io_dtype != desc->io_dtype)
    return GDN_ERR_BAD_SHAPE;
  if (n_layers <= 0 || desc->num_seqs == 0) return GDN_OK;
  // every previous tree holds at least one node, so its rows are addressable
  if (prev_desc->total_nodes < 1) return GDN_ERR_BAD_SHAPE;
  if (!layers || !prev_layers || !prev_offsets || !prev_parents || !accepted || !offsets ||
      !tree_status)
    return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  if (ws_bytes < workspace_bytes(desc) || prev_ws_bytes < workspace_bytes(prev_desc))
    return GDN_ERR_WORKSPACE;
  for (int l = 0; l < n_layers; ++l) {
    const gdn_layer_io& y = layers[l];
    const gdn_layer_io& p = prev_layers[l];
    if (!y.S0 || !y.S_out || !p.k || !p.workspace) return GDN_ERR_NULL_PTR;
    if (desc->total_nodes > 0 && (!y.q || !y.k || !y.v || !y.alpha || !y.beta || !y.o ||
                                  !y.workspace))
      return GDN_ERR_NULL_PTR;
    // this round's workspace is written while the previous one is read
    if (y.workspace) {
      const char* w0 = static_cast<const char*>(y.workspace);
      const char* p0 = static_cast<const char*>(p.workspace);
      if (w0 < p0 + prev_ws_bytes && p0 < w0 + ws_bytes) return GDN_ERR_BAD_SHAPE;
    }
  }
  if ((long long)desc->num_seqs * desc->num_heads * gdn::kMaxFusedLayersPerLaunch > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mt = (desc->max_nodes + 15) / 16;
  gdn::CommitVerifyLayersArgs a{};
  a.base = gdn::VerifyArgs{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                           offsets, parents, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, tree_status};
  a.prev = gdn::PendingTree{prev_desc->total_nodes, prev_desc->max_nodes, prev_offsets,
                            prev_parents, accepted};
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxFusedLayersPerLaunch) {
    a.layers = std::min(n_layers - l0, gdn::kMaxFusedLayersPerLaunch);
    for (int i = 0; i < a.layers; ++i) {
      const gdn_layer_io& y = layers[l0 + i];
      const gdn_layer_io& p = prev_layers[l0 + i];
      float* U = static_cast<float*>(y.workspace);
      float* g2 = U ? reinterpret_cast<float*>(static_cast<char*>(y.workspace) + wy_u_bytes(desc))
                    : nullptr;
      a.L[i] = gdn::VerifyLayer{y.q, y.k, y.v, y.alpha, y.beta, y.S0, y.o, U, g2};
      const float* pU = static_cast<const float*>(p.workspace);
      const float* pg2 = reinterpret_cast<const float*>(static_cast<const char*>(p.workspace) +
                                                        wy_u_bytes(prev_desc));
      a.P[i] = gdn::PendingLayer{p.k, pU, pg2, nullptr, nullptr, nullptr, y.S_out};
    }
    st = launched(gdn::launch_wy_commit_verify_layers(desc->io_dtype, desc->dk, mt, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

gdn_status gdn_tree_commit_verify(const gdn_tree_desc* prev_desc, const int32_t* prev_offsets,
                                  const int32_t* prev_parents, const int32_t* accepted,
                                  const void* prev_k, const void* prev_workspace,
                                  size_t prev_ws_bytes, const gdn_tree_desc* desc,
                                  const int32_t* offsets, const int32_t* parents, const void* q,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* S0, float* S_out, void* o,
                                  void* workspace, size_t ws_bytes, int32_t* tree_status,
                                  void* stream) {
  gdn_layer_io prev{};
  prev.k = prev_k;
  prev.workspace = const_cast<void*>(prev_workspace);
  gdn_layer_io cur{q, k, v, alpha, beta, S0, o, S_out, workspace};
  return gdn_tree_commit_verify_layers(prev_desc, desc, 1, prev_offsets, prev_parents, accepted,
                                       offsets, parents, &prev, prev_ws_bytes, &cur, ws_bytes,
                                       tree_status, stream);
}

}  // extern "C"

namespace gdn {

gdn_status replay_verify_layers_impl(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    const gdn_layer_io* layers, int32_t* tree_status, void* stream, int merge) {
  gdn_status st = check_desc(prev_desc);
  if (st != GDN_OK) return st;
  st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (prev_desc->mode != GDN_MODE_WY || desc->mode != GDN_MODE_WY) return GDN_ERR_UNSUPPORTED;
  if (prev_desc->num_seqs != desc->num_seqs || prev_desc->num_heads != desc->num_heads ||
      prev_desc->dk != desc->dk || prev_desc->dv != desc->dv ||
      prev_desc->io_dtype != desc->io_dtype)
    return GDN_ERR_BAD_SHAPE;
  if (n_layers <= 0 || desc->num_seqs == 0) return GDN_OK;
  if (prev_desc->total_nodes < 1) return GDN_ERR_BAD_SHAPE;
  if (!layers || !prev_layers || !prev_offsets || !prev_parents || !accepted || !offsets ||
      !tree_status)
    return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  for (int l = 0; l < n_layers; ++l) {
    const gdn_layer_io& y = layers[l];
    const gdn_layer_io& p = prev_layers[l];
    if (!y.S0 || !y.S_out || !p.k || !p.v || !p.alpha || !p.beta) return GDN_ERR_NULL_PTR;
    if (desc->total_nodes > 0 && (!y.q || !y.k || !y.v || !y.alpha || !y.beta || !y.o))
      return GDN_ERR_NULL_PTR;
  }
  if ((long long)desc->num_seqs * desc->num_heads * gdn::kMaxFusedLayersPerLaunch > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mt = (desc->max_nodes + 15) / 16;
  gdn::ReplayVerifyLayersArgs a{};
  a.base = gdn::VerifyArgs{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                           offsets, parents, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, tree_status};
  a.base.merge = merge;
  a.prev = gdn::PendingTree{prev_desc->total_nodes, prev_desc->max_nodes, prev_offsets,
                            prev_parents, accepted};
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxFusedLayersPerLaunch) {
    a.layers = std::min(n_layers - l0, gdn::kMaxFusedLayersPerLaunch);
    for (int i = 0; i < a.layers; ++i) {
      const gdn_layer_io& y = layers[l0 + i];
      const gdn_layer_io& p = prev_layers[l0 + i];
      a.L[i] = gdn::VerifyLayer{y.q, y.k, y.v, y.alpha, y.beta, y.S0, y.o, nullptr, nullptr};
      a.P[i] = gdn::PendingLayer{p.k, nullptr, nullptr, p.v, p.alpha, p.beta, y.S_out};
    }
    st = launched(gdn::launch_wy_replay_verify_layers(desc->io_dtype, desc->dk, mt, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_replay_verify_layers(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    const gdn_layer_io* layers, int32_t* tree_status, void* stream) {
  return gdn::replay_verify_layers_impl(prev_desc, desc, n_layers, prev_offsets, prev_parents,
                                        accepted, offsets, parents, prev_layers, layers,
                                        tree_status, stream, 0);
}

gdn_status gdn_tree_replay_verify(const gdn_tree_desc* prev_desc, const int32_t* prev_offsets,
                                  const int32_t* prev_parents, const int32_t* accepted,
                                  const void* prev_k, const void* prev_v,
                                  const float* prev_alpha, const float* prev_beta,
                                  const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const float* S0, float* S_out, void* o, int32_t* tree_status,
                                  void* stream) {
  gdn_layer_io prev{};
  prev.k = prev_k;
  prev.v = prev_v;
  prev.alpha = prev_alpha;
  prev.beta = prev_beta;
  gdn_layer_io cur{q, k, v, alpha, beta, S0, o, S_out, nullptr};
  return gdn_tree_replay_verify_layers(prev_desc, desc, 1, prev_offsets, prev_parents, accepted,
                                       offsets, parents, &prev, &cur, tree_status, stream);
}

gdn_status gdn_tree_replay_commit_layers(const gdn_tree_desc* desc, int32_t n_layers,
                                         const int32_t* offsets, const int32_t* parents,
                                         const int32_t* accepted, const gdn_layer_io* layers,
                                         int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (n_layers <= 0 || desc->num_seqs == 0) return GDN_OK;
  if (!layers || !offsets || !accepted || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && !parents) return GDN_ERR_NULL_PTR;
  for (int l = 0; l < n_layers; ++l) {
    const gdn_layer_io& y = layers[l];
    if (!y.S0 || !y.S_out) return GDN_ERR_NULL_PTR;
    if (desc->total_nodes > 0 && (!y.k || !y.v || !y.alpha || !y.beta)) return GDN_ERR_NULL_PTR;
  }
  if ((long long)desc->num_seqs * desc->num_heads * gdn::kMaxLayersPerLaunch > INT_MAX)
    return GDN_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  gdn::CommitLayersArgs a{};
  a.base = gdn::CommitArgs{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                           offsets, parents, accepted, nullptr, nullptr, nullptr, nullptr,
                           nullptr, tree_status, -1};
  for (int l0 = 0; l0 < n_layers; l0 += gdn::kMaxLayersPerLaunch) {
    a.layers = std::min(n_layers - l0, gdn::kMaxLayersPerLaunch);
    for (int i = 0; i < a.layers; ++i) {
      const gdn_layer_io& y = layers[l0 + i];
      a.L[i] = gdn::CommitLayer{y.k, y.S0, y.S_out, nullptr, nullptr, y.v, y.alpha, y.beta};
    }
    st = launched(gdn::launch_replay_commit_layers(desc->io_dtype, desc->dk, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

gdn_status gdn_tree_replay_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const int32_t* accepted,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* S0, float* S_out,
                                  int32_t* tree_status, void* stream) {
  gdn_layer_io y{};
  y.k = k;
  y.v = v;
  y.alpha = alpha;
  y.beta = beta;
  y.S0 = S0;
  y.S_out = S_out;
  return gdn_tree_replay_commit_layers(desc, 1, offsets, parents, accepted, &y, tree_status,
                                       stream);
}

size_t gdn_tree_fork_selective_workspace_bytes(const gdn_tree_desc* desc, int32_t max_kept) {
  if (check_desc(desc) != GDN_OK || max_kept < 0 || max_kept > desc->max_nodes) return 0;
  return round_up((size_t)desc->num_seqs * max_kept * desc->num_heads * desc->dv * desc->dk *
                  sizeof(float));
}

gdn_status gdn_tree_fork_selective_verify(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const float* confidence,
                                          float threshold, int32_t max_kept, const void* q,
                                          const void* k, const void* v, const float* alpha,
                                          const float* beta, const float* S0, void* o,
                                          void* workspace, size_t ws_bytes,
                                          int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (max_kept < 0 || max_kept > desc->max_nodes) return GDN_ERR_BAD_SHAPE;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !tree_status || !S0) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 &&
      (!parents || !confidence || !q || !k || !v || !alpha || !beta || !o))
    return GDN_ERR_NULL_PTR;
  const size_t need = gdn_tree_fork_selective_workspace_bytes(desc, max_kept);
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (need > 0 && !workspace) return GDN_ERR_NULL_PTR;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = levels(desc);
  for (int level = 0; level < L; ++level) {
    gdn::ForkArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes, desc->max_nodes,
                    L - 1, level, offsets, parents, q, k, v, alpha, beta, S0, o,
                    static_cast<float*>(workspace), tree_status, nullptr, nullptr};
    a.conf = confidence;
    a.threshold = threshold;
    a.max_kept = max_kept;
    st = launched(gdn::launch_fork_selective_level(desc->io_dtype, desc->dk, a, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

gdn_status gdn_tree_fork_selective_commit(const gdn_tree_desc* desc, const int32_t* offsets,
                                          const int32_t* parents, const float* confidence,
                                          float threshold, int32_t max_kept,
                                          const int32_t* accepted, const void* k, const void* v,
                                          const float* alpha, const float* beta,
                                          const float* S0, float* S_out, const void* workspace,
                                          size_t ws_bytes, int32_t* tree_status, void* stream) {
  gdn_status st = check_desc(desc);
  if (st != GDN_OK) return st;
  if (max_kept < 0 || max_kept > desc->max_nodes) return GDN_ERR_BAD_SHAPE;
  if (desc->num_seqs == 0) return GDN_OK;
  if (!offsets || !accepted || !S0 || !S_out || !tree_status) return GDN_ERR_NULL_PTR;
  if (desc->total_nodes > 0 && (!parents || !confidence || !k || !v || !alpha || !beta))
    return GDN_ERR_NULL_PTR;
  const size_t need = gdn_tree_fork_selective_workspace_bytes(desc, max_kept);
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (need > 0 && !workspace) return GDN_ERR_NULL_PTR;
  gdn::SelectiveCommitArgs a{desc->num_seqs, desc->num_heads, desc->total_nodes,
                             desc->max_nodes, levels(desc) - 1, offsets, parents, accepted,
                             confidence, threshold, max_kept, k, v, alpha, beta, S0, S_out,
                             static_cast<const float*>(workspace), tree_status};
  return launched(gdn::launch_fork_selective_commit(desc->io_dtype, desc->dk, a,
                                                    static_cast<hipStream_t>(stream)));
}

const char* gdn_tree_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_PTR: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "invalid sizes in the descriptor";
    case GDN_ERR_UNSUPPORTED: return "unsupported head size, io dtype, mode or head grouping";
    case GDN_ERR_WORKSPACE: return "workspace smaller than the entry point's workspace_bytes()";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_GRAPH: return "graph capture, instantiation or launch failed";
    case GDN_ERR_SCRATCH: return "the call needs more scratch than the library's fixed buffer";
  }
  return "unknown status";
}

}  // extern "C"
