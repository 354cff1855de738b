// api_internal.h -- descriptor checks shared by the host-side C ABI files of
// libgdntree (not installed, not part of the ABI, not exported).
#pragma once

#include "gdn_tree.h"
#include "gdn_tree_attn.h"

namespace gdn {

// The synchronous checks every entry point of gdn_tree.h / gdn_tree_attn.h
// makes on its descriptor before anything is enqueued.
__attribute__((visibility("hidden"))) gdn_status check_tree_desc(const gdn_tree_desc* d);
__attribute__((visibility("hidden"))) gdn_status check_attn_desc(const gdn_attn_desc* d);

// The entry points a captured round composes, with one more argument: merge
// != 0 for every step after the round's first, so that a sequence keeps the
// first nonzero code any step of the round reported (an acceptance run with
// merge != 0 then accepts nothing for it). The public entry points pass 0.
#define GDN_HIDDEN __attribute__((visibility("hidden")))
GDN_HIDDEN gdn_status verify_impl(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const float* S0, void* o, void* workspace, size_t ws_bytes,
                                  int32_t* tree_status, void* stream, int merge);
GDN_HIDDEN gdn_status commit_impl(const gdn_tree_desc* desc, const int32_t* offsets,
                                  const int32_t* parents, const int32_t* accepted,
                                  const void* k, const float* S0, float* S_out,
                                  const void* workspace, size_t ws_bytes, int32_t* tree_status,
                                  void* stream, int merge);
GDN_HIDDEN gdn_status commit_layers_impl(const gdn_tree_desc* desc, int32_t n_layers,
                                         const int32_t* offsets, const int32_t* parents,
                                         const int32_t* accepted, const gdn_layer_io* layers,
                                         size_t ws_bytes, int32_t* tree_status, void* stream,
                                         int merge);
GDN_HIDDEN gdn_status replay_verify_layers_impl(
    const gdn_tree_desc* prev_desc, const gdn_tree_desc* desc, int32_t n_layers,
    const int32_t* prev_offsets, const int32_t* prev_parents, const int32_t* accepted,
    const int32_t* offsets, const int32_t* parents, const gdn_layer_io* prev_layers,
    const gdn_layer_io* layers, int32_t* tree_status, void* stream, int merge);
GDN_HIDDEN gdn_status attn_verify_impl(const gdn_attn_desc* desc, const int32_t* offsets,
                                       const int32_t* parents, const void* q, const void* k,
                                       const void* v, const void* k_cache, const void* v_cache,
                                       const int32_t* cache_len, float scale, void* o,
                                       void* workspace, size_t ws_bytes, int32_t* tree_status,
                                       void* stream, int merge);
GDN_HIDDEN gdn_status attn_commit_layers_impl(const gdn_attn_desc* desc, int32_t n_layers,
                                              const int32_t* offsets, const int32_t* parents,
                                              const int32_t* accepted,
                                              const gdn_attn_layer_io* layers,
                                              int32_t* cache_len, int32_t* tree_status,
                                              void* stream, int merge);
#undef GDN_HIDDEN

}  // namespace gdn
