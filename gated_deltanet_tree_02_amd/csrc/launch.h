// launch.h -- internal interface between the C ABI host code and the kernel
// translation units of libgdntree (not installed, not part of the ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

struct TreeArgs {
  int B, T, max_nodes;
  const int32_t* offsets;
  const int32_t* parents;
  int32_t* depth;
  uint64_t* anc;
  int32_t* status;
};

struct VerifyArgs {
  int B, H, T, max_nodes;
  const int32_t* offsets;
  const int32_t* parents;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  void* o;
  float* U;      // [T,H,dv] pseudo-values
  float* g2;     // [T,H] base-2 gate prefixes
  int32_t* status;
  int merge = 0;  // keep a code an earlier step of the round set (put_status)
};

struct CommitArgs {
  int B, H, T, max_nodes;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
  const void* k;
  const float* S0;
  float* S_out;
  const float* U;
  const float* g2;
  int32_t* status;
  int max_depth;   // >= 0: a tree deeper than this is rejected (FORK_DELTA); -1: no limit
  // commit by replay: the path's own inputs instead of U and g2
  const void* v = nullptr;          // [T,H,dv] io
  const float* alpha = nullptr;     // [T,H]
  const float* beta = nullptr;      // [T,H]
  int merge = 0;
};

struct ForkArgs {
  int B, H, T, max_nodes, max_depth, level;
  const int32_t* offsets;
  const int32_t* parents;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  void* o;
  float* ckpt;   // [T,H,dv,dk]
  int32_t* status;
  float* U;      // FORK_DELTA: [T,H,dv] the per-node deltas, else null
  float* g2;     // FORK_DELTA: [T,H] base-2 gate prefixes, else null
  int merge = 0;
  // selective fork: a node saves its state iff conf <= threshold, in slot
  // b * max_kept + (its rank among the sequence's saved nodes); ckpt is
  // then [B * max_kept, H, dv, dk]
  const float* conf = nullptr;
  float threshold = 0.f;
  int max_kept = 0;
};

// Commit after a selective-fork verify: the accepted node's saved state, or
// the state rebuilt from its nearest saved ancestor (S0 when none) by
// replaying the path's steps from k, v, alpha, beta.
struct SelectiveCommitArgs {
  int B, H, T, max_nodes, max_depth;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
  const float* conf;
  float threshold;
  int max_kept;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  float* S_out;
  const float* ckpt;     // [B * max_kept, H, dv, dk]
  int32_t* status;
};

struct ForkCommitArgs {
  int B, H, T, max_nodes, max_depth;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
  const float* S0;
  float* S_out;
  const float* ckpt;
  int32_t* status;
  int merge = 0;
};

// io: 0 = fp32, 1 = bf16 (gdn_dtype); d = dk = dv; mt = ceil(max_nodes / 16).
hipError_t launch_tree_build(const TreeArgs& a, hipStream_t s);
// tree-masked attention (bf16 io)
struct AttnArgs {
  int B, Hq, Hkv, T, max_nodes, cap, max_len;
  int NS;            // splits of the cache per (sequence, K/V head)
  int CL;            // cache rows per split (a multiple of 64)
  float scale_log2;  // scale * log2(e)
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* cache_len;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kc;
  const uint16_t* vc;
  uint16_t* o;
  float* part_o;     // [T, Hq, NS, d] (NS > 1)
  float* part_ml;    // [T, Hq, NS, 2] (NS > 1)
  int32_t* status;
  int merge = 0;
};

// Layer-batched verify / commit: one launch covers several layers that share
// the tree (offsets, parents, accepted, status); workgroup i works on layer
// i / (B * H) with that layer's pointers.
constexpr int kMaxLayersPerLaunch = 32;

// Accepted-path KV append for `layers` attention layers that share the tree
// and the committed length: every layer's rows go to rows cache_len[b] ..,
// and cache_len advances (once) only when `advance` is set.
struct AttnCommitLayer {
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* kc;
  uint16_t* vc;
};

struct AttnCommitArgs {
  int B, Hkv, T, max_nodes, cap;
  int layers;
  int advance;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
  int32_t* cache_len;
  int32_t* status;
  AttnCommitLayer L[kMaxLayersPerLaunch];
  int merge = 0;
};

// Sampling-mode acceptance: rejection sampling of the candidates down the
// tree against the target's and the draft's distributions per node.
struct AcceptSampleArgs {
  int B, T, max_nodes, V;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* draft;
  const float* p;        // [T, V] target distribution after each node
  const float* q;        // [T, V] draft distribution the node's children were drawn from
  const float* u;        // [T, 2] uniforms: as a candidate, for the final draw
  int32_t* accepted;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* status;
  // split form: `splits` workgroups per sequence (a divisor of
  // kSamplingGroups) trade group sums through xch (per sequence, two
  // alternating sets of [group sums | q group sums], kSamplingGroups 64-bit
  // words each: the pass number above the value's bits; then one arrival
  // count per sequence), all zero between calls
  int splits = 1;
  unsigned long long* xch = nullptr;
};

// Greedy acceptance of the verified trees.
struct AcceptArgs {
  int B, T, max_nodes;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* draft;
  const int32_t* target;
  int32_t* accepted;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* status;
  // a later step of a captured round: a sequence whose status an earlier step
  // set keeps it and accepts nothing (accepted -1)
  int merge = 0;
};

struct VerifyLayer {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  void* o;
  float* U;
  float* g2;
};

struct VerifyLayersArgs {
  VerifyArgs base;   // sizes and the shared tree; its per-layer pointers are unused
  int layers;
  VerifyLayer L[kMaxLayersPerLaunch];
};

struct CommitLayer {
  const void* k;
  const float* S0;
  float* S_out;
  const float* U;
  const float* g2;
  const void* v = nullptr;          // commit by replay
  const float* alpha = nullptr;
  const float* beta = nullptr;
};

struct CommitLayersArgs {
  CommitArgs base;
  int layers;
  CommitLayer L[kMaxLayersPerLaunch];
};

// Commit of the previous round fused into this round's verify: before a
// workgroup verifies its (b, h), it applies the previous round's accepted
// path to S0 in registers (the commit's rank-|path| update), writes that
// committed state to S_out and verifies against it, so the state is read
// once per round instead of twice. `prev` is the previous round's tree.
struct PendingTree {
  int T, max_nodes;
  const int32_t* offsets;
  const int32_t* parents;
  const int32_t* accepted;
};
struct PendingLayer {
  const void* k;     // previous round's k [T', H, dk]
  const float* U;    // previous round's pseudo-values [T', H, dv] (commit from U)
  const float* g2;   // previous round's base-2 gate prefixes [T', H] (commit from U)
  const void* v;     // previous round's v [T', H, dv] (replay)
  const float* alpha;  // previous round's gates [T', H] (replay)
  const float* beta;
  float* S_out;      // committed state (may equal the layer's S0)
};
constexpr int kMaxFusedLayersPerLaunch = 24;
struct CommitVerifyLayersArgs {
  VerifyArgs base;
  PendingTree prev;
  int layers;
  VerifyLayer L[kMaxFusedLayersPerLaunch];
  PendingLayer P[kMaxFusedLayersPerLaunch];
};
// The same, with the previous round's accepted path replayed on the state
// (the gated delta rule step by step from its k, v, alpha, beta) instead of
// rebuilt from pseudo-values; this round's verify then writes no workspace.
struct ReplayVerifyLayersArgs : CommitVerifyLayersArgs {};

__device__ __forceinline__ VerifyArgs layer_args(const VerifyArgs& a, int) { return a; }
__device__ __forceinline__ VerifyArgs layer_args(const VerifyLayersArgs& la, int layer) {
  VerifyArgs a = la.base;
  const VerifyLayer& l = la.L[layer];
  a.q = l.q;
  a.k = l.k;
  a.v = l.v;
  a.alpha = l.alpha;
  a.beta = l.beta;
  a.S0 = l.S0;
  a.o = l.o;
  a.U = l.U;
  a.g2 = l.g2;
  return a;
}
__device__ __forceinline__ VerifyArgs layer_args(const CommitVerifyLayersArgs& la, int layer) {
  VerifyArgs a = la.base;
  const VerifyLayer& l = la.L[layer];
  a.q = l.q;
  a.k = l.k;
  a.v = l.v;
  a.alpha = l.alpha;
  a.beta = l.beta;
  a.S0 = l.S0;
  a.o = l.o;
  a.U = l.U;
  a.g2 = l.g2;
  return a;
}
__device__ __forceinline__ VerifyArgs layer_args(const ReplayVerifyLayersArgs& la, int layer) {
  return layer_args(static_cast<const CommitVerifyLayersArgs&>(la), layer);
}
__device__ __forceinline__ CommitArgs layer_args(const CommitArgs& a, int) { return a; }
__device__ __forceinline__ CommitArgs layer_args(const CommitLayersArgs& la, int layer) {
  CommitArgs a = la.base;
  const CommitLayer& l = la.L[layer];
  a.k = l.k;
  a.S0 = l.S0;
  a.S_out = l.S_out;
  a.U = l.U;
  a.g2 = l.g2;
  a.v = l.v;
  a.alpha = l.alpha;
  a.beta = l.beta;
  return a;
}
__device__ __forceinline__ const VerifyArgs& base_args(const VerifyArgs& a) { return a; }
__device__ __forceinline__ const VerifyArgs& base_args(const VerifyLayersArgs& a) { return a.base; }
__device__ __forceinline__ const VerifyArgs& base_args(const CommitVerifyLayersArgs& a) {
  return a.base;
}
__device__ __forceinline__ const VerifyArgs& base_args(const ReplayVerifyLayersArgs& a) {
  return a.base;
}
__device__ __forceinline__ const CommitArgs& base_args(const CommitArgs& a) { return a; }
__device__ __forceinline__ const CommitArgs& base_args(const CommitLayersArgs& a) { return a.base; }

hipError_t launch_wy_verify(int io, int d, int mt, const VerifyArgs& a, hipStream_t s);
hipError_t launch_wy_verify_layers(int io, int d, int mt, const VerifyLayersArgs& a,
                                   hipStream_t s);
hipError_t launch_wy_commit_verify_layers(int io, int d, int mt, const CommitVerifyLayersArgs& a,
                                          hipStream_t s);
hipError_t launch_wy_replay_verify_layers(int io, int d, int mt, const ReplayVerifyLayersArgs& a,
                                          hipStream_t s);
hipError_t launch_tree_attn(int d, const AttnArgs& a, hipStream_t s);
// Bytes of the fixed per-GPU scratch of the no-allocation attention verify,
// and its device address on the current device (taken once per device).
constexpr size_t kAttnScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;
__attribute__((visibility("hidden"))) hipError_t attn_scratch(void** ptr);
hipError_t launch_tree_attn_commit(int d, const AttnCommitArgs& a, hipStream_t s);
hipError_t launch_wy_commit(int io, int d, const CommitArgs& a, hipStream_t s);
hipError_t launch_wy_commit_layers(int io, int d, const CommitLayersArgs& a, hipStream_t s);
// commit by replaying the accepted path (CommitArgs v, alpha, beta set; U, g2 unused)
hipError_t launch_replay_commit(int io, int d, const CommitArgs& a, hipStream_t s);
hipError_t launch_replay_commit_layers(int io, int d, const CommitLayersArgs& a, hipStream_t s);
hipError_t launch_fork_level(int io, int d, const ForkArgs& a, hipStream_t s);
hipError_t launch_fork_commit(int d, const ForkCommitArgs& a, hipStream_t s);
hipError_t launch_fork_selective_level(int io, int d, const ForkArgs& a, hipStream_t s);
hipError_t launch_fork_selective_commit(int io, int d, const SelectiveCommitArgs& a,
                                        hipStream_t s);
hipError_t launch_accept_greedy(const AcceptArgs& a, hipStream_t s);
hipError_t launch_accept_sampling(const AcceptSampleArgs& a, hipStream_t s);
// split form: clears the exchange words, then launches B * splits
// workgroups
hipError_t launch_accept_sampling_split(const AcceptSampleArgs& a, hipStream_t s);
// workgroups of the split kernel that fit on the current device at once
int accept_sampling_split_capacity();
constexpr int kSamplingTile = 256;            // tokens per tile of a row pass
constexpr int kSamplingGroups = 16;           // fixed groups of tiles per row

// Kernel launch that reports its own error (no reliance on the sticky
// last-error state, which other libraries in the process also use).
template <class Arg>
inline hipError_t launch_kernel(const void* kernel, unsigned grid, unsigned block, hipStream_t s,
                                const Arg& arg) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(kernel, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace gdn
