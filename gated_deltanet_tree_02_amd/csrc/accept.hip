// accept.hip -- greedy acceptance of verified draft trees on gfx950.
//
// One wave per sequence, one lane per node (handbook, anrans.github.io
// ai-infra-handbooks "speculative", implementation section, generation
// loop): from the root, the target's predicted token at the current node is
// matched against the draft tokens of that node's children; the first child
// in node order that matches becomes the current node, and the walk ends at a
// node none of whose children match. Each step is one ballot over the lanes
// (child of the current node and token equal to the prediction); a child has
// a larger index than its parent, so the walk takes at most N_b - 1 steps.
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void accept_greedy_kernel(const AcceptArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + wave;
  if (b >= a.B) return;  // wave-uniform
  const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
  if (tl.status != GDN_TREE_OK) {
    if (lane == 0) {
      a.status[b] = tl.status;
      a.accepted[b] = -1;
      a.accept_len[b] = 0;
      a.next_token[b] = -1;
    }
    return;
  }
  const int n = tl.n;
  const bool live = lane >= 1 && lane < n;
  const int tok = live ? a.draft[tl.lo + lane] : 0;
  const int tgt = lane < n ? a.target[tl.lo + lane] : 0;
  int cur = 0;
  int len = 1;
  for (;;) {
    const int pred = __shfl(tgt, cur, kWave);
    const uint64_t hit = __ballot(live && tl.parent == cur && tok == pred);
    if (hit == 0ull) break;
    cur = __builtin_ctzll(hit);  // the first matching child in node order
    ++len;
  }
  const int next = __shfl(tgt, cur, kWave);
  if (lane == 0) {
    a.status[b] = GDN_TREE_OK;
    a.accepted[b] = cur;
    a.accept_len[b] = len;
    a.next_token[b] = next;
  }
}

}  // namespace

hipError_t launch_accept_greedy(const AcceptArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&accept_greedy_kernel),
                       (unsigned)((a.B + 3) / 4), 256u, s, a);
}

}  // namespace gdn
