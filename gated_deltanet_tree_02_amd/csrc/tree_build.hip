// tree_build.hip -- ancestor masks and depths of every draft node.
//
// One wave per sequence, one lane per node: the row of the tree attention
// mask (a node sees itself and its ancestors, never a sibling: fork page
// section 2; handbook implementation section, tree_mask) as a 64-bit set, and
// the depth with the root at 0 (handbook depths()). The construction itself
// is the pointer-jumping prologue every kernel of the library shares.
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void tree_build_kernel(const TreeArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + wave;
  if (b >= a.B) return;  // wave-uniform
  const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
  if (lane == 0) a.status[b] = tl.status;
  if (tl.status == GDN_TREE_BAD_SIZE) return;
  if (lane < tl.n) {
    const bool ok = tl.status == GDN_TREE_OK;
    a.depth[tl.lo + lane] = ok ? tl.depth : -1;
    a.anc[tl.lo + lane] = ok ? tl.anc : 0ull;
  }
}

}  // namespace

hipError_t launch_tree_build(const TreeArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&tree_build_kernel),
                       (unsigned)((a.B + 3) / 4), 256u, s, a);
}

}  // namespace gdn
