// fork.hip -- the fork/checkpoint baseline (fork page, section 4, with its
// depth-by-depth subsection; section 5 for the rollback copy).
//
// Verify runs one launch per depth level. A workgroup owns 32 state rows of
// one (sequence, head) and steps every node of that level in the sequence:
// it reads the parent's checkpoint (S0 for the root), applies
//     w = C_p k_t,   C_t = alpha_t C_p + beta_t (v_t - alpha_t w) k_t^T,
//     o_t = C_t q_t,
// and stores C_t as the node's checkpoint. Rows of the state evolve
// independently under the gated delta rule, so splitting rows across
// workgroups is exact. Commit copies the accepted node's checkpoint.
//
// With delta-compressed checkpoints (DELTA; fork page, section 8, checkpoint
// compression: keep only what a child adds to its parent's state), the kept
// part of node t is what C_t adds to alpha_t C_p: the rank-one term
// u_t k_t^T, u_t = beta_t (v_t - alpha_t w), and the gate. Verify stores u_t
// and the base-2 gate prefix g2_t in the WY workspace layout, and a node's full
// state only while its children still need it (nodes without children are
// never written); commit rebuilds the accepted state from S0 and the deltas
// of its path, which is the WY commit.
//
// With selective fork (SEL; fork page, section 8, selective fork: a node whose
// draft confidence is above 0.95 keeps no rollback point) a node saves its
// state only when its confidence is at most the threshold, into a per-sequence
// slot. A node then starts from its nearest saved proper ancestor (S0 when
// there is none) and applies the steps of every path node below it, its own
// last: an unsaved parent's state is rebuilt, not stored. The plain fork is
// the case where every node is saved and the only step is the node's own.
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

// Sum over the `width` consecutive lanes that share one state row.
template <int W>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Selective fork: the saved nodes of a sequence (confidence at most the
// threshold), one lane per node; lanes >= n give 0.
__device__ __forceinline__ uint64_t saved_nodes(const float* __restrict__ conf, float threshold,
                                                int lo, int n, int lane) {
  const float c = conf[lo + (lane < n ? lane : 0)];
  return __ballot(lane < n && c <= threshold);
}

// Slot of saved node j of sequence b: b * max_kept + its rank among the saved.
__device__ __forceinline__ size_t saved_slot(int b, int max_kept, uint64_t saved, int j) {
  return (size_t)b * max_kept + __popcll(saved & ((1ull << j) - 1ull));
}

template <class IO, int DK, int DV, bool DELTA, bool SEL>
__global__ __launch_bounds__(256) void fork_level_kernel(const ForkArgs a) {
  constexpr int TPR = DK / 4;        // threads per state row (one float4 each)
  constexpr int RPP = 256 / TPR;     // rows per pass
  constexpr int CR = 32;             // rows per workgroup
  constexpr int NCH = DV / CR;
  constexpr int NPASS = CR / RPP;
  using io = io_traits<IO>;
  static_assert(!(DELTA && SEL), "one checkpoint scheme at a time");

  __shared__ int sPar[64];
  __shared__ int sInfo[3];
  __shared__ uint64_t sLevel;
  __shared__ uint64_t sHasChild;   // DELTA: nodes whose state a child reads
  __shared__ float sG2[64];        // DELTA: base-2 gate prefixes
  __shared__ uint64_t sAnc[SEL ? 64 : 1];   // SEL: each node's root path
  __shared__ uint64_t sSaved;               // SEL: nodes that keep a checkpoint

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int bh = blockIdx.x / NCH;
  const int ch = blockIdx.x - bh * NCH;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;

  if (tid < 64) {
    const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
    int st = tl.status;
    if (st == GDN_TREE_OK) {
      int dmax = tl.depth;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off, kWave));
      if (dmax > a.max_depth) st = GDN_TREE_TOO_DEEP;
    }
    uint64_t saved = 0ull;
    if constexpr (SEL) {
      if (st == GDN_TREE_OK) {
        saved = saved_nodes(a.conf, a.threshold, tl.lo, tl.n, lane);
        if (__popcll(saved) > a.max_kept) st = GDN_TREE_TOO_MANY_KEPT;
      }
      sAnc[lane] = tl.anc;
    }
    const uint64_t lvl = __ballot(st == GDN_TREE_OK && lane < tl.n && tl.depth == a.level);
    sPar[lane] = tl.parent;
    if constexpr (DELTA) {
      // gate prefix along the path (the same pointer-jumping sum the WY
      // verify uses, so both write identical g2), and which nodes have children
      const int n0 = st == GDN_TREE_BAD_SIZE ? 0 : tl.n;
      const float x = lane < n0 ? gate_log2(a.alpha[(size_t)(tl.lo + lane) * a.H + h]) : 0.f;
      uint64_t anc;
      float g2;
      path_scan(lane < n0 ? tl.parent : -1, lane, n0, x, anc, g2);
      sG2[lane] = g2;
      uint64_t kids = 0ull;
      for (int j = 1; j < n0; ++j) {
        const int pj = __shfl(tl.parent, j, kWave);
        if (pj >= 0 && pj < 64) kids |= 1ull << pj;
      }
      if (lane == 0) sHasChild = kids;
    }
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = tl.lo;
      sInfo[2] = tl.n;
      sLevel = lvl;
      sSaved = saved;
      if (a.level == 0 && h == 0 && ch == 0) put_status(a.status, b, st, a.merge);
    }
  }
  __syncthreads();
  const int st = sInfo[0];
  const int lo = sInfo[1];
  const int n = sInfo[2];
  const int rin = tid / TPR;
  const int c = 4 * (tid - rin * TPR);
  IO* __restrict__ o = static_cast<IO*>(a.o);
  if (st != GDN_TREE_OK) {
    // rows of a rejected sequence are zero (written once, by the level-0 launch)
    if (st != GDN_TREE_BAD_SIZE && a.level == 0 && c == 0) {
      for (int t = 0; t < n; ++t)
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const size_t r = ((size_t)(lo + t) * H + h) * DV + ch * CR + ps * RPP + rin;
          io::store1(o + r, 0.f);
          if constexpr (DELTA) a.U[r] = 0.f;
        }
      if constexpr (DELTA) {
        if (ch == 0 && rin == 0)
          for (int t = 0; t < n; ++t) a.g2[(size_t)(lo + t) * H + h] = 0.f;
      }
    }
    return;
  }

  const IO* __restrict__ q = static_cast<const IO*>(a.q);
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  const IO* __restrict__ v = static_cast<const IO*>(a.v);
  const uint64_t saved = SEL ? sSaved : 0ull;
  uint64_t msk = sLevel;
  while (msk) {
    const int t = __builtin_ctzll(msk);
    msk &= msk - 1;
    const int p = sPar[t];
    const size_t gt = (size_t)(lo + t) * H + h;
    // the state to start from (node s, -1 = S0) and the steps to apply: the
    // parent and the node's own step (plain fork), or the nearest saved
    // proper ancestor and every path node below it (selective fork)
    int s_node = p;
    uint64_t steps = 1ull << t;
    if constexpr (SEL) {
      const uint64_t path = sAnc[t];
      const uint64_t up = path & ~(1ull << t) & saved;
      s_node = up ? 63 - __builtin_clzll(up) : -1;
      steps = s_node < 0 ? path : path & ~((2ull << s_node) - 1ull);
    }
    const size_t src_slot = SEL ? saved_slot(b, a.max_kept, saved, s_node < 0 ? 0 : s_node)
                                : (size_t)(lo + (s_node < 0 ? 0 : s_node));
    const float* __restrict__ src =
        s_node < 0 ? a.S0 + (size_t)bh * DV * DK : a.ckpt + (src_slot * H + h) * DV * DK;
    // DELTA: a leaf's state is never read again and is not stored
    const bool keep = SEL ? ((saved >> t) & 1ull) : (!DELTA || ((sHasChild >> t) & 1ull));
    float* __restrict__ dst =
        a.ckpt + ((SEL ? saved_slot(b, a.max_kept, saved, t) : (size_t)(lo + t)) * H + h) * DV * DK;
    if constexpr (DELTA) {
      if (ch == 0 && tid == 0) a.g2[gt] = sG2[t];
    }
    float4 C[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int row = ch * CR + ps * RPP + rin;
      C[ps] = *reinterpret_cast<const float4*>(src + (size_t)row * DK + c);
    }
    const float4 qq = io::load4(q + gt * DK + c);
    float coef[NPASS];
    while (steps) {   // root first: along a path, indices grow with depth
      const int j = __builtin_ctzll(steps);
      steps &= steps - 1ull;
      const size_t gj = (size_t)(lo + j) * H + h;
      const float4 kk = io::load4(k + gj * DK + c);
      const float al = a.alpha[gj];
      const float be = a.beta[gj];
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ch * CR + ps * RPP + rin;
        const float w =
            row_sum<TPR>(C[ps].x * kk.x + C[ps].y * kk.y + C[ps].z * kk.z + C[ps].w * kk.w);
        coef[ps] = be * (io::load1(v + gj * DV + row) - al * w);
        C[ps].x = al * C[ps].x + coef[ps] * kk.x;
        C[ps].y = al * C[ps].y + coef[ps] * kk.y;
        C[ps].z = al * C[ps].z + coef[ps] * kk.z;
        C[ps].w = al * C[ps].w + coef[ps] * kk.w;
      }
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int row = ch * CR + ps * RPP + rin;
      if (keep) *reinterpret_cast<float4*>(dst + (size_t)row * DK + c) = C[ps];
      const float ov =
          row_sum<TPR>(C[ps].x * qq.x + C[ps].y * qq.y + C[ps].z * qq.z + C[ps].w * qq.w);
      if (c == 0) io::store1(o + gt * DV + row, ov);
      if constexpr (DELTA) {
        if (c == 0) a.U[gt * DV + row] = coef[ps];
      }
    }
  }
}

// Commit after a selective-fork verify: the accepted node's state from its
// own slot when it is saved, else from its nearest saved ancestor (S0 when
// none) with the steps of the path nodes below it replayed. Same workgroup
// shape as the level kernel; in place (S_out == S0) is safe, every element
// being read and written by one thread.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void fork_selective_commit_kernel(const SelectiveCommitArgs a) {
  constexpr int TPR = DK / 4;
  constexpr int RPP = 256 / TPR;
  constexpr int CR = 32;
  constexpr int NCH = DV / CR;
  constexpr int NPASS = CR / RPP;
  using io = io_traits<IO>;

  __shared__ int sInfo[3];
  __shared__ uint64_t sPath, sSaved;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int bh = blockIdx.x / NCH;
  const int ch = blockIdx.x - bh * NCH;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  if (tid < 64) {
    const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
    int st = tl.status;
    if (st == GDN_TREE_OK) {
      int dmax = tl.depth;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off, kWave));
      if (dmax > a.max_depth) st = GDN_TREE_TOO_DEEP;
    }
    uint64_t saved = 0ull;
    if (st == GDN_TREE_OK) {
      saved = saved_nodes(a.conf, a.threshold, tl.lo, tl.n, lane);
      if (__popcll(saved) > a.max_kept) st = GDN_TREE_TOO_MANY_KEPT;
    }
    const int acc = a.accepted[b];
    if (st == GDN_TREE_OK && (acc < -1 || acc >= tl.n)) st = GDN_TREE_BAD_ACCEPTED;
    const uint64_t path = st == GDN_TREE_OK && acc >= 0 ? shfl_u64(tl.anc, acc) : 0ull;
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = acc;
      sInfo[2] = tl.lo;
      sPath = path;
      sSaved = saved;
      if (h == 0 && ch == 0) a.status[b] = st;
    }
  }
  __syncthreads();
  const int st = sInfo[0], acc = sInfo[1], lo = sInfo[2];
  if (st != GDN_TREE_OK) return;
  if (acc < 0 && a.S_out == a.S0) return;       // keep S0 in place: nothing to write
  const uint64_t path = sPath, saved = sSaved;
  const uint64_t up = path & saved;             // the accepted node itself included
  const int s_node = up ? 63 - __builtin_clzll(up) : -1;
  uint64_t steps = s_node < 0 ? path : path & ~((2ull << s_node) - 1ull);
  const float* __restrict__ src =
      s_node < 0 ? a.S0 + (size_t)bh * DV * DK
                 : a.ckpt + (saved_slot(b, a.max_kept, saved, s_node) * H + h) * DV * DK;
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  const IO* __restrict__ v = static_cast<const IO*>(a.v);
  const int rin = tid / TPR;
  const int c = 4 * (tid - rin * TPR);
  float4 C[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int row = ch * CR + ps * RPP + rin;
    C[ps] = *reinterpret_cast<const float4*>(src + (size_t)row * DK + c);
  }
  while (steps) {
    const int j = __builtin_ctzll(steps);
    steps &= steps - 1ull;
    const size_t gj = (size_t)(lo + j) * H + h;
    const float4 kk = io::load4(k + gj * DK + c);
    const float al = a.alpha[gj];
    const float be = a.beta[gj];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int row = ch * CR + ps * RPP + rin;
      const float w =
          row_sum<TPR>(C[ps].x * kk.x + C[ps].y * kk.y + C[ps].z * kk.z + C[ps].w * kk.w);
      const float cf = be * (io::load1(v + gj * DV + row) - al * w);
      C[ps].x = al * C[ps].x + cf * kk.x;
      C[ps].y = al * C[ps].y + cf * kk.y;
      C[ps].z = al * C[ps].z + cf * kk.z;
      C[ps].w = al * C[ps].w + cf * kk.w;
    }
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int row = ch * CR + ps * RPP + rin;
    *reinterpret_cast<float4*>(a.S_out + (size_t)bh * DV * DK + (size_t)row * DK + c) = C[ps];
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void fork_commit_kernel(const ForkCommitArgs a) {
  constexpr int CR0 = 4096 / DK;
  constexpr int CR = CR0 < DV ? CR0 : DV;
  constexpr int NCH = DV / CR;
  constexpr int F4 = CR * DK / 4;
  constexpr int NF = (F4 + 255) / 256;

  __shared__ int sInfo[3];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int bh = blockIdx.x / NCH;
  const int ch = blockIdx.x - bh * NCH;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  if (tid < 64) {
    const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
    int st = tl.status;
    if (st == GDN_TREE_OK) {
      int dmax = tl.depth;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off, kWave));
      if (dmax > a.max_depth) st = GDN_TREE_TOO_DEEP;
    }
    const int acc = a.accepted[b];
    if (st == GDN_TREE_OK && (acc < -1 || acc >= tl.n)) st = GDN_TREE_BAD_ACCEPTED;
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = acc;
      sInfo[2] = tl.lo;
      if (h == 0 && ch == 0) put_status(a.status, b, st, a.merge);
    }
  }
  __syncthreads();
  const int st = sInfo[0], acc = sInfo[1], lo = sInfo[2];
  if (st != GDN_TREE_OK) return;
  const size_t off = (size_t)bh * DV * DK + (size_t)ch * CR * DK;
  if (acc < 0 && a.S_out == a.S0) return;
  const float* __restrict__ src =
      acc < 0 ? a.S0 + off
              : a.ckpt + ((size_t)(lo + acc) * a.H + h) * DV * DK + (size_t)ch * CR * DK;
  float4 x[NF];
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = tid + 256 * it;
    if (f < F4) x[it] = *reinterpret_cast<const float4*>(src + 4 * (size_t)f);
  }
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = tid + 256 * it;
    if (f < F4) *reinterpret_cast<float4*>(a.S_out + off + 4 * (size_t)f) = x[it];
  }
}

template <class IO, int D, bool SEL>
hipError_t launch_level(const ForkArgs& a, hipStream_t s) {
  const void* kern =
      SEL  ? reinterpret_cast<const void*>(&fork_level_kernel<IO, D, D, false, true>)
      : a.U ? reinterpret_cast<const void*>(&fork_level_kernel<IO, D, D, true, false>)
            : reinterpret_cast<const void*>(&fork_level_kernel<IO, D, D, false, false>);
  return launch_kernel(kern, (unsigned)(a.B * a.H * (D / 32)), 256u, s, a);
}

template <class IO, bool SEL>
hipError_t launch_level_d(int d, const ForkArgs& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_level<IO, 32, SEL>(a, s);
    case 64: return launch_level<IO, 64, SEL>(a, s);
    case 128: return launch_level<IO, 128, SEL>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class IO, int D>
hipError_t launch_sel_commit(const SelectiveCommitArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&fork_selective_commit_kernel<IO, D, D>),
                       (unsigned)(a.B * a.H * (D / 32)), 256u, s, a);
}

template <class IO>
hipError_t launch_sel_commit_d(int d, const SelectiveCommitArgs& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_sel_commit<IO, 32>(a, s);
    case 64: return launch_sel_commit<IO, 64>(a, s);
    case 128: return launch_sel_commit<IO, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_commit(const ForkCommitArgs& a, hipStream_t s) {
  constexpr int CR0 = 4096 / D;
  constexpr int CR = CR0 < D ? CR0 : D;
  return launch_kernel(reinterpret_cast<const void*>(&fork_commit_kernel<D, D>),
                       (unsigned)(a.B * a.H * (D / CR)), 256u, s, a);
}

}  // namespace

hipError_t launch_fork_level(int io, int d, const ForkArgs& a, hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_level_d<uint16_t, false>(d, a, s)
                              : launch_level_d<float, false>(d, a, s);
}

hipError_t launch_fork_selective_level(int io, int d, const ForkArgs& a, hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_level_d<uint16_t, true>(d, a, s)
                              : launch_level_d<float, true>(d, a, s);
}

hipError_t launch_fork_selective_commit(int io, int d, const SelectiveCommitArgs& a,
                                        hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_sel_commit_d<uint16_t>(d, a, s)
                              : launch_sel_commit_d<float>(d, a, s);
}

hipError_t launch_fork_commit(int d, const ForkCommitArgs& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_commit<32>(a, s);
    case 64: return launch_commit<64>(a, s);
    case 128: return launch_commit<128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
