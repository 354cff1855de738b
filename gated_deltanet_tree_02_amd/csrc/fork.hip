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

template <class IO, int DK, int DV, bool DELTA>
__global__ __launch_bounds__(256) void fork_level_kernel(const ForkArgs a) {
  constexpr int TPR = DK / 4;        // threads per state row (one float4 each)
  constexpr int RPP = 256 / TPR;     // rows per pass
  constexpr int CR = 32;             // rows per workgroup
  constexpr int NCH = DV / CR;
  constexpr int NPASS = CR / RPP;
  using io = io_traits<IO>;

  __shared__ int sPar[64];
  __shared__ int sInfo[3];
  __shared__ uint64_t sLevel;
  __shared__ uint64_t sHasChild;   // DELTA: nodes whose state a child reads
  __shared__ float sG2[64];        // DELTA: base-2 gate prefixes

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
  uint64_t msk = sLevel;
  while (msk) {
    const int t = __builtin_ctzll(msk);
    msk &= msk - 1;
    const int p = sPar[t];
    const size_t gt = (size_t)(lo + t) * H + h;
    const float* __restrict__ src =
        p < 0 ? a.S0 + (size_t)bh * DV * DK : a.ckpt + ((size_t)(lo + p) * H + h) * DV * DK;
    float* __restrict__ dst = a.ckpt + gt * DV * DK;
    // DELTA: a leaf's state is never read again and is not stored
    const bool keep = !DELTA || ((sHasChild >> t) & 1ull);
    if constexpr (DELTA) {
      if (ch == 0 && tid == 0) a.g2[gt] = sG2[t];
    }
    float4 C[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int row = ch * CR + ps * RPP + rin;
      C[ps] = *reinterpret_cast<const float4*>(src + (size_t)row * DK + c);
    }
    const float4 kk = io::load4(k + gt * DK + c);
    const float4 qq = io::load4(q + gt * DK + c);
    const float al = a.alpha[gt];
    const float be = a.beta[gt];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int row = ch * CR + ps * RPP + rin;
      const float w = row_sum<TPR>(C[ps].x * kk.x + C[ps].y * kk.y + C[ps].z * kk.z + C[ps].w * kk.w);
      const float coef = be * (io::load1(v + gt * DV + row) - al * w);
      float4 Ct;
      Ct.x = al * C[ps].x + coef * kk.x;
      Ct.y = al * C[ps].y + coef * kk.y;
      Ct.z = al * C[ps].z + coef * kk.z;
      Ct.w = al * C[ps].w + coef * kk.w;
      if (keep) *reinterpret_cast<float4*>(dst + (size_t)row * DK + c) = Ct;
      const float ov = row_sum<TPR>(Ct.x * qq.x + Ct.y * qq.y + Ct.z * qq.z + Ct.w * qq.w);
      if (c == 0) io::store1(o + gt * DV + row, ov);
      if constexpr (DELTA) {
        if (c == 0) a.U[gt * DV + row] = coef;
      }
    }
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

template <class IO, int D>
hipError_t launch_level(const ForkArgs& a, hipStream_t s) {
  const void* kern = a.U ? reinterpret_cast<const void*>(&fork_level_kernel<IO, D, D, true>)
                         : reinterpret_cast<const void*>(&fork_level_kernel<IO, D, D, false>);
  return launch_kernel(kern, (unsigned)(a.B * a.H * (D / 32)), 256u, s, a);
}

template <class IO>
hipError_t launch_level_d(int d, const ForkArgs& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_level<IO, 32>(a, s);
    case 64: return launch_level<IO, 64>(a, s);
    case 128: return launch_level<IO, 128>(a, s);
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
  return io == GDN_DTYPE_BF16 ? launch_level_d<uint16_t>(d, a, s) : launch_level_d<float>(d, a, s);
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
