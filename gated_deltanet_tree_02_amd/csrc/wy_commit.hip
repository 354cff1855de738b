// wy_commit.hip -- rebuild the accepted node's state from pseudo-values.
//
// For the last accepted node a of sequence b (TreeWY abstract: only the one
// accepted state is reconstructed; fork page section 5: the kept state is the
// last accepted token's), head h:
//     S_out = G_a S0 + sum_{i in A(a)} (G_a / G_i) u_i k_i^T
// with G = 2^g2 from the verify workspace. accepted = -1 keeps S0.
//
// A streaming kernel: each workgroup owns a 16 KiB slab of one (b, h) state
// (CR rows x dk), puts all of it in flight at once with 16-byte loads, then
// applies the rank-|path| update from path data staged in LDS and writes the
// slab back with 16-byte stores. In-place (S_out == S0) is safe: every
// element is read and written by the same thread.
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void wy_commit_kernel(const CommitArgs a) {
  constexpr int CR0 = 4096 / DK;
  constexpr int CR = CR0 < DV ? CR0 : DV;   // state rows per workgroup
  constexpr int NCH = DV / CR;              // workgroups per (b, h)
  constexpr int F4 = CR * DK / 4;           // float4 per workgroup
  constexpr int NF = (F4 + 255) / 256;      // float4 per thread
  constexpr int PCH = 16;                   // path nodes staged per round
  using io = io_traits<IO>;

  __shared__ float sK[PCH * DK];
  __shared__ float sW[PCH * CR];
  __shared__ int sPath[64];
  __shared__ float sCoef[64];
  __shared__ int sInfo[4];
  __shared__ float sGA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int bh = blockIdx.x / NCH;
  const int ch = blockIdx.x - bh * NCH;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const size_t sbase = (size_t)bh * DV * DK + (size_t)ch * CR * DK;

  float4 s[NF];
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = tid + 256 * it;
    if (f < F4) s[it] = *reinterpret_cast<const float4*>(a.S0 + sbase + 4 * (size_t)f);
  }

  if (tid < 64) {
    const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
    int st = tl.status;
    const int acc = a.accepted[b];
    if (st == GDN_TREE_OK && (acc < -1 || acc >= tl.n)) st = GDN_TREE_BAD_ACCEPTED;
    int P = 0;
    float gA = 0.f;
    if (st == GDN_TREE_OK && acc >= 0) {
      const uint64_t path = shfl_u64(tl.anc, acc);
      gA = a.g2[(size_t)(tl.lo + acc) * H + h];
      if ((path >> lane) & 1ull) {
        const int rank = __popcll(path & ((1ull << lane) - 1ull));
        const float gi = a.g2[(size_t)(tl.lo + lane) * H + h];
        sPath[rank] = lane;
        sCoef[rank] = exp2f(gA - gi);
      }
      P = __popcll(path);
    }
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = acc;
      sInfo[2] = P;
      sInfo[3] = tl.lo;
      sGA = exp2f(gA);
      if (h == 0 && ch == 0) a.status[b] = st;
    }
  }
  __syncthreads();
  const int st = sInfo[0];
  const int acc = sInfo[1];
  const int P = sInfo[2];
  const int lo = sInfo[3];
  if (st != GDN_TREE_OK) return;
  float* __restrict__ dst = a.S_out + sbase;
  if (acc < 0) {
    if (a.S_out != a.S0) {
#pragma unroll
      for (int it = 0; it < NF; ++it) {
        const int f = tid + 256 * it;
        if (f < F4) *reinterpret_cast<float4*>(dst + 4 * (size_t)f) = s[it];
      }
    }
    return;
  }

  const float GA = sGA;
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    s[it].x *= GA;
    s[it].y *= GA;
    s[it].z *= GA;
    s[it].w *= GA;
  }
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  for (int p0 = 0; p0 < P; p0 += PCH) {
    const int pc = P - p0 < PCH ? P - p0 : PCH;
    for (int idx = tid; idx < pc * DK; idx += 256) {
      const int p = idx / DK;
      const int c = idx - p * DK;
      sK[idx] = io::load1(k + ((size_t)(lo + sPath[p0 + p]) * H + h) * DK + c);
    }
    for (int idx = tid; idx < pc * CR; idx += 256) {
      const int p = idx / CR;
      const int r = idx - p * CR;
      sW[idx] = sCoef[p0 + p] *
                a.U[((size_t)(lo + sPath[p0 + p]) * H + h) * DV + (size_t)ch * CR + r];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NF; ++it) {
      const int f = tid + 256 * it;
      if (f < F4) {
        const int row = f / (DK / 4);
        const int c = 4 * (f - row * (DK / 4));
        for (int p = 0; p < pc; ++p) {
          const float w = sW[p * CR + row];
          const float4 kk = *reinterpret_cast<const float4*>(sK + p * DK + c);
          s[it].x += w * kk.x;
          s[it].y += w * kk.y;
          s[it].z += w * kk.z;
          s[it].w += w * kk.w;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = tid + 256 * it;
    if (f < F4) *reinterpret_cast<float4*>(dst + 4 * (size_t)f) = s[it];
  }
}

template <class IO, int D>
hipError_t launch_t(const CommitArgs& a, hipStream_t s) {
  constexpr int CR0 = 4096 / D;
  constexpr int CR = CR0 < D ? CR0 : D;
  return launch_kernel(reinterpret_cast<const void*>(&wy_commit_kernel<IO, D, D>),
                       (unsigned)(a.B * a.H * (D / CR)), 256u, s, a);
}

template <class IO>
hipError_t launch_d(int d, const CommitArgs& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_t<IO, 32>(a, s);
    case 64: return launch_t<IO, 64>(a, s);
    case 128: return launch_t<IO, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_wy_commit(int io, int d, const CommitArgs& a, hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t>(d, a, s) : launch_d<float>(d, a, s);
}

}  // namespace gdn
