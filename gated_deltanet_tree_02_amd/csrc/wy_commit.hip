// wy_commit.hip -- rebuild the accepted node's state from pseudo-values.
//
// For the last accepted node a of sequence b (TreeWY abstract: only the one
// accepted state is reconstructed; fork page section 5: the kept state is the
// last accepted token's), head h:
//     S_out = G_a S0 + sum_{i in A(a)} (G_a / G_i) u_i k_i^T
// with G = 2^g2 from the verify workspace. accepted = -1 keeps S0.
//
// A streaming kernel with one workgroup (256 threads) per (b, h): every
// thread puts its 16-byte pieces of the state in flight first (each load
// instruction of the workgroup covers one contiguous stretch of rows), while
// wave 0 reads the sequence's parents, all of its nodes' gate prefixes and the
// accepted node in one round and forms the path coefficients without a
// further load; the path's k rows and pseudo-values follow in one more round.
// The rank-|path| update runs in registers and the state goes back with
// 16-byte stores. In-place (S_out == S0) is safe: every element is read and
// written by the same thread.
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kCommitThreads = 256;

template <class IO, int DK, int DV>
__global__ __launch_bounds__(kCommitThreads) void wy_commit_kernel(const CommitArgs a) {
  constexpr int NT = kCommitThreads;
  constexpr int CPROW = DK / 4;             // float4 per state row
  constexpr int F4 = DV * DK / 4;           // float4 per (b, h) state
  constexpr int NF = F4 / NT;               // float4 per thread
  constexpr int RSTEP = NT / CPROW;         // rows between a thread's pieces
  constexpr int PCH = 16;                   // path nodes staged per round
  constexpr int EPC = 16 / (int)sizeof(IO); // io elements per 16-byte chunk
  static_assert(F4 % NT == 0 && NT % CPROW == 0, "state tiles the workgroup");
  using io = io_traits<IO>;

  __shared__ __align__(16) float sK[PCH * DK];
  __shared__ __align__(16) float sW[PCH * DV];
  __shared__ int sPath[64];
  __shared__ float sCoef[64];
  __shared__ int sInfo[4];
  __shared__ float sGA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const size_t sbase = (size_t)bh * DV * DK;
  const int c4 = tid % CPROW;               // this thread's float4 column
  const int row0 = tid / CPROW;             // its rows: row0 + RSTEP * i

  float4 s[NF];
  const float* __restrict__ src0 = a.S0 + sbase;
#pragma unroll
  for (int i = 0; i < NF; ++i) s[i] = *reinterpret_cast<const float4*>(src0 + 4 * (tid + NT * i));

  if (tid < 64) {
    // node range, then parents, gate prefixes and the accepted node together
    const int lo = a.offsets[b];
    const int hi = a.offsets[b + 1];
    const int n = hi - lo;
    int st = GDN_TREE_OK;
    int acc = -1, P = 0;
    float gA = 0.f;
    if (lo < 0 || hi > a.T || n < 1 || n > a.max_nodes) {
      st = GDN_TREE_BAD_SIZE;
    } else {
      const int nl = lane < n ? lane : 0;
      const int par_raw = a.parents[lo + nl];
      const float g2_raw = a.g2[(size_t)(lo + nl) * H + h];
      acc = a.accepted[b];
      const int par = lane < n ? par_raw : -1;
      if (__shfl(par, 0, kWave) != -1)
        st = GDN_TREE_BAD_ROOT;
      else if (__ballot(lane >= 1 && lane < n && (par < 0 || par >= lane)) != 0ull)
        st = GDN_TREE_BAD_PARENT;
      else if (acc < -1 || acc >= n)
        st = GDN_TREE_BAD_ACCEPTED;
      if (st == GDN_TREE_OK && acc >= 0) {
        uint64_t anc;
        float unused;
        path_scan(par, lane, n, 0.f, anc, unused);
        const uint64_t path = shfl_u64(anc, acc);
        gA = __shfl(g2_raw, acc, kWave);
        if ((path >> lane) & 1ull) {
          const int rank = __popcll(path & ((1ull << lane) - 1ull));
          sPath[rank] = lane;
          sCoef[rank] = exp2f(gA - g2_raw);
        }
        P = __popcll(path);
      }
    }
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = acc;
      sInfo[2] = P;
      sInfo[3] = lo;
      sGA = exp2f(gA);
      if (h == 0) a.status[b] = st;
    }
  }
  __syncthreads();
  const int st = sInfo[0];
  const int acc = sInfo[1];
  const int P = sInfo[2];
  const int lo = sInfo[3];
  if (st != GDN_TREE_OK) return;
  if (acc < 0 && a.S_out == a.S0) return;   // keep S0, in place: nothing to write
  float* __restrict__ dst = a.S_out + sbase;
  // accepted = -1 copies S0: factor 1 (exact) and an empty path (P = 0), so
  // both cases share one register set
  const float GA = acc < 0 ? 1.f : sGA;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    s[i].x *= GA;
    s[i].y *= GA;
    s[i].z *= GA;
    s[i].w *= GA;
  }
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  for (int p0 = 0; p0 < P; p0 += PCH) {
    const int pc = P - p0 < PCH ? P - p0 : PCH;
    // k rows of the chunk's path nodes, 16-byte pieces, widened to fp32
    for (int idx = tid; idx < pc * (DK / EPC); idx += NT) {
      const int p = idx / (DK / EPC);
      const int c = idx - p * (DK / EPC);
      const IO* src = k + ((size_t)(lo + sPath[p0 + p]) * H + h) * DK + c * EPC;
      float* d = sK + p * DK + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) *reinterpret_cast<float4*>(d + e) = io::load4(src + e);
    }
    // coefficient-scaled pseudo-values of the chunk, 16-byte pieces
    for (int idx = tid; idx < pc * (DV / 4); idx += NT) {
      const int p = idx / (DV / 4);
      const int r = 4 * (idx - p * (DV / 4));
      const float cf = sCoef[p0 + p];
      float4 u = *reinterpret_cast<const float4*>(
          a.U + ((size_t)(lo + sPath[p0 + p]) * H + h) * DV + r);
      u.x *= cf;
      u.y *= cf;
      u.z *= cf;
      u.w *= cf;
      *reinterpret_cast<float4*>(sW + p * DV + r) = u;
    }
    __syncthreads();
    for (int p = 0; p < pc; ++p) {
      const float4 kk = *reinterpret_cast<const float4*>(sK + p * DK + 4 * c4);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const float w = sW[p * DV + row0 + RSTEP * i];
        s[i].x += w * kk.x;
        s[i].y += w * kk.y;
        s[i].z += w * kk.z;
        s[i].w += w * kk.w;
      }
    }
    __syncthreads();
  }
  // (the store addresses are recomputed from an opaque copy of the thread
  // index instead of being held in registers since the loads)
  int t2 = tid;
  asm volatile("" : "+v"(t2));
#pragma unroll
  for (int i = 0; i < NF; ++i)
    *reinterpret_cast<float4*>(dst + 4 * (t2 + NT * i)) = s[i];
}

template <class IO, int D>
hipError_t launch_t(const CommitArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&wy_commit_kernel<IO, D, D>),
                       (unsigned)(a.B * a.H), (unsigned)kCommitThreads, s, a);
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
