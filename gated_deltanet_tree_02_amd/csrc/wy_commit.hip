// wy_commit.hip -- rebuild the accepted node's state from pseudo-values.
//
// For the last accepted node a of sequence b (TreeWY abstract: only the one
// accepted state is reconstructed; fork page section 5: the kept state is the
// last accepted token's), head h:
//     S_out = G_a S0 + sum_{i in A(a)} (G_a / G_i) u_i k_i^T
// with G = 2^g2 from the verify workspace. accepted = -1 keeps S0.
//
// A streaming kernel with one workgroup (four waves) per (b, h). Each thread
// holds 16 float4 of the 64 KiB state, rows interleaved so that each load
// instruction of the workgroup covers one contiguous stretch of rows. Waves
// 1-3 put their state in flight at once. Wave 0 first reads the sequence's
// parents, all of its nodes' gate prefixes and the accepted node in one round,
// forms the path coefficients and stages the path's k rows and scaled
// pseudo-values in LDS. With kPathFirst it issues its own state loads only
// after that, so that no wave's wait for path data also waits for state:
// because loads complete in order per wave, every wave then takes its state
// in four pieces as they land, applying the rank-|path| update to each and
// storing it while the later pieces are still in flight, and the writes
// overlap the reads. That pays when every workgroup of the launch is resident
// at once; when workgroups run in several generations, wave 0 loads its state
// first and each workgroup takes its whole state as one piece
// (kPathFirst = false), which keeps workgroups short and their reads and
// writes in long runs. In-place
// (S_out == S0) is safe: every element is read and written by the same thread.
//
// The same kernel commits by replay (kReplay) when verify kept no
// pseudo-values: the gated delta rule is run along the accepted path, root
// first, on every state row the thread holds,
//     w = S_r . k_j,   S_r <- alpha_j S_r + beta_j (v_j[r] - alpha_j w) k_j^T,
// from the path's own k, v, alpha and beta (fork page, section 5: the kept
// state is the last accepted token's). A row is spread over DK/4 consecutive
// lanes, so its dot product is a butterfly over those lanes.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kCommitThreads = 256;

// Args: CommitArgs (one layer) or CommitLayersArgs (workgroup i takes layer
// i / (B * H) of a layer-batched launch).
template <class IO, int DK, int DV, bool kPathFirst, bool kReplay, class Args>
__global__ __launch_bounds__(kCommitThreads) void wy_commit_kernel(const Args args) {
  constexpr int NT = kCommitThreads;
  constexpr int CPROW = DK / 4;             // float4 per state row
  constexpr int F4 = DV * DK / 4;           // float4 per (b, h) state
  constexpr int NF = F4 / NT;               // float4 per state thread
  // pieces the state is taken in: four when the launch is resident at once,
  // else one (all reads, then all writes, per workgroup)
  constexpr int NPC = kPathFirst ? (NF >= 4 ? 4 : NF) : 1;
  constexpr int FPC = NF / NPC;             // float4 per piece
  constexpr int RSTEP = NT / CPROW;         // rows between a thread's float4s
  constexpr int PCH = 16;                   // path nodes staged per round
  constexpr int EPC = 16 / (int)sizeof(IO); // io elements per 16-byte chunk
  static_assert(F4 % NT == 0 && NT % CPROW == 0 && NF % NPC == 0, "state tiles the waves");
  using io = io_traits<IO>;

  __shared__ __align__(16) float sK[PCH * DK];
  // scaled pseudo-values, or (replay) the path's v rows
  __shared__ __align__(16) float sW[PCH * DV];
  __shared__ int sPath[64];
  __shared__ float sCoef[64];     // path coefficients, or (replay) alpha
  __shared__ float sBeta[kReplay ? 64 : 1];
  __shared__ int sInfo[4];
  __shared__ float sGA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool path_wave = tid < kWave;       // wave 0 (wave-uniform)
  const int nbh = base_args(args).B * base_args(args).H;
  const int layer = blockIdx.x / nbh;
  const CommitArgs a = layer_args(args, layer);
  const int bh = blockIdx.x - layer * nbh;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const size_t sbase = (size_t)bh * DV * DK;
  const IO* __restrict__ k = static_cast<const IO*>(a.k);

  // threads [0, nthr) stage path rows [p0, p0 + pc) of the path in sK / sW
  auto stage_path_rows = [&](int lo, int p0, int pc, int t, int nthr) {
    for (int idx = t; idx < pc * (DK / EPC); idx += nthr) {
      const int p = idx / (DK / EPC);
      const int c = idx - p * (DK / EPC);
      const IO* src = k + ((size_t)(lo + sPath[p0 + p]) * H + h) * DK + c * EPC;
      float* d = sK + p * DK + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) *reinterpret_cast<float4*>(d + e) = io::load4(src + e);
    }
    for (int idx = t; idx < pc * (DV / 4); idx += nthr) {
      const int p = idx / (DV / 4);
      const int r = 4 * (idx - p * (DV / 4));
      const size_t row = ((size_t)(lo + sPath[p0 + p]) * H + h) * DV + r;
      if constexpr (kReplay) {
        *reinterpret_cast<float4*>(sW + p * DV + r) = io::load4(static_cast<const IO*>(a.v) + row);
      } else {
        const float cf = sCoef[p0 + p];
        float4 u = *reinterpret_cast<const float4*>(a.U + row);
        u.x *= cf;
        u.y *= cf;
        u.z *= cf;
        u.w *= cf;
        *reinterpret_cast<float4*>(sW + p * DV + r) = u;
      }
    }
  };

  float4 s[NF];
  auto load_state = [&]() {
    const float* __restrict__ src0 = a.S0 + sbase;
#pragma unroll
    for (int i = 0; i < NF; ++i) s[i] = *reinterpret_cast<const float4*>(src0 + 4 * (tid + NT * i));
  };
  if (!path_wave || !kPathFirst) {
    load_state();
  }
  if (path_wave) {
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
      // the gate prefix (pseudo-values), or (replay) the node's gates
      const float g2_raw = kReplay ? a.alpha[(size_t)(lo + nl) * H + h]
                                   : a.g2[(size_t)(lo + nl) * H + h];
      const float beta_raw = kReplay ? a.beta[(size_t)(lo + nl) * H + h] : 0.f;
      acc = a.accepted[b];
      const int par = lane < n ? par_raw : -1;
      if (__shfl(par, 0, kWave) != -1)
        st = GDN_TREE_BAD_ROOT;
      else if (__ballot(lane >= 1 && lane < n && (par < 0 || par >= lane)) != 0ull)
        st = GDN_TREE_BAD_PARENT;
      if (st == GDN_TREE_OK && a.max_depth >= 0) {
        // the depth limit of the level-by-level verify that wrote the workspace
        uint64_t anc0;
        float unused0;
        path_scan(par, lane, n, 0.f, anc0, unused0);
        int dep = lane < n ? __popcll(anc0) - 1 : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dep = max(dep, __shfl_xor(dep, off, kWave));
        if (dep > a.max_depth) st = GDN_TREE_TOO_DEEP;
      }
      if (st == GDN_TREE_OK && (acc < -1 || acc >= n)) st = GDN_TREE_BAD_ACCEPTED;
      if (st == GDN_TREE_OK && acc >= 0) {
        uint64_t anc;
        float unused;
        path_scan(par, lane, n, 0.f, anc, unused);
        const uint64_t path = shfl_u64(anc, acc);
        if (!kReplay) gA = __shfl(g2_raw, acc, kWave);
        if ((path >> lane) & 1ull) {
          const int rank = __popcll(path & ((1ull << lane) - 1ull));
          sPath[rank] = lane;
          if constexpr (kReplay) {
            sCoef[rank] = g2_raw;
            sBeta[rank] = beta_raw;
          } else {
            sCoef[rank] = exp2f(gA - g2_raw);
          }
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
      if (h == 0) put_status(a.status, b, st, a.merge);
    }
    wave_lds_sync();   // sPath / sCoef written by other lanes of this wave
    if (kPathFirst && st == GDN_TREE_OK && P > 0) stage_path_rows(lo, 0, P < PCH ? P : PCH, lane, kWave);
    // the staged rows are complete (their loads were waited for) before this
    // wave's state loads go out
    if constexpr (kPathFirst) load_state();
  }
  __syncthreads();
  const int st = sInfo[0];
  const int acc = sInfo[1];
  const int P = sInfo[2];
  const int lo = sInfo[3];
  if (st != GDN_TREE_OK) return;
  if (acc < 0 && a.S_out == a.S0) return;   // keep S0, in place: nothing to write
  float* __restrict__ dst = a.S_out + sbase;
  // accepted = -1 copies S0: factor 1 (exact) and an empty path (P = 0)
  const float GA = (acc < 0 || kReplay) ? 1.f : sGA;
  if constexpr (!kPathFirst) {
    // the whole workgroup stages the first round of path rows
    if (P > 0) stage_path_rows(lo, 0, P < PCH ? P : PCH, tid, NT);
    __syncthreads();
  }
  // per-lane offsets are taken from an opaque copy of the thread index, so
  // that they are recomputed here rather than held since the loads
  int t2 = tid;
  asm volatile("" : "+v"(t2));
  const int c4 = t2 % CPROW;                // this thread's float4 column
  const int row0 = t2 / CPROW;              // its rows: row0 + RSTEP * i

  // Each piece of the state is scaled, updated with every path row and stored
  // as soon as it has landed. Paths longer than PCH nodes (rare: deep chains)
  // walk the path in rounds per piece, the path wave re-staging each round.
#pragma unroll
  for (int pcx = 0; pcx < NPC; ++pcx) {
#pragma unroll
    for (int j = 0; j < FPC; ++j) {
      const int i = pcx * FPC + j;
      s[i].x *= GA;
      s[i].y *= GA;
      s[i].z *= GA;
      s[i].w *= GA;
    }
    for (int p0 = 0; p0 < P; p0 += PCH) {
      const int pc = P - p0 < PCH ? P - p0 : PCH;
      if (P > PCH) {
        __syncthreads();   // the rows of the previous round are consumed
        if (path_wave) stage_path_rows(lo, p0, pc, lane, kWave);
        __syncthreads();
      }
      if constexpr (kReplay) {
        for (int p = 0; p < pc; ++p) {
          const float4 kk = *reinterpret_cast<const float4*>(sK + p * DK + 4 * c4);
          const float al = sCoef[p0 + p];
          const float be = sBeta[p0 + p];
#pragma unroll
          for (int j = 0; j < FPC; ++j) {
            const int i = pcx * FPC + j;
            float w = s[i].x * kk.x + s[i].y * kk.y + s[i].z * kk.z + s[i].w * kk.w;
            // the row's DK/4 lanes are consecutive: a butterfly over them
#pragma unroll
            for (int off = CPROW / 2; off > 0; off >>= 1) w += __shfl_xor(w, off, kWave);
            const float cf = be * (sW[p * DV + row0 + RSTEP * i] - al * w);
            s[i].x = al * s[i].x + cf * kk.x;
            s[i].y = al * s[i].y + cf * kk.y;
            s[i].z = al * s[i].z + cf * kk.z;
            s[i].w = al * s[i].w + cf * kk.w;
          }
        }
      } else {
        for (int p = 0; p < pc; ++p) {
          const float4 kk = *reinterpret_cast<const float4*>(sK + p * DK + 4 * c4);
#pragma unroll
          for (int j = 0; j < FPC; ++j) {
            const int i = pcx * FPC + j;
            const float w = sW[p * DV + row0 + RSTEP * i];
            s[i].x += w * kk.x;
            s[i].y += w * kk.y;
            s[i].z += w * kk.z;
            s[i].w += w * kk.w;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < FPC; ++j) {
      const int i = pcx * FPC + j;
      *reinterpret_cast<float4*>(dst + 4 * (t2 + NT * i)) = s[i];
    }
  }
}

// Workgroups of `kernel` the current device holds at once (occupancy per CU
// times the CU count), cached per kernel and device.
hipError_t resident_workgroups(const void* kernel, int block, int* out) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kernel, dev);
  auto f = cache.find(key);
  if (f == cache.end()) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
    if (e != hipSuccess) return e;
    f = cache.emplace(key, std::max(1, per_cu) * std::max(1, cus)).first;
  }
  *out = f->second;
  return hipSuccess;
}

inline int grid_of(const CommitArgs& a) { return a.B * a.H; }
inline int grid_of(const CommitLayersArgs& a) { return a.base.B * a.base.H * a.layers; }

template <class IO, int D, bool kReplay, class Args>
hipError_t launch_t(const Args& a, hipStream_t s) {
  const void* first =
      reinterpret_cast<const void*>(&wy_commit_kernel<IO, D, D, true, kReplay, Args>);
  const void* state_first =
      reinterpret_cast<const void*>(&wy_commit_kernel<IO, D, D, false, kReplay, Args>);
  int slots = 0;
  const hipError_t e = resident_workgroups(first, kCommitThreads, &slots);
  if (e != hipSuccess) return e;
  const int grid = grid_of(a);
  return launch_kernel(grid <= slots ? first : state_first, (unsigned)grid,
                       (unsigned)kCommitThreads, s, a);
}

template <class IO, bool kReplay, class Args>
hipError_t launch_d(int d, const Args& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_t<IO, 32, kReplay>(a, s);
    case 64: return launch_t<IO, 64, kReplay>(a, s);
    case 128: return launch_t<IO, 128, kReplay>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool kReplay, class Args>
hipError_t launch_io(int io, int d, const Args& a, hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t, kReplay>(d, a, s)
                              : launch_d<float, kReplay>(d, a, s);
}

}  // namespace

hipError_t launch_wy_commit(int io, int d, const CommitArgs& a, hipStream_t s) {
  return launch_io<false>(io, d, a, s);
}

hipError_t launch_wy_commit_layers(int io, int d, const CommitLayersArgs& a, hipStream_t s) {
  return launch_io<false>(io, d, a, s);
}

hipError_t launch_replay_commit(int io, int d, const CommitArgs& a, hipStream_t s) {
  return launch_io<true>(io, d, a, s);
}

hipError_t launch_replay_commit_layers(int io, int d, const CommitLayersArgs& a, hipStream_t s) {
  return launch_io<true>(io, d, a, s);
}

}  // namespace gdn
