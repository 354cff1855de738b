// tree_attn.hip -- tree-masked attention verify and the accepted-path KV
// commit for the full-attention layers of a hybrid model (gfx950).
//
// Node t of sequence b, query head h (K/V head j = h / G, G = Hq / Hkv) sees
// the committed cache rows 0 .. L_b - 1 and the tree nodes on its own root
// path (anrans handbook "speculative", implementation section: the cached
// prefix is visible to every new token, the tree mask decides among the new
// tokens, query heads share K/V heads in groups):
//     o[t,h] = softmax_x(scale <q[t,h], key_x>) . value_x .
//
// Verify kernel. One workgroup (16 waves) per (sequence, K/V head, split of
// the cache). The G * N_b query rows that share the K/V head (<= 256) are
// 16-row tiles, one per wave. Keys stream through LDS in blocks of 64: the
// cache rows of the split, then (in the last split) the 64 tree slots, masked
// per query row by the node's ancestor bits. Per block a wave computes the
// transposed scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = staged K
// rows, B = the wave's query rows held in registers), so that a lane owns one
// query row: the online softmax (running max and sum, base-2 exponentials)
// needs only two cross-lane shuffles, and the probabilities come out in the
// B-operand layout of v_mfma_f32_16x16x16_bf16, which accumulates
// O^T += V^T P^T with V staged transposed. Two blocks of K/V are in flight in
// registers while one is computed. A split's unnormalised output, running max
// and sum go to the workspace when the cache is split over several
// workgroups, and a combine kernel merges them.
//
// Commit kernel. One workgroup per sequence copies the K/V rows of the
// accepted path, root first, behind the sequence's committed rows and
// advances its length (handbook, same section: the accepted path's K/V rows
// were computed at the right positions during verification and are appended
// as they are; rainlin-top "Qwen3.5 tree spec", section 7 step 4).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "gdn_tree_attn.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kAttnThreads = 1024;   // 16 waves, one 16-row query tile each
constexpr int KB = 64;               // keys per staged block
constexpr int PF = 2;                // key blocks in flight in registers
constexpr float kMasked = -1.0e30f;  // score of an invisible key (base-2 domain)

__device__ __forceinline__ f32x4 mfma_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void tree_attn_kernel(const AttnArgs a) {
  constexpr int KSD = D / 32;                 // 16x16x32 steps over d
  constexpr int DT = D / 16;                  // 16-row tiles of O^T (over d)
  constexpr int KP = D + 8;                   // staged K row, 16 spare bytes (bank spread)
  constexpr int VP = KB + 8;                  // staged V^T row (keys), 16 spare bytes
  constexpr int CPB = KB * D / 8;             // 16-byte chunks of K (and of V) per block
  constexpr int CPT = 2 * CPB / kAttnThreads; // chunks per thread per block
  static_assert(2 * CPB % kAttnThreads == 0, "every thread stages whole chunks");

  __shared__ __align__(16) uint16_t sK[KB * KP];
  __shared__ __align__(16) uint16_t sVt[D * VP];
  __shared__ uint64_t sAnc[64];
  __shared__ int sStatus;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int NS = a.NS;
  const int split = blockIdx.x % NS;
  const int bkv = blockIdx.x / NS;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int G = a.Hq / a.Hkv;

  // ---- sequence checks and ancestor masks (wave 0)
  const int lo = a.offsets[b];
  const int hi = a.offsets[b + 1];
  const int n = hi - lo;
  const int L = a.cache_len[b];
  const bool range_ok = lo >= 0 && hi <= a.T && n >= 1 && n <= a.max_nodes;
  if (wave == 0) {
    int st = GDN_TREE_OK;
    uint64_t anc = 0;
    if (!range_ok || L < 0 || L > a.max_len) {
      st = GDN_TREE_BAD_SIZE;
    } else {
      const int par_raw = a.parents[lo + (lane < n ? lane : 0)];
      const int par = lane < n ? par_raw : -1;
      if (__shfl(par, 0, kWave) != -1)
        st = GDN_TREE_BAD_ROOT;
      else if (__ballot(lane >= 1 && lane < n && (par < 0 || par >= lane)) != 0ull)
        st = GDN_TREE_BAD_PARENT;
      float unused;
      path_scan(par, lane, n, 0.f, anc, unused);
    }
    sAnc[lane] = anc;
    if (lane == 0) sStatus = st;
  }
  __syncthreads();
  const int st = __builtin_amdgcn_readfirstlane(sStatus);
  if (split == 0 && kvh == 0 && tid == 0) a.status[b] = st;

  // ---- this lane's query row: the transposed score / output column
  const int R = range_ok ? G * n : 0;
  const int r = 16 * wave + l16;
  const bool rv = r < R;
  const int hg = rv ? r / n : 0;
  const int t = rv ? r - hg * n : 0;
  const int h = kvh * G + hg;
  const size_t orow = ((size_t)(lo + t) * a.Hq + h);   // row of o / the partials

  if (st != GDN_TREE_OK) {
    // rows of a rejected sequence (with a valid node range) are zero
    if (rv) {
      if (NS == 1) {
        for (int c = 4 * g; c < D; c += 16)
          *reinterpret_cast<uint2*>(a.o + orow * D + c) = make_uint2(0u, 0u);
      } else {
        for (int c = 4 * g; c < D; c += 16)
          *reinterpret_cast<float4*>(a.part_o + (orow * NS + split) * D + c) =
              make_float4(0.f, 0.f, 0.f, 0.f);
        if (g == 0) *reinterpret_cast<float2*>(a.part_ml + (orow * NS + split) * 2) =
            make_float2(kMasked, 0.f);
      }
    }
    return;
  }

  // ---- key range of this split: cache rows [c0, c1), then the tree slots
  // (last split only)
  const int c0 = min(split * a.CL, L);
  const int c1 = min(c0 + a.CL, L);
  const int ncb = (c1 - c0 + KB - 1) / KB;
  const int nblk = ncb + (split == NS - 1 ? 1 : 0);

  const size_t kvbase = ((size_t)b * a.Hkv + kvh) * a.cap;   // cache row 0 of (b, kvh)
  // The chunks this thread stages per block: chunk id = tid + 1024 i; ids
  // below CPB are K chunks, the rest V chunks; within a matrix, consecutive
  // ids walk the 64 keys first, so a wave stages one 16-byte column of 64 rows.
  // Keys that are masked (past the split's cache rows, or unused tree slots)
  // read a valid row instead: finite values whose weight is exactly zero.
  auto issue_block = [&](int j, u32x4 (&reg)[CPT]) {
    const bool tree = j >= ncb;
    const int p0 = c0 + j * KB;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int id = tid + kAttnThreads * i;
      const int mat = id >= CPB ? 1 : 0;
      const int rem = id - mat * CPB;
      const int kk = rem % KB;
      const int c = rem / KB;
      const uint16_t* base;
      if (!tree) {
        const int p = min(p0 + kk, c1 - 1);
        base = (mat ? a.vc : a.kc) + (kvbase + p) * D;
      } else {
        const int node = kk < n ? kk : 0;
        base = (mat ? a.v : a.k) + ((size_t)(lo + node) * a.Hkv + kvh) * D;
      }
      reg[i] = *reinterpret_cast<const u32x4*>(base + 8 * c);
    }
  };
  auto stage_block = [&](const u32x4 (&reg)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int id = tid + kAttnThreads * i;
      const int mat = id >= CPB ? 1 : 0;
      const int rem = id - mat * CPB;
      const int kk = rem % KB;
      const int c = rem / KB;
      if (mat == 0) {
        *reinterpret_cast<u32x4*>(sK + kk * KP + 8 * c) = reg[i];
      } else {
        const uint32_t w[4] = {reg[i][0], reg[i][1], reg[i][2], reg[i][3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sVt[(8 * c + 2 * e) * VP + kk] = (uint16_t)(w[e] & 0xffffu);
          sVt[(8 * c + 2 * e + 1) * VP + kk] = (uint16_t)(w[e] >> 16);
        }
      }
    }
  };

  // query fragments: B operand of S^T = K Q^T (lane: column = query row,
  // k = d 32s + 8g .. +7); issued before the key blocks
  bf16x8 qf[KSD];
  {
    const uint16_t* qrow = a.q + orow * D;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const uint4 u = rv ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g)
                         : make_uint4(0u, 0u, 0u, 0u);
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // two blocks in flight: ring0 holds even blocks, ring1 odd ones; a block
  // past the last is re-issued as the last (never computed), so every step
  // issues the same loads and the waits for in-flight blocks stay exact
  u32x4 ring0[CPT], ring1[CPT];
  if (nblk > 0) {
    issue_block(0, ring0);
    issue_block(min(1, nblk - 1), ring1);
  }
  const uint64_t anc_t = sAnc[t];
  const bool active = 16 * wave < R;          // wave-uniform: the tile holds query rows

  float m = kMasked;                          // running max (base-2 domain)
  float lsum = 0.f;                           // this lane's part of the running sum
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int j, u32x4 (&reg)[CPT]) {
    __syncthreads();                          // the previous block is consumed
    stage_block(reg);
    issue_block(min(j + PF, nblk - 1), reg);
    __syncthreads();
    if (!active || j >= nblk) return;
    const bool tree = j >= ncb;
    const int p0 = c0 + j * KB;
    // S^T tiles: lane holds query row l16 and keys 16 kt + 4g + e
    float x[4][4];
    float mb = kMasked;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(sK + (16 * kt + l16) * KP + 32 * s + 8 * g));
        acc = mfma_k32(ka, qf[s], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 16 * kt + 4 * g + e;
        const bool vis = rv && (tree ? ((anc_t >> kk) & 1ull) != 0 : p0 + kk < c1);
        x[kt][e] = vis ? acc[e] * a.scale_log2 : kMasked;
        mb = fmaxf(mb, x[kt][e]);
      }
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
    mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
    const float m_new = fmaxf(m, mb);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      oacc[dt][0] *= alpha;
      oacc[dt][1] *= alpha;
      oacc[dt][2] *= alpha;
      oacc[dt][3] *= alpha;
    }
    bf16x4 pk[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = x[kt][e] > 0.5f * kMasked ? exp2f(x[kt][e] - m_new) : 0.f;
        lsum += p;
        pk[kt][e] = (__bf16)p;
      }
    }
    // O^T += V^T P^T: A = V^T rows 16 dt + l16, keys 16 kt + 4g .. +3
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x4 va = __builtin_bit_cast(
            bf16x4, *reinterpret_cast<const uint2*>(sVt + (16 * dt + l16) * VP + 16 * kt + 4 * g));
        oacc[dt] = mfma_k16(va, pk[kt], oacc[dt]);
      }
    }
  };
  for (int j = 0; j < nblk; j += 2) {
    step(j, ring0);
    step(j + 1, ring1);
  }

  // ---- results: lane (g, l16) holds O^T rows d = 16 dt + 4g + e of query row r
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (!rv) return;
  if (NS == 1) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t w0 = (uint32_t)float_to_bf16_bits(oacc[dt][0] * inv) |
                          ((uint32_t)float_to_bf16_bits(oacc[dt][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)float_to_bf16_bits(oacc[dt][2] * inv) |
                          ((uint32_t)float_to_bf16_bits(oacc[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(a.o + orow * D + 16 * dt + 4 * g) = make_uint2(w0, w1);
    }
  } else {
    float* po = a.part_o + (orow * NS + split) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
          make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
    if (g == 0)
      *reinterpret_cast<float2*>(a.part_ml + (orow * NS + split) * 2) = make_float2(m, lsum);
  }
}

// o[row] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits
// (zero when no split saw a key: the rows of a rejected sequence). One
// workgroup per sequence (rows of an invalid node range are left alone), one
// wave per output row, 64 lanes over d.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(const AttnArgs a) {
  const int b = blockIdx.x;
  const int lo = a.offsets[b];
  const int hi = a.offsets[b + 1];
  if (lo < 0 || hi > a.T || hi - lo < 1 || hi - lo > a.max_nodes) return;
  const int lane = threadIdx.x & 63;
  const int NS = a.NS;
  for (int row = lo * a.Hq + (threadIdx.x >> 6); row < hi * a.Hq; row += 4) {
    const float* ml = a.part_ml + (size_t)row * NS * 2;
    float M = kMasked;
    for (int s = 0; s < NS; ++s) M = fmaxf(M, ml[2 * s]);
    float den = 0.f;
    float acc[D / 64];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] = 0.f;
    for (int s = 0; s < NS; ++s) {
      const float w = ml[2 * s + 1] > 0.f ? exp2f(ml[2 * s] - M) : 0.f;
      den += w * ml[2 * s + 1];
      const float* po = a.part_o + ((size_t)row * NS + s) * D;
#pragma unroll
      for (int c = 0; c < D / 64; ++c) acc[c] += w * po[lane + 64 * c];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c)
      a.o[(size_t)row * D + lane + 64 * c] = float_to_bf16_bits(acc[c] * inv);
  }
}

// One workgroup per sequence: validate, find the accepted path, append its
// K/V rows (root first) for every K/V head, advance the length.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_commit_kernel(const AttnCommitArgs a) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  __shared__ int sPath[64];
  __shared__ int sInfo[3];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (tid < 64) {
    const int lo = a.offsets[b];
    const int hi = a.offsets[b + 1];
    const int n = hi - lo;
    const int L = a.cache_len[b];
    int st = GDN_TREE_OK, P = 0;
    if (lo < 0 || hi > a.T || n < 1 || n > a.max_nodes || L < 0 || L > a.cap) {
      st = GDN_TREE_BAD_SIZE;
    } else {
      const int par_raw = a.parents[lo + (lane < n ? lane : 0)];
      const int par = lane < n ? par_raw : -1;
      const int acc = a.accepted[b];
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
        P = __popcll(path);
        if (L + P > a.cap) {
          st = GDN_TREE_CACHE_FULL;
          P = 0;
        } else if ((path >> lane) & 1ull) {
          sPath[__popcll(path & ((1ull << lane) - 1ull))] = lo + lane;   // root first
        }
      }
    }
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = P;
      sInfo[2] = L;
      a.status[b] = st;
    }
  }
  __syncthreads();
  const int st = sInfo[0];
  const int P = sInfo[1];
  const int L = sInfo[2];
  if (st != GDN_TREE_OK || P == 0) return;
  const int work = 2 * a.Hkv * P * CPR;
  for (int id = tid; id < work; id += 256) {
    const int mat = id / (a.Hkv * P * CPR);
    int rem = id - mat * a.Hkv * P * CPR;
    const int kvh = rem / (P * CPR);
    rem -= kvh * P * CPR;
    const int pr = rem / CPR;
    const int c = rem - pr * CPR;
    const uint16_t* src = (mat ? a.v : a.k) + ((size_t)sPath[pr] * a.Hkv + kvh) * D + 8 * c;
    uint16_t* dst = (mat ? a.vc : a.kc) + (((size_t)b * a.Hkv + kvh) * a.cap + L + pr) * D + 8 * c;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  __syncthreads();
  if (tid == 0) a.cache_len[b] = L + P;
}

template <int D>
hipError_t launch_attn_d(const AttnArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.Hkv * a.NS);
  hipError_t e = launch_kernel(reinterpret_cast<const void*>(&tree_attn_kernel<D>), grid,
                               (unsigned)kAttnThreads, s, a);
  if (e != hipSuccess || a.NS == 1) return e;
  return launch_kernel(reinterpret_cast<const void*>(&tree_attn_combine_kernel<D>),
                       (unsigned)a.B, 256u, s, a);
}

}  // namespace

hipError_t launch_tree_attn(int d, const AttnArgs& a, hipStream_t s) {
  switch (d) {
    case 64: return launch_attn_d<64>(a, s);
    case 128: return launch_attn_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tree_attn_commit(int d, const AttnCommitArgs& a, hipStream_t s) {
  switch (d) {
    case 64:
      return launch_kernel(reinterpret_cast<const void*>(&tree_attn_commit_kernel<64>),
                           (unsigned)a.B, 256u, s, a);
    case 128:
      return launch_kernel(reinterpret_cast<const void*>(&tree_attn_commit_kernel<128>),
                           (unsigned)a.B, 256u, s, a);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
