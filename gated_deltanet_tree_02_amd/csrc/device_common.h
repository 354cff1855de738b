// device_common.h -- helpers shared by the gfx950 kernels of libgdntree:
// io element access, bf16 conversion, the per-sequence tree prologue
// (validation, ancestor masks, depths) and wave-level LDS ordering.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- io types
// q, k, v and o are stored either as fp32 or as bf16 bit patterns (uint16).

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, h);
}

template <class IO> struct io_traits;

template <> struct io_traits<float> {
  // four consecutive elements -> fp32
  __device__ __forceinline__ static float4 load4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ static void store4(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <> struct io_traits<uint16_t> {
  __device__ __forceinline__ static float4 load4(const uint16_t* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_bits_to_float(u.x & 0xffffu), bf16_bits_to_float(u.x >> 16),
                       bf16_bits_to_float(u.y & 0xffffu), bf16_bits_to_float(u.y >> 16));
  }
  __device__ __forceinline__ static void store4(uint16_t* p, float4 v) {
    uint2 u;
    u.x = (uint32_t)float_to_bf16_bits(v.x) | ((uint32_t)float_to_bf16_bits(v.y) << 16);
    u.y = (uint32_t)float_to_bf16_bits(v.z) | ((uint32_t)float_to_bf16_bits(v.w) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) {
    return bf16_bits_to_float(*p);
  }
  __device__ __forceinline__ static void store1(uint16_t* p, float v) { *p = float_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  lo = (uint32_t)__shfl((int)lo, src, kWave);
  hi = (uint32_t)__shfl((int)hi, src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// LDS written by some lanes of a wave, then read by other lanes of the same
// wave: keep the compiler from moving accesses across this point. The LDS
// executes one wave's DS instructions in issue order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-sequence result code. merge == 0: the code is written. merge != 0 (a
// later step of a captured round): a code already set by an earlier step of
// the round is kept, so the round reports the first failure of a sequence.
__device__ __forceinline__ void put_status(int32_t* status, int b, int code, int merge) {
  if (!merge)
    status[b] = code;
  else if (code != GDN_TREE_OK && status[b] == GDN_TREE_OK)
    status[b] = code;
}

// Base-2 logarithm of a decay gate, clamped so that a gate of 0 (or a
// denormal) stays finite: 2^-64 is far below fp32 resolution of any other
// term, so the clamp does not change a result.
__device__ __forceinline__ float gate_log2(float alpha) {
  return fmaxf(log2f(alpha), -64.0f);
}

// ---------------------------------------------------------------- tree prologue
// One wave, lane t = local node t. Checks sequence b's node range and
// parents (handbook implementation section: root first with parent -1,
// parents before children) and builds each node's visible set (itself and
// its ancestors, fork page section 2) by pointer jumping: after j rounds a
// lane has merged the sets of the 2^j nearest nodes on its path, so six
// rounds cover any depth below 64.

struct TreeLane {
  int lo;          // first global node of the sequence
  int n;           // nodes in the sequence (meaningful unless status == BAD_SIZE)
  int status;      // GDN_TREE_* (wave-uniform)
  int parent;      // lane's parent (local), -1 for the root, 0 for lanes >= n
  uint64_t anc;    // lane's visible set (0 for lanes >= n)
  int depth;       // lane's depth (-1 for lanes >= n)
};

__device__ __forceinline__ TreeLane load_tree(int b, int T, int max_nodes,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ parents, int lane) {
  TreeLane tl;
  const int lo = offsets[b];
  const int hi = offsets[b + 1];
  tl.lo = lo;
  tl.n = hi - lo;
  tl.parent = 0;
  tl.anc = 0;
  tl.depth = -1;
  if (lo < 0 || hi > T || hi - lo < 1 || hi - lo > max_nodes) {
    tl.status = GDN_TREE_BAD_SIZE;
    return tl;
  }
  const int n = tl.n;
  const int par = lane < n ? parents[lo + lane] : 0;
  const int root_par = __shfl(par, 0, kWave);
  const bool bad = lane >= 1 && lane < n && (par < 0 || par >= lane);
  if (root_par != -1) {
    tl.status = GDN_TREE_BAD_ROOT;
    return tl;
  }
  if (__ballot(bad) != 0ull) {
    tl.status = GDN_TREE_BAD_PARENT;
    return tl;
  }
  tl.status = GDN_TREE_OK;
  tl.parent = lane < n ? par : 0;
  uint64_t anc = lane < n ? (1ull << lane) : 0ull;
  int jmp = lane < n ? par : -1;
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    const int src = jmp < 0 ? lane : jmp;
    const uint64_t a2 = shfl_u64(anc, src);
    const int j2 = __shfl(jmp, src, kWave);
    if (jmp >= 0) {
      anc |= a2;
      jmp = j2;
    }
  }
  tl.anc = anc;
  tl.depth = lane < n ? (__popcll(anc) - 1) : -1;
  return tl;
}

// Pointer jumping over already-loaded parents (lane t holds parent(t), -1 for
// the root, lanes >= n hold -1): visible set and the sum of x over the path
// (x = 0 on lanes >= n). Six rounds cover depths below 64; the scan stops once
// every lane has reached the root (after ceil(log2(depth + 1)) rounds).
__device__ __forceinline__ void path_scan(int par, int lane, int n, float x, uint64_t& anc,
                                          float& sum) {
  anc = lane < n ? (1ull << lane) : 0ull;
  sum = x;
  int jmp = lane < n ? par : -1;
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    if (__ballot(jmp >= 0) == 0ull) break;
    const int src = jmp < 0 ? lane : jmp;
    const uint64_t a2 = shfl_u64(anc, src);
    const float s2 = __shfl(sum, src, kWave);
    const int j2 = __shfl(jmp, src, kWave);
    if (jmp >= 0) {
      anc |= a2;
      sum += s2;
      jmp = j2;
    }
  }
}

// Sum of x over each lane's path, in increasing node order (root first):
// every lane reads node j's value by a shuffle and keeps it when j is on its
// path. n is the (wave-uniform) node count.
__device__ __forceinline__ float path_sum(uint64_t anc, float x, int n) {
  float acc = 0.0f;
  for (int j = 0; j < n; ++j) {
    const float xj = __shfl(x, j, kWave);
    if ((anc >> j) & 1ull) acc += xj;
  }
  return acc;
}

}  // namespace gdn
