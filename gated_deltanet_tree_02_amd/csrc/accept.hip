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
#include <type_traits>

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
  // in a captured round, a sequence an earlier step rejected keeps its code
  // and accepts nothing, so that no commit changes its state
  const int earlier = a.merge ? a.status[b] : GDN_TREE_OK;
  if (tl.status != GDN_TREE_OK || earlier != GDN_TREE_OK) {
    if (lane == 0) {
      put_status(a.status, b, tl.status, a.merge);
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
    put_status(a.status, b, GDN_TREE_OK, a.merge);
    a.accepted[b] = cur;
    a.accept_len[b] = len;
    a.next_token[b] = next;
  }
}

// ---------------------------------------------------------------- sampling mode
//
// Multi-candidate rejection sampling down the tree (handbook, same chapter,
// exercise on sampling with a tree). At the current node with target p and
// draft q (the distribution its children were drawn from, without
// replacement, in node order), candidate x is accepted iff u q_k(x) < p_k(x);
// after rejecting it the target becomes p_{k+1} = norm(max(0, p_k - q_k))
// (unchanged when that has no mass) and the proposal q_{k+1} = q without the
// rejected tokens, renormalised. An accepted child starts afresh with its own
// rows; when no candidate is accepted, one token is drawn from p_k by inverse
// CDF and the walk ends.
//
// One workgroup per sequence, or (split form) several, which divide every
// pass over a node's rows by tiles and trade their tile sums after it. p_k and
// q_k are never stored: for any token they follow from p(j), q(j) and the
// per-stage scalars (1/Z_i, the rejected tokens, the renormalisation of q). A
// rejection costs one pass over the node's two rows, which yields the
// normaliser Z as a sum of per-tile sums of max(0, p_k - q_k) (the first one
// at a node also the row's q mass, per tile); those tile sums, scaled by 1/Z,
// are the tile sums of the next p, so a final draw after a rejection needs no
// further pass (a draw with no rejection at the node takes one pass over p).
// The draw then finds the tile where the cumulative mass crosses the target
// and re-reads that tile alone. Each wave works on whole 256-token tiles and
// keeps kTilesInFlight tiles' loads in flight. Decisions are taken in fp32;
// totals run over the tile sums in a fixed order, so they do not depend on how
// the tiles were divided.

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr int kTile = kSamplingTile;             // tokens per tile (64 lanes x 4)
static_assert(kTile == 256, "a tile is 64 lanes x 4 tokens");
constexpr int kTilesInFlight = 4;
// (the split form takes fewer tiles per wave per pass, and more of them in
// flight at once pays there)
constexpr int kSplitTilesInFlight = 5;
constexpr int kMaxTiles = (1 << 20) / kTile;     // vocabularies up to 2^20 tokens

struct Stages {
  int k;                  // rejections so far at this node
  const int* rem;         // rejected tokens x_0 .. x_{k-1}
  const float* zinv;      // 1 / Z_{i+1}, or 0 when that residual had no mass
  const float* qscale;    // q_i = q restricted to tokens not in x_0..x_{i-1}, times qscale[i]
};

__device__ __forceinline__ bool removed(int j, const int* rem, int upto) {
  bool r = false;
  for (int i = 0; i < upto; ++i) r |= rem[i] == j;
  return r;
}

// (p_k(j), q_k(j)) from the row values p(j), q(j)
__device__ __forceinline__ float2 stage_pq(float pj, float qj, int j, const Stages& s) {
  float pk = pj;
  for (int i = 0; i < s.k; ++i) {
    const float qi = removed(j, s.rem, i) ? 0.f : qj * s.qscale[i];
    if (s.zinv[i] > 0.f) pk = fmaxf(pk - qi, 0.f) * s.zinv[i];
  }
  const float qk = removed(j, s.rem, s.k) ? 0.f : qj * s.qscale[s.k];
  return make_float2(pk, qk);
}

// The same for exactly K stages, their scalars in scalar registers: a pass
// evaluates it for every token of a row. A token is in the removed set of
// stage i when it is one of x_0 .. x_{i-1}.
template <int K>
struct StageRegs {
  int rem[K > 0 ? K : 1];
  float zinv[K > 0 ? K : 1];
  float qscale[K + 1];
};

__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <int K>
__device__ __forceinline__ StageRegs<K> stage_regs(const Stages& s) {
  StageRegs<K> r;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    r.rem[i] = __builtin_amdgcn_readfirstlane(s.rem[i]);
    r.zinv[i] = uniform_f(s.zinv[i]);
  }
#pragma unroll
  for (int i = 0; i <= K; ++i) r.qscale[i] = uniform_f(s.qscale[i]);
  return r;
}

template <int K>
__device__ __forceinline__ float2 stage_pq_reg(float pj, float qj, int j, const StageRegs<K>& r) {
  float pk = pj;
  bool gone = false;          // j in the removed set of the stage at hand
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const float qi = gone ? 0.f : qj * r.qscale[i];
    if (r.zinv[i] > 0.f) pk = fmaxf(pk - qi, 0.f) * r.zinv[i];
    gone |= j == r.rem[i];
  }
  return make_float2(pk, gone ? 0.f : qj * r.qscale[K]);
}

// Sum over the 64 lanes of a wave in DPP steps, with no LDS traffic: an
// inclusive scan within each row of 16 lanes (shifts by 1, 2, 4, 8; lanes
// shifted in from outside the row read 0), then lane 15 of rows 0 and 2
// carried into rows 1 and 3, then lane 31 into rows 2 and 3. Lane 63 ends
// with the total.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xf,
                                            true);
  return x + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float wave_sum_lane63(float x) {
  x = dpp_add<0x111, 0xf>(x);   // row_shr:1
  x = dpp_add<0x112, 0xf>(x);   // row_shr:2
  x = dpp_add<0x114, 0xf>(x);   // row_shr:4
  x = dpp_add<0x118, 0xf>(x);   // row_shr:8
  x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
// The same total in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_lane63(x)), 63));
}

// What a tile pass sums per token.
enum TileSum { kResidual, kTarget };

// One pass over tiles [tbeg, tend) of a node's rows: sTile[t] = sum over tile t
// of max(0, p_k - q_k) (kResidual) or of p_k (kTarget), and with kQSum sQ[t] =
// the tile's q mass. Wave w takes tiles tbeg + w, tbeg + w + waves, ... through
// a ring of kTilesInFlight tiles: a tile's slot is refilled with the wave's
// next-but-(kTilesInFlight - 1) tile as soon as it is summed, so every wave
// keeps that many tiles' loads in flight for the whole pass. K >= 0: exactly
// K rejections so far, the stage scalars in registers; K < 0: any number, read
// from LDS. A tile's sums are the same whichever workgroup takes it.
template <TileSum WHAT, int K, bool kQSum, int W>
__device__ __forceinline__ void tile_pass_t(const float* __restrict__ prow,
                                            const float* __restrict__ qrow, int V, int tbeg,
                                            int tend, const Stages& s, float* sTile, float* sQ) {
  const StageRegs<K < 0 ? 0 : K> r = stage_regs<K < 0 ? 0 : K>(s);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int span = tend - tbeg;
  const int mine = wave < span ? (span - 1 - wave) / kSampleWaves + 1 : 0;
  // p_0 needs no q: a draw with no rejection reads the target row alone
  constexpr bool need_q = WHAT == kResidual || K != 0 || kQSum;
  // element offsets are clamped into the row (V >= 4), so that every load is
  // issued unconditionally; tiles past the wave's last one are not summed
  auto off = [&](int i) {
    const int j = (tbeg + wave + i * kSampleWaves) * kTile + 4 * lane;
    return j < V - 4 ? j : V - 4;
  };
  float4 pv[W], qv[W];
#pragma unroll
  for (int u = 0; u < W; ++u) {
    pv[u] = *reinterpret_cast<const float4*>(prow + off(u));
    qv[u] = need_q ? *reinterpret_cast<const float4*>(qrow + off(u))
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int i0 = 0; i0 < mine; i0 += W) {
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int i = i0 + u;
      const int t = tbeg + wave + i * kSampleWaves;
      const int j = t * kTile + 4 * lane;
      const bool in_row = i < mine && j < V;
      const float pe[4] = {in_row ? pv[u].x : 0.f, in_row ? pv[u].y : 0.f,
                           in_row ? pv[u].z : 0.f, in_row ? pv[u].w : 0.f};
      const float qe[4] = {in_row ? qv[u].x : 0.f, in_row ? qv[u].y : 0.f,
                           in_row ? qv[u].z : 0.f, in_row ? qv[u].w : 0.f};
      // the slot's next tile
      pv[u] = *reinterpret_cast<const float4*>(prow + off(i + W));
      if (need_q) qv[u] = *reinterpret_cast<const float4*>(qrow + off(i + W));
      float m = 0.f, qm = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 pq = K >= 0 ? stage_pq_reg<K < 0 ? 0 : K>(pe[e], qe[e], j + e, r)
                                 : stage_pq(pe[e], qe[e], j + e, s);
        m += WHAT == kResidual ? fmaxf(pq.x - pq.y, 0.f) : pq.x;
        qm += qe[e];
      }
      m = wave_sum_lane63(m);
      if (kQSum) qm = wave_sum_lane63(qm);
      if (lane == 63 && i < mine) {
        sTile[t] = m;
        if (kQSum) sQ[t] = qm;
      }
    }
  }
}

template <TileSum WHAT, int W>
__device__ __forceinline__ void tile_pass(const float* __restrict__ prow,
                                          const float* __restrict__ qrow, int V, int tbeg,
                                          int tend, const Stages& s, float* sTile, float* sQ) {
  switch (s.k) {
    // the first rejection's pass also gives the q mass of the row, per tile
    case 0:
      if constexpr (WHAT == kResidual)
        return tile_pass_t<WHAT, 0, true, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
      else
        return tile_pass_t<WHAT, 0, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
    case 1: return tile_pass_t<WHAT, 1, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
    case 2: return tile_pass_t<WHAT, 2, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
    case 3: return tile_pass_t<WHAT, 3, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
    case 4: return tile_pass_t<WHAT, 4, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
    default: return tile_pass_t<WHAT, -1, false, W>(prow, qrow, V, tbeg, tend, s, sTile, sQ);
  }
}

// A sum over tiles [0, ntiles) of `v` (times `scale`) in a fixed order, by wave
// 0: lane l adds its block of ceil(ntiles / 64) tiles in order, then the lanes
// are added in DPP steps. Every lane of wave 0 gets the total.
__device__ __forceinline__ float tiles_total(const float* v, int ntiles, float scale) {
  const int lane = threadIdx.x & 63;
  const int per = (ntiles + 63) / 64;
  const int t0 = min(lane * per, ntiles), t1 = min(t0 + per, ntiles);
  float ls = 0.f;
  for (int t = t0; t < t1; ++t) ls += v[t] * scale;
  return wave_sum(ls);
}

// How long a workgroup of the split form waits for the others' tile sums
// (polls, each after a short sleep; a poll takes about a microsecond) before
// it sums every tile of the row itself. The sums are the same either way, so
// the wait only costs time: with every workgroup resident it never runs out;
// a workgroup that is not resident yet (the device busy with other work)
// cannot hold the others up.
constexpr unsigned kPatience = 256;

// The split form's exchange after a pass over tiles [tbeg, tend). Every tile
// sum travels as one 64-bit word, the value's bits in the low half and the
// pass number (from 1) in the high half, written and read with single atomic
// accesses at device scope (coherent across the XCDs' L2s): a reader that
// sees the pass number sees the value, so no fence or counter is needed. Wave
// 0 publishes this workgroup's tiles once the pass is done (stores issued
// during the pass would share the load counter the pass waits on); then every
// thread polls its share of all tiles of the row until each carries this
// pass's number, and copies the values into sTile (and sQ). Each sequence has
// two sets of words that alternate between passes. A word holds the value of
// the pass its number names (every writer computes the same value), so a
// workgroup that reads a word another one has already reused for a later pass
// only sees a number that is not its pass's and keeps waiting, then sums the
// tiles itself. The words are cleared before every call. Returns false if the
// wait ran out.
__device__ bool exchange_tiles(const AcceptSampleArgs& a, int b, int tbeg, int tend, int ntiles,
                               bool with_q, unsigned& nsync, float* sTile, float* sQ) {
  const int tid = threadIdx.x;
  const unsigned long long tag = (unsigned long long)(nsync + 1u) << 32;
  unsigned long long* words =
      a.xch + ((size_t)b * 2 + (nsync & 1u)) * 2 * (size_t)a.xch_stride;
  unsigned long long* qwords = words + a.xch_stride;
  __syncthreads();                       // this workgroup's tiles are in LDS
  if (tid < 64) {
    for (int t = tbeg + tid; t < tend; t += 64) {
      __hip_atomic_store(words + t, tag | __builtin_bit_cast(unsigned, sTile[t]),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (with_q)
        __hip_atomic_store(qwords + t, tag | __builtin_bit_cast(unsigned, sQ[t]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  ++nsync;
  for (unsigned polls = 0;; ++polls) {
    int missing = 0;
    for (int t = tid; t < ntiles; t += kSampleThreads) {
      if (t >= tbeg && t < tend) continue;   // this workgroup's own
      const unsigned long long w = __hip_atomic_load(words + t, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      if ((w & ~0xffffffffull) == tag) sTile[t] = __builtin_bit_cast(float, (unsigned)w);
      else missing = 1;
      if (with_q) {
        const unsigned long long u = __hip_atomic_load(qwords + t, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        if ((u & ~0xffffffffull) == tag) sQ[t] = __builtin_bit_cast(float, (unsigned)u);
        else missing = 1;
      }
    }
    if (!__syncthreads_or(missing)) return true;
    if (polls == kPatience) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// One workgroup per sequence (kSplit false), or a.splits workgroups per
// sequence, workgroup i taking part i % splits of sequence i / splits: every
// workgroup of a sequence takes the same decisions (from the same sums in the
// same order), and a pass over a node's rows is divided among them by tiles.
template <bool kSplit>
__global__ __launch_bounds__(kSampleThreads) void accept_sampling_kernel(const AcceptSampleArgs a) {
  __shared__ int sPar[64];
  __shared__ int sTok[64];
  __shared__ int sRem[64];
  __shared__ float sZinv[64];
  __shared__ float sQscale[65];
  __shared__ float sPX[64], sQX[64], sUX[64];   // candidates: p(x), q(x), uniform
  __shared__ float sTile[kMaxTiles];
  __shared__ float sQ[kMaxTiles];
  __shared__ int sInfo[4];              // status, lo, n, decision / crossing tile
  __shared__ float sF[2];               // crossing: mass before the tile, draw target

  // (the divisions by runtime values go through vector registers: their
  // uniform results are moved back to scalar ones)
  const int S = kSplit ? a.splits : 1;
  const int b = kSplit ? __builtin_amdgcn_readfirstlane((int)blockIdx.x / S) : (int)blockIdx.x;
  const int part = kSplit ? (int)blockIdx.x - b * S : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < 64) {
    const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
    sPar[lane] = tl.parent;
    const int tok = (tl.status != GDN_TREE_BAD_SIZE && lane < tl.n) ? a.draft[tl.lo + lane] : 0;
    sTok[lane] = tok;
    // a candidate's token indexes the probability rows: it must be a token
    const bool bad_tok = lane >= 1 && lane < tl.n && (tok < 0 || tok >= a.V);
    const int st = tl.status == GDN_TREE_OK && __ballot(bad_tok) != 0ull ? GDN_TREE_BAD_TOKEN
                                                                           : tl.status;
    if (lane == 0) {
      sInfo[0] = st;
      sInfo[1] = tl.lo;
      sInfo[2] = tl.n;
    }
  }
  if (tid == 0) sQscale[0] = 1.f;
  __syncthreads();
  const int st = sInfo[0], lo = sInfo[1], n = sInfo[2];
  if (st != GDN_TREE_OK) {             // (the same for every workgroup of the sequence)
    if (part == 0 && tid == 0) {
      a.status[b] = st;
      a.accepted[b] = -1;
      a.accept_len[b] = 0;
      a.next_token[b] = -1;
    }
    return;
  }
  const int V = a.V;
  const int ntiles = (V + kTile - 1) / kTile;
  const int tbeg = __builtin_amdgcn_readfirstlane(part * ntiles / S);
  const int tend = __builtin_amdgcn_readfirstlane((part + 1) * ntiles / S);
  unsigned nsync = 0;                   // exchanges passed (split form)
  // A pass over this workgroup's tiles, then every tile's sums in sTile (sQ):
  // from the others' words, or, if they do not come, from a second pass here
  // over all tiles (the same call site, so the pass is inlined once).
  auto pass_all = [&](auto what, const float* prow, const float* qrow, const Stages& st,
                      bool with_q) {
    int tb = tbeg, te = tend;
    for (;;) {
      tile_pass<decltype(what)::value, kSplit ? kSplitTilesInFlight : kTilesInFlight>(
          prow, qrow, V, tb, te, st, sTile, sQ);
      if (!kSplit || (tb == 0 && te == ntiles)) {
        __syncthreads();
        return;
      }
      if (exchange_tiles(a, b, tbeg, tend, ntiles, with_q, nsync, sTile, sQ)) return;
      tb = 0;
      te = ntiles;
    }
  };
  int cur = 0, len = 1, token = V - 1;
  for (;;) {
    const float* __restrict__ prow = a.p + (size_t)(lo + cur) * V;
    const float* __restrict__ qrow = a.q + (size_t)(lo + cur) * V;
    Stages s{0, sRem, sZinv, sQscale};
    float qtot = 0.f, qrem = 0.f;
    bool tiles_ready = false;             // sTile holds the current p's tile sums / Z
    int next = -1;
    // every candidate's p(x), q(x) and uniform, one lane per child, in one
    // round trip when the walk enters the node
    if (tid > cur && tid < n && sPar[tid] == cur) {
      const int x = sTok[tid];
      sPX[tid] = prow[x];
      sQX[tid] = qrow[x];
      sUX[tid] = a.u[2 * (size_t)(lo + tid)];
    }
    __syncthreads();
    for (int c = cur + 1; c < n; ++c) {   // children have larger indices, in node order
      if (sPar[c] != cur) continue;       // uniform
      const int x = sTok[c];
      // (every thread takes the decision alike, from the same values)
      const float2 pq = stage_pq(sPX[c], sQX[c], x, s);
      const bool take = sUX[c] * pq.y < pq.x;
      if (take) {
        next = c;
        break;
      }
      // rejected: tile sums of the residual max(0, p_k - q_k), and its mass Z
      // (the first pass at a node also sums the row's q mass)
      pass_all(std::integral_constant<TileSum, kResidual>{}, prow, qrow, s, s.k == 0);
      if (wave == 0) {
        const float z = tiles_total(sTile, ntiles, 1.f);
        if (s.k == 0) qtot = tiles_total(sQ, ntiles, 1.f);
        qrem += sQX[c];
        if (lane == 0) {
          sZinv[s.k] = z > 0.f ? 1.f / z : 0.f;
          sRem[s.k] = x;
          const float left = qtot - qrem;
          sQscale[s.k + 1] = left > 0.f ? 1.f / left : 1.f;
        }
      }
      __syncthreads();
      tiles_ready = sZinv[s.k] > 0.f;     // else p is unchanged and has no tile sums here
      s.k += 1;
    }
    if (next >= 0) {
      cur = next;
      ++len;
      continue;
    }
    // final draw from p_k: tile sums (from the last rejection's pass, scaled,
    // or from one pass over p), the crossing tile, then the token in it
    float scale = 1.f;
    if (tiles_ready) {
      scale = sZinv[s.k - 1];
    } else {
      pass_all(std::integral_constant<TileSum, kTarget>{}, prow, qrow, s, false);
    }
    if (wave == 0) {
      // lane l owns tiles [l*per, (l+1)*per)
      const int per = (ntiles + 63) / 64;
      const int t0 = min(lane * per, ntiles), t1 = min(t0 + per, ntiles);
      float ls = 0.f;
      for (int t = t0; t < t1; ++t) ls += sTile[t] * scale;
      float incl = ls;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      const float total = __shfl(incl, 63, kWave);
      const float target = a.u[2 * (size_t)(lo + cur) + 1] * total;
      const uint64_t over = __ballot(incl > target && t1 > t0);
      const int L = over ? __builtin_ctzll(over) : -1;
      if (lane == (L < 0 ? 63 : L)) {
        float run = incl - ls;
        int tile = t1 > t0 ? t1 - 1 : ntiles - 1;
        float before = run;
        for (int t = t0; t < t1; ++t) {
          if (run + sTile[t] * scale > target) {
            tile = t;
            before = run;
            break;
          }
          run += sTile[t] * scale;
          before = run;
        }
        sInfo[3] = tile;
        sF[0] = before;
        sF[1] = target;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int tile = sInfo[3];
      const float before = sF[0], target = sF[1];
      const int j0 = tile * kTile + 4 * lane;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (j0 < V) {
        const float4 p4 = *reinterpret_cast<const float4*>(prow + j0);
        const float4 q4 = *reinterpret_cast<const float4*>(qrow + j0);
        v[0] = stage_pq(p4.x, q4.x, j0, s).x;
        v[1] = stage_pq(p4.y, q4.y, j0 + 1, s).x;
        v[2] = stage_pq(p4.z, q4.z, j0 + 2, s).x;
        v[3] = stage_pq(p4.w, q4.w, j0 + 3, s).x;
      }
      const float ls = v[0] + v[1] + v[2] + v[3];
      float incl = ls;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      float run = before + incl - ls;
      int hit = -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        run += v[e];
        if (hit < 0 && j0 + e < V && run > target) hit = j0 + e;
      }
      const uint64_t any = __ballot(hit >= 0);
      const int first = any ? __builtin_ctzll(any) : -1;
      const int hit_first = __shfl(hit, first < 0 ? 0 : first, kWave);
      if (lane == 0) token = first >= 0 ? hit_first : min(tile * kTile + kTile, V) - 1;
    }
    break;
  }
  if (part == 0 && tid == 0) {
    a.status[b] = GDN_TREE_OK;
    a.accepted[b] = cur;
    a.accept_len[b] = len;
    a.next_token[b] = token;
  }
}

// The split form's exchange words start every call at pass number 0 (none).
__global__ __launch_bounds__(256) void sampling_xch_clear_kernel(const AcceptSampleArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (size_t)a.B * 4 * a.xch_stride) a.xch[i] = 0ull;
}

}  // namespace

hipError_t launch_accept_sampling(const AcceptSampleArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&accept_sampling_kernel<false>),
                       (unsigned)a.B, (unsigned)kSampleThreads, s, a);
}

int accept_sampling_split_capacity() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&accept_sampling_kernel<true>),
          kSampleThreads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

hipError_t launch_accept_sampling_split(const AcceptSampleArgs& a, hipStream_t s) {
  const size_t words = (size_t)a.B * 4 * a.xch_stride;
  const hipError_t e = launch_kernel(reinterpret_cast<const void*>(&sampling_xch_clear_kernel),
                                     (unsigned)((words + 255) / 256), 256u, s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(reinterpret_cast<const void*>(&accept_sampling_kernel<true>),
                       (unsigned)(a.B * a.splits), (unsigned)kSampleThreads, s, a);
}

hipError_t launch_accept_greedy(const AcceptArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&accept_greedy_kernel),
                       (unsigned)((a.B + 3) / 4), 256u, s, a);
}

}  // namespace gdn
