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
// p_k and q_k are never stored. After k rejections at a node they have a
// closed form in the row values p(j), q(j) and a few per-stage scalars:
//   p_k(j) = max(0, p(j) - L_k(j) q(j)) / U_k,   q_k(j) = s_k q(j) or 0,
// with L_k(j) = lam_k and q_k(j) = s_k q(j) for a token not rejected yet, and
// L_k(j) = lam_{m+1}, q_k(j) = 0 for the token x_m rejected at stage m; s_k
// renormalises q over the tokens left, lam_0 = 0 and U_0 = 1. It follows by
// induction from max(0, max(0, a) / c - b) = max(0, a - b c) / c (c > 0,
// b >= 0): rejecting x_k leaves the residual max(0, p_k - q_k) =
// max(0, p - lam' q) / U_k with lam' = lam_k + s_k U_k on the tokens not
// rejected before (x_k among them), and p_k itself on the others; so
// lam_{k+1} = lam' and U_{k+1} = U', the sum of the numerators, when U' > 0,
// and nothing changes when the residual has no mass. A pass over a node's rows
// therefore costs the same few operations per token at every stage: a
// rejection sums the numerators max(0, p - lam' q) tile by tile (the first one
// at a node also the row's q mass), and each tile holding an earlier rejected
// token is then corrected for that token alone. Those tile sums are the
// numerators of the next p, so a final draw after a rejection needs no further
// pass (a draw with no rejection at the node takes one pass over p).
//
// One workgroup per sequence, or (split form) several, which divide every
// pass over a node's rows by fixed groups of tiles and trade their group sums
// after it. The draw finds the group, then the tile where the cumulative mass
// crosses the target, and re-reads that tile alone. Each wave works on whole
// 256-token tiles and keeps several tiles' loads in flight. Decisions
// are taken in fp32; totals run over group sums in a fixed order, so they do
// not depend on how the tiles were divided.

constexpr int kSampleThreads = 1024;             // one workgroup per sequence
// The split form's workgroups are smaller: a sequence's passes then spread
// over more CUs (with 64 sequences: 4 waves on each of 16 CUs, not 16 waves
// on each of 4), which is what a sequence left to walk alone on an otherwise
// idle device can use.
constexpr int kSplitThreads = 256;
constexpr int kTile = kSamplingTile;             // tokens per tile (64 lanes x 4)
static_assert(kTile == 256, "a tile is 64 lanes x 4 tokens");
constexpr int kTilesInFlight = 4;
// (the split form takes fewer tiles per wave per pass, and more of them in
// flight at once pays there)
constexpr int kSplitTilesInFlight = 6;
constexpr int kMaxTiles = (1 << 20) / kTile;     // vocabularies up to 2^20 tokens

// The stage after k rejections at the current node (in LDS, but u).
struct Stages {
  int k;                  // rejections so far at this node
  const int* rem;         // rejected tokens x_0 .. x_{k-1}
  const float* lam;       // lam_0 .. lam_k
  const float* qscale;    // s_0 .. s_k
  float u;                // U_k
};

// A value every lane holds alike, moved to a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Index of the first rejection of token j among x_0 .. x_{upto-1}, else -1.
__device__ __forceinline__ int rejected_at(int j, const int* rem, int upto) {
  int at = -1;
  for (int i = upto - 1; i >= 0; --i)
    if (rem[i] == j) at = i;
  return at;
}

// (U_k p_k(j), q_k(j)) from the row values p(j), q(j). With lam = 0 the
// target is p itself, whatever q holds (a leaf's draft row is never read as a
// distribution).
__device__ __forceinline__ float2 stage_pq(float pj, float qj, int j, const Stages& s) {
  const int m = rejected_at(j, s.rem, s.k);
  const float lam = m < 0 ? s.lam[s.k] : s.lam[m + 1];
  return make_float2(lam != 0.f ? fmaxf(fmaf(-lam, qj, pj), 0.f) : pj,
                     m < 0 ? qj * s.qscale[s.k] : 0.f);
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

// One pass over tiles [tbeg, tend) of a node's rows: sTile[t] = sum over tile
// t of max(0, p(j) - lam q(j)) (every token taken as not rejected), and with
// kQSum sQ[t] = the tile's q mass; kNeedQ false reads the target row alone
// (lam = 0). Wave w takes tiles tbeg + w, tbeg + w + waves, ... through a ring
// of W tiles: a tile's slot is refilled with the wave's next-but-(W - 1) tile
// as soon as it is summed, so every wave keeps that many tiles' loads in
// flight for the whole pass. A tile's sums are the same whichever workgroup
// takes it.
template <bool kQSum, bool kNeedQ, int W, int NWV>
__device__ __forceinline__ void tile_pass(const float* __restrict__ prow,
                                          const float* __restrict__ qrow, int V, int tbeg,
                                          int tend, float lam, float* sTile, float* sQ) {
  static_assert(kNeedQ || !kQSum, "the q mass needs the q row");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int span = tend - tbeg;
  const int mine =
      __builtin_amdgcn_readfirstlane(wave < span ? (span - 1 - wave) / NWV + 1 : 0);
  // element offsets are clamped into the row (V >= 4): the row's last tile
  // may be partial; its tokens past the row are not summed. A slot is loaded
  // only for a tile the wave has (a uniform branch): loads left in flight at
  // the end of a pass would hold up the next wait on the load counter.
  auto off = [&](int i) {
    const int j = (tbeg + wave + i * NWV) * kTile + 4 * lane;
    return j < V - 4 ? j : V - 4;
  };
  float4 pv[W], qv[W];
#pragma unroll
  for (int u = 0; u < W; ++u) {
    pv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    qv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (u < mine) {
      pv[u] = *reinterpret_cast<const float4*>(prow + off(u));
      if (kNeedQ) qv[u] = *reinterpret_cast<const float4*>(qrow + off(u));
    }
  }
  for (int i0 = 0; i0 < mine; i0 += W) {
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int i = i0 + u;
      if (i >= mine) break;             // the wave's tiles are done (uniform)
      const int t = tbeg + wave + i * NWV;
      const int j = t * kTile + 4 * lane;
      const float pe[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
      const float qe[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
      // the slot's next tile
      if (i + W < mine) {
        pv[u] = *reinterpret_cast<const float4*>(prow + off(i + W));
        if (kNeedQ) qv[u] = *reinterpret_cast<const float4*>(qrow + off(i + W));
      }
      float m = 0.f, qm = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m += kNeedQ ? fmaxf(fmaf(-lam, qe[e], pe[e]), 0.f) : pe[e];
        qm += qe[e];
      }
      // a lane past the row's end (in its partial last tile) read clamped
      // duplicates: it adds nothing (a lane's 4 tokens are all in or all out)
      if (j >= V) {
        m = 0.f;
        qm = 0.f;
      }
      m = wave_sum_lane63(m);
      if (kQSum) qm = wave_sum_lane63(qm);
      if (lane == 63) {
        sTile[t] = m;
        if (kQSum) sQ[t] = qm;
      }
    }
  }
}

// The row's tiles fall into kGroups fixed groups, group g being tiles
// [g * ntiles / kGroups, (g + 1) * ntiles / kGroups). Every total is taken over
// the group sums in group order, and every group sum over its tiles in a fixed
// order, so neither depends on how the tiles are divided among workgroups: a
// workgroup of the split form takes whole groups.
constexpr int kGroups = kSamplingGroups;

__device__ __forceinline__ int group_begin(int g, int ntiles) { return g * ntiles / kGroups; }

// Sum of v[t0, t1) by one wave in a fixed order: lane l adds its block of
// ceil((t1 - t0) / 64) tiles in order, then the lanes are added in DPP steps.
// Every lane gets the sum.
__device__ __forceinline__ float wave_tiles_sum(const float* v, int t0, int t1) {
  const int lane = threadIdx.x & 63;
  const int per = (t1 - t0 + 63) / 64;
  const int lo = min(t0 + lane * per, t1), hi = min(lo + per, t1);
  float ls = 0.f;
  for (int t = lo; t < hi; ++t) ls += v[t];
  return wave_sum(ls);
}

// The total of the kGroups group sums, in group order.
__device__ __forceinline__ float groups_total(const float* g) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kGroups; ++i) s += g[i];
  return s;
}

// How many of the other workgroups' words a workgroup of the split form reads
// (four loads in flight per word, so one read ends about every quarter of a
// memory round trip) before it sums every tile of the row itself. The sums are
// the same either way, so the wait only costs time: with every workgroup
// resident it never runs out; a workgroup that is not resident yet (the device
// busy with other work) cannot hold the others up.
constexpr unsigned kPatience = 1024;

// The split form's exchange words of sequence b for pass number `pass` (from
// 0): per sequence two sets of [group sums | q group sums] that alternate
// between passes, one 64-bit word per group, the pass number (from 1) in the
// high half and the value's bits in the low half. After every sequence's
// words, one arrival count per sequence.
constexpr int kSeqWords = 4 * kGroups;
__device__ __forceinline__ unsigned long long* xch_words(const AcceptSampleArgs& a, int b,
                                                         unsigned pass) {
  return a.xch + (size_t)b * kSeqWords + (pass & 1u) * 2 * kGroups;
}

// The end of a split-form workgroup: it counts itself in, and the last of the
// sequence's workgroups to arrive (all others are done reading and writing the
// words) clears the words and the count, so that the next call finds them zero
// without a clearing pass of its own. Before its workgroup counts in, every
// wave waits until its own stores are acknowledged: the words are written
// through to memory at device scope, so a word another workgroup published
// cannot land after the clearing store. (A device-scope fence would also write
// back and invalidate the L2 of the XCD, which the workgroups still walking
// their rows there would pay for.)
__device__ void seq_done(const AcceptSampleArgs& a, int b) {
  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left free (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    unsigned long long* count = a.xch + (size_t)a.B * kSeqWords + b;
    unsigned long long before = 0ull;
    if (lane == 0)
      before = __hip_atomic_fetch_add(count, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    before = __shfl(before, 0, kWave);
    if (before == (unsigned long long)(a.splits - 1)) {
      static_assert(kSeqWords == 64, "one word per lane");
      __hip_atomic_store(a.xch + (size_t)b * kSeqWords + lane, 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) __hip_atomic_store(count, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The split form's exchange after a pass over groups [gbeg, gend), whose sums
// this workgroup has published (each word written with a single atomic store
// at device scope, coherent across the XCDs' L2s, by the wave that summed the
// group). Wave 0 reads the other groups' words, one word per lane, keeping four
// loads of each in flight until every word carries this pass's number: a
// reader that sees the pass number sees the value, so no fence or counter is
// needed. The values go to sG (and sGQ). A word holds the value of the pass
// its number names (every writer computes the same value), so a workgroup that
// reads a word another one has already reused for a later pass only sees a
// number that is not its pass's and keeps waiting, then sums the row itself.
// Every word is zero when a call starts: the last workgroup of a sequence to
// finish clears the sequence's words (seq_done). Returns false (in every
// thread) if the wait ran out.
__device__ bool exchange_groups(const unsigned long long* words, unsigned long long tag,
                                int gbeg, int gend, bool with_q, float* sG, float* sGQ) {
  int missing = 0;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int g = lane & (kGroups - 1);
    const bool isq = lane >= kGroups;
    const bool wanted = lane < 2 * kGroups && (!isq || with_q) && (g < gbeg || g >= gend);
    // every lane reads a word of the sequence (lanes that want none ignore it)
    const unsigned long long* src = words + (isq ? kGroups : 0) + g;
    auto load = [&]() {
      return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    bool got = !wanted;
    unsigned val = 0u;
    unsigned long long w[4] = {load(), load(), load(), load()};
    // one returned read: keep it if it is this pass's, and issue the next read
    // into its register (the scheduling barrier keeps each read's wait and
    // reissue in place, so four reads stay in flight); true once every lane
    // has its word
    auto take = [&](unsigned long long& x) {
      const bool hit = !got && (x & ~0xffffffffull) == tag;
      val = hit ? (unsigned)x : val;
      got = got || hit;
      x = load();
      __builtin_amdgcn_sched_barrier(0);
      return __ballot(!got) == 0ull;
    };
    // (sixteen reads per loop trip: only the first waits for all four)
    bool done = false;
    for (unsigned reads = 0; reads < kPatience && !done; reads += 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (take(w[i & 3])) {
          done = true;
          break;
        }
      }
    }
    if (wanted && got) (isq ? sGQ : sG)[g] = __builtin_bit_cast(float, val);
    missing = !got;
  }
  return !__syncthreads_or(missing);
}

// One workgroup per sequence (kSplit false), or a.splits workgroups per
// sequence (a divisor of kGroups), workgroup i taking part i % splits of
// sequence i / splits and with it groups [part, part + 1) * kGroups / splits:
// every workgroup of a sequence takes the same decisions (from the same sums in
// the same order), and a pass over a node's rows is divided among them by
// groups of tiles.
template <bool kSplit>
__global__ __launch_bounds__(kSplit ? kSplitThreads : kSampleThreads) void accept_sampling_kernel(
    const AcceptSampleArgs a) {
  constexpr int NWV = (kSplit ? kSplitThreads : kSampleThreads) / 64;   // waves
  __shared__ int sPar[64];
  __shared__ int sTok[64];
  __shared__ int sRem[64];              // rejected tokens of the current node
  __shared__ float sRemP[64], sRemQ[64];  // their p and q
  __shared__ float sLam[65], sU[65];      // lam_k, U_k
  __shared__ float sQscale[65];           // s_k
  __shared__ int sReady;                  // the last pass's sums are p_k's numerators
  __shared__ float sPX[64], sQX[64], sUX[64];   // candidates: p(x), q(x), uniform
  __shared__ float sTile[kMaxTiles];
  __shared__ float sQ[kMaxTiles];
  __shared__ float sG[kGroups], sGQ[kGroups];   // group sums of sTile, sQ
  __shared__ int sInfo[3];              // status, lo, n

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
    // every candidate's p(x) and q(x) from its parent's rows, and its
    // uniform, one lane per node, all in the walk's first round trip (a node
    // has one parent, so this is each value the walk can ask for)
    if (st == GDN_TREE_OK && lane >= 1 && lane < tl.n) {
      const size_t at = (size_t)(tl.lo + tl.parent) * a.V + tok;
      sPX[lane] = a.p[at];
      sQX[lane] = a.q[at];
      sUX[lane] = a.u[2 * (size_t)(tl.lo + lane)];
    }
  }
  if (tid == 0) {
    sLam[0] = 0.f;
    sU[0] = 1.f;
    sQscale[0] = 1.f;
  }
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
  const int gbeg = part * (kGroups / S), gend = gbeg + kGroups / S;
  unsigned nsync = 0;                   // passes exchanged (split form)
  // The group sums of groups [g0, g1) from sTile (sQ) into sG (sGQ), wave w
  // taking groups g0 + w, g0 + w + waves, ...; with `words`, each is published
  // as soon as it is summed.
  auto group_sums = [&](int g0, int g1, bool with_q, unsigned long long* words,
                        unsigned long long tag) {
    for (int g = g0 + wave; g < g1; g += NWV) {
      const int t0 = group_begin(g, ntiles), t1 = group_begin(g + 1, ntiles);
      const float gs = wave_tiles_sum(sTile, t0, t1);
      const float gq = with_q ? wave_tiles_sum(sQ, t0, t1) : 0.f;
      if (lane == 0) {
        sG[g] = gs;
        if (with_q) sGQ[g] = gq;
        if (words != nullptr) {
          __hip_atomic_store(words + g, tag | __builtin_bit_cast(unsigned, gs), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          if (with_q)
            __hip_atomic_store(words + kGroups + g, tag | __builtin_bit_cast(unsigned, gq),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  // A pass over this workgroup's groups summing max(0, p - lam q) (with_q: and
  // q; need_q false: p alone, lam = 0), each tile holding a token rejected
  // earlier at the node corrected for it; then every group's sums in sG (sGQ):
  // from the others' words, or, if they do not come, from a second pass here
  // over every tile (the same call site, so the pass is inlined once).
  constexpr int RW = kSplit ? kSplitTilesInFlight : kTilesInFlight;
  auto pass_all = [&](const float* prow, const float* qrow, float lam, bool need_q, bool with_q,
                      const Stages& st) {
    int g0 = gbeg, g1 = gend;
    for (;;) {
      const int t0 = group_begin(g0, ntiles), t1 = group_begin(g1, ntiles);
      if (with_q)
        tile_pass<true, true, RW, NWV>(prow, qrow, V, t0, t1, lam, sTile, sQ);
      else if (need_q)
        tile_pass<false, true, RW, NWV>(prow, qrow, V, t0, t1, lam, sTile, sQ);
      else
        tile_pass<false, false, RW, NWV>(prow, qrow, V, t0, t1, 0.f, sTile, sQ);
      __syncthreads();                  // the pass's tile sums are in LDS
      if (st.k > 0) {
        // a token rejected at stage m keeps lam_{m+1}: its term in its tile
        // is replaced (once, at its first rejection)
        if (tid == 0) {
          for (int m = 0; m < st.k; ++m) {
            const int x = st.rem[m];
            const int t = x / kTile;
            if (t < t0 || t >= t1 || rejected_at(x, st.rem, m) >= 0) continue;
            const float px = sRemP[m], qx = sRemQ[m];
            sTile[t] += fmaxf(fmaf(-st.lam[m + 1], qx, px), 0.f) - fmaxf(fmaf(-lam, qx, px), 0.f);
          }
        }
        __syncthreads();
      }
      const bool whole = !kSplit || (g0 == 0 && g1 == kGroups);
      unsigned long long* words = whole ? nullptr : xch_words(a, b, nsync);
      const unsigned long long tag = (unsigned long long)(nsync + 1u) << 32;
      group_sums(g0, g1, with_q, words, tag);
      if (whole) {
        __syncthreads();
        return;
      }
      ++nsync;
      if (exchange_groups(words, tag, g0, g1, with_q, sG, sGQ)) return;
      g0 = 0;
      g1 = kGroups;
    }
  };
  int cur = 0, len = 1;
  for (;;) {
    const float* __restrict__ prow = a.p + (size_t)(lo + cur) * V;
    const float* __restrict__ qrow = a.q + (size_t)(lo + cur) * V;
    Stages s{0, sRem, sLam, sQscale, 1.f};
    float qtot = 0.f, qrem = 0.f;
    bool tiles_ready = false;             // sTile, sG hold the numerators of the current p
    int next = -1;
    for (int c = cur + 1; c < n; ++c) {   // children have larger indices, in node order
      if (sPar[c] != cur) continue;       // uniform
      const int x = sTok[c];
      // (every thread takes the decision alike, from the same values)
      const float2 pq = stage_pq(sPX[c], sQX[c], x, s);
      const bool take = sUX[c] * pq.y < pq.x / s.u;
      if (take) {
        next = c;
        break;
      }
      // rejected: the residual's numerators max(0, p - lam' q), tile by tile,
      // and their total U' (the first pass at a node also sums the row's q
      // mass)
      const float lam = uniform_f(s.lam[s.k] + s.qscale[s.k] * s.u);
      pass_all(prow, qrow, lam, true, s.k == 0, s);
      if (wave == 0) {
        const float u2 = groups_total(sG);
        if (s.k == 0) qtot = groups_total(sGQ);
        // (a token drawn twice has left q already)
        if (rejected_at(x, sRem, s.k) < 0) qrem += sQX[c];
        if (lane == 0) {
          sRem[s.k] = x;
          sRemP[s.k] = sPX[c];
          sRemQ[s.k] = sQX[c];
          sLam[s.k + 1] = u2 > 0.f ? lam : sLam[s.k];
          sU[s.k + 1] = u2 > 0.f ? u2 : s.u;
          sReady = u2 > 0.f;              // else p is unchanged and has no tile sums here
          const float left = qtot - qrem;
          sQscale[s.k + 1] = left > 0.f ? 1.f / left : 1.f;
        }
      }
      __syncthreads();
      tiles_ready = sReady != 0;
      s.k += 1;
      s.u = uniform_f(sU[s.k]);
    }
    if (next >= 0) {
      cur = next;
      ++len;
      continue;
    }
    // final draw from p_k: the tile sums of its numerators (from the last
    // rejection's pass, or from one pass over the rows), scaled by 1 / U_k;
    // the group where the cumulative mass crosses u times the total, then (by
    // the workgroup that summed that group, whose tile sums it holds) the
    // tile, then the token in it
    if (!tiles_ready) {
      const float lam = uniform_f(s.lam[s.k]);
      pass_all(prow, qrow, lam, lam != 0.f, false, s);
    }
    const float scale = 1.f / s.u;
    if (wave != 0) break;
    const float gv = lane < kGroups ? sG[lane] * scale : 0.f;
    float gincl = gv;
#pragma unroll
    for (int off = 1; off < kGroups; off <<= 1) {
      const float y = __shfl_up(gincl, off, kWave);
      if (lane >= off) gincl += y;
    }
    const float total = __shfl(gincl, kGroups - 1, kWave);
    const float target = a.u[2 * (size_t)(lo + cur) + 1] * total;
    const uint64_t gover = __ballot(lane < kGroups && gincl > target);
    const int G = gover ? __builtin_ctzll(gover) : kGroups - 1;
    if (G < gbeg || G >= gend) break;     // another workgroup's group (uniform)
    const float before_g = __shfl(gincl - gv, G, kWave);
    // the tile: lane l owns the group's tiles [l*per, (l+1)*per)
    const int gt0 = group_begin(G, ntiles), gt1 = group_begin(G + 1, ntiles);
    const int per = (gt1 - gt0 + 63) / 64;
    const int t0 = min(gt0 + lane * per, gt1), t1 = min(t0 + per, gt1);
    float ls = 0.f;
    for (int t = t0; t < t1; ++t) ls += sTile[t] * scale;
    float incl = ls;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    incl += before_g;
    const uint64_t over = __ballot(incl > target && t1 > t0);
    const int L = over ? __builtin_ctzll(over) : 63;
    // lane L walks its block: the crossing tile and the mass before it (with
    // no crossing, the group's last tile and the mass through it)
    int tile = gt1 - 1;
    float before = incl;
    if (lane == L) {
      float run = incl - ls;
      tile = t1 > t0 ? t1 - 1 : gt1 - 1;
      before = run;
      for (int t = t0; t < t1; ++t) {
        if (run + sTile[t] * scale > target) {
          tile = t;
          before = run;
          break;
        }
        run += sTile[t] * scale;
        before = run;
      }
    }
    tile = __shfl(tile, L, kWave);
    before = __shfl(before, L, kWave);
    // the token: the first whose cumulative mass exceeds the target (with
    // none, the tile's last token)
    const int j0 = tile * kTile + 4 * lane;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (j0 < V) {
      const float4 p4 = *reinterpret_cast<const float4*>(prow + j0);
      const float4 q4 = *reinterpret_cast<const float4*>(qrow + j0);
      v[0] = stage_pq(p4.x, q4.x, j0, s).x * scale;
      v[1] = stage_pq(p4.y, q4.y, j0 + 1, s).x * scale;
      v[2] = stage_pq(p4.z, q4.z, j0 + 2, s).x * scale;
      v[3] = stage_pq(p4.w, q4.w, j0 + 3, s).x * scale;
    }
    const float vs = v[0] + v[1] + v[2] + v[3];
    float vincl = vs;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(vincl, off, kWave);
      if (lane >= off) vincl += y;
    }
    float run = before + vincl - vs;
    int hit = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      run += v[e];
      if (hit < 0 && j0 + e < V && run > target) hit = j0 + e;
    }
    const uint64_t any = __ballot(hit >= 0);
    const int first = any ? __builtin_ctzll(any) : -1;
    const int hit_first = __shfl(hit, first < 0 ? 0 : first, kWave);
    if (lane == 0) a.next_token[b] = first >= 0 ? hit_first : min(tile * kTile + kTile, V) - 1;
    break;
  }
  // (next_token is written by the workgroup that drew it)
  if (part == 0 && tid == 0) {
    a.status[b] = GDN_TREE_OK;
    a.accepted[b] = cur;
    a.accept_len[b] = len;
  }
  if constexpr (kSplit) seq_done(a, b);
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
          kSplitThreads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

hipError_t launch_accept_sampling_split(const AcceptSampleArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&accept_sampling_kernel<true>),
                       (unsigned)(a.B * a.splits), (unsigned)kSplitThreads, s, a);
}

hipError_t launch_accept_greedy(const AcceptArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&accept_greedy_kernel),
                       (unsigned)((a.B + 3) / 4), 256u, s, a);
}

}  // namespace gdn
