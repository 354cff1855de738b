// wy_verify.hip -- tree-WY verification of one GDN layer on gfx950.
//
// One workgroup (8 waves) per (sequence b, head h). With A(t) = t and its
// ancestors, G_t = prod_{j in A(t)} alpha_j, the gated delta rule along every
// root-to-node path is rewritten (TreeWY abstract, arxivdaily 2608.20961:
// one triangular solve per draft tree, pseudo-values instead of per-node
// states) as
//     (I + A_kk) U = diag(beta) (V - diag(G) K S0^T)
//     O = diag(G) Q S0^T + A_qk U
//     A_kk[t,i] = beta_t (G_t/G_i) k_t.k_i   for i a proper ancestor of t
//     A_qk[t,i] =        (G_t/G_i) q_t.k_i   for i in A(t)
// and every entry outside the ancestor relation is an exact zero (select, not
// multiply), so siblings never see each other (fork page, section 2 mask;
// section 4 isolation of branches).
//
// Schedule of one workgroup:
//  1. issue every global read up front: parents and gates, q, k and v rows
//     (16-byte chunks with consecutive lanes on consecutive chunks, stored to
//     LDS with an XOR swizzle so that MFMA operand reads are bank-conflict
//     free), and this wave's 16 rows of S0 straight into MFMA operand
//     registers.
//  2. wave 0: tree prologue by pointer jumping (ancestor sets, depths, base-2
//     gate prefixes g2 with G_t = 2^g2_t).
//  3. A_kk and A_qk as 16x16 tiles of v_mfma_f32_16x16x32_bf16 over the lower
//     triangle of node tiles, masked and decayed.
//  4. X = K S0^T and Y = Q S0^T on MFMA: S0 is fp32 and is split into bf16
//     hi + lo parts (about 16 significant bits) at bf16 MFMA rate; fp32 io
//     also splits q and k.
//  5. R = diag(beta)(V - diag(G) X) in registers, then the solve level by
//     level (all nodes of one depth at once; a node at depth l has exactly l
//     proper ancestors), each wave on its own dv columns, pseudo-values in LDS,
//     fused with the output o_t = G_t Y_t + sum_{i in A(t)} A_qk[t,i] u_i.
//  6. o (staged in LDS) and U leave as whole contiguous rows (16 bytes per
//     lane), never as the 32-64 byte pieces the MFMA result layout would give.
//
// The same kernel also joins the previous round's commit to this round's
// verify (the fork page's section 7: step 4 of one round, then step 2 of the
// next), so a round reads each state once: once a wave's S0 fragment has
// landed it applies the previous accepted path to it in registers (phase 4b),
// writes the committed fragment out and verifies against it. The path is
// applied either from the previous round's pseudo-values and gate prefixes
// (CommitVerifyLayersArgs: S = G_a S0 + sum_i (G_a/G_i) u_i k_i^T), or by
// replaying the gated delta rule along it from its own k, v, alpha, beta
// (ReplayVerifyLayersArgs), in which case this round writes no U and no g.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split_hi_lo(const float (&f)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)f[e];
    hi[e] = h;
    lo[e] = (__bf16)(f[e] - (float)h);
  }
}

// Staged rows: row-major 16-byte chunks with one spare chunk per row, so that
// 16 lanes on 16 consecutive rows at one chunk index hit disjoint banks and
// every operand address is a per-lane base plus a compile-time offset.
template <int CPR>
__device__ __forceinline__ int chunk_slot(int row, int c) {
  return row * (CPR + 1) + c;
}

// MFMA operand fragment = 8 consecutive k-elements of one staged row
// (k-step s, lane group g = lane/16 -> elements 32s + 8g .. +7).
template <class IO, int CPR> struct Frag;

template <int CPR> struct Frag<uint16_t, CPR> {
  bf16x8 hi;
  __device__ __forceinline__ void load(const uint4* rows, int row, int s, int g) {
    hi = __builtin_bit_cast(bf16x8, rows[chunk_slot<CPR>(row, 4 * s + g)]);
  }
};

template <int CPR> struct Frag<float, CPR> {
  bf16x8 hi, lo;
  __device__ __forceinline__ void load(const uint4* rows, int row, int s, int g) {
    const float4 x = __builtin_bit_cast(float4, rows[chunk_slot<CPR>(row, 8 * s + 2 * g)]);
    const float4 y = __builtin_bit_cast(float4, rows[chunk_slot<CPR>(row, 8 * s + 2 * g + 1)]);
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    split_hi_lo(f, hi, lo);
  }
};

// acc += A * B (bf16: one product; fp32: the four hi/lo cross products).
template <int CPR>
__device__ __forceinline__ f32x4 mma(const Frag<uint16_t, CPR>& a, const Frag<uint16_t, CPR>& b,
                                     f32x4 acc) {
  return mfma16(a.hi, b.hi, acc);
}
template <int CPR>
__device__ __forceinline__ f32x4 mma(const Frag<float, CPR>& a, const Frag<float, CPR>& b,
                                     f32x4 acc) {
  acc = mfma16(a.hi, b.hi, acc);
  acc = mfma16(a.hi, b.lo, acc);
  acc = mfma16(a.lo, b.hi, acc);
  return mfma16(a.lo, b.lo, acc);
}
// Staged fragment times S0 fragment (hi, lo): result rows = nodes, columns = dv.
template <int CPR>
__device__ __forceinline__ f32x4 mma_state_t(const Frag<uint16_t, CPR>& a, const bf16x8& shi,
                                             const bf16x8& slo, f32x4 acc) {
  acc = mfma16(a.hi, shi, acc);
  return mfma16(a.hi, slo, acc);
}
template <int CPR>
__device__ __forceinline__ f32x4 mma_state_t(const Frag<float, CPR>& a, const bf16x8& shi,
                                             const bf16x8& slo, f32x4 acc) {
  acc = mfma16(a.hi, shi, acc);
  acc = mfma16(a.lo, shi, acc);
  acc = mfma16(a.hi, slo, acc);
  return mfma16(a.lo, slo, acc);
}

// 2^x with the hardware transcendental (about 1 ulp; results below the
// smallest normal flush to 0, far below fp32 resolution of any sum here).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 hi | lo packed in one 32-bit word (hi in the low half)
__device__ __forceinline__ uint32_t pack_hi_lo(float x) {
  const __bf16 h = (__bf16)x;
  const __bf16 l = (__bf16)(x - (float)h);
  return (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
}
// four packed words -> bf16x4 hi and bf16x4 lo
__device__ __forceinline__ void unpack_hi_lo(const uint4& w, bf16x4& hi, bf16x4& lo) {
  const uint32_t h01 = __builtin_amdgcn_perm(w.y, w.x, 0x05040100u);
  const uint32_t h23 = __builtin_amdgcn_perm(w.w, w.z, 0x05040100u);
  const uint32_t l01 = __builtin_amdgcn_perm(w.y, w.x, 0x07060302u);
  const uint32_t l23 = __builtin_amdgcn_perm(w.w, w.z, 0x07060302u);
  hi = __builtin_bit_cast(bf16x4, make_uint2(h01, h23));
  lo = __builtin_bit_cast(bf16x4, make_uint2(l01, l23));
}

// 16x16x16 bf16 MFMA: A lane l holds A[l%16][4(l/16)..+3], B lane l holds
// B[4(l/16)..+3][l%16]; the result lane l holds D[4(l/16)..+3][l%16], so a
// result tile is directly the B operand of the next product.
__device__ __forceinline__ f32x4 mfma16k(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split4(const f32x4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// acc += A * B with both operands carried as bf16 hi + lo (the lo*lo term is
// below fp32 resolution of the sum and is dropped).
__device__ __forceinline__ f32x4 mma3(const bf16x4& ah, const bf16x4& al, const bf16x4& bh,
                                      const bf16x4& bl, f32x4 acc) {
  acc = mfma16k(ah, bh, acc);
  acc = mfma16k(ah, bl, acc);
  return mfma16k(al, bh, acc);
}

constexpr int kVerifyWaves = 8;

// Row t of T = (I + A_kk)^-1 for a node whose path p_0 (root) .. p_d = t has
// at most P nodes. Row t is nonzero only on that path, where it is the last
// row of the inverse of the path's own unit-lower block: y_t = 1 and, from the
// deepest proper ancestor up to the root, y_j = -sum_{i on the path below j}
// y_i A_kk[i,j]. Every A_kk entry of the path is loaded at once, then the
// substitution runs in registers; the path entries are written into the
// (zeroed) row as packed bf16 hi|lo words, the form U = T R consumes.
template <int P, int TTS>
__device__ __forceinline__ void t_row_in_registers(uint64_t anc, int d, const float* sAkk,
                                                   float* Tbase) {
  int p[P];
  uint64_t m = anc;
#pragma unroll
  for (int s2 = 0; s2 < P; ++s2) {
    p[s2] = m ? __builtin_ctzll(m) : 0;
    m &= m - 1;
  }
  float akk[P][P];
#pragma unroll
  for (int s2 = 1; s2 < P; ++s2)
#pragma unroll
    for (int r2 = 0; r2 < s2; ++r2)
      akk[s2][r2] = s2 <= d ? sAkk[p[s2] * (p[s2] + 1) / 2 + p[r2]] : 0.f;
  float y[P];
#pragma unroll
  for (int s2 = 0; s2 < P; ++s2) y[s2] = s2 == d ? 1.f : 0.f;
#pragma unroll
  for (int r2 = P - 2; r2 >= 0; --r2) {
    if (r2 < d) {
      float acc = 0.f;
#pragma unroll
      for (int s2 = r2 + 1; s2 < P; ++s2) acc += y[s2] * akk[s2][r2];
      y[r2] = -acc;
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < P; ++s2)
    if (s2 <= d)
      *reinterpret_cast<uint32_t*>(Tbase + (p[s2] >> 4) * TTS + (p[s2] & 15)) = pack_hi_lo(y[s2]);
}

// Path rows of the previous round staged at once when its commit is fused
// into this verify (longer paths are applied in rounds of this many).
constexpr int kFusedPathRows = 4;
template <class Args>
constexpr bool replay_args() {
  return std::is_same<Args, ReplayVerifyLayersArgs>::value;
}
template <class Args>
constexpr bool fused_args() {
  return std::is_same<Args, CommitVerifyLayersArgs>::value || replay_args<Args>();
}

// LDS bytes of one workgroup with the v staging rows unpadded (the layout
// declared in the kernel below).
template <class IO, int DK, int DV, int MT, bool kFused>
constexpr int verify_lds_bytes() {
  constexpr int NP = MT * 16, EPC = 16 / (int)sizeof(IO), CPR = DK / EPC, CPV = DV / EPC;
  constexpr int st1 = 16 * (2 * NP * (CPR + 1) + NP * CPV);
  constexpr int st2 = NP * DV * (4 + (int)sizeof(IO));
  constexpr int nqt = MT * (MT + 1) / 2;
  constexpr int path = kFused ? kFusedPathRows * (4 * DK + 4 * DV) : 0;
  return (st1 > st2 ? st1 : st2) + 4 * (NP * (NP + 1) / 2) + 4 * 256 * nqt +
         (int)sizeof(IO) * 256 * nqt + 16 * NP + path;
}
// Three workgroups per CU (6 waves per SIMD, at most 80 VGPRs, the v rows
// staged unpadded) where the LDS allows three; else the default register
// budget and padded v rows, which read faster at the same occupancy.
template <class IO, int DK, int DV, int MT, bool kFused>
constexpr bool verify_three_per_cu() {
  return verify_lds_bytes<IO, DK, DV, MT, kFused>() <= 52 * 1024;
}
template <class IO, int DK, int DV, int MT, bool kFused>
constexpr int verify_waves_per_simd() {
  // (the fused kernel with 128-wide rows needs about 100 VGPRs: no cap)
  return verify_three_per_cu<IO, DK, DV, MT, kFused>() && !(kFused && DK == 128) ? 6 : 1;
}

// One 16-byte io chunk (8 bf16 or 4 fp32 values) widened to fp32 at dst.
template <class IO>
__device__ __forceinline__ void widen_chunk(const uint4& c, float* dst) {
  if constexpr (std::is_same<IO, float>::value) {
    *reinterpret_cast<float4*>(dst) = __builtin_bit_cast(float4, c);
  } else {
    *reinterpret_cast<float4*>(dst) =
        make_float4(bf16_bits_to_float(c.x & 0xffffu), bf16_bits_to_float(c.x >> 16),
                    bf16_bits_to_float(c.y & 0xffffu), bf16_bits_to_float(c.y >> 16));
    *reinterpret_cast<float4*>(dst + 4) =
        make_float4(bf16_bits_to_float(c.z & 0xffffu), bf16_bits_to_float(c.z >> 16),
                    bf16_bits_to_float(c.w & 0xffffu), bf16_bits_to_float(c.w >> 16));
  }
}

// Rank p (0 = the root) of a path given as a node bit set: its p-th lowest bit.
__device__ __forceinline__ int nth_path_node(uint64_t path, int p) {
  for (int j = 0; j < p; ++j) path &= path - 1ull;
  return path ? __builtin_ctzll(path) : 0;
}

// The previous round's side of a fused round boundary, one lane per previous
// node: the node range and accepted node (uniform), the lane's parent and
// either its gates (replay) or its base-2 gate prefix (pseudo-values).
struct PrevLane {
  int lo, n, acc, size_status;
  int par_raw;
  float g2_raw, alpha, beta;
};

// The previous round's node range and accepted node (scalar loads). Loaded
// together with this round's node range, so that the previous tree's
// per-node loads need no further round trip to memory.
struct PrevHead {
  int lo_r, hi_r, acc;
};
__device__ __forceinline__ PrevHead load_prev_head(const PendingTree& pt, int b) {
  return PrevHead{pt.offsets[b], pt.offsets[b + 1], pt.accepted[b]};
}

template <bool kReplay>
__device__ __forceinline__ PrevLane load_prev(const PendingTree& pt, const PendingLayer& pl,
                                              const PrevHead& ph, int h, int H, int lane) {
  PrevLane p;
  p.g2_raw = 0.f;
  p.alpha = 1.f;
  p.beta = 0.f;
  p.acc = ph.acc;
  // (selects, not branches: the per-node loads below follow without a wait)
  const bool bad = ph.lo_r < 0 || ph.hi_r > pt.T || ph.hi_r - ph.lo_r < 1 ||
                   ph.hi_r - ph.lo_r > pt.max_nodes;
  p.size_status = bad ? GDN_TREE_BAD_SIZE : GDN_TREE_OK;
  p.lo = bad ? 0 : ph.lo_r;
  p.n = bad ? 1 : ph.hi_r - ph.lo_r;
  const int nl = lane < p.n ? lane : 0;
  p.par_raw = pt.parents[p.lo + nl];
  const size_t gl = (size_t)(p.lo + nl) * H + h;
  if constexpr (kReplay) {
    p.alpha = pl.alpha[gl];
    p.beta = pl.beta[gl];
  } else {
    p.g2_raw = pl.g2[gl];
  }
  return p;
}

// Checks of the previous round before its commit (uniform result): nothing
// is checked for accepted == -1; otherwise the previous tree (size, root,
// parents) and then the accepted index.
__device__ __forceinline__ int prev_status(const PrevLane& p, int lane) {
  if (p.acc == -1) return GDN_TREE_OK;
  int ps = p.size_status;
  const int par = lane < p.n ? p.par_raw : -1;
  if (ps == GDN_TREE_OK) {
    if (__shfl(par, 0, kWave) != -1)
      ps = GDN_TREE_BAD_ROOT;
    else if (__ballot(lane >= 1 && lane < p.n && (par < 0 || par >= lane)) != 0ull)
      ps = GDN_TREE_BAD_PARENT;
    else if (p.acc < -1 || p.acc >= p.n)
      ps = GDN_TREE_BAD_ACCEPTED;
  }
  return __builtin_amdgcn_readfirstlane(ps);
}
// The accepted node's path (root first, as a node set) of a previous tree
// that passed prev_status with accepted >= 0; one full wave.
__device__ __forceinline__ uint64_t prev_path(const PrevLane& p, int lane) {
  uint64_t anc;
  float unused;
  path_scan(lane < p.n ? p.par_raw : -1, lane, p.n, 0.f, anc, unused);
  return shfl_u64(anc, p.acc);
}
// Both: the status, and in `path` the accepted path (0 if none is committed).
__device__ __forceinline__ int check_prev(const PrevLane& p, int lane, uint64_t& path) {
  const int ps = prev_status(p, lane);
  path = (ps == GDN_TREE_OK && p.acc >= 0) ? prev_path(p, lane) : 0ull;
  return ps;
}

// The previous round's commit alone, S0 -> S_out, for a sequence whose own
// tree this round is rejected: the accepted tokens' update is kept all the
// same (fork page, section 5: the state is the last accepted token's). A cold
// path kept small in registers: 16 lanes per state row, DK/16 consecutive
// elements per lane, 32 rows per pass; path rows are read straight from
// memory. Returns the previous round's code.
template <class IO, int DK, int DV, bool kReplay>
__device__ int commit_prev_only(const CommitVerifyLayersArgs& args, const PrevHead& ph, int layer,
                                int h, int bh, const float* __restrict__ S0) {
  constexpr int NT = 64 * kVerifyWaves;
  constexpr int TPR = 16;                     // lanes per state row
  constexpr int CPT = DK / TPR;               // columns per lane
  constexpr int RPP = NT / TPR;               // rows per pass
  static_assert(DV % RPP == 0 && DK % TPR == 0, "rows and columns tile the workgroup");
  using io = io_traits<IO>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int H = args.base.H;
  const PendingLayer& pl = args.P[layer];
  const PrevLane p = load_prev<kReplay>(args.prev, pl, ph, h, H, lane);
  uint64_t path0;
  const int ps = check_prev(p, lane, path0);
  float* __restrict__ S_out = pl.S_out;
  if (ps != GDN_TREE_OK || (p.acc < 0 && S_out == S0)) return ps;
  const IO* __restrict__ pk = static_cast<const IO*>(pl.k);
  const int rr = tid / TPR;
  const int c0 = (tid - rr * TPR) * CPT;
  const float gA = (!kReplay && p.acc >= 0) ? __shfl(p.g2_raw, p.acc, kWave) : 0.f;
  const float GA = (!kReplay && p.acc >= 0) ? exp2f(gA) : 1.f;
  for (int r = rr; r < DV; r += RPP) {
    const size_t base = (size_t)bh * DV * DK + (size_t)r * DK + c0;
    float s[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) s[c] = GA * S0[base + c];
    uint64_t path = path0;
    while (path) {   // root first (a parent's index is below its children's)
      const int j = __builtin_ctzll(path);
      path &= path - 1ull;
      const size_t prow = (size_t)(p.lo + j) * H + h;
      float kk[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) kk[c] = io::load1(pk + prow * DK + c0 + c);
      if constexpr (kReplay) {
        const float al = __shfl(p.alpha, j, kWave);
        const float be = __shfl(p.beta, j, kWave);
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) dot += s[c] * kk[c];
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, kWave);
        const float vr = io::load1(static_cast<const IO*>(pl.v) + prow * DV + r);
        const float cf = be * (vr - al * dot);
#pragma unroll
        for (int c = 0; c < CPT; ++c) s[c] = al * s[c] + cf * kk[c];
      } else {
        const float w = exp2f(gA - __shfl(p.g2_raw, j, kWave)) * pl.U[prow * DV + r];
#pragma unroll
        for (int c = 0; c < CPT; ++c) s[c] += w * kk[c];
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) S_out[base + c] = s[c];
  }
  return ps;
}

// Args: VerifyArgs (one layer) or VerifyLayersArgs (workgroup i takes layer
// i / (B * H) of a layer-batched launch), or CommitVerifyLayersArgs (the same,
// with the previous round's commit applied to S0 first).
template <class IO, int DK, int DV, int MT, class Args>
__global__ __launch_bounds__(64 * kVerifyWaves,
                             (verify_waves_per_simd<IO, DK, DV, MT, fused_args<Args>()>()))
void wy_verify_kernel(const Args args) {
  constexpr int NW = kVerifyWaves;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int NP = MT * 16;                 // padded node rows
  constexpr int KS = DK / 32;                 // 16x16x32 k-steps over dk
  constexpr int DVT = DV / 16;                // 16-column tiles of dv; wave w owns tile w
  constexpr int EPC = 16 / (int)sizeof(IO);   // io elements per 16-byte chunk
  constexpr int CPR = DK / EPC;               // chunks per q/k row
  constexpr int CPV = DV / EPC;               // chunks per v/o row
  // U and o staging rows are unpadded; column r of node row t is stored at
  // r ^ (16 * ((t >> 2) & 3)) (when dv >= 64), so that the four row groups of
  // an MFMA result tile touch disjoint banks while every 16-byte chunk of a
  // row stays contiguous for the row-wise global loads and stores.
  constexpr int SWZ = DV >= 64 ? 1 : 0;
  // v rows: unpadded with the swizzle above when that buys the third
  // workgroup per CU, else one spare chunk per row (like the k / q rows)
  constexpr bool kVSwz = verify_three_per_cu<IO, DK, DV, MT, fused_args<Args>()>();
  constexpr int kVPad = kVSwz ? 0 : 1;
  constexpr int TTW = 16;                     // row of a stored 16x16 tile
  constexpr int TTS = 16 * TTW;               // stored tile size
  constexpr int NTRI = NP * (NP + 1) / 2;     // packed lower triangle
  constexpr int NQT = MT * (MT + 1) / 2;      // lower-triangular 16x16 node tiles
  constexpr int NSTAGE = NP * (2 * CPR + CPV);  // staged q, k, v chunks
  constexpr int NLD = (NSTAGE + NT - 1) / NT;   // per thread (a spare one repeats the last)
  constexpr bool kF32 = std::is_same<IO, float>::value;
  constexpr bool kFused = fused_args<Args>();
  constexpr bool kReplay = replay_args<Args>();
  constexpr int PCH = kFusedPathRows;
  constexpr int PKC = PCH * CPR;              // io chunks of the staged path k rows
  // then per path row: its scaled pseudo-values (float4), or its v row (io chunks, replay)
  constexpr int SEC = kReplay ? CPV : DV / 4;
  constexpr int PUC = PCH * SEC;
  using io = io_traits<IO>;
  static_assert(DVT <= NW, "one 16-column dv tile per wave");
  static_assert(PKC + PUC <= NT, "one staged path piece per thread");

  struct Stage1 {             // until the state products are done
    uint4 k[NP * (CPR + 1)];
    uint4 q[NP * (CPR + 1)];
    uint4 v[NP * (CPV + kVPad)];
  };
  struct Stage2 {             // products with T and A_qk, output staging
    float u[NP * DV];
    IO o[NP * DV];
  };
  union SMem {
    Stage1 s1;
    Stage2 s2;
  };
  __shared__ SMem sm;
  __shared__ float sAkk[NTRI];
  // T (fp32 while it is computed, then packed bf16 hi|lo words) and A_qk as
  // their lower-triangular 16x16 node tiles (mi, ki), ki <= mi,
  // tile qt = mi(mi+1)/2 + ki, unpadded 16x16 (the few operand reads take a
  // 4-way bank conflict; the bytes saved keep three 48-node workgroups per
  // CU within the LDS). A_qk is kept in io
  // precision for bf16 io (its product with U is rounded to bf16 anyway) and
  // as fp32 for fp32 io.
  using AqT = typename std::conditional<std::is_same<IO, float>::value, float, __bf16>::type;
  __shared__ __align__(16) float sT[NQT * TTS];
  __shared__ __align__(16) AqT sAqk[NQT * TTS];
  __shared__ uint64_t sAnc[NP];
  __shared__ uint64_t sPath[1];   // (fused) the accepted path of the previous round
  __shared__ float sG2[NP];
  __shared__ float sBeta[NP];
  // previous round's path (fused commit): k rows widened to fp32 once here
  // (every lane reads 32 of them per path row), and the pseudo-values scaled
  // by their path coefficients, or (replay) the v rows as io
  __shared__ __align__(16) float sPK[kFused ? PCH * DK : 4];
  __shared__ __align__(16) float sPW[kFused ? PCH * DV : 4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;      // lane group of an MFMA operand / result
  const int l16 = lane & 15;
  // ---- 0. The prologue's scalar loads go out in two batches, each in full
  // before its one wait (an empty asm statement takes the batch's values as
  // operands; it has no side effects, so the loads stay scalar): the kernel
  // arguments that locate the workgroup's sequence, then the layer's
  // pointers together with the node ranges. Step 1 then issues every
  // per-node load. Left alone, the compiler loads each field next to its
  // first use: about eight dependent round trips before the first row is
  // requested, each a memory latency when the scalar cache is cold.
  int nB = base_args(args).B;
  if constexpr (kFused)
    asm("" : "+s"(nB) : "s"(base_args(args).H), "s"(base_args(args).offsets),
        "s"(args.prev.offsets), "s"(args.prev.accepted));
  else
    asm("" : "+s"(nB) : "s"(base_args(args).H), "s"(base_args(args).offsets));
  const int nbh = nB * base_args(args).H;
  const int layer = blockIdx.x / nbh;
  const VerifyArgs a = layer_args(args, layer);
  const int bh = blockIdx.x - layer * nbh;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const IO* __restrict__ q = static_cast<const IO*>(a.q);
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  const IO* __restrict__ v = static_cast<const IO*>(a.v);
  IO* __restrict__ o = static_cast<IO*>(a.o);

  // ---- node range, and (fused) the previous round's (uniform, scalar loads)
  int lo = a.offsets[b];
  const int hi = a.offsets[b + 1];
  PrevHead phd{0, 1, -1};
  if constexpr (kFused) {
    phd = load_prev_head(args.prev, b);
    const PendingLayer& pl = args.P[layer];
    asm("" : "+s"(lo) : "s"(hi), "s"(phd.lo_r), "s"(phd.hi_r), "s"(phd.acc), "s"(a.T),
        "s"(a.max_nodes), "s"(a.parents), "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.alpha),
        "s"(a.beta), "s"(args.prev.T), "s"(args.prev.max_nodes), "s"(args.prev.parents),
        "s"(kReplay ? pl.alpha : pl.g2), "s"(pl.beta));
  } else {
    asm("" : "+s"(lo) : "s"(hi), "s"(a.T), "s"(a.max_nodes), "s"(a.parents), "s"(a.q),
        "s"(a.k), "s"(a.v), "s"(a.alpha), "s"(a.beta));
  }
  if (lo < 0 || hi > a.T || hi - lo < 1 || hi - lo > a.max_nodes) {
    // (fused) the previous round's commit is applied all the same
    int code = GDN_TREE_BAD_SIZE;
    if constexpr (kFused) {
      const int pcode = commit_prev_only<IO, DK, DV, kReplay>(args, phd, layer, h, bh, a.S0);
      code |= GDN_TREE_PREV(pcode);
    }
    if (h == 0 && tid == 0) put_status(a.status, b, code, a.merge);
    return;
  }
  const int n = hi - lo;
  const int mt = (n + 15) >> 4;

  // ---- 1. every global read of the workgroup, issued before any is used
  // (addresses clamped into the sequence, so the issue is unconditional).
  // 1a. parents and gates, one lane per node
  const int nl = lane < n ? lane : 0;
  const size_t gl = (size_t)(lo + nl) * H + h;
  const int par_raw = a.parents[lo + nl];
  const float alpha_l = a.alpha[gl];
  const float beta_raw = a.beta[gl];
  // 1b. k, q and v rows in 16-byte chunks, consecutive lanes on consecutive
  // chunks of a row. Rows past the last node repeat row n-1: finite values
  // whose products land only in results that are never used.
  uint4 stg[NLD];
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int idx = min(tid + NT * it, NSTAGE - 1);
    const int mat = idx < NP * CPR ? 0 : (idx < 2 * NP * CPR ? 1 : 2);
    const int rel = idx - mat * NP * CPR;
    const int cpr = mat == 2 ? CPV : CPR;
    const int row = rel / cpr;
    const int c = rel - row * cpr;
    const int srow = row < n ? row : n - 1;
    const IO* base = mat == 0 ? k : (mat == 1 ? q : v);
    const int dd = mat == 2 ? DV : DK;
    stg[it] = *reinterpret_cast<const uint4*>(base + ((size_t)(lo + srow) * H + h) * dd + c * EPC);
  }
  // 1c. (fused commit) the previous round's node range and accepted node,
  // and one lane per previous node: its parent and gate prefix (or gates).
  // Issued after the rows: nothing waits on these loads before the rows are
  // in flight.
  PrevLane prv{0, 1, -1, GDN_TREE_OK, -1, 0.f, 1.f, 0.f};
  const IO* __restrict__ pk = nullptr;
  const IO* __restrict__ pv = nullptr;
  const float* __restrict__ pU = nullptr;
  float* __restrict__ S_out = nullptr;
  if constexpr (kFused) {
    const PendingLayer& pl = args.P[layer];
    pk = static_cast<const IO*>(pl.k);
    pv = static_cast<const IO*>(pl.v);
    pU = pl.U;
    S_out = pl.S_out;
    prv = load_prev<kReplay>(args.prev, pl, phd, h, H, lane);
  }
  const int plo = prv.lo, pacc = prv.acc;
  const float pg2_raw = prv.g2_raw, palpha = prv.alpha, pbeta = prv.beta;
  const bool owns = wave < DVT;                 // dv < 128: the last waves own no columns
  const int jt = owns ? wave : DVT - 1;

  float4 sraw[KS][2];
  auto load_S0 = [&]() {
    const float* rowp = a.S0 + (size_t)bh * DV * DK + (size_t)(16 * jt + l16) * DK + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sraw[s][0] = *reinterpret_cast<const float4*>(rowp + 32 * s);
      sraw[s][1] = *reinterpret_cast<const float4*>(rowp + 32 * s + 4);
    }
  };
  // (fused from pseudo-values) odd workgroups take the state first, even ones
  // after their rows, so that the two workgroups of a CU do not load in step;
  // the replay kernel, which writes less at its end, does best with all late
  const bool early_S0 = kFused && !kReplay && (blockIdx.x & 1);
  if (early_S0) load_S0();
  // ---- 2. staged chunks to LDS (swizzled), then the tree prologue, computed
  // by every wave so that no branch separates the loads from their first use.
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int idx = min(tid + NT * it, NSTAGE - 1);
    const int mat = idx < NP * CPR ? 0 : (idx < 2 * NP * CPR ? 1 : 2);
    const int rel = idx - mat * NP * CPR;
    if (mat == 2) {
      const int row = rel / CPV;
      if constexpr (kVSwz) {
        const int cs = ((rel - row * CPV) * EPC) ^ (SWZ * 16 * ((row >> 2) & 3));
        *reinterpret_cast<uint4*>(reinterpret_cast<IO*>(sm.s1.v) + row * DV + cs) = stg[it];
      } else {
        sm.s1.v[chunk_slot<CPV>(row, rel - row * CPV)] = stg[it];
      }
    } else {
      const int row = rel / CPR;
      (mat == 0 ? sm.s1.k : sm.s1.q)[chunk_slot<CPR>(row, rel - row * CPR)] = stg[it];
    }
  }
  // The tree checks run in every wave (a shuffle and a ballot each), the
  // scans in wave 0 only: they are chains of LDS shuffles, and eight waves
  // running the same ones slow each other down. (The checks also keep the
  // parent and gate loads ahead of wave 0's branch.)
  const int par = lane < n ? par_raw : -1;
  int st = GDN_TREE_OK;
  if (__shfl(par, 0, kWave) != -1)
    st = GDN_TREE_BAD_ROOT;
  else if (__ballot(lane >= 1 && lane < n && (par < 0 || par >= lane)) != 0ull)
    st = GDN_TREE_BAD_PARENT;
  st = __builtin_amdgcn_readfirstlane(st);
  const float lg = lane < n ? gate_log2(alpha_l) : 0.f;
  int ps = GDN_TREE_OK;   // the previous round's commit (fused)
  if constexpr (kFused) ps = prev_status(prv, lane);
  uint64_t anc = 0ull;
  float g2 = 0.f;
  if (wave == 0) {
    // (on a bad tree the scan still terminates; its results are not used)
    path_scan(par, lane, n, lg, anc, g2);
    if constexpr (kFused) {
      // the accepted node's path, root first (a rejected tree this round:
      // committed on the cold path below)
      const uint64_t pp =
          (st == GDN_TREE_OK && ps == GDN_TREE_OK && pacc >= 0) ? prev_path(prv, lane) : 0ull;
      if (lane == 0) sPath[0] = pp;
    }
    if (lane < NP) {
      sAnc[lane] = anc;
      sG2[lane] = g2;
      sBeta[lane] = lane < n ? beta_raw : 0.f;
    }
  }
  __syncthreads();
  // (fused commit) the path, and its gate prefix and path coefficients
  // 2^(gA - g2_i) (commit from pseudo-values)
  uint64_t ppath = 0ull;
  float pgA = 0.f, pcoef = 0.f;
  if constexpr (kFused) {
    const uint64_t pp = sPath[0];
    ppath = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(pp >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pp);
    if constexpr (!kReplay) {
      if (ppath) {
        pgA = __shfl(pg2_raw, pacc, kWave);
        pcoef = exp2f(pgA - pg2_raw);
      }
    }
  }
  // 1c. this wave's S0 rows 16w + lane%16, columns 32s + 8g .. +7. Issued only
  // now, once the q, k, v rows have arrived: when every resident workgroup
  // loads at once, the rows that the first phases need are not queued behind
  // the state, which then streams in while the node products are computed.
  // 1d. (fused commit) the first PCH path rows: one 16-byte piece per thread
  // (a k chunk, or four pseudo-values), issued before the state so that
  // waiting for them does not wait for the state.
  const int P = kFused ? __popcll(ppath) : 0;
  const int pidx = tid < PKC ? tid / CPR : (tid - PKC) / SEC;
  uint4 pld = make_uint4(0u, 0u, 0u, 0u);
  float pcf = 0.f;
  if constexpr (kFused) {
    const int pnode = nth_path_node(ppath, pidx < P ? pidx : 0);
    pcf = __shfl(pcoef, pnode, kWave);
    if (pidx < P && tid < PKC + PUC) {
      const size_t prow = (size_t)(plo + pnode) * H + h;
      if (tid < PKC)
        pld = *reinterpret_cast<const uint4*>(pk + prow * DK + (tid - pidx * CPR) * EPC);
      else if constexpr (kReplay)
        pld = *reinterpret_cast<const uint4*>(pv + prow * DV + (tid - PKC - pidx * CPV) * EPC);
      else
        pld = *reinterpret_cast<const uint4*>(pU + prow * DV + 4 * (tid - PKC - pidx * (DV / 4)));
    }
  }
  if (!early_S0) load_S0();
  if (st != GDN_TREE_OK || ps != GDN_TREE_OK) {
    // this round's tree, or the previous round's commit, is rejected: zero
    // output rows (and workspace). With only this round's tree rejected, the
    // previous commit is still applied (cold path); a rejected previous
    // commit leaves S_out unwritten and nothing is verified against a state
    // that lacks it.
    for (int idx = tid; idx < n * (DV / 4); idx += NT) {
      const int t = idx / (DV / 4);
      const int r = 4 * (idx - t * (DV / 4));
      const size_t row = ((size_t)(lo + t) * H + h) * DV + r;
      io::store4(o + row, make_float4(0.f, 0.f, 0.f, 0.f));
      if constexpr (!kReplay) *reinterpret_cast<float4*>(a.U + row) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (!kReplay)
      for (int t = tid; t < n; t += NT) a.g2[(size_t)(lo + t) * H + h] = 0.f;
    int code = st;
    if constexpr (kFused) {
      if (st != GDN_TREE_OK && ps == GDN_TREE_OK)
        ps = commit_prev_only<IO, DK, DV, kReplay>(args, phd, layer, h, bh, a.S0);
      code |= GDN_TREE_PREV(ps);
    }
    if (h == 0 && tid == 0) put_status(a.status, b, code, a.merge);
    return;
  }

  // ---- 3. The masked, decayed products over the lower-triangular node tiles,
  // spread over the waves:
  //   A_kk[t,i] = beta_t 2^(g2_t - g2_i) k_t.k_i  (i a proper ancestor of t),
  //     as K K^T: result column i = 16mj + lane%16, rows t = 16mi + 4g + e,
  //     stored packed, entry (t, i) at t(t+1)/2 + i;
  //   A_qk[t,i] = 2^(g2_t - g2_i) q_t.k_i  (i in A(t)),
  //     as K Q^T: lane holds t = 16mi + lane%16, i = 16mj + 4g + e, i.e. the
  //     A-operand layout of the product A_qk U, stored as tile (mi, mj).
  {
    const int ntile = mt * (mt + 1) / 2;
    for (int tt2 = wave; tt2 < 2 * ntile; tt2 += NW) {
      const bool is_qk = tt2 >= ntile;
      const int tt = is_qk ? tt2 - ntile : tt2;
      int mi = 0;
      while ((mi + 1) * (mi + 2) / 2 <= tt) ++mi;
      const int mj = tt - mi * (mi + 1) / 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<IO, CPR> fa, fb;
        fa.load(sm.s1.k, 16 * (is_qk ? mj : mi) + l16, s, g);
        fb.load(is_qk ? sm.s1.q : sm.s1.k, 16 * (is_qk ? mi : mj) + l16, s, g);
        acc = mma(fa, fb, acc);
      }
      if (!is_qk) {
        const int i = 16 * mj + l16;
        const float g2i = sG2[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * mi + 4 * g + e;
          const bool vis = ((sAnc[t] >> i) & 1ull) && i != t;
          const float val = vis ? sBeta[t] * fast_exp2(sG2[t] - g2i) * acc[e] : 0.f;
          if (i <= t) sAkk[t * (t + 1) / 2 + i] = val;
        }
      } else {
        const int t = 16 * mi + l16;
        const uint64_t at = sAnc[t];
        const float g2t = sG2[t];
        AqT* dst = sAqk + tt * TTS + l16 * TTW + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * mj + 4 * g + e;
          const bool vis = (at >> i) & 1ull;
          dst[e] = (AqT)(vis ? fast_exp2(g2t - sG2[i]) * acc[e] : 0.f);
        }
      }
    }
  }
  if constexpr (kFused) {
    if (pidx < P && tid < PKC + PUC) {
      if (tid < PKC) {
        widen_chunk<IO>(pld, sPK + tid * EPC);
      } else if constexpr (kReplay) {
        reinterpret_cast<uint4*>(sPW)[tid - PKC] = pld;
      } else {
        float4 u = __builtin_bit_cast(float4, pld);
        u.x *= pcf;
        u.y *= pcf;
        u.z *= pcf;
        u.w *= pcf;
        reinterpret_cast<float4*>(sPW)[tid - PKC] = u;
      }
    }
  }
  __syncthreads();

  // ---- 4. wave 0: T = (I + A_kk)^-1, one lane per row. Row t is nonzero only
  // on t's path p_0 (root) .. p_d = t, where it is the last row of the inverse
  // of the path's own unit-lower block: y_t = 1 and, from the deepest proper
  // ancestor up to the root, y_j = -sum_{i on the path below j} y_i A_kk[i,j].
  // Rows of padding nodes are zero.
  if (wave == 0 && lane < NP) {
    // row t lives in tiles (t/16, ki), ki <= t/16, at row t%16
    const int t = lane;
    const int mrow = t >> 4;
    float* Tbase = sT + (mrow * (mrow + 1) / 2) * TTS + (t & 15) * TTW;   // tile (mrow, 0)
#pragma unroll
    for (int ki = 0; ki < MT; ++ki)
      if (ki <= mrow)
#pragma unroll
        for (int c = 0; c < 16; c += 4)
          *reinterpret_cast<float4*>(Tbase + ki * TTS + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    // every path of at most 4 nodes (a wave-uniform test): the short solve
    const int d = __popcll(anc) - 1;
    const bool shallow4 = __ballot(t < n && d >= 4) == 0ull;
    if (t < n) {
      if (shallow4) {
        t_row_in_registers<4, TTS>(anc, d, sAkk, Tbase);
      } else if (d < 8) {
        t_row_in_registers<8, TTS>(anc, d, sAkk, Tbase);
      } else {
        // deep paths: the same substitution with the row kept in LDS
        Tbase[(t >> 4) * TTS + (t & 15)] = 1.f;
        uint64_t rest = anc & ~(1ull << t);
        while (rest) {
          const int j = 63 - __builtin_clzll(rest);
          rest &= ~(1ull << j);
          uint64_t below = anc & ~((2ull << j) - 1ull);
          float acc = 0.f;
          while (below) {
            const int i = __builtin_ctzll(below);
            below &= below - 1;
            acc += Tbase[(i >> 4) * TTS + (i & 15)] * sAkk[i * (i + 1) / 2 + j];
          }
          Tbase[(j >> 4) * TTS + (j & 15)] = -acc;
        }
        // the row's nonzero entries (t's path) become packed bf16 hi|lo words,
        // the form the product U = T R consumes
        uint64_t path = anc;
        while (path) {
          const int i = __builtin_ctzll(path);
          path &= path - 1;
          float* e = Tbase + (i >> 4) * TTS + (i & 15);
          *reinterpret_cast<uint32_t*>(e) = pack_hi_lo(*e);
        }
      }
    }
  }

  // ---- 4b. (fused commit) S0 <- G_a S0 + sum over the accepted path of
  // (G_a/G_i) u_i k_i^T on this wave's fragment (row 16w + lane%16, columns
  // 32s + 8g .. +7), written out as the committed state and verified against.
  // Replay instead runs the gated delta rule along the path, root first:
  // w = S k_j, S <- alpha_j S + beta_j (v_j - alpha_j w) k_j^T.
  if constexpr (kFused) {
    const float GA = pacc >= 0 ? exp2f(pgA) : 1.f;
    // (replay) the fragment is carried as S = gam * Shat: a step is then one
    // FMA per element, Shat += (c / gam') k^T with gam' = alpha gam, and gam
    // is applied once at the end (or folded in early, before it underflows)
    float gam = 1.f;
    if (owns && !kReplay) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sraw[s][0].x *= GA; sraw[s][0].y *= GA; sraw[s][0].z *= GA; sraw[s][0].w *= GA;
        sraw[s][1].x *= GA; sraw[s][1].y *= GA; sraw[s][1].z *= GA; sraw[s][1].w *= GA;
      }
    }
    for (int p0 = 0; p0 < P; p0 += PCH) {
      const int pc = P - p0 < PCH ? P - p0 : PCH;
      if (p0 > 0) {
        // a path longer than PCH rows (deep chains): the next rows, staged
        // by the whole workgroup once the previous ones are consumed
        __syncthreads();
        const int pnode = nth_path_node(ppath, p0 + (pidx < pc ? pidx : 0));
        const float cf = __shfl(pcoef, pnode, kWave);
        if (pidx < pc && tid < PKC + PUC) {
          const size_t prow = (size_t)(plo + pnode) * H + h;
          if (tid < PKC) {
            widen_chunk<IO>(
                *reinterpret_cast<const uint4*>(pk + prow * DK + (tid - pidx * CPR) * EPC),
                sPK + tid * EPC);
          } else if constexpr (kReplay) {
            reinterpret_cast<uint4*>(sPW)[tid - PKC] = *reinterpret_cast<const uint4*>(
                pv + prow * DV + (tid - PKC - pidx * CPV) * EPC);
          } else {
            float4 u = *reinterpret_cast<const float4*>(pU + prow * DV +
                                                        4 * (tid - PKC - pidx * (DV / 4)));
            u.x *= cf;
            u.y *= cf;
            u.z *= cf;
            u.w *= cf;
            reinterpret_cast<float4*>(sPW)[tid - PKC] = u;
          }
        }
        __syncthreads();
      }
      if (owns && kReplay) {
        const int r = 16 * jt + l16;
        for (int p = 0; p < pc; ++p) {
          const int node = nth_path_node(ppath, p0 + p);
          const float al = __shfl(palpha, node, kWave);
          const float be = __shfl(pbeta, node, kWave);
          const float* krow = sPK + p * DK + 8 * g;
          float4 kk[KS][2];
          float dot = 0.f;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            kk[s][0] = *reinterpret_cast<const float4*>(krow + 32 * s);
            kk[s][1] = *reinterpret_cast<const float4*>(krow + 32 * s + 4);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              dot += sraw[s][hh].x * kk[s][hh].x + sraw[s][hh].y * kk[s][hh].y +
                     sraw[s][hh].z * kk[s][hh].z + sraw[s][hh].w * kk[s][hh].w;
          }
          // the row's 128 columns are spread over the lanes l16 + 16g
          dot += __shfl_xor(dot, 16, kWave);
          dot += __shfl_xor(dot, 32, kWave);
          const float vr = io::load1(reinterpret_cast<const IO*>(sPW) + p * DV + r);
          const float c = be * (vr - al * (gam * dot));
          const float ng = al * gam;                 // wave-uniform
          if (ng < 0x1p-30f) {
            // fold the product into the fragment before it can underflow
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                sraw[s][hh].x = ng * sraw[s][hh].x + c * kk[s][hh].x;
                sraw[s][hh].y = ng * sraw[s][hh].y + c * kk[s][hh].y;
                sraw[s][hh].z = ng * sraw[s][hh].z + c * kk[s][hh].z;
                sraw[s][hh].w = ng * sraw[s][hh].w + c * kk[s][hh].w;
              }
            }
            gam = 1.f;
          } else {
            const float f = c * (1.f / ng);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                sraw[s][hh].x += f * kk[s][hh].x;
                sraw[s][hh].y += f * kk[s][hh].y;
                sraw[s][hh].z += f * kk[s][hh].z;
                sraw[s][hh].w += f * kk[s][hh].w;
              }
            }
            gam = ng;
          }
        }
      }
      if (owns && !kReplay) {
        const int r = 16 * jt + l16;
        for (int p = 0; p < pc; ++p) {
          const float w = sPW[p * DV + r];
          const float* krow = sPK + p * DK + 8 * g;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const float4 k0 = *reinterpret_cast<const float4*>(krow + 32 * s);
            const float4 k1 = *reinterpret_cast<const float4*>(krow + 32 * s + 4);
            sraw[s][0].x += w * k0.x; sraw[s][0].y += w * k0.y;
            sraw[s][0].z += w * k0.z; sraw[s][0].w += w * k0.w;
            sraw[s][1].x += w * k1.x; sraw[s][1].y += w * k1.y;
            sraw[s][1].z += w * k1.z; sraw[s][1].w += w * k1.w;
          }
        }
      }
    }
    if (owns && kReplay && gam != 1.f) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          sraw[s][hh].x *= gam;
          sraw[s][hh].y *= gam;
          sraw[s][hh].z *= gam;
          sraw[s][hh].w *= gam;
        }
      }
    }
    if (owns && !(pacc < 0 && S_out == a.S0)) {
      float* rowo = S_out + (size_t)bh * DV * DK + (size_t)(16 * jt + l16) * DK + 8 * g;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        *reinterpret_cast<float4*>(rowo + 32 * s) = sraw[s][0];
        *reinterpret_cast<float4*>(rowo + 32 * s + 4) = sraw[s][1];
      }
    }
  }

  // ---- 5. per wave: X = K S0^T and Y = Q S0^T for node tiles m, with the
  // wave's 16 dv columns (A = staged k / q rows, B = S0 hi/lo); result lane
  // holds column r = 16w + lane%16 of nodes t = 16m + 4g + e. Then
  // R = diag(beta)(V - diag(G) X) and G*Y.
  f32x4 rX[MT], rY[MT];
  if (owns) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      rX[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      rY[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4 x0 = sraw[s][0], x1 = sraw[s][1];
      const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 shi, slo;
      split_hi_lo(f, shi, slo);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mt) {
          Frag<IO, CPR> fk, fq;
          fk.load(sm.s1.k, 16 * m + l16, s, g);
          fq.load(sm.s1.q, 16 * m + l16, s, g);
          rX[m] = mma_state_t(fk, shi, slo, rX[m]);
          rY[m] = mma_state_t(fq, shi, slo, rY[m]);
        }
      }
    }
    const int r = 16 * jt + l16;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * m + 4 * g + e;
        const float G = fast_exp2(sG2[t]);
        const float vv =
            kVSwz ? io::load1(reinterpret_cast<const IO*>(sm.s1.v) + t * DV +
                              (r ^ (SWZ * 16 * ((t >> 2) & 3))))
                  : io::load1(reinterpret_cast<const IO*>(sm.s1.v) +
                              chunk_slot<CPV>(t, r / EPC) * EPC + r % EPC);
        rX[m][e] = sBeta[t] * (vv - G * rX[m][e]);
        rY[m][e] = G * rY[m][e];
      }
    }
  }
  __syncthreads();  // T is complete; staged q, k, v are dead (stage 2 reuses the LDS)

  // ---- 6. U = T R and O = G*Y + A_qk U on MFMA (16x16x16, node tiles as the
  // k dimension); U and O leave through LDS staging rows.
  if (owns) {
    bf16x4 rh[MT], rl[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) split4(rX[m], rh[m], rl[m]);
    f32x4 uu[MT];
    bf16x4 uh[MT], ul[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      uu[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m < mt) {
#pragma unroll
        for (int ki = 0; ki <= m; ++ki) {
          const uint4 tw = *reinterpret_cast<const uint4*>(
              sT + (m * (m + 1) / 2 + ki) * TTS + l16 * TTW + 4 * g);
          bf16x4 th, tl;
          unpack_hi_lo(tw, th, tl);
          uu[m] = mma3(th, tl, rh[ki], rl[ki], uu[m]);
        }
      }
      split4(uu[m], uh[m], ul[m]);
    }
    const int r = 16 * jt + l16;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f32x4 oo = rY[m];
      if (m < mt) {
#pragma unroll
        for (int ki = 0; ki <= m; ++ki) {
          const AqT* src = sAqk + (m * (m + 1) / 2 + ki) * TTS + l16 * TTW + 4 * g;
          if constexpr (kF32) {
            const float4 av = *reinterpret_cast<const float4*>(src);
            bf16x4 ah, al;
            split4(f32x4{av.x, av.y, av.z, av.w}, ah, al);
            oo = mma3(ah, al, uh[ki], ul[ki], oo);
          } else {
            const bf16x4 ah = *reinterpret_cast<const bf16x4*>(src);
            oo = mfma16k(ah, uh[ki], oo);
            oo = mfma16k(ah, ul[ki], oo);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * m + 4 * g + e;
        const int rs = r ^ (SWZ * 16 * ((t >> 2) & 3));
        if constexpr (!kReplay) sm.s2.u[t * DV + rs] = uu[m][e];
        io::store1(sm.s2.o + t * DV + rs, oo[e]);
      }
    }
  }
  __syncthreads();

  // ---- 7. o, U and g2 to memory, consecutive lanes on consecutive chunks of a row
  for (int idx = tid; idx < n * CPV; idx += NT) {
    const int t = idx / CPV;
    const int c = idx - t * CPV;
    const int cs = (c * EPC) ^ (SWZ * 16 * ((t >> 2) & 3));
    *reinterpret_cast<uint4*>(o + ((size_t)(lo + t) * H + h) * DV + c * EPC) =
        *reinterpret_cast<const uint4*>(sm.s2.o + t * DV + cs);
  }
  // (replay: the next round replays from this round's inputs; no workspace)
  for (int idx = tid; !kReplay && idx < n * (DV / 4); idx += NT) {
    const int t = idx / (DV / 4);
    const int c = idx - t * (DV / 4);
    const int cs = (4 * c) ^ (SWZ * 16 * ((t >> 2) & 3));
    *reinterpret_cast<float4*>(a.U + ((size_t)(lo + t) * H + h) * DV + 4 * c) =
        *reinterpret_cast<const float4*>(sm.s2.u + t * DV + cs);
  }
  if (!kReplay && wave == 0 && lane < n) a.g2[(size_t)(lo + lane) * H + h] = g2;
  if (h == 0 && tid == 0) put_status(a.status, b, GDN_TREE_OK, a.merge);
}

inline unsigned grid_of(const VerifyArgs& a) { return (unsigned)(a.B * a.H); }
inline unsigned grid_of(const VerifyLayersArgs& a) {
  return (unsigned)(a.base.B * a.base.H * a.layers);
}
inline unsigned grid_of(const CommitVerifyLayersArgs& a) {
  return (unsigned)(a.base.B * a.base.H * a.layers);
}
inline unsigned grid_of(const ReplayVerifyLayersArgs& a) {
  return (unsigned)(a.base.B * a.base.H * a.layers);
}

template <class IO, int D, int MT, class Args>
hipError_t launch_t(const Args& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&wy_verify_kernel<IO, D, D, MT, Args>),
                       grid_of(a), 64u * kVerifyWaves, s, a);
}

template <class IO, int D, class Args>
hipError_t launch_mt(int mt, const Args& a, hipStream_t s) {
  switch (mt) {
    case 1: return launch_t<IO, D, 1>(a, s);
    case 2: return launch_t<IO, D, 2>(a, s);
    case 3: return launch_t<IO, D, 3>(a, s);
    case 4: return launch_t<IO, D, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class IO, class Args>
hipError_t launch_d(int d, int mt, const Args& a, hipStream_t s) {
  switch (d) {
    case 32: return launch_mt<IO, 32>(mt, a, s);
    case 64: return launch_mt<IO, 64>(mt, a, s);
    case 128: return launch_mt<IO, 128>(mt, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_wy_verify(int io, int d, int mt, const VerifyArgs& a, hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t>(d, mt, a, s) : launch_d<float>(d, mt, a, s);
}

hipError_t launch_wy_verify_layers(int io, int d, int mt, const VerifyLayersArgs& a,
                                   hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t>(d, mt, a, s) : launch_d<float>(d, mt, a, s);
}

hipError_t launch_wy_commit_verify_layers(int io, int d, int mt, const CommitVerifyLayersArgs& a,
                                          hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t>(d, mt, a, s) : launch_d<float>(d, mt, a, s);
}

hipError_t launch_wy_replay_verify_layers(int io, int d, int mt, const ReplayVerifyLayersArgs& a,
                                          hipStream_t s) {
  return io == GDN_DTYPE_BF16 ? launch_d<uint16_t>(d, mt, a, s) : launch_d<float>(d, mt, a, s);
}

}  // namespace gdn
