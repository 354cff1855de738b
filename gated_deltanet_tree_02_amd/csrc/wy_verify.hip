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

// Staged rows: row-major 16-byte chunks, chunk c of row r stored at position
// c ^ (r mod chunks-per-row), so that 16 lanes on 16 consecutive rows at one
// chunk index hit 16 different bank groups.
template <int CPR>
__device__ __forceinline__ int chunk_slot(int row, int c) {
  return row * CPR + (c ^ (row & (CPR - 1)));
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
// S0 fragment (hi, lo) times a staged fragment.
template <int CPR>
__device__ __forceinline__ f32x4 mma_state(const bf16x8& shi, const bf16x8& slo,
                                           const Frag<uint16_t, CPR>& b, f32x4 acc) {
  acc = mfma16(shi, b.hi, acc);
  return mfma16(slo, b.hi, acc);
}
template <int CPR>
__device__ __forceinline__ f32x4 mma_state(const bf16x8& shi, const bf16x8& slo,
                                           const Frag<float, CPR>& b, f32x4 acc) {
  acc = mfma16(shi, b.hi, acc);
  acc = mfma16(shi, b.lo, acc);
  acc = mfma16(slo, b.hi, acc);
  return mfma16(slo, b.lo, acc);
}

__device__ __forceinline__ void fma4(float4& acc, float c, const float4& u) {
  acc.x += c * u.x;
  acc.y += c * u.y;
  acc.z += c * u.z;
  acc.w += c * u.w;
}

constexpr int kVerifyWaves = 8;

template <class IO, int DK, int DV, int MT>
__global__ __launch_bounds__(64 * kVerifyWaves) void wy_verify_kernel(const VerifyArgs a) {
  constexpr int NW = kVerifyWaves;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int NP = MT * 16;                 // padded node rows
  constexpr int KS = DK / 32;                 // MFMA k-steps over dk
  constexpr int DVT = DV / 16;                // 16-row tiles of S0 (dv direction)
  constexpr int TPW = (DVT + NW - 1) / NW;    // S0 tiles per wave
  constexpr int EPC = 16 / (int)sizeof(IO);   // io elements per 16-byte chunk
  constexpr int CPR = DK / EPC;               // chunks per q/k row
  constexpr int CPV = DV / EPC;               // chunks per v/o row
  constexpr int UROW = DV + 4;                // U row, floats
  constexpr int NTRI = NP * (NP + 1) / 2;     // packed lower triangle
  constexpr int NSTAGE = NP * (2 * CPR + CPV);  // staged q, k, v chunks
  constexpr int NLD = (NSTAGE + NT - 1) / NT;   // per thread (a spare one repeats the last)
  using io = io_traits<IO>;
  static_assert(DVT % NW == 0 || TPW == 1, "every wave with S0 rows owns whole tiles");

  struct Stage1 {             // until the state products are done
    uint4 k[NP * CPR];
    uint4 q[NP * CPR];
    uint4 v[NP * CPV];
  };
  struct Stage2 {             // solve and output
    float u[NP * UROW];
    uint4 o[NP * CPV];
  };
  union SMem {
    Stage1 s1;
    Stage2 s2;
  };
  __shared__ SMem sm;
  __shared__ float sAkk[NTRI];
  __shared__ float sAqk[NTRI];
  __shared__ uint64_t sAnc[64];
  __shared__ float sG2[64];
  __shared__ float sBeta[64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;      // lane group of an MFMA operand / result
  const int l16 = lane & 15;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const IO* __restrict__ q = static_cast<const IO*>(a.q);
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  const IO* __restrict__ v = static_cast<const IO*>(a.v);
  IO* __restrict__ o = static_cast<IO*>(a.o);

  // ---- node range (uniform, scalar loads)
  const int lo = a.offsets[b];
  const int hi = a.offsets[b + 1];
  if (lo < 0 || hi > a.T || hi - lo < 1 || hi - lo > a.max_nodes) {
    if (h == 0 && tid == 0) a.status[b] = GDN_TREE_BAD_SIZE;
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
  // 1c. this wave's S0 rows 16jt + lane%16, columns 32s + 8g .. +7
  const int jt0 = min(wave * TPW, DVT - TPW);   // waves without a tile of their own repeat one
  const float* __restrict__ S0bh = a.S0 + (size_t)bh * DV * DK;
  float4 sraw[TPW][KS][2];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const float* rowp = S0bh + (size_t)(16 * (jt0 + jj) + l16) * DK + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sraw[jj][s][0] = *reinterpret_cast<const float4*>(rowp + 32 * s);
      sraw[jj][s][1] = *reinterpret_cast<const float4*>(rowp + 32 * s + 4);
    }
  }

  // ---- 2. staged chunks to LDS (swizzled), then the tree prologue, computed
  // by every wave so that no branch separates the loads from their first use.
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int idx = min(tid + NT * it, NSTAGE - 1);
    const int mat = idx < NP * CPR ? 0 : (idx < 2 * NP * CPR ? 1 : 2);
    const int rel = idx - mat * NP * CPR;
    if (mat == 2) {
      const int row = rel / CPV;
      sm.s1.v[chunk_slot<CPV>(row, rel - row * CPV)] = stg[it];
    } else {
      const int row = rel / CPR;
      (mat == 0 ? sm.s1.k : sm.s1.q)[chunk_slot<CPR>(row, rel - row * CPR)] = stg[it];
    }
  }
  const int par = lane < n ? par_raw : -1;
  const float beta_l = lane < n ? beta_raw : 0.f;
  int st = GDN_TREE_OK;
  if (__shfl(par, 0, kWave) != -1)
    st = GDN_TREE_BAD_ROOT;
  else if (__ballot(lane >= 1 && lane < n && (par < 0 || par >= lane)) != 0ull)
    st = GDN_TREE_BAD_PARENT;
  uint64_t anc;
  float g2;
  // (on a bad tree the scan still terminates; its results are not used)
  path_scan(par, lane, n, lane < n ? gate_log2(alpha_l) : 0.f, anc, g2);
  int maxd = lane < n ? __popcll(anc) - 1 : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) maxd = max(maxd, __shfl_xor(maxd, off, kWave));
  if (wave == 0) {
    sAnc[lane] = anc;
    sG2[lane] = g2;
    sBeta[lane] = beta_l;
  }
  __syncthreads();
  if (st != GDN_TREE_OK) {
    for (int idx = tid; idx < n * (DV / 4); idx += NT) {
      const int t = idx / (DV / 4);
      const int r = 4 * (idx - t * (DV / 4));
      const size_t row = ((size_t)(lo + t) * H + h) * DV + r;
      io::store4(o + row, make_float4(0.f, 0.f, 0.f, 0.f));
      *reinterpret_cast<float4*>(a.U + row) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int t = tid; t < n; t += NT) a.g2[(size_t)(lo + t) * H + h] = 0.f;
    if (h == 0 && tid == 0) a.status[b] = st;
    return;
  }

  // ---- 3. masked, decayed K K^T and Q K^T (lower triangle of node tiles),
  // stored packed: entry (t, i), i <= t, at t(t+1)/2 + i
  {
    const int ntile = mt * (mt + 1) / 2;
    for (int ti = wave; ti < 2 * ntile; ti += NW) {
      const bool is_qk = ti >= ntile;
      const int tt = is_qk ? ti - ntile : ti;
      int mi = 0;
      while ((mi + 1) * (mi + 2) / 2 <= tt) ++mi;
      const int mj = tt - mi * (mi + 1) / 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<IO, CPR> fa, fb;
        fa.load(is_qk ? sm.s1.q : sm.s1.k, 16 * mi + l16, s, g);
        fb.load(sm.s1.k, 16 * mj + l16, s, g);
        acc = mma(fa, fb, acc);
      }
      // result: column i = 16mj + lane%16, rows t = 16mi + 4g + e
      const int i = 16 * mj + l16;
      const float g2i = sG2[i];
      float* dstA = is_qk ? sAqk : sAkk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mi + 4 * g + e;
        if (i <= t) {
          const bool vis = t < n && ((sAnc[t] >> i) & 1ull) && (is_qk || i != t);
          float val = 0.f;
          if (vis) val = exp2f(sG2[t] - g2i) * acc[e] * (is_qk ? 1.f : sBeta[t]);
          dstA[t * (t + 1) / 2 + i] = val;
        }
      }
    }
  }

  // ---- 4. X = K S0^T, Y = Q S0^T (A operand = S0 hi/lo, B = staged k / q)
  const bool owns = wave * TPW < DVT;           // (dv = 32) waves 2, 3 own no S0 rows
  f32x4 accX[TPW][MT], accY[TPW][MT];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      accX[jj][m] = f32x4{0.f, 0.f, 0.f, 0.f};
      accY[jj][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  if (owns) {
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float4 x0 = sraw[jj][s][0], x1 = sraw[jj][s][1];
        const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 shi, slo;
        split_hi_lo(f, shi, slo);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < mt) {
            Frag<IO, CPR> fk, fq;
            fk.load(sm.s1.k, 16 * m + l16, s, g);
            fq.load(sm.s1.q, 16 * m + l16, s, g);
            accX[jj][m] = mma_state(shi, slo, fk, accX[jj][m]);
            accY[jj][m] = mma_state(shi, slo, fq, accY[jj][m]);
          }
        }
      }
    }
  }

  // ---- 5. per item (node t = 16m + lane%16, columns r..r+3): R into accX,
  // G*Y into accY
  int tdep[MT];
  uint64_t tanc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = 16 * m + l16;
    const bool live = owns && m < mt && t < n;
    tanc[m] = live ? sAnc[t] : 0ull;
    tdep[m] = live ? __popcll(tanc[m]) - 1 : -1;
    const float G = live ? exp2f(sG2[t]) : 0.f;
    const float bt = live ? sBeta[t] : 0.f;
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
      const int r = 16 * (jt0 + jj) + 4 * g;
      const float4 vv = io::load4(reinterpret_cast<const IO*>(sm.s1.v) +
                                  chunk_slot<CPV>(t, r / EPC) * EPC + r % EPC);
      const f32x4 x = accX[jj][m];
      accX[jj][m] = f32x4{bt * (vv.x - G * x[0]), bt * (vv.y - G * x[1]), bt * (vv.z - G * x[2]),
                          bt * (vv.w - G * x[3])};
      accY[jj][m] = accY[jj][m] * G;
    }
  }
  __syncthreads();  // staged q, k, v are dead: U and the o staging reuse that LDS

  // ---- 6. level-by-level solve of (I + A_kk) U = R on this wave's columns,
  // fused with the output: all nodes of one depth at once (a node at depth l
  // has exactly l proper ancestors, visited root first); each ancestor's
  // pseudo-value is read once and serves both
  //     u_t = r_t - sum_{i in A(t), i != t} A_kk[t,i] u_i
  //     o_t = G_t y_t + sum_{i in A(t), i != t} A_qk[t,i] u_i + A_qk[t,t] u_t
  float* __restrict__ sU = sm.s2.u;
  if (owns) {
    float4 out[TPW][MT];
    for (int lvl = 0; lvl <= maxd; ++lvl) {
      float4 un[TPW][MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int t = 16 * m + l16;
        if (tdep[m] == lvl) {
          uint64_t msk = tanc[m] & ~(1ull << (t & 63));
#pragma unroll
          for (int jj = 0; jj < TPW; ++jj) {
            const f32x4 rr = accX[jj][m];
            const f32x4 yy = accY[jj][m];
            un[jj][m] = make_float4(rr[0], rr[1], rr[2], rr[3]);
            out[jj][m] = make_float4(yy[0], yy[1], yy[2], yy[3]);
          }
          const int trow = t * (t + 1) / 2;
          for (int d = 0; d < lvl; ++d) {
            const int i = __builtin_ctzll(msk);
            msk &= msk - 1;
            const float ckk = -sAkk[trow + i];
            const float cqk = sAqk[trow + i];
#pragma unroll
            for (int jj = 0; jj < TPW; ++jj) {
              const int r = 16 * (wave * TPW + jj) + 4 * g;
              const float4 ui = *reinterpret_cast<const float4*>(sU + i * UROW + r);
              fma4(un[jj][m], ckk, ui);
              fma4(out[jj][m], cqk, ui);
            }
          }
          const float cself = sAqk[trow + t];
#pragma unroll
          for (int jj = 0; jj < TPW; ++jj) fma4(out[jj][m], cself, un[jj][m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int t = 16 * m + l16;
        if (tdep[m] == lvl) {
#pragma unroll
          for (int jj = 0; jj < TPW; ++jj)
            *reinterpret_cast<float4*>(sU + t * UROW + 16 * (wave * TPW + jj) + 4 * g) = un[jj][m];
        }
      }
      wave_lds_sync();
    }
    // o in io precision into the LDS staging rows
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = 16 * m + l16;
      if (tdep[m] >= 0) {
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
          const int r = 16 * (wave * TPW + jj) + 4 * g;
          io::store4(reinterpret_cast<IO*>(sm.s2.o) + chunk_slot<CPV>(t, r / EPC) * EPC + r % EPC,
                     out[jj][m]);
        }
      }
    }
  }
  __syncthreads();

  // ---- 8. o, U and g2 to memory, consecutive lanes on consecutive chunks of a row
  for (int idx = tid; idx < n * CPV; idx += NT) {
    const int t = idx / CPV;
    const int c = idx - t * CPV;
    *reinterpret_cast<uint4*>(o + ((size_t)(lo + t) * H + h) * DV + c * EPC) =
        sm.s2.o[chunk_slot<CPV>(t, c)];
  }
  for (int idx = tid; idx < n * (DV / 4); idx += NT) {
    const int t = idx / (DV / 4);
    const int c = idx - t * (DV / 4);
    *reinterpret_cast<float4*>(a.U + ((size_t)(lo + t) * H + h) * DV + 4 * c) =
        *reinterpret_cast<const float4*>(sU + t * UROW + 4 * c);
  }
  if (wave == 0 && lane < n) a.g2[(size_t)(lo + lane) * H + h] = g2;
  if (h == 0 && tid == 0) a.status[b] = GDN_TREE_OK;
}

template <class IO, int D, int MT>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&wy_verify_kernel<IO, D, D, MT>),
                       (unsigned)(a.B * a.H), 64u * kVerifyWaves, s, a);
}

template <class IO, int D>
hipError_t launch_mt(int mt, const VerifyArgs& a, hipStream_t s) {
  switch (mt) {
    case 1: return launch_t<IO, D, 1>(a, s);
    case 2: return launch_t<IO, D, 2>(a, s);
    case 3: return launch_t<IO, D, 3>(a, s);
    case 4: return launch_t<IO, D, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class IO>
hipError_t launch_d(int d, int mt, const VerifyArgs& a, hipStream_t s) {
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

}  // namespace gdn
