// wy_verify.hip -- tree-WY verification of one GDN layer on gfx950.
//
// One workgroup (4 waves) per (sequence b, head h). With A(t) = t and its
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
// Work split:
//  * tree prologue: one lane per node, ancestor bitmasks by pointer jumping,
//    base-2 gate prefixes g2 (G_t = 2^g2_t) summed along each path;
//  * q and k staged in LDS; A_kk and A_qk as 16x16 tiles of
//    v_mfma_f32_16x16x32_bf16 over the lower triangle of node tiles;
//  * the state products X = K S0^T and Y = Q S0^T on MFMA. S0 is fp32 and is
//    streamed from HBM straight into MFMA operand registers (each wave owns
//    32 rows of S0), split into bf16 hi + lo parts so that the product keeps
//    about 16 significant bits of S0 at bf16 MFMA rate (fp32 io also splits
//    q and k);
//  * R = diag(beta)(V - diag(G) X) into LDS, then a per-column forward
//    substitution over the ancestor lists (at most depth(t) terms per row);
//  * o_t = G_t Y_t + sum_{i in A(t)} A_qk[t,i] u_i, written in io precision;
//    U and g2 are written to the workspace for the commit kernel.
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

// An MFMA operand fragment of 8 consecutive k-elements of one staged row.
template <class IO> struct Frag;

template <> struct Frag<uint16_t> {
  bf16x8 hi;
  __device__ __forceinline__ void load(const uint16_t* p) {
    hi = *reinterpret_cast<const bf16x8*>(p);
  }
};

template <> struct Frag<float> {
  bf16x8 hi, lo;
  __device__ __forceinline__ void load(const float* p) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    split_hi_lo(f, hi, lo);
  }
};

// acc += A * B for operands held as fragments (bf16: one product; fp32: the
// four hi/lo cross products).
__device__ __forceinline__ f32x4 mma(const Frag<uint16_t>& a, const Frag<uint16_t>& b, f32x4 acc) {
  return mfma16(a.hi, b.hi, acc);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 acc) {
  acc = mfma16(a.hi, b.hi, acc);
  acc = mfma16(a.hi, b.lo, acc);
  acc = mfma16(a.lo, b.hi, acc);
  return mfma16(a.lo, b.lo, acc);
}
// S0 fragment (hi, lo) times a staged fragment.
__device__ __forceinline__ f32x4 mma_state(const bf16x8& shi, const bf16x8& slo,
                                           const Frag<uint16_t>& b, f32x4 acc) {
  acc = mfma16(shi, b.hi, acc);
  return mfma16(slo, b.hi, acc);
}
__device__ __forceinline__ f32x4 mma_state(const bf16x8& shi, const bf16x8& slo,
                                           const Frag<float>& b, f32x4 acc) {
  acc = mfma16(shi, b.hi, acc);
  acc = mfma16(shi, b.lo, acc);
  acc = mfma16(slo, b.hi, acc);
  return mfma16(slo, b.lo, acc);
}

template <class IO, int DK, int DV, int MT>
__global__ __launch_bounds__(256) void wy_verify_kernel(const VerifyArgs a) {
  constexpr int NW = 4;
  constexpr int NP = MT * 16;                 // padded node rows
  constexpr int KS = DK / 32;                 // MFMA k-steps over dk
  constexpr int DVT = DV / 16;                // 16-row tiles of S0 (dv direction)
  constexpr int TPW = (DVT + NW - 1) / NW;    // S0 tiles per wave
  constexpr int KPAD = 16 / (int)sizeof(IO);  // 16-byte row padding against bank conflicts
  constexpr int KROW = DK + KPAD;             // staged q/k row, elements
  constexpr int UROW = DV + 4;                // U row, floats
  constexpr int AROW = NP + 1;                // A_kk / A_qk row, floats
  constexpr int EPC = 16 / (int)sizeof(IO);   // elements per 16-byte chunk
  constexpr int CPR = DK / EPC;               // chunks per q/k row
  using io = io_traits<IO>;

  struct KQ {
    IO k[NP * KROW];
    IO q[NP * KROW];
  };
  union SMem {
    KQ kq;
    float u[NP * UROW];
  };
  __shared__ SMem sm;
  __shared__ float sAkk[NP * AROW];
  __shared__ float sAqk[NP * AROW];
  __shared__ uint64_t sAnc[64];
  __shared__ float sG2[64];
  __shared__ float sBeta[64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int H = a.H;
  const IO* __restrict__ q = static_cast<const IO*>(a.q);
  const IO* __restrict__ k = static_cast<const IO*>(a.k);
  const IO* __restrict__ v = static_cast<const IO*>(a.v);
  IO* __restrict__ o = static_cast<IO*>(a.o);

  // ---- 1. Put this wave's share of S0 in flight first: rows 16*jt + (lane%16),
  // columns 32*s + 8*(lane/16) .. +7 -- exactly the MFMA A-operand fragments.
  const float* __restrict__ S0bh = a.S0 + (size_t)bh * DV * DK;
  float4 sraw[TPW][KS][2];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int jt = wave * TPW + jj;
    if (jt < DVT) {
      const float* rowp = S0bh + (size_t)(16 * jt + (lane & 15)) * DK + 8 * (lane >> 4);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sraw[jj][s][0] = *reinterpret_cast<const float4*>(rowp + 32 * s);
        sraw[jj][s][1] = *reinterpret_cast<const float4*>(rowp + 32 * s + 4);
      }
    }
  }

  // ---- 2. Tree of sequence b (every wave holds it; wave 0 publishes it).
  const TreeLane tl = load_tree(b, a.T, a.max_nodes, a.offsets, a.parents, lane);
  if (tl.status != GDN_TREE_OK) {
    if (tl.status != GDN_TREE_BAD_SIZE) {
      const int n = tl.n, lo = tl.lo;
      for (int idx = tid; idx < n * (DV / 4); idx += 256) {
        const int t = idx / (DV / 4);
        const int r = 4 * (idx - t * (DV / 4));
        const size_t row = ((size_t)(lo + t) * H + h) * DV + r;
        io::store4(o + row, make_float4(0.f, 0.f, 0.f, 0.f));
        *reinterpret_cast<float4*>(a.U + row) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      for (int t = tid; t < n; t += 256) a.g2[(size_t)(lo + t) * H + h] = 0.f;
    }
    if (h == 0 && tid == 0) a.status[b] = tl.status;
    return;
  }
  const int n = tl.n;
  const int lo = tl.lo;
  const int mt = (n + 15) >> 4;

  float beta_l = 0.f, l2a = 0.f;
  if (lane < n) {
    const size_t gi = (size_t)(lo + lane) * H + h;
    l2a = gate_log2(a.alpha[gi]);
    beta_l = a.beta[gi];
  }
  const float g2_l = path_sum(tl.anc, l2a, n);
  if (wave == 0) {
    sAnc[lane] = tl.anc;
    sG2[lane] = g2_l;
    sBeta[lane] = beta_l;
  }

  // ---- 3. Stage k and q rows (zero rows up to the tile edge).
  for (int idx = tid; idx < 2 * 16 * mt * CPR; idx += 256) {
    const int which = idx >= 16 * mt * CPR;
    const int rem = idx - which * 16 * mt * CPR;
    const int row = rem / CPR;
    const int ch = rem - row * CPR;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < n)
      val = *reinterpret_cast<const uint4*>((which ? q : k) + ((size_t)(lo + row) * H + h) * DK +
                                            ch * EPC);
    *reinterpret_cast<uint4*>((which ? sm.kq.q : sm.kq.k) + row * KROW + ch * EPC) = val;
  }

  // ---- 4. v in the output layout: node t = 16m + lane%16, dv r = 16jt + 4*(lane/16) + 0..3.
  float4 vreg[TPW][MT];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      vreg[jj][m] = make_float4(0.f, 0.f, 0.f, 0.f);
      const int jt = wave * TPW + jj;
      const int t = 16 * m + (lane & 15);
      if (jt < DVT && m < mt && t < n)
        vreg[jj][m] = io::load4(v + ((size_t)(lo + t) * H + h) * DV + 16 * jt + 4 * (lane >> 4));
    }
  }
  __syncthreads();

  // ---- 5. Masked, decayed K K^T and Q K^T on MFMA (lower triangle of node tiles).
  {
    const int ntile = mt * (mt + 1) / 2;
    for (int ti = wave; ti < 2 * ntile; ti += NW) {
      const bool is_qk = ti >= ntile;
      const int tt = is_qk ? ti - ntile : ti;
      int mi = 0;
      while ((mi + 1) * (mi + 2) / 2 <= tt) ++mi;
      const int mj = tt - mi * (mi + 1) / 2;
      const IO* arow = (is_qk ? sm.kq.q : sm.kq.k) + (16 * mi + (lane & 15)) * KROW + 8 * (lane >> 4);
      const IO* brow = sm.kq.k + (16 * mj + (lane & 15)) * KROW + 8 * (lane >> 4);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<IO> fa, fb;
        fa.load(arow + 32 * s);
        fb.load(brow + 32 * s);
        acc = mma(fa, fb, acc);
      }
      // D layout: column i = 16*mj + lane%16, rows t = 16*mi + 4*(lane/16) + e.
      const int i = 16 * mj + (lane & 15);
      const float g2i = sG2[i];
      float* dstA = is_qk ? sAqk : sAkk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mi + 4 * (lane >> 4) + e;
        const bool vis = t < n && i < n && ((sAnc[t] >> i) & 1ull) && (is_qk || i != t);
        float val = 0.f;
        if (vis) val = exp2f(sG2[t] - g2i) * acc[e] * (is_qk ? 1.f : sBeta[t]);
        dstA[t * AROW + i] = val;
      }
    }
  }

  // ---- 6. X = K S0^T, Y = Q S0^T: A operand = S0 fragment (hi, lo), B = staged k / q.
  f32x4 accX[TPW][MT], accY[TPW][MT];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      accX[jj][m] = f32x4{0.f, 0.f, 0.f, 0.f};
      accY[jj][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int jt = wave * TPW + jj;
    if (jt >= DVT) continue;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4 x0 = sraw[jj][s][0], x1 = sraw[jj][s][1];
      const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 shi, slo;
      split_hi_lo(f, shi, slo);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mt) {
          Frag<IO> fk, fq;
          fk.load(sm.kq.k + (16 * m + (lane & 15)) * KROW + 32 * s + 8 * (lane >> 4));
          fq.load(sm.kq.q + (16 * m + (lane & 15)) * KROW + 32 * s + 8 * (lane >> 4));
          accX[jj][m] = mma_state(shi, slo, fk, accX[jj][m]);
          accY[jj][m] = mma_state(shi, slo, fq, accY[jj][m]);
        }
      }
    }
  }
  __syncthreads();  // every read of staged k/q is done: U may now reuse that LDS

  // ---- 7. R = diag(beta)(V - diag(G) X) -> LDS; keep G*Y for the output.
  float* __restrict__ sU = sm.u;
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int jt = wave * TPW + jj;
    if (jt >= DVT) continue;
    const int r = 16 * jt + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = 16 * m + (lane & 15);
      if (m < mt && t < n) {
        const float G = exp2f(sG2[t]);
        const float bt = sBeta[t];
        const f32x4 x = accX[jj][m];
        const float4 vv = vreg[jj][m];
        float4 R;
        R.x = bt * (vv.x - G * x[0]);
        R.y = bt * (vv.y - G * x[1]);
        R.z = bt * (vv.z - G * x[2]);
        R.w = bt * (vv.w - G * x[3]);
        *reinterpret_cast<float4*>(sU + t * UROW + r) = R;
        accY[jj][m] = accY[jj][m] * G;
      }
    }
  }
  wave_lds_sync();

  // ---- 8. Forward substitution on this wave's columns: u_t = r_t - sum A_kk[t,i] u_i
  // over the proper ancestors i of t, nodes in index (= topological) order.
  {
    const int col0 = 16 * wave * TPW;
    const int col = col0 + lane;
    if (col0 < DV && lane < 16 * TPW && col < DV) {
      for (int t = 1; t < n; ++t) {
        float acc = sU[t * UROW + col];
        uint64_t msk = sAnc[t] & ~(1ull << t);
        while (msk) {
          const int i = __builtin_ctzll(msk);
          msk &= msk - 1;
          acc -= sAkk[t * AROW + i] * sU[i * UROW + col];
        }
        sU[t * UROW + col] = acc;
      }
    }
  }
  wave_lds_sync();

  // ---- 9. o_t = G_t Y_t + sum_{i in A(t)} A_qk[t,i] u_i; store o, U and g2.
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int jt = wave * TPW + jj;
    if (jt >= DVT) continue;
    const int r = 16 * jt + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = 16 * m + (lane & 15);
      if (m < mt && t < n) {
        const f32x4 y = accY[jj][m];
        float4 acc = make_float4(y[0], y[1], y[2], y[3]);
        uint64_t msk = sAnc[t];
        while (msk) {
          const int i = __builtin_ctzll(msk);
          msk &= msk - 1;
          const float c = sAqk[t * AROW + i];
          const float4 u = *reinterpret_cast<const float4*>(sU + i * UROW + r);
          acc.x += c * u.x;
          acc.y += c * u.y;
          acc.z += c * u.z;
          acc.w += c * u.w;
        }
        const size_t row = ((size_t)(lo + t) * H + h) * DV + r;
        io::store4(o + row, acc);
        *reinterpret_cast<float4*>(a.U + row) = *reinterpret_cast<const float4*>(sU + t * UROW + r);
      }
    }
  }
  if (wave == 0 && lane < n) a.g2[(size_t)(lo + lane) * H + h] = g2_l;
  if (h == 0 && tid == 0) a.status[b] = GDN_TREE_OK;
}

template <class IO, int D, int MT>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s) {
  return launch_kernel(reinterpret_cast<const void*>(&wy_verify_kernel<IO, D, D, MT>),
                       (unsigned)(a.B * a.H), 256u, s, a);
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
