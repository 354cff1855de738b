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
// Verify kernels. One workgroup per (sequence, K/V head, split of the cache).
// The G * N_b query rows that share the K/V head (<= 256) are split into
// tiles, one per wave (16-row tiles on 12 waves up to 192 rows, 32-row tiles
// on 8 waves beyond). Keys stream through a 4-stage LDS ring in blocks of 64,
// loaded straight from HBM into LDS: the cache rows of the split, then (in the
// last split) the 64 tree slots, masked per query row by the node's ancestor
// bits. Per block a wave computes the transposed scores S^T = K Q^T on MFMA
// (A = staged K rows, B = the wave's query rows held in registers), so that a
// lane owns one query row: the online softmax needs at most two cross-lane
// shuffles, and the weights come out in the B-operand layout of the same MFMA,
// which accumulates O^T += V^T P^T with V read column-wise from LDS by the
// transposing read. A split's unnormalised output, reference and sum go to the
// workspace when the cache is split over several workgroups, and a combine
// kernel merges them.
//
// Commit kernel. One workgroup per sequence copies the K/V rows of the
// accepted path, root first, behind the sequence's committed rows and
// advances its length (handbook, same section: the accepted path's K/V rows
// were computed at the right positions during verification and are appended
// as they are; rainlin-top "Qwen3.5 tree spec", section 7 step 4).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "gdn_tree_attn.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int KB = 64;                           // keys per staged block
constexpr int kStages = 4;                       // key blocks resident in LDS (three in flight)
constexpr float kMasked = -1.0e30f;              // score of an invisible key
constexpr float kSlack = 8.f;                    // see attend_block

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt with the export and LDS counters left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// the wave's 64 lanes fill 1 KiB of LDS at lds_base + 16 * lane, lane l
// reading base + offset_l. Issued as inline assembly so that the compiler
// does not wait for every such load before each LDS read; the kernel waits
// for them itself (vmcnt, then a barrier). M0 holds the LDS base for the
// instruction and is restored afterwards.
// The address is a wave-uniform base plus the lane's 32-bit byte offset.
__device__ __forceinline__ void load_lds_16(const void* base, uint32_t offset,
                                            uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(offset), "s"(base)
      : "memory");
}

// Transposing LDS read (gfx950): in each group of 16 lanes, lane i receives
// element i % 4 of the 8 bytes read by lanes 4e + i / 4, e = 0..3. With lane
// j of the group reading row R0 + j / 4, columns C0 + 4 (j % 4) .. +3 of a
// row-major bf16 matrix, lane i therefore holds column C0 + i of rows
// R0 .. R0 + 3: a column of four consecutive rows, the MFMA operand layout.
__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_char* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// LDS layout of a staged block: 64 key rows of D bf16, row-major, the 16-byte
// chunk c of row r stored at chunk position c ^ f(r). The LDS serves 256
// bytes (64 banks) per cycle; f is chosen so that the 16 rows of a K
// fragment read (same logical chunk) fill 16 different 16-byte bank groups,
// and so that the 8 rows of a half transposing read (two chunks each) fill
// them as well: for 256-byte rows f is a bijection on r mod 16 with f / 2 a
// bijection on r mod 8; for 128-byte rows (two per bank window) the same
// holds per row parity.
template <int D>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

// Online-softmax state and output accumulator of one 16-row query tile.
template <int D>
struct Tile {
  bf16x8 qf[D / 32];     // B operand of S^T = K Q^T: column = query row, k = d 32s + 8g .. +7,
                         // holding q * scale * log2(e)
  f32x4 o[D / 16];       // O^T rows d = 16 dt + 4g + e, column = query row
  f32x4 l;               // row sums of P^T as an MFMA result: element 0 of the g = 0 lanes
  float m;               // row reference (base-2 units)
  uint64_t anc;          // ancestor bits of the lane's node
};

// Lane byte offsets of the MFMA operand reads inside a staged block. A row
// starts at a multiple of 2D bytes and the permuted chunk index occupies the
// address bits just below, so a chunk permutation is an XOR on the address:
// K fragment (kt, s) at (k ^ 64 s) + 32 D kt, V^T fragment (mg, dt, half) at
// (v ^ 32 dt) + 64 D mg + 32 D half.
struct LaneOffsets {
  int k, v;
};

template <int D>
__device__ __forceinline__ LaneOffsets lane_offsets(int g, int l16) {
  constexpr int RB = 2 * D;
  LaneOffsets o;
  // K fragment: rows 16 kt + l16, logical chunk 4s + g
  o.k = l16 * RB | ((swz_key<D>(l16) ^ g) << 4);
  // V^T fragment: transposing reads of rows 32 mg + 4g + i (+16), i = l16 / 4,
  // columns 16 dt + 4 (l16 % 4) .. +3: logical chunk 2 dt + h, h = (l16 % 4) / 2,
  // byte 8 (l16 % 2) of it
  const int row = 4 * g + (l16 >> 2);
  const int h = (l16 & 3) >> 1;
  o.v = row * RB | ((swz_key<D>(row) ^ h) << 4) | ((l16 & 1) << 3);
  return o;
}

// Scores, online softmax and output update of one staged key block (K at
// sK, V right after it) for the wave's 16-row query tile. The query fragments
// hold q * scale * log2(e), so a score is already in base-2 units; the MFMA
// starts from -m, the lane's reference, and returns x - m directly.
//
// FULL: every key of the block is visible; otherwise bit 16 kt + e of vm says
// whether key 16 kt + 4g + e is visible to the lane's row (the row's ancestor
// bits shifted by 4g for the tree block, a prefix of keys for the last cache
// block), and invisible keys get x - m = -1e30, weight 0.
//
// A row takes its maximum as its reference at its first visible key; later
// halves raise it only when some lane of the wave sees x - m > kSlack, so the
// O^T rescale is rare and every weight stays below 2^kSlack; the final
// o = O^T / l does not depend on the reference.
template <int D, bool FULL, int HALF>
__device__ __forceinline__ void attend_block(Tile<D>& T, const lds_char* sK,
                                             const LaneOffsets& lo, uint64_t vm,
                                             const bf16x8& ones) {
  constexpr int KSD = D / 32;
  constexpr int DT = D / 16;
  constexpr int RB = 2 * D;
  const lds_char* sV = sK + KB * RB;

  // the block in two halves of 32 keys (key group mg = key tiles 2mg, 2mg+1);
  // HALF >= 0: this wave takes only that half (another wave takes the other)
#pragma unroll
  for (int mg = (HALF == 1 ? 1 : 0); mg < (HALF == 0 ? 1 : 2); ++mg) {
    // S^T tiles: lane holds query row l16 and keys 16 kt + 4g + e, as x - m
    // (as x while the row has no reference yet)
    const float c0 = T.m > 0.5f * kMasked ? -T.m : 0.f;
    f32x4 acc[2];
    acc[0] = f32x4{c0, c0, c0, c0};
    acc[1] = acc[0];
    __builtin_amdgcn_s_setprio(1);            // MFMA phases first
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 ka[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ka[h] = *(const lds_bf16x8*)(sK + (lo.k ^ (64 * s)) + 16 * RB * (2 * mg + h));
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h] = mfma_k32(ka[h], T.qf[s], acc[h]);
    }
    __builtin_amdgcn_s_setprio(0);
    if (!FULL) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (((vm >> (32 * mg + 16 * h + e)) & 1ull) == 0) acc[h][e] = kMasked;
    }
    float mx = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                     fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
    const bool has = T.m > 0.5f * kMasked;
    if (__ballot(has ? mx > kSlack : mx > 0.5f * kMasked) != 0ull) {   // wave-uniform
      // the four lanes of a row, g = 0..3, hold its keys between them
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const bool seen = mx > 0.5f * kMasked;
      const float delta = has ? fmaxf(mx, 0.f) : (seen ? mx : 0.f);
      T.m = has ? T.m + delta : (seen ? mx : T.m);
      acc[0] -= delta;
      acc[1] -= delta;
      const float alpha = has ? __builtin_amdgcn_exp2f(-delta) : 1.f;
      T.l[0] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) T.o[dt] *= alpha;
    }
    // P^T as the B operand of 16x16x32 over the 32 keys: k slot 8g + i holds
    // key 32 mg + 4g + i (i < 4) or 32 mg + 16 + 4g + i - 4
    bf16x8 pk;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[4 * h + e] = (__bf16)__builtin_amdgcn_exp2f(acc[h][e]);
    // row sums of the same bf16 weights the output uses: a ones row (row 0
    // of the A operand) against P^T
    T.l = mfma_k32(ones, pk, T.l);
    // O^T += V^T P^T: A = V^T rows d = 16 dt + l16 over the same key slots,
    // read column-wise from the row-major V block
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const lds_char* p1 = sV + (lo.v ^ (32 * dt)) + 32 * RB * mg;
      const bf16x4 v1 = lds_read_tr16(p1);
      const bf16x4 v2 = lds_read_tr16(p1 + 16 * RB);
      const bf16x8 va = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
      T.o[dt] = mfma_k32(va, pk, T.o[dt]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

template <int N>
__device__ __forceinline__ void wait_blocks_ahead(int ahead) {
  if (ahead >= 3) wait_vmem<3 * N>();
  else if (ahead == 2) wait_vmem<2 * N>();
  else if (ahead == 1) wait_vmem<N>();
  else wait_vmem<0>();
}

// W waves of one 16-row query tile each (W * 16 >= the rows of a (sequence,
// K/V head)); see the tile assignment below.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void tree_attn_kernel(const AttnArgs a) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int KSD = D / 32;                 // 16x16x32 steps over d (scores)
  constexpr int DT = D / 16;                  // 16-row tiles of O^T (over d)
  constexpr int MAT = KB * 2 * D;             // bytes of one staged matrix (K or V)
  constexpr int STAGE = 2 * MAT;              // K block then V block
  constexpr int NU = STAGE / 1024;            // 1 KiB wave loads per block
  constexpr int LMAX = (NU + W - 1) / W;      // loads per thread per block: LMAX or LMAX - 1
  static_assert(MAT % 1024 == 0, "a wave's 1 KiB load falls in one matrix");

  __shared__ __align__(16) char smem[kStages * STAGE];
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
  if (split == 0 && kvh == 0 && tid == 0) put_status(a.status, b, st, a.merge);

  // ---- query rows: wave w owns tiles w, w + waves, ... (rows 16 tile + l16
  // of the G * n rows of the K/V head, query-head-major, node inner)
  const int R = range_ok ? G * n : 0;
  const int ntiles = (R + 15) >> 4;
  // Tiles [0, nfull) get a wave each, and each of the last nsplit tiles gets
  // two waves, one per 32-key half of every block (merged at the end), so that
  // the four SIMDs carry equal work when the tiles do not divide evenly
  // (10 tiles on 12 waves: 2.5 tiles per SIMD).
  const int nsplit = max(0, min(ntiles, W - ntiles));   // workgroup-uniform
  const int nfull = ntiles - nsplit;
  int tile = wave, half = -1;                 // wave-uniform role
  if (wave >= nfull) {
    const int q2 = wave - nfull;
    tile = q2 < 2 * nsplit ? nfull + (q2 >> 1) : ntiles;   // ntiles: idle
    half = q2 & 1;
  }
  const bool active = tile < ntiles;          // wave-uniform
  const int r = 16 * tile + l16;
  const bool rv = r < R;
  const int hg = rv ? r / n : 0;
  const int t = rv ? r - hg * n : 0;
  const size_t orow = (size_t)(lo + t) * a.Hq + kvh * G + hg;   // row of o / the partials
  Tile<D> T;
  T.anc = sAnc[t];
  T.m = kMasked;                              // no reference yet
  T.l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) T.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (st != GDN_TREE_OK) {
    // rows of a rejected sequence (with a valid node range) are zero
    if (rv && half <= 0) {
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

  // query fragments, scaled to base-2 score units and rounded to bf16,
  // waited for before the key blocks are issued (the block waits below count
  // only the block loads)
  {
    const uint16_t* qrow = a.q + orow * D;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const uint4 v = rv ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g)
                         : make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 x = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) T.qf[s][e] = (__bf16)((float)x[e] * a.scale_log2);
    }
  }
  wait_vmem<0>();
  const LaneOffsets lofs = lane_offsets<D>(g, l16);
  const __bf16 one = l16 == 0 ? (__bf16)1.f : (__bf16)0.f;
  const bf16x8 ones = {one, one, one, one, one, one, one, one};

  // ---- key range of this split: cache rows [c0, c1), then the tree slots
  // (last split only)
  const int c0 = min(split * a.CL, L);
  const int c1 = min(c0 + a.CL, L);
  const int ncb = (c1 - c0 + KB - 1) / KB;
  const int nblk = ncb + (split == NS - 1 ? 1 : 0);
  const size_t kvbase = ((size_t)b * a.Hkv + kvh) * a.cap;   // cache row 0 of (b, kvh)
  const uint32_t smem_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char*)smem);

  // Loads of block j into stage s. Wave w issues the 1 KiB units
  // w, w + W, ... of the stage; in unit u lane l fills LDS slot q = 64 u + l
  // (16 bytes; consecutive per wave, as the instruction requires): slots
  // below 64 * CPR are K, the rest V; slot q holds row q / CPR, stored chunk
  // q % CPR, i.e. logical chunk (q % CPR) ^ f(row). Keys past the split's
  // cache rows, and unused tree slots, read a valid row instead: finite
  // values that the mask gives zero weight.
  const int nload = (NU - wave + W - 1) / W;  // this wave's loads per block (wave-uniform)
  // lane byte offset of load i inside a full cache block (row r at r * 2D)
  uint32_t loff[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    const int rem = (64 * (wave + W * i) + lane) % (KB * CPR);
    const int row = rem / CPR;
    loff[i] = (uint32_t)(row * D + 8 * ((rem % CPR) ^ swz_key<D>(row))) * 2u;
  }
  const uint16_t* kc_seq = a.kc + kvbase * D;      // cache row 0 of (b, kvh)
  const uint16_t* vc_seq = a.vc + kvbase * D;
  const size_t tree0 = ((size_t)lo * a.Hkv + kvh) * D;   // tree node 0 of (b, kvh)
  auto issue_block = [&](int j, int s) {
    const bool tree = j >= ncb;
    const int p0 = c0 + j * KB;
    const bool partial = !tree && p0 + KB > c1;   // wave-uniform
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      if (i == LMAX - 1 && i >= nload) break;
      const int wbase = 64 * (wave + W * i);  // wave-uniform
      const int mat = wbase >= KB * CPR ? 1 : 0;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + s * STAGE + 16 * wbase);
      if (!tree && !partial) {
        load_lds_16((mat ? vc_seq : kc_seq) + (size_t)p0 * D, loff[i], lds);
      } else {
        const int rem = wbase + lane - mat * KB * CPR;
        const int row = rem / CPR;
        const int chunk = (rem % CPR) ^ swz_key<D>(row);
        if (!tree) {
          const int p = min(row, c1 - 1 - p0);
          load_lds_16((mat ? vc_seq : kc_seq) + (size_t)p0 * D,
                      (uint32_t)(p * D + 8 * chunk) * 2u, lds);
        } else {
          const int node = row < n ? row : 0;
          load_lds_16((mat ? a.v : a.k) + tree0,
                      (uint32_t)(node * a.Hkv * D + 8 * chunk) * 2u, lds);
        }
      }
    }
  };

#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < nblk) issue_block(j, j);

  for (int j = 0; j < nblk; ++j) {
    // block j's loads are this thread's oldest outstanding ones
    const int ahead = min(kStages - 2, nblk - 1 - j);
    static_assert(kStages - 2 <= 3, "wait_blocks_ahead covers three blocks ahead");
    if (nload == LMAX) wait_blocks_ahead<LMAX>(ahead);
    else wait_blocks_ahead<(LMAX > 1 ? LMAX - 1 : 1)>(ahead);
    __syncthreads();                          // every thread's part landed; stage j-1 is free
    if (j + kStages - 1 < nblk) issue_block(j + kStages - 1, (j + kStages - 1) % kStages);
    if (!active) continue;

    const lds_char* sK = (const lds_char*)smem + (j % kStages) * STAGE;
    const bool tree = j >= ncb;
    const int lim = tree ? KB : c1 - (c0 + j * KB);   // cache keys below lim are visible
    if (!tree && lim >= KB) {
      if (half < 0) attend_block<D, true, -1>(T, sK, lofs, 0ull, ones);
      else if (half == 0) attend_block<D, true, 0>(T, sK, lofs, 0ull, ones);
      else attend_block<D, true, 1>(T, sK, lofs, 0ull, ones);
    } else {
      const int lm = lim - 4 * g;             // lane keys 16 kt + e below lm are visible
      const uint64_t vm = tree ? T.anc >> (4 * g)
                               : (lm >= 64 ? ~0ull : lm <= 0 ? 0ull : (1ull << lm) - 1ull);
      if (half < 0) attend_block<D, false, -1>(T, sK, lofs, vm, ones);
      else if (half == 0) attend_block<D, false, 0>(T, sK, lofs, vm, ones);
      else attend_block<D, false, 1>(T, sK, lofs, vm, ones);
    }
  }

  // ---- split tiles: the half-1 wave hands its (m, l, O^T) to the half-0
  // wave through LDS (the stages are free once every wave passed the loop)
  if (nsplit > 0) {
    constexpr int SLOT = 64 * (DT * 4 + 8);   // floats per split tile: O^T, l, m
    __syncthreads();
    float* xs = reinterpret_cast<float*>(smem) + (tile - nfull) * SLOT;
    if (active && half == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(xs + (dt * 64 + lane) * 4) = T.o[dt];
      *reinterpret_cast<f32x4*>(xs + (DT * 64 + lane) * 4) = T.l;
      xs[DT * 256 + 256 + lane] = T.m;
    }
    __syncthreads();
    if (active && half == 0) {
      const float m1 = xs[DT * 256 + 256 + lane];
      const float M = fmaxf(T.m, m1);
      const float a0 = T.m > 0.5f * kMasked ? __builtin_amdgcn_exp2f(T.m - M) : 0.f;
      const float a1 = m1 > 0.5f * kMasked ? __builtin_amdgcn_exp2f(m1 - M) : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        T.o[dt] = T.o[dt] * a0 + *reinterpret_cast<const f32x4*>(xs + (dt * 64 + lane) * 4) * a1;
      T.l = T.l * a0 + *reinterpret_cast<const f32x4*>(xs + (DT * 64 + lane) * 4) * a1;
      T.m = M;
    }
  }

  // ---- results: lane (g, l16) holds O^T rows d = 16 dt + 4g + e of row r
  const float lsum = __shfl(T.l[0], l16, kWave);   // from lane (g = 0, l16)
  if (!rv || half == 1) return;
  if (NS == 1) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t w0 = (uint32_t)float_to_bf16_bits(T.o[dt][0] * inv) |
                          ((uint32_t)float_to_bf16_bits(T.o[dt][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)float_to_bf16_bits(T.o[dt][2] * inv) |
                          ((uint32_t)float_to_bf16_bits(T.o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(a.o + orow * D + 16 * dt + 4 * g) = make_uint2(w0, w1);
    }
  } else {
    float* po = a.part_o + (orow * NS + split) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
          make_float4(T.o[dt][0], T.o[dt][1], T.o[dt][2], T.o[dt][3]);
    if (g == 0)
      *reinterpret_cast<float2*>(a.part_ml + (orow * NS + split) * 2) = make_float2(T.m, lsum);
  }
}

// ---------------------------------------------------------------------------
// 32-row query tiles on v_mfma_f32_32x32x16_bf16. A K or V fragment read from
// LDS then serves 32 query rows instead of 16, halving the LDS reads per row.
// Layouts (A: lane = row l % 32, k = 8 (l / 32) .. +7; B: lane = column
// l % 32, the same k; D: lane = column l % 32, rows 8 (i / 4) + 4 (l / 32) +
// i % 4 for result element i = 0..15).

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Chunk permutation of the 32-row kernels' staged blocks: chunk c of row r at
// c ^ f(r). A K fragment read touches rows 0..15 (16 lanes per LDS cycle) at
// one logical chunk, so f is a bijection on r mod 16 (256-byte rows) or on
// r / 2 mod 8 per row parity (128-byte rows, two per 256-byte bank window);
// a transposing V read touches rows 0..3 at four consecutive chunks, so the
// bits of f above the lowest two differ between those rows.
template <int D>
__device__ __forceinline__ int swz32_key(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
struct Tile32 {
  bf16x8 qf[D / 16];     // B operand of S^T = K Q^T: column = query row l % 32,
                         // k = d 16s + 8 (l / 32) .. +7, holding q * scale * log2(e)
  f32x16 o[D / 32];      // O^T rows d = 32 dt + 8 (i / 4) + 4 (l / 32) + i % 4
  float l;               // this lane's part of the row sum
  float m;               // row reference (base-2 units); kMasked: none yet
  uint64_t anc;          // ancestor bits of the lane's node
};

// K fragment (key tile mg, step s) at (k ^ 32 s) + 32 RB mg; V^T fragment
// (key group mg, 16-key step ms, d tile dt) at (v1 ^ 64 dt) + (32 mg + 16 ms) RB
// and (v2 ^ 64 dt) + the same, RB = 2D bytes per row.
struct LaneOffsets32 {
  int k, v1, v2;
};

template <int D>
__device__ __forceinline__ LaneOffsets32 lane_offsets32(int lane) {
  constexpr int RB = 2 * D;
  LaneOffsets32 o;
  const int r32 = lane & 31, hh = lane >> 5;
  o.k = r32 * RB | ((swz32_key<D>(r32) ^ hh) << 4);      // logical chunk 2s + hh
  // transposing reads: 16-lane group (dsub, hh) = ((lane >> 4) & 1, lane >> 5);
  // lane j of the group reads row 4 hh + j / 4 (+8 for the second read),
  // columns 32 dt + 16 dsub + 4 (j % 4) .. +3: logical chunk 4 dt + c',
  // c' = 2 dsub + (j % 4) / 2, byte 8 (j % 2) of it
  const int j = lane & 15;
  const int c = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
  const int r1 = 4 * hh + (j >> 2), r2 = r1 + 8;
  o.v1 = r1 * RB | ((c ^ swz32_key<D>(r1)) << 4) | ((j & 1) << 3);
  o.v2 = r2 * RB | ((c ^ swz32_key<D>(r2)) << 4) | ((j & 1) << 3);
  return o;
}

// One 64-key block for a wave's 32-row tile. FULL and vm as in attend_block,
// with bit 32 mg + 8 q + r of vm for the lane's key 32 mg + 8 q + 4 (l / 32) + r
// (vm = the row's ancestor bits shifted by 4 (l / 32), or a prefix).
template <int D, bool FULL>
__device__ __forceinline__ void attend_block32(Tile32<D>& T, const lds_char* sK,
                                               const LaneOffsets32& lo, uint64_t vm) {
  constexpr int KS = D / 16;                  // 32x32x16 steps over d (scores)
  constexpr int DT = D / 32;                  // 32-row tiles of O^T
  constexpr int RB = 2 * D;
  const lds_char* sV = sK + KB * RB;
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    const float c0 = T.m > 0.5f * kMasked ? -T.m : 0.f;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = c0;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 ka = *(const lds_bf16x8*)(sK + (lo.k ^ (32 * s)) + 32 * RB * mg);
      acc = mfma32(ka, T.qf[s], acc);
    }
    __builtin_amdgcn_s_setprio(0);
    if (!FULL) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (((vm >> (32 * mg + 8 * (i >> 2) + (i & 3))) & 1ull) == 0) acc[i] = kMasked;
    }
    float mx = acc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[i]);
    const bool has = T.m > 0.5f * kMasked;
    if (__ballot(has ? mx > kSlack : mx > 0.5f * kMasked) != 0ull) {   // wave-uniform
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));   // lanes l, l ^ 32 hold the same row
      const bool seen = mx > 0.5f * kMasked;
      const float delta = has ? fmaxf(mx, 0.f) : (seen ? mx : 0.f);
      T.m = has ? T.m + delta : (seen ? mx : T.m);
      acc -= delta;
      const float alpha = has ? __builtin_amdgcn_exp2f(-delta) : 1.f;
      T.l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) T.o[dt] *= alpha;
    }
    // P^T as the B operand of 32x32x16 over 16-key steps: step ms holds the
    // results 8 ms .. 8 ms + 7 (keys 16 ms + 4 (l / 32) + 0..3, then + 8)
    bf16x8 pk[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(acc[i]);
      T.l += p;
      pk[i >> 3][i & 7] = (__bf16)p;
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int rows = (32 * mg + 16 * ms) * RB;
        const bf16x4 v1 = lds_read_tr16(sV + (lo.v1 ^ (64 * dt)) + rows);
        const bf16x4 v2 = lds_read_tr16(sV + (lo.v2 ^ (64 * dt)) + rows);
        const bf16x8 va = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        T.o[dt] = mfma32(va, pk[ms], T.o[dt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

// W waves, the 32-row tile t on wave t (W * 32 >= the rows of a (sequence,
// K/V head)); the rest as in tree_attn_kernel.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void tree_attn32_kernel(const AttnArgs a) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int MAT = KB * 2 * D;             // bytes of one staged matrix (K or V)
  constexpr int STAGE = 2 * MAT;              // K block then V block
  constexpr int NU = STAGE / 1024;            // 1 KiB wave loads per block
  constexpr int LMAX = (NU + W - 1) / W;      // loads per thread per block: LMAX or LMAX - 1
  static_assert(MAT % 1024 == 0, "a wave's 1 KiB load falls in one matrix");

  __shared__ __align__(16) char smem[kStages * STAGE];
  __shared__ uint64_t sAnc[64];
  __shared__ int sStatus;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int r32 = lane & 31;
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
  if (split == 0 && kvh == 0 && tid == 0) put_status(a.status, b, st, a.merge);

  // ---- this wave's tile: rows 32 wave + l % 32 of the G * n rows of the
  // K/V head (query-head-major, node inner)
  const int R = range_ok ? G * n : 0;
  const bool active = 32 * wave < R;          // wave-uniform
  const int r = 32 * wave + r32;
  const bool rv = r < R;
  const int hg = rv ? r / n : 0;
  const int t = rv ? r - hg * n : 0;
  const size_t orow = (size_t)(lo + t) * a.Hq + kvh * G + hg;

  if (st != GDN_TREE_OK) {
    // rows of a rejected sequence (with a valid node range) are zero
    if (rv) {
      if (NS == 1) {
        for (int c = 4 * hh; c < D; c += 8)
          *reinterpret_cast<uint2*>(a.o + orow * D + c) = make_uint2(0u, 0u);
      } else {
        for (int c = 4 * hh; c < D; c += 8)
          *reinterpret_cast<float4*>(a.part_o + (orow * NS + split) * D + c) =
              make_float4(0.f, 0.f, 0.f, 0.f);
        if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + (orow * NS + split) * 2) =
            make_float2(kMasked, 0.f);
      }
    }
    return;
  }

  Tile32<D> T;
  T.anc = sAnc[t];
  T.m = kMasked;
  T.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) T.o[dt][i] = 0.f;
  {
    // query fragments, scaled to base-2 score units and rounded to bf16,
    // waited for before the key blocks are issued
    const uint16_t* qrow = a.q + orow * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = rv ? *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hh)
                         : make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 x = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) T.qf[s][e] = (__bf16)((float)x[e] * a.scale_log2);
    }
  }
  wait_vmem<0>();
  const LaneOffsets32 lofs = lane_offsets32<D>(lane);

  // ---- key range of this split: cache rows [c0, c1), then the tree slots
  const int c0 = min(split * a.CL, L);
  const int c1 = min(c0 + a.CL, L);
  const int ncb = (c1 - c0 + KB - 1) / KB;
  const int nblk = ncb + (split == NS - 1 ? 1 : 0);
  const size_t kvbase = ((size_t)b * a.Hkv + kvh) * a.cap;
  const uint32_t smem_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char*)smem);

  // Block loads, as in tree_attn_kernel (slot q of a stage holds row q / CPR,
  // stored chunk q % CPR, i.e. logical chunk (q % CPR) ^ f(row)).
  const int nload = (NU - wave + W - 1) / W;
  uint32_t loff[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    const int rem = (64 * (wave + W * i) + lane) % (KB * CPR);
    const int row = rem / CPR;
    loff[i] = (uint32_t)(row * D + 8 * ((rem % CPR) ^ swz32_key<D>(row))) * 2u;
  }
  const uint16_t* kc_seq = a.kc + kvbase * D;
  const uint16_t* vc_seq = a.vc + kvbase * D;
  const size_t tree0 = ((size_t)lo * a.Hkv + kvh) * D;
  auto issue_block = [&](int j, int s) {
    const bool tree = j >= ncb;
    const int p0 = c0 + j * KB;
    const bool partial = !tree && p0 + KB > c1;
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      if (i == LMAX - 1 && i >= nload) break;
      const int wbase = 64 * (wave + W * i);
      const int mat = wbase >= KB * CPR ? 1 : 0;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + s * STAGE + 16 * wbase);
      if (!tree && !partial) {
        load_lds_16((mat ? vc_seq : kc_seq) + (size_t)p0 * D, loff[i], lds);
      } else {
        const int rem = wbase + lane - mat * KB * CPR;
        const int row = rem / CPR;
        const int chunk = (rem % CPR) ^ swz32_key<D>(row);
        if (!tree) {
          const int p = min(row, c1 - 1 - p0);
          load_lds_16((mat ? vc_seq : kc_seq) + (size_t)p0 * D,
                      (uint32_t)(p * D + 8 * chunk) * 2u, lds);
        } else {
          const int node = row < n ? row : 0;
          load_lds_16((mat ? a.v : a.k) + tree0,
                      (uint32_t)(node * a.Hkv * D + 8 * chunk) * 2u, lds);
        }
      }
    }
  };

#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < nblk) issue_block(j, j);

  for (int j = 0; j < nblk; ++j) {
    const int ahead = min(kStages - 2, nblk - 1 - j);
    if (nload == LMAX) wait_blocks_ahead<LMAX>(ahead);
    else wait_blocks_ahead<(LMAX > 1 ? LMAX - 1 : 1)>(ahead);
    __syncthreads();
    if (j + kStages - 1 < nblk) issue_block(j + kStages - 1, (j + kStages - 1) % kStages);
    if (!active) continue;

    const lds_char* sK = (const lds_char*)smem + (j % kStages) * STAGE;
    const bool tree = j >= ncb;
    const int lim = tree ? KB : c1 - (c0 + j * KB);
    if (!tree && lim >= KB) {
      attend_block32<D, true>(T, sK, lofs, 0ull);
    } else {
      const int lm = lim - 4 * hh;            // lane keys 8 q + r below lm are visible
      const uint64_t vm = tree ? T.anc >> (4 * hh)
                               : (lm >= 64 ? ~0ull : lm <= 0 ? 0ull : (1ull << lm) - 1ull);
      attend_block32<D, false>(T, sK, lofs, vm);
    }
  }

  // ---- results: lane (hh, r32) holds O^T rows d = 32 dt + 8 q + 4 hh + 0..3
  const float lsum = T.l + __shfl_xor(T.l, 32, kWave);
  if (!rv) return;
  if (NS == 1) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = (uint32_t)float_to_bf16_bits(T.o[dt][4 * q] * inv) |
                            ((uint32_t)float_to_bf16_bits(T.o[dt][4 * q + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)float_to_bf16_bits(T.o[dt][4 * q + 2] * inv) |
                            ((uint32_t)float_to_bf16_bits(T.o[dt][4 * q + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(a.o + orow * D + 32 * dt + 8 * q + 4 * hh) = make_uint2(w0, w1);
      }
  } else {
    float* po = a.part_o + (orow * NS + split) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(po + 32 * dt + 8 * q + 4 * hh) =
            make_float4(T.o[dt][4 * q], T.o[dt][4 * q + 1], T.o[dt][4 * q + 2], T.o[dt][4 * q + 3]);
    if (hh == 0)
      *reinterpret_cast<float2*>(a.part_ml + (orow * NS + split) * 2) = make_float2(T.m, lsum);
  }
}

// o[row] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits
// (zero when no split saw a key: the rows of a rejected sequence). One wave
// per output row, 64 lanes over d; workgroup (b, c) takes 4 of sequence b's
// rows (node-major, query heads inner); rows of an invalid node range are
// left alone.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(const AttnArgs a) {
  const int chunks = (a.max_nodes * a.Hq + 3) / 4;
  const int b = blockIdx.x / chunks;
  const int lo = a.offsets[b];
  const int hi = a.offsets[b + 1];
  if (lo < 0 || hi > a.T || hi - lo < 1 || hi - lo > a.max_nodes) return;
  const int row = lo * a.Hq + 4 * (blockIdx.x - b * chunks) + (threadIdx.x >> 6);
  if (row >= hi * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int NS = a.NS;
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

// One workgroup per sequence: validate, find the accepted path, append its
// K/V rows (root first) for every K/V head of every layer of the launch, then
// advance the length.
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
      put_status(a.status, b, st, a.merge);
    }
  }
  __syncthreads();
  const int st = sInfo[0];
  const int P = sInfo[1];
  const int L = sInfo[2];
  if (st != GDN_TREE_OK || P == 0) return;
  // the same rows of up to kGroup layers per pass: all their loads are in
  // flight before the first store (a layer alone is one short dependent
  // load-store round trip per thread)
  constexpr int kGroup = 8;   // the named registers below
  const int half = a.Hkv * P * CPR;            // chunks of K (then of V) per layer
  if (a.layers == 1) {
    const AttnCommitLayer& ly = a.L[0];
    for (int id = tid; id < 2 * half; id += 256) {
      const int mat = id / half;
      const int rem0 = id - mat * half;
      const int kvh = rem0 / (P * CPR);
      const int rem = rem0 - kvh * P * CPR;
      const int pr = rem / CPR;
      const int c = rem - pr * CPR;
      const uint16_t* src = (mat ? ly.v : ly.k) + ((size_t)sPath[pr] * a.Hkv + kvh) * D + 8 * c;
      uint16_t* dst =
          (mat ? ly.vc : ly.kc) + (((size_t)b * a.Hkv + kvh) * a.cap + L + pr) * D + 8 * c;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
  for (int l0 = 0; a.layers > 1 && l0 < a.layers; l0 += kGroup) {
    // layer pointers are wave-uniform: K first, then V, so that the choice
    // between them is uniform too and the pointers stay in scalar registers
    for (int mat = 0; mat < 2; ++mat) {
      for (int id = tid; id < half; id += 256) {
        const int kvh = id / (P * CPR);
        const int rem = id - kvh * P * CPR;
        const int pr = rem / CPR;
        const int c = rem - pr * CPR;
        const size_t src = ((size_t)sPath[pr] * a.Hkv + kvh) * D + 8 * c;
        const size_t dst = (((size_t)b * a.Hkv + kvh) * a.cap + L + pr) * D + 8 * c;
        // (past the last layer the last one repeats: the same bytes to the
        // same place, so no branch is needed; named registers, not an array,
        // which the compiler would keep in scratch)
        auto in = [&](int j) {
          const AttnCommitLayer& ly = a.L[min(l0 + j, a.layers - 1)];
          return *reinterpret_cast<const uint4*>((mat ? ly.v : ly.k) + src);
        };
        auto out = [&](int j, const uint4& x) {
          const AttnCommitLayer& ly = a.L[min(l0 + j, a.layers - 1)];
          *reinterpret_cast<uint4*>((mat ? ly.vc : ly.kc) + dst) = x;
        };
        const uint4 x0 = in(0), x1 = in(1), x2 = in(2), x3 = in(3);
        const uint4 x4 = in(4), x5 = in(5), x6 = in(6), x7 = in(7);
        out(0, x0), out(1, x1), out(2, x2), out(3, x3);
        out(4, x4), out(5, x5), out(6, x6), out(7, x7);
      }
    }
  }
  __syncthreads();
  if (tid == 0 && a.advance) a.cache_len[b] = L + P;
}

// Kernel from the most query rows a (sequence, K/V head) can have: up to 192
// rows, 16-row tiles on 12 waves (three per SIMD); beyond, 32-row tiles on 8
// waves (measured faster there: each LDS fragment serves twice the rows, and
// 8 tiles of 32 spread evenly over the SIMDs).
template <int D>
hipError_t launch_attn_d(const AttnArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.Hkv * a.NS);
  const int rows = (a.Hq / a.Hkv) * a.max_nodes;
  hipError_t e = rows <= 192
      ? launch_kernel(reinterpret_cast<const void*>(&tree_attn_kernel<D, 12>), grid, 768u, s, a)
      : launch_kernel(reinterpret_cast<const void*>(&tree_attn32_kernel<D, 8>), grid, 512u, s, a);
  if (e != hipSuccess || a.NS == 1) return e;
  const unsigned chunks = (unsigned)((a.max_nodes * a.Hq + 3) / 4);
  return launch_kernel(reinterpret_cast<const void*>(&tree_attn_combine_kernel<D>),
                       (unsigned)a.B * chunks, 256u, s, a);
}

}  // namespace

hipError_t launch_tree_attn(int d, const AttnArgs& a, hipStream_t s) {
  switch (d) {
    case 64: return launch_attn_d<64>(a, s);
    case 128: return launch_attn_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

// Scratch of the no-allocation verify (gdn_tree_attn_verify_noalloc): the
// split-cache partials of one call, written and then read by that call's own
// kernels. One array per GPU, held until the process ends; every call on a
// GPU shares it, so calls that overlap on one GPU race. In host code the
// name is a host-side stand-in: kernels get the device address taken below.
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

hipError_t attn_scratch(void** ptr) {
  static std::mutex mu;
  static void* by_device[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (by_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // this device's copy
    if (e != hipSuccess) return e;
    by_device[dev] = p;
  }
  *ptr = by_device[dev];
  return hipSuccess;
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
