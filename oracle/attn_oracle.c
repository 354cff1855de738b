/*
 * attn_oracle.c -- plain, slow CPU oracle for tree-masked attention verify
 * and the accepted-path KV-cache commit (the full-attention layers of a
 * hybrid model under a speculative draft tree).
 *
 * TEST INFRASTRUCTURE ONLY, like gdn_oracle.c: tests, the smoke check and the
 * benchmark's CPU-baseline leg use it; the library never calls it.
 *
 * What is computed (anrans handbook "speculative", implementation section:
 * the tree tokens see the whole cached prefix and, among the tree tokens,
 * themselves and their ancestors; K/V heads are shared by groups of query
 * heads; after verification only the K/V rows of the accepted path are
 * appended to the cache, in path order, without recomputation. rainlin-top
 * "Qwen3.5 tree spec", section 7 step 4: the full-attention layers keep the
 * accepted tokens' KV cache and drop the rejected ones):
 *
 *   for sequence b with cached length L_b, tree node t, query head h, and the
 *   KV head j = h / (Hq / Hkv):
 *     visible keys  = cache positions 0 .. L_b-1, then the tree nodes on the
 *                     path from the root to t (t included);
 *     score_x       = scale * <q[t,h], key_x>;
 *     o[t,h]        = sum_x softmax(score)_x * value_x.
 *
 *   commit: for the accepted node a, the path root = p_0, ..., p_m = a is
 *   appended: cache[b, j, L_b + r] = (k[p_r, j], v[p_r, j]), r = 0..m, and
 *   L_b += m + 1. a = -1 appends nothing.
 *
 * Arithmetic: IEEE double; inputs arrive as doubles holding the stored bf16
 * values exactly. Every output is computed separately, with the maximum
 * score subtracted before exponentiation.
 *
 * Status codes per sequence: 0 ok; 3 bad size (checked first); 1 root not at
 * index 0; 2 a parent out of range or not smaller than its child; 4 accepted
 * node out of range (commit); 6 the cache would overflow its capacity
 * (commit).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { AO_OK = 0, AO_BAD_ROOT = 1, AO_BAD_PARENT = 2, AO_BAD_SIZE = 3, AO_BAD_ACCEPTED = 4,
       AO_CACHE_FULL = 6 };

static int attn_check_seq(int b, int T, int max_nodes, const int32_t* offsets,
                          const int32_t* parents) {
  int lo = offsets[b], hi = offsets[b + 1];
  if (lo < 0 || hi > T || hi - lo < 1 || hi - lo > max_nodes || hi - lo > 64) return AO_BAD_SIZE;
  const int32_t* p = parents + lo;
  if (p[0] != -1) return AO_BAD_ROOT;
  for (int i = 1; i < hi - lo; ++i)
    if (p[i] < 0 || p[i] >= i) return AO_BAD_PARENT;
  return AO_OK;
}

/* Tree-masked attention for every node of every sequence.
 * q [T,Hq,d], k/v [T,Hkv,d], kc/vc [B,Hkv,cap,d], cache_len [B]; o [T,Hq,d].
 * Rows of a sequence with a nonzero status are set to zero. */
void oracle_tree_attn(int B, int Hq, int Hkv, int d, int T, int max_nodes, int cap,
                      const int32_t* offsets, const int32_t* parents, const double* q,
                      const double* k, const double* v, const double* kc, const double* vc,
                      const int32_t* cache_len, double scale, double* o, int32_t* status) {
  const int G = Hq / Hkv;
  for (int b = 0; b < B; ++b) {
    int st = attn_check_seq(b, T, max_nodes, offsets, parents);
    const int L = cache_len[b];
    if (st == AO_OK && (L < 0 || L > cap)) st = AO_BAD_SIZE;
    status[b] = st;
    if (st != AO_OK) {
      int lo = offsets[b], hi = offsets[b + 1];
      if (lo >= 0 && hi <= T)
        for (int t = lo; t < hi; ++t) memset(o + (size_t)t * Hq * d, 0, sizeof(double) * Hq * d);
      continue;
    }
    const int lo = offsets[b], n = offsets[b + 1] - lo;
#pragma omp parallel for collapse(2) schedule(static) if (n * Hq > 8)
    for (int t = 0; t < n; ++t) {
      for (int h = 0; h < Hq; ++h) {
        /* (each (t, h) uses its own score buffer) */
        double* s = (double*)malloc(sizeof(double) * (size_t)(L + n));
        int pth[64], m = 0;
        for (int j = t; j != -1; j = parents[lo + j]) pth[m++] = j;
        const int kv = h / G;
        const double* qv = q + ((size_t)(lo + t) * Hq + h) * d;
        double mx = -INFINITY;
        for (int x = 0; x < L + m; ++x) {
          const double* key = x < L ? kc + (((size_t)b * Hkv + kv) * cap + x) * d
                                    : k + ((size_t)(lo + pth[x - L]) * Hkv + kv) * d;
          double dot = 0.0;
          for (int c = 0; c < d; ++c) dot += qv[c] * key[c];
          s[x] = scale * dot;
          if (s[x] > mx) mx = s[x];
        }
        double den = 0.0;
        for (int x = 0; x < L + m; ++x) {
          s[x] = exp(s[x] - mx);
          den += s[x];
        }
        double* out = o + ((size_t)(lo + t) * Hq + h) * d;
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        for (int x = 0; x < L + m; ++x) {
          const double* val = x < L ? vc + (((size_t)b * Hkv + kv) * cap + x) * d
                                    : v + ((size_t)(lo + pth[x - L]) * Hkv + kv) * d;
          const double w = s[x] / den;
          for (int c = 0; c < d; ++c) out[c] += w * val[c];
        }
        free(s);
      }
    }
  }
}

/* Append the accepted path's K/V rows to the cache (kc/vc [B,Hkv,cap,d],
 * updated in place) and advance cache_len. */
void oracle_tree_attn_commit(int B, int Hkv, int d, int T, int max_nodes, int cap,
                             const int32_t* offsets, const int32_t* parents,
                             const int32_t* accepted, const double* k, const double* v,
                             double* kc, double* vc, int32_t* cache_len, int32_t* status) {
  for (int b = 0; b < B; ++b) {
    int st = attn_check_seq(b, T, max_nodes, offsets, parents);
    const int L = cache_len[b];
    if (st == AO_OK && (L < 0 || L > cap)) st = AO_BAD_SIZE;
    const int lo = offsets[b];
    const int n = st == AO_OK ? offsets[b + 1] - lo : 0;
    const int a = accepted[b];
    if (st == AO_OK && (a < -1 || a >= n)) st = AO_BAD_ACCEPTED;
    int pth[64], m = 0;
    if (st == AO_OK && a >= 0) {
      for (int j = a; j != -1; j = parents[lo + j]) pth[m++] = j;
      if (L + m > cap) st = AO_CACHE_FULL;
    }
    status[b] = st;
    if (st != AO_OK || a < 0) continue;
    /* pth holds a .. root; the cache receives root first */
    for (int r = 0; r < m; ++r) {
      const int node = pth[m - 1 - r];
      for (int kv = 0; kv < Hkv; ++kv) {
        memcpy(kc + (((size_t)b * Hkv + kv) * cap + L + r) * d,
               k + ((size_t)(lo + node) * Hkv + kv) * d, sizeof(double) * d);
        memcpy(vc + (((size_t)b * Hkv + kv) * cap + L + r) * d,
               v + ((size_t)(lo + node) * Hkv + kv) * d, sizeof(double) * d);
      }
    }
    cache_len[b] = L + m;
  }
}
