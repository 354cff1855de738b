/*
 * gdn_oracle.c -- plain, slow CPU oracle for tree-verified Gated DeltaNet.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may call,
 * link or load this file; it exists so that tests, the smoke check and the
 * CPU-baseline leg of the benchmark can check the GPU results against a
 * definition that a reader can compare with the pages by eye.
 *
 * Arithmetic: IEEE double throughout. Inputs arrive as doubles that hold the
 * stored fp32/bf16 values exactly. No blocking, no reuse of work between
 * nodes: every node's output is obtained by running the gated delta rule from
 * the initial state along that node's own root-to-node path.
 *
 * What is computed, and where the pages define it:
 *  - Tree topology: nodes are flattened into one sequence with a parent index
 *    per node, the root first with parent -1 (rainlin-top "Qwen3.5 tree
 *    spec", section 7 step 2 "flatten the draft tree"; anrans handbook
 *    "speculative", implementation section, tree_mask/depths). A node sees
 *    itself and its ancestors and never a sibling (rainlin-top section 2,
 *    "tree attention mask review"; anrans implementation section). Depth is
 *    counted from the root = 0, as the handbook's depths() does.
 *  - Recurrence: the gated delta rule, one step per token,
 *        S_t = alpha_t * S_parent * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *        o_t = S_t q_t,
 *    with S of shape dv x dk (row r, column c; S k is a dv-vector). The
 *    formula itself is stripped from rainlin-top section 3 ("hybrid
 *    architecture challenge", the GDN state update); this reading is the
 *    standard gated delta rule that the TreeWY abstract (arxivdaily
 *    2608.20961) says its derivation depends on.
 *  - Branch isolation: each branch evolves from its own copy of the parent
 *    state (rainlin-top section 4, "Fork/Checkpoint", including its
 *    depth-by-depth batching subsection).
 *  - Commit / rollback: the state kept after verification is the state of the
 *    last accepted node (rainlin-top section 5, "dual use of checkpoints",
 *    the root->A->C example; TreeWY abstract: only the accepted state is
 *    reconstructed on commit).
 *
 * Status codes per sequence (same specification the library documents,
 * written independently here): 0 ok; 3 bad size / offsets (checked first);
 * 1 root not at index 0; 2 a parent is out of range or not smaller than its
 * child's index; 4 accepted node out of range (commit only).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAX_NODES 64

enum { ORC_OK = 0, ORC_BAD_ROOT = 1, ORC_BAD_PARENT = 2, ORC_BAD_SIZE = 3, ORC_BAD_ACCEPTED = 4 };

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Sequence b's node range [lo, hi) is valid and its parents array is a tree
 * in topological order. */
static int check_seq(int b, int T, int max_nodes, const int32_t* offsets,
                     const int32_t* parents) {
  int lo = offsets[b], hi = offsets[b + 1];
  if (lo < 0 || hi > T || hi - lo < 1 || hi - lo > max_nodes || hi - lo > ORC_MAX_NODES)
    return ORC_BAD_SIZE;
  const int32_t* p = parents + lo;
  if (p[0] != -1) return ORC_BAD_ROOT;
  for (int i = 1; i < hi - lo; ++i)
    if (p[i] < 0 || p[i] >= i) return ORC_BAD_PARENT;
  return ORC_OK;
}

/* Depth (root = 0) and the set of visible nodes (ancestors and itself, one bit
 * per local node index) of every node, by walking up to the root. */
void oracle_tree(int B, int T, int max_nodes, const int32_t* offsets, const int32_t* parents,
                 int32_t* depth, uint64_t* anc, int32_t* status) {
  for (int b = 0; b < B; ++b) {
    int st = check_seq(b, T, max_nodes, offsets, parents);
    status[b] = st;
    if (st != ORC_OK) continue;
    int lo = offsets[b], n = offsets[b + 1] - lo;
    for (int i = 0; i < n; ++i) {
      uint64_t mask = 0;
      int d = -1;
      for (int j = i; j != -1; j = parents[lo + j]) {
        mask |= (uint64_t)1 << j;
        d += 1;
      }
      depth[lo + i] = d;
      anc[lo + i] = mask;
    }
  }
}

/* One token of the gated delta rule applied to S (dv x dk, row-major):
 *   w = S k;  S <- alpha * (S - beta * w k^T) + beta * v k^T
 * which is alpha * S (I - beta k k^T) + beta v k^T written out. */
static void delta_step(int dk, int dv, double* S, const double* k, const double* v,
                       double alpha, double beta) {
  for (int r = 0; r < dv; ++r) {
    double* row = S + (size_t)r * dk;
    double w = 0.0;
    for (int c = 0; c < dk; ++c) w += row[c] * k[c];
    for (int c = 0; c < dk; ++c)
      row[c] = alpha * (row[c] - beta * w * k[c]) + beta * v[r] * k[c];
  }
}

/* out = S q */
static void read_out(int dk, int dv, const double* S, const double* q, double* out) {
  for (int r = 0; r < dv; ++r) {
    double acc = 0.0;
    for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * q[c];
    out[r] = acc;
  }
}

/* S <- S0[b,h], then one delta step per node on the root..node path of
 * sequence b (local node `node`), head h. */
static void replay_path(int H, int dk, int dv, int lo, const int32_t* parents, int node, int b,
                        int h, const double* k, const double* v, const double* alpha,
                        const double* beta, const double* S0, double* S) {
  int path[ORC_MAX_NODES];
  int len = 0;
  for (int j = node; j != -1; j = parents[lo + j]) path[len++] = j;
  memcpy(S, S0 + ((size_t)b * H + h) * dv * dk, sizeof(double) * dv * dk);
  for (int s = len - 1; s >= 0; --s) {
    size_t g = (size_t)(lo + path[s]) * H + h;
    delta_step(dk, dv, S, k + g * dk, v + g * dv, alpha[g], beta[g]);
  }
}

/* Verification of a whole batch of draft trees through one GDN layer: every
 * node's output from its own path replay. Layouts: q,k [T,H,dk]; v,o
 * [T,H,dv]; alpha,beta [T,H]; S0 [B,H,dv,dk]. Rows of sequences whose tree is
 * invalid are zero when the node range itself is valid. */
void oracle_verify(int B, int H, int dk, int dv, int T, int max_nodes, const int32_t* offsets,
                   const int32_t* parents, const double* q, const double* k, const double* v,
                   const double* alpha, const double* beta, const double* S0, double* o,
                   int32_t* status) {
  for (int b = 0; b < B; ++b) status[b] = check_seq(b, T, max_nodes, offsets, parents);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      int lo = offsets[b], hi = offsets[b + 1];
      if (status[b] != ORC_OK) {
        if (status[b] != ORC_BAD_SIZE)
          for (int t = lo; t < hi; ++t) memset(o + ((size_t)t * H + h) * dv, 0, sizeof(double) * dv);
        continue;
      }
      double* S = (double*)malloc(sizeof(double) * dv * dk);
      for (int t = 0; t < hi - lo; ++t) {
        replay_path(H, dk, dv, lo, parents, t, b, h, k, v, alpha, beta, S0, S);
        size_t g = (size_t)(lo + t) * H + h;
        read_out(dk, dv, S, q + g * dk, o + g * dv);
      }
      free(S);
    }
  }
}

/* Commit: the state of the last accepted node (local index accepted[b]);
 * -1 keeps S0. On a bad tree or a bad accepted index, S_out is not written. */
void oracle_commit(int B, int H, int dk, int dv, int T, int max_nodes, const int32_t* offsets,
                   const int32_t* parents, const int32_t* accepted, const double* k,
                   const double* v, const double* alpha, const double* beta, const double* S0,
                   double* S_out, int32_t* status) {
  for (int b = 0; b < B; ++b) {
    int st = check_seq(b, T, max_nodes, offsets, parents);
    if (st == ORC_OK) {
      int n = offsets[b + 1] - offsets[b];
      if (accepted[b] < -1 || accepted[b] >= n) st = ORC_BAD_ACCEPTED;
    }
    status[b] = st;
  }
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      if (status[b] != ORC_OK) continue;
      size_t base = ((size_t)b * H + h) * dv * dk;
      if (accepted[b] == -1) {
        memcpy(S_out + base, S0 + base, sizeof(double) * dv * dk);
        continue;
      }
      replay_path(H, dk, dv, offsets[b], parents, accepted[b], b, h, k, v, alpha, beta, S0,
                  S_out + base);
    }
  }
}

/* Depth-by-depth fork/checkpoint replay of one batch (rainlin-top section 4,
 * depth-by-depth subsection): level 0 is the root, stepped from S0; every
 * node of level l > 0 starts from a copy of its parent's checkpoint. ckpt is
 * [T,H,dv,dk] and receives every node's state; o is [T,H,dv]. Used to check
 * that fork replay and per-path replay agree. Invalid sequences are skipped. */
void oracle_fork_replay(int B, int H, int dk, int dv, int T, int max_nodes,
                        const int32_t* offsets, const int32_t* parents, const double* q,
                        const double* k, const double* v, const double* alpha,
                        const double* beta, const double* S0, double* o, double* ckpt,
                        int32_t* status) {
  for (int b = 0; b < B; ++b) status[b] = check_seq(b, T, max_nodes, offsets, parents);
  const size_t SS = (size_t)dv * dk;
  for (int b = 0; b < B; ++b) {
    if (status[b] != ORC_OK) continue;
    int lo = offsets[b], n = offsets[b + 1] - lo;
    int level[ORC_MAX_NODES];
    int maxlevel = 0;
    for (int i = 0; i < n; ++i) {
      int d = 0;
      for (int j = parents[lo + i]; j != -1; j = parents[lo + j]) d++;
      level[i] = d;
      if (d > maxlevel) maxlevel = d;
    }
    for (int l = 0; l <= maxlevel; ++l) {
      for (int i = 0; i < n; ++i) {
        if (level[i] != l) continue;
        for (int h = 0; h < H; ++h) {
          size_t g = (size_t)(lo + i) * H + h;
          double* C = ckpt + g * SS;
          int p = parents[lo + i];
          const double* src = (p == -1) ? S0 + ((size_t)b * H + h) * SS
                                        : ckpt + ((size_t)(lo + p) * H + h) * SS;
          memcpy(C, src, sizeof(double) * SS);
          delta_step(dk, dv, C, k + g * dk, v + g * dv, alpha[g], beta[g]);
          read_out(dk, dv, C, q + g * dk, o + g * dv);
        }
      }
    }
  }
}

/* Plain sequential recurrence over n tokens of one head (no tree): token t is
 * the t-th row of q,k [n,dk], v [n,dv], gates [n]. Returns every output and
 * the state after all n tokens. */
void oracle_chain(int n, int dk, int dv, const double* q, const double* k, const double* v,
                  const double* alpha, const double* beta, const double* S0, double* o,
                  double* S_final) {
  memcpy(S_final, S0, sizeof(double) * dv * dk);
  for (int t = 0; t < n; ++t) {
    delta_step(dk, dv, S_final, k + (size_t)t * dk, v + (size_t)t * dv, alpha[t], beta[t]);
    read_out(dk, dv, S_final, q + (size_t)t * dk, o + (size_t)t * dv);
  }
}

/* ---------------------------------------------------------------- selective fork
 *
 * Selective fork (rainlin-top section 8, "selective fork"): the draft's
 * confidence in each node decides whether the depth-by-depth fork keeps a
 * rollback point for it. A node whose confidence is above the threshold
 * (the page: 0.95) is processed without saving a checkpoint; one at or below
 * it forks and saves one, as in section 4. Reading taken here: a node whose
 * state was not saved is never lost, only not stored; where it is needed
 * later (as a parent during verify, or as the accepted node at commit) it is
 * recomputed from the nearest saved ancestor (S0 above the root) by applying
 * the delta steps of the unsaved nodes in between. */

/* State of local node `node` of sequence b, head h, rebuilt from the saved
 * checkpoints: start at the nearest saved node on its root path (the node
 * itself included), or at S0 when none is saved, and apply the steps of the
 * path nodes below that start. */
static void rebuild_state(int H, int dk, int dv, int lo, const int32_t* parents,
                          const int32_t* kept, const double* ckpt, int node, int b, int h,
                          const double* k, const double* v, const double* alpha,
                          const double* beta, const double* S0, double* S) {
  const size_t SS = (size_t)dv * dk;
  int path[ORC_MAX_NODES];
  int len = 0;
  int start = -1;                   /* a saved node on the path, or -1 */
  for (int j = node; j != -1; j = parents[lo + j]) {
    if (kept[lo + j]) {
      start = j;
      break;
    }
    path[len++] = j;                /* unsaved nodes, deepest first */
  }
  if (start >= 0)
    memcpy(S, ckpt + ((size_t)(lo + start) * H + h) * SS, sizeof(double) * SS);
  else
    memcpy(S, S0 + ((size_t)b * H + h) * SS, sizeof(double) * SS);
  for (int s = len - 1; s >= 0; --s) {
    size_t g = (size_t)(lo + path[s]) * H + h;
    delta_step(dk, dv, S, k + g * dk, v + g * dv, alpha[g], beta[g]);
  }
}

/* Verify with selective fork, depth by depth: every node of level l starts
 * from its parent's state (the saved checkpoint, or rebuilt as above; S0 for
 * the root), takes its own delta step, emits o = S q, and saves its state
 * iff conf <= threshold (kept[t] = 1). ckpt [T,H,dv,dk]: saved states at the
 * node's own index, other entries untouched. */
void oracle_selective_fork(int B, int H, int dk, int dv, int T, int max_nodes,
                           const int32_t* offsets, const int32_t* parents, const double* conf,
                           double threshold, const double* q, const double* k, const double* v,
                           const double* alpha, const double* beta, const double* S0, double* o,
                           double* ckpt, int32_t* kept, int32_t* status) {
  for (int b = 0; b < B; ++b) status[b] = check_seq(b, T, max_nodes, offsets, parents);
  const size_t SS = (size_t)dv * dk;
  for (int b = 0; b < B; ++b) {
    if (status[b] != ORC_OK) continue;
    int lo = offsets[b], n = offsets[b + 1] - lo;
    int level[ORC_MAX_NODES];
    int maxlevel = 0;
    for (int i = 0; i < n; ++i) {
      int d = 0;
      for (int j = parents[lo + i]; j != -1; j = parents[lo + j]) d++;
      level[i] = d;
      if (d > maxlevel) maxlevel = d;
      kept[lo + i] = 0;
    }
    double* S = (double*)malloc(sizeof(double) * SS);
    for (int l = 0; l <= maxlevel; ++l) {
      for (int i = 0; i < n; ++i) {
        if (level[i] != l) continue;
        const int keep = conf[lo + i] <= threshold;
        for (int h = 0; h < H; ++h) {
          size_t g = (size_t)(lo + i) * H + h;
          int p = parents[lo + i];
          if (p == -1)
            memcpy(S, S0 + ((size_t)b * H + h) * SS, sizeof(double) * SS);
          else
            rebuild_state(H, dk, dv, lo, parents, kept, ckpt, p, b, h, k, v, alpha, beta, S0, S);
          delta_step(dk, dv, S, k + g * dk, v + g * dv, alpha[g], beta[g]);
          read_out(dk, dv, S, q + g * dk, o + g * dv);
          if (keep) memcpy(ckpt + g * SS, S, sizeof(double) * SS);
        }
        kept[lo + i] = keep;
      }
    }
    free(S);
  }
}

/* Commit after a selective-fork verify: the accepted node's state, from its
 * saved checkpoint when it has one, else rebuilt from the nearest saved
 * ancestor (S0 when none); -1 keeps S0. kept and ckpt as verify left them.
 * Status as oracle_commit. */
void oracle_selective_commit(int B, int H, int dk, int dv, int T, int max_nodes,
                             const int32_t* offsets, const int32_t* parents, const int32_t* kept,
                             const int32_t* accepted, const double* ckpt, const double* k,
                             const double* v, const double* alpha, const double* beta,
                             const double* S0, double* S_out, int32_t* status) {
  for (int b = 0; b < B; ++b) {
    int st = check_seq(b, T, max_nodes, offsets, parents);
    if (st == ORC_OK) {
      int n = offsets[b + 1] - offsets[b];
      if (accepted[b] < -1 || accepted[b] >= n) st = ORC_BAD_ACCEPTED;
    }
    status[b] = st;
  }
  const size_t SS = (size_t)dv * dk;
  for (int b = 0; b < B; ++b) {
    if (status[b] != ORC_OK) continue;
    for (int h = 0; h < H; ++h) {
      size_t base = ((size_t)b * H + h) * SS;
      if (accepted[b] == -1)
        memcpy(S_out + base, S0 + base, sizeof(double) * SS);
      else
        rebuild_state(H, dk, dv, offsets[b], parents, kept, ckpt, accepted[b], b, h, k, v,
                      alpha, beta, S0, S_out + base);
    }
  }
}
