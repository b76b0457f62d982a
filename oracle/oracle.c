/*
 * oracle.c -- plain, slow CPU reference for the target-model verification step of
 * EAGLE-style tree speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker for the HIP
 * library: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper with
 * the GPU path, and the GPU path never calls it.
 *
 * Everything is computed in double precision with scalar loops in the order the
 * definitions state.  Inputs arrive in the dtype the GPU path consumes (fp32
 * logits, fp32/bf16 activations) and are widened to double exactly on read.
 *
 * Sources (the four pages this build follows):
 *   [GL]  "Eagle vs DFlash: Best speculative decoding methods" (gingerlabs.ai),
 *         section "Target-model decoding is serial" (acceptance rule and residual)
 *         and "A useful performance model" (tau counts the bonus token).
 *   [FAL] "EAGLE-4 Technical Deepdive" (blog.fal.ai), section "EAGLE-4
 *         verification trees and harness" (prefix + ancestors + self mask).
 *   [ZS]  "EAGLE 演化史 (1 → 2 → 3) 与 DFlash 的回答" (zhangshuibai.github.io paper
 *         notes), section "Tree Verification 详解", parts A-G.
 *   [CE]  "The EAGLE Family: Speculating in Feature Space" (consciousengines.com),
 *         "Why predict features instead of tokens?" (softmax of the LM head) and
 *         "EAGLE-1: feature-level autoregression" (ancestor-only tree attention).
 *
 * Parity status per function:
 *   oracle_mask             pinned (hand-built 7-node tree, chain, star)
 *   oracle_tree_attention   pinned (causal equivalence vs a library attention)
 *   oracle_softmax          pinned (library softmax, row sums)
 *   oracle_reject_sample    pinned (worked example, chi-square, alpha^d, product of
 *                           per-level alphas, greedy vs target-only decode, special
 *                           cases; near-tie bands: hand-derived first-order widths of
 *                           a later-sibling test and of draws from p and from a
 *                           residual, each probed just inside and just outside)
 *   oracle_accept_path      pinned (worked example)
 *   oracle_kv_commit        pinned (hand-checked moves on a small cache, both
 *                           layouts; untouched positions; page release)
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Return codes (the oracle's own; they mirror nothing). */
#define ORC_OK 0
#define ORC_EARG -1
#define ORC_EDATA -2
#define ORC_ENOMEM -3

/* Per-node markers in the sampling outputs. */
#define ORC_NOT_EVALUATED -2 /* node not visited by the walk (lazy mode)   */
#define ORC_NONE -1          /* no child accepted / no next node           */
#define ORC_BAD_REQUEST -3   /* request rejected: malformed tree or tokens */

/* Near-tie flag bits, per node. */
#define ORC_TIE_TEST 1 /* an acceptance test landed inside its uncertainty band */
#define ORC_TIE_DRAW 2 /* an inverse-CDF draw landed inside a bin-edge band     */

/* ------------------------------------------------------------------------- */
/* O1. Ancestor sets.                                                          */
/* [ZS] part B: the tree is flattened in BFS order and each node may see only   */
/* its own ancestors and itself (never siblings or cousins).  [FAL] states the  */
/* same mask.  Node 0 is the root.  Any order with parent[i] < i is accepted,   */
/* since BFS order is one such order.                                           */
/* ------------------------------------------------------------------------- */

/* Returns 1 when request b's parent links form a tree rooted at node 0. */
static int tree_is_valid(const int32_t* par, int32_t n, int32_t n_max) {
  if (n < 1 || n > n_max || n > 64) return 0;
  if (par[0] != -1) return 0;
  for (int32_t i = 1; i < n; ++i)
    if (par[i] < 0 || par[i] >= i) return 0;
  return 1;
}

int oracle_mask(const int32_t* parent, const int32_t* n_nodes, int32_t batch, int32_t n_max,
                uint64_t* anc, uint64_t* child, int32_t* depth, int32_t* valid) {
  if (!parent || !n_nodes || !anc || !child || !depth || !valid) return ORC_EARG;
  if (batch < 0 || n_max < 1 || n_max > 64) return ORC_EARG;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t* par = parent + (int64_t)b * n_max;
    uint64_t* A = anc + (int64_t)b * n_max;
    uint64_t* C = child + (int64_t)b * n_max;
    int32_t* D = depth + (int64_t)b * n_max;
    int32_t n = n_nodes[b];
    for (int32_t i = 0; i < n_max; ++i) {
      A[i] = 0;
      C[i] = 0;
      D[i] = -1;
    }
    valid[b] = tree_is_valid(par, n, n_max);
    if (!valid[b]) continue;
    /* anc(0) = {0}; anc(i) = anc(parent(i)) + {i}; depth(i) = depth(parent(i)) + 1 */
    A[0] = 1ull;
    D[0] = 0;
    for (int32_t i = 1; i < n; ++i) {
      A[i] = A[par[i]] | (1ull << i);
      D[i] = D[par[i]] + 1;
      C[par[i]] |= (1ull << i);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O2. Tree-masked attention.                                                  */
/* [ZS] part B: a node's hidden state equals what an ordinary causal run of     */
/* prompt + Path(root, node) would give, because the node attends to exactly    */
/* the prompt, its ancestors and itself.  [ZS] part D.2: the node-to-prompt     */
/* part is O(N*P), the node-to-tree part is sparse.                             */
/*                                                                              */
/* For request b, node i, query head h (KV head g = h / (hq/hkv)):               */
/*   keys  = prompt positions [0, ctx_b)  +  tree slots ctx_b + j, j in anc(i)    */
/*   s_t   = scale * <q, k_t>,  w = softmax(s),  o = sum_t w_t v_t               */
/* K/V hold logical positions [0, ctx_b + n_b); tree node j lives at ctx_b + j.  */
/* ------------------------------------------------------------------------- */

static double load_act(const void* base, int64_t idx, int32_t dtype) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Element offset of (request b, logical position t, KV head g, dim 0), or -1. */
static int64_t kv_offset(int32_t b, int32_t t, int32_t g, const int32_t* block_table, int32_t page_size,
                         int32_t kv_capacity, int32_t n_pages, int32_t hkv, int32_t d) {
  if (!block_table) {
    if (t < 0 || t >= kv_capacity) return -1;
    return (((int64_t)b * kv_capacity + t) * hkv + g) * d;
  }
  int32_t slot = t / page_size;
  if (t < 0 || slot >= kv_capacity) return -1;
  int32_t page = block_table[(int64_t)b * kv_capacity + slot];
  if (page < 0 || page >= n_pages) return -1;
  return (((int64_t)page * page_size + t % page_size) * hkv + g) * d;
}

/*
 * Computes output rows listed in rows[r] = (b, i, h).  Padding nodes (i >= n_b) and
 * requests whose tree is invalid produce zero rows.  q is [B, n_max, hq, d]; k and v
 * are [B, kv_capacity, hkv, d] (block_table == NULL) or a paged pool
 * [n_pages, page_size, hkv, d] with block_table [B, kv_capacity] (pages per request).
 * Returns ORC_EDATA if a listed row needs a position outside the cache.
 */
int oracle_tree_attention(const void* q, const void* k, const void* v, int32_t dtype,
                          const int32_t* block_table, int32_t page_size, int32_t kv_capacity, int32_t n_pages,
                          const int32_t* ctx_len, const int32_t* n_nodes, const uint64_t* anc, int32_t batch,
                          int32_t n_max, int32_t hq, int32_t hkv, int32_t d, double scale, const int32_t* rows,
                          int32_t n_rows, double* out) {
  if (!q || !k || !v || !ctx_len || !n_nodes || !anc || !rows || !out) return ORC_EARG;
  if (hkv < 1 || hq < hkv || hq % hkv != 0 || d < 1 || n_max < 1 || n_max > 64) return ORC_EARG;
  if (block_table && page_size < 1) return ORC_EARG;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < n_rows; ++r) {
    int32_t b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
    double* o = out + (int64_t)r * d;
    for (int32_t x = 0; x < d; ++x) o[x] = 0.0;
    if (b < 0 || b >= batch || i < 0 || i >= n_max || h < 0 || h >= hq) continue;
    int32_t n = n_nodes[b], ctx = ctx_len[b];
    uint64_t mask = anc[(int64_t)b * n_max + i];
    if (i >= n || mask == 0) continue;
    int32_t g = h / (hq / hkv);
    int32_t n_keys = ctx + n;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_keys > 0 ? n_keys : 1));
    if (!s || !off) {
      free(s);
      free(off);
#pragma omp atomic write
      status = ORC_ENOMEM;
      continue;
    }
    /* gather the visible key positions in logical order: prompt, then ancestors */
    int32_t m = 0;
    int bad = 0;
    for (int32_t t = 0; t < ctx; ++t) off[m++] = kv_offset(b, t, g, block_table, page_size, kv_capacity, n_pages, hkv, d);
    for (int32_t j = 0; j < n; ++j)
      if ((mask >> j) & 1ull) off[m++] = kv_offset(b, ctx + j, g, block_table, page_size, kv_capacity, n_pages, hkv, d);
    for (int32_t t = 0; t < m; ++t)
      if (off[t] < 0) bad = 1;
    if (bad) {
      free(s);
      free(off);
#pragma omp atomic write
      status = ORC_EDATA;
      continue;
    }
    int64_t qoff = (((int64_t)b * n_max + i) * hq + h) * d;
    double smax = -INFINITY;
    for (int32_t t = 0; t < m; ++t) {
      double dot = 0.0;
      for (int32_t x = 0; x < d; ++x) dot += load_act(q, qoff + x, dtype) * load_act(k, off[t] + x, dtype);
      s[t] = scale * dot;
      if (s[t] > smax) smax = s[t];
    }
    double z = 0.0;
    for (int32_t t = 0; t < m; ++t) {
      s[t] = exp(s[t] - smax);
      z += s[t];
    }
    for (int32_t t = 0; t < m; ++t) {
      double w = s[t] / z;
      for (int32_t x = 0; x < d; ++x) o[x] += w * load_act(v, off[t] + x, dtype);
    }
    free(s);
    free(off);
  }
  return status;
}

/* ------------------------------------------------------------------------- */
/* O3. Per-node vocabulary softmax at temperature T.                           */
/* [CE] "Why predict features instead of tokens?": the next-token distribution   */
/* is the softmax of the LM-head output.  [ZS] part A / D.2: one softmax per     */
/* tree node, N*|V| elements per verify.                                        */
/*   m = max_x l(x);  Z = sum_x exp((l(x) - m)/T);  p(x) = exp((l(x) - m)/T) / Z  */
/* T == 0 is greedy: argmax, lowest index on ties.  -inf logits are allowed     */
/* (probability 0); NaN or +inf make the row invalid.                           */
/* ------------------------------------------------------------------------- */

/* Returns 0 when the row is usable, and fills max, sum of exp, argmax. */
static int row_stats(const float* l, int32_t vocab, double T, double* m_out, double* z_out, int32_t* am_out) {
  double m = -INFINITY;
  int32_t am = -1;
  for (int32_t x = 0; x < vocab; ++x) {
    double lx = (double)l[x];
    if (isnan(lx) || lx == INFINITY) return -1;
    if (lx > m) {
      m = lx;
      am = x;
    }
  }
  if (am < 0) return -1; /* every logit is -inf */
  double z = 0.0;
  if (T > 0.0)
    for (int32_t x = 0; x < vocab; ++x) z += exp(((double)l[x] - m) / T);
  *m_out = m;
  *z_out = z;
  *am_out = am;
  return 0;
}

int oracle_softmax(const float* logits, int64_t rows, int32_t vocab, double T, double* probs, double* row_max,
                   double* row_sumexp, int32_t* row_argmax, int32_t* row_valid) {
  if (!logits || vocab < 1 || rows < 0 || !(T >= 0.0)) return ORC_EARG;
  for (int64_t r = 0; r < rows; ++r) {
    const float* l = logits + r * vocab;
    double m = NAN, z = NAN;
    int32_t am = -1;
    int ok = row_stats(l, vocab, T, &m, &z, &am) == 0;
    if (row_valid) row_valid[r] = ok;
    if (row_max) row_max[r] = ok ? m : NAN;
    if (row_sumexp) row_sumexp[r] = ok ? z : NAN;
    if (row_argmax) row_argmax[r] = ok ? am : -1;
    if (probs && T > 0.0)
      for (int32_t x = 0; x < vocab; ++x) probs[r * vocab + x] = ok ? exp(((double)l[x] - m) / T) / z : NAN;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O4. Tree rejection sampling, one parent node at a time.                      */
/*                                                                              */
/* [GL] "Target-model decoding is serial": a drafted token x is accepted with    */
/* probability min(1, p(x)/q(x)); on rejection the replacement comes from the    */
/* normalised residual max(0, p - q).                                            */
/* [ZS] part C: the draft distribution of a node is the one produced at its      */
/* parent (siblings share it).  Children are tried one after another; after a    */
/* rejection the rejected draft mass is taken out of the parent's target         */
/* distribution (residual) and the next sibling is tested against that residual; */
/* if every sibling fails, the bonus token is drawn from the residual at the     */
/* parent.  [ZS] part G, step 6: at a leaf the bonus comes from the target       */
/* distribution of that leaf.  The committed path is the unique walk from the    */
/* root to the first rejection or a leaf.                                        */
/*                                                                              */
/* Readings where the pages are silent (each stated once here):                  */
/*  - children are tested in ascending node index (the producer orders them);    */
/*  - the test of child c consumes u_accept[c]; the terminal draw at node n      */
/*    consumes u_sample[n], so results do not depend on evaluation order;        */
/*  - acceptance is the strict comparison u < r(x)/q(x); when q(x) = 0 the ratio */
/*    is +inf if r(x) > 0 and 0 otherwise;                                       */
/*  - a zero-mass residual (r <= q everywhere) leaves r unchanged;               */
/*  - the inverse-CDF draw returns the smallest k whose running sum (ascending   */
/*    token order) exceeds u * S; if rounding leaves none, the largest token     */
/*    with positive mass;                                                        */
/*  - T == 0 is greedy: the first child whose token equals argmax p is accepted, */
/*    and the terminal token is that argmax.                                     */
/*                                                                              */
/* Near-tie bookkeeping.  The decisions above use the plain iterated residual.  */
/* Separately, every probability is given an uncertainty box [x(1-eps),        */
/* x(1+eps)] and each decision boundary is enclosed over that box; a decision  */
/* whose uniform falls inside its enclosure is flagged, since an implementation */
/* whose probabilities carry relative error below eps may take either branch.   */
/* Accept tests are also flagged when |u - ratio| < 1e-5.                       */
/*                                                                              */
/* The enclosure uses an identity of the iterated residual with a fixed q: after */
/* j rejections r_j = max(0, p - c_j q) / W(c_j), W(c) = sum_x max(0, p - c q),  */
/* c_0 = 0 and c_{j+1} = c_j + W(c_j) (a zero-mass step leaves c unchanged, as   */
/* it leaves r unchanged).  Enclosing the scalar c instead of the whole vector r */
/* keeps the bands from compounding across sibling levels.                      */
/* ------------------------------------------------------------------------- */

typedef struct {
  int32_t vocab;
  double eps;
  /* scratch, length vocab each */
  double *p, *q, *r, *w, *p_lo, *p_hi, *q_lo, *q_hi, *w_lo, *w_hi;
} node_ws;

static int ws_alloc(node_ws* ws, int32_t vocab, double eps) {
  ws->vocab = vocab;
  ws->eps = eps;
  double** f[] = {&ws->p, &ws->q, &ws->r, &ws->w, &ws->p_lo, &ws->p_hi, &ws->q_lo, &ws->q_hi, &ws->w_lo, &ws->w_hi};
  int ok = 1;
  for (size_t j = 0; j < sizeof f / sizeof f[0]; ++j) {
    *f[j] = (double*)malloc(sizeof(double) * (size_t)vocab);
    if (!*f[j]) ok = 0;
  }
  return ok;
}

static void ws_free(node_ws* ws) {
  double* f[] = {ws->p, ws->q, ws->r, ws->w, ws->p_lo, ws->p_hi, ws->q_lo, ws->q_hi, ws->w_lo, ws->w_hi};
  for (size_t j = 0; j < sizeof f / sizeof f[0]; ++j) free(f[j]);
}

/* p(x) = exp((l(x) - m)/T) / Z, written into out; returns -1 on an invalid row. */
static int row_probs(const float* l, int32_t vocab, double T, double* out) {
  double m, z;
  int32_t am;
  if (row_stats(l, vocab, T, &m, &z, &am) != 0) return -1;
  for (int32_t x = 0; x < vocab; ++x) out[x] = exp(((double)l[x] - m) / T) / z;
  return 0;
}

/* Ratio r/q with the q == 0 convention. */
static double accept_ratio(double r, double q) {
  if (q > 0.0) return r / q;
  return r > 0.0 ? INFINITY : 0.0;
}

/* Smallest / largest W(c) = sum max(0, p - c q) over the box, at a fixed c. */
static double W_min(const node_ws* ws, double c) {
  double s = 0.0;
  for (int32_t x = 0; x < ws->vocab; ++x) s += fmax(0.0, ws->p_lo[x] - c * ws->q_hi[x]);
  return s;
}
static double W_max(const node_ws* ws, double c) {
  double s = 0.0;
  for (int32_t x = 0; x < ws->vocab; ++x) s += fmax(0.0, ws->p_hi[x] - c * ws->q_lo[x]);
  return s;
}

/*
 * Inverse-CDF draw from unnormalised masses w (ascending token order).  Also
 * reports whether u lies inside the enclosure of either edge of the chosen bin,
 * given element-wise bounds [w_lo, w_hi].
 */
static int32_t invcdf_draw(const double* w, const double* w_lo, const double* w_hi, int32_t vocab, double u,
                           int* tie) {
  double S = 0.0;
  for (int32_t x = 0; x < vocab; ++x) S += w[x];
  double target = u * S;
  double F = 0.0;
  int32_t k = -1;
  for (int32_t x = 0; x < vocab; ++x) {
    F += w[x];
    if (F > target) {
      k = x;
      break;
    }
  }
  if (k < 0) {
    for (int32_t x = vocab - 1; x >= 0; --x)
      if (w[x] > 0.0) {
        k = x;
        break;
      }
  }
  *tie = 0;
  if (k < 0) return k;
  /* Edges F(k-1)/S and F(k)/S.  F/S = F/(F + R) grows with F and falls with R, so
     the extreme values pair the low sums on one side with the high sums on the other. */
  double Fl_lo = 0.0, Fl_hi = 0.0; /* tokens below k */
  double Rr_lo = 0.0, Rr_hi = 0.0; /* tokens above k */
  for (int32_t x = 0; x < k; ++x) {
    Fl_lo += w_lo[x];
    Fl_hi += w_hi[x];
  }
  for (int32_t x = k + 1; x < vocab; ++x) {
    Rr_lo += w_lo[x];
    Rr_hi += w_hi[x];
  }
  double den;
  den = Fl_lo + w_hi[k] + Rr_hi;
  double e0_lo = den > 0.0 ? Fl_lo / den : 0.0;
  den = Fl_hi + w_lo[k] + Rr_lo;
  double e0_hi = den > 0.0 ? Fl_hi / den : 1.0;
  den = Fl_lo + w_lo[k] + Rr_hi;
  double e1_lo = den > 0.0 ? (Fl_lo + w_lo[k]) / den : 0.0;
  den = Fl_hi + w_hi[k] + Rr_lo;
  double e1_hi = den > 0.0 ? (Fl_hi + w_hi[k]) / den : 1.0;
  if (u >= e0_lo && u <= e0_hi) *tie = 1;
  if (u >= e1_lo && u <= e1_hi) *tie = 1;
  return k;
}

typedef struct {
  const float *tgt, *dft; /* [B, n_max, vocab] */
  double T, Td;
  const int32_t *tokens, *parent, *n_nodes;
  const float *u_accept, *u_sample;
  int32_t n_max, vocab;
} verify_in;

/*
 * Outcome of node n of request b: the accepted child (or ORC_NONE) and, when no
 * child is accepted, the terminal token.  Returns -1 on an invalid logit row.
 */
static int eval_node(const verify_in* in, int32_t b, int32_t n, node_ws* ws, int32_t* acc_out, int32_t* term_out,
                     int32_t* flags) {
  const int32_t V = in->vocab;
  const int64_t row = (int64_t)b * in->n_max + n;
  const float* lt = in->tgt + row * V;
  const int32_t nb = in->n_nodes[b];
  const int32_t* par = in->parent + (int64_t)b * in->n_max;
  const int32_t* tok = in->tokens + (int64_t)b * in->n_max;
  *flags = 0;
  *acc_out = ORC_NONE;
  *term_out = ORC_NOT_EVALUATED;

  if (in->T == 0.0) { /* greedy */
    double m, z;
    int32_t am;
    if (row_stats(lt, V, 0.0, &m, &z, &am) != 0) return -1;
    for (int32_t c = n + 1; c < nb; ++c)
      if (par[c] == n && tok[c] == am) {
        *acc_out = c;
        return 0;
      }
    *term_out = am;
    return 0;
  }

  const float* ua = in->u_accept + (int64_t)b * in->n_max;
  const float* us = in->u_sample + (int64_t)b * in->n_max;
  const double eps = ws->eps;
  if (row_probs(lt, V, in->T, ws->p) != 0) return -1;
  /* [ZS] part C: q is the draft distribution produced at this node and serves only
     to test this node's children; a leaf has none, so its draft row takes no part
     (its bonus is drawn from p, part G) and is not read */
  int has_kids = 0;
  for (int32_t c = n + 1; c < nb && !has_kids; ++c) has_kids = par[c] == n;
  if (has_kids) {
    if (row_probs(in->dft + row * V, V, in->Td, ws->q) != 0) return -1;
  } else {
    for (int32_t x = 0; x < V; ++x) ws->q[x] = 0.0;
  }
  for (int32_t x = 0; x < V; ++x) {
    ws->r[x] = ws->p[x];
    ws->p_lo[x] = ws->p[x] * (1.0 - eps);
    ws->p_hi[x] = ws->p[x] * (1.0 + eps);
    ws->q_lo[x] = ws->q[x] * (1.0 - eps);
    ws->q_hi[x] = ws->q[x] * (1.0 + eps);
  }
  double c_lo = 0.0, c_hi = 0.0; /* enclosure of the residual threshold */

  for (int32_t c = n + 1; c < nb; ++c) {
    if (par[c] != n) continue;
    int32_t x = tok[c];
    double u = (double)ua[c];
    /* the decision: accept with probability min(1, r(x)/q(x)) */
    double ratio = accept_ratio(ws->r[x], ws->q[x]);
    /* its enclosure: r(x) = max(0, p - c q)(x) / W(c) */
    double Wl = W_min(ws, c_hi), Wh = W_max(ws, c_lo);
    double num_lo = fmax(0.0, ws->p_lo[x] - c_hi * ws->q_hi[x]);
    double num_hi = fmax(0.0, ws->p_hi[x] - c_lo * ws->q_lo[x]);
    double ratio_lo = (Wh > 0.0) ? accept_ratio(num_lo / Wh, ws->q_hi[x]) : 0.0;
    double ratio_hi = (Wl > 0.0) ? accept_ratio(num_hi / Wl, ws->q_lo[x]) : INFINITY;
    if ((u >= ratio_lo && u <= ratio_hi) || fabs(u - ratio) < 1e-5) *flags |= ORC_TIE_TEST;
    if (u < ratio) {
      *acc_out = c;
      return 0;
    }
    /* rejected: r <- norm(max(0, r - q)); a zero-mass residual leaves r as it is */
    double S = 0.0;
    for (int32_t y = 0; y < V; ++y) {
      ws->w[y] = fmax(0.0, ws->r[y] - ws->q[y]);
      S += ws->w[y];
    }
    if (S > 0.0)
      for (int32_t y = 0; y < V; ++y) ws->r[y] = ws->w[y] / S;
    /* c <- c + W(c); c + W(c) has slope >= -eps in c over the box */
    double width = c_hi - c_lo;
    double nlo = c_lo + W_min(ws, c_lo) - eps * width;
    double nhi = c_hi + W_max(ws, c_hi) + eps * width;
    c_lo = nlo;
    c_hi = nhi;
  }
  /* Leaf: bonus from p of this node.  All children rejected: from the residual. */
  for (int32_t y = 0; y < V; ++y) {
    ws->w_lo[y] = fmax(0.0, ws->p_lo[y] - c_hi * ws->q_hi[y]);
    ws->w_hi[y] = fmax(0.0, ws->p_hi[y] - c_lo * ws->q_lo[y]);
  }
  int tie = 0;
  *term_out = invcdf_draw(ws->r, ws->w_lo, ws->w_hi, V, (double)us[n], &tie);
  if (tie) *flags |= ORC_TIE_DRAW;
  return 0;
}

static int request_is_usable(const verify_in* in, int32_t b) {
  const int32_t* par = in->parent + (int64_t)b * in->n_max;
  const int32_t* tok = in->tokens + (int64_t)b * in->n_max;
  int32_t n = in->n_nodes[b];
  if (!tree_is_valid(par, n, in->n_max)) return 0;
  for (int32_t i = 1; i < n; ++i)
    if (tok[i] < 0 || tok[i] >= in->vocab) return 0;
  return 1;
}

/*
 * mode 0: lazy walk -- only nodes on the committed path are evaluated.
 * mode 1: every node of every request is evaluated (speculative evaluation).
 * Because uniforms are indexed by node, both modes agree on every evaluated node.
 * Outputs (all [B, n_max]): accepted_child (-1 none, -2 not evaluated, -3 bad
 * request at node 0), term_token (-2 when not evaluated or a child was accepted),
 * tie_flags (bit 0 test, bit 1 draw).
 */
int oracle_reject_sample(const float* tgt_logits, const float* dft_logits, double T, double Td,
                         const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                         const float* u_accept, const float* u_sample, int32_t batch, int32_t n_max, int32_t vocab,
                         double eps, int32_t mode, int32_t* accepted_child, int32_t* term_token, int32_t* tie_flags) {
  if (!tgt_logits || !tokens || !parent || !n_nodes || !accepted_child || !term_token || !tie_flags) return ORC_EARG;
  if (!(T >= 0.0) || batch < 0 || n_max < 1 || n_max > 64 || vocab < 1) return ORC_EARG;
  if (T > 0.0 && (!dft_logits || !u_accept || !u_sample || !(Td > 0.0))) return ORC_EARG;
  verify_in in = {tgt_logits, dft_logits, T, Td, tokens, parent, n_nodes, u_accept, u_sample, n_max, vocab};
  int status = ORC_OK;
#pragma omp parallel
  {
    node_ws ws;
    int ok = ws_alloc(&ws, vocab, eps);
    if (!ok) {
#pragma omp atomic write
      status = ORC_ENOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < batch; ++b) {
      int32_t* acc = accepted_child + (int64_t)b * n_max;
      int32_t* term = term_token + (int64_t)b * n_max;
      int32_t* fl = tie_flags + (int64_t)b * n_max;
      for (int32_t i = 0; i < n_max; ++i) {
        acc[i] = ORC_NOT_EVALUATED;
        term[i] = ORC_NOT_EVALUATED;
        fl[i] = 0;
      }
      if (!ok) continue;
      if (!request_is_usable(&in, b)) {
        acc[0] = ORC_BAD_REQUEST;
        continue;
      }
      int32_t nb = n_nodes[b];
      if (mode == 1) {
        for (int32_t i = 0; i < nb; ++i)
          if (eval_node(&in, b, i, &ws, &acc[i], &term[i], &fl[i]) != 0) {
            for (int32_t j = 0; j < n_max; ++j) {
              acc[j] = ORC_NOT_EVALUATED;
              term[j] = ORC_NOT_EVALUATED;
              fl[j] = 0;
            }
            acc[0] = ORC_BAD_REQUEST;
            break;
          }
      } else {
        int32_t cur = 0;
        for (;;) {
          if (eval_node(&in, b, cur, &ws, &acc[cur], &term[cur], &fl[cur]) != 0) {
            for (int32_t j = 0; j < n_max; ++j) {
              acc[j] = ORC_NOT_EVALUATED;
              term[j] = ORC_NOT_EVALUATED;
              fl[j] = 0;
            }
            acc[0] = ORC_BAD_REQUEST;
            break;
          }
          if (acc[cur] < 0) break;
          cur = acc[cur];
        }
      }
    }
    if (ok) ws_free(&ws);
  }
  return status;
}

/* ------------------------------------------------------------------------- */
/* O5. Commit the accepted path plus the bonus token.                           */
/* [ZS] part C: walk from the root to the first rejection or a leaf; the path is */
/* unique.  [ZS] part G, step 6: the output is the accepted tokens followed by   */
/* the bonus.  [GL] "A useful performance model": tau counts the bonus.          */
/* path_nodes [B, n_max] (root first, -1 padded); out_tokens [B, n_max]          */
/* (accepted tokens then the bonus, -1 padded); accept_len [B] = accepted nodes, */
/* -1 for a rejected request.                                                    */
/* ------------------------------------------------------------------------- */
int oracle_accept_path(const int32_t* accepted_child, const int32_t* term_token, const int32_t* tokens,
                       const int32_t* n_nodes, int32_t batch, int32_t n_max, int32_t* path_nodes,
                       int32_t* out_tokens, int32_t* accept_len) {
  if (!accepted_child || !term_token || !tokens || !n_nodes || !path_nodes || !out_tokens || !accept_len)
    return ORC_EARG;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t* acc = accepted_child + (int64_t)b * n_max;
    const int32_t* term = term_token + (int64_t)b * n_max;
    const int32_t* tok = tokens + (int64_t)b * n_max;
    int32_t* pn = path_nodes + (int64_t)b * n_max;
    int32_t* ot = out_tokens + (int64_t)b * n_max;
    for (int32_t i = 0; i < n_max; ++i) {
      pn[i] = -1;
      ot[i] = -1;
    }
    accept_len[b] = -1;
    if (acc[0] == ORC_BAD_REQUEST || n_nodes[b] < 1 || n_nodes[b] > n_max) continue;
    int32_t cur = 0, len = 0;
    pn[0] = 0;
    while (acc[cur] >= 0) {
      int32_t nxt = acc[cur];
      if (nxt <= cur || nxt >= n_nodes[b] || len + 1 >= n_max) break; /* malformed input */
      cur = nxt;
      pn[++len] = cur;
      ot[len - 1] = tok[cur];
    }
    if (acc[cur] != ORC_NONE || term[cur] < 0) { /* the walk must end at an evaluated terminal */
      for (int32_t i = 0; i < n_max; ++i) {
        pn[i] = -1;
        ot[i] = -1;
      }
      continue;
    }
    ot[len] = term[cur];
    accept_len[b] = len;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O6. KV commit and rollback after the path.                                   */
/* [FAL] "EAGLE-4 verification trees and harness": after verification the       */
/* accepted continuation is kept and the rejected KV-cache entries are freed.    */
/* [ZS] part D.2: every tree node writes its own K/V, and rejected nodes must    */
/* not stay in the cache (rollback; paged caches free whole pages).              */
/* Reading: node j's K/V sits at logical position ctx + j; the root (node 0) is  */
/* committed where it is, and path node i (i = 1..L) moves from ctx + path[i] to */
/* ctx + i, so the committed length becomes ctx + 1 + L.  All sources are read   */
/* before any destination is written.  With a page table, the pages whose slots  */
/* hold only positions in [new_len, ctx + n) are released: their table entries   */
/* become -1 and their ids are listed in freed[b][0..] (-1 padded, 64 entries).  */
/* A request with accept_len < 0, an invalid path or a position outside the      */
/* cache is left untouched with new_len = -1 (ORC_EDATA is returned if any).     */
/* elem = bytes per element (2 for bf16, 4 for fp32); k, v in the layouts of O2. */
/* Reading for a model with several layers: every layer's cache holds the tree    */
/* at the same positions, so layer l (at k, v + l * layer_stride elements) takes  */
/* the same moves; the page table is shared and released once.                   */
/* ------------------------------------------------------------------------- */
int oracle_kv_commit(void* k, void* v, int32_t elem, int32_t n_layers, int64_t layer_stride, int32_t* block_table,
                     int32_t page_size, int32_t kv_capacity,
                     int32_t n_pages, const int32_t* ctx_len, const int32_t* n_nodes, const int32_t* path_nodes,
                     const int32_t* accept_len, int32_t batch, int32_t n_max, int32_t hkv, int32_t d,
                     int32_t* new_len, int32_t* freed) {
  if (!k || !v || !ctx_len || !n_nodes || !path_nodes || !accept_len || !new_len || !freed) return ORC_EARG;
  if (elem != 2 && elem != 4) return ORC_EARG;
  if (n_layers < 1 || (n_layers > 1 && layer_stride < 1)) return ORC_EARG;
  const size_t row = (size_t)d * (size_t)elem; /* bytes of one (position, head) vector */
  unsigned char* tmp = (unsigned char*)malloc((size_t)2 * n_max * hkv * row);
  if (!tmp) return ORC_ENOMEM;
  int rc = ORC_OK;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t* fr = freed + (int64_t)b * 64;
    for (int j = 0; j < 64; ++j) fr[j] = -1;
    new_len[b] = -1;
    const int32_t L = accept_len[b], n = n_nodes[b], ctx = ctx_len[b];
    const int32_t* path = path_nodes + (int64_t)b * n_max;
    if (L < 0) continue;
    int ok = n >= 1 && n <= n_max && ctx >= 0 && L < n && path[0] == 0;
    for (int32_t i = 1; ok && i <= L; ++i) ok = path[i] > path[i - 1] && path[i] < n;
    /* every position the commit touches must exist */
    for (int32_t t = ctx; ok && t < ctx + n; ++t)
      for (int32_t g = 0; ok && g < hkv; ++g)
        ok = kv_offset(b, t, g, block_table, page_size, kv_capacity, n_pages, hkv, d) >= 0;
    if (!ok) {
      rc = ORC_EDATA;
      continue;
    }
    for (int32_t l = 0; l < n_layers; ++l) {
      unsigned char* lk = (unsigned char*)k + (size_t)l * (size_t)layer_stride * elem;
      unsigned char* lv = (unsigned char*)v + (size_t)l * (size_t)layer_stride * elem;
      /* read every source first ... */
      for (int32_t i = 1; i <= L; ++i)
        for (int32_t g = 0; g < hkv; ++g) {
          const int64_t off = kv_offset(b, ctx + path[i], g, block_table, page_size, kv_capacity, n_pages, hkv, d);
          memcpy(tmp + ((size_t)(2 * i) * hkv + g) * row, lk + off * elem, row);
          memcpy(tmp + ((size_t)(2 * i + 1) * hkv + g) * row, lv + off * elem, row);
        }
      /* ... then write every destination */
      for (int32_t i = 1; i <= L; ++i)
        for (int32_t g = 0; g < hkv; ++g) {
          const int64_t off = kv_offset(b, ctx + i, g, block_table, page_size, kv_capacity, n_pages, hkv, d);
          memcpy(lk + off * elem, tmp + ((size_t)(2 * i) * hkv + g) * row, row);
          memcpy(lv + off * elem, tmp + ((size_t)(2 * i + 1) * hkv + g) * row, row);
        }
    }
    new_len[b] = ctx + 1 + L;
    if (block_table) { /* release the pages left holding only freed positions */
      int32_t* tab = block_table + (int64_t)b * kv_capacity;
      const int32_t first = (new_len[b] + page_size - 1) / page_size, end = (ctx + n + page_size - 1) / page_size;
      int j = 0;
      for (int32_t slot = first; slot < end; ++slot) {
        fr[j++] = tab[slot];
        tab[slot] = -1;
      }
    }
  }
  free(tmp);
  return rc;
}

/* Thread plumbing for timing runs (no arithmetic). */
int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
