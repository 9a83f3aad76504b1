/* CPU oracle: draft-tree construction (RheoSampling expansion with a top-R prune
 * or SMART's keep rule) and lossless probe-first tree verification.
 *
 * TEST INFRASTRUCTURE ONLY (see vrt_oracle.h): plain loops, fp64 for sampling
 * quantities, a fixed fp32 recipe for ranking quantities. Build with
 * -O2 -ffp-contract=off, no fast-math.
 */
#include "vrt_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Counter-based uniforms: Philox4x32-10 as defined by Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds of
 * two 32x32->64 multiplies with a Weyl-sequence key schedule. */
void orc_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u; /* golden ratio */
      k1 += 0xBB67AE85u; /* sqrt(3) - 1 */
    }
    uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)x0;
    uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* One uniform in [0, 1 - 2^-24] from counter (idx, b, step, purpose) and the
 * 64-bit seed as key: the top 24 bits of the first output word times 2^-24
 * (exact in fp32 and fp64). */
double orc_uniform(uint64_t seed, uint32_t idx, uint32_t b, uint32_t step, uint32_t purpose) {
  uint32_t ctr[4] = {idx, b, step, purpose};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox(ctr, key, out);
  return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------- */
/* exp for ranking, fixed recipe (x <= 0):
 *   x < -80 -> 0
 *   k = rint(x * 1.44269504f)                      (fp32 multiply, round half even)
 *   r = fma(-k, ln2_hi, x); r = fma(-k, ln2_lo, r)  (ln2_hi = 0x3f317200, ln2_lo = 0x35bfbe8e)
 *   p = Taylor series of e^r to degree 7 in Horner form with fma, coefficients
 *       the fp32-rounded 1/n!
 *   result = p * 2^k                               (exact scaling)
 */
float orc_exp_rank(float x) {
  if (!(x >= -80.0f)) return 0.0f; /* also maps -inf (and NaN) to 0 */
  const float log2e = 1.44269504f;
  const float ln2_hi = 0.693145751953125f;
  const float ln2_lo = 1.428606765330187e-06f;
  float k = rintf(x * log2e);
  float r = fmaf(-k, ln2_hi, x);
  r = fmaf(-k, ln2_lo, r);
  float p = 1.0f / 5040.0f;
  p = fmaf(p, r, 1.0f / 720.0f);
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

void orc_exp_rank_array(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_exp_rank(x[i]);
}

/* Pairwise sum over a zero-padded power-of-two array: level by level, element
 * 2i plus element 2i+1. Padding with more zeros leaves the result unchanged. */
static float pairwise(const float* v, int32_t n) {
  int32_t w = 1;
  while (w < n) w <<= 1;
  float* s = (float*)calloc((size_t)w, sizeof(float));
  for (int32_t i = 0; i < n; ++i) s[i] = v[i];
  while (w > 1) {
    w >>= 1;
    for (int32_t i = 0; i < w; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  }
  float r = s[0];
  free(s);
  return r;
}

float orc_pairwise128(const float* v) { return pairwise(v, 128); }

/* ------------------------------------------------------------------------- */
/* Support (RheoSampling key design 1): the min(trunc, V) largest logits of a
 * row, ordered by value descending and token id ascending. Every other logit
 * is treated as -inf. Plain full sort. */
typedef struct {
  float v;
  int32_t id;
} vi_pair;

static int cmp_vi(const void* a, const void* b) {
  const vi_pair* x = (const vi_pair*)a;
  const vi_pair* y = (const vi_pair*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

int32_t orc_support(const float* row, int32_t V, int32_t trunc, int32_t* ids, float* vals) {
  vi_pair* a = (vi_pair*)malloc(sizeof(vi_pair) * (size_t)V);
  for (int32_t v = 0; v < V; ++v) {
    a[v].v = row[v];
    a[v].id = v;
  }
  qsort(a, (size_t)V, sizeof(vi_pair), cmp_vi);
  const int32_t n = V < trunc ? V : trunc;
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = a[i].id;
    vals[i] = a[i].v;
  }
  free(a);
  return n;
}

double orc_support_mass(const float* row, int32_t V, int32_t trunc) {
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
  float* vals = (float*)malloc(sizeof(float) * (size_t)V);
  orc_support(row, V, V, ids, vals);
  const double M = (double)vals[0];
  double top = 0.0, all = 0.0;
  if (!(isinf(vals[0]) && vals[0] < 0)) {
    const int32_t n = V < trunc ? V : trunc;
    for (int32_t i = 0; i < V; ++i) { /* in rank order */
      const double e = exp((double)vals[i] - M);
      all += e;
      if (i < n) top += e;
    }
  }
  free(ids);
  free(vals);
  return all > 0.0 ? top / all : 0.0;
}

/* ------------------------------------------------------------------------- */
struct orc_tree {
  orc_cfg cfg;
  uint64_t seed;
  int32_t b;
  uint32_t step;
  int32_t maxpar, n_cand_cap, n_row_cap, flags, n_exempt;
  orc_cand* cand;
  orc_exp* rows;
  int32_t* front; /* creation indices of the nodes to expand next (-1 = root) */
  int32_t n_front;
  int32_t layers_done;
  /* SMART state */
  double L;
  int64_t n_size, n_paths;
  int32_t* has_child; /* [n_cand_cap + 1], index c + 1, root at 0 */
  int32_t* admitted;
  int32_t n_adm;
  /* emitted tree: node_cand[i] = creation index of node i (root = -1) */
  int32_t n_nodes;
  int32_t* node_cand;
  /* exact enumeration (orc_exact_law): force[r] is the support rank row r's probe takes
   * instead of a draw, and weight the product of the forced draws' probabilities; NULL
   * when drawing */
  int32_t* force;
  double weight;
};

static int32_t width_of(const orc_cfg* c) { return c->W > 0 ? c->W : c->K; }

int32_t orc_layer_base(const orc_tree* t, int32_t layer) {
  return layer == 0 ? 0 : t->cfg.K + (layer - 1) * t->maxpar * t->cfg.K;
}

int32_t orc_row_base(const orc_tree* t, int32_t layer) {
  return layer == 0 ? 0 : 1 + (layer - 1) * t->maxpar;
}

orc_tree* orc_tree_create(const orc_cfg* cfg, uint64_t seed, int32_t b, uint32_t step) {
  orc_tree* t = (orc_tree*)calloc(1, sizeof(orc_tree));
  t->cfg = *cfg;
  t->seed = seed;
  t->b = b;
  t->step = step;
  t->maxpar = (cfg->mode == ORC_SMART) ? cfg->budget : width_of(cfg);
  t->n_cand_cap = cfg->K + (cfg->D - 1) * t->maxpar * cfg->K;
  t->n_row_cap = 1 + (cfg->D - 1) * t->maxpar;
  t->cand = (orc_cand*)calloc((size_t)t->n_cand_cap, sizeof(orc_cand));
  t->rows = (orc_exp*)calloc((size_t)t->n_row_cap, sizeof(orc_exp));
  t->front = (int32_t*)malloc(sizeof(int32_t) * (size_t)(t->maxpar + 1));
  t->front[0] = -1;
  t->n_front = 1;
  t->has_child = (int32_t*)calloc((size_t)t->n_cand_cap + 1, sizeof(int32_t));
  t->admitted = (int32_t*)malloc(sizeof(int32_t) * (size_t)(t->n_cand_cap + 1));
  t->node_cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(t->n_cand_cap + 1));
  t->n_size = 1;
  t->n_paths = 1;
  t->L = 0.0;
  t->weight = 1.0;
  return t;
}

void orc_tree_free(orc_tree* t) {
  if (!t) return;
  for (int32_t r = 0; r < t->n_row_cap; ++r) free(t->rows[r].dense_q);
  free(t->cand);
  free(t->rows);
  free(t->front);
  free(t->has_child);
  free(t->admitted);
  free(t->node_cand);
  free(t);
}

static float score_of(const orc_tree* t, int32_t node) {
  return node < 0 ? 1.0f : t->cand[node].score;
}

static int32_t depth_of(const orc_tree* t, int32_t node) {
  return node < 0 ? 0 : t->cand[node].depth;
}

static void add_child(orc_tree* t, int32_t layer, int32_t pos, int32_t slot, int32_t parent,
                      int32_t row, int32_t token, int32_t kind, float q) {
  const int32_t c = orc_layer_base(t, layer) + pos * t->cfg.K + slot;
  orc_cand* x = &t->cand[c];
  x->token = token;
  x->parent = parent;
  x->depth = depth_of(t, parent) + 1;
  x->kind = kind;
  x->slot = slot;
  x->row = row;
  x->live = 1;
  x->score = score_of(t, parent) * q; /* path product, fp32 */
}

/* Exact enumeration: the share of u in [0, 1) for which the inverse CDF used by every
 * draw here (the smallest k with u z < q[0] + .. + q[k], sums in index order; if rounding
 * leaves none, the last k with mass, else 0) returns k. z is the mass the draw scales u
 * by (exactly the sum of q for the method's own draws). */
static double draw_share(const double* q, int32_t n, double z, int32_t k) {
  int32_t last = 0, first = -1;
  double cum = 0.0, before = 0.0, at = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    if (q[j] > 0.0) {
      last = j;
      if (first < 0) first = j;
    }
    if (j == k) before = cum;
    cum += q[j];
    if (j == k) at = cum;
  }
  if (z != z) return k == last ? 1.0 : 0.0;             /* u z is NaN: never below */
  if (z < 0.0) return k == 0 ? 1.0 : 0.0;               /* u z < 0 <= q[0] */
  if (z == 0.0) return k == (first >= 0 ? first : last) ? 1.0 : 0.0;
  if (k < 0 || k >= n) return 0.0;
  const double hi = at / z < 1.0 ? at / z : 1.0, lo = before / z < 1.0 ? before / z : 1.0;
  double share = hi > lo ? hi - lo : 0.0;
  if (k == last) share += 1.0 - (cum / z < 1.0 ? cum / z : 1.0); /* the fallback */
  return share;
}

/* Proxy probability of the probe (key design 2): min{q(x_m), z}, or min(1, q(x_1) + eps)
 * when m = 0. t0 is the number of deterministic children; probe last, x_m is the last of
 * them (the last filler) and z the mass after it. */
static float proxy_of(const orc_cfg* c, const orc_exp* e, int32_t t0) {
  if (t0 >= 1) return e->q_raw[t0 - 1] < e->z_raw ? e->q_raw[t0 - 1] : e->z_raw;
  const float a = e->q_raw[0] + c->eps_m0;
  return a < 1.0f ? a : 1.0f;
}

/* Expansion of one node over the whole vocabulary (trunc = ORC_DENSE): the dense
 * baseline of RheoSampling's support-size ablation. Ranks, deterministic and filler
 * slots, the probe's tail and its proxy follow key design 2 as on a truncated support,
 * with the support being every token. Two readings fix what the sorted 128-entry
 * support left implicit:
 *   - the ranking normaliser E and the raw tail mass are fp32 pairwise sums over the
 *     row in token-id order (zero-padded to a power of two), and z = E_tail / E;
 *   - the probe is drawn from the tempered tail by inverse CDF in token-id order (every
 *     order gives the same law; id order needs no sort of the row).
 * Tempered values are fp64 as on the truncated path. */
static void expand_dense(orc_tree* t, int32_t layer, int32_t pos, int32_t node, const float* row,
                         orc_exp* e, int32_t r) {
  const orc_cfg* c = &t->cfg;
  const int32_t V = c->V;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
  float* vals = (float*)malloc(sizeof(float) * (size_t)V);
  orc_support(row, V, V, ids, vals);
  const float M = vals[0];
  if (isinf(M) && M < 0) e->flags |= 2;
  if (e->flags) {
    t->flags |= e->flags;
    free(ids);
    free(vals);
    return;
  }
  e->n_sup = V;
  const int32_t keep = V < ORC_MAXSUP ? V : ORC_MAXSUP; /* ranks recorded in the row */

  /* untempered, fp32 recipe, sums in id order */
  float* ex = (float*)malloc(sizeof(float) * (size_t)V);
  float* tx = (float*)malloc(sizeof(float) * (size_t)V);
  uint8_t* det = (uint8_t*)calloc((size_t)V, 1);
  for (int32_t v = 0; v < V; ++v) ex[v] = orc_exp_rank(row[v] - M);
  const float E = pairwise(ex, V);
  const int32_t m = c->probe ? c->m : 0;
  const int32_t t0 = c->order == ORC_PROBE_LAST ? (c->K - 1 < V ? c->K - 1 : V) : m;
  for (int32_t i = 0; i < t0; ++i) det[ids[i]] = 1; /* the deterministic children */
  for (int32_t v = 0; v < V; ++v) tx[v] = det[v] ? 0.0f : ex[v];
  e->z_raw = pairwise(tx, V) / E;
  for (int32_t i = 0; i < keep; ++i) {
    e->sup_id[i] = ids[i];
    e->sup_logit[i] = vals[i];
    e->q_raw[i] = ex[ids[i]] / E;
  }

  /* tempered, fp64 */
  const double invT = (double)(1.0f / c->T);
  double* et = (double*)malloc(sizeof(double) * (size_t)V);
  double Z = 0.0, zT = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    et[v] = exp(((double)row[v] - (double)M) * invT);
    Z += et[v];
    if (!det[v]) zT += et[v];
  }
  for (int32_t i = 0; i < keep; ++i) e->q_T[i] = et[ids[i]] / Z;
  e->z_T = zT / Z;

  /* probe: x_s ~ the tempered tail renormalised, inverse CDF in token-id order */
  int32_t s = -1;
  const int32_t draws = c->probe && V > t0 && zT > 0.0;
  if (t->force && !(draws ? (t->force[r] >= t0 && t->force[r] < V) : t->force[r] == t0))
    t->weight = 0.0; /* a forced branch that does not exist (no draw: only rank t0 stands) */
  if (draws && t->force && t->weight > 0.0) {
    /* exact enumeration: the token at the forced rank, weighted by the share of u in
     * [0, 1) that the id-order inverse CDF below sends to it (the deterministic children
     * hold no mass there) */
    s = ids[t->force[r]];
    double* qt = (double*)malloc(sizeof(double) * (size_t)V);
    for (int32_t v = 0; v < V; ++v) qt[v] = det[v] ? 0.0 : et[v];
    t->weight *= draw_share(qt, V, zT, s);
    free(qt);
  } else if (draws && !t->force) {
    const double u = orc_uniform(t->seed, (uint32_t)(node + 1), (uint32_t)t->b, t->step,
                                 ORC_PURPOSE_PROBE);
    e->u = u;
    const double target = u * zT;
    double cum = 0.0, before = 0.0;
    for (int32_t v = 0; v < V; ++v) {
      if (det[v]) continue;
      before = cum;
      cum += et[v];
      if (target < cum) {
        s = v;
        break;
      }
    }
    if (s < 0) { /* rounding exhausted the sum: the last tail token with mass */
      for (int32_t v = V - 1; v >= 0; --v)
        if (!det[v] && et[v] > 0.0) {
          s = v;
          break;
        }
      before = zT - et[s];
      cum = zT;
    }
    int32_t has_after = 0;
    for (int32_t v = s + 1; v < V; ++v)
      if (!det[v] && et[v] > 0.0) has_after = 1;
    if ((before > 0.0 && fabs(u - before / zT) < ORC_EXEMPT_BAND) ||
        (has_after && fabs(u - cum / zT) < ORC_EXEMPT_BAND)) {
      e->exempt = 1;
      t->n_exempt++;
    }
  }
  if (s >= 0) {
    e->probe_token = s;
    for (int32_t i = 0; i < keep; ++i)
      if (ids[i] == s) e->probe_rank = i;
    e->proxy = proxy_of(c, e, t0);
    /* the probe's tail for verification: q~ = et / zT off the deterministic children */
    e->dense_q = (double*)malloc(sizeof(double) * (size_t)V);
    for (int32_t v = 0; v < V; ++v) e->dense_q[v] = det[v] ? 0.0 : et[v] / zT;
  }

  /* slots: top-m deterministic, the probe, then the next ranks as fillers (probe last:
   * the fillers, then the probe) */
  int32_t slot = 0;
  if (!c->probe) {
    for (int32_t i = 0; i < V && slot < c->K; ++i)
      add_child(t, layer, pos, slot++, node, r, ids[i], ORC_DET, e->q_raw[i]);
  } else {
    for (int32_t i = 0; i < m && i < V && slot < c->K; ++i)
      add_child(t, layer, pos, slot++, node, r, ids[i], ORC_DET, e->q_raw[i]);
    if (c->order == ORC_PROBE_LAST) {
      for (int32_t i = m; i < t0 && slot < c->K; ++i)
        add_child(t, layer, pos, slot++, node, r, ids[i], ORC_FILL, e->q_raw[i]);
      if (s >= 0 && slot < c->K) add_child(t, layer, pos, slot++, node, r, s, ORC_PROBE, e->proxy);
    } else {
      if (s >= 0 && slot < c->K) add_child(t, layer, pos, slot++, node, r, s, ORC_PROBE, e->proxy);
      for (int32_t i = m; i < V && slot < c->K; ++i)
        if (ids[i] != s) add_child(t, layer, pos, slot++, node, r, ids[i], ORC_FILL, e->q_raw[i]);
    }
  }
  e->n_child = slot;
  free(ids);
  free(vals);
  free(ex);
  free(tx);
  free(det);
  free(et);
}

/* Expansion of one node (RheoSampling key designs 1 and 2; temperature policy
 * of its settings paragraph). */
static void expand_node(orc_tree* t, int32_t layer, int32_t pos, int32_t node, const float* row) {
  const orc_cfg* c = &t->cfg;
  const int32_t r = orc_row_base(t, layer) + pos;
  orc_exp* e = &t->rows[r];
  free(e->dense_q);
  memset(e, 0, sizeof(*e));
  e->node = node;
  e->probe_rank = -1;
  e->probe_token = -1;

  for (int32_t v = 0; v < c->V; ++v)
    if (isnan(row[v]) || (isinf(row[v]) && row[v] > 0)) e->flags |= 1;
  if (c->trunc == ORC_DENSE) {
    expand_dense(t, layer, pos, node, row, e, r);
    return;
  }
  /* 1. support: the top-trunc logits; the rest are -inf */
  const int32_t n = orc_support(row, c->V, c->trunc, e->sup_id, e->sup_logit);
  e->n_sup = n;
  const float M = e->sup_logit[0];
  if (isinf(M) && M < 0) e->flags |= 2; /* every logit is -inf */
  if (e->flags) {
    t->flags |= e->flags;
    return;
  }

  /* 2a. untempered probabilities on the support (ranking recipe, fp32) */
  float ex[ORC_MAXSUP];
  for (int32_t i = 0; i < n; ++i) ex[i] = orc_exp_rank(e->sup_logit[i] - M);
  const float E = pairwise(ex, n);
  for (int32_t i = 0; i < n; ++i) e->q_raw[i] = ex[i] / E;
  const int32_t m = c->probe ? c->m : 0;
  /* the probe's tail starts after the deterministic children: after the top m, or,
   * probe last, after the fillers too */
  const int32_t t0 = c->order == ORC_PROBE_LAST ? (c->K - 1 < n ? c->K - 1 : n) : m;
  float tail[ORC_MAXSUP];
  for (int32_t i = 0; i < n; ++i) tail[i] = (i < t0) ? 0.0f : e->q_raw[i];
  e->z_raw = pairwise(tail, n);

  /* 2b. tempered probabilities on the same support (sampling, fp64) */
  const double invT = (double)(1.0f / c->T);
  double et[ORC_MAXSUP], Z = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    et[i] = exp(((double)e->sup_logit[i] - (double)M) * invT);
    Z += et[i];
  }
  for (int32_t i = 0; i < n; ++i) e->q_T[i] = et[i] / Z;
  double zT = 0.0;
  for (int32_t i = t0; i < n; ++i) zT += e->q_T[i];
  e->z_T = zT;

  /* 3. probe: x_s ~ q_T restricted to ranks > m and renormalised by z_T,
   *    drawn by inverse CDF in rank order with one uniform. */
  int32_t js = -1;
  const int32_t draws = c->probe && n > t0 && zT > 0.0;
  if (t->force && !(draws ? (t->force[r] >= t0 && t->force[r] < n) : t->force[r] == t0))
    t->weight = 0.0; /* a forced branch that does not exist (no draw: only rank t0 stands) */
  if (draws && t->force && t->weight > 0.0) {
    /* exact enumeration: the forced rank, weighted by the share of u in [0, 1) that the
     * inverse CDF below sends to it */
    js = t->force[r];
    t->weight *= draw_share(e->q_T + t0, n - t0, zT, js - t0);
    e->probe_rank = js;
    e->probe_token = e->sup_id[js];
    e->proxy = proxy_of(c, e, t0);
  } else if (draws && !t->force) {
    const double u = orc_uniform(t->seed, (uint32_t)(node + 1), (uint32_t)t->b, t->step,
                                 ORC_PURPOSE_PROBE);
    e->u = u;
    const double target = u * zT;
    double cum = 0.0, before = 0.0;
    for (int32_t j = t0; j < n; ++j) {
      before = cum;
      cum += e->q_T[j];
      if (target < cum) {
        js = j;
        break;
      }
    }
    if (js < 0) { /* rounding exhausted the sum: the last rank with mass */
      for (int32_t j = n - 1; j >= t0; --j)
        if (e->q_T[j] > 0.0) {
          js = j;
          break;
        }
      before = zT - e->q_T[js];
      cum = zT;
    }
    /* exemption: u within the band of an interior CDF boundary */
    int32_t has_after = 0;
    for (int32_t j = js + 1; j < n; ++j)
      if (e->q_T[j] > 0.0) has_after = 1;
    if ((before > 0.0 && fabs(u - before / zT) < ORC_EXEMPT_BAND) ||
        (has_after && fabs(u - cum / zT) < ORC_EXEMPT_BAND)) {
      e->exempt = 1;
      t->n_exempt++;
    }
    e->probe_rank = js;
    e->probe_token = e->sup_id[js];
    e->proxy = proxy_of(c, e, t0);
  }

  /* 4. slots: top-m deterministic, the probe, then the next ranks as fillers */
  int32_t slot = 0;
  if (!c->probe) {
    for (int32_t i = 0; i < n && slot < c->K; ++i)
      add_child(t, layer, pos, slot++, node, r, e->sup_id[i], ORC_DET, e->q_raw[i]);
  } else {
    for (int32_t i = 0; i < m && i < n && slot < c->K; ++i)
      add_child(t, layer, pos, slot++, node, r, e->sup_id[i], ORC_DET, e->q_raw[i]);
    if (c->order == ORC_PROBE_LAST) {
      for (int32_t i = m; i < t0 && slot < c->K; ++i)
        add_child(t, layer, pos, slot++, node, r, e->sup_id[i], ORC_FILL, e->q_raw[i]);
      if (js >= 0 && slot < c->K)
        add_child(t, layer, pos, slot++, node, r, e->sup_id[js], ORC_PROBE, e->proxy);
    } else {
      if (js >= 0 && slot < c->K)
        add_child(t, layer, pos, slot++, node, r, e->sup_id[js], ORC_PROBE, e->proxy);
      for (int32_t i = m; i < n && slot < c->K; ++i)
        if (i != js) add_child(t, layer, pos, slot++, node, r, e->sup_id[i], ORC_FILL, e->q_raw[i]);
    }
  }
  e->n_child = slot;
}

/* Ranking key: path score descending, creation index ascending. */
static _Thread_local const orc_tree* g_sort_tree;
static int cmp_key(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  const float sx = g_sort_tree->cand[x].score, sy = g_sort_tree->cand[y].score;
  if (sx > sy) return -1;
  if (sx < sy) return 1;
  return (x < y) ? -1 : (x > y);
}

static void sort_by_key(const orc_tree* t, int32_t* idx, int32_t n) {
  g_sort_tree = t;
  qsort(idx, (size_t)n, sizeof(int32_t), cmp_key);
}

static double cost_C(const orc_cfg* c, double n) {
  return c->lambda_ * n + c->gamma_ * (exp(c->delta_ * pow(n, c->rho_)) - 1.0);
}

static double cost_dC(const orc_cfg* c, double n) {
  return c->lambda_ + c->gamma_ * c->delta_ * c->rho_ * pow(n, c->rho_ - 1.0) *
                          exp(c->delta_ * pow(n, c->rho_));
}

/* Expand the current frontier with its draft rows (row j of `rows` belongs to
 * frontier position j), then choose the next frontier: the top-W of this
 * layer's candidates (top-R mode) or the candidates SMART admits. */
int32_t orc_expand_layer(orc_tree* t, int32_t layer, const float* rows, int64_t ld) {
  const orc_cfg* c = &t->cfg;
  if (layer != t->layers_done || layer >= c->D) return -1;
  for (int32_t j = 0; j < t->n_front; ++j) expand_node(t, layer, j, t->front[j], rows + (int64_t)j * ld);
  t->layers_done++;

  const int32_t base = orc_layer_base(t, layer);
  const int32_t span = (layer == 0 ? 1 : t->maxpar) * c->K;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)span);
  int32_t n = 0;
  for (int32_t i = 0; i < span; ++i)
    if (t->cand[base + i].live) idx[n++] = base + i;
  sort_by_key(t, idx, n);

  if (c->mode == ORC_SMART) {
    /* SMART key design 3: scan candidates best-first; keep u iff
     * alpha * dC_target/dC_spec > C_target/C_spec, i.e.
     * alpha * g * C(|T|) > L * C'(|T|), g = P(path) / |P|. The first rejection
     * ends the layer (state is unchanged and later gains are not larger). */
    int32_t nf = 0;
    for (int32_t k = 0; k < n; ++k) {
      if (t->n_adm >= c->budget) break;
      const int32_t u = idx[k];
      const double g = (double)t->cand[u].score / (double)t->n_paths;
      const double nn = (double)t->n_size;
      const double lhs = c->alpha * g * cost_C(c, nn);
      const double rhs = t->L * cost_dC(c, nn);
      if (!(lhs > rhs)) break;
      const int32_t par = t->cand[u].parent;
      t->L += g;
      t->n_size += 1;
      if (t->has_child[par + 1]) t->n_paths += 1;
      t->has_child[par + 1] = 1;
      t->admitted[t->n_adm++] = u;
      t->front[nf++] = u;
    }
    t->n_front = (layer + 1 < c->D) ? nf : 0;
  } else {
    const int32_t W = width_of(c);
    int32_t nf = 0;
    if (layer + 1 < c->D)
      for (int32_t k = 0; k < n && k < W; ++k) t->front[nf++] = idx[k];
    t->n_front = nf;
  }
  free(idx);
  return t->n_front;
}

int32_t orc_frontier(const orc_tree* t, int32_t* cand_out) {
  for (int32_t j = 0; j < t->n_front; ++j) cand_out[j] = t->front[j];
  return t->n_front;
}

/* Emit the final tree. Top-R: the R best candidates by key (parents rank
 * before their children, so the kept set is a subtree). SMART: the admitted
 * candidates in (layer, admission) order. */
int32_t orc_finish(orc_tree* t) {
  const orc_cfg* c = &t->cfg;
  t->node_cand[0] = -1;
  int32_t nn = 1;
  if (c->mode == ORC_SMART) {
    for (int32_t k = 0; k < t->n_adm; ++k) t->node_cand[nn++] = t->admitted[k];
  } else {
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)t->n_cand_cap);
    int32_t n = 0;
    for (int32_t i = 0; i < t->n_cand_cap; ++i)
      if (t->cand[i].live) idx[n++] = i;
    sort_by_key(t, idx, n);
    for (int32_t k = 0; k < n && k < c->R; ++k) t->node_cand[nn++] = idx[k];
    free(idx);
  }
  t->n_nodes = nn;
  return nn;
}

int32_t orc_n_cand(const orc_tree* t) { return t->n_cand_cap; }
const orc_cand* orc_cands(const orc_tree* t) { return t->cand; }
int32_t orc_n_rows(const orc_tree* t) { return t->n_row_cap; }
const orc_exp* orc_row(const orc_tree* t, int32_t row) { return &t->rows[row]; }
int32_t orc_n_exempt(const orc_tree* t) { return t->n_exempt; }
int32_t orc_flags(const orc_tree* t) { return t->flags; }

int32_t orc_tree_view(const orc_tree* t, int32_t cap, int32_t tail_cap, int32_t* n_nodes,
                      int32_t* token, int32_t* parent, int32_t* depth, int32_t* kind,
                      int32_t* cand, int32_t* child_off, int32_t* child, int32_t* tail_n,
                      int32_t* tail_id, double* tail_q) {
  const int32_t n = t->n_nodes;
  if (n > cap) return -1;
  *n_nodes = n;
  int32_t* node_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(t->n_cand_cap + 1));
  for (int32_t i = 0; i <= t->n_cand_cap; ++i) node_of[i] = -1;
  for (int32_t i = 0; i < n; ++i) node_of[t->node_cand[i] + 1] = i;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t ci = t->node_cand[i];
    cand[i] = ci;
    tail_n[i] = 0;
    if (ci < 0) {
      token[i] = -1;
      parent[i] = -1;
      depth[i] = 0;
      kind[i] = ORC_ROOT;
    } else {
      token[i] = t->cand[ci].token;
      parent[i] = node_of[t->cand[ci].parent + 1];
      depth[i] = t->cand[ci].depth;
      kind[i] = t->cand[ci].kind;
    }
  }
  /* child lists in slot order: a counting pass, then fill by ascending slot */
  int32_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    child_off[i] = off;
    for (int32_t s = 0; s < t->cfg.K; ++s)
      for (int32_t j = 1; j < n; ++j)
        if (parent[j] == i && t->cand[t->node_cand[j]].slot == s) child[off++] = j;
  }
  child_off[n] = off;
  /* tails for nodes whose probe child is kept */
  for (int32_t j = 1; j < n; ++j) {
    if (kind[j] != ORC_PROBE) continue;
    const int32_t i = parent[j];
    const orc_exp* e = &t->rows[t->cand[t->node_cand[j]].row];
    const int32_t K1 = t->cfg.K - 1 < e->n_sup ? t->cfg.K - 1 : e->n_sup;
    const int32_t t0 = t->cfg.order == ORC_PROBE_LAST ? K1 : t->cfg.m;
    int32_t k = 0;
    if (t->cfg.trunc == ORC_DENSE) { /* every token off the deterministic children, id order */
      for (int32_t v = 0; v < t->cfg.V; ++v) {
        int32_t is_det = 0;
        for (int32_t r = 0; r < t0; ++r) is_det |= e->sup_id[r] == v;
        if (is_det) continue;
        if (k >= tail_cap) {
          free(node_of);
          return -2;
        }
        tail_id[(int64_t)i * tail_cap + k] = v;
        tail_q[(int64_t)i * tail_cap + k] = e->dense_q[v];
        ++k;
      }
      tail_n[i] = k;
      continue;
    }
    for (int32_t r = t0; r < e->n_sup; ++r) {
      if (k >= tail_cap) {
        free(node_of);
        return -2;
      }
      tail_id[(int64_t)i * tail_cap + k] = e->sup_id[r];
      tail_q[(int64_t)i * tail_cap + k] = e->q_T[r] / e->z_T;
      ++k;
    }
    tail_n[i] = k;
  }
  free(node_of);
  return n;
}

/* ------------------------------------------------------------------------- */
/* Exact enumeration of a node's decision: instead of drawing, decide_node follows the
 * forced branch (the test at index accept_at accepts, the ones before it reject; with
 * accept_at = -1 every test rejects and the final sample returns `token`) and multiplies
 * the branch's probability under u uniform on [0, 1) into weight. */
typedef struct {
  int32_t accept_at, token, n;
  double weight;
} orc_force;

/* One accept/reject test: u < ratio when drawing; forced, P(u < ratio) = clip(ratio). */
static int32_t take_test(orc_force* f, double u, double ratio) {
  if (!f) return u < ratio;
  const double pa = ratio >= 1.0 ? 1.0 : (ratio > 0.0 ? ratio : 0.0); /* NaN: 0 */
  const int32_t acc = f->n++ == f->accept_at;
  f->weight *= acc ? pa : 1.0 - pa;
  return acc;
}

/* ------------------------------------------------------------------------- */
/* Verification of one node (RheoSampling key design 3). p is the full-vocab
 * temperature softmax of the node's target row. If the probe child is kept it
 * is tested first with min(1, p/q~); on rejection the residual is
 * w = max(0, p - q~) on the probe's tail (p elsewhere) with mass
 * W = 1 - sum_tail min(p, q~). The remaining kept children are then tested in
 * slot order: accept x iff u < w(x)/W, else W -= w(x), w(x) = 0. With no kept
 * probe, w = p and W = 1. If nothing is accepted (or the node has no kept
 * children) a token is drawn from w/W by inverse CDF in token-id order.
 * Probe last (the RRSw baseline of key design 3): the other kept children are tested
 * first, in slot order, against w = p and W = 1 (each rejection removes its point mass);
 * then the probe with min(1, w/(W q~)), and a rejection leaves max(0, w - W q~) on the
 * tail (which holds none of those children). */
static void decide_node(const orc_cfg* c, int32_t i, const int32_t* token, const int32_t* depth,
                        const int32_t* kind, const int32_t* child_off, const int32_t* child,
                        const int32_t* tail_n, const int32_t* tail_id, const double* tail_q,
                        int32_t tail_cap, const float* x, uint64_t seed, int32_t b, uint32_t step,
                        double* w, orc_node_out* o, orc_force* f) {
  const int32_t V = c->V;
  const double invT = (double)(1.0f / c->T);
  float M = x[0];
  for (int32_t v = 1; v < V; ++v)
    if (x[v] > M) M = x[v];
  double S = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    w[v] = exp(((double)x[v] - (double)M) * invT);
    S += w[v];
  }
  for (int32_t v = 0; v < V; ++v) w[v] /= S; /* w = p */

  o->accept = -1;
  o->token = -1;
  o->exempt = 0;
  o->n_tests = 0;
  double W = 1.0;
  const uint32_t d = (uint32_t)depth[i];
  int32_t probe = -1;
  for (int32_t k = child_off[i]; k < child_off[i + 1]; ++k)
    if (kind[child[k]] == ORC_PROBE) probe = child[k];

  /* draws: 32*depth + j, j = 0 for the probe, 1.. for the other children in slot order */
  const double u0 = orc_uniform(seed, 32u * d, (uint32_t)b, step, ORC_PURPOSE_TEST);
  double qs = 0.0;
  if (probe >= 0)
    for (int32_t k = 0; k < tail_n[i]; ++k)
      if (tail_id[(int64_t)i * tail_cap + k] == token[probe]) qs = tail_q[(int64_t)i * tail_cap + k];

  if (c->order != ORC_PROBE_LAST && probe >= 0) {
    /* probe first: accept with min(1, p/q~); else the residual max(0, p - q~) on the tail */
    const double a = w[token[probe]] / qs;
    o->n_tests++;
    if (fabs(u0 - a) < ORC_EXEMPT_BAND) o->exempt++;
    if (take_test(f, u0, a)) {
      o->accept = probe;
      o->W = 0.0;
      return;
    }
    double overlap = 0.0;
    for (int32_t k = 0; k < tail_n[i]; ++k) {
      const int32_t y = tail_id[(int64_t)i * tail_cap + k];
      const double q = tail_q[(int64_t)i * tail_cap + k];
      const double p = w[y];
      overlap += (p < q) ? p : q;
      w[y] = (p > q) ? p - q : 0.0;
    }
    W = 1.0 - overlap;
  }

  /* the other kept children, in slot order, against the residual w / W; a rejected child
   * leaves the residual */
  uint32_t j = 1;
  for (int32_t k = child_off[i]; k < child_off[i + 1]; ++k) {
    const int32_t ch = child[k];
    if (ch == probe) continue;
    const int32_t xt = token[ch];
    const double wx = w[xt];
    const double ratio = wx / W;
    const double uj = orc_uniform(seed, 32u * d + j, (uint32_t)b, step, ORC_PURPOSE_TEST);
    ++j;
    o->n_tests++;
    if (fabs(uj - ratio) < ORC_EXEMPT_BAND) o->exempt++;
    if (take_test(f, uj, ratio)) {
      o->accept = ch;
      o->W = 0.0;
      return;
    }
    W -= wx;
    w[xt] = 0.0;
  }

  if (c->order == ORC_PROBE_LAST && probe >= 0) {
    /* probe last (RRSw): the residual w / W (every other kept child rejected) against the
     * probe's tail distribution q~: accept with min(1, w/(W q~)); else w - W q~ clipped at
     * 0 on the tail */
    const double a = w[token[probe]] / (W * qs);
    o->n_tests++;
    if (fabs(u0 - a) < ORC_EXEMPT_BAND) o->exempt++;
    if (take_test(f, u0, a)) {
      o->accept = probe;
      o->W = 0.0;
      return;
    }
    double overlap = 0.0;
    for (int32_t k = 0; k < tail_n[i]; ++k) {
      const int32_t y = tail_id[(int64_t)i * tail_cap + k];
      const double q = W * tail_q[(int64_t)i * tail_cap + k];
      const double p = w[y];
      overlap += (p < q) ? p : q;
      w[y] = (p > q) ? p - q : 0.0;
    }
    W -= overlap;
  }

  /* final residual (or bonus) sample by inverse CDF in token-id order */
  o->W = W;
  if (f) { /* forced: the branch exists only if no test was to accept */
    f->weight *= f->accept_at < 0 ? draw_share(w, V, W, f->token) : 0.0;
    o->token = f->token;
    return;
  }
  const double uf = orc_uniform(seed, d, (uint32_t)b, step, ORC_PURPOSE_FINAL);
  const double tgt = uf * W;
  double cum = 0.0, before = 0.0;
  int32_t y = -1;
  for (int32_t v = 0; v < V; ++v) {
    before = cum;
    cum += w[v];
    if (tgt < cum) {
      y = v;
      break;
    }
  }
  if (y < 0) {
    for (int32_t v = V - 1; v >= 0; --v)
      if (w[v] > 0.0) {
        y = v;
        break;
      }
    if (y < 0) y = 0;
    before = cum - w[y];
  }
  int32_t has_after = 0;
  for (int32_t v = y + 1; v < V && !has_after; ++v)
    if (w[v] > 0.0) has_after = 1;
  if ((before > 0.0 && fabs(uf - before / W) < ORC_EXEMPT_BAND) ||
      (has_after && fabs(uf - cum / W) < ORC_EXEMPT_BAND))
    o->exempt++;
  o->token = y;
}

int32_t orc_verify(const orc_cfg* cfg, int32_t n_nodes, const int32_t* token, const int32_t* parent,
                   const int32_t* depth, const int32_t* kind, const int32_t* child_off,
                   const int32_t* child, const int32_t* tail_n, const int32_t* tail_id,
                   const double* tail_q, int32_t tail_cap, const float* target, int64_t ld,
                   uint64_t seed, int32_t b, uint32_t step, int32_t* out_tokens,
                   int32_t* out_nodes, int32_t* out_len, orc_node_out* per_node) {
  (void)parent;
  double* w = (double*)malloc(sizeof(double) * (size_t)cfg->V);
  orc_node_out* outs = per_node;
  if (!outs) outs = (orc_node_out*)malloc(sizeof(orc_node_out) * (size_t)n_nodes);
  for (int32_t i = 0; i < n_nodes; ++i)
    decide_node(cfg, i, token, depth, kind, child_off, child, tail_n, tail_id, tail_q, tail_cap,
                target + (int64_t)i * ld, seed, b, step, w, &outs[i], NULL);
  /* the walk: follow accepted children from the root; emit the final token */
  int32_t cur = 0, len = 0, exempt = 0;
  for (;;) {
    exempt += outs[cur].exempt;
    if (outs[cur].accept >= 0) {
      out_nodes[len] = outs[cur].accept;
      out_tokens[len] = token[outs[cur].accept];
      ++len;
      cur = outs[cur].accept;
    } else {
      out_tokens[len] = outs[cur].token;
      ++len;
      break;
    }
  }
  *out_len = len;
  if (!per_node) free(outs);
  free(w);
  return exempt;
}

/* ------------------------------------------------------------------------- */
/* Repeated single decoding steps on a context-table model, for the
 * losslessness and acceptance tests. Logit rows are indexed by context path
 * (t_1..t_k): row = (V^k - 1)/(V - 1) + sum_i t_i V^(k-i), for k <= max_len.
 * Trial t runs step step0 + t from the empty context and records its first
 * emitted token. With two != 0 it also records the second emitted token: the
 * step's own second token if it emitted one, else the first token of a second
 * step (step step0 + n_trials + t) rooted at the first token. n_first[t] is the
 * number of tokens the first step took from the tree. */
static int64_t ctx_row(int32_t V, const int32_t* path, int32_t k) {
  int64_t off = 0, pw = 1;
  for (int32_t i = 0; i < k; ++i) {
    off += pw;
    pw *= V;
  }
  int64_t pos = 0;
  for (int32_t i = 0; i < k; ++i) pos = pos * V + path[i];
  return off + pos;
}

static int32_t path_of(const orc_tree* t, int32_t node, const int32_t* prefix, int32_t np,
                       int32_t* path) {
  int32_t rev[64], n = 0;
  for (int32_t c = node; c >= 0; c = t->cand[c].parent) rev[n++] = t->cand[c].token;
  for (int32_t i = 0; i < np; ++i) path[i] = prefix[i];
  for (int32_t i = 0; i < n; ++i) path[np + i] = rev[n - 1 - i];
  return np + n;
}

static int32_t one_step(const orc_cfg* cfg, int32_t max_len, const float* dtab, const float* ttab,
                        const int32_t* prefix, int32_t np, uint64_t seed, int32_t b, uint32_t step,
                        int32_t* out_tok, int32_t* out_len, int32_t* n_exempt) {
  const int32_t V = cfg->V;
  orc_tree* t = orc_tree_create(cfg, seed, b, step);
  float* rows = (float*)malloc(sizeof(float) * (size_t)V * (size_t)(t->maxpar + 1));
  int32_t path[64];
  for (int32_t layer = 0; layer < cfg->D && t->n_front > 0; ++layer) {
    for (int32_t j = 0; j < t->n_front; ++j) {
      const int32_t k = path_of(t, t->front[j], prefix, np, path);
      if (k > max_len) return -1;
      memcpy(rows + (int64_t)j * V, dtab + ctx_row(V, path, k) * V, sizeof(float) * (size_t)V);
    }
    orc_expand_layer(t, layer, rows, V);
  }
  orc_finish(t);
  const int32_t N = t->n_nodes, TC = cfg->trunc == ORC_DENSE ? V : cfg->trunc;
  int32_t* iv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(8 * N + 8));
  int32_t *token = iv, *parent = iv + N, *depth = iv + 2 * N, *kind = iv + 3 * N,
          *cand = iv + 4 * N, *child_off = iv + 5 * N, *child = iv + 6 * N + 1,
          *tail_n = iv + 7 * N + 1;
  int32_t* tail_id = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * TC);
  double* tail_q = (double*)malloc(sizeof(double) * (size_t)N * TC);
  int32_t nn;
  orc_tree_view(t, N, TC, &nn, token, parent, depth, kind, cand, child_off, child, tail_n, tail_id,
                tail_q);
  float* target = (float*)malloc(sizeof(float) * (size_t)V * (size_t)N);
  for (int32_t i = 0; i < N; ++i) {
    const int32_t k = path_of(t, cand[i], prefix, np, path);
    if (k > max_len) return -1;
    memcpy(target + (int64_t)i * V, ttab + ctx_row(V, path, k) * V, sizeof(float) * (size_t)V);
  }
  int32_t out_nodes[64];
  const int32_t ex = orc_verify(cfg, N, token, parent, depth, kind, child_off, child, tail_n,
                                tail_id, tail_q, TC, target, V, seed, b, step, out_tok, out_nodes,
                                out_len, NULL);
  *n_exempt += ex + t->n_exempt;
  free(target);
  free(tail_q);
  free(tail_id);
  free(iv);
  free(rows);
  orc_tree_free(t);
  return 0;
}

int32_t orc_table_trials(const orc_cfg* cfg, int32_t max_len, const float* draft_tab,
                         const float* target_tab, uint64_t seed, int32_t b, uint32_t step0,
                         int32_t n_trials, int32_t two, int32_t* out, int32_t* n_first,
                         int32_t* n_exempt) {
  int32_t bad = 0, exempt = 0;
#pragma omp parallel for schedule(dynamic, 256) reduction(+ : bad, exempt)
  for (int32_t tr = 0; tr < n_trials; ++tr) {
    int32_t tok[64], len = 0, ex = 0;
    if (one_step(cfg, max_len, draft_tab, target_tab, NULL, 0, seed, b, step0 + (uint32_t)tr, tok,
                 &len, &ex) != 0) {
      bad++;
      continue;
    }
    out[2 * tr] = tok[0];
    out[2 * tr + 1] = -1;
    n_first[tr] = len - 1;
    if (two) {
      if (len >= 2) {
        out[2 * tr + 1] = tok[1];
      } else {
        int32_t tok2[64], len2 = 0;
        if (one_step(cfg, max_len, draft_tab, target_tab, tok, 1, seed, b,
                     step0 + (uint32_t)n_trials + (uint32_t)tr, tok2, &len2, &ex) != 0) {
          bad++;
          continue;
        }
        out[2 * tr + 1] = tok2[0];
      }
    }
    exempt += ex;
  }
  *n_exempt = exempt;
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Exact laws by enumeration on a context-table model (tiny configurations). Every probe
 * draw of the build, and every test and final sample of the verification, becomes a
 * branch weighted by its probability under a uniform u on [0, 1); the branches run the
 * same expansion and decision code as the sampler (forced). */
typedef struct {
  const orc_cfg* cfg;
  int32_t max_len;
  const float *dtab, *ttab;
  const int32_t* prefix;
  int32_t np, two, err;
  double *law1, *law2, acc;
  double* fresh; /* [V][V]: row a = first-token law of the step at prefix + a (NaN: not yet) */
} enum_ctx;

/* The first `layers` layers of a tree at E's context, with the probes forced. */
/* Tokens in every expanded row's support: min(trunc, V), or all V when dense. */
static int32_t enum_sup(const orc_cfg* c) {
  return c->trunc == ORC_DENSE || c->V < c->trunc ? c->V : c->trunc;
}

static orc_tree* enum_build(enum_ctx* E, int32_t* force, int32_t layers) {
  const int32_t V = E->cfg->V;
  orc_tree* t = orc_tree_create(E->cfg, 0, 0, 0);
  t->force = force;
  float* rows = (float*)malloc(sizeof(float) * (size_t)V * (size_t)(t->maxpar + 1));
  int32_t path[64];
  for (int32_t layer = 0; layer < layers && t->n_front > 0 && t->weight > 0.0; ++layer) {
    for (int32_t j = 0; j < t->n_front; ++j) {
      const int32_t k = path_of(t, t->front[j], E->prefix, E->np, path);
      if (k > E->max_len) E->err = -1;
      if (E->err) break;
      memcpy(rows + (int64_t)j * V, E->dtab + ctx_row(V, path, k) * V, sizeof(float) * (size_t)V);
    }
    if (E->err) break;
    orc_expand_layer(t, layer, rows, V);
  }
  free(rows);
  return t;
}

typedef struct {
  int32_t accept, token;
  double p;
} enum_out;

/* Every outcome of node i's decision with its probability: out holds up to K + V entries. */
static int32_t node_outcomes(const orc_cfg* c, int32_t i, const int32_t* iv, int32_t N, const int32_t* tail_id,
                             const double* tail_q, int32_t TC, const float* x, double* w, enum_out* out) {
  const int32_t *token = iv, *depth = iv + 2 * N, *kind = iv + 3 * N, *child_off = iv + 5 * N,
                *child = iv + 6 * N + 1, *tail_n = iv + 7 * N + 1;
  int32_t n = 0;
  orc_node_out o;
  for (int32_t a = -1; a < c->K; ++a) {
    for (int32_t y = 0; y < (a < 0 ? c->V : 1); ++y) {
      orc_force f = {a, y, 0, 1.0};
      decide_node(c, i, token, depth, kind, child_off, child, tail_n, tail_id, tail_q, TC, x, 0, 0, 0, w,
                  &o, &f);
      if (f.weight > 0.0) {
        out[n].accept = a < 0 ? -1 : o.accept;
        out[n].token = a < 0 ? y : token[o.accept];
        out[n].p = f.weight;
        ++n;
      }
    }
  }
  return n;
}

static void enum_law(enum_ctx* E);

/* A complete tree of weight t->weight: its verification's outcomes into E's laws. */
static void enum_verify(enum_ctx* E, orc_tree* t) {
  const orc_cfg* c = E->cfg;
  const int32_t V = c->V, TC = enum_sup(c);
  orc_finish(t);
  const int32_t N = t->n_nodes;
  int32_t* iv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(8 * N + 8));
  int32_t* tail_id = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * TC);
  double* tail_q = (double*)malloc(sizeof(double) * (size_t)N * TC);
  float* target = (float*)malloc(sizeof(float) * (size_t)V * (size_t)N);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  enum_out* o1 = (enum_out*)malloc(sizeof(enum_out) * (size_t)(c->K + V));
  enum_out* o2 = (enum_out*)malloc(sizeof(enum_out) * (size_t)(c->K + V));
  int32_t nn, path[64];
  orc_tree_view(t, N, TC, &nn, iv, iv + N, iv + 2 * N, iv + 3 * N, iv + 4 * N, iv + 5 * N, iv + 6 * N + 1,
                iv + 7 * N + 1, tail_id, tail_q);
  for (int32_t i = 0; i < N && !E->err; ++i) {
    const int32_t k = path_of(t, iv[4 * N + i], E->prefix, E->np, path);
    if (k > E->max_len) E->err = -1;
    else memcpy(target + (int64_t)i * V, E->ttab + ctx_row(V, path, k) * V, sizeof(float) * (size_t)V);
  }
  const int32_t n1 = E->err ? 0 : node_outcomes(c, 0, iv, N, tail_id, tail_q, TC, target, w, o1);
  for (int32_t a = 0; a < n1; ++a) {
    const double p1 = t->weight * o1[a].p;
    const int32_t t1 = o1[a].token;
    E->law1[t1] += p1;
    if (o1[a].accept >= 0) E->acc += p1;
    if (!E->two) continue;
    if (o1[a].accept >= 0) { /* the step goes on at the accepted child */
      const int32_t ch = o1[a].accept;
      const int32_t n2 = node_outcomes(c, ch, iv, N, tail_id, tail_q, TC, target + (int64_t)ch * V, w, o2);
      for (int32_t b2 = 0; b2 < n2; ++b2) E->law2[(int64_t)t1 * V + o2[b2].token] += p1 * o2[b2].p;
    } else { /* one token emitted: the next step starts at the extended context */
      double* fr = E->fresh + (int64_t)t1 * V;
      if (fr[0] != fr[0]) {
        int32_t* pre = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E->np + 1));
        for (int32_t q = 0; q < E->np; ++q) pre[q] = E->prefix[q];
        pre[E->np] = t1;
        enum_ctx F = {c, E->max_len, E->dtab, E->ttab, pre, E->np + 1, 0, 0, fr, NULL, 0.0, NULL};
        for (int32_t v = 0; v < V; ++v) fr[v] = 0.0;
        enum_law(&F);
        if (F.err) E->err = F.err;
        free(pre);
      }
      for (int32_t v = 0; v < V; ++v) E->law2[(int64_t)t1 * V + v] += p1 * fr[v];
    }
  }
  free(o2);
  free(o1);
  free(w);
  free(target);
  free(tail_q);
  free(tail_id);
  free(iv);
}

/* Layer `layer` onwards, the probes of earlier layers fixed in force: one branch per
 * combination of the probe ranks of this layer's expanded rows. */
static void enum_layers(enum_ctx* E, int32_t* force, int32_t layer) {
  const orc_cfg* c = E->cfg;
  orc_tree* t = enum_build(E, force, layer);
  if (E->err || t->weight == 0.0) {
    orc_tree_free(t);
    return;
  }
  if (layer == c->D || t->n_front == 0) {
    enum_verify(E, t);
    orc_tree_free(t);
    return;
  }
  const int32_t nf = t->n_front, r0 = orc_row_base(t, layer);
  orc_tree_free(t);
  const int32_t n_sup = enum_sup(c);
  const int32_t t0 = c->order == ORC_PROBE_LAST ? (c->K - 1 < n_sup ? c->K - 1 : n_sup) : (c->probe ? c->m : 0);
  const int32_t radix = (c->probe && n_sup > t0) ? n_sup - t0 : 1;
  int32_t digit[64] = {0};
  for (;;) {
    for (int32_t j = 0; j < nf; ++j) force[r0 + j] = t0 + digit[j];
    enum_layers(E, force, layer + 1);
    int32_t j = 0;
    while (j < nf && ++digit[j] == radix) digit[j++] = 0;
    if (j == nf) break;
  }
  for (int32_t j = 0; j < nf; ++j) force[r0 + j] = t0;
}

/* Parents a layer may expand: the beam width, or SMART's node budget. */
static int32_t enum_maxpar(const orc_cfg* c) { return c->mode == ORC_SMART ? c->budget : width_of(c); }

static void enum_law(enum_ctx* E) {
  const orc_cfg* c = E->cfg;
  const int32_t maxpar = enum_maxpar(c);
  const int32_t n_rows = 1 + (c->D - 1) * maxpar;
  const int32_t n_sup = enum_sup(c);
  const int32_t t0 = c->order == ORC_PROBE_LAST ? (c->K - 1 < n_sup ? c->K - 1 : n_sup) : (c->probe ? c->m : 0);
  int32_t* force = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_rows);
  for (int32_t r = 0; r < n_rows; ++r) force[r] = t0;
  enum_layers(E, force, 0);
  free(force);
}

int32_t orc_exact_law(const orc_cfg* cfg, int32_t max_len, const float* draft_tab, const float* target_tab,
                      const int32_t* prefix, int32_t np, int32_t two, double* law1, double* law2,
                      double* accept) {
  if (enum_maxpar(cfg) > 64) return -2;
  const int32_t V = cfg->V;
  double* fresh = (double*)malloc(sizeof(double) * (size_t)V * (size_t)V);
  for (int64_t k = 0; k < (int64_t)V * V; ++k) fresh[k] = NAN;
  for (int32_t v = 0; v < V; ++v) law1[v] = 0.0;
  if (two)
    for (int64_t k = 0; k < (int64_t)V * V; ++k) law2[k] = 0.0;
  enum_ctx E = {cfg, max_len, draft_tab, target_tab, prefix, np, two, 0, law1, law2, 0.0, fresh};
  enum_law(&E);
  *accept = E.acc;
  free(fresh);
  return E.err;
}

int32_t orc_tree_mask(int32_t n, const int32_t* parent, uint8_t* mask, int32_t* pos) {
  if (n < 1 || parent[0] != -1) return -1;
  for (int32_t i = 1; i < n; ++i)
    if (parent[i] < 0 || parent[i] >= i) return -1;
  memset(mask, 0, (size_t)n * (size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    int32_t a = i, depth = 0;
    while (a >= 0) {
      mask[(size_t)i * (size_t)n + (size_t)a] = 1;
      a = parent[a];
      if (a >= 0) ++depth;
    }
    pos[i] = depth;
  }
  return 0;
}

int32_t orc_accepted_kv(int32_t len, const int32_t* nodes, int32_t* keep) {
  if (len < 1) return 0;
  keep[0] = 0;
  for (int32_t k = 1; k < len; ++k) keep[k] = nodes[k - 1];
  return len;
}
