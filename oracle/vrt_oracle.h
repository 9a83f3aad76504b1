/* CPU oracle for draft-tree construction and lossless tree verification.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant generator with the HIP path; it is written from
 * the method's definition:
 *   - RheoSampling (NeurIPS 2026 paper notes): key design 1 (top-128 truncation
 *     of the draft logits), key design 2 (dual-identity slot fill, proxy
 *     probability, the local-ranking lemma), key design 3 (probe-first
 *     optimal-transport verification, residual recursion, final residual
 *     sample), and the training-free settings paragraph (raw probabilities
 *     for ranking, temperature for the probe draw and verification).
 *   - SMART (ECCV 2026 paper notes): key designs 1-3 (speedup objective, cost
 *     models, marginal keep rule with discount alpha), framework flowchart
 *     (layer-wise greedy loop).
 *
 * Precision: sampling quantities (tempered draft probabilities, target
 * probabilities, residuals, CDFs) are fp64. Ranking quantities (untempered
 * draft probabilities, proxies, path scores) follow a fixed fp32 recipe so
 * that tree topology is a well-defined integer result: exp via exp_rank (a
 * Cody-Waite reduction plus degree-7 Taylor polynomial, pinned against the
 * fp64 exponential), 128-wide pairwise sums, IEEE division, no contraction.
 *
 * Parity pins: every function is pinned by the tests in tests/test_oracle_*.py
 * (Philox known-answer vectors, exp_rank error bound, support vs lexsort,
 * the lemma, chi-square losslessness, closed-form acceptance, the textbook
 * speculative-sampling case, the identity case, the T->0 limit; the beam and
 * the top-R prune by hand-worked trees and by invariants against lexsort
 * order; build and verification together by exact enumeration of the first-
 * and two-token laws, which losslessness fixes to the target's softmax). The
 * SMART keep rule's readings (|P| = leaf count, L starts at 0, |T| counts the
 * root) are pinned only by hand-worked cases: parity unpinned beyond those.
 * Which parents a layer expands (the top W of the layer by path score) is a
 * reading of the pages; the pins fix that the oracle implements this reading.
 */
#ifndef VRT_ORACLE_H
#define VRT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_ROOT = 0, ORC_DET = 1, ORC_PROBE = 2, ORC_FILL = 3 };
enum { ORC_TOPR = 0, ORC_SMART = 1 };
enum { ORC_PURPOSE_PROBE = 1, ORC_PURPOSE_TEST = 2, ORC_PURPOSE_FINAL = 3 };
#define ORC_MAXSUP 1024
#define ORC_EXEMPT_BAND 1e-6

/* order: ORC_PROBE_FIRST, RheoSampling's layout and verification (top-m, the probe,
 * then fillers; the probe is tested first); or ORC_PROBE_LAST, the RRSw baseline the
 * pages compare against (key design 3 and the verification ablation): top-m, then the
 * fillers, then the probe, drawn from the ranks after the fillers so that the kept
 * deterministic children never lie in its tail, and tested after them. */
enum { ORC_PROBE_FIRST = 0, ORC_PROBE_LAST = 1 };

/* trunc = ORC_DENSE: no truncation, the support is the whole vocabulary (the dense
 * baseline of RheoSampling's support-size ablation, full-vocabulary softmax and
 * sampling). See expand_dense in vrt_oracle.c for the two readings it takes. */
#define ORC_DENSE 0

typedef struct {
  int32_t V, trunc, K, m, probe, D, W, R, mode, budget;
  float T, eps_m0;
  double alpha, lambda_, gamma_, delta_, rho_;
  int32_t order;
} orc_cfg;

/* One candidate: a child created by one expansion. */
typedef struct {
  int32_t token, parent, depth, kind, slot, row, live;
  float score;
} orc_cand;

/* One expansion of a node over its draft row. */
typedef struct {
  int32_t node; /* creation index of the expanded node, -1 for the root */
  int32_t n_sup, probe_rank, n_child, exempt, flags;
  int32_t sup_id[ORC_MAXSUP];
  float sup_logit[ORC_MAXSUP];
  float q_raw[ORC_MAXSUP];
  double q_T[ORC_MAXSUP];
  float z_raw, proxy;
  double z_T, u;
  int32_t probe_token; /* the probe's token, -1 if none */
  double* dense_q;     /* dense rows with a probe: q~ of every token (0 off the tail) */
} orc_exp;

typedef struct orc_tree orc_tree;

/* Per-node verification outcome. */
typedef struct {
  int32_t accept;  /* accepted child (node index) or -1 */
  int32_t token;   /* residual/bonus token if accept == -1, else -1 */
  int32_t exempt;  /* number of draws at this node within the exemption band */
  int32_t n_tests; /* number of uniforms consumed by accept/reject tests */
  double W;        /* residual mass when the final sample was taken (1 at a leaf) */
} orc_node_out;

void orc_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
double orc_uniform(uint64_t seed, uint32_t idx, uint32_t b, uint32_t step, uint32_t purpose);
float orc_exp_rank(float x);
void orc_exp_rank_array(const float* x, float* y, int64_t n);
float orc_pairwise128(const float* v);
int32_t orc_support(const float* row, int32_t V, int32_t trunc, int32_t* ids, float* vals);

/* Coverage of a truncated support (RheoSampling's support-size ablation): the share of
 * the untempered draft softmax of one row that its min(trunc, V) largest logits hold,
 * in fp64. A row with no finite logit has coverage 0. */
double orc_support_mass(const float* row, int32_t V, int32_t trunc);

orc_tree* orc_tree_create(const orc_cfg* cfg, uint64_t seed, int32_t b, uint32_t step);
void orc_tree_free(orc_tree* t);
int32_t orc_expand_layer(orc_tree* t, int32_t layer, const float* rows, int64_t ld);
int32_t orc_frontier(const orc_tree* t, int32_t* cand_out);
int32_t orc_finish(orc_tree* t);
int32_t orc_n_cand(const orc_tree* t);
const orc_cand* orc_cands(const orc_tree* t);
int32_t orc_n_rows(const orc_tree* t);
const orc_exp* orc_row(const orc_tree* t, int32_t row);
int32_t orc_layer_base(const orc_tree* t, int32_t layer);
int32_t orc_row_base(const orc_tree* t, int32_t layer);
int32_t orc_n_exempt(const orc_tree* t);
int32_t orc_flags(const orc_tree* t);

/* Verification view of the emitted tree. Arrays have n_nodes entries, node 0
 * is the root; child lists are in slot order; tail tables hold (token, q~) of
 * the probe's tail for nodes whose probe child is kept (tail_n = 0 otherwise). */
int32_t orc_tree_view(const orc_tree* t, int32_t cap, int32_t tail_cap, int32_t* n_nodes,
                      int32_t* token, int32_t* parent, int32_t* depth, int32_t* kind,
                      int32_t* cand, int32_t* child_off, int32_t* child, int32_t* tail_n,
                      int32_t* tail_id, double* tail_q);

int32_t orc_verify(const orc_cfg* cfg, int32_t n_nodes, const int32_t* token, const int32_t* parent,
                   const int32_t* depth, const int32_t* kind, const int32_t* child_off,
                   const int32_t* child, const int32_t* tail_n, const int32_t* tail_id,
                   const double* tail_q, int32_t tail_cap, const float* target, int64_t ld,
                   uint64_t seed, int32_t b, uint32_t step, int32_t* out_tokens,
                   int32_t* out_nodes, int32_t* out_len, orc_node_out* per_node);

int32_t orc_table_trials(const orc_cfg* cfg, int32_t max_len, const float* draft_tab,
                         const float* target_tab, uint64_t seed, int32_t b, uint32_t step0,
                         int32_t n_trials, int32_t two, int32_t* out, int32_t* n_first,
                         int32_t* n_exempt);

/* Exact laws of one step on a context-table model (rows indexed as for
 * orc_table_trials), for tiny configurations (top-R or SMART, truncated or dense support): every probe
 * draw and every accept/reject or final sample is taken as a branch weighted by its
 * probability, through the same expansion and decision code the sampler runs.
 *   law1[V]     P(first emitted token = v) of the step at context prefix[0..np)
 *   law2[V*V]   (two != 0) P(first = a, second = b): the step's second token, or when the
 *               step emitted one token the first token of the next step at prefix + a
 *   accept      P(the first token comes from the tree)
 * RheoSampling's highlights state that the step is lossless for any prune budget: law1 is
 * then the target's tempered softmax at the context and law2 its two-step product.
 * Returns 0, -1 if the table is too short for the paths, -2 for an unsupported
 * configuration (more than 64 parents per layer: W, or SMART's budget). */
int32_t orc_exact_law(const orc_cfg* cfg, int32_t max_len, const float* draft_tab, const float* target_tab,
                      const int32_t* prefix, int32_t np, int32_t two, double* law1, double* law2,
                      double* accept);

/* The step after the prune (the target forward over the emitted tree, RheoSampling
 * framework flowchart: one target pass verifies the whole tree): node i may attend to
 * node j iff j lies on the path from the root to i, i included. Written out by
 * following parents from i. mask: n*n bytes, row i, column j; pos[i]: the number of
 * ancestors of i (its depth). Returns 0, or -1 if a parent is out of range (the root's
 * parent is -1, every other node's lies in [0, i)). */
int32_t orc_tree_mask(int32_t n, const int32_t* parent, uint8_t* mask, int32_t* pos);

/* The KV entries kept after verification: the root's, then the accepted nodes' in path
 * order: keep[0] = 0, keep[k] = nodes[k-1] for 1 <= k < len. Returns len. */
int32_t orc_accepted_kv(int32_t len, const int32_t* nodes, int32_t* keep);

#ifdef __cplusplus
}
#endif
#endif
