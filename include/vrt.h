/* vrt.h — C ABI of libvrt: one speculative-decoding step on MI355X (gfx950).
 *
 * The library builds a dynamic draft tree from batched draft logits and verifies
 * it losslessly against batched target logits:
 *
 *   build (per layer, then finish)             RheoSampling, framework flowchart
 *     - top-`trunc` truncation of each expanded parent's draft row (key design 1)
 *     - dual-identity slot fill: top-m deterministic tokens, one probe drawn from
 *       the renormalised tempered tail carrying proxy min{q(x_m), z}, then the
 *       next-ranked filler tokens (key design 2)
 *     - path-product scores; per-layer beam and global top-R prune, or SMART's
 *       marginal keep rule (SMART key designs 1-3) in VRT_MODE_SMART
 *   verify                                      RheoSampling, key design 3
 *     - full-vocabulary temperature softmax of every node's target row
 *     - probe-first optimal-transport test, recursive rejection of the remaining
 *       kept siblings under norm(max(0, p - q~)), final residual (or bonus) sample
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers owned by the caller; the
 *     library never allocates or frees memory and keeps no device state between
 *     calls except what the caller's tree blob and workspace hold.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream) and is
 *     asynchronous: the return code covers host-side validation and launch errors
 *     only. No entry point synchronises the device.
 *   - Data faults in the logits (NaN, +Inf, an all -inf row) do not abort: they set
 *     bits in the per-tree status word (stats[b][0]); outputs of that tree are then
 *     unspecified but every access stays in bounds.
 *   - On error the call enqueues nothing and vrt_last_error() describes the cause
 *     (thread-local, valid until the next call on that thread).
 *   - Random draws are Philox4x32-10 (Salmon et al., SC'11) with key = seed and
 *     counter (idx, b, step, purpose): purpose 1 = probe draw (idx = creation index
 *     of the expanded node + 1, root 0), 2 = accept/reject test (idx = 32*depth + j,
 *     j = 0 probe, 1.. remaining siblings in slot order), 3 = final sample
 *     (idx = depth). u = (out0 >> 8) * 2^-24; a draw accepts iff u < threshold.
 */
#ifndef VRT_H
#define VRT_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VRT_OK = 0,
  VRT_EINVAL = -1,  /* invalid argument or configuration */
  VRT_EDTYPE = -2,  /* unsupported logits dtype */
  VRT_ENOMEM = -3,  /* workspace or tree blob smaller than the sizing call returned */
  VRT_EHIP = -4     /* a HIP launch failed */
} vrt_status;

typedef enum { VRT_F32 = 0, VRT_BF16 = 1 } vrt_dtype;
typedef enum { VRT_MODE_TOPR = 0, VRT_MODE_SMART = 1 } vrt_mode;
enum { VRT_ROOT = 0, VRT_DET = 1, VRT_PROBE = 2, VRT_FILL = 3 };
#define VRT_FINISH (-1)
#define VRT_DENSE 0 /* vrt_config.trunc: no truncation (see trunc below) */

/* status bits, stats[b][0] */
#define VRT_ST_DRAFT_NONFINITE 0x1u  /* NaN or +Inf in an expanded draft row */
#define VRT_ST_DRAFT_EMPTY 0x2u      /* a draft row is entirely -inf */
#define VRT_ST_TARGET_BAD 0x4u       /* NaN/+Inf in a target row, or a row entirely -inf */

/* Method configuration (plain data; identical for every call on one tree blob).
 *   B        trees in the batch (>= 1)
 *   V        vocabulary size (1 .. 2^20)
 *   dtype    VRT_F32 or VRT_BF16 logits
 *   trunc    support size of the draft truncation (1 .. 1024; the pages use 128), or
 *            VRT_DENSE: no truncation, the support is the whole vocabulary (the dense
 *            baseline of RheoSampling's support-size ablation). Dense rows rank their
 *            top K exactly as a truncated support would, sum the ranking exponentials
 *            pairwise in token-id order and draw the probe by inverse CDF in token-id
 *            order; they write no tail table: trees with the probe on are verified by
 *            vrt_verify_dense (the other verification entry points return VRT_EINVAL)
 *   K        slots per expanded parent (1 .. 30)
 *   m        deterministic top-m slots (probe mode: 0 <= m <= K-1)
 *   probe    1 = RheoSampling dual-identity slots, 0 = plain top-K (all deterministic)
 *   D        tree depth, the number of expansion layers (1 .. 32)
 *   W        parents expanded per layer in top-R mode (0 -> K); W*K <= 4096 and
 *            K + (D-1)*W*K <= 4096
 *   R        nodes kept by the global prune, root excluded (top-R mode, 1 .. 1024)
 *   mode     VRT_MODE_TOPR or VRT_MODE_SMART
 *   budget   SMART: maximum kept nodes, root excluded (1 .. 1024); budget*K <= 4096
 *   T        temperature of the probe draw and of verification (> 0)
 *   eps_m0   proxy offset for m = 0 (proxy = min(1, q(x_1) + eps_m0))
 *   alpha, lambda_, gamma_, delta_, rho_
 *            SMART discount and cost models C(n) = lambda n + gamma (exp(delta n^rho) - 1),
 *            C'(n) = lambda + gamma delta rho n^(rho-1) exp(delta n^rho) (SMART key design 2) */
/* Order of the probe among a node's children (the probe on; ignored with probe = 0):
 *   VRT_PROBE_FIRST  RheoSampling (key designs 2-3): slots top-m, the probe, then the
 *                    fillers; the probe is tested first with min(1, p/q~), the others
 *                    under the residual norm(max(0, p - q~))
 *   VRT_PROBE_LAST   the RRSw baseline of key design 3: slots top-m, the fillers (the next
 *                    K-1-m ranks), then the probe drawn from the ranks after them (tail
 *                    q~ = tempered mass there, renormalised; proxy min{q of the last
 *                    deterministic child, the raw mass after it}); the deterministic
 *                    children are tested first as point masses, then the probe with
 *                    min(1, p_D/q~), p_D the target with the rejected children removed */
typedef enum { VRT_PROBE_FIRST = 0, VRT_PROBE_LAST = 1 } vrt_order;
/* tree_base: every draw of tree b (the probe draws of the build, the verification's tests
 * and final samples) is keyed by tree index tree_base + b. A batch issued as several
 * calls, each on its own trees (B = its tree count; its own blob, workspace and row
 * pointers; say one call per stream, so that one call's dependent phases overlap another's
 * row streams), with tree_base set to the index of each call's first tree, gives the whole
 * batch's trees and tokens bit for bit. 0 for a single call. */

typedef struct {
  int32_t B, V, dtype, trunc, K, m, probe, D, W, R, mode, budget;
  float T, eps_m0;
  double alpha, lambda_, gamma_, delta_, rho_;
  int32_t order;  /* vrt_order: where the probe sits and when it is tested */
  int32_t tree_base;  /* >= 0: the tree index of this call's tree 0 in the draws' keys */
} vrt_config;

/* Byte offsets of the arrays inside the caller-owned tree blob. Every array is
 * [B][...] row-major, 256-byte aligned. Capacities:
 *   NC  = K + (D-1)*P*K candidates (P = W in top-R mode, budget in SMART mode)
 *   NR  = 1 + (D-1)*P expansion rows
 *   N   = R + 1 (top-R) or budget + 1 (SMART) emitted nodes, root included
 *   TC  = trunc tail entries
 *   FP  = P frontier slots
 * Candidate c of layer l sits at c = base(l) + pos*K + slot with base(0) = 0,
 * base(l) = K + (l-1)*P*K; pos is the expanding parent's frontier position, slot its
 * slot. Expansion row r = 0 (root) or 1 + (l-1)*P + pos expanded frontier position
 * pos at layer l >= 1.
 *
 * Build state (written by vrt_build_tree, read by the next layer and by finish):
 *   cand_token  i32 [B][NC]  token of the candidate
 *   cand_parent i32 [B][NC]  creation index of its parent, -1 = root
 *   cand_score  f32 [B][NC]  path score (fp32 product of ranking probabilities)
 *   cand_kind   i32 [B][NC]  bits 0-7: 0 = no candidate in this slot, else
 *                            VRT_DET/PROBE/FILL; bit 8 (SMART): it has an admitted child
 *   row_tail_n  i32 [B][NR]  number of tail entries of the row's support (0: no probe)
 *   row_tail_id i32 [B][NR][TC]  tail tokens in rank order (support ranks m+1..)
 *   row_tail_q  f32 [B][NR][TC]  q~ = q_T / z_T of those tokens
 *   front       i32 [B][FP]  creation indices of the parents the next layer expands,
 *                            in frontier-position order (the caller supplies their
 *                            draft rows in this order)
 *   n_front     i32 [B]      number of valid entries of front (0: no further layer)
 *   smart       f64 [B][8]   SMART state (L, |T|, |P|, admitted count, root has a child)
 *   admitted    i32 [B][N]   SMART: admitted creation indices in admission order
 *   layer_sync  i32 [B]      rows of the current layer done (set to 0 by layer 0 and
 *                            by the block that ranks each layer)
 * Emitted tree (written by finish; the verification input, writable by the caller):
 *   n_nodes     i32 [B]      emitted nodes, root included (1 .. N)
 *   node_token  i32 [B][N]   token (root: -1)
 *   node_parent i32 [B][N]   parent node index (root: -1); parent < child
 *   node_depth  i32 [B][N]   depth (root 0)
 *   node_kind   i32 [B][N]   VRT_ROOT/DET/PROBE/FILL
 *   node_cand   i32 [B][N]   creation index (root: -1)
 *   child_off   i32 [B][N+1] children of node i are child[child_off[i] .. child_off[i+1])
 *   child       i32 [B][N]   child node indices, in slot order
 *   tail_n      i32 [B][N]   tail entries of node i's expansion if its probe child is
 *                            kept, else 0
 *   tail_id     i32 [B][N][TC], tail_q f32 [B][N][TC]  that tail (q~ values)
 * Dense rows (trunc = VRT_DENSE; the three arrays are empty otherwise), whose probe
 * tail is the whole row but its deterministic children, kept as what regenerates it
 * from the draft row:
 *   row_dense   f64 [B][NR][2]   the row's largest logit and its tempered tail mass
 *                                sum_{v in tail} exp((x_v - max)/T) (0: no probe)
 *   row_det     i32 [B][NR][32]  tokens of the deterministic children (the t0 best:
 *                                the top m, or probe last the top K-1)
 *   node_row    i32 [B][N]       expansion row of node i if its probe child is kept,
 *                                else -1
 * Build scratch:
 *   row_sync    u64 [B][FP]  where a layer's rows are split over 2 or 4 blocks (rows
 *                            too long for one block; rows beyond one per CU), the
 *                            launch's tag and how many parts have finished (needs
 *                            no initial value; the last part sets it back to 0)
 * SMART mode only (empty otherwise), one table for the whole batch, not per tree:
 *   smart_cost  f64 [budget+2][2]  C(n) and C'(n) of SMART key design 2 for tree sizes
 *                            n = 0 .. budget+1, evaluated in fp64 by the host's libm
 *                            and written by layer 0, so that the keep rule's decisions
 *                            do not depend on the device's exp and pow */
typedef struct {
  int64_t NC, NR, N, TC, FP;
  int64_t cand_token, cand_parent, cand_score, cand_kind;
  int64_t row_tail_n, row_tail_id, row_tail_q;
  int64_t front, n_front, smart, admitted, layer_sync;
  int64_t n_nodes, node_token, node_parent, node_depth, node_kind, node_cand;
  int64_t child_off, child, tail_n, tail_id, tail_q;
  int64_t row_dense, row_det, node_row;
  int64_t row_sync;
  int64_t smart_cost;
  int64_t total_bytes;
} vrt_tree_layout;

/* Checks the configuration. Returns VRT_OK or VRT_EINVAL (reason in vrt_last_error). */
vrt_status vrt_check_config(const vrt_config* cfg);

/* Fills *out with the tree-blob layout for cfg. */
vrt_status vrt_tree_layout_of(const vrt_config* cfg, vrt_tree_layout* out);

/* Size in bytes of the tree blob (the caller allocates it on the device). 0 if cfg is invalid. */
size_t vrt_tree_bytes(const vrt_config* cfg);

/* Size in bytes of the device workspace both entry points need. 0 if cfg is invalid.
 * The workspace needs no initialisation and holds nothing between calls. */
size_t vrt_workspace_bytes(const vrt_config* cfg);

/* One layer of tree construction (RheoSampling framework flowchart, key designs 1-2;
 * SMART key design 3 in VRT_MODE_SMART), or the final prune.
 *   layer         0 .. D-1 in order (layer 0 resets the tree), or VRT_FINISH after the
 *                 last layer (or once n_front is 0 for every tree) to emit the tree
 *   draft_logits  device, dtype cfg->dtype: the draft row of frontier position j of
 *                 tree b starts at element b*tree_stride + j*ld. Layer 0 reads one row
 *                 per tree (the root); layer l reads n_front[b] rows. Unused for
 *                 VRT_FINISH (may be NULL). Rows must be 16-byte aligned: the base
 *                 pointer 16-byte aligned and ld, tree_stride multiples of 16 bytes;
 *                 every row read must have ld addressable elements.
 *   ld, tree_stride  in elements, ld >= V
 *   seed, step    Philox key and counter word (the step counter, low 32 bits used)
 *   tree          device, vrt_tree_bytes(cfg) bytes, caller-owned, persists across
 *                 the layers of one step
 *   ws            device workspace of ws_bytes >= vrt_workspace_bytes(cfg)
 *   stats         device u32 [B][8] or NULL: status bits are OR-ed into stats[b][0]
 *   stream        hipStream_t
 * Layers must be called 0, 1, .., then VRT_FINISH: each layer expands the frontier
 * the previous one stored in the blob (indices read back from the blob are
 * range-checked on the device, so a wrong order gives wrong trees, never an
 * out-of-bounds access).
 * Errors: VRT_EINVAL (config, layer number, alignment, NULL pointers), VRT_ENOMEM
 * (ws_bytes too small), VRT_EHIP. */
vrt_status vrt_build_tree(const vrt_config* cfg, int32_t layer, const void* draft_logits,
                          int64_t ld, int64_t tree_stride, uint64_t seed, uint64_t step,
                          void* tree, void* ws, size_t ws_bytes, uint32_t* stats, void* stream);

/* Measurement helper, not a step of the method: streams `bytes` bytes of device
 * memory at buf once with the same 16-byte non-temporal loads the row kernels use
 * and ORs a checksum into *sink (device u32), so that the read cannot be elided. Its
 * achieved GB/s is this device's practical streaming-read ceiling.
 *   buf    device, 16-byte aligned;  bytes  a multiple of 16
 * Errors: VRT_EINVAL (alignment, NULL), VRT_EHIP. */
vrt_status vrt_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Verification of an emitted tree (RheoSampling key design 3).
 *   target_logits device, dtype cfg->dtype: the target row of node i of tree b starts
 *                 at element b*tree_stride + i*ld (rows i < n_nodes[b] are read);
 *                 same alignment rules as the draft rows
 *   tree          device tree blob whose emitted-tree arrays are filled (by finish or
 *                 by the caller following the layout)
 *   out_tokens    device i32 [B][D+1]: emitted tokens (accepted path, then the final
 *                 residual or bonus token); entries past out_len[b] are -1
 *   out_nodes     device i32 [B][D]: accepted node indices (entries past out_len[b]-1 are -1)
 *   out_len       device i32 [B]: number of emitted tokens (1 .. D+1)
 *   stats         device u32 [B][8]: [0] status bits, [1] accepted tree tokens,
 *                 [2] 1 if the probe was accepted somewhere on the path,
 *                 [3] draws on the path within 1e-6 of their threshold (near ties),
 *                 [4] nodes visited; [5..7] reserved (0)
 *   node_out      device i32 [B][N][4] or NULL: per node, decided as if the walk
 *                 reached it: [0] accepted child node or -1, [1] residual/bonus token
 *                 or -1, [2] tests taken (bits 0-7) | near ties (bits 8-15) | status
 *                 bits (from bit 16), [3] fp32 bits of the residual mass W the final
 *                 sample used (0 if a child was accepted)
 * Errors: as vrt_build_tree. */
vrt_status vrt_verify_tree(const vrt_config* cfg, const void* target_logits, int64_t ld,
                           int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                           void* ws, size_t ws_bytes, int32_t* out_tokens, int32_t* out_nodes,
                           int32_t* out_len, uint32_t* stats, int32_t* node_out, void* stream);

/* vrt_verify_tree for callers that cannot allocate device memory (code under graph
 * capture, serving loops, harnesses that forbid hipMalloc): the same arguments and outputs
 * without ws and ws_bytes. Its workspace is a static array of 4 MiB on each GPU, held until
 * the process ends and shared by every call on that GPU: calls that overlap on one GPU (two
 * streams, two threads) race and must not be issued. The call allocates nothing; it needs
 * vrt_workspace_bytes(cfg) <= 4 MiB (B * ((R+1) * 16 + 4096) bytes, plus alignment), else
 * VRT_ENOMEM. The GPU is the stream's (the current device for a NULL stream). Errors: as
 * vrt_verify_tree. */
vrt_status vrt_verify_tree_static(const vrt_config* cfg, const void* target_logits, int64_t ld,
                                  int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                                  int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                                  int32_t* node_out, void* stream);

/* The verification in its two parts, for callers that time or schedule them apart:
 * vrt_verify_nodes decides every node of every tree (its row statistics, the probe-first
 * test, the rejections of the other kept children, the final sample as if the walk
 * reached it) into node_out; vrt_verify_walk then follows the accepted children from
 * each root and writes out_tokens, out_nodes, out_len and stats. Together they do
 * exactly what vrt_verify_tree does. Arguments as there; both calls must get the same
 * ws and node_out (node_out NULL: the decisions stay in ws between the two calls).
 * vrt_verify_walk reads no logits. Errors: as vrt_verify_tree. */
vrt_status vrt_verify_nodes(const vrt_config* cfg, const void* target_logits, int64_t ld,
                            int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                            void* ws, size_t ws_bytes, int32_t* node_out, void* stream);
vrt_status vrt_verify_walk(const vrt_config* cfg, const void* tree, void* ws, size_t ws_bytes,
                           int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                           int32_t* node_out, void* stream);

/* Verification of a dense tree (trunc = VRT_DENSE, the dense baseline of RheoSampling's
 * support-size ablation): key design 3 as in vrt_verify_tree, with each kept probe's tail
 * (its expansion row but the deterministic children, q~ = the tempered softmax of that
 * draft row renormalised over the tail) regenerated from the draft rows the tree was
 * built from, since no tail table is kept. A node whose probe child is kept costs a second
 * pass over its target row together with that draft row.
 *   draft_logits       host array of D device pointers: layer l's draft rows exactly as
 *                      passed to vrt_build_tree for that layer (they must still hold them)
 *   draft_ld, draft_tree_stride  their strides (the same for every layer, as for the build)
 * Other arguments and outputs as vrt_verify_tree. Errors: as vrt_verify_tree, and
 * VRT_EINVAL if trunc is not VRT_DENSE or a draft pointer or stride is invalid. */
vrt_status vrt_verify_dense(const vrt_config* cfg, const void* target_logits, int64_t ld,
                            int64_t tree_stride, const void* const* draft_logits, int64_t draft_ld,
                            int64_t draft_tree_stride, const void* tree, uint64_t seed, uint64_t step,
                            void* ws, size_t ws_bytes, int32_t* out_tokens, int32_t* out_nodes,
                            int32_t* out_len, uint32_t* stats, int32_t* node_out, void* stream);

/* Lazy verification: the same outputs as vrt_verify_tree (RheoSampling key design 3:
 * the walk from the root, each visited node's probe-first test, the recursive rejection of
 * its other kept children and the final residual or bonus sample) computed by deciding
 * only the nodes the walk reaches, one tree per block, depth after depth. Only the target
 * rows of the visited nodes (as many as the emitted tokens) are read, instead of every
 * emitted node's row; the price is one dependent row pass per depth, so it pays where the
 * batch is small or the trees are large against the accepted length. Arguments as for
 * vrt_verify_tree. Differences: node_out (or the workspace) receives decisions for the
 * visited nodes only, and stats[b][0] reports a bad target row (VRT_ST_TARGET_BAD) only
 * for visited rows. Errors: as vrt_verify_tree. */
vrt_status vrt_verify_lazy(const vrt_config* cfg, const void* target_logits, int64_t ld,
                           int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                           void* ws, size_t ws_bytes, int32_t* out_tokens, int32_t* out_nodes,
                           int32_t* out_len, uint32_t* stats, int32_t* node_out, void* stream);

/* Coverage of the truncated support (RheoSampling's support-size ablation, whose
 * coverage column is the draft probability mass inside the support): for each of the
 * n_rows rows of each tree, the share of the untempered softmax of the row held by its
 * cfg->trunc largest logits (ties at the boundary hold equal mass, so which of them is
 * taken does not matter), in fp64 with exponentials to about 1e-7 relative. trunc =
 * VRT_DENSE, or trunc >= V, gives 1.
 *   draft_logits  device rows, laid out as for vrt_build_tree (row j of tree b at
 *                 b*tree_stride + j*ld elements; ld >= V; 16-byte aligned strides)
 *   n_rows        rows per tree (1 .. 65535)
 *   coverage      device f64 [B][n_rows]; 0 for a row with no finite logit, NaN for a row
 *                 holding NaN or +inf
 * A measurement of the inputs: the tree build does not need it. Errors: VRT_EINVAL
 * (config, pointers, strides, n_rows), VRT_EHIP. */
vrt_status vrt_support_coverage(const vrt_config* cfg, const void* draft_logits, int64_t ld,
                                int64_t tree_stride, int32_t n_rows, double* coverage, void* stream);

/* The step after the prune (RheoSampling framework flowchart: one target forward
 * verifies the whole tree): attention inputs of that forward over the emitted tree.
 * Node i of tree b attends to node j iff j lies on the path from the root to i, i
 * included (parents precede children, so the mask is lower triangular).
 *   tree  device tree blob whose emitted-tree arrays (n_nodes, node_parent) are filled;
 *         a parent index out of range [0, i) ends that node's path
 *   mask  device u32 [B][N][(N+31)/32]: bit j%32 of word j/32 of row i set iff j is on
 *         i's path; rows and columns at or past n_nodes[b] are 0
 *   pos   device i32 [B][N] or NULL: the number of ancestors of node i (its depth; add
 *         the context length for absolute positions), -1 past n_nodes[b]
 * Errors: VRT_EINVAL (config, NULL or misaligned pointers), VRT_EHIP. */
vrt_status vrt_tree_mask(const vrt_config* cfg, const void* tree, uint32_t* mask, int32_t* pos,
                         void* stream);

/* The KV entries to keep once a tree is verified: keep[b][0] = 0 (the root), then
 * keep[b][k] = out_nodes[b][k-1] for 1 <= k < out_len[b], -1 after (keep is device i32
 * [B][D+1]); keep_n[b] = out_len[b] (device i32 [B]). out_nodes and out_len as
 * vrt_verify_tree writes them (out_len clamped to 1 .. D+1).
 * Errors: VRT_EINVAL (config, NULL or misaligned pointers), VRT_EHIP. */
vrt_status vrt_accepted_kv(const vrt_config* cfg, const int32_t* out_nodes, const int32_t* out_len,
                           int32_t* keep, int32_t* keep_n, void* stream);

/* Description of the last error on this host thread ("" if none). */
const char* vrt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
