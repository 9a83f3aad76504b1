// Internal types shared by the host entry points and the kernels of libvrt.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vrt.h"

namespace vrt {

// Kernel-side copy of the configuration with derived capacities.
struct Cfg {
  int B, V, dtype, trunc, K, m, probe, D, W, R, mode, budget;
  int P;   // parents per layer >= 1 (W in top-R mode, budget in SMART mode)
  int NC;  // candidates per tree
  int NR;  // expansion rows per tree
  int N;   // emitted nodes per tree, root included
  int TC;  // tail capacity (= trunc)
  int FP;  // frontier slots
  float invT;  // fl32(1 / T)
  float c2;    // fl32(invT * log2(e)): exp((x - M)/T) = exp2(x*c2 - M*c2)
  float eps_m0;
  double alpha, lam, gam, del, rho;
  int order;  // VRT_PROBE_FIRST / VRT_PROBE_LAST (probe on only)
  uint32_t tree_base;  // tree index of tree 0 in the draws' keys
};

// Typed views of the caller's tree blob (see vrt_tree_layout in vrt.h).
struct TreePtrs {
  int* cand_token;
  int* cand_parent;
  float* cand_score;
  int* cand_kind;
  int* row_tail_n;
  int* row_tail_id;
  float* row_tail_q;
  int* front;
  int* n_front;
  double* smart;
  int* admitted;
  int* layer_sync;
  int* n_nodes;
  int* node_token;
  int* node_parent;
  int* node_depth;
  int* node_kind;
  int* node_cand;
  int* child_off;
  int* child;
  int* tail_n;
  int* tail_id;
  float* tail_q;
  double* row_dense;  // dense rows: [NR][2] (largest logit, tempered tail mass)
  int* row_det;       // dense rows: [NR][32] deterministic children's tokens
  int* node_row;      // dense rows: [N] expansion row of a node whose probe is kept
  uint64_t* row_sync;  // [FP] tag of the half of a split row that finished first
  double* smart_cost;  // SMART: [budget+2][2] C(n), C'(n) for n = 0 .. budget+1 (one table)
};

// Per-node verification outcome: accepted child node (-1: none), final token
// (-1: none), flags = tests taken (bits 0-7) | near ties (bits 8-15) | status
// bits (from bit 16), and the residual mass W of the final sample (0 otherwise).
struct NodeOut {
  int accept, token, flags;
  float W;
};

Cfg make_cfg(const vrt_config& c);
TreePtrs tree_ptrs(const vrt_config& c, void* blob);

// Device scratch of the verification: per-chunk row statistics and per-tree counters.
size_t verify_ws_bytes(const Cfg& c);

hipError_t launch_tree_mask(const Cfg& c, const TreePtrs& t, uint32_t* mask, int32_t* pos,
                            hipStream_t stream);
hipError_t launch_accepted_kv(const Cfg& c, const int32_t* out_nodes, const int32_t* out_len,
                              int32_t* keep, int32_t* keep_n, hipStream_t stream);

// parts: 1 = decide every node (k_vnode), 2 = walk (k_vwalk), 3 = both, 4 = the lazy walk
// (k_vlazy: decide only the nodes the walk reaches); + 8: dense rows, the nodes decided by
// k_vnode_dense with the probe tails regenerated from draft[l] (layer l's draft rows,
// row j of tree b at b*dstride + j*dld elements)
hipError_t launch_verify(int parts, const Cfg& c, const TreePtrs& t, const void* logits, int64_t ld,
                         int64_t tstride, uint64_t seed, uint32_t step, NodeOut* node_out,
                         int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                         void* ws, const void* const* draft, int64_t dld, int64_t dstride,
                         hipStream_t stream);

// Device scratch of the build: each row segment's sorted top-trunc keys and counts.
size_t build_ws_bytes(const Cfg& c);

hipError_t launch_coverage(const Cfg& c, const void* logits, int64_t ld, int64_t tstride, int n_rows,
                           double* out, hipStream_t stream);
hipError_t launch_build_layer(const Cfg& c, const TreePtrs& t, int layer, const void* logits,
                              int64_t ld, int64_t tstride, uint64_t seed, uint32_t step,
                              uint32_t* stats, void* ws, hipStream_t stream);
hipError_t launch_build_finish(const Cfg& c, const TreePtrs& t, void* ws, hipStream_t stream);

// Copies n host-computed doubles into device memory at dst through kernel arguments (no
// host buffer outlives the call, and the copy is an ordinary kernel on the stream).
hipError_t launch_fill_f64(double* dst, const double* vals, int n, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace vrt
