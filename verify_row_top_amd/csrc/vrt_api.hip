// Host side of the C ABI: validation, blob layout, workspace sizing, launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "vrt_internal.hpp"

namespace {

thread_local char g_err[256] = "";

vrt_status fail(vrt_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vrt_status fail(vrt_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int parents_per_layer(const vrt_config& c) {
  return c.mode == VRT_MODE_SMART ? c.budget : (c.W > 0 ? c.W : c.K);
}

bool compute_layout(const vrt_config& c, vrt_tree_layout* L) {
  const int64_t B = c.B, P = parents_per_layer(c);
  L->NC = c.K + (int64_t)(c.D - 1) * P * c.K;
  L->NR = 1 + (int64_t)(c.D - 1) * P;
  L->N = (c.mode == VRT_MODE_SMART ? c.budget : c.R) + 1;
  L->TC = c.trunc;
  L->FP = P;
  int64_t off = 0;
  auto take = [&](int64_t* field, int64_t bytes) {
    *field = off;
    off = align256(off + bytes);
  };
  take(&L->cand_token, B * L->NC * 4);
  take(&L->cand_parent, B * L->NC * 4);
  take(&L->cand_score, B * L->NC * 4);
  take(&L->cand_kind, B * L->NC * 4);
  take(&L->row_tail_n, B * L->NR * 4);
  take(&L->row_tail_id, B * L->NR * L->TC * 4);
  take(&L->row_tail_q, B * L->NR * L->TC * 4);
  take(&L->front, B * L->FP * 4);
  take(&L->n_front, B * 4);
  take(&L->smart, B * 8 * 8);
  take(&L->admitted, B * L->N * 4);
  take(&L->layer_sync, B * 4);
  take(&L->n_nodes, B * 4);
  take(&L->node_token, B * L->N * 4);
  take(&L->node_parent, B * L->N * 4);
  take(&L->node_depth, B * L->N * 4);
  take(&L->node_kind, B * L->N * 4);
  take(&L->node_cand, B * L->N * 4);
  take(&L->child_off, B * (L->N + 1) * 4);
  take(&L->child, B * L->N * 4);
  take(&L->tail_n, B * L->N * 4);
  take(&L->tail_id, B * L->N * L->TC * 4);
  take(&L->tail_q, B * L->N * L->TC * 4);
  const int64_t dense = c.trunc == VRT_DENSE ? 1 : 0;
  take(&L->row_dense, dense * B * L->NR * 2 * 8);
  take(&L->row_det, dense * B * L->NR * 32 * 4);
  take(&L->node_row, dense * B * L->N * 4);
  take(&L->row_sync, B * L->FP * 8);
  take(&L->smart_cost, c.mode == VRT_MODE_SMART ? (int64_t)(c.budget + 2) * 2 * 8 : 0);
  L->total_bytes = off;
  return true;
}

// Workspace: verification node outcomes [B][N], the verification's row statistics,
// then build scratch.
struct WsLayout {
  int64_t node_out, verify, build, total;
};

WsLayout ws_layout(const vrt_config& c) {
  vrt_tree_layout L;
  compute_layout(c, &L);
  WsLayout w;
  int64_t off = 0;
  w.node_out = off;
  off = align256(off + (int64_t)c.B * L.N * (int64_t)sizeof(vrt::NodeOut));
  w.verify = off;
  off = align256(off + (int64_t)vrt::verify_ws_bytes(vrt::make_cfg(c)));
  w.build = off;
  off = align256(off + (int64_t)vrt::build_ws_bytes(vrt::make_cfg(c)));
  w.total = off;
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// SMART key design 2's cost models and the derivative the keep rule uses, in fp64 with
// this host's libm, for tree sizes n = 0 .. budget+1: C(n) = lambda n + gamma (e^{delta
// n^rho} - 1) and C'(n) = lambda + gamma delta rho n^{rho-1} e^{delta n^rho}, each
// evaluated left to right as written.
void smart_cost_table(const vrt_config& c, double* tab) {
  for (int n = 0; n <= c.budget + 1; ++n) {
    const double x = (double)n;
    tab[2 * n] = c.lambda_ * x + c.gamma_ * (exp(c.delta_ * pow(x, c.rho_)) - 1.0);
    tab[2 * n + 1] = c.lambda_ + c.gamma_ * c.delta_ * c.rho_ * pow(x, c.rho_ - 1.0) * exp(c.delta_ * pow(x, c.rho_));
  }
}

vrt_status check_rows(const vrt_config& c, const void* p, int64_t ld, int64_t tstride,
                      const char* what) {
  if (!p) return fail(VRT_EINVAL, "%s logits pointer is NULL", what);
  const int64_t esz = c.dtype == VRT_BF16 ? 2 : 4;
  if (!aligned16(p)) return fail(VRT_EINVAL, "%s logits pointer is not 16-byte aligned", what);
  if (ld < c.V) return fail(VRT_EINVAL, "%s ld (%lld) < V (%d)", what, (long long)ld, c.V);
  if ((ld * esz) % 16 != 0 || (tstride * esz) % 16 != 0)
    return fail(VRT_EINVAL, "%s ld and tree_stride must be multiples of 16 bytes", what);
  if (tstride < 0) return fail(VRT_EINVAL, "%s tree_stride is negative", what);
  return VRT_OK;
}

}  // namespace

namespace vrt {

Cfg make_cfg(const vrt_config& c) {
  vrt_tree_layout L;
  compute_layout(c, &L);
  Cfg k;
  k.B = c.B; k.V = c.V; k.dtype = c.dtype; k.trunc = c.trunc; k.K = c.K; k.m = c.m;
  k.probe = c.probe; k.D = c.D; k.W = c.W > 0 ? c.W : c.K; k.R = c.R; k.mode = c.mode;
  k.budget = c.budget;
  k.P = parents_per_layer(c);
  k.NC = (int)L.NC; k.NR = (int)L.NR; k.N = (int)L.N; k.TC = (int)L.TC; k.FP = (int)L.FP;
  k.invT = 1.0f / c.T;
  k.c2 = k.invT * 1.44269504088896341f;
  k.eps_m0 = c.eps_m0;
  k.alpha = c.alpha; k.lam = c.lambda_; k.gam = c.gamma_; k.del = c.delta_; k.rho = c.rho_;
  k.order = c.probe ? c.order : VRT_PROBE_FIRST;
  k.tree_base = (uint32_t)c.tree_base;
  return k;
}

TreePtrs tree_ptrs(const vrt_config& c, void* blob) {
  vrt_tree_layout L;
  compute_layout(c, &L);
  char* p = (char*)blob;
  TreePtrs t;
  t.cand_token = (int*)(p + L.cand_token);
  t.cand_parent = (int*)(p + L.cand_parent);
  t.cand_score = (float*)(p + L.cand_score);
  t.cand_kind = (int*)(p + L.cand_kind);
  t.row_tail_n = (int*)(p + L.row_tail_n);
  t.row_tail_id = (int*)(p + L.row_tail_id);
  t.row_tail_q = (float*)(p + L.row_tail_q);
  t.front = (int*)(p + L.front);
  t.n_front = (int*)(p + L.n_front);
  t.smart = (double*)(p + L.smart);
  t.admitted = (int*)(p + L.admitted);
  t.layer_sync = (int*)(p + L.layer_sync);
  t.n_nodes = (int*)(p + L.n_nodes);
  t.node_token = (int*)(p + L.node_token);
  t.node_parent = (int*)(p + L.node_parent);
  t.node_depth = (int*)(p + L.node_depth);
  t.node_kind = (int*)(p + L.node_kind);
  t.node_cand = (int*)(p + L.node_cand);
  t.child_off = (int*)(p + L.child_off);
  t.child = (int*)(p + L.child);
  t.tail_n = (int*)(p + L.tail_n);
  t.tail_id = (int*)(p + L.tail_id);
  t.tail_q = (float*)(p + L.tail_q);
  t.row_dense = (double*)(p + L.row_dense);
  t.row_det = (int*)(p + L.row_det);
  t.node_row = (int*)(p + L.node_row);
  t.row_sync = (uint64_t*)(p + L.row_sync);
  t.smart_cost = (double*)(p + L.smart_cost);
  return t;
}

}  // namespace vrt

extern "C" {

const char* vrt_last_error(void) { return g_err; }

vrt_status vrt_check_config(const vrt_config* cp) {
  g_err[0] = 0;
  if (!cp) return fail(VRT_EINVAL, "config is NULL");
  const vrt_config& c = *cp;
  if (c.B < 1 || c.B > 65535) return fail(VRT_EINVAL, "B must be in [1, 65535] (got %d)", c.B);
  if (c.V < 1 || c.V > (1 << 20)) return fail(VRT_EINVAL, "V must be in [1, 2^20] (got %d)", c.V);
  if (c.dtype != VRT_F32 && c.dtype != VRT_BF16) return fail(VRT_EDTYPE, "dtype must be VRT_F32 or VRT_BF16");
  if (c.trunc != VRT_DENSE && (c.trunc < 1 || c.trunc > 1024))
    return fail(VRT_EINVAL, "trunc must be VRT_DENSE or in [1, 1024] (got %d)", c.trunc);
  if (c.K < 1 || c.K > 30) return fail(VRT_EINVAL, "K must be in [1, 30] (got %d)", c.K);
  if (c.probe != 0 && c.probe != 1) return fail(VRT_EINVAL, "probe must be 0 or 1");
  if (c.m < 0 || (c.probe && c.m > c.K - 1))
    return fail(VRT_EINVAL, "m must be in [0, K-1] with the probe on (m=%d, K=%d)", c.m, c.K);
  if (c.D < 1 || c.D > 32) return fail(VRT_EINVAL, "D must be in [1, 32] (got %d)", c.D);
  if (c.tree_base < 0) return fail(VRT_EINVAL, "tree_base must be >= 0 (got %d)", c.tree_base);
  if (c.order != VRT_PROBE_FIRST && c.order != VRT_PROBE_LAST)
    return fail(VRT_EINVAL, "order must be VRT_PROBE_FIRST or VRT_PROBE_LAST (got %d)", c.order);
  if (c.mode != VRT_MODE_TOPR && c.mode != VRT_MODE_SMART) return fail(VRT_EINVAL, "unknown mode %d", c.mode);
  if (c.mode == VRT_MODE_TOPR) {
    if (c.W < 0 || c.W > 1024) return fail(VRT_EINVAL, "W must be in [0, 1024] (got %d)", c.W);
    if (c.R < 1 || c.R > 1024) return fail(VRT_EINVAL, "R must be in [1, 1024] (got %d)", c.R);
  } else {
    if (c.budget < 1 || c.budget > 1024) return fail(VRT_EINVAL, "budget must be in [1, 1024] (got %d)", c.budget);
    if (!(c.alpha > 0.0 && c.alpha <= 1.0)) return fail(VRT_EINVAL, "alpha must be in (0, 1]");
    if (!isfinite(c.lambda_) || !isfinite(c.gamma_) || !isfinite(c.delta_) || !isfinite(c.rho_) ||
        c.lambda_ < 0 || c.gamma_ < 0 || c.delta_ < 0)
      return fail(VRT_EINVAL, "SMART cost constants must be finite and non-negative");
  }
  if (!(c.T > 0.0f) || !isfinite(c.T)) return fail(VRT_EINVAL, "T must be positive and finite");
  if (!(1.0f / c.T < INFINITY)) return fail(VRT_EINVAL, "T too small: 1/T overflows");
  if (!(c.eps_m0 >= 0.0f) || !isfinite(c.eps_m0)) return fail(VRT_EINVAL, "eps_m0 must be finite, >= 0");
  vrt_tree_layout L;
  compute_layout(c, &L);
  // per-layer candidate sets and the top-R candidate pool are sorted in LDS
  if (L.FP * c.K > 4096) return fail(VRT_EINVAL, "parents per layer times K must be <= 4096");
  if (c.mode == VRT_MODE_TOPR && L.NC > 4096)
    return fail(VRT_EINVAL, "K + (D-1) W K must be <= 4096 in top-R mode (got %lld)", (long long)L.NC);
  if (L.NC > (1 << 20) || L.N > 4097) return fail(VRT_EINVAL, "tree capacity too large");
  return VRT_OK;
}

vrt_status vrt_tree_layout_of(const vrt_config* c, vrt_tree_layout* out) {
  const vrt_status s = vrt_check_config(c);
  if (s != VRT_OK) return s;
  if (!out) return fail(VRT_EINVAL, "layout output is NULL");
  compute_layout(*c, out);
  return VRT_OK;
}

size_t vrt_tree_bytes(const vrt_config* c) {
  if (vrt_check_config(c) != VRT_OK) return 0;
  vrt_tree_layout L;
  compute_layout(*c, &L);
  return (size_t)L.total_bytes;
}

size_t vrt_workspace_bytes(const vrt_config* c) {
  if (vrt_check_config(c) != VRT_OK) return 0;
  return (size_t)ws_layout(*c).total;
}

vrt_status vrt_build_tree(const vrt_config* cp, int32_t layer, const void* draft_logits,
                          int64_t ld, int64_t tree_stride, uint64_t seed, uint64_t step,
                          void* tree, void* ws, size_t ws_bytes, uint32_t* stats, void* stream) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  const vrt_config& c = *cp;
  if (layer != VRT_FINISH && (layer < 0 || layer >= c.D))
    return fail(VRT_EINVAL, "layer must be in [0, D) or VRT_FINISH (got %d)", layer);
  if (!tree || !ws) return fail(VRT_EINVAL, "tree and workspace pointers must not be NULL");
  if (!aligned16(tree) || !aligned16(ws)) return fail(VRT_EINVAL, "tree and workspace must be 16-byte aligned");
  const WsLayout wl = ws_layout(c);
  if (ws_bytes < (size_t)wl.total)
    return fail(VRT_ENOMEM, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)wl.total);
  if (layer != VRT_FINISH) {
    s = check_rows(c, draft_logits, ld, tree_stride, "draft");
    if (s != VRT_OK) return s;
  }
  const vrt::Cfg k = vrt::make_cfg(c);
  const vrt::TreePtrs t = vrt::tree_ptrs(c, tree);
  hipError_t e;
  if (layer == VRT_FINISH) {
    e = vrt::launch_build_finish(k, t, (char*)ws + wl.build, (hipStream_t)stream);
  } else {
    e = hipSuccess;
    if (layer == 0 && c.mode == VRT_MODE_SMART) {  // the keep rule's cost table, for this step
      double tab[2 * (1024 + 2)];
      smart_cost_table(c, tab);
      e = vrt::launch_fill_f64(t.smart_cost, tab, 2 * (c.budget + 2), (hipStream_t)stream);
    }
    if (e == hipSuccess)
      e = vrt::launch_build_layer(k, t, layer, draft_logits, ld, tree_stride, seed, (uint32_t)step,
                                  stats, (char*)ws + wl.build, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

vrt_status vrt_support_coverage(const vrt_config* cp, const void* draft_logits, int64_t ld,
                                int64_t tree_stride, int32_t n_rows, double* coverage, void* stream) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  const vrt_config& c = *cp;
  if (n_rows < 1 || n_rows > 65535) return fail(VRT_EINVAL, "n_rows must be in [1, 65535] (got %d)", n_rows);
  if (!coverage || ((uintptr_t)coverage & 7u)) return fail(VRT_EINVAL, "coverage must be a non-NULL, 8-byte aligned pointer");
  s = check_rows(c, draft_logits, ld, tree_stride, "draft");
  if (s != VRT_OK) return s;
  const hipError_t e = vrt::launch_coverage(vrt::make_cfg(c), draft_logits, ld, tree_stride, n_rows, coverage,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

namespace {

// Validation and launch shared by the verification entry points (parts as in
// launch_verify). Pointers a part does not use may be NULL.
vrt_status verify_parts(int parts, const vrt_config* cp, const void* target_logits, int64_t ld,
                        int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step, void* ws,
                        size_t ws_bytes, int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len,
                        uint32_t* stats, int32_t* node_out, void* stream, const void* const* draft = nullptr,
                        int64_t dld = 0, int64_t dstride = 0) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  const vrt_config& c = *cp;
  if (c.trunc == VRT_DENSE && c.probe && !(parts & 8))
    return fail(VRT_EINVAL, "trees built with trunc = VRT_DENSE and the probe on carry no tail table: "
                            "verify them with vrt_verify_dense, which regenerates the tails from the "
                            "draft rows");
  if (parts & 8) {
    if (c.trunc != VRT_DENSE) return fail(VRT_EINVAL, "vrt_verify_dense needs trunc = VRT_DENSE");
    if (!draft) return fail(VRT_EINVAL, "draft row pointer array is NULL");
    for (int l = 0; l < c.D; ++l) {
      s = check_rows(c, draft[l], dld, dstride, "draft");
      if (s != VRT_OK) return s;
    }
  }
  if (!tree || !ws) return fail(VRT_EINVAL, "tree and workspace pointers must not be NULL");
  if (!aligned16(tree) || !aligned16(ws)) return fail(VRT_EINVAL, "tree and workspace must be 16-byte aligned");
  if ((parts & 6) && (!out_tokens || !out_nodes || !out_len || !stats))
    return fail(VRT_EINVAL, "output pointers must not be NULL");
  if (node_out && ((uintptr_t)node_out & 15u)) return fail(VRT_EINVAL, "node_out must be 16-byte aligned");
  const WsLayout wl = ws_layout(c);
  if (ws_bytes < (size_t)wl.total)
    return fail(VRT_ENOMEM, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)wl.total);
  if (parts & 5) {
    s = check_rows(c, target_logits, ld, tree_stride, "target");
    if (s != VRT_OK) return s;
  }
  const vrt::Cfg k = vrt::make_cfg(c);
  const vrt::TreePtrs t = vrt::tree_ptrs(c, (void*)tree);
  vrt::NodeOut* no = node_out ? (vrt::NodeOut*)node_out : (vrt::NodeOut*)((char*)ws + wl.node_out);
  const hipError_t e = vrt::launch_verify(parts, k, t, target_logits, ld, tree_stride, seed,
                                          (uint32_t)step, no, out_tokens, out_nodes, out_len, stats,
                                          (char*)ws + wl.verify, draft, dld, dstride, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

}  // namespace

vrt_status vrt_verify_tree(const vrt_config* cp, const void* target_logits, int64_t ld,
                           int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                           void* ws, size_t ws_bytes, int32_t* out_tokens, int32_t* out_nodes,
                           int32_t* out_len, uint32_t* stats, int32_t* node_out, void* stream) {
  return verify_parts(3, cp, target_logits, ld, tree_stride, tree, seed, step, ws, ws_bytes, out_tokens,
                      out_nodes, out_len, stats, node_out, stream);
}

namespace {

// The verification's workspace for callers that cannot allocate: one array per GPU, held
// until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory: the kernels get the device address hipGetSymbolAddress gives for the GPU the
// stream belongs to, looked up once per device with that device current.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

vrt_status scratch_of(void* stream, void** out) {
  int dev = 0, cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(VRT_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice((hipStream_t)stream, &dev);
    if (e != hipSuccess) return fail(VRT_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(VRT_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(VRT_EHIP, "hipSetDevice failed: %s", hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess && e == hipSuccess)
      return fail(VRT_EHIP, "hipSetDevice could not restore device %d", cur);
    if (e != hipSuccess || !ptr)
      return fail(VRT_EHIP, "hipGetSymbolAddress of the static workspace failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VRT_OK;
}

}  // namespace

vrt_status vrt_verify_tree_static(const vrt_config* cp, const void* target_logits, int64_t ld,
                                  int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                                  int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                                  int32_t* node_out, void* stream) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  const size_t need = (size_t)ws_layout(*cp).total;
  if (need > kScratchBytes)
    return fail(VRT_ENOMEM, "vrt_verify_tree_static needs a %zu-byte workspace; its static one holds %zu "
                            "bytes (use vrt_verify_tree with a workspace of your own)", need, kScratchBytes);
  void* ws = nullptr;
  s = scratch_of(stream, &ws);
  if (s != VRT_OK) return s;
  return verify_parts(3, cp, target_logits, ld, tree_stride, tree, seed, step, ws, kScratchBytes, out_tokens,
                      out_nodes, out_len, stats, node_out, stream);
}

vrt_status vrt_verify_dense(const vrt_config* cp, const void* target_logits, int64_t ld, int64_t tree_stride,
                            const void* const* draft_logits, int64_t draft_ld, int64_t draft_tree_stride,
                            const void* tree, uint64_t seed, uint64_t step, void* ws, size_t ws_bytes,
                            int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                            int32_t* node_out, void* stream) {
  return verify_parts(3 | 8, cp, target_logits, ld, tree_stride, tree, seed, step, ws, ws_bytes, out_tokens,
                      out_nodes, out_len, stats, node_out, stream, draft_logits, draft_ld, draft_tree_stride);
}

vrt_status vrt_verify_lazy(const vrt_config* cp, const void* target_logits, int64_t ld, int64_t tree_stride,
                           const void* tree, uint64_t seed, uint64_t step, void* ws, size_t ws_bytes,
                           int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                           int32_t* node_out, void* stream) {
  return verify_parts(4, cp, target_logits, ld, tree_stride, tree, seed, step, ws, ws_bytes, out_tokens,
                      out_nodes, out_len, stats, node_out, stream);
}

vrt_status vrt_verify_nodes(const vrt_config* cp, const void* target_logits, int64_t ld,
                            int64_t tree_stride, const void* tree, uint64_t seed, uint64_t step,
                            void* ws, size_t ws_bytes, int32_t* node_out, void* stream) {
  return verify_parts(1, cp, target_logits, ld, tree_stride, tree, seed, step, ws, ws_bytes, nullptr,
                      nullptr, nullptr, nullptr, node_out, stream);
}

vrt_status vrt_verify_walk(const vrt_config* cp, const void* tree, void* ws, size_t ws_bytes,
                           int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                           int32_t* node_out, void* stream) {
  return verify_parts(2, cp, nullptr, 0, 0, tree, 0, 0, ws, ws_bytes, out_tokens, out_nodes, out_len,
                      stats, node_out, stream);
}

vrt_status vrt_tree_mask(const vrt_config* cp, const void* tree, uint32_t* mask, int32_t* pos,
                         void* stream) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  if (!tree || !mask) return fail(VRT_EINVAL, "tree and mask pointers must not be NULL");
  if (!aligned16(tree) || ((uintptr_t)mask & 3u) || ((uintptr_t)pos & 3u))
    return fail(VRT_EINVAL, "tree must be 16-byte and mask, pos 4-byte aligned");
  const hipError_t e = vrt::launch_tree_mask(vrt::make_cfg(*cp), vrt::tree_ptrs(*cp, (void*)tree), mask,
                                             pos, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

vrt_status vrt_accepted_kv(const vrt_config* cp, const int32_t* out_nodes, const int32_t* out_len,
                           int32_t* keep, int32_t* keep_n, void* stream) {
  vrt_status s = vrt_check_config(cp);
  if (s != VRT_OK) return s;
  if (!out_nodes || !out_len || !keep || !keep_n)
    return fail(VRT_EINVAL, "pointers must not be NULL");
  if (((uintptr_t)out_nodes | (uintptr_t)out_len | (uintptr_t)keep | (uintptr_t)keep_n) & 3u)
    return fail(VRT_EINVAL, "pointers must be 4-byte aligned");
  const hipError_t e = vrt::launch_accepted_kv(vrt::make_cfg(*cp), out_nodes, out_len, keep, keep_n,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

vrt_status vrt_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(VRT_EINVAL, "buffer and sink must not be NULL");
  if (!aligned16(buf) || (bytes & 15u)) return fail(VRT_EINVAL, "buffer and size must be 16-byte aligned");
  const hipError_t e = vrt::launch_read_probe(buf, bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VRT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return VRT_OK;
}

}  // extern "C"
