// The step after the prune (RheoSampling framework flowchart: one target forward verifies
// the whole tree): the attention structure of that forward over the emitted tree, and the
// KV entries kept once the tree is verified.
//
// k_tree_mask: one block per tree. The tree's parents are staged in LDS; thread (i, w)
// follows node i's parents to the root (parents precede children, so the walk ends) and
// writes word w of row i: bit j set iff node j lies on the path from the root to i.
// k_accepted_kv: one wave per tree copies the root and the accepted path.
#include "vrt_dev.hpp"
#include "vrt_internal.hpp"

namespace vrt {
namespace {

constexpr int kMT = 256;  // threads of a mask block

__global__ __launch_bounds__(kMT) void k_tree_mask(const Cfg c, const TreePtrs t, uint32_t* mask,
                                                   int32_t* pos) {
  const int b = blockIdx.x;
  const int N = c.N;
  const int W32 = (N + 31) / 32;
  const int64_t nb = (int64_t)b * N;
  int nn = t.n_nodes[b];
  nn = nn < 1 ? 1 : (nn > N ? N : nn);
  extern __shared__ int s_par[];  // [N]
  for (int i = threadIdx.x; i < nn; i += kMT) {
    const int p = t.node_parent[nb + i];
    // a parent out of range ends the node's path there
    s_par[i] = (i > 0 && p >= 0 && p < i) ? p : -1;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < N * W32; x += kMT) {
    const int i = x / W32, w = x - i * W32;
    uint32_t word = 0u;
    int depth = -1;
    if (i < nn) {
      for (int a = i; a >= 0; a = s_par[a]) {
        if ((a >> 5) == w) word |= 1u << (a & 31);
        ++depth;
      }
    }
    mask[(nb + i) * W32 + w] = word;
    if (w == 0 && pos) pos[nb + i] = depth;
  }
}

__global__ __launch_bounds__(kWave) void k_accepted_kv(const Cfg c, const int32_t* out_nodes,
                                                       const int32_t* out_len, int32_t* keep,
                                                       int32_t* keep_n) {
  const int b = blockIdx.x;
  int len = out_len[b];
  len = len < 1 ? 1 : (len > c.D + 1 ? c.D + 1 : len);
  for (int k = lane_id(); k <= c.D; k += kWave)
    keep[(int64_t)b * (c.D + 1) + k] = k == 0 ? 0 : (k < len ? out_nodes[(int64_t)b * c.D + k - 1] : -1);
  if (lane_id() == 0) keep_n[b] = len;
}

}  // namespace

hipError_t launch_tree_mask(const Cfg& c, const TreePtrs& t, uint32_t* mask, int32_t* pos,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_mask, dim3(c.B), dim3(kMT), (size_t)c.N * 4, stream, c, t, mask, pos);
  return hipGetLastError();
}

hipError_t launch_accepted_kv(const Cfg& c, const int32_t* out_nodes, const int32_t* out_len,
                              int32_t* keep, int32_t* keep_n, hipStream_t stream) {
  hipLaunchKernelGGL(k_accepted_kv, dim3(c.B), dim3(kWave), 0, stream, c, out_nodes, out_len, keep,
                     keep_n);
  return hipGetLastError();
}

}  // namespace vrt
