// Seeded synthetic logits: the stand-in for the draft and target language models.
//
// This module is the only code that both the CPU oracle's tests and the HIP
// path's tests/benchmark use. It holds none of the tree-building or
// verification arithmetic: it only turns (seed, node key, token id) into
// logits. Every routine is written once as __host__ __device__ code, so the
// host loop (used to feed the oracle) and the device kernel (used to fill HBM
// for the benchmark) produce bit-identical values. The file must be compiled
// with -ffp-contract=off so that no multiply-add is fused on either side.
//
// Recipe (per node row, node key h, vocabulary size V):
//   * A keyed affine permutation rank(v) = (A*v + C) mod V, gcd(A, V) = 1.
//   * Base logit: a Zipf table z[rank] = -a*ln(rank+1) (passed in as data), or 0.
//   * Jitter n(h, v): Irwin-Hall sum of four 16-bit uniforms from Philox4x32-10,
//     centred and scaled to unit variance (support +-3.46): a stated stand-in
//     for a standard normal draw.
//   * draft  = round(z[rank(v)] + s_draft * n(h, v))     (bf16 RNE or fp32)
//   * target = round(float(draft) + sigma * n'(h, v))     (independent jitter n')
// A node key is a splitmix64 chain over the token path from a per-tree root key,
// so the logits at a context depend only on that context.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYN_HD __host__ __device__ inline

namespace {

struct SynParams {
  int32_t V;
  int32_t dtype;        // 0 = fp32 rows, 1 = bf16 rows
  int32_t n_tables;     // 0: no Zipf base; 1 or 2 Zipf tables of length V
  int32_t split;        // trees b < split use table 0, the others table n_tables-1
  float draft_scale;    // multiplier on the draft jitter
  float target_sigma;   // standard deviation of the target's extra jitter
  uint64_t seed;
};

SYN_HD uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): the generator's own copy.
SYN_HD void philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                   uint32_t k1, uint32_t out[4]) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

SYN_HD uint32_t gcd_u32(uint32_t a, uint32_t b) {
  while (b) {
    const uint32_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

SYN_HD void perm_of(const SynParams& p, uint64_t h, uint32_t* A, uint32_t* C) {
  uint32_t o[4];
  philox(0xFFFFFFFFu, (uint32_t)h, (uint32_t)(h >> 32), 16u, (uint32_t)p.seed,
         (uint32_t)(p.seed >> 32), o);
  const uint32_t V = (uint32_t)p.V;
  if (V <= 1) {
    *A = 1; *C = 0;
    return;
  }
  uint32_t a = 1u + o[0] % (V - 1u);
  while (gcd_u32(a, V) != 1u) a = (a + 1u == V) ? 1u : a + 1u;
  *A = a;
  *C = o[1] % V;
}

SYN_HD float jitter(const SynParams& p, uint64_t h, uint32_t v, uint32_t stream) {
  uint32_t o[4];
  philox(v, (uint32_t)h, (uint32_t)(h >> 32), stream, (uint32_t)p.seed, (uint32_t)(p.seed >> 32), o);
  const int32_t s = (int32_t)((o[0] >> 16) + (o[1] >> 16) + (o[2] >> 16) + (o[3] >> 16)) - 131072;
  const float scale = 1.7320508075688772f / 65536.0f;
  return (float)s * scale;
}

SYN_HD uint16_t bf16_rne(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

SYN_HD float bf16_to_f(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

// One logit. which = 0: draft, 1: target.
SYN_HD void gen_one(const SynParams& p, const float* zipf, int32_t tree, uint64_t h, uint32_t A,
                    uint32_t C, uint32_t v, int which, void* out, int64_t off) {
  const uint32_t V = (uint32_t)p.V;
  const uint32_t rank = (uint32_t)(((uint64_t)A * v + C) % V);
  float base = 0.0f;
  if (p.n_tables > 0) {
    const int tab = (tree < p.split) ? 0 : (p.n_tables - 1);
    base = zipf[(int64_t)tab * V + rank];
  }
  const float jd = p.draft_scale * jitter(p, h, v, 17u);
  float d = base + jd;
  if (p.dtype == 1) {
    const uint16_t db = bf16_rne(d);
    if (which == 0) {
      ((uint16_t*)out)[off] = db;
      return;
    }
    const float jt = p.target_sigma * jitter(p, h, v, 18u);
    ((uint16_t*)out)[off] = bf16_rne(bf16_to_f(db) + jt);
  } else {
    if (which == 0) {
      ((float*)out)[off] = d;
      return;
    }
    const float jt = p.target_sigma * jitter(p, h, v, 18u);
    ((float*)out)[off] = d + jt;
  }
}

SYN_HD uint64_t node_key(uint64_t parent, int32_t token) {
  return sm64(parent ^ sm64((uint64_t)(uint32_t)token + 0x632BE59BD9B4E019ull));
}

__global__ void k_rows(SynParams p, const float* __restrict__ zipf, int32_t n_rows,
                       const uint64_t* __restrict__ keys, const int32_t* __restrict__ tree_of_row,
                       void* out, int64_t ld, int which) {
  const int32_t row = blockIdx.y;
  if (row >= n_rows) return;
  const uint64_t h = keys[row];
  if (h == 0ull) return;  // key 0 marks an unused row: left untouched
  uint32_t A, C;
  perm_of(p, h, &A, &C);
  const int32_t tree = tree_of_row ? tree_of_row[row] : 0;
  for (uint32_t v = blockIdx.x * blockDim.x + threadIdx.x; v < (uint32_t)p.V;
       v += gridDim.x * blockDim.x)
    gen_one(p, zipf, tree, h, A, C, v, which, out, (int64_t)row * ld + v);
}

// Keys of the next frontier: child key = node_key(key of the row that created it, token).
// next[b][j] is a candidate creation index c; its creating row within the layer
// is (c - base) / K, and its token is cand_token[b][c].
__global__ void k_frontier_keys(int32_t B, int32_t K, int32_t base, int32_t prev_stride,
                                const uint64_t* __restrict__ prev_keys,
                                const int32_t* __restrict__ next, const int32_t* __restrict__ n_next,
                                int32_t next_stride, const int32_t* __restrict__ cand_token,
                                int32_t cand_stride, uint64_t* out) {
  const int32_t b = blockIdx.x;
  if (b >= B) return;
  for (int32_t j = threadIdx.x; j < next_stride; j += blockDim.x) {
    uint64_t key = 0ull;
    if (j < n_next[b]) {
      const int32_t c = next[(int64_t)b * next_stride + j];
      const int32_t pos = (c - base) / K;
      key = node_key(prev_keys[(int64_t)b * prev_stride + pos],
                     cand_token[(int64_t)b * cand_stride + c]);
    }
    out[(int64_t)b * next_stride + j] = key;
  }
}

// Keys of every node of an emitted tree (parents precede children).
__global__ void k_tree_keys(int32_t B, int32_t N, const uint64_t* __restrict__ root_keys,
                            const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ token,
                            const int32_t* __restrict__ parent, uint64_t* out) {
  const int32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t o = (int64_t)b * N;
  const int32_t n = n_nodes[b];
  out[o] = root_keys[b];
  for (int32_t i = 1; i < N; ++i)
    out[o + i] = (i < n) ? node_key(out[o + parent[o + i]], token[o + i]) : 0ull;
}

}  // namespace

extern "C" {

struct syn_params_c {
  int32_t V, dtype, n_tables, split;
  float draft_scale, target_sigma;
  uint64_t seed;
};

static SynParams to_p(const syn_params_c* c) {
  SynParams p;
  p.V = c->V;
  p.dtype = c->dtype;
  p.n_tables = c->n_tables;
  p.split = c->split;
  p.draft_scale = c->draft_scale;
  p.target_sigma = c->target_sigma;
  p.seed = c->seed;
  return p;
}

uint64_t syn_node_key(uint64_t parent, int32_t token) { return node_key(parent, token); }

uint64_t syn_root_key(uint64_t seed, int32_t b) {
  uint64_t k = sm64(sm64(seed ^ 0xA0761D6478BD642Full) + (uint64_t)(uint32_t)b);
  return k ? k : 1ull;
}

// Host generation: n_rows rows with the given node keys into out (row stride ld elements).
void syn_rows_host(const syn_params_c* pc, const float* zipf, int32_t n_rows, const uint64_t* keys,
                   const int32_t* tree_of_row, void* out, int64_t ld, int32_t which) {
  const SynParams p = to_p(pc);
  for (int32_t r = 0; r < n_rows; ++r) {
    const uint64_t h = keys[r];
    if (h == 0ull) continue;
    uint32_t A, C;
    perm_of(p, h, &A, &C);
    const int32_t tree = tree_of_row ? tree_of_row[r] : 0;
    for (uint32_t v = 0; v < (uint32_t)p.V; ++v)
      gen_one(p, zipf, tree, h, A, C, v, which, out, (int64_t)r * ld + v);
  }
}

// Device generation on the given stream. All pointers are device pointers.
int32_t syn_rows_dev(const syn_params_c* pc, const float* zipf, int32_t n_rows, const uint64_t* keys,
                     const int32_t* tree_of_row, void* out, int64_t ld, int32_t which, void* stream) {
  if (n_rows <= 0) return 0;
  const SynParams p = to_p(pc);
  int gx = (p.V + 255) / 256;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(k_rows, dim3(gx, n_rows), dim3(256), 0, (hipStream_t)stream, p, zipf, n_rows,
                     keys, tree_of_row, out, ld, which);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t syn_frontier_keys_dev(int32_t B, int32_t K, int32_t base, int32_t prev_stride,
                              const uint64_t* prev_keys, const int32_t* next, const int32_t* n_next,
                              int32_t next_stride, const int32_t* cand_token, int32_t cand_stride,
                              uint64_t* out, void* stream) {
  hipLaunchKernelGGL(k_frontier_keys, dim3(B), dim3(64), 0, (hipStream_t)stream, B, K, base,
                     prev_stride, prev_keys, next, n_next, next_stride, cand_token, cand_stride, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t syn_tree_keys_dev(int32_t B, int32_t N, const uint64_t* root_keys, const int32_t* n_nodes,
                          const int32_t* token, const int32_t* parent, uint64_t* out, void* stream) {
  hipLaunchKernelGGL(k_tree_keys, dim3((B + 63) / 64), dim3(64), 0, (hipStream_t)stream, B, N,
                     root_keys, n_nodes, token, parent, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
