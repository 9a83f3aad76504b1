// Draft-tree construction on gfx950 (RheoSampling framework flowchart, key designs
// 1-2; SMART key design 3 as the switchable keep rule).
//
// k_support_expand: one 1024-thread block per expanded parent. The block streams the
//   parent's draft row once (four 16-byte loads per thread in flight) and keeps the
//   row's top-`trunc` entries by (logit desc, token id asc) in an LDS candidate buffer
//   behind a running threshold: the first pass seeds the threshold with the
//   trunc-th largest of the threads' own maxima, later elements are appended only if
//   they beat it, and a full buffer is compacted by a bitonic sort that raises it.
//   Wave 0 then expands the parent: untempered softmax on the support with the fixed
//   ranking recipe, tempered softmax in fp64, the probe draw from the tempered tail,
//   the proxy min{q(x_m), z}, the K child slots and the parent's tail table.
// k_beam / k_smart: one block per tree ranks the layer's children by (path score
//   desc, creation index asc) and keeps the top W (top-R mode) or runs SMART's
//   sequential keep rule over them.
// k_finish: one block per tree emits the tree: the global top R by the same key
//   (or SMART's admitted nodes), parents before children, child lists in slot
//   order, and the probe tails the verifier needs.
#include "vrt_dev.hpp"
#include "vrt_internal.hpp"

namespace vrt {
namespace {

constexpr int kSB = 1024;  // threads per support block
constexpr int kSU = 4;     // 16-byte loads per thread per pass

__device__ __forceinline__ int layer_base(const Cfg& c, int l) {
  return l == 0 ? 0 : c.K + (l - 1) * c.P * c.K;
}
__device__ __forceinline__ int row_base(const Cfg& c, int l) { return l == 0 ? 0 : 1 + (l - 1) * c.P; }
__device__ __forceinline__ int layer_span(const Cfg& c, int l) { return (l == 0 ? 1 : c.P) * c.K; }
__device__ __forceinline__ int layer_of(const Cfg& c, int cidx) {
  return cidx < c.K ? 0 : 1 + (cidx - c.K) / (c.P * c.K);
}
__device__ __forceinline__ int row_of(const Cfg& c, int cidx) {
  const int l = layer_of(c, cidx);
  return row_base(c, l) + (cidx - layer_base(c, l)) / c.K;
}

struct BArgs {
  Cfg c;
  TreePtrs t;
  int layer;
  const void* logits;
  int64_t ld, tstride;
  uint64_t seed;
  uint32_t step;
  uint32_t* stats;
};

// Wave-aggregated append of `key` into the LDS buffer when `pass`. Returns true if
// stored; sets *ovf when the buffer is full (the key is then retried later).
__device__ __forceinline__ bool append(bool pass, uint64_t key, uint64_t* buf, int cap, int* cnt,
                                       int* ovf) {
  const uint64_t mask = ballot(pass);
  if (!mask) return false;
  const int lane = lane_id();
  const int leader = __builtin_ctzll(mask);
  int base = 0;
  if (lane == leader) base = atomicAdd(cnt, __builtin_popcountll(mask));
  base = __shfl(base, leader, kWave);
  if (!pass) return false;
  const int slot = base + __builtin_popcountll(mask & ((1ull << lane) - 1ull));
  if (slot < cap) {
    buf[slot] = key;
    return true;
  }
  *ovf = 1;
  return false;
}

// Sort the first min(*cnt, cap) keys descending (zero padded to a power of two).
__device__ void sort_buffer(uint64_t* buf, int cap, int* cnt, int* n_out) {
  __syncthreads();
  const int n = min(*cnt, cap);
  const int np = next_pow2(max(n, 2));
  for (int t = n + threadIdx.x; t < np; t += blockDim.x) buf[t] = 0ull;
  __syncthreads();
  bitonic_desc(buf, np);
  *n_out = n;
}

template <int DT>
__global__ __launch_bounds__(kSB) void k_support_expand(const BArgs a) {
  const Cfg& c = a.c;
  const int b = blockIdx.y;
  const int j = blockIdx.x;
  const int layer = a.layer;
  const int tid = threadIdx.x;
  const int64_t ncb = (int64_t)b * c.NC;
  const int cbase = layer_base(c, layer) + j * c.K;
  const int ridx = row_base(c, layer) + j;

  // which node this block expands (root at layer 0)
  int node = -1;
  bool active = true;
  if (layer == 0) {
    // a new step: forget every candidate of the previous one, reset SMART's state
    for (int t = c.K + tid; t < c.NC; t += blockDim.x) a.t.cand_kind[ncb + t] = 0;
    if (tid == 0) {
      double* sm = a.t.smart + (int64_t)b * 8;
      sm[0] = 0.0; sm[1] = 1.0; sm[2] = 1.0; sm[3] = 0.0; sm[4] = 0.0;
      sm[5] = sm[6] = sm[7] = 0.0;
    }
  } else {
    const int nf = a.t.n_front[b];
    active = j < min(max(nf, 0), c.FP);
    if (active) {
      node = a.t.front[(int64_t)b * c.FP + j];
      const int pl = layer - 1;
      const int lo = layer_base(c, pl), hi = lo + layer_span(c, pl);
      active = node >= lo && node < hi && (a.t.cand_kind[ncb + node] & 0xFF) != 0;
    }
  }
  if (!active) {
    for (int s = tid; s < c.K; s += blockDim.x) a.t.cand_kind[ncb + cbase + s] = 0;
    if (tid == 0) a.t.row_tail_n[(int64_t)b * c.NR + ridx] = 0;
    return;
  }

  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  constexpr int EPL = 16 / esz;       // elements per 16-byte load
  constexpr int NE = kSU * EPL;       // elements per thread per pass
  const int V = c.V;
  const char* row = (const char*)a.logits + ((int64_t)b * a.tstride + (int64_t)j * a.ld) * esz;
  const int cap = 4096;
  const int TCp = max(128, next_pow2(c.trunc));

  extern __shared__ uint64_t s_buf[];           // [cap] candidate keys
  float* s_q = (float*)(s_buf + cap);           // [TCp] ranking probabilities
  __shared__ int s_cnt, s_ovf, s_bad;
  __shared__ uint64_t s_thr;
  if (tid == 0) {
    s_cnt = 0;
    s_ovf = 0;
    s_bad = 0;
    s_thr = 0ull;
  }
  __syncthreads();

  const int per_pass = kSB * NE;
  bool first = true;
  int bad = 0;
  for (int base = 0; base < V; base += per_pass) {
    float x[NE];
#pragma unroll
    for (int q = 0; q < kSU; ++q) {
      const int e0 = base + (q * kSB + tid) * EPL;
      if constexpr (DT == VRT_BF16) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e0 < V) v = *(const uint4*)((const uint16_t*)row + e0);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[q * 8 + 2 * k] = bf16_lo(w[k]);
          x[q * 8 + 2 * k + 1] = bf16_hi(w[k]);
        }
      } else {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e0 < V) v = *(const float4*)((const float*)row + e0);
        x[q * 4 + 0] = v.x;
        x[q * 4 + 1] = v.y;
        x[q * 4 + 2] = v.z;
        x[q * 4 + 3] = v.w;
      }
    }
    auto id_of = [&](int k) { return base + ((k / EPL) * kSB + tid) * EPL + (k % EPL); };
#pragma unroll
    for (int k = 0; k < NE; ++k)
      if (id_of(k) < V) bad |= __builtin_isnan(x[k]) || x[k] == INFINITY;

    if (first) {
      // seed the threshold: the trunc-th largest of the threads' maxima is a key
      // that at least trunc elements reach
      first = false;
      uint64_t mk = 0ull;
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int id = id_of(k);
        if (id < V && !__builtin_isnan(x[k])) {
          const uint64_t key = sup_key(x[k], (uint32_t)id);
          mk = key > mk ? key : mk;
        }
      }
      if (c.trunc <= kSB) {
        s_buf[tid] = mk;
        __syncthreads();
        bitonic_desc(s_buf, kSB);
        if (tid == 0) {
          const uint64_t t0 = s_buf[c.trunc - 1];
          s_thr = t0 ? t0 - 1ull : 0ull;
        }
        __syncthreads();
      }
    }

    uint32_t done = 0u;
    for (;;) {
      const uint64_t thr = s_thr;
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int id = id_of(k);
        const bool ok = id < V && !__builtin_isnan(x[k]) && !((done >> k) & 1u);
        const uint64_t key = ok ? sup_key(x[k], (uint32_t)id) : 0ull;
        if (append(ok && key > thr, key, s_buf, cap, &s_cnt, &s_ovf)) done |= 1u << k;
      }
      __syncthreads();
      const int ov = s_ovf;
      __syncthreads();
      if (!ov) break;
      // compaction: keep the best trunc keys, raise the threshold to the trunc-th
      int n;
      sort_buffer(s_buf, cap, &s_cnt, &n);
      if (tid == 0) {
        if (n >= c.trunc) s_thr = s_buf[c.trunc - 1];
        s_cnt = min(n, c.trunc);
        s_ovf = 0;
      }
      __syncthreads();
    }
  }
  if (bad) atomicOr(&s_bad, 1);
  int n;
  sort_buffer(s_buf, cap, &s_cnt, &n);  // final: sorted support in s_buf[0..n)
  const int n_sup = min(n, c.trunc);
  if (threadIdx.x >= kWave) return;

  // ---- expansion by wave 0
  const int lane = lane_id();
  const int64_t ktb = (int64_t)b * c.NR + ridx;
  uint32_t st = s_bad ? VRT_ST_DRAFT_NONFINITE : 0u;
  const float M = n_sup > 0 ? sup_key_val(s_buf[0]) : -INFINITY;
  if (n_sup == 0 || M == -INFINITY) st |= VRT_ST_DRAFT_EMPTY;
  if (st) {
    if (lane == 0 && a.stats) atomicOr(a.stats + (int64_t)b * 8, st);
    for (int s = lane; s < c.K; s += kWave) a.t.cand_kind[ncb + cbase + s] = 0;
    if (lane == 0) a.t.row_tail_n[ktb] = 0;
    return;
  }
  const int bs = TCp / kWave;  // ranks per lane: lane owns [lane*bs, lane*bs + bs)
  const int m = c.probe ? c.m : 0;
  float e[16], tmp[16];
  double et[16];
  for (int k = 0; k < bs; ++k) {
    const int r = lane * bs + k;
    const float v = r < n_sup ? sup_key_val(s_buf[r]) : -INFINITY;
    e[k] = r < n_sup ? exp_rank(v - M) : 0.0f;
    et[k] = r < n_sup ? exp(((double)v - (double)M) * (double)c.invT) : 0.0;
  }
  // aligned pairwise sums: inside the lane's block, then across lanes
  auto pairwise = [&](const float* in) -> float {
    for (int k = 0; k < bs; ++k) tmp[k] = in[k];
    for (int w = bs >> 1; w >= 1; w >>= 1)
      for (int k = 0; k < w; ++k) tmp[k] = tmp[2 * k] + tmp[2 * k + 1];
    return wave_sum(tmp[0]);
  };
  const float E = pairwise(e);
  float q[16], qt[16];
  for (int k = 0; k < bs; ++k) {
    const int r = lane * bs + k;
    q[k] = e[k] / E;
    qt[k] = r < m ? 0.0f : q[k];
    if (r < TCp) s_q[r] = q[k];
  }
  const float zr = pairwise(qt);
  double zl = 0.0;
  for (int k = 0; k < bs; ++k) zl += et[k];
  const double Z = wave_sum(zl);
  double tl = 0.0;
  for (int k = 0; k < bs; ++k) {
    et[k] = et[k] / Z;  // q_T
    if (lane * bs + k >= m) tl += et[k];
  }
  const double zT = wave_sum(tl);
  wave_sync();

  int js = -1;
  float proxy = 0.0f;
  if (c.probe && n_sup > m && zT > 0.0) {
    const double u =
        (double)uniform24(a.seed, (uint32_t)(node + 1), (uint32_t)b, a.step, kPurposeProbe);
    const double tgt = u * zT;
    const double incl = wave_incl_scan(tl);
    const double excl = incl - tl;
    const uint64_t hit = ballot(tl > 0.0 && tgt < incl);
    int pick = -1;
    if (hit) {
      const int src = __builtin_ctzll(hit);
      if (lane == src) {
        double cum = excl;
        for (int k = 0; k < bs; ++k) {
          const int r = lane * bs + k;
          if (r < m) continue;
          cum += et[k];
          if (tgt < cum) {
            pick = r;
            break;
          }
        }
      }
      pick = __shfl(pick, src, kWave);
    }
    if (pick < 0) {  // rounding exhausted the sum: the last tail rank with mass
      int last = -1;
      for (int k = 0; k < bs; ++k) {
        const int r = lane * bs + k;
        if (r >= m && r < n_sup && et[k] > 0.0) last = r;
      }
      for (int o = 1; o < kWave; o <<= 1) last = max(last, __shfl_xor(last, o, kWave));
      pick = last;
    }
    js = pick;
    if (m >= 1) {
      const float qm = s_q[m - 1];
      proxy = qm < zr ? qm : zr;
    } else {
      const float t1 = s_q[0] + c.eps_m0;
      proxy = t1 < 1.0f ? t1 : 1.0f;
    }
  }

  // tail table of this row: ranks m.. with q~ = q_T / z_T
  const int ntail = (js >= 0) ? n_sup - m : 0;
  if (lane == 0) a.t.row_tail_n[ktb] = ntail;
  for (int k = 0; k < bs; ++k) {
    const int r = lane * bs + k;
    if (r >= m && r < m + ntail) {
      a.t.row_tail_id[ktb * c.TC + (r - m)] = (int)sup_key_id(s_buf[r]);
      a.t.row_tail_q[ktb * c.TC + (r - m)] = (float)(et[k] / zT);
    }
  }

  // child slots (one lane): DET ranks, the probe, then fillers in rank order
  if (lane == 0) {
    const float sp = node < 0 ? 1.0f : a.t.cand_score[ncb + node];
    int slot = 0;
    auto put = [&](int r, int kind, float qv) {
      const int64_t ci = ncb + cbase + slot;
      a.t.cand_token[ci] = (int)sup_key_id(s_buf[r]);
      a.t.cand_parent[ci] = node;
      a.t.cand_score[ci] = sp * qv;
      a.t.cand_kind[ci] = kind;
      ++slot;
    };
    if (!c.probe) {
      for (int r = 0; r < n_sup && slot < c.K; ++r) put(r, VRT_DET, s_q[r]);
    } else {
      for (int r = 0; r < m && r < n_sup && slot < c.K; ++r) put(r, VRT_DET, s_q[r]);
      if (js >= 0 && slot < c.K) put(js, VRT_PROBE, proxy);
      for (int r = m; r < n_sup && slot < c.K; ++r)
        if (r != js) put(r, VRT_FILL, s_q[r]);
    }
    for (; slot < c.K; ++slot) a.t.cand_kind[ncb + cbase + slot] = 0;
  }
}

// Per-tree ranking of the layer's children: top-W frontier (top-R mode) or SMART.
__global__ __launch_bounds__(256) void k_rank_layer(const Cfg c, const TreePtrs t, int layer) {
  const int b = blockIdx.x;
  const int64_t ncb = (int64_t)b * c.NC;
  const int base = layer_base(c, layer);
  const int span = layer_span(c, layer);
  const int np = next_pow2(max(span, 2));
  extern __shared__ uint64_t s_keys[];
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    uint64_t k = 0ull;
    if (i < span && (t.cand_kind[ncb + base + i] & 0xFF) != 0)
      k = node_key(t.cand_score[ncb + base + i], (uint32_t)(base + i));
    s_keys[i] = k;
  }
  __syncthreads();
  bitonic_desc(s_keys, np);
  if (threadIdx.x != 0) return;
  const bool more = layer + 1 < c.D;
  int* front = t.front + (int64_t)b * c.FP;
  int nf = 0;
  if (c.mode == VRT_MODE_TOPR) {
    if (more)
      for (int i = 0; i < span && nf < c.W && s_keys[i] != 0ull; ++i)
        front[nf++] = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i]);
  } else {
    // SMART key design 3: keep u iff alpha * g * C(|T|) > L * C'(|T|), g = P(path)/|P|;
    // the first rejection ends the layer
    double* sm = t.smart + (int64_t)b * 8;
    double L = sm[0], n = sm[1], P = sm[2], nadm = sm[3], root_has = sm[4];
    int* adm = t.admitted + (int64_t)b * c.N;
    for (int i = 0; i < span && s_keys[i] != 0ull; ++i) {
      if (nadm >= (double)c.budget) break;
      const int cu = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i]);
      const double g = (double)t.cand_score[ncb + cu] / P;
      const double Cn = c.lam * n + c.gam * (exp(c.del * pow(n, c.rho)) - 1.0);
      const double dC = c.lam + c.gam * c.del * c.rho * pow(n, c.rho - 1.0) * exp(c.del * pow(n, c.rho));
      if (!(c.alpha * g * Cn > L * dC)) break;
      const int par = t.cand_parent[ncb + cu];
      const bool has = par < 0 ? root_has != 0.0 : (t.cand_kind[ncb + par] & 0x100) != 0;
      L += g;
      n += 1.0;
      if (has) P += 1.0;
      if (par < 0) root_has = 1.0;
      else t.cand_kind[ncb + par] |= 0x100;
      adm[(int)nadm] = cu;
      nadm += 1.0;
      if (more) front[nf++] = cu;
    }
    sm[0] = L; sm[1] = n; sm[2] = P; sm[3] = nadm; sm[4] = root_has;
  }
  t.n_front[b] = nf;
}

// Emit the tree: node 0 = root, then the kept candidates (parents first).
__global__ __launch_bounds__(256) void k_finish(const Cfg c, const TreePtrs t) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t ncb = (int64_t)b * c.NC;
  const int64_t nb = (int64_t)b * c.N;
  // dynamic LDS: top-R keys [np] (top-R mode), node -> candidate [N], child counts [N+1]
  extern __shared__ uint64_t s_keys[];
  const int np = c.mode == VRT_MODE_TOPR ? next_pow2(max(c.NC, 2)) : 0;
  int* s_ncand = (int*)(s_keys + np);
  int* s_cnt = s_ncand + c.N;
  __shared__ int s_n;

  if (c.mode == VRT_MODE_TOPR) {
    for (int i = tid; i < np; i += blockDim.x) {
      uint64_t k = 0ull;
      if (i < c.NC && (t.cand_kind[ncb + i] & 0xFF) != 0) k = node_key(t.cand_score[ncb + i], (uint32_t)i);
      s_keys[i] = k;
    }
    __syncthreads();
    bitonic_desc(s_keys, np);
    if (tid == 0) {
      int n = 1;
      while (n - 1 < c.R && n - 1 < np && s_keys[n - 1] != 0ull) ++n;
      s_n = n;
    }
    __syncthreads();
    for (int i = 1 + tid; i < s_n; i += blockDim.x)
      s_ncand[i] = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i - 1]);
  } else {
    if (tid == 0) {
      const int nadm = (int)t.smart[(int64_t)b * 8 + 3];
      s_n = 1 + min(max(nadm, 0), c.N - 1);
    }
    __syncthreads();
    for (int i = 1 + tid; i < s_n; i += blockDim.x) {
      int cu = t.admitted[nb + i - 1];
      s_ncand[i] = (cu < 0 || cu >= c.NC) ? 0 : cu;
    }
  }
  if (tid == 0) s_ncand[0] = -1;
  const int n = s_n;
  for (int i = tid; i <= n; i += blockDim.x) s_cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    t.tail_n[nb + i] = 0;
    if (i == 0) {
      t.node_token[nb] = -1;
      t.node_parent[nb] = -1;
      t.node_depth[nb] = 0;
      t.node_kind[nb] = VRT_ROOT;
      t.node_cand[nb] = -1;
      continue;
    }
    const int cu = s_ncand[i];
    const int pc = t.cand_parent[ncb + cu];
    int pn = 0;  // parents precede children, so the parent is among nodes 1..i-1
    if (pc >= 0)
      for (int j = i - 1; j >= 1; --j)
        if (s_ncand[j] == pc) {
          pn = j;
          break;
        }
    t.node_cand[nb + i] = cu;
    t.node_token[nb + i] = t.cand_token[ncb + cu];
    t.node_parent[nb + i] = pn;
    t.node_depth[nb + i] = layer_of(c, cu) + 1;
    t.node_kind[nb + i] = t.cand_kind[ncb + cu] & 0xFF;
    atomicAdd(&s_cnt[pn], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int i = 0; i < n; ++i) {
      const int k = s_cnt[i];
      s_cnt[i] = off;
      t.child_off[(int64_t)b * (c.N + 1) + i] = off;
      off += k;
    }
    t.child_off[(int64_t)b * (c.N + 1) + n] = off;
    t.n_nodes[b] = n;
  }
  __syncthreads();
  // child lists in slot order; the probe's tail goes to its parent
  for (int i = 1 + tid; i < n; i += blockDim.x) {
    const int pn = t.node_parent[nb + i];
    const int cu = s_ncand[i];
    const int slot = (cu - layer_base(c, layer_of(c, cu))) % c.K;
    int before = 0;
    for (int j = 1; j < n; ++j) {
      if (j == i || t.node_parent[nb + j] != pn) continue;
      const int cj = s_ncand[j];
      if ((cj - layer_base(c, layer_of(c, cj))) % c.K < slot) ++before;
    }
    t.child[nb + s_cnt[pn] + before] = i;
    if (t.node_kind[nb + i] == VRT_PROBE) {
      const int64_t rr = (int64_t)b * c.NR + row_of(c, cu);
      const int nt = min(max(t.row_tail_n[rr], 0), c.TC);
      for (int k = 0; k < nt; ++k) {
        t.tail_id[(nb + pn) * c.TC + k] = t.row_tail_id[rr * c.TC + k];
        t.tail_q[(nb + pn) * c.TC + k] = t.row_tail_q[rr * c.TC + k];
      }
      t.tail_n[nb + pn] = nt;
    }
  }
}

}  // namespace

hipError_t launch_build_layer(const Cfg& c, const TreePtrs& t, int layer, const void* logits,
                              int64_t ld, int64_t tstride, uint64_t seed, uint32_t step,
                              uint32_t* stats, void* ws, hipStream_t stream) {
  (void)ws;
  BArgs a{c, t, layer, logits, ld, tstride, seed, step, stats};
  const int cap = 4096;
  const size_t lds = (size_t)cap * 8 + (size_t)max(128, next_pow2(c.trunc)) * 4;
  const dim3 grid(layer == 0 ? 1 : c.FP, c.B);
  if (c.dtype == VRT_BF16)
    hipLaunchKernelGGL(k_support_expand<VRT_BF16>, grid, dim3(kSB), lds, stream, a);
  else
    hipLaunchKernelGGL(k_support_expand<VRT_F32>, grid, dim3(kSB), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int span = (layer == 0 ? 1 : c.P) * c.K;
  const size_t lds2 = (size_t)next_pow2(max(span, 2)) * 8;
  hipLaunchKernelGGL(k_rank_layer, dim3(c.B), dim3(256), lds2, stream, c, t, layer);
  return hipGetLastError();
}

hipError_t launch_build_finish(const Cfg& c, const TreePtrs& t, void* ws, hipStream_t stream) {
  (void)ws;
  const int np = c.mode == VRT_MODE_TOPR ? next_pow2(max(c.NC, 2)) : 0;
  const size_t lds = (size_t)np * 8 + (size_t)(2 * c.N + 1) * 4;
  hipLaunchKernelGGL(k_finish, dim3(c.B), dim3(256), lds, stream, c, t);
  return hipGetLastError();
}

}  // namespace vrt
