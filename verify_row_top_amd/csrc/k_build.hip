// Draft-tree construction on gfx950 (RheoSampling framework flowchart, key designs
// 1-2; SMART key design 3 as the switchable keep rule). Per layer, three kernels:
//
// k_seg_topk: one wave per 16 KB segment of an expanded parent's draft row streams
//   the segment once (non-temporal 16-byte loads, next batch in flight) and keeps the
//   segment's best keys (logit desc, token id asc) sorted in registers: one compare
//   per element against a threshold, exact keys only for survivors, bitonic sorts and
//   merges by cross-lane shuffles.
// k_merge_expand: one wave per parent merges its segments' lists into the row's
//   top-trunc support and expands the parent: untempered softmax on the support with
//   the fixed ranking recipe, tempered softmax in fp64, the probe draw from the
//   tempered tail, the proxy min{q(x_m), z}, the K child slots and the parent's tail
//   table.
// k_rank_layer: one block per tree ranks the layer's children by (path score desc,
//   creation index asc) and keeps the top W (top-R mode) or runs SMART's sequential
//   keep rule over them.
// k_finish: one block per tree emits the tree: the global top R by the same key
//   (or SMART's admitted nodes), parents before children, child lists in slot
//   order, and the probe tails the verifier needs.
#include "vrt_dev.hpp"
#include "vrt_internal.hpp"

namespace vrt {
namespace {

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
__device__ __forceinline__ int slot_of(const Cfg& c, int cidx) {
  return (cidx - layer_base(c, layer_of(c, cidx))) % c.K;
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
  int G;               // segments per row
  uint64_t* seg_keys;  // [B][FP][G][N] sorted top keys of each segment, N = 64 * PL
  int* seg_bad;        // [B][FP][G] a NaN or +inf logit was seen
};

// The node frontier position j of tree b expands at this layer (-1 = root), or -2
// if the position is empty (fewer parents) or holds an index the previous layer did
// not produce.
__device__ __forceinline__ int row_node(const BArgs& a, int b, int j) {
  const Cfg& c = a.c;
  if (a.layer == 0) return j == 0 ? -1 : -2;
  const int nf = a.t.n_front[b];
  if (j >= min(max(nf, 0), c.FP)) return -2;
  const int node = a.t.front[(int64_t)b * c.FP + j];
  const int lo = layer_base(c, a.layer - 1), hi = lo + layer_span(c, a.layer - 1);
  if (node < lo || node >= hi) return -2;
  if ((a.t.cand_kind[(int64_t)b * c.NC + node] & 0xFF) == 0) return -2;
  return node;
}

constexpr int kSegWaves = 4;  // waves (one segment each) per selection block
constexpr int kSegLoads = 16; // 16-byte loads per lane per segment, all in flight at once

template <int DT>
constexpr int seg_elems() { return kWave * kSegLoads * (DT == VRT_BF16 ? 8 : 4); }

// Segment top-N (N = 64*PL >= trunc): one wave per segment of an expanded parent's
// draft row. The wave issues all of its loads at once (the segment lives in 64
// registers per lane), then:
//  1. every lane finds the PL-th largest of its own values; the minimum of these over
//     the wave, v0, is reached by at least N elements of the segment, so nothing
//     below v0 can be among its N best;
//  2. elements at or above the current threshold value have their exact keys (logit
//     desc, token id asc) staged in wave-local LDS;
//  3. once N keys are staged they are sorted and merged into a sorted list of N keys
//     held in registers (bitonic networks over cross-lane shuffles), whose N-th key
//     becomes the exact threshold.
// No block barriers; the merge code is emitted once (the load loop resumes after it).
template <int DT, int PL>
__global__ __launch_bounds__(kSegWaves * kWave) void k_seg_topk(const BArgs a) {
  const Cfg& c = a.c;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int g = blockIdx.x * kSegWaves + wave;
  const int j = blockIdx.y, b = blockIdx.z;
  if (g >= a.G || row_node(a, b, j) == -2) return;
  constexpr int N = PL * kWave;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  constexpr int EPL = 16 / esz;         // elements per load
  constexpr int CAP = N + EPL * kWave;  // stage capacity: one load's worth past N
  const int V = c.V;
  const int seg0 = g * seg_elems<DT>();
  const char* row = (const char*)a.logits + ((int64_t)b * a.tstride + (int64_t)j * a.ld) * esz;
  __shared__ uint64_t s_stage[kSegWaves][CAP];
  uint64_t* stage = s_stage[wave];

  // load q of this lane covers elements [seg0 + (q*64 + lane)*EPL, +EPL); elements at
  // or past V read as -inf
  u32x4_t d[kSegLoads];
  static_for<kSegLoads>([&](auto q) {
    const int e0 = seg0 + (q * kWave + lane) * EPL;
    const uint32_t ninf = DT == VRT_BF16 ? 0xFF80FF80u : 0xFF800000u;
    u32x4_t v = {ninf, ninf, ninf, ninf};
    if (e0 < V) v = __builtin_nontemporal_load((const u32x4_t*)(row + (int64_t)e0 * esz));
    d[q] = v;
  });
  auto val = [&](const u32x4_t& v, int e) -> float {  // e: compile-time in every use
    if constexpr (DT == VRT_BF16) return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    else return __uint_as_float(v[e]);
  };
  if (seg0 + seg_elems<DT>() > V) {  // the row's last segment: mask a straddling load
    static_for<kSegLoads>([&](auto q) {
      const int e0 = seg0 + (q * kWave + lane) * EPL;
      if (e0 < V && e0 + EPL > V) {
        static_for<EPL>([&](auto e) {
          if (e0 + e >= V) {
            if constexpr (DT == VRT_BF16)
              d[q][e >> 1] = (e & 1) ? ((d[q][e >> 1] & 0xFFFFu) | 0xFF800000u)
                                     : ((d[q][e >> 1] & 0xFFFF0000u) | 0xFF80u);
            else
              d[q][(int)e] = 0xFF800000u;
          }
        });
      }
    });
  }

  // 1. non-finite scan and the lane's PL largest values
  bool bad = false;
  float lv[PL];
  static_for<PL>([&](auto s) { lv[s] = -INFINITY; });
  static_for<kSegLoads>([&](auto q) {
    static_for<EPL>([&](auto e) {
      float x = val(d[q], e);
      bad |= __builtin_amdgcn_classf(x, 0x203);  // NaN or +inf
      static_for<PL>([&](auto s) {
        const float hi = fmaxf(lv[s], x);
        x = fminf(lv[s], x);
        lv[s] = hi;
      });
    });
  });
  const bool any_bad = ballot(bad) != 0ull;
  float v0 = lv[PL - 1];
  for (int o = 1; o < kWave; o <<= 1) v0 = fminf(v0, __shfl_xor(v0, o, kWave));

  uint64_t top[PL];
  static_for<PL>([&](auto s) { top[s] = 0ull; });
  uint64_t thr = 0ull;  // N-th key of the list once it is full
  float thr_f = v0;
  int nst = 0;          // staged keys (wave-uniform)
  int q_next = 0;       // first load not yet scanned (wave-uniform)
  for (;;) {
    // the data is opaque to the optimiser here, so that unpacked values are not kept
    // live across the phases (they are recomputed: one ALU op each)
#pragma unroll
    for (int q = 0; q < kSegLoads; ++q) asm volatile("" : "+v"(d[q]));
    // 2. scan loads q_next.. until the stage holds N keys
    static_for<kSegLoads>([&](auto q) {
      if (q >= q_next && nst < N) {
        uint32_t cm = 0;
        static_for<EPL>([&](auto e) { cm |= (val(d[q], e) >= thr_f ? 1u : 0u) << e; });
        while (ballot(cm != 0u)) {
          const bool has = cm != 0u;
          const int e = has ? __builtin_ctz(cm) : 0;
          const uint32_t w = d[q][DT == VRT_BF16 ? (e >> 1) : e];
          const float x = DT == VRT_BF16 ? ((e & 1) ? bf16_hi(w) : bf16_lo(w)) : __uint_as_float(w);
          const int id = seg0 + (q * kWave + lane) * EPL + e;
          const uint64_t key = sup_key(x, (uint32_t)id);
          const bool pass = has && id < V && key > thr;
          const uint64_t mask = ballot(pass);
          if (pass) stage[nst + __builtin_popcountll(mask & ((1ull << lane) - 1ull))] = key;
          nst += __builtin_popcountll(mask);
          if (has) cm &= cm - 1u;
        }
        q_next = q + 1;
      }
    });
    const bool last = q_next >= kSegLoads;
    // 3. merge full stages (all of it after the last load) into the list
    int off = 0;
    while (nst - off >= N || (last && nst > off)) {
      const int cnt = min(N, nst - off);
      wave_sync();
      uint64_t add[PL];
      static_for<PL>([&](auto s) {
        const int p = lane * PL + s;
        add[s] = p < cnt ? stage[off + p] : 0ull;
      });
      wave_sort_desc<PL>(add);
      wave_merge_top<PL>(top, add);
      off += cnt;
      const uint64_t t = shfl64(top[PL - 1], kWave - 1);
      if (t) {
        thr = t;
        thr_f = sup_key_val(t);
      }
    }
    if (last) break;
    // the rest (fewer than N keys, at positions >= N) moves to the front
    const int rem = nst - off;
    wave_sync();
    for (int i = lane; i < rem; i += kWave) stage[i] = stage[off + i];
    nst = rem;
  }
  // the segment's list, positions >= trunc cleared
  const int64_t sg = ((int64_t)b * c.FP + j) * a.G + g;
  static_for<PL>([&](auto s) {
    const int p = lane * PL + s;
    a.seg_keys[sg * N + p] = p < c.TC ? top[s] : 0ull;
  });
  if (lane == 0) a.seg_bad[sg] = any_bad ? 1 : 0;
}

// Expansion of one parent by wave 0 (RheoSampling key design 2), BS support ranks
// per lane: lane l owns ranks [l*BS, l*BS + BS).
template <int BS>
__device__ void expand_row(const BArgs& a, int b, int node, int n_sup, const uint64_t* s_buf,
                           float* s_q, int64_t ncb, int cbase, int64_t ktb) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const float M = sup_key_val(s_buf[0]);
  const int m = c.probe ? c.m : 0;
  float e[BS];
  double et[BS];
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    const int r = lane * BS + k;
    const float v = r < n_sup ? sup_key_val(s_buf[r]) : -INFINITY;
    e[k] = r < n_sup ? exp_rank(v - M) : 0.0f;
    et[k] = r < n_sup ? exp(((double)v - (double)M) * (double)c.invT) : 0.0;
  }
  // aligned pairwise sums: inside the lane's block, then across lanes
  auto pairwise = [&](const float (&in)[BS]) -> float {
    float t[BS];
#pragma unroll
    for (int k = 0; k < BS; ++k) t[k] = in[k];
#pragma unroll
    for (int w = BS >> 1; w >= 1; w >>= 1)
#pragma unroll
      for (int k = 0; k < w; ++k) t[k] = t[2 * k] + t[2 * k + 1];
    return wave_sum(t[0]);
  };
  const float E = pairwise(e);
  float qt[BS];
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    const int r = lane * BS + k;
    const float q = e[k] / E;
    qt[k] = r < m ? 0.0f : q;
    s_q[r] = q;
  }
  const float zr = pairwise(qt);
  double zl = 0.0;
#pragma unroll
  for (int k = 0; k < BS; ++k) zl += et[k];
  const double Z = wave_sum(zl);
  double tl = 0.0;
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    et[k] = et[k] / Z;  // q_T
    if (lane * BS + k >= m) tl += et[k];
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
#pragma unroll
        for (int k = 0; k < BS; ++k) {
          const int r = lane * BS + k;
          if (r >= m && pick < 0) {
            cum += et[k];
            if (tgt < cum) pick = r;
          }
        }
      }
      pick = __shfl(pick, src, kWave);
    }
    if (pick < 0) {  // rounding exhausted the sum: the last tail rank with mass
      int last = -1;
#pragma unroll
      for (int k = 0; k < BS; ++k) {
        const int r = lane * BS + k;
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
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    const int r = lane * BS + k;
    if (r >= m && r < m + ntail) {
      a.t.row_tail_id[ktb * c.TC + (r - m)] = (int)sup_key_id(s_buf[r]);
      a.t.row_tail_q[ktb * c.TC + (r - m)] = (float)(et[k] / zT);
    }
  }

  // child slots: DET ranks, the probe, then fillers in rank order. Lane s writes slot s.
  const float sp = node < 0 ? 1.0f : a.t.cand_score[ncb + node];
  int r_of_slot = -1, kind = 0;
  {
    const int m_det = c.probe ? min(m, n_sup) : 0;
    const int s = lane;
    if (!c.probe) {
      if (s < n_sup) r_of_slot = s, kind = VRT_DET;
    } else if (s < m_det) {
      r_of_slot = s, kind = VRT_DET;
    } else if (js >= 0 && s == m_det) {
      r_of_slot = js, kind = VRT_PROBE;
    } else {
      const int f = s - m_det - (js >= 0 ? 1 : 0);  // filler index
      int r = m + f;
      if (js >= 0 && r >= js) ++r;
      if (r < n_sup) r_of_slot = r, kind = VRT_FILL;
    }
  }
  if (lane < c.K) {
    const int64_t ci = ncb + cbase + lane;
    if (r_of_slot >= 0) {
      a.t.cand_token[ci] = (int)sup_key_id(s_buf[r_of_slot]);
      a.t.cand_parent[ci] = node;
      a.t.cand_score[ci] = sp * (kind == VRT_PROBE ? proxy : s_q[r_of_slot]);
      a.t.cand_kind[ci] = kind;
    } else {
      a.t.cand_kind[ci] = 0;
    }
  }
}

// One wave per parent: merge its segments' sorted lists (the row's top trunc is in
// the union of the segments' top trunc), then expand the parent.
template <int PL>
__global__ __launch_bounds__(kWave) void k_merge_expand(const BArgs a) {
  const Cfg& c = a.c;
  const int j = blockIdx.x, b = blockIdx.y;
  const int lane = lane_id();
  constexpr int N = PL * kWave;
  const int64_t ncb = (int64_t)b * c.NC;
  const int cbase = layer_base(c, a.layer) + j * c.K;
  const int ridx = row_base(c, a.layer) + j;
  const int64_t ktb = (int64_t)b * c.NR + ridx;

  if (a.layer == 0) {
    // a new step: forget every candidate of the previous one, reset SMART's state
    for (int t = c.K + lane; t < c.NC; t += kWave) a.t.cand_kind[ncb + t] = 0;
    if (lane == 0) {
      double* sm = a.t.smart + (int64_t)b * 8;
      sm[0] = 0.0; sm[1] = 1.0; sm[2] = 1.0; sm[3] = 0.0; sm[4] = 0.0;
      sm[5] = sm[6] = sm[7] = 0.0;
    }
  }
  const int node = row_node(a, b, j);
  if (node == -2) {
    for (int s = lane; s < c.K; s += kWave) a.t.cand_kind[ncb + cbase + s] = 0;
    if (lane == 0) a.t.row_tail_n[ktb] = 0;
    return;
  }

  __shared__ uint64_t s_buf[N];
  __shared__ float s_q[N];
  const int64_t sg0 = ((int64_t)b * c.FP + j) * a.G;
  auto load_list = [&](int g, uint64_t (&l)[PL]) {
    const uint64_t* src = a.seg_keys + (sg0 + g) * N + lane * PL;
    static_for<PL>([&](auto s) { l[s] = src[s]; });
  };
  uint64_t top[PL], nxt[PL];
  load_list(0, top);
  if (a.G > 1) load_list(1, nxt);
  for (int g = 1; g < a.G; ++g) {
    uint64_t cur[PL];
    static_for<PL>([&](auto s) { cur[s] = nxt[s]; });
    if (g + 1 < a.G) load_list(g + 1, nxt);
    wave_merge_top<PL>(top, cur);
  }
  int bad = 0;
  for (int g = lane; g < a.G; g += kWave) bad |= a.seg_bad[sg0 + g];
  // support: the non-empty keys among the first trunc positions
  int cnt = 0;
  static_for<PL>([&](auto s) {
    const int p = lane * PL + s;
    const uint64_t k = p < c.TC ? top[s] : 0ull;
    s_buf[p] = k;
    cnt += k != 0ull;
  });
  const int n_sup = wave_sum_i(cnt);
  wave_sync();

  uint32_t st = ballot(bad != 0) ? VRT_ST_DRAFT_NONFINITE : 0u;
  const float M = n_sup > 0 ? sup_key_val(s_buf[0]) : -INFINITY;
  if (n_sup == 0 || M == -INFINITY) st |= VRT_ST_DRAFT_EMPTY;
  if (st) {
    if (lane == 0 && a.stats) atomicOr(a.stats + (int64_t)b * 8, st);
    for (int s = lane; s < c.K; s += kWave) a.t.cand_kind[ncb + cbase + s] = 0;
    if (lane == 0) a.t.row_tail_n[ktb] = 0;
    return;
  }
  expand_row<PL>(a, b, node, n_sup, s_buf, s_q, ncb, cbase, ktb);
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

constexpr int kFT = 1024;  // threads of the finish block

// Emit the tree: node 0 = root, then the kept candidates (parents first).
__global__ __launch_bounds__(kFT) void k_finish(const Cfg c, const TreePtrs t) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t ncb = (int64_t)b * c.NC;
  const int64_t nb = (int64_t)b * c.N;
  // dynamic LDS: top-R keys [np] (top-R mode), then per node: candidate, parent node,
  // slot, expansion row holding its tail, tail length, child counts [N+1]
  extern __shared__ uint64_t s_keys[];
  const int np = c.mode == VRT_MODE_TOPR ? next_pow2(max(c.NC, 2)) : 0;
  int* s_ncand = (int*)(s_keys + np);
  int* s_par = s_ncand + c.N;
  int* s_slot = s_par + c.N;
  int* s_trow = s_slot + c.N;
  int* s_tn = s_trow + c.N;
  int* s_cnt = s_tn + c.N;
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
      const int cu = t.admitted[nb + i - 1];
      s_ncand[i] = (cu < 0 || cu >= c.NC) ? 0 : cu;
    }
  }
  const int n = s_n;
  if (tid == 0) s_ncand[0] = -1;
  for (int i = tid; i <= n; i += blockDim.x) s_cnt[i] = 0;
  for (int i = tid; i < n; i += blockDim.x) {
    s_trow[i] = -1;
    s_tn[i] = 0;
  }
  __syncthreads();
  // nodes: parent node (parents precede children, so it is among nodes 1..i-1)
  for (int i = 1 + tid; i < n; i += blockDim.x) {
    const int cu = s_ncand[i];
    const int pc = t.cand_parent[ncb + cu];
    int pn = 0;
    if (pc >= 0)
      for (int jj = i - 1; jj >= 1; --jj)
        if (s_ncand[jj] == pc) {
          pn = jj;
          break;
        }
    s_par[i] = pn;
    s_slot[i] = slot_of(c, cu);
    const int kind = t.cand_kind[ncb + cu] & 0xFF;
    if (kind == VRT_PROBE) {
      const int r = row_of(c, cu);
      s_trow[pn] = r;
      s_tn[pn] = min(max(t.row_tail_n[(int64_t)b * c.NR + r], 0), c.TC);
    }
    t.node_cand[nb + i] = cu;
    t.node_token[nb + i] = t.cand_token[ncb + cu];
    t.node_parent[nb + i] = pn;
    t.node_depth[nb + i] = layer_of(c, cu) + 1;
    t.node_kind[nb + i] = kind;
    atomicAdd(&s_cnt[pn], 1);
  }
  if (tid == 0) {
    t.node_token[nb] = -1;
    t.node_parent[nb] = -1;
    t.node_depth[nb] = 0;
    t.node_kind[nb] = VRT_ROOT;
    t.node_cand[nb] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    const int64_t cob = (int64_t)b * (c.N + 1);
    for (int i = 0; i < n; ++i) {
      const int k = s_cnt[i];
      s_cnt[i] = off;
      t.child_off[cob + i] = off;
      off += k;
    }
    t.child_off[cob + n] = off;
    t.n_nodes[b] = n;
  }
  __syncthreads();
  // child lists in slot order
  for (int i = 1 + tid; i < n; i += blockDim.x) {
    const int pn = s_par[i], slot = s_slot[i];
    int before = 0;
    for (int jj = 1; jj < n; ++jj) before += (s_par[jj] == pn && s_slot[jj] < slot);
    t.child[nb + s_cnt[pn] + before] = i;
  }
  // probe tails, copied to the probe's parent
  for (int i = tid; i < n; i += blockDim.x) t.tail_n[nb + i] = s_tn[i];
  for (int64_t x = tid; x < (int64_t)n * c.TC; x += blockDim.x) {
    const int i = (int)(x / c.TC), k = (int)(x % c.TC);
    if (k >= s_tn[i]) continue;
    const int64_t rr = (int64_t)b * c.NR + s_trow[i];
    t.tail_id[(nb + i) * c.TC + k] = t.row_tail_id[rr * c.TC + k];
    t.tail_q[(nb + i) * c.TC + k] = t.row_tail_q[rr * c.TC + k];
  }
}

template <int DT>
int segments(int V) {
  return (V + seg_elems<DT>() - 1) / seg_elems<DT>();
}

int list_len(const Cfg& c) { return max(128, next_pow2(c.trunc)); }

template <int DT>
hipError_t launch_layer(const BArgs& a, int rows, hipStream_t stream) {
  const Cfg& c = a.c;
  const dim3 g1((a.G + kSegWaves - 1) / kSegWaves, rows, c.B);
  const dim3 g2(rows, c.B);
  const dim3 t1(kSegWaves * kWave), t2(kWave);
  switch (list_len(c) / kWave) {
    case 2:
      hipLaunchKernelGGL((k_seg_topk<DT, 2>), g1, t1, 0, stream, a);
      hipLaunchKernelGGL(k_merge_expand<2>, g2, t2, 0, stream, a);
      break;
    case 4:
      hipLaunchKernelGGL((k_seg_topk<DT, 4>), g1, t1, 0, stream, a);
      hipLaunchKernelGGL(k_merge_expand<4>, g2, t2, 0, stream, a);
      break;
    case 8:
      hipLaunchKernelGGL((k_seg_topk<DT, 8>), g1, t1, 0, stream, a);
      hipLaunchKernelGGL(k_merge_expand<8>, g2, t2, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((k_seg_topk<DT, 16>), g1, t1, 0, stream, a);
      hipLaunchKernelGGL(k_merge_expand<16>, g2, t2, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

int segments_of(const Cfg& c) {
  return c.dtype == VRT_BF16 ? segments<VRT_BF16>(c.V) : segments<VRT_F32>(c.V);
}

}  // namespace

size_t build_ws_bytes(const Cfg& c) {
  const size_t lists = (size_t)c.B * c.FP * segments_of(c);
  return lists * list_len(c) * sizeof(uint64_t) + ((lists * sizeof(int) + 255) & ~(size_t)255);
}

hipError_t launch_build_layer(const Cfg& c, const TreePtrs& t, int layer, const void* logits,
                              int64_t ld, int64_t tstride, uint64_t seed, uint32_t step,
                              uint32_t* stats, void* ws, hipStream_t stream) {
  const int G = segments_of(c);
  const size_t lists = (size_t)c.B * c.FP * G;
  uint64_t* seg_keys = (uint64_t*)ws;
  int* seg_bad = (int*)((char*)ws + lists * list_len(c) * sizeof(uint64_t));
  BArgs a{c, t, layer, logits, ld, tstride, seed, step, stats, G, seg_keys, seg_bad};
  const int rows = layer == 0 ? 1 : c.FP;
  hipError_t e = c.dtype == VRT_BF16 ? launch_layer<VRT_BF16>(a, rows, stream)
                                     : launch_layer<VRT_F32>(a, rows, stream);
  if (e != hipSuccess) return e;
  const int span = (layer == 0 ? 1 : c.P) * c.K;
  const size_t lds2 = (size_t)next_pow2(max(span, 2)) * 8;
  hipLaunchKernelGGL(k_rank_layer, dim3(c.B), dim3(256), lds2, stream, c, t, layer);
  return hipGetLastError();
}

hipError_t launch_build_finish(const Cfg& c, const TreePtrs& t, void* ws, hipStream_t stream) {
  (void)ws;
  const int np = c.mode == VRT_MODE_TOPR ? next_pow2(max(c.NC, 2)) : 0;
  const size_t lds = (size_t)np * 8 + (size_t)(6 * c.N + 1) * 4;
  hipLaunchKernelGGL(k_finish, dim3(c.B), dim3(kFT), lds, stream, c, t);
  return hipGetLastError();
}

}  // namespace vrt
