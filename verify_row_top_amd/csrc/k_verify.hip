// Tree verification (RheoSampling, key design 3) on gfx950: one launch per call (the
// node pass with the walk fused into its last block of each tree), or the two parts
// apart, or the lazy walk.
//
// k_vnode: one 512-thread block per (node row, tree).
//   - The eight waves stream the node's target row from HBM once, in 2048-element
//     chunks taken two at a time (four 16-byte loads per lane per chunk, 8 bf16 each),
//     keeping per chunk fl(max*c2) and the sum of exp2(x*c2 - fl(max*c2)) in LDS,
//     where c2 = log2(e)/T. Every element costs one conversion, a third of a max3,
//     one fma, one native exp2 and one add.
//   - Meanwhile the last wave gathers what the decision needs besides the row
//     statistics: the kept children (node, token, logit) and the probe tail (token,
//     q~, logit). Those dependent loads overlap the other waves' stream.
//   - Wave 0 then forms p = softmax(x/T) where needed and decides the node exactly as
//     the walk would if it reached it: the probe-first test min(1, p/q~), recursive
//     rejection of the other kept children under w = max(0, p - q~) on the probe's
//     tail (p elsewhere), and, when nothing is accepted, the final residual (or bonus)
//     sample by inverse CDF in token-id order (adjusted chunk masses locate the chunk,
//     one 2048-element re-read finds the token). Every draw is keyed by (depth, test
//     index), so each node's decision is a pure function of its own row; other blocks'
//     streams hide its latency.
//   With the walk fused (vrt_verify_tree), each block writes its decision device-
//   coherently and counts itself on its tree's word in the workspace; the block that
//   counts the tree's last node follows the accepted children from the root.
// k_vwalk: one wave per tree follows the accepted children from the root and writes
//   the emitted tokens and statistics (the walk as a launch of its own).
// k_vlazy: one block per tree decides the root, then the accepted child, ... each node
//   by k_vnode's pass, so only the rows on the walk are read.
#include <atomic>
#include <random>

#include "vrt_dev.hpp"
#include "vrt_internal.hpp"

namespace vrt {
namespace {

constexpr int kVB = 512;        // threads per streaming block
constexpr int kCH = 2048;       // elements per chunk (one wave at a time)
constexpr int kChildMax = 32;   // K <= 30
constexpr float kBand = 1e-6f;  // near-tie band reported in the stats
constexpr double kFix = 1152921504606846976.0;  // 2^60: fixed point of the mass changes
// Per-tree counters of the fused walk, one 4 KB line apart: the device-coherent atomics
// on one line are executed one after another, so the trees' counters must not share one.
constexpr int kSyncStride = 512;  // u64 words

// What the decision of one node needs besides its row statistics (gathered by the
// streaming kernel): kept children in slot order and their logits.
struct VRec {
  int nc;     // kept children (validated)
  int probe;  // slot of the probe child, -1 if none
  int nt;     // probe tail entries (0 without a probe)
  int depth;  // depth of the node (0 = root)
  float u0, uf;  // draws of the probe test and of the final sample
  int node[kChildMax];
  int tok[kChildMax];
  float x[kChildMax];
  float u[kChildMax];  // draw of each non-probe kept child's test
  NodeOut res;         // the decision, also written here for the block (lazy walk)
  // dense rows (the probe's tail regenerated from the expansion's draft row)
  const char* drow;    // that draft row, NULL if the probe child is not kept
  double dzt;          // its tempered tail mass
  float dmax;          // its largest logit
  int nd;              // deterministic children: the tokens off the tail
  int det[kChildMax];
  float mc;            // pass 2's p: fl(max*c2) and 1/S of the target row,
  double invs, qscale; // and the scale of q~ (probe last: the residual mass W_D)
};

struct VArgs {
  Cfg c;
  TreePtrs t;
  const void* logits;
  int64_t ld, tstride;
  uint64_t seed;
  uint32_t step;
  NodeOut* node_out;
  int32_t* out_tokens;
  int32_t* out_nodes;
  int32_t* out_len;
  uint32_t* stats;
  const void* draft[32];  // dense rows: layer l's draft rows (as passed to the build)
  int64_t dld, dstride;
  uint64_t* vsync;  // fused walk: per tree (kSyncStride words apart), tag << 32 | status << 24 | done
  uint32_t tag;     // fused walk: this launch's tag (never 0)
};

// A node's decision into node_out, device-coherently (the fused walk reads it from
// another block), and into the block's record.
__device__ __forceinline__ void put_out(const VArgs& a, int64_t at, const NodeOut& out, VRec& R) {
  int* o = (int*)&a.node_out[at];
  st_dev(o, out.accept);
  st_dev(o + 1, out.token);
  st_dev(o + 2, out.flags);
  st_dev((float*)(o + 3), out.W);
  R.res = out;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clamp_nodes(int nn, int N) { return nn < 1 ? 1 : (nn > N ? N : nn); }

// One chunk of a lane in flight: NL 16-byte loads, load q covering elements
// lo + q*64*EPL + lane*EPL .. +EPL (bf16: 4 loads of 8, fp32: 8 loads of 4).
template <int DT>
struct ChunkRegs {
  static constexpr int NL = DT == VRT_BF16 ? 4 : 8;
  static constexpr int EPL = DT == VRT_BF16 ? 8 : 4;
  u32x4_t w[NL];
};

template <int DT>
__device__ __forceinline__ void issue_chunk(const char* row, int lo, int V, ChunkRegs<DT>& r) {
  using CR = ChunkRegs<DT>;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  const int lane = lane_id();
  static_for<CR::NL>([&](auto q) {
    const int e0 = lo + (q * kWave + lane) * CR::EPL;
    const uint32_t ninf = DT == VRT_BF16 ? 0xFF80FF80u : 0xFF800000u;
    u32x4_t v = {ninf, ninf, ninf, ninf};
    if (e0 < V) v = __builtin_nontemporal_load((const u32x4_t*)(row + (int64_t)e0 * esz));
    r.w[q] = v;
  });
}

// (fl(max*c2), sum exp2(x*c2 - fl(max*c2))) of two chunks at once (their reductions
// interleave, so no lane-exchange step waits on the one before it); `ragged` masks
// elements >= V.
template <int DT>
__device__ __forceinline__ void chunk_stats2(const ChunkRegs<DT>& ra, const ChunkRegs<DT>& rb, int loa,
                                             int lob, int V, float c2, bool rga, bool rgb, float2& oa,
                                             float2& ob) {
  using CR = ChunkRegs<DT>;
  const int lane = lane_id();
  float xa[32], xb[32];
  auto unpack = [&](const ChunkRegs<DT>& r, float (&x)[32], int lo, bool ragged) {
    static_for<CR::NL>([&](auto q) {
      static_for<4>([&](auto k) {
        if constexpr (DT == VRT_BF16) {
          x[q * 8 + 2 * k] = bf16_lo(r.w[q][(int)k]);
          x[q * 8 + 2 * k + 1] = bf16_hi(r.w[q][(int)k]);
        } else {
          x[q * 4 + k] = __uint_as_float(r.w[q][(int)k]);
        }
      });
    });
    if (ragged) {
      static_for<CR::NL>([&](auto q) {
        static_for<CR::EPL>([&](auto k) {
          if (lo + (q * kWave + lane) * CR::EPL + k >= V) x[q * CR::EPL + k] = -INFINITY;
        });
      });
    }
  };
  unpack(ra, xa, loa, rga);
  unpack(rb, xb, lob, rgb);
  float ma = xa[0], mb = xb[0];
#pragma unroll
  for (int k = 1; k < 32; ++k) {
    ma = fmaxf(ma, xa[k]);
    mb = fmaxf(mb, xb[k]);
  }
  auto mx = [](float x, float y) { return fmaxf(x, y); };
  ma = mx(ma, xchg<1>(ma)); mb = mx(mb, xchg<1>(mb));
  ma = mx(ma, xchg<2>(ma)); mb = mx(mb, xchg<2>(mb));
  ma = mx(ma, xchg<4>(ma)); mb = mx(mb, xchg<4>(mb));
  ma = mx(ma, xchg<8>(ma)); mb = mx(mb, xchg<8>(mb));
  ma = mx(ma, xchg<16>(ma)); mb = mx(mb, xchg<16>(mb));
  ma = mx(ma, xchg<32>(ma)); mb = mx(mb, xchg<32>(mb));
  const float mca = ma * c2, mcb = mb * c2;
  float sa = 0.0f, sb = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    sa += fast_exp2(__builtin_fmaf(xa[k], c2, -mca));
    sb += fast_exp2(__builtin_fmaf(xb[k], c2, -mcb));
  }
  // a chunk whose maximum is -inf (all masked) summed exp2(-inf + inf): it holds 0
  sa = ma > -INFINITY ? sa : 0.0f;
  sb = mb > -INFINITY ? sb : 0.0f;
  sa = sa + xchg<1>(sa); sb = sb + xchg<1>(sb);
  sa = sa + xchg<2>(sa); sb = sb + xchg<2>(sb);
  sa = sa + xchg<4>(sa); sb = sb + xchg<4>(sb);
  sa = sa + xchg<8>(sa); sb = sb + xchg<8>(sb);
  sa = sa + xchg<16>(sa); sb = sb + xchg<16>(sb);
  sa = sa + xchg<32>(sa); sb = sb + xchg<32>(sb);
  oa = make_float2(mca, sa);
  ob = make_float2(mcb, sb);
}

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int v) {
  if constexpr (DT == VRT_BF16) return __uint_as_float((uint32_t)((const uint16_t*)row)[v] << 16);
  else return ((const float*)row)[v];
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Per-wave LDS of the decision: chunk masses and their fixed-point changes [nch], the
// probe tail (token, q~, p, child slot) [TC], children's q~ [32], the changes inside
// the sampled chunk [TC + 32].
struct DLds {
  double* pm;
  long long* dfix;
  int* tid;
  float* tq;
  double* tp;
  int* tslot;
  double* qc;
  int* itok;
  double* idel;
  float* w;    // [64][33] weights of the sampled chunk
  double* ov;  // dense rows: per chunk, sum over the tail of min(p, s q~) [nch]
};

__host__ __device__ size_t decide_lds_bytes(const Cfg& c) {
  const size_t nch = (size_t)(c.V + kCH - 1) / kCH;
  const size_t TC = (size_t)c.TC;
  const size_t bytes = nch * 16 + TC * (4 + 4 + 8 + 4) + kChildMax * 8 + (TC + kChildMax) * (4 + 8) +
                       kWave * 33 * 4 + 72 + (c.trunc == VRT_DENSE ? nch * 8 + 8 : 0);
  return (bytes + 15) & ~(size_t)15;
}

__device__ DLds carve(char* base, int nch, int TC) {
  DLds L;
  char* p = base;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += (bytes + 7) & ~(size_t)7;
    return r;
  };
  L.pm = (double*)take((size_t)nch * 8);
  L.dfix = (long long*)take((size_t)nch * 8);
  L.tp = (double*)take((size_t)TC * 8);
  L.qc = (double*)take(kChildMax * 8);
  L.idel = (double*)take((size_t)(TC + kChildMax) * 8);
  L.tid = (int*)take((size_t)TC * 4);
  L.tq = (float*)take((size_t)TC * 4);
  L.tslot = (int*)take((size_t)TC * 4);
  L.itok = (int*)take((size_t)(TC + kChildMax) * 4);
  L.w = (float*)take((size_t)kWave * 33 * 4);
  L.ov = (double*)take((size_t)nch * 8);  // dense rows only (not reserved otherwise)
  return L;
}

// The decision inputs of node i other than its row statistics, gathered into the
// block's LDS by one wave: kept children (node, token, logit) in slot order and the
// probe tail (token, q~, logit).
template <int DT, bool DENSE>
__device__ void gather_node(const VArgs& a, int b, int i, int nn, const char* row, VRec& r,
                            const DLds& L) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const int64_t nb = (int64_t)b * c.N;
  const int64_t cob = (int64_t)b * (c.N + 1);  // child_off rows hold N + 1 entries
  const int co = a.t.child_off[cob + i], ce = a.t.child_off[cob + i + 1];
  int nc = ce - co;
  if (co < 0 || co > c.N || nc < 0) nc = 0;
  if (nc > c.K) nc = c.K;
  if (co + nc > c.N) nc = c.N - co > 0 ? c.N - co : 0;
  int node = -1, tok = -1;
  bool probe = false;
  if (lane < nc) {
    node = a.t.child[nb + co + lane];
    if (node > i && node < nn) {
      tok = a.t.node_token[nb + node];
      probe = a.t.node_kind[nb + node] == VRT_PROBE;
    }
    if (tok < 0 || tok >= c.V) node = -1, tok = -1, probe = false;
  }
  const uint64_t pm = ballot(probe);
  const int pl = pm ? __builtin_ctzll(pm) : -1;
  const float x = tok >= 0 ? load_one<DT>(row, tok) : -INFINITY;
  const int nt = pl >= 0 ? min(max(a.t.tail_n[nb + i], 0), c.TC) : 0;
  const int64_t tb = (nb + i) * c.TC;
  if (lane < kChildMax) L.qc[lane] = -1.0;
  wave_sync();
  for (int e = lane; e < nt; e += kWave) {
    int y = a.t.tail_id[tb + e];
    if (y < 0 || y >= c.V) y = -1;
    const float q = a.t.tail_q[tb + e];
    L.tid[e] = y;
    L.tq[e] = q;
    L.tp[e] = y >= 0 ? (double)load_one<DT>(row, y) : -INFINITY;  // the logit for now
    // which kept child (slot) has this token; that child's q~
    int slot = -1;
    for (int k = 0; k < nc; ++k)
      if (slot < 0 && y >= 0 && __builtin_amdgcn_readlane(tok, k) == y) slot = k;
    L.tslot[e] = slot;
    if (slot >= 0) L.qc[slot] = q;
  }
  if constexpr (DENSE) {
    // the probe's tail is its expansion row but the deterministic children: q~ of the
    // kept children in it, from that draft row
    const char* drow = nullptr;
    double dzt = 0.0;
    float dmax = 0.0f;
    int nd = 0;
    const int rr = pl >= 0 ? a.t.node_row[nb + i] : -1;
    if (rr >= 0 && rr < c.NR) {
      const int l = rr == 0 ? 0 : 1 + (rr - 1) / c.P;
      const int jr = rr == 0 ? 0 : rr - 1 - (l - 1) * c.P;
      const int64_t rb = (int64_t)b * c.NR + rr;
      dzt = a.t.row_dense[rb * 2 + 1];
      dmax = (float)a.t.row_dense[rb * 2];
      if (l < c.D && a.draft[l] && dzt > 0.0) {
        constexpr int esz = DT == VRT_BF16 ? 2 : 4;
        drow = (const char*)a.draft[l] + ((int64_t)b * a.dstride + (int64_t)jr * a.dld) * esz;
        nd = c.order == VRT_PROBE_LAST ? min(c.K - 1, c.V) : c.m;
        if (lane < nd) r.det[lane] = a.t.row_det[rb * 32 + lane];
      }
    }
    wave_sync();
    if (drow && lane < nc && tok >= 0) {
      bool in_tail = true;
      for (int k = 0; k < nd; ++k) in_tail &= r.det[k] != tok;
      if (in_tail) L.qc[lane] = dense_tempered(load_one<DT>(drow, tok), dmax, (double)a.c.invT) / dzt;
    }
    if (lane == 0) {
      r.drow = drow;
      r.dzt = dzt;
      r.dmax = dmax;
      r.nd = nd;
    }
  }
  // the draws (keyed by depth and test index): probe test j = 0, the other kept
  // children j = 1, 2, .. in slot order, the final sample
  const uint32_t depth = (uint32_t)min(max(a.t.node_depth[nb + i], 0), 63);
  const bool cand = lane < nc && lane != pl && node >= 0;
  const uint64_t cmask = ballot(cand);
  const uint32_t j = 1u + (uint32_t)__builtin_popcountll(cmask & ((1ull << lane) - 1ull));
  const uint32_t tree = a.c.tree_base + (uint32_t)b;  // the tree's index in the draws' keys
  const float u = cand ? uniform24(a.seed, 32u * depth + j, tree, a.step, kPurposeTest) : 1.0f;
  if (lane < kChildMax) {
    r.node[lane] = node;
    r.tok[lane] = tok;
    r.x[lane] = x;
    r.u[lane] = u;
  }
  if (lane == 0) {
    r.nc = nc;
    r.probe = pl;
    r.nt = nt;
    r.depth = (int)depth;
    r.u0 = uniform24(a.seed, 32u * depth, tree, a.step, kPurposeTest);
    r.uf = uniform24(a.seed, depth, tree, a.step, kPurposeFinal);
  }
}


// The target row's normaliser from its chunk statistics, by one wave: MC = the largest
// fl(max*c2), S = sum of the chunk masses scaled to MC (each also written to pm).
__device__ __forceinline__ void target_norm(const float2* cs, int nch, double* pm, float& MC, double& S) {
  const int lane = lane_id();
  constexpr int kCPL = 8;  // chunks per lane: V <= 2^20
  float2 st[kCPL];
  static_for<kCPL>([&](auto k) {
    const int ch = lane + k * kWave;
    st[k] = ch < nch ? cs[ch] : make_float2(-INFINITY, 0.0f);
  });
  float mcl = -INFINITY;
  static_for<kCPL>([&](auto k) { mcl = fmaxf(mcl, st[k].x); });
  MC = wave_max(mcl);
  double sl = 0.0;
  static_for<kCPL>([&](auto k) {
    const int ch = lane + k * kWave;
    if (ch < nch) {
      const double m = (double)st[k].y * (double)fast_exp2(st[k].x - MC);
      pm[ch] = m;
      sl += m;
    }
  });
  S = wave_sum(sl);
}

// Dense rows, by wave 0 before the overlap pass: the target normaliser and the scale of
// q~ exactly as decide_node forms them (probe last: W_D = 1 - p of the other kept
// children), into R.
__device__ __forceinline__ void dense_prepare(const Cfg& c, const float2* cs, VRec& R, const DLds& L) {
  const int lane = lane_id();
  const int nch = (c.V + kCH - 1) / kCH;
  float MC;
  double S;
  target_norm(cs, nch, L.pm, MC, S);
  const bool ok = S > 0.0 && S < INFINITY && MC < INFINITY;
  const double invS = ok ? 1.0 / S : 0.0;
  const int nc = R.nc, probe = R.probe;
  const int tok = lane < nc ? R.tok[lane] : -1;
  const double pc = tok >= 0 ? (double)fast_exp2(__builtin_fmaf(R.x[lane], c.c2, -MC)) * invS : 0.0;
  const uint64_t cmask = ballot(lane < nc && lane != probe && R.node[lane] >= 0);
  double WD = 1.0;
  for (uint64_t m = cmask; m; m &= m - 1ull) WD -= readlane_d(pc, __builtin_ctzll(m));
  if (lane == 0) {
    R.mc = MC;
    R.invs = invS;
    R.qscale = c.order == VRT_PROBE_LAST ? WD : 1.0;
  }
}

// Dense rows, all waves: per 2048-token chunk, the sum over the probe's tail of
// min(p, s q~), with p from the target row and q~ regenerated from the draft row.
template <int DT, int NT>
__device__ __forceinline__ void dense_overlap(const Cfg& c, const char* row, const VRec& R, const DLds& L) {
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  constexpr int EPL = 16 / esz;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int V = c.V, nch = (V + kCH - 1) / kCH, nd = R.nd;
  const float MC = R.mc;
  const double invS = R.invs, qs = R.qscale / R.dzt, invT = (double)c.invT;
  const float dmax = R.dmax;
  for (int ch = wave; ch < nch; ch += NT / kWave) {
    const int my0 = ch * kCH + lane * 32;  // lane l owns tokens [my0, my0 + 32)
    u32x4_t xt[32 / EPL], xd[32 / EPL];
    static_for<32 / EPL>([&](auto q) {
      const int e0 = my0 + q * EPL;
      xt[q] = u32x4_t{0u, 0u, 0u, 0u};
      xd[q] = u32x4_t{0u, 0u, 0u, 0u};
      if (e0 < V) {
        xt[q] = *(const u32x4_t*)(row + (int64_t)e0 * esz);
        xd[q] = *(const u32x4_t*)(R.drow + (int64_t)e0 * esz);
      }
    });
    bool hd = false;  // the chunk holds a deterministic child (uniform)
    for (int k = 0; k < nd; ++k) hd |= R.det[k] >= ch * kCH && R.det[k] < (ch + 1) * kCH;
    double ov = 0.0;
    static_for<32 / EPL>([&](auto q) {
      static_for<EPL>([&](auto k) {
        float x, d;
        if constexpr (DT == VRT_BF16) {
          x = (k & 1) ? bf16_hi(xt[q][k >> 1]) : bf16_lo(xt[q][k >> 1]);
          d = (k & 1) ? bf16_hi(xd[q][k >> 1]) : bf16_lo(xd[q][k >> 1]);
        } else {
          x = __uint_as_float(xt[q][(int)k]);
          d = __uint_as_float(xd[q][(int)k]);
        }
        const int v = my0 + q * EPL + (int)k;
        bool tail = v < V;
        if (hd)
          for (int t = 0; t < nd; ++t) tail &= R.det[t] != v;
        if (tail) {
          const double p = (double)fast_exp2(__builtin_fmaf(x, c.c2, -MC)) * invS;
          const double qv = qs * dense_tempered(d, dmax, invT);
          ov += fmin(p, qv);
        }
      });
    });
    ov = wave_sum(ov);
    if (lane == 0) L.ov[ch] = ov;
  }
}

// The decision of node i by one wave, from the chunk statistics and gathered inputs
// in LDS (see the file comment). DENSE: the probe's tail is regenerated from the
// expansion's draft row (R.drow) instead of a tail table.
template <int DT, bool DENSE>
__device__ void decide_node(const VArgs& a, int b, int i, const char* row, const float2* cs,
                            VRec& R, const DLds& L) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const int V = c.V;
  const int nch = (V + kCH - 1) / kCH;
  const float c2 = c.c2;
  const int64_t nb = (int64_t)b * c.N;
  const int nc = R.nc, probe = R.probe, nt = R.nt;
  int r_node = -1, r_tok = -1;
  float r_x = -INFINITY, r_u = 1.0f;
  if (lane < kChildMax) {
    r_node = R.node[lane];
    r_tok = R.tok[lane];
    r_x = R.x[lane];
    r_u = R.u[lane];
  }
  const int ch_node = lane < nc ? r_node : -1;
  const int ch_tok = lane < nc ? r_tok : -1;
  const float ch_x = lane < nc ? r_x : -INFINITY;
  float MC;
  double S;
  target_norm(cs, nch, L.pm, MC, S);
  NodeOut out{-1, -1, 0, 0.0f};
  if (!(S > 0.0) || !(S < INFINITY) || !(MC < INFINITY)) {
    out.flags = (int)(VRT_ST_TARGET_BAD << 16);
    if (lane == 0) put_out(a, nb + i, out, R);
    return;
  }
  const double invS = 1.0 / S;
  auto p_of_x = [&](float x) -> double { return (double)fast_exp2(__builtin_fmaf(x, c2, -MC)) * invS; };
  const double pc = ch_tok >= 0 ? p_of_x(ch_x) : 0.0;

  // ---- probe tail: p, the overlap sum min(p, s q~), which kept child each token is.
  // Probe first: s = 1 and the probe is tested before the others. Probe last (the RRSw
  // order): the others are tested first as point masses, and the probe meets the
  // residual mass W_D = 1 - p(those children), so its tail is weighed with s = W_D.
  const bool last = c.order == VRT_PROBE_LAST;
  int tests = 0, near = 0;
  int accept = -1;
  double W = 1.0;  // mass of the residual the tests run against
  double q_child = lane < nc ? L.qc[lane] : -1.0;  // q~ of this lane's child, -1: not in the tail
  const bool cand = lane < nc && lane != probe && ch_node >= 0;
  const uint64_t cmask = ballot(cand);
  double WD = 1.0;  // residual mass once every other kept child is rejected (probe last)
  if (last)
    for (uint64_t m = cmask; m; m &= m - 1ull) WD -= readlane_d(pc, __builtin_ctzll(m));
  const double qscale = last ? WD : 1.0;
  double overlap = 0.0;
  const bool dense_tail = DENSE && R.drow != nullptr;  // the overlap pass ran
  if (probe >= 0) {
    double ov = 0.0;
    if constexpr (DENSE) {
      const int cpl = (nch + kWave - 1) / kWave;
      if (dense_tail)
        for (int ch = lane * cpl; ch < min(nch, (lane + 1) * cpl); ++ch) ov += L.ov[ch];
    }
    for (int e = lane; e < nt; e += kWave) {
      const int y = L.tid[e];
      const double p = y >= 0 ? p_of_x((float)L.tp[e]) : 0.0;
      const double q = qscale * (double)L.tq[e];
      L.tp[e] = p;
      ov += fmin(p, q);
    }
    overlap = wave_sum(ov);
    wave_sync();
    if (!last) W = 1.0 - overlap;
  }
  // weight of this lane's child when it is tested: probe first, its residual once the
  // probe is rejected; probe last, its p. The children are tested in slot order, each
  // lane's uniform drawn up front.
  const bool in_tail = q_child >= 0.0;
  const double wc = (in_tail && !last) ? (pc > q_child ? pc - q_child : 0.0) : pc;
  const float uc = r_u;

  // ---- the final residual (or bonus) sample's preparation: the residual's chunk masses,
  // the chunk holding u * Wf, its re-read issued, and the residual's changes inside it.
  // Taken only if every test rejects, against the residual with all of them rejected.
  // (Preparing it before the tests, so that the re-read overlaps them, measured the same
  // for the full pass and slower for the lazy walk.)
  const float uf = R.uf;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  constexpr int EPL = 16 / esz;
  double tgt = 0.0, before = 0.0;
  bool clamp = false;
  int lo = 0, my0 = 0, nitem = 0;
  u32x4_t raw[32 / EPL];
  u32x4_t rawd[DENSE ? 32 / EPL : 1];  // dense rows: the same tokens of the draft row
  const double W0 = W;  // the residual mass the tests start from
  auto prepare_final = [&]() {
    double Wf = W0;
    if (last) Wf = WD - overlap;
    else
      for (uint64_t m = cmask; m; m &= m - 1ull) Wf -= readlane_d(wc, __builtin_ctzll(m));
    tgt = (double)uf * Wf;
    for (int ch = lane; ch < nch; ch += kWave) L.dfix[ch] = 0;
    wave_sync();
    // changes of mass relative to p: the probe's tail (clipped residual, or zero for a
    // rejected child) and the rejected children outside it (zero). Fixed-point atomics
    // keep the per-chunk sums independent of the order of arrival. Dense rows: the tail's
    // clipping is the overlap pass's per-chunk sums, and each rejected child removes its
    // residual w (its p off the tail).
    if (!DENSE && probe >= 0) {
      for (int e = lane; e < nt; e += kWave) {
        const int y = L.tid[e];
        if (y < 0) continue;
        const double p = L.tp[e], q = qscale * (double)L.tq[e];
        const int slot = L.tslot[e];
        const bool rej = slot >= 0 && ((cmask >> slot) & 1ull);
        const double d = rej ? -p : -(p < q ? p : q);
        atomicAdd((unsigned long long*)&L.dfix[y / kCH], (unsigned long long)__double2ll_rn(d * kFix));
      }
    }
    const bool mine = DENSE ? cand : (cand && !in_tail);
    const double mdel = (DENSE && in_tail) ? -wc : -pc;
    if (mine) atomicAdd((unsigned long long*)&L.dfix[ch_tok / kCH], (unsigned long long)__double2ll_rn(mdel * kFix));
    wave_sync();
    // adjusted chunk masses, lane-blocked contiguous chunks
    const int cpl = (nch + kWave - 1) / kWave;
    const int c0 = lane * cpl, c1 = min(c0 + cpl, nch);
    double lmass = 0.0;
    for (int ch = c0; ch < c1; ++ch) {
      double mch = L.pm[ch] * invS + (double)L.dfix[ch] * (1.0 / kFix);
      if (dense_tail) mch -= L.ov[ch];
      if (mch < 0.0) mch = 0.0;
      L.pm[ch] = mch;
      lmass += mch;
    }
    const double incl = wave_incl_scan(lmass);
    const double excl = incl - lmass;
    // lane holding the crossing chunk; if rounding leaves none, the last lane with mass
    const uint64_t hit = ballot(tgt < incl && lmass > 0.0);
    int src = hit ? __builtin_ctzll(hit) : -1;
    clamp = false;
    if (src < 0) {
      const uint64_t pos = ballot(lmass > 0.0);
      src = pos ? 63 - __builtin_clzll(pos) : 0;
      clamp = true;
    }
    int cstar = -1;
    before = 0.0;
    if (lane == src) {
      double cum = excl;
      for (int ch = c0; ch < c1; ++ch) {
        if (L.pm[ch] > 0.0) {
          cstar = ch;
          before = cum;
          if (!clamp && tgt < cum + L.pm[ch]) break;
        }
        cum += L.pm[ch];
      }
      if (cstar < 0) cstar = c0 < nch ? c0 : nch - 1;
    }
    cstar = __shfl(cstar, src, kWave);
    before = __shfl(before, src, kWave);
    lo = cstar * kCH;
    // re-read the chunk; lane l owns tokens [lo + 32 l, lo + 32 l + 32)
    my0 = lo + lane * 32;
    static_for<32 / EPL>([&](auto q) {
      const int e0 = my0 + q * EPL;
      raw[q] = u32x4_t{0u, 0u, 0u, 0u};
      if (e0 < V) raw[q] = *(const u32x4_t*)(row + (int64_t)e0 * esz);
    });
    if constexpr (DENSE) {
      static_for<32 / EPL>([&](auto q) {
        const int e0 = my0 + q * EPL;
        rawd[q] = u32x4_t{0u, 0u, 0u, 0u};
        if (dense_tail && e0 < V) rawd[q] = *(const u32x4_t*)(R.drow + (int64_t)e0 * esz);
      });
    }
    // the changes that fall inside the chunk, listed for the owners of their tokens
    nitem = 0;
    wave_sync();
    if (!DENSE && probe >= 0) {
      for (int e0 = 0; e0 < nt; e0 += kWave) {
        const int e = e0 + lane;
        bool inside = false;
        int y = -1;
        double d = 0.0;
        if (e < nt) {
          y = L.tid[e];
          inside = y >= lo && y < lo + kCH;
          if (inside) {
            const double p = L.tp[e], q = qscale * (double)L.tq[e];
            const int slot = L.tslot[e];
            const bool rej = slot >= 0 && ((cmask >> slot) & 1ull);
            d = rej ? -p : -(p < q ? p : q);
          }
        }
        const uint64_t m = ballot(inside);
        if (inside) {
          const int at = nitem + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
          L.itok[at] = y;
          L.idel[at] = d;
        }
        nitem += (int)__builtin_popcountll(m);
      }
    }
    {
      const bool inside = mine && ch_tok >= lo && ch_tok < lo + kCH;
      const uint64_t m = ballot(inside);
      if (inside) {
        const int at = nitem + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
        L.itok[at] = ch_tok;
        L.idel[at] = mdel;
      }
      nitem += (int)__builtin_popcountll(m);
    }
  };

  // ---- the tests: the probe with min(1, p/(s q~)) (first, or after the others), the
  // others under the residual
  auto probe_test = [&](double sc) {
    const double qp = readlane_d(q_child, probe);
    const double qs = qp < 0.0 ? 0.0 : qp;  // a probe outside its tail has q~ = 0
    const double ps = readlane_d(pc, probe);
    const double ratio = ps / (sc * qs);
    const float u0 = R.u0;
    ++tests;
    if (fabs((double)u0 - ratio) < kBand) ++near;
    if ((double)u0 < ratio) accept = __builtin_amdgcn_readlane(ch_node, probe);
  };
  if (probe >= 0 && !last) probe_test(1.0);
  if (accept < 0) {
    for (uint64_t m = cmask; m; m &= m - 1ull) {
      const int k = __builtin_ctzll(m);
      const double wk = readlane_d(wc, k);
      const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(uc), k));
      ++tests;
      const double ratio = wk / W;
      if (fabs((double)u - ratio) < kBand) ++near;
      if ((double)u < ratio) {
        accept = __builtin_amdgcn_readlane(ch_node, k);
        break;
      }
      W -= wk;
    }
  }
  if (probe >= 0 && last && accept < 0) {
    probe_test(W);     // W == WD here: every other kept child was rejected
    W = WD - overlap;  // the mass the final sample runs against
  }

  // ---- nothing accepted: the final residual (or bonus) sample, inverse CDF of w / W in
  // token-id order against the residual with every test rejected (W == Wf now)
  if (accept < 0) {
    prepare_final();
    float* sw = L.w + lane * 33;  // stride 33: conflict-free per-lane walks
    {
      const float invSf = (float)invS;
      static_for<32 / EPL>([&](auto q) {
        static_for<EPL>([&](auto k) {
          float x;
          if constexpr (DT == VRT_BF16) x = (k & 1) ? bf16_hi(raw[q][k >> 1]) : bf16_lo(raw[q][k >> 1]);
          else x = __uint_as_float(raw[q][(int)k]);
          const int e = q * EPL + k;
          sw[e] = (my0 + e < V && x > -INFINITY) ? fast_exp2(__builtin_fmaf(x, c2, -MC)) * invSf : 0.0f;
          if constexpr (DENSE) {
            if (dense_tail && my0 + e < V) {  // a tail token keeps p - min(p, s q~)
              bool tail = true;
              for (int t = 0; t < R.nd; ++t) tail &= R.det[t] != my0 + e;
              if (tail) {
                const float d = (DT == VRT_BF16) ? ((k & 1) ? bf16_hi(rawd[q][k >> 1]) : bf16_lo(rawd[q][k >> 1]))
                                                 : __uint_as_float(rawd[q][(int)k]);
                const double pd = (double)fast_exp2(__builtin_fmaf(x, c2, -MC)) * invS;
                const double qv = qscale * dense_tempered(d, R.dmax, (double)c.invT) / R.dzt;
                sw[e] = (float)(pd - fmin(pd, qv));
              }
            }
          }
        });
      });
    }
    wave_sync();
    // the changes inside the chunk, one per lane (distinct tokens)
    for (int it = lane; it < nitem; it += kWave) {
      const int off = L.itok[it] - lo;
      float* pw = L.w + (off >> 5) * 33 + (off & 31);
      const double v = (double)*pw + L.idel[it];
      *pw = v > 0.0 ? (float)v : 0.0f;
    }
    wave_sync();
    double lsum = 0.0;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) lsum += (double)sw[k];
    const double lincl = wave_incl_scan(lsum) + before;
    const double lexcl = lincl - lsum;
    const uint64_t hit2 = ballot(tgt < lincl && lsum > 0.0);
    int src2 = (hit2 && !clamp) ? __builtin_ctzll(hit2) : -1;
    bool clamp2 = clamp;
    if (src2 < 0) {
      const uint64_t pos = ballot(lsum > 0.0);
      src2 = pos ? 63 - __builtin_clzll(pos) : 0;
      clamp2 = true;
    }
    // the token: lane src2's 32 weights, one per lane, scanned by the whole wave; the
    // first with weight whose inclusive sum passes tgt (clamped, or if rounding leaves
    // none: the last with weight)
    const float wk = lane < 32 ? L.w[src2 * 33 + lane] : 0.0f;
    const double kincl = wave_incl_scan((double)wk) + __shfl(lexcl, src2, kWave);
    const uint64_t pos = ballot(wk > 0.0f);
    const uint64_t hit3 = clamp2 ? 0ull : ballot(wk > 0.0f && tgt < kincl);
    const int kk = hit3 ? __builtin_ctzll(hit3) : (pos ? 63 - __builtin_clzll(pos) : -1);
    const int base_tok = lo + src2 * 32;
    if (kk >= 0) {
      const double b1 = __shfl(kincl, kk, kWave);
      const double b0 = b1 - (double)__shfl(wk, kk, kWave);
      out.token = base_tok + kk;
      if (W > 0.0 && (fabs((double)uf - b0 / W) < kBand || fabs((double)uf - b1 / W) < kBand)) ++near;
    } else {
      out.token = min(base_tok, V - 1);
      const double b = __shfl(lexcl, src2, kWave);
      if (W > 0.0 && fabs((double)uf - b / W) < kBand) ++near;
    }
  }
  out.accept = accept;
  out.flags = min(tests, 255) | (min(near, 255) << 8);
  if (accept < 0) out.W = (float)W;
  if (lane == 0) put_out(a, nb + i, out, R);
}

constexpr int kMaxChunks = (1 << 20) / kCH;  // V <= 2^20

// One node's pass by a block of NT threads: stream the row (all waves), gather the
// decision inputs (last wave, overlapping the others' stream), then decide (wave 0).
template <int DT, int NT, bool DENSE = false>
__device__ __forceinline__ void node_pass(const VArgs& a, int b, int i, int nn, float2* s_cs, VRec& s_rec,
                                          const DLds& L, int& s_next) {
  const Cfg& c = a.c;
  const int V = c.V;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + ((int64_t)b * a.tstride + (int64_t)i * a.ld) * esz;
  const int nch = (V + kCH - 1) / kCH;
  const int nfull = V / kCH;
  const int wave = threadIdx.x >> 6;
  constexpr int NW = NT / kWave;
  if (threadIdx.x == 0) s_next = NW;
  __syncthreads();
  if (wave == NW - 1) gather_node<DT, DENSE>(a, b, i, nn, row, s_rec, L);
  // pairs of chunks are handed out as waves become free (the gathering wave takes
  // fewer); both chunks' loads are in flight together
  const int npair = (nch + 1) / 2;
  for (int pr = wave; pr < npair;) {
    const int ca = 2 * pr, cb = 2 * pr + 1;
    ChunkRegs<DT> ra, rb;
    issue_chunk<DT>(row, ca * kCH, V, ra);
    issue_chunk<DT>(row, cb * kCH, V, rb);  // past the row end: all -inf, not stored
    int nx = 0;
    if (lane_id() == 0) nx = atomicAdd(&s_next, 1);
    nx = __builtin_amdgcn_readfirstlane(nx);
    float2 sa, sb;
    chunk_stats2<DT>(ra, rb, ca * kCH, cb * kCH, V, c.c2, ca >= nfull, cb >= nfull, sa, sb);
    if (lane_id() == 0) {
      s_cs[ca] = sa;
      if (cb < nch) s_cs[cb] = sb;
    }
    pr = nx;
  }
  __syncthreads();
  if constexpr (DENSE) {
    // a kept probe on a dense row: its tail's overlap with p in a second pass over the
    // target row and the expansion's draft row
    if (s_rec.drow != nullptr) {  // uniform
      if (wave == 0) dense_prepare(c, s_cs, s_rec, L);
      __syncthreads();
      dense_overlap<DT, NT>(c, row, s_rec, L);
      __syncthreads();
    }
  }
  if (wave == 0) decide_node<DT, DENSE>(a, b, i, row, s_cs, s_rec, L);
}

__device__ void install_tag(const VArgs& a, int b);
__device__ void walk_if_last(const VArgs& a, int b, int nn, uint32_t st_node);

// One block per (node, tree): that node's pass; WALK: then the tree's walk if this block
// is the last of its tree to finish.
template <int DT, bool WALK>
__global__ __launch_bounds__(kVB) void k_vnode(const VArgs a) {
  const Cfg& c = a.c;
  const int b = blockIdx.x;  // trees vary fastest: blocks that finish together belong to
  const int i = blockIdx.y;  // different trees, whose counters sit on different lines
  const int nn = clamp_nodes(a.t.n_nodes[b], c.N);
  if (i >= nn) return;
  __shared__ float2 s_cs[kMaxChunks];
  __shared__ VRec s_rec;
  __shared__ int s_next;
  extern __shared__ double s_dyn[];
  const DLds L = carve((char*)s_dyn, (c.V + kCH - 1) / kCH, c.TC);
  // the tree's counter word carries this launch's tag before any block counts on it;
  // the gathering wave (whose dependent loads have slack behind the stream) sees to it
  if (WALK && threadIdx.x == kVB - kWave) install_tag(a, b);
  node_pass<DT, kVB>(a, b, i, nn, s_cs, s_rec, L, s_next);
  if constexpr (WALK) {
    if ((threadIdx.x >> 6) == 0) {
      wave_sync();  // s_rec.res, written by lane 0
      walk_if_last(a, b, nn, (uint32_t)s_rec.res.flags >> 16);
    }
  }
}

// Dense rows: the same pass with the probe tails regenerated from the draft rows.
template <int DT, bool WALK>
__global__ __launch_bounds__(kVB) void k_vnode_dense(const VArgs a) {
  const Cfg& c = a.c;
  const int b = blockIdx.x;
  const int i = blockIdx.y;
  const int nn = clamp_nodes(a.t.n_nodes[b], c.N);
  if (i >= nn) return;
  __shared__ float2 s_cs[kMaxChunks];
  __shared__ VRec s_rec;
  __shared__ int s_next;
  extern __shared__ double s_dyn[];
  const DLds L = carve((char*)s_dyn, (c.V + kCH - 1) / kCH, c.TC);
  if (WALK && threadIdx.x == kVB - kWave) install_tag(a, b);
  node_pass<DT, kVB, true>(a, b, i, nn, s_cs, s_rec, L, s_next);
  if constexpr (WALK) {
    if ((threadIdx.x >> 6) == 0) {
      wave_sync();
      walk_if_last(a, b, nn, (uint32_t)s_rec.res.flags >> 16);
    }
  }
}

// Emitted tokens, nodes and statistics of tree b once its walk has ended (len tokens).
__device__ __forceinline__ void walk_outputs(const VArgs& a, int b, int len, uint32_t st, int probe, int near,
                                             int visited) {
  const Cfg& c = a.c;
  for (int k = len; k <= c.D; ++k) a.out_tokens[(int64_t)b * (c.D + 1) + k] = -1;
  for (int k = len - 1; k < c.D; ++k) a.out_nodes[(int64_t)b * c.D + k] = -1;
  a.out_len[b] = len;
  if (a.stats) {
    uint32_t* s = a.stats + (int64_t)b * 8;
    s[0] |= st;
    s[1] = (uint32_t)(len - 1);
    s[2] = (uint32_t)probe;
    s[3] = (uint32_t)near;
    s[4] = (uint32_t)visited;
    s[5] = s[6] = s[7] = 0;
  }
}

// Lazy verification: one block per tree walks from the root and decides only the nodes
// the walk reaches, each exactly as k_vnode decides it (its row streamed once), so the
// rows of the other nodes are never read. Bytes per tree: (emitted tokens) rows instead
// of n_nodes rows; the cost is one dependent pass per depth.
constexpr int kVL = 1024;  // threads of a lazy-walk block

template <int DT>
__global__ __launch_bounds__(kVL) void k_vlazy(const VArgs a) {
  const Cfg& c = a.c;
  const int b = blockIdx.x;
  const int nn = clamp_nodes(a.t.n_nodes[b], c.N);
  const int64_t nb = (int64_t)b * c.N;
  __shared__ float2 s_cs[kMaxChunks];
  __shared__ VRec s_rec;
  __shared__ int s_next;
  extern __shared__ double s_dyn[];
  const DLds L = carve((char*)s_dyn, (c.V + kCH - 1) / kCH, c.TC);
  const bool t0 = threadIdx.x == 0;
  int cur = 0, len = 0, near = 0, probe = 0, visited = 0;
  uint32_t st = 0;
  for (int step = 0; step <= c.D; ++step) {
    node_pass<DT, kVL>(a, b, cur, nn, s_cs, s_rec, L, s_next);
    __syncthreads();  // the decision is in s_rec.res
    const NodeOut o = s_rec.res;
    ++visited;
    near += (o.flags >> 8) & 0xFF;
    st |= (uint32_t)o.flags >> 16;
    if (o.accept > cur && o.accept < nn && len < c.D) {
      if (t0) {
        a.out_nodes[(int64_t)b * c.D + len] = o.accept;
        a.out_tokens[(int64_t)b * (c.D + 1) + len] = a.t.node_token[nb + o.accept];
      }
      if (a.t.node_kind[nb + o.accept] == VRT_PROBE) probe = 1;
      ++len;
      cur = o.accept;
    } else {
      if (t0) a.out_tokens[(int64_t)b * (c.D + 1) + len] = o.token;
      ++len;
      break;
    }
  }
  if (t0) walk_outputs(a, b, len, st, probe, near, visited);
}

// One wave per tree: the walk over the decided nodes. The tree's decisions, tokens
// and kinds are first loaded into LDS (one round of parallel loads), then lane 0
// follows the accepted children from the root.
__global__ __launch_bounds__(kWave) void k_vwalk(const VArgs a) {
  const Cfg& c = a.c;
  const int b = blockIdx.x;
  const int nn = clamp_nodes(a.t.n_nodes[b], c.N);
  const int lane = lane_id();
  const int64_t nb = (int64_t)b * c.N;
  extern __shared__ int4 s_walk[];  // [N] decisions, then [N] tokens, then [N] kinds
  int* s_tok = (int*)(s_walk + c.N);
  int* s_kind = s_tok + c.N;
  uint32_t st = 0;
  for (int i = lane; i < nn; i += kWave) {
    const NodeOut o = a.node_out[nb + i];
    s_walk[i] = make_int4(o.accept, o.token, o.flags, 0);
    s_tok[i] = a.t.node_token[nb + i];
    s_kind[i] = a.t.node_kind[nb + i];
    st |= (uint32_t)o.flags >> 16;
  }
  st = wave_reduce(st, [](uint32_t x, uint32_t y) { return x | y; });
  wave_sync();
  if (lane != 0) return;
  int cur = 0, len = 0, near = 0, probe = 0, visited = 0;
  for (int step = 0; step <= c.D; ++step) {
    const int4 o = s_walk[cur];
    ++visited;
    near += (o.z >> 8) & 0xFF;
    if (o.x > cur && o.x < nn && len < c.D) {
      a.out_nodes[(int64_t)b * c.D + len] = o.x;
      a.out_tokens[(int64_t)b * (c.D + 1) + len] = s_tok[o.x];
      if (s_kind[o.x] == VRT_PROBE) probe = 1;
      ++len;
      cur = o.x;
    } else {
      a.out_tokens[(int64_t)b * (c.D + 1) + len] = o.y;
      ++len;
      break;
    }
  }
  walk_outputs(a, b, len, st, probe, near, visited);
}

// The walk of tree b by one wave, reading the decisions written device-coherently by the
// tree's node blocks: the decisions of 64 consecutive nodes are loaded at a time (one lane
// each), and the walk moves to the chunk holding the next node when it leaves the loaded
// one (children follow their parents, so chunks are visited in order).
__device__ void walk_tree(const VArgs& a, int b, int nn, uint32_t st) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const int64_t nb = (int64_t)b * c.N;
  int c0 = -1, m_acc = -1, m_tok = -1, m_fl = 0, m_ntok = -1, m_kind = 0;
  auto load_chunk = [&](int cc) {
    c0 = cc;
    const int i = cc + lane;
    m_acc = -1, m_tok = -1, m_fl = 0, m_ntok = -1, m_kind = 0;
    if (i < nn) {
      const int* o = (const int*)&a.node_out[nb + i];
      m_acc = ld_dev(o);
      m_tok = ld_dev(o + 1);
      m_fl = ld_dev(o + 2);
      m_ntok = a.t.node_token[nb + i];
      m_kind = a.t.node_kind[nb + i];
    }
  };
  load_chunk(0);
  int cur = 0, len = 0, near = 0, probe = 0, visited = 0;
  for (int step = 0; step <= c.D; ++step) {
    const int l = cur - c0;
    const int acc = __builtin_amdgcn_readlane(m_acc, l);
    const int tok = __builtin_amdgcn_readlane(m_tok, l);
    const int fl = __builtin_amdgcn_readlane(m_fl, l);
    ++visited;
    near += (fl >> 8) & 0xFF;
    if (acc > cur && acc < nn && len < c.D) {
      if ((acc & ~(kWave - 1)) != c0) load_chunk(acc & ~(kWave - 1));
      const int l2 = acc - c0;
      const int ntok = __builtin_amdgcn_readlane(m_ntok, l2);
      if (__builtin_amdgcn_readlane(m_kind, l2) == VRT_PROBE) probe = 1;
      if (lane == 0) {
        a.out_nodes[(int64_t)b * c.D + len] = acc;
        a.out_tokens[(int64_t)b * (c.D + 1) + len] = ntok;
      }
      ++len;
      cur = acc;
    } else {
      if (lane == 0) a.out_tokens[(int64_t)b * (c.D + 1) + len] = tok;
      ++len;
      break;
    }
  }
  if (lane == 0) walk_outputs(a, b, len, st, probe, near, visited);
}

// The fused walk's per-tree word: tag << 32 | status << 24 | nodes counted. At its start
// each node block makes sure the word carries this launch's tag: a word left by another
// launch, or garbage, is replaced by the bare tag by compare-and-swap (only the first
// blocks of a tree find it stale; a failed swap returns the word another block installed).
// Every block checks this before it counts, so no count precedes the tree's install, and
// the word keeps the tag until the tree's last block resets it.
__device__ void install_tag(const VArgs& a, int b) {
  unsigned long long* p = (unsigned long long*)(a.vsync + (int64_t)b * kSyncStride);
  const unsigned long long tag = (unsigned long long)a.tag << 32;
  unsigned long long v = ld_dev64((const uint64_t*)p);
  while ((v & 0xFFFFFFFF00000000ull) != tag) {
    const unsigned long long seen = atomicCAS(p, v, tag);
    v = seen == v ? tag : seen;
  }
}

// Wave 0 of a node block once its decision is stored: status bits are OR-ed into the
// tree's word and one atomic add counts the node, so no block retries against the others.
// The block that counts the tree's last node sets the word back to 0 (a replay with the
// same tag then starts afresh) and walks the tree.
__device__ void walk_if_last(const VArgs& a, int b, int nn, uint32_t st_node) {
  const int lane = lane_id();
  wait_stores();  // this node's decision is written before it is counted
  unsigned long long word = 0ull;
  if (lane == 0) {
    unsigned long long* p = (unsigned long long*)(a.vsync + (int64_t)b * kSyncStride);
    if (st_node & 0xFFu) atomicOr(p, (unsigned long long)(st_node & 0xFFu) << 24);
    word = atomicAdd(p, 1ull) + 1ull;
  }
  word = shfl64(word, 0);
  if ((int)(word & 0xFFFFFFull) != nn) return;
  if (lane == 0) st_dev64(a.vsync + (int64_t)b * kSyncStride, 0ull);
  walk_tree(a, b, nn, (uint32_t)(word >> 24) & 0xFFu);
}

// Tags of fused launches: a process-wide counter from a random start, never 0.
std::atomic<uint32_t> g_vtag{(uint32_t)std::random_device{}()};

}  // namespace

size_t verify_ws_bytes(const Cfg& c) { return (size_t)c.B * kSyncStride * 8; }

hipError_t launch_verify(int parts, const Cfg& c, const TreePtrs& t, const void* logits, int64_t ld,
                         int64_t tstride, uint64_t seed, uint32_t step, NodeOut* node_out,
                         int32_t* out_tokens, int32_t* out_nodes, int32_t* out_len, uint32_t* stats,
                         void* ws, const void* const* draft, int64_t dld, int64_t dstride,
                         hipStream_t stream) {
  VArgs a{c, t, logits, ld, tstride, seed, step, node_out, out_tokens, out_nodes, out_len, stats, {}, dld,
          dstride, (uint64_t*)ws, 0u};
  for (int l = 0; l < c.D && l < 32 && draft; ++l) a.draft[l] = draft[l];
  const bool fused = (parts & 3) == 3;  // the nodes and the walk in one launch
  if (fused) {
    uint32_t tag;
    do tag = g_vtag.fetch_add(1); while (tag == 0u);
    a.tag = tag;
  }
  if (parts & 1) {
    const dim3 grid(c.B, c.N);
    const size_t lds = decide_lds_bytes(c);
    const bool dense = (parts & 8) != 0;
    if (c.dtype == VRT_BF16) {
      if (dense) {
        if (fused) hipLaunchKernelGGL((k_vnode_dense<VRT_BF16, true>), grid, dim3(kVB), lds, stream, a);
        else hipLaunchKernelGGL((k_vnode_dense<VRT_BF16, false>), grid, dim3(kVB), lds, stream, a);
      } else {
        if (fused) hipLaunchKernelGGL((k_vnode<VRT_BF16, true>), grid, dim3(kVB), lds, stream, a);
        else hipLaunchKernelGGL((k_vnode<VRT_BF16, false>), grid, dim3(kVB), lds, stream, a);
      }
    } else {
      if (dense) {
        if (fused) hipLaunchKernelGGL((k_vnode_dense<VRT_F32, true>), grid, dim3(kVB), lds, stream, a);
        else hipLaunchKernelGGL((k_vnode_dense<VRT_F32, false>), grid, dim3(kVB), lds, stream, a);
      } else {
        if (fused) hipLaunchKernelGGL((k_vnode<VRT_F32, true>), grid, dim3(kVB), lds, stream, a);
        else hipLaunchKernelGGL((k_vnode<VRT_F32, false>), grid, dim3(kVB), lds, stream, a);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((parts & 2) && !fused)
    hipLaunchKernelGGL(k_vwalk, dim3(c.B), dim3(kWave), (size_t)c.N * (16 + 4 + 4), stream, a);
  if (parts & 4) {
    const size_t lds = decide_lds_bytes(c);
    if (c.dtype == VRT_BF16)
      hipLaunchKernelGGL(k_vlazy<VRT_BF16>, dim3(c.B), dim3(kVL), lds, stream, a);
    else
      hipLaunchKernelGGL(k_vlazy<VRT_F32>, dim3(c.B), dim3(kVL), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace vrt
