// Draft-tree construction on gfx950 (RheoSampling framework flowchart, key designs
// 1-2; SMART key design 3 as the switchable keep rule). Per layer one kernel, then one
// to emit the tree:
//
// k_select_expand: one 8-wave block per expanded parent. Short lists (trunc <= 256):
//   the waves stream the parent's draft row once (all of a segment's loads in flight,
//   non-temporal), keep each lane's largest group maxima, find one threshold for the
//   whole row from a histogram of their distance below the largest, re-read only the
//   groups that reach it and rank the exact keys; rows with many ties take an exact
//   radix selection instead. Lists of 512 and 1024 keys sort the staged keys by wave
//   slices in registers and pairwise merges.
//   Wave 0 then expands the parent: untempered softmax on the top-trunc support with
//   the fixed ranking recipe, tempered softmax in fp64, the probe draw from the
//   tempered tail, the proxy min{q(x_m), z}, the K child slots and the parent's tail
//   table. The last row block of each tree ranks the layer's children by (path score
//   desc, creation index asc) and keeps the top W (top-R mode) or runs SMART's
//   sequential keep rule (k_rank_layer does this for layers of more than 256 children).
// k_dense_expand: the same per parent with no truncation (the dense baseline): the K best
//   keys, one pass of exact-order sums over the whole row, the probe drawn in token order.
// k_finish: one block per tree emits the tree: the global top R by the same key
//   (or SMART's admitted nodes), parents before children, child lists in slot
//   order, and the probe tails the verifier needs.
// k_coverage: the share of each row's softmax inside its top-trunc support (a
//   measurement of the inputs, not a step of the build).
#include <atomic>
#include <random>

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
  int fuse_rank;  // the layer's ranking runs in its row blocks
  int split;      // blocks per row: 1, or 2 (each selects from half of the row's segments)
  uint64_t* half_keys;  // split rows: [B][FP][4][list length] each part's sorted support
  int* half_meta;       // split rows: [B][FP][4] each part's support size | non-finite << 30
  uint64_t epoch;       // split rows: this launch's tag base, unique within the process
  int rpt;              // rows per tree at this layer (1 at the root, else FP)
  int mixed;            // > 0: a 1-D grid whose first `mixed` rows (tree-major) are whole
                        // and whose other rows are split over `parts` blocks each
  int parts;            // 2 or 4
  int compact;          // > 0: a compact grid of this many blocks over the layer's expanded
                        // rows (SMART layers)
  int rest;             // compact grids: blocks of the kernel that takes the rows beyond them
                        // (0: the ranking kernel takes each tree's own rows beyond them)
  int* cpre;            // compact grids: the prefix sums pre[0 .. B] of the frontier sizes
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

constexpr int kSegLoads = 16;  // 16-byte loads per lane per segment, all in flight at once

template <int DT>
constexpr int seg_elems() { return kWave * kSegLoads * (DT == VRT_BF16 ? 8 : 4); }

constexpr int kSelWaves = 8;  // waves of a row block
// segments per wave the row-wide path of a row block takes (rows up to 24 bf16 or 16 fp32
// segments; longer rows are split over two blocks, or take the exact path)
template <int DT>
constexpr int seg_per_wave() { return DT == VRT_BF16 ? 3 : 2; }

__device__ __forceinline__ float max3n(float a, float b, float c) {  // NaN-propagating
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// One wave's load of segment g of a row: load q of this lane covers elements
// [seg0 + (q*64 + lane)*EPL, +EPL), all 16 loads in flight at once; elements at or
// past V read as -inf.
template <int DT>
__device__ __forceinline__ void load_segment(const char* row, int g, int V, u32x4_t (&d)[kSegLoads]) {
  constexpr bool BF = DT == VRT_BF16;
  constexpr int esz = BF ? 2 : 4;
  constexpr int EPL = 16 / esz;
  const int lane = lane_id();
  const int seg0 = g * seg_elems<DT>();
  static_for<kSegLoads>([&](auto q) {
    const int e0 = seg0 + (q * kWave + lane) * EPL;
    const uint32_t ninf = BF ? 0xFF80FF80u : 0xFF800000u;
    u32x4_t v = {ninf, ninf, ninf, ninf};
    if (e0 < V) v = __builtin_nontemporal_load((const u32x4_t*)(row + (int64_t)e0 * esz));
    d[q] = v;
  });
  if (V - seg0 < seg_elems<DT>()) {  // the row's last segment: mask a straddling load
    static_for<kSegLoads>([&](auto q) {
      const int e0 = seg0 + (q * kWave + lane) * EPL;
      if (e0 < V && e0 + EPL > V) {
        static_for<EPL>([&](auto e) {
          if (e0 + e >= V) {
            if constexpr (BF)
              d[q][e >> 1] = (e & 1) ? ((d[q][e >> 1] & 0xFFFFu) | 0xFF800000u)
                                     : ((d[q][e >> 1] & 0xFFFF0000u) | 0xFF80u);
            else
              d[q][(int)e] = 0xFF800000u;
          }
        });
      }
    });
  }
}

// Maximum of each group (one lane's load), NaN-propagating so that one class test per
// group flags a non-finite row.
template <int DT>
__device__ __forceinline__ void group_maxima(const u32x4_t (&d)[kSegLoads], float (&gm)[kSegLoads]) {
  static_for<kSegLoads>([&](auto q) {
    if constexpr (DT == VRT_BF16) {
      auto lo = [&](int i) { return bf16_lo(d[q][i]); };
      auto hi = [&](int i) { return bf16_hi(d[q][i]); };
      const float t1 = max3n(lo(0), hi(0), lo(1));
      const float t2 = max3n(hi(1), lo(2), hi(2));
      gm[q] = __builtin_elementwise_maximum(max3n(lo(3), hi(3), t1), t2);
    } else {
      auto f = [&](int i) { return __uint_as_float(d[q][i]); };
      gm[q] = __builtin_elementwise_maximum(max3n(f(0), f(1), f(2)), f(3));
    }
  });
}

// Order-preserving image of a row value: 16 bits for bf16 values (the low half of the
// fp32 image carries nothing), 32 bits for fp32; NaN maps to 0. value_of inverts it.
template <int DT>
using Img = std::conditional_t<DT == VRT_BF16, uint16_t, uint32_t>;
template <int DT>
__device__ __forceinline__ uint32_t img_of(float x) {
  if constexpr (DT == VRT_BF16) return ord32(x) >> 16;
  else return ord32(x);
}
template <int DT>
__device__ __forceinline__ float value_of(uint32_t img) {
  if constexpr (DT == VRT_BF16) {
    const uint32_t h = (img & 0x8000u) ? (img & 0x7FFFu) : (~img & 0xFFFFu);
    return __uint_as_float(h << 16);
  } else {
    return unord32(img);
  }
}

// ---------------------------------------------------------------------------
// Row-wide selection: one threshold for the whole row. The usual threshold search is
// one histogram of the candidates' distance below the largest one, in 1/kDistScale
// steps of value, kDistBins bins.
constexpr int kDistBins = 1024;
constexpr float kDistScale = 64.0f;

template <int DT, int PL>
struct FastLds {
  static constexpr int LV = 4;                         // candidates per lane and segment
  // staged keys held: 4N, 6N for supports of 1024 keys (bf16 rows hold many ties near
  // their 1024th value: 4N staged keys overflowed on a few rows in a hundred; 6N keeps
  // the block's LDS small enough for two blocks per CU)
  static constexpr int KCAP = (PL >= 16 ? 6 : 4) * PL * kWave;
  // a candidate: group maximum's image << 8 | its load index q
  using CK = std::conditional_t<DT == VRT_BF16, uint32_t, uint64_t>;
  alignas(16) uint64_t keys[KCAP];        // row keys of the elements that reach it
  int hist[kDistBins];  // distance histogram; its first 256 bins serve the radix levels
  int sel[2];
  int wmax[16];
  int nk, ng, bad;
};

// The row's top TC keys (value desc, token id asc) into s_sup (positions < N, sorted,
// zero-padded), by all waves of the block. Thread (wave, lane) owns the lane-segments
// (wave + j*SW, lane): lane's loads of those segments.
//  A. each wave loads its segments (16 KB each, all loads in flight); each lane keeps,
//     per lane-segment, every group maximum and the LV largest with their load indices;
//  B. the TC-th largest of all these candidates, t (a radix selection, one byte per
//     block-wide histogram), is reached by at least TC distinct elements, so no element
//     below it is among the row's TC best; on Zipf-shaped rows with jitter it is the
//     row's TC-th value itself;
//  C. each thread re-reads its candidate groups that reach t (16 bytes each, all in
//     flight; where all LV candidates of a lane-segment reach t, its other groups that
//     do too) and stages the exact keys of their elements that reach t;
//  D. the staged keys are distinct: below 512-key supports each one's rank among them
//     places it in s_sup; from 512 keys on, sorted 256-key slices are merged pairwise.
// Returns 0 on success, 1 for a non-finite row, 2 when more keys reach t than the path
// holds (ties, flat rows; floor_img is then t's image) or fewer than TC (tiny rows):
// the caller then takes the exact path. The result is uniform over the block.
template <int DT, int PL, int SW, int LSPT>
__device__ __forceinline__ int row_select_fast(const char* row, int g0, int g1, int V, int TC,
                                               FastLds<DT, PL>& F, uint64_t* s_sup, int& n_sup,
                                               uint32_t& floor_img) {
  using FL = FastLds<DT, PL>;
  using CK = typename FL::CK;
  constexpr bool BF = DT == VRT_BF16;
  constexpr int N = PL * kWave;
  constexpr int LV = FL::LV;
  constexpr int NT = SW * kWave;
  constexpr int RB = BF ? 16 : 32;
  constexpr int esz = BF ? 2 : 4;
  constexpr int EPL = 16 / esz;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  if (tid == 0) {
    F.nk = 0;
    F.ng = 0;
    F.bad = 0;
  }
  for (int i = tid; i < kDistBins; i += NT) F.hist[i] = 0;
  for (int i = tid; i < FL::KCAP; i += NT) F.keys[i] = 0ull;
  __syncthreads();

  // A. (the thread's lane-segments are (g0 + wave + j*SW, lane): the same in every phase)
  CK cand[LSPT][LV];
  constexpr int GPW = BF ? 2 : 1;              // group maxima images per word
  uint32_t gmi[LSPT][kSegLoads / GPW];         // every group maximum's image
  bool nf = false;
  static_for<LSPT>([&](auto j) {
    const int g = g0 + wave + j * SW;
    static_for<LV>([&](auto s) { cand[j][s] = 0; });
    static_for<kSegLoads / GPW>([&](auto h) { gmi[j][h] = 0u; });
    if (g < g1) {  // uniform
      u32x4_t d[kSegLoads];
      load_segment<DT>(row, g, V, d);
      float gm[kSegLoads];
      group_maxima<DT>(d, gm);
      static_for<kSegLoads>([&](auto q) {
        nf |= __builtin_amdgcn_classf(gm[q], 0x203);  // NaN, +inf
        const uint32_t im = img_of<DT>(gm[q]);
        gmi[j][q / GPW] |= im << (16 * (q % GPW));
        CK x = ((CK)im << 8) | (CK)q;
        static_for<LV>([&](auto s) {
          const CK h = cand[j][s] > x ? cand[j][s] : x;
          x = cand[j][s] > x ? x : cand[j][s];
          cand[j][s] = h;
        });
      });
    }
  });
  {
    uint32_t mx = 0u;  // the wave's largest candidate image
    static_for<LSPT>([&](auto j) { mx = max(mx, (uint32_t)(cand[j][0] >> 8)); });
    mx = wave_reduce(mx, [](uint32_t x, uint32_t y) { return max(x, y); });
    if (lane == 0) F.wmax[wave] = mx;
  }
  if (ballot(nf) != 0ull && lane == 0) F.bad = 1;
  __syncthreads();
  if (F.bad) return 1;

  // B. Usually one histogram of the candidates' value distance below the largest, Mv
  // (bin = floor(kDistScale * (Mv - x))), finds the smallest bin d that TC candidates
  // reach; t is then the smallest image whose value falls in bins 0..d (a binary search:
  // the bin is monotone in the value). When fewer than TC candidates lie in the window,
  // a radix selection over the images.
  uint32_t M = 0u;
  static_for<SW>([&](auto w) { M = max(M, (uint32_t)F.wmax[w]); });
  const float Mv = value_of<DT>(M);
  auto dist = [&](uint32_t im) { return (Mv - value_of<DT>(im)) * kDistScale; };
  static_for<LSPT>([&](auto j) {
    if (g0 + wave + j * SW < g1) {  // uniform
      static_for<LV>([&](auto s) {
        const float dd = dist((uint32_t)(cand[j][s] >> 8));
        if (dd < (float)(kDistBins - 1)) atomicAdd(&F.hist[(int)dd], 1);
      });
    }
  });
  __syncthreads();
  if (wave == 0) {
    constexpr int HB = kDistBins / kWave;
    int h[HB];
    static_for<HB>([&](auto i) { h[i] = F.hist[lane * HB + i]; });  // ascending distance
    int ls = 0;
    static_for<HB>([&](auto i) { ls += h[i]; });
    int cum = wave_incl_scan(ls) - ls;
    int pick = -1;
    static_for<HB>([&](auto i) {
      cum += h[i];
      if (pick < 0 && cum >= TC) pick = lane * HB + i;
    });
    const uint64_t has = ballot(pick >= 0);
    const int d = __shfl(pick, has ? __builtin_ctzll(has) : 0, kWave);
    if (lane == 0) F.sel[0] = has ? d : -1;
  }
  __syncthreads();
  const int dsel = F.sel[0];
  uint32_t pre = 0u;   // image bits fixed so far (the high ones)
  if (dsel >= 0) {
    // smallest image in bins 0..dsel: dist(lo) is outside (or NaN), dist(hi) inside; a
    // 64-way search, each lane testing one point per round (the inside points form a
    // suffix: the distance falls as the image grows)
    const float lim = (float)(dsel + 1);
    uint32_t lo = BF ? 0x007Eu : 0x007FFFFEu, hi = M;
    while (hi - lo > 1u) {
      const uint64_t step = ((uint64_t)(hi - lo) + 63u) / 64u;
      const uint64_t pt = (uint64_t)lo + (uint64_t)(lane + 1) * step;  // the last lane's >= hi
      const uint64_t in = ballot(pt >= hi || dist((uint32_t)pt) < lim);
      const int f = __builtin_ctzll(in);
      hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + (uint64_t)(f + 1) * step);
      lo = (uint32_t)((uint64_t)lo + (uint64_t)f * step);
    }
    pre = hi;
  } else {
  if (tid < 256) F.hist[tid] = 0;
  __syncthreads();
  int above = 0;       // candidates whose fixed bits exceed pre's
  static_for<RB / 8>([&](auto lvl) {
    constexpr int sh = RB - 8 * (lvl + 1);
    // the top byte takes few values: a wave counts each with ballots and adds once (same-
    // address LDS atomics from every lane would serialise); the next byte spreads out
    bool lanewise = lvl > 0;
    if constexpr (lvl == 0) {
      uint32_t bmin = 255u, bmax = 0u;
      static_for<LSPT>([&](auto j) {
        if (g0 + wave + j * SW < g1) {  // uniform
          static_for<LV>([&](auto s) {
            const uint32_t bt = (uint32_t)(cand[j][s] >> 8) >> sh;
            bmin = min(bmin, bt);
            bmax = max(bmax, bt);
          });
        }
      });
      bmin = wave_reduce(bmin, [](uint32_t x, uint32_t y) { return min(x, y); });
      bmax = wave_reduce(bmax, [](uint32_t x, uint32_t y) { return max(x, y); });
      if (bmax >= bmin && bmax - bmin < 8u) {
        for (uint32_t bt = bmin; bt <= bmax; ++bt) {
          int cnt = 0;
          static_for<LSPT>([&](auto j) {
            if (g0 + wave + j * SW < g1) {
              static_for<LV>([&](auto s) {
                cnt += __builtin_popcountll(ballot(((uint32_t)(cand[j][s] >> 8) >> sh) == bt));
              });
            }
          });
          if (lane == 0 && cnt > 0) atomicAdd(&F.hist[bt], cnt);
        }
      } else {
        lanewise = bmax >= bmin;
      }
    }
    if (lanewise) {
      static_for<LSPT>([&](auto j) {
        if (g0 + wave + j * SW < g1) {
          static_for<LV>([&](auto s) {
            const uint32_t v = (uint32_t)(cand[j][s] >> 8);
            if (((uint64_t)(v ^ pre) >> (sh + 8)) == 0u) atomicAdd(&F.hist[(v >> sh) & 0xFFu], 1);
          });
        }
      });
    }
    __syncthreads();
    // wave 0 finds the byte value b: the largest with above + #(byte >= b) >= TC
    if (wave == 0) {
      int h[4];
      static_for<4>([&](auto i) { h[i] = F.hist[255 - (lane * 4 + i)]; });  // descending bytes
      const int ls = h[0] + h[1] + h[2] + h[3];
      int cum = wave_incl_scan(ls) - ls + above;
      int pick = -1, excl = 0;
      static_for<4>([&](auto i) {
        if (pick < 0 && cum + h[i] >= TC) {
          pick = 255 - (lane * 4 + i);
          excl = cum;
        }
        cum += h[i];
      });
      const uint64_t has = ballot(pick >= 0);
      if (lane == 0) F.sel[0] = -1;
      if (has) {
        const int src = __builtin_ctzll(has);
        const int bsel = __shfl(pick, src, kWave);
        const int bex = __shfl(excl, src, kWave);
        if (lane == 0) {
          F.sel[0] = bsel;
          F.sel[1] = bex;
        }
      }
    }
    __syncthreads();
    const int bsel = F.sel[0];
    if (bsel >= 0) {
      pre |= (uint32_t)bsel << sh;
      above = F.sel[1];
    }
    // clear the histogram for the next byte (the reads above are done: one more barrier)
    if (tid < 256) F.hist[tid] = 0;
    __syncthreads();
    if (bsel < 0) pre = 0xFFFFFFFFu;  // marks "fewer than TC candidates"
  });
  }
  if (pre == 0u || pre == 0xFFFFFFFFu) return 2;  // fewer than TC candidates carry a value

  // C. Lists up to 256 keys: the groups whose maximum reaches t (each lane-segment's group
  // maxima name them) go to one list in LDS, a wave reserving its places with one atomic;
  // then each thread takes one listed group, reads its 16 bytes again and stages its
  // elements that reach t. Longer lists: each thread re-reads its own lane-segments'
  // candidate groups that reach t (all loads in flight at once), and the other groups
  // that do where all LV candidates of a lane-segment reach t.
  if constexpr (PL <= 4) {
    int* glist = F.hist;  // the histogram is done with: it holds the list
    constexpr int GCAP = kDistBins;
    uint32_t gsel[LSPT];  // bit q: group q of lane-segment j reaches t
    int cnt = 0;
    static_for<LSPT>([&](auto j) {
      gsel[j] = 0u;
      if (g0 + wave + j * SW < g1) {  // uniform
        static_for<kSegLoads>([&](auto q) {
          const uint32_t im = (gmi[j][q / GPW] >> (16 * (q % GPW))) & (BF ? 0xFFFFu : 0xFFFFFFFFu);
          gsel[j] |= (uint32_t)(im >= pre) << q;
        });
        cnt += __builtin_popcount(gsel[j]);
      }
    });
    {
      const int incl = wave_incl_scan(cnt);
      int base = 0;
      if (lane == kWave - 1 && incl > 0) base = atomicAdd(&F.ng, incl);
      int at = __shfl(base, kWave - 1, kWave) + incl - cnt;
      static_for<LSPT>([&](auto j) {
        uint32_t m = gsel[j];
        const int s0 = (g0 + wave + j * SW) * seg_elems<DT>();
        while (m != 0u) {
          const int q = __builtin_ctz(m);
          m &= m - 1u;
          if (at < GCAP) glist[at] = s0 + (q * kWave + lane) * EPL;
          ++at;
        }
      });
    }
    __syncthreads();
    const int ng = F.ng;
    if (ng > GCAP) {  // more groups than keys the path holds reach t
      floor_img = pre;
      return 2;
    }
    auto elem = [](const u32x4_t& w, auto e) -> float {  // e: a compile-time index
      constexpr int E = decltype(e)::value;
      if constexpr (BF) return (E & 1) ? bf16_hi(w[E >> 1]) : bf16_lo(w[E >> 1]);
      else return __uint_as_float(w[E]);
    };
    for (int r0 = wave * kWave; r0 < ng; r0 += NT) {  // uniform per wave
      const int gi = r0 + lane;
      u32x4_t w = {0u, 0u, 0u, 0u};
      int e0 = V;
      if (gi < ng) {
        e0 = glist[gi];
        w = *(const u32x4_t*)(row + (int64_t)e0 * esz);
      }
      uint32_t k = 0u;
      static_for<EPL>([&](auto e) {
        if (e0 + (int)e < V && img_of<DT>(elem(w, e)) >= pre) k |= 1u << e;
      });
      const int c = __builtin_popcount(k);
      const int incl = wave_incl_scan(c);
      int base = 0;
      if (lane == kWave - 1 && incl > 0) base = atomicAdd(&F.nk, incl);
      int at = __shfl(base, kWave - 1, kWave) + incl - c;
      static_for<EPL>([&](auto e) {
        if (k & (1u << e)) {
          if (at < FL::KCAP) F.keys[at] = sup_key(elem(w, e), (uint32_t)(e0 + (int)e));
          ++at;
        }
      });
    }
  } else {
    {
      constexpr int SL = LSPT * LV;
      static_assert(SL <= 32, "slot mask");
      u32x4_t gw[LSPT][LV];
      uint32_t lst = 0u;  // bit j*LV + s: slot (j, s) is listed
      bool sat_any = false;
      uint32_t satm = 0u;  // bit j: lane-segment j has all LV candidates at or above t
      static_for<LSPT>([&](auto j) {
        const int g = g0 + wave + j * SW;
        const bool vj = g < g1;
        const bool sat = vj && (uint32_t)(cand[j][LV - 1] >> 8) >= pre;
        sat_any |= sat;
        satm |= (uint32_t)sat << j;
        static_for<LV>([&](auto s) {
          gw[j][s] = u32x4_t{0u, 0u, 0u, 0u};
          const int e0 = g * seg_elems<DT>() + ((int)(cand[j][s] & 0xFF) * kWave + lane) * EPL;
          if (vj && (uint32_t)(cand[j][s] >> 8) >= pre && e0 < V) {
            gw[j][s] = *(const u32x4_t*)(row + (int64_t)e0 * esz);
            lst |= 1u << (j * LV + s);
          }
        });
      });
      auto elem = [](const u32x4_t& w, auto e) -> float {  // e: a compile-time index
        constexpr int E = decltype(e)::value;
        if constexpr (BF) return (E & 1) ? bf16_hi(w[E >> 1]) : bf16_lo(w[E >> 1]);
        else return __uint_as_float(w[E]);
      };
      uint32_t keep[LSPT][LV];
      int cnt = 0;
      static_for<LSPT>([&](auto j) {
        static_for<LV>([&](auto s) {
          keep[j][s] = 0u;
          if (ballot((lst >> (j * LV + s)) & 1u) != 0ull) {  // uniform skip
            const int g = g0 + wave + j * SW;
            const int e0 = g * seg_elems<DT>() + ((int)(cand[j][s] & 0xFF) * kWave + lane) * EPL;
            uint32_t k = 0u;
            static_for<EPL>([&](auto e) {
              if (((lst >> (j * LV + s)) & 1u) && e0 + (int)e < V && img_of<DT>(elem(gw[j][s], e)) >= pre)
                k |= 1u << e;
            });
            keep[j][s] = k;
            cnt += __builtin_popcount(k);
          }
        });
      });
      const int incl = wave_incl_scan(cnt);
      int base = 0;
      if (lane == kWave - 1 && incl > 0) base = atomicAdd(&F.nk, incl);
      int at = __shfl(base, kWave - 1, kWave) + incl - cnt;
      static_for<LSPT>([&](auto j) {
        static_for<LV>([&](auto s) {
          if (ballot(keep[j][s] != 0u) != 0ull) {
            const int g = g0 + wave + j * SW;
            const int e0 = g * seg_elems<DT>() + ((int)(cand[j][s] & 0xFF) * kWave + lane) * EPL;
            static_for<EPL>([&](auto e) {
              if (keep[j][s] & (1u << e)) {
                if (at < FL::KCAP) F.keys[at] = sup_key(elem(gw[j][s], e), (uint32_t)(e0 + (int)e));
                ++at;
              }
            });
          }
        });
      });
      // a lane-segment whose LV candidates all reach t may hold more groups that do: their
      // maxima name them, read four at a time
      if (ballot(sat_any) != 0ull) {
        static_for<LSPT>([&](auto j) {
          uint32_t extra = 0u;  // bit q: group q of the lane-segment, not a candidate
          if ((satm >> j) & 1u) {
            static_for<kSegLoads>([&](auto q) {
              const uint32_t im = (gmi[j][q / GPW] >> (16 * (q % GPW))) & (BF ? 0xFFFFu : 0xFFFFFFFFu);
              if (im >= pre) extra |= 1u << q;
            });
            static_for<LV>([&](auto s) { extra &= ~(1u << (uint32_t)(cand[j][s] & 0xFF)); });
          }
          const int s0 = (g0 + wave + j * SW) * seg_elems<DT>();
          while (ballot(extra != 0u) != 0ull) {
            u32x4_t w[4];
            int e0[4];
            static_for<4>([&](auto u) {
              w[u] = u32x4_t{0u, 0u, 0u, 0u};
              e0[u] = V;
              if (extra != 0u) {
                const int q = __builtin_ctz(extra);
                extra &= extra - 1u;
                e0[u] = s0 + (q * kWave + lane) * EPL;
                if (e0[u] < V) w[u] = *(const u32x4_t*)(row + (int64_t)e0[u] * esz);
              }
            });
            uint32_t kp[4];
            int c2 = 0;
            static_for<4>([&](auto u) {
              uint32_t k = 0u;
              static_for<EPL>([&](auto e) {
                if (e0[u] + (int)e < V && img_of<DT>(elem(w[u], e)) >= pre) k |= 1u << e;
              });
              kp[u] = k;
              c2 += __builtin_popcount(k);
            });
            const int inc2 = wave_incl_scan(c2);
            int b2 = 0;
            if (lane == kWave - 1 && inc2 > 0) b2 = atomicAdd(&F.nk, inc2);
            int at2 = __shfl(b2, kWave - 1, kWave) + inc2 - c2;
            static_for<4>([&](auto u) {
              static_for<EPL>([&](auto e) {
                if (kp[u] & (1u << e)) {
                  if (at2 < FL::KCAP) F.keys[at2] = sup_key(elem(w[u], e), (uint32_t)(e0[u] + (int)e));
                  ++at2;
                }
              });
            });
          }
        });
      }
    }
  }
  __syncthreads();
  const int nk = F.nk;
  if (nk > FL::KCAP) floor_img = pre;  // at least TC row elements reach t
  if (nk > FL::KCAP || nk < TC) return 2;

  // D. Lists of 512 keys or more: every wave sorts 256-key slices of the staged keys in
  // registers, then rounds of pairwise merges in LDS keep the top N of each pair (ranking
  // every key against every other would cost nk^2 LDS reads). A merge writes output k of
  // a pair from its co-rank (a binary search over the two sorted inputs, "merge path");
  // each thread holds its outputs in registers until the whole round has read its inputs,
  // so the outputs overwrite them in place.
  if constexpr (PL >= 8) {
    constexpr int QS = 256;                  // keys per slice: 4 per lane
    constexpr int MO = FL::KCAP / NT;        // outputs per thread and round, at most
    const int ns = (nk + QS - 1) / QS;       // slices (<= KCAP / QS)
    for (int sl = wave; sl < ns; sl += SW) {  // uniform per wave
      uint64_t k[QS / kWave];
      static_for<QS / kWave>([&](auto q) {
        const int p = sl * QS + lane * (QS / kWave) + (int)q;
        k[q] = p < nk ? F.keys[p] : 0ull;
      });
      wave_sort_desc<QS / kWave>(k);
      static_for<QS / kWave>([&](auto q) { F.keys[sl * QS + lane * (QS / kWave) + q] = k[q]; });
    }
    __syncthreads();
    // round r: list i starts at i * QS * 2^r
    int nl = ns;
    int stride = QS;
    while (nl > 1) {  // uniform
      const int np = nl / 2;  // pairs merged this round
      uint64_t out[MO];
      int opos[MO];
      static_for<MO>([&](auto u) { opos[u] = -1; });
      // list li holds the top min(N, keys it covers) of the staged keys it covers; pair
      // q's outputs follow those of the pairs before it
      int total = 0;
      auto len_of = [&](int li) {
        const int start = li * stride;
        const int rest = nk - start;  // keys a list covers before capping
        return max(0, min(min(rest, stride), N));
      };
      for (int q = 0; q < np; ++q) total += min(len_of(2 * q) + len_of(2 * q + 1), N);
      static_for<MO>([&](auto u) {
        const int gk = tid + (int)u * NT;  // this thread's output index in the round
        if (gk < total) {
          int q = 0, before = 0;
          while (true) {
            const int cq = min(len_of(2 * q) + len_of(2 * q + 1), N);
            if (gk < before + cq) break;
            before += cq;
            ++q;
          }
          const int kk = gk - before;
          const uint64_t* A = F.keys + (2 * q) * stride;
          const uint64_t* Bv = F.keys + (2 * q + 1) * stride;
          const int na = len_of(2 * q), nb = len_of(2 * q + 1);
          int lo = max(0, kk - nb), hi = min(kk, na);  // A's share of the kk keys above
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (A[mid] > Bv[kk - mid - 1]) lo = mid + 1;
            else hi = mid;
          }
          const int ia = lo, ib = kk - lo;
          const bool fromA = ib >= nb || (ia < na && A[ia] > Bv[ib]);
          out[u] = fromA ? A[ia] : Bv[ib];
          opos[u] = (2 * q) * stride + kk;
        }
      });
      __syncthreads();  // the round's inputs are read
      static_for<MO>([&](auto u) {
        if (opos[u] >= 0) F.keys[opos[u]] = out[u];
      });
      // an odd last list (index nl-1, even) already starts where list (nl-1)/2 of the
      // next round does: it stays in place
      __syncthreads();
      nl = (nl + 1) / 2;
      stride *= 2;
    }
    for (int p = tid; p < N; p += NT) s_sup[p] = (p < TC && p < nk) ? F.keys[p] : 0ull;
    n_sup = TC;
    __syncthreads();
    return 0;
  }
  {
    // H consecutive threads per key (as many as the block holds, up to 8), each counting
    // the larger keys in its share of the list; two keys per read, eight reads in flight
    // (slots past nk hold 0, below every key)
    const int H = nk <= NT / 8 ? 8 : (nk <= NT / 4 ? 4 : (nk <= NT / 2 ? 2 : 1));
    const int nk2 = (nk + 1) >> 1;
    const int len = (nk2 + H - 1) / H;
    const u64x2_t* kp = (const u64x2_t*)F.keys;
    for (int i0 = 0; i0 < nk; i0 += NT / H) {  // uniform
      const int i = i0 + tid / H, h = tid % H;
      const uint64_t my = i < nk ? F.keys[i] : ~0ull;
      const int j1 = min(nk2, (h + 1) * len);
      int r = 0;
      int jj = h * len;
      for (; jj + 8 <= j1; jj += 8) {
        u64x2_t w[8];
        static_for<8>([&](auto u) { w[u] = kp[jj + u]; });
        static_for<8>([&](auto u) { r += (w[u][0] > my) + (w[u][1] > my); });
      }
      for (; jj < j1; ++jj) {
        const u64x2_t w = kp[jj];
        r += (w[0] > my) + (w[1] > my);
      }
      for (int o = 1; o < H; o <<= 1) r += __shfl_xor(r, o, kWave);
      if (i < nk && h == 0 && r < TC) s_sup[r] = my;
    }
  }
  for (int p = TC + tid; p < N; p += NT) s_sup[p] = 0ull;
  n_sup = TC;
  __syncthreads();
  return 0;
}

// LDS of the exact row selection.
template <int PL>
struct ExactLds {
  uint64_t keys[PL * kWave];
  int hist[2][256];
  int wtot[2][16];
  int sel[2];
  int nk, bad;
};

// The top TC keys (value desc, token id asc) of the V values at row (token ids id0 ..
// id0 + V - 1) into s_sup, exactly, where the fast path does not hold (many ties, flat
// rows, long rows), by all SW waves of the block with few registers:
//  1. a radix selection fixes the image t of the TC-th largest value, one byte per pass
//     over the row (re-read; the first pass also flags NaN and +inf), and how many
//     elements equal to t belong to the top TC;
//  2. a last pass stages every element above t and, in token order (a block-wide scan
//     per chunk of the row), that many elements equal to t;
//  3. wave 0 sorts the staged keys.
// Elements below floor_img (an image the TC-th largest value is known to reach) are not
// counted. Returns 1 for a row holding NaN or +inf, else 0; uniform over the block.
template <int DT, int PL, int SW>
__device__ __forceinline__ int row_select_exact(const char* row, int id0, int V, int TC, uint32_t floor_img,
                                                ExactLds<PL>& X, uint64_t* s_sup, int& n_sup) {
  constexpr bool BF = DT == VRT_BF16;
  constexpr int EPL = BF ? 8 : 4;             // elements per 16-byte vector
  constexpr int IB = BF ? 16 : 32;            // image bits
  constexpr uint32_t PINF = BF ? 0xFF80u : 0xFF800000u;  // image of +inf
  constexpr uint32_t NINF = BF ? 0x007Fu : 0x007FFFFFu;  // image of -inf
  constexpr int NT = SW * kWave;
  constexpr int N = PL * kWave;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int nv = (V + EPL - 1) / EPL;
  const int take = min(TC, V);
  // images of vector v's elements; 0 marks an element past V (a valid element with image
  // 0 is a NaN, which flags the row)
  auto images = [&](int v, uint32_t (&im)[EPL]) {
    const u32x4_t d = *(const u32x4_t*)(row + (int64_t)v * 16);
    static_for<EPL>([&](auto e) {
      uint32_t x;
      if constexpr (BF) {
        const uint32_t h = (d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        x = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
      } else {
        x = ord32(__uint_as_float(d[(int)e]));
      }
      im[e] = v * EPL + (int)e < V ? x : 0u;
    });
  };
  if (tid < 256) {
    X.hist[0][tid] = 0;
    X.hist[1][tid] = 0;
  }
  if (tid == 0) {
    X.nk = 0;
    X.bad = 0;
  }
  __syncthreads();

  // 1.
  uint32_t pre = 0u;  // the image bits fixed so far
  int need = take;    // elements matching pre still to take
  bool bad = false;
  static_for<IB / 8>([&](auto lvl) {
    constexpr int sh = IB - 8 * (lvl + 1);
    int* H = X.hist[lvl & 1];
    if (lvl >= 1 && tid < 256) X.hist[(lvl + 1) & 1][tid] = 0;  // last read two bytes ago
    bool nf = false;
    for (int v = tid; v < nv; v += NT) {
      uint32_t im[EPL];
      images(v, im);
      static_for<EPL>([&](auto e) {
        const uint32_t x = im[e];
        // a row element with image 0 is a NaN (fp32 rows map NaN to 0)
        if (lvl == 0) nf |= v * EPL + (int)e < V && (x == 0u || x >= PINF || x < NINF);
        if (x >= floor_img && x != 0u && ((uint64_t)(x ^ pre) >> (sh + 8)) == 0u)
          atomicAdd(&H[(x >> sh) & 0xFF], 1);
      });
    }
    if (lvl == 0 && ballot(nf) != 0ull && lane == 0) X.bad = 1;
    __syncthreads();
    if (lvl == 0 && X.bad) bad = true;
    if (!bad) {
      // wave 0: the largest byte b with #(matching elements with byte >= b) >= need
      if (wave == 0) {
        int h[4];
        static_for<4>([&](auto i) { h[i] = H[255 - (lane * 4 + i)]; });
        const int ls = h[0] + h[1] + h[2] + h[3];
        int cum = wave_incl_scan(ls) - ls;
        int pick = -1, excl = 0;
        static_for<4>([&](auto i) {
          if (pick < 0 && cum + h[i] >= need) {
            pick = 255 - (lane * 4 + i);
            excl = cum;
          }
          cum += h[i];
        });
        const uint64_t has = ballot(pick >= 0);  // never empty: need <= matching elements
        const int src = has ? __builtin_ctzll(has) : 0;
        const int bsel = __shfl(pick, src, kWave);
        const int bex = __shfl(excl, src, kWave);
        if (lane == 0) {
          X.sel[0] = bsel < 0 ? 0 : bsel;
          X.sel[1] = need - bex;
        }
      }
      __syncthreads();
      pre |= (uint32_t)X.sel[0] << sh;
      need = X.sel[1];
    }
  });
  if (bad) return 1;

  // 2.
  auto stage = [&](uint32_t x, int id) {
    const int at = atomicAdd(&X.nk, 1);
    if (at < N) X.keys[at] = sup_key(value_of<DT>(x), (uint32_t)id);
  };
  int rem = need;  // elements equal to t still to take
  for (int c0 = 0, it = 0; c0 < nv; c0 += NT, ++it) {
    const int v = c0 + tid;
    uint32_t im[EPL];
    int nt = 0;
    if (v < nv) {
      images(v, im);
      static_for<EPL>([&](auto e) {
        if (im[e] > pre) stage(im[e], id0 + v * EPL + (int)e);
        nt += im[e] == pre;
      });
    }
    if (rem > 0) {  // uniform
      const int incl = wave_incl_scan(nt);
      if (lane == kWave - 1) X.wtot[it & 1][wave] = incl;
      __syncthreads();
      int off = incl - nt, tot = 0;
      static_for<SW>([&](auto w) {
        const int t = X.wtot[it & 1][w];
        off += (int)w < wave ? t : 0;
        tot += t;
      });
      if (nt > 0 && off < rem) {
        static_for<EPL>([&](auto e) {
          if (im[e] == pre) {
            if (off < rem) stage(im[e], id0 + v * EPL + (int)e);
            ++off;
          }
        });
      }
      rem -= tot;
    }
  }
  __syncthreads();

  // 3.
  if (wave == 0) {
    const int nk = min(X.nk, N);
    uint64_t k[PL];
    static_for<PL>([&](auto s) {
      const int p = lane * PL + s;
      k[s] = p < nk ? X.keys[p] : 0ull;
    });
    wave_sort_desc<PL>(k);
    int cnt = 0;
    static_for<PL>([&](auto s) {
      const int p = lane * PL + s;
      const uint64_t x = p < TC ? k[s] : 0ull;
      s_sup[p] = x;
      cnt += x != 0ull;
    });
    n_sup = wave_sum_i(cnt);
  }
  return 0;
}

// Expansion of one parent by wave 0 (RheoSampling key design 2), BS support ranks
// per lane: lane l owns ranks [l*BS, l*BS + BS).
template <int BS>
__device__ __forceinline__ void expand_row(const BArgs& a, int b, int node, float sp, int n_sup,
                                           const uint64_t* s_buf, float* s_q, int64_t ncb, int cbase,
                                           int64_t ktb) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const float M = sup_key_val(s_buf[0]);
  const int m = c.probe ? c.m : 0;
  // the probe's tail starts after the deterministic children: the top m, or, probe last,
  // the fillers too
  const int t0 = c.order == VRT_PROBE_LAST ? min(c.K - 1, n_sup) : m;
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
  // E (the fp32 pairwise sum) and the tempered tail's mass in one butterfly. The tail
  // mass stays unnormalised: the tempered normaliser cancels out of q~ = q_T / z_T and
  // out of the draw (u z_T against partial sums of q_T, all scaled alike).
  double tl = 0.0;
#pragma unroll
  for (int k = 0; k < BS; ++k)
    if (lane * BS + k >= t0) tl += et[k];
  float te;
  {
    float t[BS];
#pragma unroll
    for (int k = 0; k < BS; ++k) t[k] = e[k];
#pragma unroll
    for (int w = BS >> 1; w >= 1; w >>= 1)
#pragma unroll
      for (int k = 0; k < w; ++k) t[k] = t[2 * k] + t[2 * k + 1];
    te = t[0];
  }
  double zT = tl;
  te += xchg<1>(te), zT += xchg<1>(zT);
  te += xchg<2>(te), zT += xchg<2>(zT);
  te += xchg<4>(te), zT += xchg<4>(zT);
  te += xchg<8>(te), zT += xchg<8>(zT);
  te += xchg<16>(te), zT += xchg<16>(zT);
  te += xchg<32>(te), zT += xchg<32>(zT);
  const float E = te;
  float qt[BS];
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    const int r = lane * BS + k;
    const float q = e[k] / E;
    qt[k] = r < t0 ? 0.0f : q;
    s_q[r] = q;
  }
  const float zr = pairwise(qt);
  wave_sync();

  int js = -1;
  float proxy = 0.0f;
  if (c.probe && n_sup > t0 && zT > 0.0) {
    const double u =
        (double)uniform24(a.seed, (uint32_t)(node + 1), c.tree_base + (uint32_t)b, a.step, kPurposeProbe);
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
          if (r >= t0 && pick < 0) {
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
        if (r >= t0 && r < n_sup && et[k] > 0.0) last = r;
      }
      for (int o = 1; o < kWave; o <<= 1) last = max(last, __shfl_xor(last, o, kWave));
      pick = last;
    }
    js = pick;
    if (t0 >= 1) {  // the last deterministic child's q, capped by the raw mass after it
      const float qm = s_q[t0 - 1];
      proxy = qm < zr ? qm : zr;
    } else {
      const float t1 = s_q[0] + c.eps_m0;
      proxy = t1 < 1.0f ? t1 : 1.0f;
    }
  }

  // tail table of this row: ranks t0.. with q~ = q_T / z_T
  const int ntail = (js >= 0) ? n_sup - t0 : 0;
  if (lane == 0) a.t.row_tail_n[ktb] = ntail;
#pragma unroll
  for (int k = 0; k < BS; ++k) {
    const int r = lane * BS + k;
    if (r >= t0 && r < t0 + ntail) {
      a.t.row_tail_id[ktb * c.TC + (r - t0)] = (int)sup_key_id(s_buf[r]);
      a.t.row_tail_q[ktb * c.TC + (r - t0)] = (float)(et[k] / zT);
    }
  }

  // child slots: DET ranks, the probe, then fillers in rank order. Lane s writes slot s.
  int r_of_slot = -1, kind = 0;
  {
    const int m_det = c.probe ? min(m, n_sup) : 0;
    const int s = lane;
    if (!c.probe) {
      if (s < n_sup) r_of_slot = s, kind = VRT_DET;
    } else if (s < m_det) {
      r_of_slot = s, kind = VRT_DET;
    } else if (c.order == VRT_PROBE_LAST) {  // the fillers (ranks up to t0), then the probe
      if (s < t0) r_of_slot = s, kind = VRT_FILL;
      else if (js >= 0 && s == t0) r_of_slot = js, kind = VRT_PROBE;
    } else if (js >= 0 && s == m_det) {
      r_of_slot = js, kind = VRT_PROBE;
    } else {
      const int f = s - m_det - (js >= 0 ? 1 : 0);  // filler index
      int r = m + f;
      if (js >= 0 && r >= js) ++r;
      if (r < n_sup) r_of_slot = r, kind = VRT_FILL;
    }
  }
  if (lane < c.K) {  // device-coherent: the layer's ranking block reads them
    const int64_t ci = ncb + cbase + lane;
    if (r_of_slot >= 0) {
      st_dev(&a.t.cand_token[ci], (int)sup_key_id(s_buf[r_of_slot]));
      st_dev(&a.t.cand_parent[ci], node);
      st_dev(&a.t.cand_score[ci], sp * (kind == VRT_PROBE ? proxy : s_q[r_of_slot]));
      st_dev(&a.t.cand_kind[ci], kind);
    } else {
      st_dev(&a.t.cand_kind[ci], 0);
    }
  }
}

// Start of a row block: at layer 0 a new step begins (every candidate of the previous
// one is forgotten and SMART's state reset, by the block of tree b's row 0, wave 0).
// Returns the node the row expands, or -2 after clearing the row's candidate slots
// (no parent at this frontier position).
// Layer 0, wave 0 of the block that expands the root: clears the later layers'
// candidate slots and starts the SMART state. (With the root row split over several
// blocks the block that expands it is known only after the join, and it is the one that
// reads the state.)
__device__ __forceinline__ void init_tree(const BArgs& a, int b) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  for (int t = c.K + lane; t < c.NC; t += kWave) a.t.cand_kind[ncb + t] = 0;
  if (lane == 0) {
    double* sm = a.t.smart + (int64_t)b * 8;
    sm[0] = 0.0; sm[1] = 1.0; sm[2] = 1.0; sm[3] = 0.0; sm[4] = 0.0;
    sm[5] = sm[6] = sm[7] = 0.0;
  }
}

__device__ __forceinline__ int begin_row(const BArgs& a, int b, int j) {
  const Cfg& c = a.c;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  if (a.layer == 0 && wave == 0 && a.split == 1) init_tree(a, b);
  const int node = row_node(a, b, j);
  if (node == -2 && wave == 0) {
    const int cbase = layer_base(c, a.layer) + j * c.K;
    for (int s = lane; s < c.K; s += kWave) st_dev(&a.t.cand_kind[ncb + cbase + s], 0);
    if (lane == 0) a.t.row_tail_n[(int64_t)b * c.NR + row_base(c, a.layer) + j] = 0;
  }
  return node;
}

// End of a row block, wave 0: the row's status (non-finite values, no finite value),
// then the parent's expansion from its support s_sup (n_sup keys).
template <int PL>
__device__ __forceinline__ void end_row(const BArgs& a, int b, int j, int node, float sp, int n_sup,
                                        bool any_bad, const uint64_t* s_sup, float* s_q) {
  const Cfg& c = a.c;
  const int lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  const int cbase = layer_base(c, a.layer) + j * c.K;
  const int64_t ktb = (int64_t)b * c.NR + row_base(c, a.layer) + j;
  uint32_t st = any_bad ? VRT_ST_DRAFT_NONFINITE : 0u;
  const float M = n_sup > 0 ? sup_key_val(s_sup[0]) : -INFINITY;
  if (n_sup == 0 || M == -INFINITY) st |= VRT_ST_DRAFT_EMPTY;
  if (st) {
    if (lane == 0 && a.stats) atomicOr(a.stats + (int64_t)b * 8, st);
    for (int s = lane; s < c.K; s += kWave) st_dev(&a.t.cand_kind[ncb + cbase + s], 0);
    if (lane == 0) a.t.row_tail_n[ktb] = 0;
    return;
  }
  expand_row<PL>(a, b, node, sp, n_sup, s_sup, s_q, ncb, cbase, ktb);
}

// Ranking fused into the layer's row blocks (wave 0 of each): every block writes its
// candidates device-coherently, waits for the stores and counts itself done on tree
// b's layer_sync word; the last one reads the layer's candidates device-coherently,
// sorts their keys in its registers and ranks them. Layer 0 has one row block per tree.
// The ranking block sets the word back to 0 for the next layer; layer 0 starts it at 0.
constexpr int kRankFused = 256;  // children per layer the fused ranking takes

__device__ void rank_sorted(const Cfg& c, const TreePtrs& t, int layer, int b, const uint64_t* keys,
                            int span);

template <int RL>
__device__ __forceinline__ void rank_wave(const BArgs& a, int b, uint64_t* s_rank) {
  const Cfg& c = a.c;
  const TreePtrs& t = a.t;
  const int lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  const int base = layer_base(c, a.layer);
  const int span = layer_span(c, a.layer);
  uint64_t k[RL];
  static_for<RL>([&](auto s) {
    const int i = lane * RL + s;
    uint64_t x = 0ull;
    if (i < span && (ld_dev(&t.cand_kind[ncb + base + i]) & 0xFF) != 0)
      x = node_key(ld_dev(&t.cand_score[ncb + base + i]), (uint32_t)(base + i));
    k[s] = x;
  });
  wave_sort_desc<RL>(k);
  if (c.mode == VRT_MODE_TOPR) {
    // the top W keys are positions 0 .. W-1 of the sorted list (lane * RL + s); the
    // nonzero keys form its prefix
    int nz = 0;
    static_for<RL>([&](auto s) { nz += __builtin_popcountll(ballot(k[s] != 0ull)); });
    const int nf = a.layer + 1 < c.D ? min(c.W, nz) : 0;
    int* front = t.front + (int64_t)b * c.FP;
    static_for<RL>([&](auto s) {
      const int p = lane * RL + s;
      if (p < nf) front[p] = (int)(0xFFFFFFFFu - (uint32_t)k[s]);
    });
    if (lane == 0) t.n_front[b] = nf;
    return;
  }
  static_for<RL>([&](auto s) { s_rank[lane * RL + s] = k[s]; });
  wave_sync();
  if (lane == 0) rank_sorted(c, t, a.layer, b, s_rank, span);
}

__device__ __forceinline__ void rank_if_last(const BArgs& a, int b, uint64_t* s_rank) {
  const int lane = lane_id();
  const int rows = a.rpt;
  if (rows > 1) {
    wait_stores();
    int old = 0;
    if (lane == 0) old = atomicAdd(&a.t.layer_sync[b], 1);
    old = __shfl(old, 0, kWave);
    if (old != rows - 1) return;
  }
  const int span = layer_span(a.c, a.layer);
  if (span <= kWave) rank_wave<1>(a, b, s_rank);
  else if (span <= 2 * kWave) rank_wave<2>(a, b, s_rank);
  else rank_wave<4>(a, b, s_rank);
  if (lane == 0) a.t.layer_sync[b] = 0;
}

// A row split over P blocks (2 or 4), wave 0 of each: every block has the top TC of its
// part of the row in s_sup (n_sup keys, sorted); the row's top TC are among the P lists.
// Each block writes its list and status device-coherently, waits for the stores and
// counts itself on the row's row_sync word, which holds this launch's tag (the low 32
// bits of its epoch) above the count: a compare-and-swap puts the tag in with count 1 if
// the word holds another tag (earlier launches, or whatever the blob held: no initial
// value is needed), else adds 1; each failed swap means another block counted, so a
// block retries at most P - 1 times (the loop's bound only matters if another launch used
// the same blob at the same time, which the ABI rules out). The block whose count is P
// is the last: it sets the
// word back to 0 (a launch repeated with the same tag, a replayed graph, starts afresh),
// merges the other lists into its own and combines the status; the others are done
// (false).
constexpr int kMaxParts = 4;

template <int PL>
__device__ __forceinline__ bool join_parts(const BArgs& a, int b, int j, int h, int P, int& n_sup,
                                           int& any_bad, uint64_t* s_sup) {
  const Cfg& c = a.c;
  constexpr int N = PL * kWave;
  const int lane = lane_id();
  const int64_t r = (int64_t)b * c.FP + j;
  uint64_t* mine = a.half_keys + (r * kMaxParts + h) * N;
  static_for<PL>([&](auto s) { st_dev64(&mine[lane * PL + s], s_sup[lane * PL + s]); });
  if (lane == 0) st_dev(&a.half_meta[r * kMaxParts + h], n_sup | (any_bad << 30));
  wait_stores();
  int last = 0;
  if (lane == 0) {
    const unsigned long long tag = (unsigned long long)(uint32_t)a.epoch << 32;
    unsigned long long* word = (unsigned long long*)&a.t.row_sync[r];
    unsigned long long w = (unsigned long long)ld_dev64(&a.t.row_sync[r]);
    for (int tries = 0; tries <= kMaxParts; ++tries) {
      const unsigned long long want = (w & 0xFFFFFFFF00000000ull) == tag ? w + 1ull : tag | 1ull;
      const unsigned long long got = atomicCAS(word, w, want);
      if (got == w) {
        last = (int)(want & 0xFFFFFFFFull) == P;
        break;
      }
      w = got;
    }
  }
  last = __shfl(last, 0, kWave);
  if (!last) return false;
  if (lane == 0) st_dev64(&a.t.row_sync[r], 0ull);
  uint64_t top[PL];
  static_for<PL>([&](auto s) { top[s] = s_sup[lane * PL + s]; });
  for (int o = 0; o < P; ++o) {
    if (o == h) continue;
    const uint64_t* other = a.half_keys + (r * kMaxParts + o) * N;
    const int om = ld_dev(&a.half_meta[r * kMaxParts + o]);
    uint64_t add[PL];
    static_for<PL>([&](auto s) { add[s] = ld_dev64(&other[lane * PL + s]); });
    wave_merge_top<PL>(top, add);
    n_sup = min(c.TC, n_sup + (om & 0xFFFF));
    any_bad |= (om >> 30) & 1;
  }
  static_for<PL>([&](auto s) {
    const int p = lane * PL + s;
    s_sup[p] = p < c.TC ? top[s] : 0ull;
  });
  wave_sync();
  return true;
}

// Part h of S of frontier position j of tree b, by one block; then wave 0 expands the
// parent: the row-wide path, the exact path behind it (ties, flat rows, rows longer
// than the row-wide path covers). Waves 1.. return once the row is read.
template <int DT, int PL, bool SPLIT>
__device__ __forceinline__ void select_expand_row(const BArgs& a, int b, int j, int h, int S) {
  const Cfg& c = a.c;
  const int wave = threadIdx.x >> 6;
  constexpr int N = PL * kWave;
  __shared__ uint64_t s_rank[kRankFused];
  const int node = begin_row(a, b, j);
  if (node == -2) {
    if (wave == 0 && a.fuse_rank && h == 0) rank_if_last(a, b, s_rank);
    return;
  }
  // the parent's path score, read now (wave 0 uses it at the end)
  const float sp = node < 0 ? 1.0f : a.t.cand_score[(int64_t)b * c.NC + node];
  constexpr int SW = kSelWaves;
  constexpr int LSPT = seg_per_wave<DT>();
  union Sel {
    FastLds<DT, PL> f;
    ExactLds<PL> x;
  };
  __shared__ __align__(16) char s_raw[sizeof(Sel)];
  __shared__ uint64_t s_sup[N];  // the support: top trunc keys, zero-padded
  __shared__ float s_q[N];
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + ((int64_t)b * a.tstride + (int64_t)j * a.ld) * esz;
  const int G = (c.V + seg_elems<DT>() - 1) / seg_elems<DT>();
  int n_sup = 0;
  Sel& P = *(Sel*)s_raw;
  int path = 2;
  uint32_t floor_img = 0u;  // the TC-th largest row value's image is at least this
  const int Gh = (G + S - 1) / S;  // this block's segments: [g0, g1)
  const int g0 = h * Gh, g1 = min(G, g0 + Gh);
  if (g1 - g0 <= LSPT * SW) path = row_select_fast<DT, PL, SW, LSPT>(row, g0, g1, c.V, c.TC, P.f, s_sup, n_sup, floor_img);
  if (path == 2) {
    __syncthreads();  // s_raw changes hands
    const int e0 = g0 * seg_elems<DT>(), e1 = min(c.V, g1 * seg_elems<DT>());
    path = row_select_exact<DT, PL, SW>(row + (int64_t)e0 * esz, e0, e1 - e0, c.TC, floor_img, P.x, s_sup, n_sup);
  }
  int any_bad = path == 1;
  if (wave != 0) return;
  wave_sync();
  if (SPLIT && S > 1) {
    if (!join_parts<PL>(a, b, j, h, S, n_sup, any_bad, s_sup)) return;
    if (a.layer == 0) init_tree(a, b);
  }
  end_row<PL>(a, b, j, node, sp, n_sup, any_bad != 0, s_sup, s_q);
  if (a.fuse_rank) rank_if_last(a, b, s_rank);
}

// The rows of a compact grid (a layer whose frontier may hold far fewer than FP parents
// per tree, as SMART's do): tree b's expanded rows are items pre[b] .. pre[b+1]-1 of a
// tree-major list, and a grid of fewer blocks than B * FP walks the list. Rows that no
// block takes hold no children: layer 0 cleared every later candidate slot.
constexpr int kCompactTrees = kSelWaves * kWave;  // trees a compact grid takes

// pre[0 .. B] in LDS from the frontier sizes (all threads; B <= kCompactTrees).
__device__ __forceinline__ int compact_prefix(const BArgs& a, int* pre) {
  __shared__ int s_wsum[kSelWaves];
  const Cfg& c = a.c;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  int x = tid < c.B ? min(max(a.t.n_front[tid], 0), c.FP) : 0;
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_wsum[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += s_wsum[w];
  if (tid < c.B) pre[tid + 1] = x;
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  return pre[c.B];
}

// Tree and frontier position of item k of the compact list (block-uniform).
__device__ __forceinline__ void compact_item(const BArgs& a, const int* pre, int k, int& b, int& j) {
  int lo = 0, hi = a.c.B - 1;  // the last tree whose rows start at or before item k
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  b = __builtin_amdgcn_readfirstlane(lo);
  j = __builtin_amdgcn_readfirstlane(k - pre[lo]);
}

// One block per expanded parent (or per part of one: split rows, the mixed grid), or a
// compact grid over the expanded rows.
template <int DT, int PL, bool SPLIT>
__global__ __launch_bounds__(kSelWaves * kWave)
__attribute__((amdgpu_waves_per_eu(PL == 2 ? 4 : 2, 8))) void k_select_expand(const BArgs a) {
  int S = SPLIT ? 2 : 1, j = blockIdx.x / S, h = blockIdx.x % S, b = blockIdx.y;
  if (SPLIT && a.mixed > 0) {
    // rows r = b * rpt + j below `mixed` are whole, the others split; the halves come
    // first in the grid: a CU's older waves win its memory pipeline, and a half that
    // streams beside a whole row must not finish last
    const int k = blockIdx.x, P = a.parts;
    const int nh = P * (a.c.B * a.rpt - a.mixed);  // blocks of split rows
    const bool whole = k >= nh;
    const int r = whole ? k - nh : a.mixed + k / P;
    S = whole ? 1 : P;
    h = whole ? 0 : k % P;
    b = r / a.rpt;
    j = r - b * a.rpt;
  }
  const bool compact = !SPLIT && a.compact > 0;
  __shared__ int s_pre[kCompactTrees + 1];
  int total = 0;
  if (compact) {
    total = __builtin_amdgcn_readfirstlane(compact_prefix(a, s_pre));
    // the list for the kernel after this one, which ranks while the frontier sizes change
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i <= a.c.B; i += blockDim.x) a.cpre[i] = s_pre[i];
    if ((int)blockIdx.x >= total) return;
    compact_item(a, s_pre, blockIdx.x, b, j);
  }
  select_expand_row<DT, PL, SPLIT>(a, b, j, h, S);
}

// Rows of a compact list beyond the first a.compact (one per block of the compact grid):
// the blocks of this grid take them in turn. A kernel of its own, so that the loop's
// register demand stays out of the one-row kernel; with no such rows it only reads the
// frontier sizes.
template <int DT, int PL>
__global__ __launch_bounds__(kSelWaves * kWave)
__attribute__((amdgpu_waves_per_eu(PL == 2 ? 4 : 2, 8))) void k_select_rest(const BArgs a) {
  __shared__ int s_pre[kCompactTrees + 1];
  const int total = __builtin_amdgcn_readfirstlane(compact_prefix(a, s_pre));
  for (int k = a.compact + blockIdx.x; k < total; k += gridDim.x) {
    int b, j;
    compact_item(a, s_pre, k, b, j);
    select_expand_row<DT, PL, false>(a, b, j, 0, 1);
    __syncthreads();  // the block's LDS changes hands
  }
}

// ---------------------------------------------------------------------------------
// Dense expansion (trunc = VRT_DENSE): the untruncated baseline of the support-size
// ablation, whose support is the whole vocabulary. One 8-wave block per parent:
//  1. the row's K best keys (value desc, token id asc) by the selection above;
//  2. one pass over the row in 512-element chunks (the waves take consecutive runs of
//     chunks, 8 consecutive elements per lane): per chunk the fp32 pairwise sum of the
//     ranking exponentials over the chunk and over its tail tokens (the deterministic
//     children excluded), and the fp64 sum of the tempered tail values;
//  3. the chunk sums combine along the zero-padded pairwise tree in token-id order
//     (E, E_tail, z = E_tail / E); the probe is drawn by inverse CDF in token-id order:
//     its chunk from a scan of the chunk sums, its token from one re-read of the chunk;
//  4. the K child slots as on a truncated support; no tail table is written.
constexpr int kDC = 512;                       // elements per chunk
constexpr int kDenseChunks = (1 << 20) / kDC;  // chunks of the largest vocabulary

struct DenseLds {
  float e[kDenseChunks];   // per chunk: pairwise sum of exp_rank(x - M)
  float et[kDenseChunks];  // the same over the chunk's tail tokens
  double z[kDenseChunks];  // per chunk: sum of exp((x - M)/T) over its tail tokens
  int det[32];             // tokens of the deterministic children (ranks < t0)
  int n_sup, bad;
};

// The 8 values of a lane in chunk c (elements c*kDC + 8*lane ..), -inf at and past V.
template <int DT>
__device__ __forceinline__ void dense_load(const char* row, int c, int V, float (&x)[8]) {
  const int e0 = c * kDC + lane_id() * 8;
  if constexpr (DT == VRT_BF16) {
    u32x4_t w = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
    if (e0 < V) w = *(const u32x4_t*)(row + (int64_t)e0 * 2);
    static_for<4>([&](auto k) {
      x[2 * k] = bf16_lo(w[(int)k]);
      x[2 * k + 1] = bf16_hi(w[(int)k]);
    });
  } else {
    static_for<2>([&](auto h) {
      u32x4_t w = {0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u};
      if (e0 + 4 * h < V) w = *(const u32x4_t*)(row + (int64_t)(e0 + 4 * h) * 4);
      static_for<4>([&](auto k) { x[4 * h + k] = __uint_as_float(w[(int)k]); });
    });
  }
  if (e0 + 8 > V)
    static_for<8>([&](auto k) {
      if (e0 + (int)k >= V) x[k] = -INFINITY;
    });
}

// Whether token v is one of the n deterministic children (wave-uniform list in LDS).
__device__ __forceinline__ bool dense_is_det(const DenseLds& L, int n, int v) {
  bool d = false;
  for (int i = 0; i < n; ++i) d |= L.det[i] == v;
  return d;
}

// The tail part of a lane's 8 values and whether its chunk holds a deterministic child.
__device__ __forceinline__ bool dense_chunk_has_det(const DenseLds& L, int n, int c) {
  bool d = false;
  for (int i = 0; i < n; ++i) d |= (L.det[i] >= c * kDC) && (L.det[i] < (c + 1) * kDC);
  return d;
}

template <int DT>
__global__ __launch_bounds__(8 * kWave) void k_dense_expand(const BArgs a) {
  const Cfg& c = a.c;
  const int j = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int lane = lane_id();
  constexpr int SW = 8, PL = 2;
  constexpr int LSPT = seg_per_wave<DT>();
  __shared__ uint64_t s_rank[kRankFused];
  const int node = begin_row(a, b, j);
  if (node == -2) {
    if (wave == 0 && a.fuse_rank) rank_if_last(a, b, s_rank);
    return;
  }
  const float sp = node < 0 ? 1.0f : a.t.cand_score[(int64_t)b * c.NC + node];
  union Sel {
    FastLds<DT, PL> f;
    ExactLds<PL> x;
  };
  __shared__ __align__(16) char s_raw[sizeof(Sel)];
  __shared__ uint64_t s_sup[PL * kWave];
  __shared__ DenseLds L;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + ((int64_t)b * a.tstride + (int64_t)j * a.ld) * esz;
  const int64_t ncb = (int64_t)b * c.NC;
  const int cbase = layer_base(c, a.layer) + j * c.K;
  const int64_t ktb = (int64_t)b * c.NR + row_base(c, a.layer) + j;
  const int TK = min(c.K, c.V);  // ranks the slots can use

  // 1. the K best keys and the row maximum
  {
    Sel& P = *(Sel*)s_raw;
    const int G = (c.V + seg_elems<DT>() - 1) / seg_elems<DT>();
    int n_sup = 0, path = 2;
    uint32_t floor_img = 0u;
    if (G <= LSPT * SW) path = row_select_fast<DT, PL, SW, LSPT>(row, 0, G, c.V, TK, P.f, s_sup, n_sup, floor_img);
    if (path == 2) {
      __syncthreads();
      path = row_select_exact<DT, PL, SW>(row, 0, c.V, TK, floor_img, P.x, s_sup, n_sup);
    }
    if (tid == 0) {
      L.n_sup = n_sup;
      L.bad = path == 1;
    }
  }
  __syncthreads();
  const int n_sup = L.n_sup;
  const float M = n_sup > 0 ? sup_key_val(s_sup[0]) : -INFINITY;
  uint32_t st = L.bad ? VRT_ST_DRAFT_NONFINITE : 0u;
  if (n_sup == 0 || M == -INFINITY) st |= VRT_ST_DRAFT_EMPTY;
  if (st) {
    if (wave == 0) {
      if (lane == 0 && a.stats) atomicOr(a.stats + (int64_t)b * 8, st);
      for (int s = lane; s < c.K; s += kWave) st_dev(&a.t.cand_kind[ncb + cbase + s], 0);
      if (lane == 0) a.t.row_tail_n[ktb] = 0;
      if (a.fuse_rank) rank_if_last(a, b, s_rank);
    }
    return;
  }
  const int m = c.probe ? c.m : 0;
  const int t0 = c.order == VRT_PROBE_LAST ? min(c.K - 1, c.V) : m;  // deterministic ranks
  if (tid < t0) L.det[tid] = (int)sup_key_id(s_sup[tid]);
  __syncthreads();

  // 2. chunk sums; wave w takes chunks [w*S, (w+1)*S) of the padded chunk range
  const int NCH = (c.V + kDC - 1) / kDC;
  const int NCP = max(1, next_pow2(c.V) / kDC);  // chunks of the zero-padded row
  const int S = NCP >= SW ? NCP / SW : 1;
  const double invT = (double)c.invT;
  for (int ci = wave * S; ci < min(NCP, (wave + 1) * S); ++ci) {
    float e = 0.0f, et = 0.0f;
    double z = 0.0;
    if (ci < NCH) {
      float x[8];
      dense_load<DT>(row, ci, c.V, x);
      const bool hd = dense_chunk_has_det(L, t0, ci);
      float ex[8], tx[8];
      double zl = 0.0;
      static_for<8>([&](auto k) {
        ex[k] = exp_rank(x[k] - M);
        const bool tail = !hd || !dense_is_det(L, t0, ci * kDC + lane * 8 + (int)k);
        tx[k] = tail ? ex[k] : 0.0f;
        zl += tail ? dense_tempered(x[k], M, invT) : 0.0;
      });
      // pairwise inside the lane's 8, then across lanes
      static_for<4>([&](auto k) { ex[k] = ex[2 * k] + ex[2 * k + 1]; tx[k] = tx[2 * k] + tx[2 * k + 1]; });
      static_for<2>([&](auto k) { ex[k] = ex[2 * k] + ex[2 * k + 1]; tx[k] = tx[2 * k] + tx[2 * k + 1]; });
      e = wave_sum(ex[0] + ex[1]);
      et = wave_sum(tx[0] + tx[1]);
      z = wave_sum(zl);
    }
    if (lane == 0) {
      L.e[ci] = e;
      L.et[ci] = et;
      L.z[ci] = z;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // 3. E and E_tail along the pairwise tree: in-place levels down to 64 chunk sums, then
  //    across lanes
  for (int w = NCP >> 1; w >= kWave; w >>= 1) {
    for (int i = lane; i < w; i += kWave) {
      L.e[i] = L.e[2 * i] + L.e[2 * i + 1];
      L.et[i] = L.et[2 * i] + L.et[2 * i + 1];
    }
    wave_sync();
  }
  const int top = min(NCP, kWave);
  const float E = wave_sum(lane < top ? L.e[lane] : 0.0f);
  const float Et = wave_sum(lane < top ? L.et[lane] : 0.0f);
  const float zr = Et / E;
  // tempered tail mass and the chunk the draw falls in (lane l scans a run of chunks)
  const int CPL = (NCH + kWave - 1) / kWave;
  double zl = 0.0;
  for (int i = lane * CPL; i < min(NCH, (lane + 1) * CPL); ++i) zl += L.z[i];
  const double incl = wave_incl_scan(zl);
  const double zT = __shfl(incl, kWave - 1, kWave);

  int probe = -1;
  float proxy = 0.0f;
  auto qraw = [&](int r) { return exp_rank(sup_key_val(s_sup[r]) - M) / E; };
  if (c.probe && c.V > t0 && zT > 0.0) {
    const double u =
        (double)uniform24(a.seed, (uint32_t)(node + 1), c.tree_base + (uint32_t)b, a.step, kPurposeProbe);
    const double tgt = u * zT;
    // the chunk: first whose inclusive prefix passes tgt (else the last with mass)
    int ch = -1;
    double before = 0.0;
    const uint64_t hit = ballot(zl > 0.0 && tgt < incl);
    const int src = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(ballot(zl > 0.0));
    if (lane == src) {
      double cum = incl - zl;
      for (int i = lane * CPL; i < min(NCH, (lane + 1) * CPL); ++i) {
        if (L.z[i] > 0.0) {
          ch = i;
          before = cum;
          if (tgt < cum + L.z[i]) break;
        }
        cum += L.z[i];
      }
    }
    ch = __shfl(ch, src, kWave);
    before = __shfl(before, src, kWave);
    // the token: re-read the chunk, tempered tail values in token order
    float x[8];
    dense_load<DT>(row, ch, c.V, x);
    double tv[8], ls = 0.0;
    static_for<8>([&](auto k) {
      const int v = ch * kDC + lane * 8 + (int)k;
      tv[k] = dense_is_det(L, t0, v) ? 0.0 : dense_tempered(x[k], M, invT);
      ls += tv[k];
    });
    const double li = wave_incl_scan(ls);
    const double rem = tgt - before;
    int pick = -1;
    const uint64_t h2 = ballot(ls > 0.0 && rem < li);
    if (h2) {
      const int s2 = __builtin_ctzll(h2);
      if (lane == s2) {
        double cum = li - ls;
        static_for<8>([&](auto k) {
          cum += tv[k];
          if (pick < 0 && tv[k] > 0.0 && rem < cum) pick = ch * kDC + lane * 8 + (int)k;
        });
      }
      pick = __shfl(pick, s2, kWave);
    }
    if (pick < 0) {  // rounding: the chunk's last tail token with mass
      int last = -1;
      static_for<8>([&](auto k) {
        if (tv[k] > 0.0) last = ch * kDC + lane * 8 + (int)k;
      });
      for (int o = 1; o < kWave; o <<= 1) last = max(last, __shfl_xor(last, o, kWave));
      pick = last;
    }
    probe = pick;
    if (t0 >= 1) {
      const float qm = qraw(t0 - 1);
      proxy = qm < zr ? qm : zr;
    } else {
      const float t1 = qraw(0) + c.eps_m0;
      proxy = t1 < 1.0f ? t1 : 1.0f;
    }
  }
  // what regenerates the probe's tail at verification: the row's largest logit, the
  // tempered tail mass and the deterministic children's tokens
  if (lane == 0) {
    a.t.row_tail_n[ktb] = 0;
    a.t.row_dense[ktb * 2] = (double)M;
    a.t.row_dense[ktb * 2 + 1] = probe >= 0 ? zT : 0.0;
  }
  if (lane < t0) a.t.row_det[ktb * 32 + lane] = L.det[lane];

  // 4. child slots: DET ranks, the probe, then fillers in rank order (lane s: slot s)
  const int rp_hit = (int)__builtin_ctzll(ballot(lane < n_sup && probe >= 0 &&
                                                 (int)sup_key_id(s_sup[min(lane, n_sup - 1)]) == probe) |
                                          (1ull << 63));
  const int rp = rp_hit < n_sup ? rp_hit : 1 << 30;  // the probe's rank if among the K best
  int r_of_slot = -1, kind = 0;
  {
    const int m_det = c.probe ? min(m, n_sup) : 0;
    const int s = lane;
    if (!c.probe) {
      if (s < n_sup) r_of_slot = s, kind = VRT_DET;
    } else if (s < m_det) {
      r_of_slot = s, kind = VRT_DET;
    } else if (c.order == VRT_PROBE_LAST) {
      if (s < t0) r_of_slot = s, kind = VRT_FILL;
      else if (probe >= 0 && s == t0) kind = VRT_PROBE;
    } else if (probe >= 0 && s == m_det) {
      kind = VRT_PROBE;
    } else {
      int r = m + s - m_det - (probe >= 0 ? 1 : 0);
      if (r >= rp) ++r;
      if (r < n_sup) r_of_slot = r, kind = VRT_FILL;
    }
  }
  if (lane < c.K) {
    const int64_t ci = ncb + cbase + lane;
    if (kind == VRT_PROBE) {
      st_dev(&a.t.cand_token[ci], probe);
      st_dev(&a.t.cand_parent[ci], node);
      st_dev(&a.t.cand_score[ci], sp * proxy);
      st_dev(&a.t.cand_kind[ci], kind);
    } else if (r_of_slot >= 0) {
      st_dev(&a.t.cand_token[ci], (int)sup_key_id(s_sup[r_of_slot]));
      st_dev(&a.t.cand_parent[ci], node);
      st_dev(&a.t.cand_score[ci], sp * qraw(r_of_slot));
      st_dev(&a.t.cand_kind[ci], kind);
    } else {
      st_dev(&a.t.cand_kind[ci], 0);
    }
  }
  if (a.fuse_rank) rank_if_last(a, b, s_rank);
}

// Coverage of the top-trunc support (the coverage column of the support-size ablation):
// per row, the share of the untempered softmax that its trunc largest logits hold, in
// fp64 with exponentials to about 1e-7 relative. One 8-wave block per row: the exact
// selection of the trunc best keys (one key when trunc covers the row), then one pass
// over the row for the total while wave 0 sums the selected keys.
template <int DT, int PL>
__global__ __launch_bounds__(8 * kWave) void k_coverage(const Cfg c, const void* logits, int64_t ld,
                                                       int64_t tstride, int n_rows, double* out) {
  constexpr int SW = 8;
  const int j = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int lane = lane_id();
  __shared__ ExactLds<PL> X;
  __shared__ uint64_t s_sup[PL * kWave];
  __shared__ double s_part[SW];
  __shared__ int s_n, s_bad;
  constexpr int esz = DT == VRT_BF16 ? 2 : 4;
  constexpr int EPL = 16 / esz;
  const char* row = (const char*)logits + ((int64_t)b * tstride + (int64_t)j * ld) * esz;
  const bool all = c.trunc == VRT_DENSE || c.trunc >= c.V;  // the support is the whole row
  int n_sup = 0;
  const int bad = row_select_exact<DT, PL, SW>(row, 0, c.V, all ? 1 : c.trunc, 0u, X, s_sup, n_sup);
  if (tid == 0) {
    s_n = n_sup;
    s_bad = bad;
  }
  __syncthreads();
  double* o = out + (int64_t)b * n_rows + j;
  const float M = s_n > 0 ? sup_key_val(s_sup[0]) : -INFINITY;
  if (s_bad || !(M > -INFINITY)) {
    if (tid == 0) *o = s_bad ? (double)NAN : 0.0;
    return;
  }
  double tot = 0.0;
  const int nv = (c.V + EPL - 1) / EPL;
  for (int v = tid; v < nv; v += SW * kWave) {
    const u32x4_t d = *(const u32x4_t*)(row + (int64_t)v * 16);
    static_for<EPL>([&](auto e) {
      float x;
      if constexpr (DT == VRT_BF16) x = (e & 1) ? bf16_hi(d[e >> 1]) : bf16_lo(d[e >> 1]);
      else x = __uint_as_float(d[(int)e]);
      if (v * EPL + (int)e < c.V) tot += dense_tempered(x, M, 1.0);
    });
  }
  tot = wave_sum(tot);
  if (lane == 0) s_part[wave] = tot;
  __syncthreads();
  if (wave != 0) return;
  double all_sum = 0.0;
  for (int w = 0; w < SW; ++w) all_sum += s_part[w];
  double top = 0.0;
  static_for<PL>([&](auto s) {
    const int r = lane * PL + (int)s;
    if (r < s_n) top += dense_tempered(sup_key_val(s_sup[r]), M, 1.0);
  });
  top = wave_sum(top);
  if (lane == 0) *o = all ? 1.0 : top / all_sum;
}

// Per-tree ranking of the layer's children, given their keys sorted (path score
// desc, creation index asc; zeros last): the top W become the frontier (top-R mode),
// or SMART's sequential keep rule runs over them. One thread.
__device__ void rank_sorted(const Cfg& c, const TreePtrs& t, int layer, int b, const uint64_t* keys,
                            int span) {
  const int64_t ncb = (int64_t)b * c.NC;
  const bool more = layer + 1 < c.D;
  int* front = t.front + (int64_t)b * c.FP;
  int nf = 0;
  if (c.mode == VRT_MODE_TOPR) {
    if (more)
      for (int i = 0; i < span && nf < c.W && keys[i] != 0ull; ++i)
        front[nf++] = (int)(0xFFFFFFFFu - (uint32_t)keys[i]);
  } else {
    // SMART key design 3: keep u iff alpha * g * C(|T|) > L * C'(|T|), g = P(path)/|P|;
    // the first rejection ends the layer
    double* sm = t.smart + (int64_t)b * 8;
    double L = sm[0], n = sm[1], P = sm[2], nadm = sm[3], root_has = sm[4];
    int* adm = t.admitted + (int64_t)b * c.N;
    for (int i = 0; i < span && keys[i] != 0ull; ++i) {
      if (nadm >= (double)c.budget) break;
      const int cu = (int)(0xFFFFFFFFu - (uint32_t)keys[i]);
      const double g = (double)ld_dev(&t.cand_score[ncb + cu]) / P;
      // C(|T|) and C'(|T|) from the host's fp64 table (|T| = n is 1 .. budget+1 here)
      const int ni = min(max((int)n, 0), c.budget + 1);
      const double Cn = t.smart_cost[2 * ni], dC = t.smart_cost[2 * ni + 1];
      if (!(c.alpha * g * Cn > L * dC)) break;
      const int par = ld_dev(&t.cand_parent[ncb + cu]);
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

// Ranking as a kernel of its own (layers of more than kRankFused children): one block
// per tree gathers the keys of the children the layer created to the front of LDS and
// sorts only those. Top-R then writes the first W as the frontier. For SMART, all
// threads first fetch what the keep rule reads per position (the child's parent, the
// cost-table entries C(|T|) and C'(|T|) at the size the tree has when that position is
// tested), so the rule's sequential pass runs on LDS alone; the admitted prefix is
// written out in parallel afterwards.
constexpr int kRankT = 256;        // threads of the ranking block
constexpr int kRankSmart = 1024;   // SMART positions it stages (the budget's maximum)
constexpr int kRestRankSpan = 2048;  // slots per layer up to which k_rest_rank's LDS holds the keys
constexpr int kRankPar = 4096;     // parents per layer it tracks (P * K is at most 4096)

template <int NT>
__device__ __forceinline__ void rank_layer_block(const Cfg& c, const TreePtrs& t, int layer, int b,
                                                 uint64_t* s_keys) {
  const int tid = threadIdx.x, lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  const int base = layer_base(c, layer);
  const int span = layer_span(c, layer);
  __shared__ int s_n, s_m;
  // a tree that expanded no parent at this layer has no children to rank: its frontier
  // stays empty and its SMART state as it is
  if (layer > 0 && t.n_front[b] <= 0) return;
  // created children, in any order (the sort fixes it): one LDS atomic per wave and pass
  if (tid == 0) s_n = 0;
  __syncthreads();
  for (int i0 = 0; i0 < span; i0 += 4 * NT) {
    uint64_t k[4];
    static_for<4>([&](auto s) {
      const int i = i0 + s * NT + tid;
      k[s] = 0ull;
      if (i < span && (ld_dev(&t.cand_kind[ncb + base + i]) & 0xFF) != 0)
        k[s] = node_key(ld_dev(&t.cand_score[ncb + base + i]), (uint32_t)(base + i));
    });
    static_for<4>([&](auto s) {
      const uint64_t m = ballot(k[s] != 0ull);
      int at = 0;
      if (lane == 0 && m != 0ull) at = atomicAdd(&s_n, __builtin_popcountll(m));
      at = __shfl(at, 0);
      const int below = __builtin_popcountll(m & ((1ull << lane) - 1ull));
      if (k[s] != 0ull) s_keys[at + below] = k[s];
    });
  }
  __syncthreads();
  const int n = s_n;
  const int np = next_pow2(max(n, 2));
  for (int i = n + tid; i < np; i += NT) s_keys[i] = 0ull;
  __syncthreads();
  bitonic_desc(s_keys, np);
  const bool more = layer + 1 < c.D;
  int* front = t.front + (int64_t)b * c.FP;
  if (c.mode == VRT_MODE_TOPR) {
    const int nf = more ? min(c.W, n) : 0;
    for (int i = tid; i < nf; i += NT) front[i] = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i]);
    if (tid == 0) t.n_front[b] = nf;
    return;
  }
  // SMART key design 3, as in rank_sorted: keep u iff alpha * g * C(|T|) > L * C'(|T|)
  // with g = P(path) / |P|, the first rejection ends the layer. Position i is tested
  // with |T| = n0 + i, since every position before it was admitted.
  __shared__ int s_par[kRankSmart];
  __shared__ double s_cn[kRankSmart], s_dc[kRankSmart];
  __shared__ uint8_t s_pf[kRankPar];  // parent has an admitted child: 1 before, 2 set now
  double* sm = t.smart + (int64_t)b * 8;
  const double n0 = sm[1], nadm0 = sm[3];
  const int stop = min(n, max(c.budget - (int)nadm0, 0));
  const int pbase = layer > 0 ? layer_base(c, layer - 1) : 0;
  const int pspan = layer > 0 ? layer_span(c, layer - 1) : 0;
  for (int p = tid; p < pspan; p += NT)
    s_pf[p] = (ld_dev(&t.cand_kind[ncb + pbase + p]) & 0x100) ? 1 : 0;
  for (int i = tid; i < stop; i += NT) {
    const int cu = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i]);
    s_par[i] = ld_dev(&t.cand_parent[ncb + cu]);
    const int ni = min(max((int)(n0 + (double)i), 0), c.budget + 1);
    s_cn[i] = t.smart_cost[2 * ni];
    s_dc[i] = t.smart_cost[2 * ni + 1];
  }
  __syncthreads();
  if (tid == 0) {
    double L = sm[0], nn = n0, P = sm[2], nadm = nadm0, root_has = sm[4];
    int m = 0;
    for (; m < stop; ++m) {
      // the key's high word is the child's fp32 path score
      const double g = (double)__uint_as_float((uint32_t)(s_keys[m] >> 32)) / P;
      if (!(c.alpha * g * s_cn[m] > L * s_dc[m])) break;
      const int par = s_par[m];
      bool has;
      if (par < 0) {
        has = root_has != 0.0;
        root_has = 1.0;
      } else if (par - pbase >= 0 && par - pbase < pspan) {
        has = s_pf[par - pbase] != 0;
        if (!has) s_pf[par - pbase] = 2;
      } else {  // not a node of the layer above: read and mark it in place
        has = (t.cand_kind[ncb + par] & 0x100) != 0;
        t.cand_kind[ncb + par] |= 0x100;
      }
      L += g;
      nn += 1.0;
      if (has) P += 1.0;
      nadm += 1.0;
    }
    sm[0] = L; sm[1] = nn; sm[2] = P; sm[3] = nadm; sm[4] = root_has;
    t.n_front[b] = more ? m : 0;
    s_m = m;
  }
  __syncthreads();
  const int m = s_m;
  int* adm = t.admitted + (int64_t)b * c.N + (int)nadm0;
  for (int i = tid; i < m; i += NT) {
    const int cu = (int)(0xFFFFFFFFu - (uint32_t)s_keys[i]);
    adm[i] = cu;
    if (more) front[i] = cu;
  }
  for (int p = tid; p < pspan; p += NT)
    if (s_pf[p] == 2) t.cand_kind[ncb + pbase + p] |= 0x100;
}


__global__ __launch_bounds__(kRankT) void k_rank_layer(const Cfg c, const TreePtrs t, int layer) {
  extern __shared__ uint64_t s_keys[];  // next_pow2(span) keys
  rank_layer_block<kRankT>(c, t, layer, blockIdx.x, s_keys);
}

// A SMART layer after its compact grid, one block per tree: the tree's expanded rows
// beyond the grid (items pre[b] .. pre[b+1]-1 of the list from a.compact on), one after
// another, then the layer's ranking. One launch instead of a kernel for the rows and one
// for the ranking; a tree's rows beyond the grid run in its own block, which suits the
// keep rule's frontiers (one or two rows per tree per layer at budget 128, top-k 8).
template <int DT, int PL>
__global__ __launch_bounds__(kSelWaves * kWave) void k_rest_rank(const BArgs a) {
  extern __shared__ uint64_t s_keys[];  // next_pow2(span) keys
  const int b = blockIdx.x;
  const int p0 = a.cpre[b], p1 = a.cpre[b + 1];
  for (int k = max(p0, a.compact); k < p1; ++k) {
    select_expand_row<DT, PL, false>(a, b, __builtin_amdgcn_readfirstlane(k - p0), 0, 1);
    __syncthreads();  // the block's LDS changes hands; the rows' candidates are stored
  }
  rank_layer_block<kSelWaves * kWave>(a.c, a.t, a.layer, b, s_keys);
}

constexpr int kFT = 1024;          // threads of the finish block
constexpr int kFW = kFT / kWave;   // its waves
constexpr int kMapMax = 16384;     // candidate -> node map in LDS up to this many candidates

// Keys per lane of the finish's wave lists (64*PL >= R), 0 when R needs the LDS sort.
__host__ __device__ inline int finish_pl(const Cfg& c) {
  if (c.mode != VRT_MODE_TOPR) return 0;
  return c.R <= 64 ? 1 : (c.R <= 128 ? 2 : 0);
}

// Finish's dynamic LDS, in 8-byte words: the key area (wave lists or the LDS sort), then
// the candidate -> node map, then per node: candidate, parent node, slot, expansion row
// holding its tail, tail length, child slot mask [N], child counts [N+1].
struct FinishLds {
  int key_words, map_ints;
  __host__ __device__ explicit FinishLds(const Cfg& c) {
    const int pl = finish_pl(c);
    if (c.mode != VRT_MODE_TOPR) key_words = 0;
    else if (pl) key_words = (kFW / 2 + 1) * pl * kWave;
    else key_words = next_pow2(max(c.NC, 2));
    // the map only where the whole area stays within 64 KB
    const size_t rest = (size_t)key_words * 8 + (size_t)(7 * c.N + 1) * 4;
    map_ints = (c.NC <= kMapMax && rest + (size_t)c.NC * 4 <= 65536) ? c.NC : 0;
  }
  __host__ __device__ size_t bytes(const Cfg& c) const {
    return (size_t)key_words * 8 + (size_t)map_ints * 4 + (size_t)(7 * c.N + 1) * 4;
  }
};

// Top 64*PL candidate keys of tree b (path score desc, creation index asc), sorted
// descending and zero-padded, into s_top: each wave sorts chunks of 64*PL candidates
// and keeps the largest 64*PL; the waves' lists then merge pairwise through LDS.
template <int PL>
__device__ void finish_top(const Cfg& c, const TreePtrs& t, int64_t ncb, uint64_t* s_list,
                           uint64_t* s_top) {
  constexpr int CH = PL * kWave;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  uint64_t acc[PL];
  static_for<PL>([&](auto s) { acc[s] = 0ull; });
  const int nch = (c.NC + CH - 1) / CH;
  for (int ch = wave; ch < nch; ch += kFW) {
    uint64_t k[PL];
    static_for<PL>([&](auto s) {
      const int i = ch * CH + lane * PL + s;
      uint64_t x = 0ull;
      if (i < c.NC && (t.cand_kind[ncb + i] & 0xFF) != 0) x = node_key(t.cand_score[ncb + i], (uint32_t)i);
      k[s] = x;
    });
    wave_sort_desc<PL>(k);
    if (ch == wave) static_for<PL>([&](auto s) { acc[s] = k[s]; });
    else wave_merge_top<PL>(acc, k);
  }
  for (int st = 1; st < kFW; st <<= 1) {
    uint64_t* slot = s_list + (wave / (2 * st)) * CH;
    if ((wave & (2 * st - 1)) == st) static_for<PL>([&](auto s) { slot[lane * PL + s] = acc[s]; });
    __syncthreads();
    if ((wave & (2 * st - 1)) == 0) {
      uint64_t oth[PL];
      static_for<PL>([&](auto s) { oth[s] = slot[lane * PL + s]; });
      wave_merge_top<PL>(acc, oth);
    }
    __syncthreads();
  }
  if (wave == 0) static_for<PL>([&](auto s) { s_top[lane * PL + s] = acc[s]; });
}

// Emit the tree: node 0 = root, then the kept candidates (parents first).
__global__ __launch_bounds__(kFT) void k_finish(const Cfg c, const TreePtrs t) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int64_t ncb = (int64_t)b * c.NC;
  const int64_t nb = (int64_t)b * c.N;
  extern __shared__ uint64_t s_keys[];
  const FinishLds FL(c);
  int* s_node_of = (int*)(s_keys + FL.key_words);
  int* s_ncand = s_node_of + FL.map_ints;
  int* s_par = s_ncand + c.N;
  int* s_slot = s_par + c.N;
  int* s_trow = s_slot + c.N;
  int* s_tn = s_trow + c.N;
  uint32_t* s_smask = (uint32_t*)(s_tn + c.N);
  int* s_cnt = (int*)(s_smask + c.N);
  __shared__ int s_n;

  for (int i = tid; i < FL.map_ints; i += kFT) s_node_of[i] = 0x7FFFFFFF;
  if (c.mode == VRT_MODE_TOPR) {
    const int pl = finish_pl(c);
    const uint64_t* top = s_keys;
    if (pl) {
      // wave lists: the 8 merge slots, then the result
      uint64_t* s_top = s_keys + (kFW / 2) * pl * kWave;
      if (pl == 1) finish_top<1>(c, t, ncb, s_keys, s_top);
      else finish_top<2>(c, t, ncb, s_keys, s_top);
      top = s_top;
    } else {
      const int np = FL.key_words;
      for (int i = tid; i < np; i += kFT) {
        uint64_t k = 0ull;
        if (i < c.NC && (t.cand_kind[ncb + i] & 0xFF) != 0) k = node_key(t.cand_score[ncb + i], (uint32_t)i);
        s_keys[i] = k;
      }
      __syncthreads();
      bitonic_desc(s_keys, np);
    }
    __syncthreads();
    // n - 1 = the nonzero keys among the first R (the list is sorted, zeros last)
    if (wave == 0) {
      const int lim = pl ? c.R : min(c.R, FL.key_words);
      int cnt = 0;
      for (int i = lane; i < lim; i += kWave) cnt += top[i] != 0ull;
      cnt = wave_sum_i(cnt);
      if (lane == 0) s_n = 1 + cnt;
    }
    __syncthreads();
    for (int i = 1 + tid; i < s_n; i += kFT) s_ncand[i] = (int)(0xFFFFFFFFu - (uint32_t)top[i - 1]);
  } else {
    if (tid == 0) {
      const int nadm = (int)t.smart[(int64_t)b * 8 + 3];
      s_n = 1 + min(max(nadm, 0), c.N - 1);
    }
    __syncthreads();
    for (int i = 1 + tid; i < s_n; i += kFT) {
      const int cu = t.admitted[nb + i - 1];
      s_ncand[i] = (cu < 0 || cu >= c.NC) ? 0 : cu;
    }
  }
  const int n = s_n;
  if (tid == 0) s_ncand[0] = -1;
  for (int i = tid; i <= n; i += kFT) s_cnt[i] = 0;
  for (int i = tid; i < n; i += kFT) {
    s_trow[i] = -1;
    s_tn[i] = 0;
    s_smask[i] = 0u;
  }
  __syncthreads();
  if (FL.map_ints)
    for (int i = 1 + tid; i < n; i += kFT) atomicMin(&s_node_of[s_ncand[i]], i);
  __syncthreads();
  // nodes: parent node (parents precede children, so it is among nodes 1..i-1)
  for (int i = 1 + tid; i < n; i += kFT) {
    const int cu = s_ncand[i];
    const int r = row_of(c, cu);
    const int pc = t.cand_parent[ncb + cu];
    const int kind = t.cand_kind[ncb + cu] & 0xFF;
    const int tok = t.cand_token[ncb + cu];
    const int rtn = t.row_tail_n[(int64_t)b * c.NR + r];
    int pn = 0;
    if (pc >= 0) {
      if (FL.map_ints) {
        const int m = s_node_of[pc];
        pn = (m >= 1 && m < i) ? m : 0;
      } else {
        for (int jj = i - 1; jj >= 1; --jj)
          if (s_ncand[jj] == pc) {
            pn = jj;
            break;
          }
      }
    }
    const int slot = slot_of(c, cu);
    s_par[i] = pn;
    s_slot[i] = slot;
    if (kind == VRT_PROBE) {
      s_trow[pn] = r;
      s_tn[pn] = min(max(rtn, 0), c.TC);
    }
    t.node_cand[nb + i] = cu;
    t.node_token[nb + i] = tok;
    t.node_parent[nb + i] = pn;
    t.node_depth[nb + i] = layer_of(c, cu) + 1;
    t.node_kind[nb + i] = kind;
    atomicAdd(&s_cnt[pn], 1);
    atomicOr(&s_smask[pn], 1u << slot);
  }
  if (tid == 0) {
    t.node_token[nb] = -1;
    t.node_parent[nb] = -1;
    t.node_depth[nb] = 0;
    t.node_kind[nb] = VRT_ROOT;
    t.node_cand[nb] = -1;
  }
  __syncthreads();
  // child offsets: exclusive scan of the counts (wave 0, 64 nodes at a time)
  if (wave == 0) {
    const int64_t cob = (int64_t)b * (c.N + 1);
    int carry = 0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
      const int i = i0 + lane;
      const int v = i < n ? s_cnt[i] : 0;
      const int incl = wave_incl_scan(v);
      if (i < n) {
        s_cnt[i] = carry + incl - v;
        t.child_off[cob + i] = carry + incl - v;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      t.child_off[cob + n] = carry;
      t.n_nodes[b] = n;
    }
  }
  __syncthreads();
  // child lists in slot order (siblings come from one expansion row: distinct slots)
  for (int i = 1 + tid; i < n; i += kFT) {
    const int pn = s_par[i], slot = s_slot[i];
    const int before = __builtin_popcount(s_smask[pn] & ((1u << slot) - 1u));
    t.child[nb + s_cnt[pn] + before] = i;
  }
  // probe tails, copied to the probe's parent (all loads of a round in flight at once);
  // dense rows: the expansion row that regenerates the tail
  for (int i = tid; i < n; i += kFT) t.tail_n[nb + i] = s_tn[i];
  if (c.trunc == VRT_DENSE)
    for (int i = tid; i < n; i += kFT) t.node_row[nb + i] = s_trow[i];
  constexpr int U = 8;
  const int64_t tot = (int64_t)n * c.TC;
  for (int64_t x0 = 0; x0 < tot; x0 += (int64_t)kFT * U) {
    int idv[U];
    float qv[U];
    int64_t dst[U];
    static_for<U>([&](auto u) {
      const int64_t x = x0 + (int64_t)u * kFT + tid;
      dst[u] = -1;
      if (x < tot) {
        const int i = (int)(x / c.TC), k = (int)(x % c.TC);
        if (k < s_tn[i]) {
          const int64_t rr = ((int64_t)b * c.NR + s_trow[i]) * c.TC + k;
          idv[u] = t.row_tail_id[rr];
          qv[u] = t.row_tail_q[rr];
          dst[u] = (nb + i) * c.TC + k;
        }
      }
    });
    static_for<U>([&](auto u) {
      if (dst[u] >= 0) {
        t.tail_id[dst[u]] = idv[u];
        t.tail_q[dst[u]] = qv[u];
      }
    });
  }
}

// Host values into device memory through kernel arguments, kFillChunk per launch.
constexpr int kFillChunk = 128;
struct FillArgs {
  double* dst;
  int n;
  double v[kFillChunk];
};

__global__ __launch_bounds__(kFillChunk) void k_fill_f64(const FillArgs f) {
  if ((int)threadIdx.x < f.n) f.dst[threadIdx.x] = f.v[threadIdx.x];
}

int list_len(const Cfg& c) { return max(128, next_pow2(c.trunc)); }

template <int DT, bool SPLIT>
hipError_t launch_select(const BArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kSelWaves * kWave);
  switch (list_len(a.c) / kWave) {
    case 2: hipLaunchKernelGGL((k_select_expand<DT, 2, SPLIT>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_select_expand<DT, 4, SPLIT>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_select_expand<DT, 8, SPLIT>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((k_select_expand<DT, 16, SPLIT>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int DT, int PL>
void launch_rest(const BArgs& a, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((k_select_rest<DT, PL>), dim3(blocks), dim3(kSelWaves * kWave), 0, stream, a);
}

template <int DT>
hipError_t launch_rest_rank(const BArgs& a, size_t lds, hipStream_t stream) {
  const dim3 grid(a.c.B), block(kSelWaves * kWave);
  switch (list_len(a.c) / kWave) {
    case 2: hipLaunchKernelGGL((k_rest_rank<DT, 2>), grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((k_rest_rank<DT, 4>), grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((k_rest_rank<DT, 8>), grid, block, lds, stream, a); break;
    default: hipLaunchKernelGGL((k_rest_rank<DT, 16>), grid, block, lds, stream, a); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_layer(const BArgs& a, int rows, hipStream_t stream) {
  if (a.compact > 0) {
    const hipError_t e = launch_select<DT, false>(a, dim3(a.compact), stream);
    const int extra = a.c.B * rows - a.compact;  // rows the compact grid may not reach
    if (e != hipSuccess || extra <= 0 || a.rest == 0) return e;  // rest 0: k_rest_rank takes them
    const int blocks = min(extra, a.rest);
    switch (list_len(a.c) / kWave) {
      case 2: launch_rest<DT, 2>(a, blocks, stream); break;
      case 4: launch_rest<DT, 4>(a, blocks, stream); break;
      case 8: launch_rest<DT, 8>(a, blocks, stream); break;
      default: launch_rest<DT, 16>(a, blocks, stream); break;
    }
    return hipGetLastError();
  }
  if (a.mixed > 0) {
    const int n_rows = a.c.B * rows;
    return launch_select<DT, true>(a, dim3(a.mixed + a.parts * (n_rows - a.mixed)), stream);
  }
  const dim3 grid(rows * a.split, a.c.B);
  if (a.c.trunc == VRT_DENSE) {
    hipLaunchKernelGGL((k_dense_expand<DT>), grid, dim3(8 * kWave), 0, stream, a);
    return hipGetLastError();
  }
  if (a.split > 1) return launch_select<DT, true>(a, grid, stream);
  return launch_select<DT, false>(a, grid, stream);
}

template <int DT>
hipError_t launch_coverage_t(const Cfg& c, const void* logits, int64_t ld, int64_t tstride, int n_rows,
                             double* out, hipStream_t stream) {
  const dim3 grid(n_rows, c.B), block(8 * kWave);
  switch (c.trunc == VRT_DENSE ? 2 : list_len(c) / kWave) {
    case 2: hipLaunchKernelGGL((k_coverage<DT, 2>), grid, block, 0, stream, c, logits, ld, tstride, n_rows, out); break;
    case 4: hipLaunchKernelGGL((k_coverage<DT, 4>), grid, block, 0, stream, c, logits, ld, tstride, n_rows, out); break;
    case 8: hipLaunchKernelGGL((k_coverage<DT, 8>), grid, block, 0, stream, c, logits, ld, tstride, n_rows, out); break;
    default: hipLaunchKernelGGL((k_coverage<DT, 16>), grid, block, 0, stream, c, logits, ld, tstride, n_rows, out); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_coverage(const Cfg& c, const void* logits, int64_t ld, int64_t tstride, int n_rows,
                           double* out, hipStream_t stream) {
  return c.dtype == VRT_BF16 ? launch_coverage_t<VRT_BF16>(c, logits, ld, tstride, n_rows, out, stream)
                             : launch_coverage_t<VRT_F32>(c, logits, ld, tstride, n_rows, out, stream);
}

// Rows split over two blocks, at every layer: rows too long for one block's row-wide
// path whose halves fit it (fp32 rows of 65537 to 131072 values, bf16 rows of 196609 to
// 393216). Splitting rows that fit one block measured slower after the root (0.450
// against 0.403 ms per step at B = 32, V = 128256, W = 10: each half pays the dependent
// phases after its loads) and no faster at the root (0.4032 against 0.4021-0.4027 ms).
bool split_rows(const Cfg& c, int layer) {
  (void)layer;
  if (c.trunc == VRT_DENSE) return false;
  const bool bf = c.dtype == VRT_BF16;
  const int seg = bf ? seg_elems<VRT_BF16>() : seg_elems<VRT_F32>();
  const int cap = (bf ? seg_per_wave<VRT_BF16>() : seg_per_wave<VRT_F32>()) * kSelWaves;
  const int G = (c.V + seg - 1) / seg;
  return G > cap && (G + 1) / 2 <= cap;
}

// Tags of split launches: a process-wide counter from a random start.
static std::atomic<uint64_t> g_epoch{((uint64_t)std::random_device{}() << 32) ^ std::random_device{}()};

// Layers of more rows than the GPU has CUs put two rows on some CUs, and those CUs finish
// their loads last (a CU streams at most ~28 GB/s). Up to 1.5 rows per CU, one row per CU
// stays whole and the rest are split over four blocks each (up to 1.25 rows per CU) or two
// (the parts' lists in the workspace): at B = 32, W = 10 (320 rows of V = 128256) 256
// whole rows and 64 split ones,
// 0.253 against 0.262 ms of build per step (quarters and halves measure the same there:
// once its part is done, a whole row streams alone at one block's rate).
// (Supports of 512 and 1024 keys stay whole: their parts' sorts and merges made the split
// rows the last ones, 0.530 against 0.509 and 0.935 against 0.796 ms of build per step.)
static bool mixable(const Cfg& c) {
  return c.trunc != VRT_DENSE && list_len(c) <= 256 && !split_rows(c, 0) && c.B * c.FP > 64;
}

static int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = -1;
    cached[dev] = v > 0 ? v : -1;
  }
  return cached[dev] > 0 ? cached[dev] : 0;
}

// The workspace: the parts' lists (split rows, the mixed grid), then for SMART the compact
// grids' prefix sums of the frontier sizes.
static size_t lists_bytes(const Cfg& c) {
  if (!split_rows(c, 0) && !mixable(c)) return 0;
  const size_t parts = (size_t)c.B * c.FP * kMaxParts;
  return parts * list_len(c) * 8 + parts * 4;
}
static size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

size_t build_ws_bytes(const Cfg& c) {
  const size_t n = lists_bytes(c);
  return c.mode == VRT_MODE_SMART ? align16(n) + (size_t)(c.B + 1) * 4 : n;
}

hipError_t launch_build_layer(const Cfg& c, const TreePtrs& t, int layer, const void* logits,
                              int64_t ld, int64_t tstride, uint64_t seed, uint32_t step,
                              uint32_t* stats, void* ws, hipStream_t stream) {
  const int span = (layer == 0 ? 1 : c.P) * c.K;
  const bool split = split_rows(c, layer);
  const int rows = layer == 0 ? 1 : c.FP;
  const int ncu = cu_count();
  const int n_rows = c.B * rows;
  // one whole row per CU, the other rows in quarters (up to 1.25 rows per CU) or halves
  // (up to 1.5) in the CUs' second slots
  const int seg = c.dtype == VRT_BF16 ? seg_elems<VRT_BF16>() : seg_elems<VRT_F32>();
  const int G = (c.V + seg - 1) / seg;
  // every part takes at least one segment: parts of ceil(G / P) segments, the last one too
  auto fits = [G](int P) { return (P - 1) * ((G + P - 1) / P) < G; };
  const int parts = (4 * (n_rows - ncu) <= ncu && fits(4)) ? 4 : 2;
  const int mixed = (layer > 0 && !split && mixable(c) && ncu > 0 && n_rows > ncu &&
                     2 * n_rows <= 3 * ncu && fits(parts))
                        ? ncu
                        : 0;
  const bool lists = split || mixed > 0;
  uint64_t* hk = (uint64_t*)ws;
  int* hm = lists ? (int*)(hk + (size_t)c.B * c.FP * kMaxParts * list_len(c)) : nullptr;
  // SMART frontiers are usually far below FP parents per tree: a compact grid of at most
  // two blocks per CU walks the expanded rows (the ranking must run in its own kernel,
  // since the grid reads every tree's frontier size)
  const bool fuse = span <= kRankFused;
  const int compact = (c.mode == VRT_MODE_SMART && layer > 0 && !fuse && !split && mixed == 0 &&
                       c.trunc != VRT_DENSE && c.B <= kCompactTrees && ncu > 0)
                          ? min(n_rows, 2 * ncu)
                          : 0;
  // rows beyond the compact grid: in the ranking kernel, each tree's own (one launch less
  // per layer), while its LDS holds the keys of the layer (up to 2048 slots); else a kernel
  // of one block per CU before the ranking
  const bool merged = compact > 0 && n_rows > compact && span <= kRestRankSpan;
  int* cpre = (int*)((char*)ws + align16(lists_bytes(c)));
  BArgs a{c, t, layer, logits, ld, tstride, seed, step, stats, fuse ? 1 : 0,
          split ? 2 : 1, lists ? hk : nullptr, hm, lists ? g_epoch.fetch_add(1) : 0, rows, mixed,
          parts, compact, merged ? 0 : ncu, cpre};
  hipError_t e = c.dtype == VRT_BF16 ? launch_layer<VRT_BF16>(a, rows, stream)
                                     : launch_layer<VRT_F32>(a, rows, stream);
  if (e != hipSuccess) return e;
  if (a.fuse_rank) return hipSuccess;
  const size_t lds2 = (size_t)next_pow2(max(span, 2)) * 8;
  if (merged)
    return c.dtype == VRT_BF16 ? launch_rest_rank<VRT_BF16>(a, lds2, stream)
                               : launch_rest_rank<VRT_F32>(a, lds2, stream);
  hipLaunchKernelGGL(k_rank_layer, dim3(c.B), dim3(kRankT), lds2, stream, c, t, layer);
  return hipGetLastError();
}

hipError_t launch_fill_f64(double* dst, const double* vals, int n, hipStream_t stream) {
  for (int o = 0; o < n; o += kFillChunk) {
    FillArgs f;
    f.dst = dst + o;
    f.n = min(kFillChunk, n - o);
    for (int k = 0; k < f.n; ++k) f.v[k] = vals[o + k];
    hipLaunchKernelGGL(k_fill_f64, dim3(1), dim3(kFillChunk), 0, stream, f);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_build_finish(const Cfg& c, const TreePtrs& t, void* ws, hipStream_t stream) {
  (void)ws;
  const size_t lds = FinishLds(c).bytes(c);
  hipLaunchKernelGGL(k_finish, dim3(c.B), dim3(kFT), lds, stream, c, t);
  return hipGetLastError();
}

}  // namespace vrt
