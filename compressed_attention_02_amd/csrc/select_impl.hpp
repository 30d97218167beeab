// Device code of the indexer: helpers shared by the score and select kernels and
// the per-row selection, which the combined selection + attention kernel of the
// decode step runs too.  The design notes are at the top of index.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

__device__ __forceinline__ void row_coords(int row, int tq, const int64_t* pos0, int& b, int& i,
                                           int64_t& pos) {
  b = row / tq;
  i = row - b * tq;
  pos = pos0[b] + i;
}

// A wave's report on its 64 elements (lane L holds block base + L with order key
// `key` when `valid`): the keys of its kWaveTop best (higher key first, then lower
// id) in ascending id order, their ids as 8-bit offsets from base (0xff = no
// element) packed in one word, and the key of the next best, an upper bound on every
// key it leaves out (0 if none).  Each round takes a 32-bit wave maximum (DPP) of
// the keys not yet taken and gives it to the lowest lane that holds it (a ballot),
// so ties go to the lower id; the taken lanes, in lane order, are the id order.
__device__ __forceinline__ void wave_top(uint32_t key, bool valid, uint32_t* keys, uint2* info) {
  static_assert(kWaveTop == 4, "four offsets per info word");
  const int lane = threadIdx.x & 63;
  bool live = valid;
  uint64_t won = 0;
#pragma unroll
  for (int r = 0; r < kWaveTop; ++r) {
    const uint32_t m = wave_max_u32(live ? key : 0u);
    const uint64_t at = __ballot(live && key == m);
    if (at) {
      const int l = __builtin_ctzll(at);
      won |= 1ull << l;
      live = live && lane != l;
    }
  }
  const uint32_t bound = wave_max_u32(live ? key : 0u);
  uint32_t k4[kWaveTop], offs = 0;
#pragma unroll
  for (int r = 0; r < kWaveTop; ++r) {
    if (won) {
      const int l = __builtin_ctzll(won);
      won &= won - 1;
      k4[r] = __builtin_amdgcn_readlane(key, l);
      offs |= (uint32_t)l << (8 * r);
    } else {
      k4[r] = 0u;
      offs |= 0xffu << (8 * r);
    }
  }
  if (lane == 0) {
    *reinterpret_cast<uint4*>(keys) = make_uint4(k4[0], k4[1], k4[2], k4[3]);
    *info = make_uint2(offs, bound);
  }
}

// ------------------------------------------------------------------ selection
constexpr int kNW = kSelThreads / 64;
constexpr int kBins = 8192;

struct SelShared {
  uint32_t hist[kBins + 64];   // + one slot per lane for branch-free passes to discard into
  uint32_t wtot[kNW];
  uint32_t wmin[kNW], wmax[kNW];
  union {
    uint32_t hist2[kBins];     // second level of the register search (zeroed up front)
    struct {
      uint32_t pool_key[kPoolCap];
      uint32_t pool_id[kPoolCap];
    };
  };
  uint32_t fail[256], fcount[256], fbase[256];
  uint32_t n_pool, n_fail, flag;
  uint32_t hit_bin, hit_before;
};

// inclusive prefix sum over the workgroup (one value per thread)
__device__ __forceinline__ uint32_t block_scan(uint32_t v, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan_u32(v);
  if (lane == 63) sh.wtot[wave] = v;
  __syncthreads();
  uint32_t tot[kNW];
#pragma unroll
  for (int w = 0; w < kNW; ++w) tot[w] = sh.wtot[w];
  uint32_t add = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) add += w < wave ? tot[w] : 0u;
  __syncthreads();
  return v + add;
}

// min and max over the workgroup
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SelShared& sh, uint32_t& omn, uint32_t& omx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) { sh.wmin[wave] = mn; sh.wmax[wave] = mx; }
  __syncthreads();
  omn = sh.wmin[0];
  omx = sh.wmax[0];
  for (int w = 1; w < kNW; ++w) { omn = min(omn, sh.wmin[w]); omx = max(omx, sh.wmax[w]); }
  __syncthreads();
}

// Bin of sh.hist[0..nb) holding the r-th element (1-based) counted from the top
// (descending) or from the bottom, and the count strictly before it.
__device__ __forceinline__ void find_rank(const uint32_t* hist, SelShared& sh, int nb, uint32_t r, bool descending,
                                          uint32_t& bin, uint32_t& before) {
  constexpr int kMaxPer = kBins / kSelThreads;
  const int t = threadIdx.x;
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  uint32_t c[kMaxPer];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    const int o = t * per + e;
    c[e] = (e < per && o < nb) ? hist[descending ? nb - 1 - o : o] : 0u;
    sum += c[e];
  }
  const uint32_t incl = block_scan(sum, sh);
  const uint32_t excl = incl - sum;
  if (excl < r && r <= incl) {
    uint32_t run = excl;
    int hit = 0;
    bool found = false;
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      if (!found && run + c[e] >= r) { hit = e; found = true; }
      if (!found) run += c[e];
    }
    const int o = t * per + hit;
    sh.hit_bin = (uint32_t)(descending ? nb - 1 - o : o);
    sh.hit_before = run;
  }
  __syncthreads();
  bin = sh.hit_bin;
  before = sh.hit_before;
  __syncthreads();
}

// Rank search over the values `val(key, id)` of the elements that `each` visits and
// `keep(key, id)` accepts: returns a value v* such that the elements at or above it
// (descending; at or below it, ascending) are the r first ones plus, when r ends
// inside a run of equal values, part of that run; through r it returns how many of
// the elements equal to v* are wanted and through n_equal how many there are (both
// equal when the search stops early at a bin that is taken whole).  Bins are power-of-two slices of the live
// [lo, hi] range, so keys that sit close together spread over many bins and the
// LDS atomics stay free of contention; at most 3 levels narrow 32 bits to one value.
template <class Each, class Keep, class Val>
__device__ __forceinline__ uint32_t rank_search(Each each, Keep keep, Val val, uint32_t& r, bool descending, SelShared& sh,
                                uint32_t& n_equal) {
  uint32_t mn = 0xffffffffu, mx = 0;
  each([&](uint32_t key, uint32_t id) {
    if (keep(key, id)) { const uint32_t v = val(key, id); mn = min(mn, v); mx = max(mx, v); }
  });
  uint32_t lo, hi;
  block_minmax(mn, mx, sh, lo, hi);
  n_equal = 0;
  if (lo > hi) return lo;   // nothing accepted (callers never ask for that)
  while (true) {
    const uint64_t range = (uint64_t)hi - lo + 1;
    int shift = 0;
    while ((range >> shift) > (uint64_t)kBins) ++shift;
    const int nb = (int)(((uint64_t)(hi - lo) >> shift) + 1);
    for (int t = threadIdx.x; t < nb; t += kSelThreads) sh.hist[t] = 0;
    __syncthreads();
    each([&](uint32_t key, uint32_t id) {
      if (keep(key, id)) {
        const uint32_t v = val(key, id);
        if (v >= lo && v <= hi) atomicAdd(&sh.hist[(v - lo) >> shift], 1u);
      }
    });
    __syncthreads();
    uint32_t bin, before;
    find_rank(sh.hist, sh, nb, r, descending, bin, before);
    r -= before;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t nhi = (uint32_t)min<uint64_t>((uint64_t)hi, (uint64_t)nlo + ((uint64_t)1 << shift) - 1);
    const uint32_t in_bin = sh.hist[bin];
    __syncthreads();
    if (shift == 0) {
      n_equal = in_bin;
      return nlo;
    }
    if (r == in_bin) {
      // the wanted rank closes the bin: every element of the bin is taken, so the
      // bin edge on the far side is an exact threshold
      n_equal = in_bin;
      return descending ? nlo : nhi;
    }
    lo = nlo;
    hi = nhi;
  }
}

// A lower bound of the r-th largest key over the visited elements from one level
// of power-of-two bins over the live key range: the lower edge of the bin that
// holds the r-th element.
template <class Each>
__device__ __forceinline__ uint32_t kth_key_floor(Each each, uint32_t r, SelShared& sh) {
  uint32_t mn = 0xffffffffu, mx = 0;
  each([&](uint32_t key, uint32_t) { mn = min(mn, key); mx = max(mx, key); });
  uint32_t lo, hi;
  block_minmax(mn, mx, sh, lo, hi);
  if (lo > hi) return 0;
  const uint64_t range = (uint64_t)hi - lo + 1;
  int shift = 0;
  while ((range >> shift) > (uint64_t)kBins) ++shift;
  const int nb = (int)(((uint64_t)(hi - lo) >> shift) + 1);
  for (int t = threadIdx.x; t < nb; t += kSelThreads) sh.hist[t] = 0;
  __syncthreads();
  each([&](uint32_t key, uint32_t) { atomicAdd(&sh.hist[(key - lo) >> shift], 1u); });
  __syncthreads();
  uint32_t bin, before;
  find_rank(sh.hist, sh, nb, r, true, bin, before);
  return lo + (bin << shift);
}

// The key threshold T and the largest tie id of the exact top-k over the visited
// elements: an element is selected iff key > T, or key == T and id <= id_max.
template <class Each>
__device__ __forceinline__ void topk_threshold(Each each, uint32_t k, SelShared& sh, uint32_t& T, uint32_t& id_max) {
  uint32_t r = k, n_tie;
  T = rank_search(each, [](uint32_t, uint32_t) { return true; },
                  [](uint32_t key, uint32_t) { return key; }, r, true, sh, n_tie);
  id_max = 0xffffffffu;
  if (r < n_tie) {      // ties at T: the r lowest ids among them
    uint32_t n_eq;
    id_max = rank_search(each, [T](uint32_t key, uint32_t) { return key == T; },
                         [](uint32_t, uint32_t id) { return id; }, r, false, sh, n_eq);
  }
}

__device__ __forceinline__ bool picked(uint32_t key, uint32_t id, uint32_t T, uint32_t id_max) {
  return key > T || (key == T && id <= id_max);
}
// the same as 0 / 1, without short-circuit branches
__device__ __forceinline__ uint32_t picked_bits(uint32_t key, uint32_t id, uint32_t T, uint32_t id_max) {
  return (uint32_t)(key > T) | ((uint32_t)(key == T) & (uint32_t)(id <= id_max));
}

constexpr int kMaxTilesPerThread = 3;

// Rank search (descending) over the report keys held in registers, keys[q][j] for
// q < tpt (0 = no element): as rank_search, but every pass is branch-free (an
// element outside the live range adds into its lane's discard slot).
__device__ __forceinline__ uint32_t reg_rank_search(const uint32_t (&keys)[kMaxTilesPerThread][kTileTop], int tpt,
                                                    uint32_t& r, SelShared& sh, uint32_t& n_equal) {
  const int lane = threadIdx.x & 63;
  uint32_t mn = 0xffffffffu, mx = 0;
#pragma unroll
  for (int q = 0; q < kMaxTilesPerThread; ++q) {
    if (q >= tpt) break;
#pragma unroll
    for (int j = 0; j < kTileTop; ++j) {
      const uint32_t v = keys[q][j];
      mx = max(mx, v);
      mn = min(mn, v ? v : 0xffffffffu);
    }
  }
  uint32_t lo, hi;
  block_minmax(mn, mx, sh, lo, hi);
  n_equal = 0;
  if (lo > hi) return lo;
  for (int level = 0;; ++level) {
    const uint64_t range = (uint64_t)hi - lo + 1;
    int shift = 0;
    while ((range >> shift) > (uint64_t)kBins) ++shift;
    const int nb = (int)(((uint64_t)(hi - lo) >> shift) + 1);
    // levels 0 and 1 count into sh.hist and sh.hist2, which the caller zeroed
    uint32_t* h = (level & 1) ? sh.hist2 : sh.hist;
    if (level >= 2) {
      for (int t = threadIdx.x; t < nb; t += kSelThreads) h[t] = 0;
      __syncthreads();
    }
    const uint32_t span = hi - lo;
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q) {
      if (q >= tpt) break;
#pragma unroll
      for (int j = 0; j < kTileTop; ++j) {
        const uint32_t d = keys[q][j] - lo;   // wraps for keys below lo (and for 0)
        atomicAdd(d <= span ? &h[d >> shift] : &sh.hist[kBins + lane], 1u);
      }
    }
    __syncthreads();
    uint32_t bin, before;
    find_rank(h, sh, nb, r, true, bin, before);
    r -= before;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t nhi = (uint32_t)min<uint64_t>((uint64_t)hi, (uint64_t)nlo + ((uint64_t)1 << shift) - 1);
    const uint32_t in_bin = h[bin];
    __syncthreads();
    if (shift == 0 || r == in_bin) {   // one value left, or the bin is taken whole
      n_equal = in_bin;
      return nlo;
    }
    lo = nlo;
    hi = nhi;
  }
}

// Emits out[0..k) from the LDS pool (ascending ids) by an order-preserving
// compaction of the picked entries; every thread owns a contiguous pool range.
__device__ __forceinline__ void emit_pool(SelShared& sh, uint32_t np, uint32_t k, uint32_t T, uint32_t id_max,
                                          int32_t* out, float* selp, const float* sc) {
  const uint32_t per = (np + kSelThreads - 1) / kSelThreads;
  const uint32_t lo = min(np, threadIdx.x * per), hi = min(np, lo + per);
  uint32_t c = 0;
  for (uint32_t t = lo; t < hi; ++t) c += picked(sh.pool_key[t], sh.pool_id[t], T, id_max) ? 1u : 0u;
  uint32_t o = block_scan(c, sh) - c;
  for (uint32_t t = lo; t < hi; ++t) {
    const uint32_t id = sh.pool_id[t];
    if (picked(sh.pool_key[t], id, T, id_max)) {
      if (o < k) {
        out[o] = (int32_t)id;
        if (selp) selp[o] = sc[id];
      }
      ++o;
    }
  }
}

// The selection of row lr of the launch (one kSelThreads-thread workgroup).
__device__ __forceinline__ void select_row(const SelectP& p, int lr, SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* RK = p.rep_key + (int64_t)lr * p.key_rs;
  const uint2* RI = p.rep_info + (int64_t)lr * p.info_rs;
  // thread t owns tiles [t*tpt, t*tpt + tpt) of the longest row; the report loads do
  // not wait for the row's position (tiles past the row's own end are dropped below)
  const int64_t ntc = p.ntiles_cap;
  const int tpt = (int)min<int64_t>(kMaxTilesPerThread + 1, (ntc + kSelThreads - 1) / kSelThreads);
  bool ok = tpt <= kMaxTilesPerThread;
  uint4 rk[kMaxTilesPerThread][kTileTop / 4], ri[kMaxTilesPerThread][2];
#pragma unroll
  for (int q = 0; q < kMaxTilesPerThread; ++q) {
    if (ok && q < tpt) {
      const int64_t tl = min<int64_t>((int64_t)tid * tpt + q, ntc - 1);
      const uint4* ks = reinterpret_cast<const uint4*>(RK + tl * kTileTop);
      const uint4* is = reinterpret_cast<const uint4*>(RI + tl * 4);
#pragma unroll
      for (int j = 0; j < kTileTop / 4; ++j) rk[q][j] = ks[j];
      ri[q][0] = is[0];
      ri[q][1] = is[1];
    } else {
#pragma unroll
      for (int j = 0; j < kTileTop / 4; ++j) rk[q][j] = make_uint4(0u, 0u, 0u, 0u);
      ri[q][0] = ri[q][1] = make_uint4(0xffffffffu, 0u, 0xffffffffu, 0u);
    }
  }
  // the two histogram levels of the register search start at zero (cleared while
  // the reports load; the search's first barrier orders this before any count)
  {
    u32x4* h1 = reinterpret_cast<u32x4*>(sh.hist);
    u32x4* h2 = reinterpret_cast<u32x4*>(sh.hist2);
    for (int t = tid; t < kBins / 4; t += kSelThreads) {
      h1[t] = u32x4{0u, 0u, 0u, 0u};
      h2[t] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int k = p.topk;
  int32_t* out = p.idx + (int64_t)b * p.idx_bs + (int64_t)i * p.idx_rs;
  float* selp = p.sel ? p.sel + (int64_t)b * p.sel_bs + (int64_t)i * p.sel_rs : nullptr;
  const float* sc = p.scores + (int64_t)lr * p.sc_rs;
  if (nvis <= k) {
    for (int t = tid; t < k; t += kSelThreads) {
      out[t] = t < nvis ? t : -1;
      if (selp) selp[t] = t < nvis ? sc[t] : 0.f;
    }
    return;
  }
  const int64_t ntiles = (nvis + kTile - 1) / kTile;
  ok = ok && ntiles <= ntc;

  // report keys, packed id offsets (the id of entry j of tile t is t*256 + (j/4)*64 +
  // offset) and the largest wave bound of each owned tile
  uint32_t uk[kMaxTilesPerThread][kTileTop], uo[kMaxTilesPerThread][kTileTop / 4], ub[kMaxTilesPerThread];
  bool own[kMaxTilesPerThread];
  int64_t tbase[kMaxTilesPerThread];
#pragma unroll
  for (int q = 0; q < kMaxTilesPerThread; ++q) {
    const int64_t t = (int64_t)tid * tpt + q;
    own[q] = ok && q < tpt && t < ntiles;
    tbase[q] = t * kTile;
#pragma unroll
    for (int w = 0; w < kTileTop / 4; ++w) {
      uk[q][4 * w] = rk[q][w].x; uk[q][4 * w + 1] = rk[q][w].y;
      uk[q][4 * w + 2] = rk[q][w].z; uk[q][4 * w + 3] = rk[q][w].w;
    }
    uo[q][0] = own[q] ? ri[q][0].x : 0xffffffffu;
    uo[q][1] = own[q] ? ri[q][0].z : 0xffffffffu;
    uo[q][2] = own[q] ? ri[q][1].x : 0xffffffffu;
    uo[q][3] = own[q] ? ri[q][1].z : 0xffffffffu;
    ub[q] = own[q] ? max(max(ri[q][0].y, ri[q][0].w), max(ri[q][1].y, ri[q][1].w)) : 0u;
    // key 0 marks no element from here on
#pragma unroll
    for (int j = 0; j < kTileTop; ++j)
      if (((uo[q][j / 4] >> (8 * (j % 4))) & 0xffu) == 0xffu) uk[q][j] = 0u;
  }
  auto rep_id = [&](int q, int j) -> uint32_t {
    return (uint32_t)tbase[q] + 64u * (j / 4) + ((uo[q][j / 4] >> (8 * (j % 4))) & 0xffu);
  };
  auto eachOwn = [&](auto&& f) {
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q)
#pragma unroll
      for (int j = 0; j < kTileTop; ++j) {
        const uint32_t off = (uo[q][j / 4] >> (8 * (j % 4))) & 0xffu;
        if (own[q] && off != 0xffu) f(uk[q][j], (uint32_t)tbase[q] + 64u * (j / 4) + off);
      }
  };
  // every wave of 64 visible blocks reports kWaveTop of them, a partial last wave
  // as many as it has
  const int64_t n_rep = kWaveTop * (nvis / 64) + min<int64_t>(kWaveTop, nvis % 64);

  if (ok && n_rep >= k) {
    // 1. the exact k-th key T of all the reports
    uint32_t r = (uint32_t)k, n_tie;
    const uint32_t T = reg_rank_search(uk, tpt, r, sh, n_tie);
    // 2. no tile hides a key >= T: the reports hold every element >= T and their top-k
    //    is the row's; compacted in id order from the registers through LDS
    bool hides = false;
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q) hides |= own[q] && ub[q] >= T;
    if (!__syncthreads_or(hides) && T != 0u) {
      uint32_t id_max = 0xffffffffu;
      if (r < n_tie)
        id_max = rank_search(eachOwn, [T](uint32_t key, uint32_t) { return key == T; },
                             [](uint32_t, uint32_t id) { return id; }, r, false, sh, n_tie);
      if (id_max == 0xffffffffu) {
        // no cut inside the ties at T: the picks are the keys >= T (keys of no element
        // are 0 < T).  A bit per entry, then only the set bits are visited.
        uint64_t mask = 0;
#pragma unroll
        for (int q = 0; q < kMaxTilesPerThread; ++q) {
          if (q >= tpt) break;
#pragma unroll
          for (int j = 0; j < kTileTop; ++j) mask |= (uint64_t)(uk[q][j] >= T) << (q * kTileTop + j);
        }
        const uint32_t c = (uint32_t)__popcll(mask);
        uint32_t o = block_scan(c, sh) - c;
        while (mask) {
          const int j = __builtin_ctzll(mask);
          mask &= mask - 1;
          const int q = j / kTileTop, wv = (j % kTileTop) / 4, e = j % 4;
          uint32_t word = uo[0][0];
#pragma unroll
          for (int qq = 0; qq < kMaxTilesPerThread; ++qq)
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) word = (q * 4 + wv == qq * 4 + ww) ? uo[qq][ww] : word;
          const uint32_t id = (uint32_t)(((int64_t)tid * tpt + q) * kTile) + 64u * wv + ((word >> (8 * e)) & 0xffu);
          if (o < (uint32_t)k) sh.pool_id[o] = id;
          ++o;
        }
      } else {
        // branch-free per entry
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < kMaxTilesPerThread; ++q) {
          if (q >= tpt) break;
#pragma unroll
          for (int j = 0; j < kTileTop; ++j) c += picked_bits(uk[q][j], rep_id(q, j), T, id_max);
        }
        uint32_t o = block_scan(c, sh) - c;
#pragma unroll
        for (int q = 0; q < kMaxTilesPerThread; ++q) {
          if (q >= tpt) break;
#pragma unroll
          for (int j = 0; j < kTileTop; ++j) {
            const uint32_t id = rep_id(q, j);
            const uint32_t pk = picked_bits(uk[q][j], id, T, id_max);
            *((pk & (o < (uint32_t)k)) ? &sh.pool_id[o] : &sh.hist[kBins + lane]) = id;
            o += pk;
          }
        }
      }
      __syncthreads();
      for (int t = tid; t < k; t += kSelThreads) {
        const uint32_t id = sh.pool_id[t];
        out[t] = (int32_t)id;
        if (selp) selp[t] = sc[id];
      }
      return;
    }
    {
      // 5. some tiles may hide elements >= T: pool = reports >= T of the other tiles
      //    plus every element >= T of those tiles (rescanned), in id order
      if (tid == 0) sh.n_fail = 0;
      __syncthreads();
      int fslot[kMaxTilesPerThread];
      uint32_t cnt[kMaxTilesPerThread];
      bool over = false;
#pragma unroll
      for (int q = 0; q < kMaxTilesPerThread; ++q) {
        fslot[q] = -1;
        cnt[q] = 0;
        if (!own[q]) continue;
#pragma unroll
        for (int j = 0; j < kTileTop; ++j)
          if (((uo[q][j / 4] >> (8 * (j % 4))) & 0xffu) != 0xffu) cnt[q] += uk[q][j] >= T ? 1u : 0u;
        if (ub[q] >= T) {
          const uint32_t slot = atomicAdd(&sh.n_fail, 1u);
          if (slot < 256u) { fslot[q] = (int)slot; sh.fail[slot] = (uint32_t)((int64_t)tid * tpt + q); }
          else over = true;
        }
      }
      over = __syncthreads_or(over);
      const uint32_t nf = min(sh.n_fail, 256u);
      if (!over) {
        // a wave counts the elements >= T of its failing tiles, all loads in flight
        for (uint32_t f = wave; f < nf; f += kNW) {
          const int64_t base = (int64_t)sh.fail[f] * kTile;
          uint32_t kk[kTile / 64];
#pragma unroll
          for (int rr = 0; rr < kTile / 64; ++rr) {
            const int64_t j = base + rr * 64 + lane;
            kk[rr] = j < nvis ? score_key(sc[j]) : 0u;
          }
          uint32_t c = 0;
#pragma unroll
          for (int rr = 0; rr < kTile / 64; ++rr) c += __popcll(__ballot(base + rr * 64 + lane < nvis && kk[rr] >= T));
          if (lane == 0) sh.fcount[f] = c;
        }
        __syncthreads();
        uint32_t mine = 0;
#pragma unroll
        for (int q = 0; q < kMaxTilesPerThread; ++q) {
          if (fslot[q] >= 0) cnt[q] = sh.fcount[fslot[q]];
          mine += cnt[q];
        }
        const uint32_t incl = block_scan(mine, sh);
        if (tid == kSelThreads - 1) sh.n_pool = incl;
        __syncthreads();
        const uint32_t np2 = sh.n_pool;
        if (np2 <= (uint32_t)kPoolCap) {
          uint32_t off = incl - mine;
#pragma unroll
          for (int q = 0; q < kMaxTilesPerThread; ++q) {
            if (fslot[q] >= 0) {
              sh.fbase[fslot[q]] = off;
              off += cnt[q];
            } else if (own[q]) {
#pragma unroll
              for (int j = 0; j < kTileTop; ++j) {
                const uint32_t wo = (uo[q][j / 4] >> (8 * (j % 4))) & 0xffu;
                if (wo != 0xffu && uk[q][j] >= T) {
                  sh.pool_key[off] = uk[q][j];
                  sh.pool_id[off] = (uint32_t)tbase[q] + 64u * (j / 4) + wo;
                  ++off;
                }
              }
            }
          }
          __syncthreads();
          for (uint32_t f = wave; f < nf; f += kNW) {
            const int64_t base = (int64_t)sh.fail[f] * kTile;
            uint32_t o = sh.fbase[f];
#pragma unroll
            for (int rr = 0; rr < kTile / 64; ++rr) {
              const int64_t j = base + rr * 64 + lane;
              const uint32_t key = j < nvis ? score_key(sc[j]) : 0u;
              const bool hit = j < nvis && key >= T;
              const uint64_t m = __ballot(hit);
              if (hit) {
                const uint32_t at = o + __popcll(m & ((1ull << lane) - 1));
                sh.pool_key[at] = key;
                sh.pool_id[at] = (uint32_t)j;
              }
              o += __popcll(m);
            }
          }
          __syncthreads();
          uint32_t T2, id2;
          auto eachP2 = [&](auto&& f) { for (uint32_t t = tid; t < np2; t += kSelThreads) f(sh.pool_key[t], sh.pool_id[t]); };
          topk_threshold(eachP2, (uint32_t)k, sh, T2, id2);
          emit_pool(sh, np2, (uint32_t)k, T2, id2, out, selp, sc);
          return;
        }
      }
    }
  }

  // whole-row path (ties everywhere, too many rescans, or more tiles than registers hold)
  uint32_t T, id_max;
  auto eachR = [&](auto&& f) {
    for (int64_t t = tid; t < nvis; t += kSelThreads) f(score_key(sc[t]), (uint32_t)t);
  };
  topk_threshold(eachR, (uint32_t)k, sh, T, id_max);
  const int64_t per = (nvis + kSelThreads - 1) / kSelThreads;
  const int64_t lo = min<int64_t>(nvis, (int64_t)tid * per), hi = min<int64_t>(nvis, lo + per);
  uint32_t c = 0;
  for (int64_t t = lo; t < hi; ++t) c += picked(score_key(sc[t]), (uint32_t)t, T, id_max) ? 1u : 0u;
  uint32_t o = block_scan(c, sh) - c;
  for (int64_t t = lo; t < hi; ++t) {
    const float v = sc[t];
    if (picked(score_key(v), (uint32_t)t, T, id_max)) {
      if (o < (uint32_t)k) {
        out[o] = (int32_t)t;
        if (selp) selp[o] = v;
      }
      ++o;
    }
  }
}

}  // namespace v4a
