// Device code of the indexer: helpers shared by the score and select kernels and
// the per-row selection, which the combined selection + attention kernel of the
// decode step runs too.  The design notes are at the top of index.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"
#include <utility>

namespace v4a {

__device__ __forceinline__ void row_coords(int row, int tq, const int64_t* pos0, int& b, int& i,
                                           int64_t& pos) {
  b = row / tq;
  i = row - b * tq;
  pos = pos0[b] + i;
}

// Reports of the score kernels, per tile of kTile = 256 blocks: the keys of the
// tile's best blocks, kTileTop of them in decode (the selection is on the step's
// critical path, so its rescans should be rare) and 4 in prefill (about one block
// per tile is picked there, and a rescan costs the selection little), in ascending
// id order (key 0 = no element); and an info word (offsets of entries 0-3, offsets
// of entries 4-7, bound, 0): 8-bit offsets from the tile's first block, and the key
// of the best block the report leaves out (0 if none), which bounds every other one.

// Lane `dst` receives v (a forward permute); every lane sends, so lanes with nothing
// to send aim at lane 63, which no caller reads.
__device__ __forceinline__ uint32_t lane_send(uint32_t v, int dst) {
  return (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)v);
}
// number of set bits of m below this lane
__device__ __forceinline__ uint32_t bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The tile report made by one wave whose lane L holds the keys kb[q] of blocks
// 64 q + L (0 for none): the entries won[q] (bit L: block 64 q + L) are written in
// id order, keys (kTileTop words, empty ones 0) and info, with the bound given.
// The winners go to lanes 0.. in id order (a forward permute per quarter).
__device__ __forceinline__ void tile_emit(const uint32_t (&kb)[4], const uint64_t (&won)[4], uint32_t bound,
                                          uint32_t* keys, uint4* info) {
  const int lane = threadIdx.x & 63;
  uint32_t base = 0, rk = 0u, ro = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool w = (won[q] >> lane) & 1ull;
    const int dst = w ? (int)(base + bits_below(won[q])) : 63;
    const uint32_t gk = lane_send(kb[q], dst), go = lane_send(64u * q + lane, dst);
    const uint32_t nq = (uint32_t)__popcll(won[q]);
    if (lane >= (int)base && lane < (int)(base + nq)) { rk = gk; ro = go; }
    base += nq;
  }
  if (lane < kTileTop) keys[lane] = lane < (int)base ? rk : 0u;
  // the offsets as bytes of two words (lanes 0..3 and 4..7): OR over each quad
  uint32_t word = lane < (int)base ? (ro & 0xffu) << (8 * (lane & 3)) : 0u;
  word |= dpp_u32<0xB1>(0u, word);   // quad_perm [1,0,3,2]
  word |= dpp_u32<0x4E>(0u, word);   // quad_perm [2,3,0,1]
  const uint32_t word1 = __builtin_amdgcn_readlane(word, 4);
  if (lane == 0) *info = make_uint4(word, word1, bound, 0u);
}

// The same report when the entries are known to be at most kTileTop: each winner
// stores its own key and its offset byte at its rank in id order, the lanes past the
// last entry clear the remaining key slots (an empty entry's offset byte is never
// read), and no value crosses lanes.
__device__ __forceinline__ void tile_emit_few(const uint32_t (&kb)[4], const uint64_t (&won)[4], uint32_t bound,
                                              uint32_t* keys, uint4* info) {
  const int lane = threadIdx.x & 63;
  unsigned char* offs = reinterpret_cast<unsigned char*>(info);
  uint32_t base = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if ((won[q] >> lane) & 1ull) {
      const uint32_t at = base + bits_below(won[q]);
      keys[at] = kb[q];
      offs[at] = (unsigned char)(64 * q + lane);
    }
    base += (uint32_t)__popcll(won[q]);
  }
  if (lane >= (int)base && lane < kTileTop) keys[lane] = 0u;
  if (lane == 0) reinterpret_cast<uint2*>(info)[1] = make_uint2(bound, 0u);
}

// The R <= kTileTop best of the wave's 256 keys (entries past R are empty).  Each of
// R rounds takes a 32-bit wave maximum (DPP) of the keys not yet taken and takes one
// block holding it: the lowest lane with it, and that lane's first quarter.  Which of
// several equal keys is taken does not matter for the selection: if one is left out,
// the bound (one more maximum) equals that key, so a threshold at it sends the tile
// to a rescan.
template <int R>
__device__ __forceinline__ void tile_rounds(const uint32_t (&kb)[4], uint64_t (&won)[4], uint32_t& bound) {
  static_assert(kTileTop == 8 && R >= 1 && R <= kTileTop, "two offset words per tile");
  const int lane = threadIdx.x & 63;
  uint32_t k[4] = {kb[0], kb[1], kb[2], kb[3]};
#pragma unroll
  for (int q = 0; q < 4; ++q) won[q] = 0ull;
#pragma unroll 1
  for (int r = 0; r < R; ++r) {
    const uint32_t lm = max(max(k[0], k[1]), max(k[2], k[3]));
    const uint32_t m = wave_max_u32(lm);
    if (m == 0u) break;
    const int l = __builtin_ctzll(__ballot(lm == m));
    const int qs = k[0] == m ? 0 : k[1] == m ? 1 : k[2] == m ? 2 : 3;   // lane-local
    const int qw = __builtin_amdgcn_readlane(qs, l);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q == qw) won[q] |= 1ull << l;
      if (lane == l && q == qs) k[q] = 0u;
    }
  }
  bound = wave_max_u32(max(max(k[0], k[1]), max(k[2], k[3])));
}

template <int R>
__device__ __forceinline__ void tile_report(const uint32_t (&kb)[4], uint32_t* keys, uint4* info) {
  uint64_t won[4];
  uint32_t bound;
  tile_rounds<R>(kb, won, bound);
  tile_emit(kb, won, bound, keys, info);
}

// Rounds of a wave maximum over one key per lane (0 = none): the lanes of the n <= R
// best keys (the lowest lane among equal ones) and, through rest, the best key left.
template <int R>
__device__ __forceinline__ uint64_t wave_best(uint32_t k, int n, uint32_t& rest) {
  const int lane = threadIdx.x & 63;
  uint64_t won = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= n) break;
    const uint32_t m = wave_max_u32(k);
    if (m == 0u) break;
    const int l = __builtin_ctzll(__ballot(k == m));
    won |= 1ull << l;
    if (lane == l) k = 0u;
  }
  rest = wave_max_u32(k);
  return won;
}

// The report of a tile whose four 64-block quarters are the four waves of a
// workgroup (lane L of wave w holds block 64 w + L).  Each wave first takes its own
// wtop best keys (wtop <= kTileTop) as candidates, in lane order; then wave 0 ranks
// the 4 wtop candidates, which are in id order, and the kTileTop best need only a
// compaction.  Every block left out is either a candidate
// that lost or a key a wave kept back, so the bound is the larger of the best losing
// candidate and the waves' best kept-back keys.  (A wave holding more than wtop of
// the tile's best makes the bound one of them: its tile is rescanned if that reaches
// the threshold.)  [parity]: a tile's candidates are read before the next tile's are
// written (a barrier separates the two).  Called by all four waves (holds a barrier).
struct TileStage {
  uint32_t key[2][4 * kTileTop];   // candidates, wave-major (key 0: none)
  uint32_t off[2][4 * kTileTop];   // their offsets in the tile
  uint32_t rest[2][4];             // each wave's best key past its candidates
};
__device__ __forceinline__ void tile_report_waves(uint32_t key, bool valid, int par, int wtop, TileStage& st,
                                                  uint32_t* keys, uint4* info) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t k = valid ? key : 0u;
  uint32_t rest;
  const uint64_t won = wave_best<kTileTop>(k, wtop, rest);
  const int cnt = __popcll(won);
  if ((won >> lane) & 1ull) {
    const int slot = wave * wtop + (int)bits_below(won);
    st.key[par][slot] = k;
    st.off[par][slot] = (uint32_t)(wave * 64 + lane);
  }
  if (lane >= cnt && lane < wtop) st.key[par][wave * wtop + lane] = 0u;
  if (lane == 0) st.rest[par][wave] = rest;
  __syncthreads();
  if (wave == 0) {
    const int nc = 4 * wtop;
    const uint32_t ck = lane < nc ? st.key[par][lane] : 0u;
    const uint32_t co = lane < nc ? st.off[par][lane] : 0u;
    const uint32_t kept = max(max(st.rest[par][0], st.rest[par][1]), max(st.rest[par][2], st.rest[par][3]));
    // each candidate counts the candidates ahead of it (a larger key, or an equal one in
    // a lower slot): independent steps, no chain of wave maxima.  The ranks are
    // distinct, so the kTileTop best win and rank kTileTop is the best one lost.
    uint32_t ahead = 0;
#pragma unroll
    for (int j = 0; j < 4 * kTileTop; ++j) {
      if (j >= nc) break;
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ck, j);
      ahead += (kj > ck || (kj == ck && j < lane)) ? 1u : 0u;
    }
    const uint64_t w2 = __ballot(ck != 0u && ahead < (uint32_t)kTileTop);
    const uint64_t l2 = __ballot(ck != 0u && ahead == (uint32_t)kTileTop);
    const uint32_t lost = l2 ? (uint32_t)__builtin_amdgcn_readlane((int)ck, (int)__builtin_ctzll(l2)) : 0u;
    const uint32_t bound = max(lost, kept);
    const int n = __popcll(w2);
    const int dst = ((w2 >> lane) & 1ull) ? (int)bits_below(w2) : 63;
    const uint32_t gk = lane_send(ck, dst), go = lane_send(co, dst);
    if (lane < kTileTop) keys[lane] = lane < n ? gk : 0u;
    // the offsets as bytes of two words (entries 0..3 and 4..7): OR over each quad
    uint32_t word = lane < n ? (go & 0xffu) << (8 * (lane & 3)) : 0u;
    word |= dpp_u32<0xB1>(0u, word);   // quad_perm [1,0,3,2]
    word |= dpp_u32<0x4E>(0u, word);   // quad_perm [2,3,0,1]
    const uint32_t word1 = __builtin_amdgcn_readlane(word, 4);
    if (lane == 0) *info = make_uint4(word, word1, bound, 0u);
  }
}

// ------------------------------------------------------------------ selection
constexpr int kNW = kSelThreads / 64;
constexpr int kBins = 8192;
constexpr int kGatherMax = 64;   // a bin of at most this many keys is ranked by one wave

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
  uint32_t n_gather, gres[3];
  uint32_t gkey[kGatherMax];   // the few keys of one histogram bin (reg_rank_search)
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

// Width (as a shift) of the power-of-two bins over [lo, hi] (lo <= hi): the
// smallest one for which the bin of hi, (hi - lo) >> shift, is below kBins, so the
// nb = ((hi - lo) >> shift) + 1 bins fit the histogram.  Bounding the rounded-up
// count of bins rather than (hi - lo + 1) >> shift matters when that quotient is
// exactly kBins with a remainder: that range needs kBins + 1 bins of that width.
__device__ __forceinline__ int bin_shift(uint32_t lo, uint32_t hi) {
  int shift = 0;
  while (((hi - lo) >> shift) >= (uint32_t)kBins) ++shift;
  return shift;
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
    const int shift = bin_shift(lo, hi);
    const int nb = (int)((hi - lo) >> shift) + 1;
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
  const int shift = bin_shift(lo, hi);
  const int nb = (int)((hi - lo) >> shift) + 1;
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
  if (threadIdx.x == 0) sh.n_gather = 0;   // (ordered before the gather by the barriers below)
  uint32_t lo, hi;
  block_minmax(mn, mx, sh, lo, hi);
  n_equal = 0;
  if (lo > hi) return lo;
  for (int level = 0;; ++level) {
    const int shift = bin_shift(lo, hi);
    const int nb = (int)((hi - lo) >> shift) + 1;
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
    if (in_bin <= (uint32_t)kGatherMax) {
      // few keys in the bin: gathered into LDS, and one wave ranks them by counting
      // (lane i holds key i and counts the keys above it and equal to it); the r-th
      // largest is the key of a lane with above < r <= above + equal
#pragma unroll
      for (int q = 0; q < kMaxTilesPerThread; ++q) {
        if (q >= tpt) break;
#pragma unroll
        for (int j = 0; j < kTileTop; ++j) {
          const uint32_t v = keys[q][j];
          if (v >= nlo && v <= nhi) sh.gkey[atomicAdd(&sh.n_gather, 1u)] = v;
        }
      }
      __syncthreads();
      if ((threadIdx.x >> 6) == 0) {
        const uint32_t mine = lane < (int)in_bin ? sh.gkey[lane] : 0u;
        uint32_t above = 0, equal = 0;
        for (uint32_t j = 0; j < in_bin; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mine, (int)j);
          above += kj > mine ? 1u : 0u;
          equal += kj == mine ? 1u : 0u;
        }
        const bool hit = lane < (int)in_bin && above < r && r <= above + equal;
        if (lane == (int)__builtin_ctzll(__ballot(hit))) {
          sh.gres[0] = mine;
          sh.gres[1] = r - above;
          sh.gres[2] = equal;
        }
      }
      __syncthreads();
      r = sh.gres[1];
      n_equal = sh.gres[2];
      return sh.gres[0];
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
  if (p.repair && p.repair[lr] == 0u) return;   // a repair pass: flagged rows only
  // threshold mode: the reports hold every key >= th of the tiles that stored no
  // scores; a row whose k-th key turns out below th is flagged (and left to an exact
  // repair pass) instead of selected.  thread 0 writes the flag, first clearing it.
  const bool tmode = p.theta != nullptr;
  const uint32_t th = tmode ? p.theta[lr] : 0u;
  if (tmode && tid == 0) p.flag[lr] = 0u;
  const uint32_t* RK = p.rep_key + (int64_t)lr * p.key_rs;
  const uint4* RI = p.rep_info + (int64_t)lr * p.info_rs;
  // thread t owns tiles [t*tpt, t*tpt + tpt) of the longest row; the report loads do
  // not wait for the row's position (tiles past the row's own end are dropped below)
  const int64_t ntc = p.ntiles_cap;
  const int tpt = (int)min<int64_t>(kMaxTilesPerThread + 1, (ntc + kSelThreads - 1) / kSelThreads);
  bool ok = tpt <= kMaxTilesPerThread;
  uint4 rk[kMaxTilesPerThread][kTileTop / 4], ri[kMaxTilesPerThread];
#pragma unroll
  for (int q = 0; q < kMaxTilesPerThread; ++q) {
    if (ok && q < tpt) {
      const int64_t tl = min<int64_t>((int64_t)tid * tpt + q, ntc - 1);
      const uint4* ks = reinterpret_cast<const uint4*>(RK + tl * kTileTop);
#pragma unroll
      for (int j = 0; j < kTileTop / 4; ++j) rk[q][j] = ks[j];
      ri[q] = RI[tl];
    } else {
#pragma unroll
      for (int j = 0; j < kTileTop / 4; ++j) rk[q][j] = make_uint4(0u, 0u, 0u, 0u);
      ri[q] = make_uint4(0u, 0u, 0u, 0u);
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

  // report keys (0: no element), packed id offsets (the id of entry j of tile t is
  // t*256 + its offset) and the bound of each owned tile
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
    uo[q][0] = ri[q].x;
    uo[q][1] = ri[q].y;
    ub[q] = own[q] ? ri[q].z : 0u;
#pragma unroll
    for (int j = 0; j < kTileTop; ++j) uk[q][j] = own[q] ? uk[q][j] : 0u;
  }
  auto rep_id = [&](int q, int j) -> uint32_t {
    return (uint32_t)tbase[q] + ((uo[q][j / 4] >> (8 * (j % 4))) & 0xffu);
  };
  auto eachOwn = [&](auto&& f) {
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q)
#pragma unroll
      for (int j = 0; j < kTileTop; ++j)
        if (uk[q][j] != 0u) f(uk[q][j], rep_id(q, j));
  };
  // every tile of 256 visible blocks reports rep_top of them, a partial last tile
  // at most as many as it has; in threshold mode the count is the reports' own
  int64_t n_rep = (int64_t)p.rep_top * (nvis / kTile) + min<int64_t>(p.rep_top, nvis % kTile);
  if (tmode) {
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q)
#pragma unroll
      for (int j = 0; j < kTileTop; ++j) c += uk[q][j] != 0u ? 1u : 0u;
    const uint32_t incl = block_scan(c, sh);
    if (tid == kSelThreads - 1) sh.n_pool = incl;
    __syncthreads();
    n_rep = sh.n_pool;
    __syncthreads();
  }

  if (ok && n_rep >= k) {
    // 1. the exact k-th key T of all the reports
    uint32_t r = (uint32_t)k, n_tie;
    const uint32_t T = reg_rank_search(uk, tpt, r, sh, n_tie);
    if (tmode && T < th) {   // keys in [T, th) may sit in tiles that stored nothing
      if (tid == 0) p.flag[lr] = 1u;
      return;
    }
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
        // (written out directly: exactly k picks, in id order across threads)
        const uint32_t c = (uint32_t)__popcll(mask);
        uint32_t o = block_scan(c, sh) - c;
        while (mask) {
          const int j = __builtin_ctzll(mask);
          mask &= mask - 1;
          constexpr int OW = kTileTop / 4;   // offset words per tile
          const int q = j / kTileTop, wv = (j % kTileTop) / 4, e = j % 4;
          uint32_t word = uo[0][0];
#pragma unroll
          for (int qq = 0; qq < kMaxTilesPerThread; ++qq)
#pragma unroll
            for (int ww = 0; ww < OW; ++ww) word = (q * OW + wv == qq * OW + ww) ? uo[qq][ww] : word;
          const uint32_t id = (uint32_t)(((int64_t)tid * tpt + q) * kTile) + ((word >> (8 * e)) & 0xffu);
          if (o < (uint32_t)k) {
            out[o] = (int32_t)id;
            if (selp) selp[o] = sc[id];
          }
          ++o;
        }
        return;
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
        for (int j = 0; j < kTileTop; ++j) cnt[q] += (uk[q][j] != 0u && uk[q][j] >= T) ? 1u : 0u;
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
                if (uk[q][j] != 0u && uk[q][j] >= T) {
                  sh.pool_key[off] = uk[q][j];
                  sh.pool_id[off] = rep_id(q, j);
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

  // whole-row path (ties everywhere, too many rescans, or more tiles than registers
  // hold); in threshold mode not every score is stored: the row is flagged instead
  if (tmode) {
    if (tid == 0) p.flag[lr] = 1u;
    return;
  }
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
