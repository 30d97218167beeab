// csa_indexer_score + topk_select.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制,
// CSA step 2: a light indexer scores every compressed block for each query token and
// the query keeps its top-k blocks (yage.ai essay on the agentic workload, three-tier
// section: k = 1024 for Pro, 512 for Flash).  Score form fixed by the layer
// configuration: s_j = sum_h w_h * ReLU(qi_h . ki_j).
//
// Two launches per group of query rows, with no global atomics and no state that
// has to be cleared between calls:
//   score   one workgroup per (tile of 256 blocks, row): bf16 MFMA 16x16x32 (indexer
//           heads on M, blocks on N) or fp32 VALU.  Writes the fp32 scores and the
//           tile's 8 best (key, id) pairs.
//   select  one 1024-thread workgroup per row.  The k-th largest key among all tile
//           summaries is a lower bound tau of the row's true k-th key (any subset's
//           k-th largest is).  A tile whose 8th best key is below tau has no other
//           element >= tau; tiles that fail this test are rescanned.  The pool of
//           every element with key >= tau (LDS) therefore holds the top-k, which a
//           rank search over power-of-two slices of the live key range (then of the
//           ids, for ties: the lower id wins) extracts exactly.  Tiles report their 8
//           in id order and the pool is built by order-preserving compaction, so the
//           k ids come out ascending without a sort.  If the pool would overflow LDS
//           (or a row has more than 2048 tiles), the same search and compaction run
//           over the whole row instead.  Rows with n_vis < k are padded with -1.
// Keys are the order-preserving uint32 image of the fp32 scores, so "larger key" is
// "larger score"; the result does not depend on launch shape or timing.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

__device__ __forceinline__ void row_coords(int row, int tq, const int64_t* pos0, int& b, int& i,
                                           int64_t& pos) {
  b = row / tq;
  i = row - b * tq;
  pos = pos0[b] + i;
}

// (key, id) packed so that the larger value is the better element: higher key, then
// lower id.  0 marks "no element".
__device__ __forceinline__ uint64_t pack_kid(uint32_t key, uint32_t id) {
  return ((uint64_t)key << 32) | (uint64_t)(~id);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = v > w ? v : w;
  }
  return v;
}

// The 8 best of a tile's 256 packed values (s_v, one per thread of a 256-thread
// workgroup) to out[0..7] as (key, id), in ascending id order (missing entries, for
// tiles with fewer than 8 elements, are (0, 0xffffffff) and come last).
__device__ void tile_top8(const uint64_t* s_v, uint64_t* s_w, uint2* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t v = s_v[threadIdx.x];
#pragma unroll
  for (int r = 0; r < kTileTop; ++r) {
    const uint64_t m = wave_max_u64(v);
    if (v == m) v = 0;
    if (lane == 0) s_w[wave * kTileTop + r] = m;
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t u = lane < 4 * kTileTop ? s_w[lane] : 0;
    uint64_t mine = 0;
#pragma unroll
    for (int r = 0; r < kTileTop; ++r) {
      const uint64_t m = wave_max_u64(u);
      if (u == m) u = 0;
      if (lane == r) mine = m;
    }
    const uint32_t id = ~(uint32_t)mine;
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kTileTop; ++q) {
      const uint32_t oid = (uint32_t)__shfl((int)id, q);
      rank += (oid < id || (oid == id && q < lane)) ? 1 : 0;
    }
    if (lane < kTileTop) out[rank] = make_uint2((uint32_t)(mine >> 32), id);
  }
}

// ------------------------------------------------------------------ score, bf16 MFMA
// S = QI (heads x d_I) . KI^T (d_I x blocks) on v_mfma_f32_16x16x32_bf16.
// Operand layout (wave64): lane l = 16*grp + col.  A (16 heads x 32 dims): lane holds
// head col, 8 dims of group grp; B (32 dims x 16 blocks): lane holds block col, the
// same 8 dims; C (16 heads x 16 blocks): lane holds block col, heads 4*grp + e.
// The dims a lane group carries only have to agree between A and B.
template <int MT, int KS>
__global__ __launch_bounds__(256) void score_bf16_kernel(ScoreP p) {
  __shared__ uint64_t s_v[kTile];
  __shared__ uint64_t s_w[4 * kTileTop];
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t tile0 = (int64_t)blockIdx.x * kTile;
  if (tile0 >= nvis) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  constexpr int DI = KS * 32;
  const uint16_t* ki = reinterpret_cast<const uint16_t*>(p.ki) + (int64_t)b * p.ki_bs;
  // blocks of this wave: tile0 + wave*16 + u*64 + col, u = 0..3
  constexpr int U = kTile / 64;
  bf16x8_t Bv[U][KS];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = tile0 + wave * 16 + u * 64 + col;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < nvis) v = *reinterpret_cast<const uint4*>(ki + j * p.ki_rs + s * 32 + grp * 8);
      Bv[u][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const uint16_t* qi = reinterpret_cast<const uint16_t*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
  bf16x8_t A[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      A[mt][s] = __builtin_bit_cast(bf16x8_t,
                   *reinterpret_cast<const uint4*>(qi + (mt * 16 + col) * DI + s * 32 + grp * 8));
  float w[MT][4];
  const float* wi = p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) w[mt][e] = wi[mt * 16 + grp * 4 + e];

  float* sc = p.scores + (int64_t)lr * p.sc_rs;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][s], Bv[u][s], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) part = fmaf(w[mt][e], fmaxf(acc[e], 0.f), part);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    const int t = wave * 16 + u * 64 + col;
    const int64_t j = tile0 + t;
    if (grp == 0) {
      if (j < nvis) sc[j] = part;
      s_v[t] = j < nvis ? pack_kid(score_key(part), (uint32_t)j) : 0ull;
    }
  }
  __syncthreads();
  tile_top8(s_v, s_w, p.summary + (int64_t)lr * p.sum_rs + (int64_t)blockIdx.x * kTileTop);
}

// ------------------------------------------------------------------ score, fp32 VALU
// One thread per block of the tile; the row's indexer queries and weights sit in LDS.
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreP p) {
  __shared__ uint64_t s_v[kTile];
  __shared__ uint64_t s_w[4 * kTileTop];
  extern __shared__ float s_q[];  // [heads*dim] then [heads]
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t tile0 = (int64_t)blockIdx.x * kTile;
  if (tile0 >= nvis) return;
  const int HD = p.heads * p.dim;
  const float* qi = reinterpret_cast<const float*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
  const float* wi = p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs;
  for (int t = threadIdx.x; t < HD; t += 256) s_q[t] = qi[t];
  for (int t = threadIdx.x; t < p.heads; t += 256) s_q[HD + t] = wi[t];
  __syncthreads();
  const float* ki = reinterpret_cast<const float*>(p.ki) + (int64_t)b * p.ki_bs;
  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int64_t j = tile0 + threadIdx.x;
  uint64_t v = 0;
  if (j < nvis) {
    const float* kj = ki + j * p.ki_rs;
    float s = 0.f;
    for (int h = 0; h < p.heads; ++h) {
      const float* qh = s_q + h * p.dim;
      float dot = 0.f;
      for (int c = 0; c < p.dim; c += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(kj + c);
        dot = fmaf(qh[c], kv.x, dot);
        dot = fmaf(qh[c + 1], kv.y, dot);
        dot = fmaf(qh[c + 2], kv.z, dot);
        dot = fmaf(qh[c + 3], kv.w, dot);
      }
      s = fmaf(s_q[HD + h], fmaxf(dot, 0.f), s);
    }
    sc[j] = s;
    v = pack_kid(score_key(s), (uint32_t)j);
  }
  s_v[threadIdx.x] = v;
  __syncthreads();
  tile_top8(s_v, s_w, p.summary + (int64_t)lr * p.sum_rs + (int64_t)blockIdx.x * kTileTop);
}

hipError_t launch_score(int dtype, const ScoreP& p, int nrows, int ntiles, hipStream_t s) {
  const dim3 grid((unsigned)ntiles, (unsigned)nrows);
  if (dtype == 0) {
    const size_t lds = (size_t)(p.heads * p.dim + p.heads) * sizeof(float);
    hipLaunchKernelGGL(score_f32_kernel, grid, dim3(256), lds, s, p);
    return hipGetLastError();
  }
  const int mt = p.heads / 16, ks = p.dim / 32;
#define V4A_SCORE_CASE(M, K) \
  if (mt == M && ks == K) { hipLaunchKernelGGL((score_bf16_kernel<M, K>), grid, dim3(256), 0, s, p); return hipGetLastError(); }
  V4A_SCORE_CASE(1, 1) V4A_SCORE_CASE(1, 2) V4A_SCORE_CASE(1, 4)
  V4A_SCORE_CASE(2, 1) V4A_SCORE_CASE(2, 2) V4A_SCORE_CASE(2, 4)
  V4A_SCORE_CASE(4, 1) V4A_SCORE_CASE(4, 2) V4A_SCORE_CASE(4, 4)
  V4A_SCORE_CASE(8, 1) V4A_SCORE_CASE(8, 2) V4A_SCORE_CASE(8, 4)
#undef V4A_SCORE_CASE
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ selection
constexpr int kNW = kSelThreads / 64;
constexpr int kBins = 4096;

struct SelShared {
  uint32_t hist[kBins];
  uint32_t wtot[kNW];
  uint32_t wmin[kNW], wmax[kNW];
  uint32_t pool_key[kPoolCap];
  uint32_t pool_id[kPoolCap];
  uint32_t fail[256], fcount[256], fbase[256];
  uint32_t n_pool, n_fail, flag;
  uint32_t hit_bin, hit_before;
};

// inclusive prefix sum over the workgroup (one value per thread)
__device__ __forceinline__ uint32_t block_scan(uint32_t v, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) sh.wtot[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += sh.wtot[w];
  __syncthreads();
  return v + add;
}

// min and max over the workgroup
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SelShared& sh, uint32_t& omn, uint32_t& omx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) { sh.wmin[wave] = mn; sh.wmax[wave] = mx; }
  __syncthreads();
  omn = sh.wmin[0];
  omx = sh.wmax[0];
  for (int w = 1; w < kNW; ++w) { omn = min(omn, sh.wmin[w]); omx = max(omx, sh.wmax[w]); }
  __syncthreads();
}

// Bin of sh.hist[0..nb) holding the r-th element (1-based) counted from the top
// (descending) or from the bottom, and the count strictly before it.
__device__ void find_rank(SelShared& sh, int nb, uint32_t r, bool descending, uint32_t& bin,
                          uint32_t& before) {
  const int t = threadIdx.x;
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  uint32_t sum = 0;
  for (int e = 0; e < per; ++e) {
    const int o = t * per + e;
    if (o < nb) sum += sh.hist[descending ? nb - 1 - o : o];
  }
  const uint32_t incl = block_scan(sum, sh);
  const uint32_t excl = incl - sum;
  if (excl < r && r <= incl) {
    uint32_t run = excl;
    for (int e = 0; e < per; ++e) {
      const int o = t * per + e;
      if (o >= nb) break;
      const int bb = descending ? nb - 1 - o : o;
      const uint32_t c = sh.hist[bb];
      if (run + c >= r) { sh.hit_bin = (uint32_t)bb; sh.hit_before = run; break; }
      run += c;
    }
  }
  __syncthreads();
  bin = sh.hit_bin;
  before = sh.hit_before;
  __syncthreads();
}

// Rank search over the values `val(key, id)` of the elements that `each` visits and
// `keep(key, id)` accepts: returns the value v* holding the r-th element counted
// from the top (descending) or the bottom, and through r the rank of the wanted
// element among those equal to v*.  Bins are power-of-two slices of the live
// [lo, hi] range, so keys that sit close together spread over many bins and the
// LDS atomics stay free of contention; at most 3 levels narrow 32 bits to one value.
template <class Each, class Keep, class Val>
__device__ uint32_t rank_search(Each each, Keep keep, Val val, uint32_t& r, bool descending, SelShared& sh,
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
    find_rank(sh, nb, r, descending, bin, before);
    r -= before;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t nhi = (uint32_t)min<uint64_t>((uint64_t)hi, (uint64_t)nlo + ((uint64_t)1 << shift) - 1);
    if (shift == 0) {
      n_equal = sh.hist[bin];
      __syncthreads();
      return nlo;
    }
    lo = nlo;
    hi = nhi;
  }
}

// The key threshold T and the largest tie id of the exact top-k over the visited
// elements: an element is selected iff key > T, or key == T and id <= id_max.
template <class Each>
__device__ void topk_threshold(Each each, uint32_t k, SelShared& sh, uint32_t& T, uint32_t& id_max) {
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

constexpr int kMaxTilesPerThread = 2;

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectP p) {
  __shared__ SelShared sh;
  const int lr = blockIdx.x;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int k = p.topk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const uint2* U = p.summary + (int64_t)lr * p.sum_rs;
  const int64_t ntiles = (nvis + kTile - 1) / kTile;
  const int tpt = ntiles <= kSelThreads ? 1 : kMaxTilesPerThread;   // tiles per thread
  bool fast = ntiles <= (int64_t)kSelThreads * kMaxTilesPerThread;

  // thread t owns tiles [t*tpt, t*tpt + tpt): their summaries (id order) in registers
  uint32_t uk[kMaxTilesPerThread][kTileTop], ui[kMaxTilesPerThread][kTileTop];
#pragma unroll
  for (int q = 0; q < kMaxTilesPerThread; ++q) {
    const int64_t t = (int64_t)tid * tpt + q;
    const bool own = fast && q < tpt && t < ntiles;
    const uint4* src = reinterpret_cast<const uint4*>(U + t * kTileTop);
#pragma unroll
    for (int j = 0; j < kTileTop / 2; ++j) {
      uint4 e = make_uint4(0u, 0xffffffffu, 0u, 0xffffffffu);
      if (own) e = src[j];
      uk[q][2 * j] = e.x; ui[q][2 * j] = e.y; uk[q][2 * j + 1] = e.z; ui[q][2 * j + 1] = e.w;
    }
  }
  uint32_t T = 0, id_max = 0xffffffffu;
  uint32_t np = 0;
  if (fast) {
    // tau: the k-th largest summary key, a lower bound of the row's k-th key (0 when the
    // summaries hold fewer than k elements)
    uint32_t tau = 0;
    if (ntiles * kTileTop >= k) {
      uint32_t r = (uint32_t)k, n_eq;
      tau = rank_search(
          [&](auto&& f) {
#pragma unroll
            for (int q = 0; q < kMaxTilesPerThread; ++q)
#pragma unroll
              for (int j = 0; j < kTileTop; ++j)
                if ((int64_t)tid * tpt + q < ntiles && q < tpt) f(uk[q][j], ui[q][j]);
          },
          [](uint32_t, uint32_t) { return true; }, [](uint32_t key, uint32_t) { return key; }, r, true, sh,
          n_eq);
    }
    // per owned tile: count of elements >= tau, or a rescan slot when the tile may hold
    // more of them than its summary shows
    if (tid == 0) { sh.n_fail = 0; sh.flag = 0; }
    __syncthreads();
    int fslot[kMaxTilesPerThread];
    uint32_t cnt[kMaxTilesPerThread];
#pragma unroll
    for (int q = 0; q < kMaxTilesPerThread; ++q) {
      fslot[q] = -1;
      cnt[q] = 0;
      const int64_t t = (int64_t)tid * tpt + q;
      if (q >= tpt || t >= ntiles) continue;
      const int64_t valid = min<int64_t>(kTile, nvis - t * kTile);
      uint32_t kmin = 0xffffffffu;
#pragma unroll
      for (int j = 0; j < kTileTop; ++j) {
        if (ui[q][j] != 0xffffffffu) {
          cnt[q] += uk[q][j] >= tau ? 1u : 0u;
          kmin = min(kmin, uk[q][j]);
        }
      }
      if (valid > kTileTop && kmin >= tau) {
        const uint32_t slot = atomicAdd(&sh.n_fail, 1u);
        if (slot < 256u) { fslot[q] = (int)slot; sh.fail[slot] = (uint32_t)t; }
        else sh.flag = 1;
      }
    }
    __syncthreads();
    const uint32_t nf = sh.n_fail;
    if (sh.flag) fast = false;
    if (fast && nf) {
      // a wave counts the elements >= tau of each failing tile
      for (uint32_t f = wave; f < nf; f += kNW) {
        const int64_t base = (int64_t)sh.fail[f] * kTile;
        uint32_t c = 0;
        for (int r = 0; r < kTile / 64; ++r) {
          const int64_t j = base + r * 64 + lane;
          const bool hit = j < nvis && score_key(sc[j]) >= tau;
          c += __popcll(__ballot(hit));
        }
        if (lane == 0) sh.fcount[f] = c;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kMaxTilesPerThread; ++q)
        if (fslot[q] >= 0) cnt[q] = sh.fcount[fslot[q]];
    }
    if (fast) {
      // order-preserving compaction: tiles in order, ids ascending inside a tile
      uint32_t mine = 0;
#pragma unroll
      for (int q = 0; q < kMaxTilesPerThread; ++q) mine += cnt[q];
      const uint32_t incl = block_scan(mine, sh);
      if (tid == kSelThreads - 1) sh.n_pool = incl;
      uint32_t off = incl - mine;
      __syncthreads();
      np = sh.n_pool;
      if (np > (uint32_t)kPoolCap) {
        fast = false;
      } else {
#pragma unroll
        for (int q = 0; q < kMaxTilesPerThread; ++q) {
          if (fslot[q] >= 0) {
            sh.fbase[fslot[q]] = off;
          } else {
#pragma unroll
            for (int j = 0; j < kTileTop; ++j)
              if (ui[q][j] != 0xffffffffu && uk[q][j] >= tau) {
                sh.pool_key[off] = uk[q][j];
                sh.pool_id[off] = ui[q][j];
                ++off;
              }
          }
          off += fslot[q] >= 0 ? cnt[q] : 0;
        }
        __syncthreads();
        for (uint32_t f = wave; f < nf; f += kNW) {
          const int64_t base = (int64_t)sh.fail[f] * kTile;
          uint32_t o = sh.fbase[f];
          for (int r = 0; r < kTile / 64; ++r) {
            const int64_t j = base + r * 64 + lane;
            const uint32_t key = j < nvis ? score_key(sc[j]) : 0u;
            const bool hit = j < nvis && key >= tau;
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
      }
    }
  }

  if (fast) {
    // the pool holds every element >= tau in id order, and at least k of them
    if (np > (uint32_t)k) {
      topk_threshold([&](auto&& f) { for (uint32_t t = tid; t < np; t += kSelThreads) f(sh.pool_key[t], sh.pool_id[t]); },
                     (uint32_t)k, sh, T, id_max);
    } else {
      T = 0;
      id_max = 0xffffffffu;
    }
    // order-preserving compaction of the picked pool entries (contiguous ranges per thread)
    const uint32_t per = (np + kSelThreads - 1) / kSelThreads;
    const uint32_t lo = min(np, tid * per), hi = min(np, lo + per);
    uint32_t c = 0;
    for (uint32_t t = lo; t < hi; ++t) c += picked(sh.pool_key[t], sh.pool_id[t], T, id_max) ? 1u : 0u;
    uint32_t o = block_scan(c, sh) - c;
    for (uint32_t t = lo; t < hi; ++t) {
      const uint32_t id = sh.pool_id[t];
      if (picked(sh.pool_key[t], id, T, id_max)) {
        if (o < (uint32_t)k) {
          out[o] = (int32_t)id;
          if (selp) selp[o] = sc[id];
        }
        ++o;
      }
    }
    return;
  }

  // slow path: the whole row (ties everywhere, or a pool too large for LDS)
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

hipError_t launch_select(const SelectP& p, int nrows, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)nrows), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
