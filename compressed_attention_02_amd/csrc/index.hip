// csa_indexer_score + topk_select.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制,
// CSA step 2: a light indexer scores every compressed block for each query token and
// the query keeps its top-k blocks (yage.ai essay on the agentic workload, three-tier
// section: k = 1024 for Pro, 512 for Flash).  Score form fixed by the layer
// configuration: s_j = sum_h w_h * ReLU(qi_h . ki_j).
//
// Pipeline per launch (rows = query tokens):
//   clear   zero the per-row radix histograms and list counters
//   score   one workgroup per (tile of blocks, row): bf16 MFMA 16x16x32 with the
//           indexer heads on M and the blocks on N, or fp32 VALU; writes fp32 scores
//           and adds the tile's histogram of the top 12 key bits into the row's one
//   filter  every workgroup re-derives the threshold bin from the histogram, then
//           compacts its slice: ids above the bin ("sure") and (key, id) pairs inside
//           the bin ("candidates")
//   final   one workgroup per row: two more radix levels over the candidates fix
//           the exact k-th key; ties at that key go to the lowest ids (radix on the
//           id); the k ids are bitonic-sorted ascending and written with -1 padding
// Keys are the order-preserving uint32 image of the fp32 scores, so "larger key"
// is "larger score"; the selection is exact and independent of launch shape.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ void row_coords(int row, int tq, const int64_t* pos0, int& b, int& i,
                                           int64_t& pos) {
  b = row / tq;
  i = row - b * tq;
  pos = pos0[b] + i;
}

// Flush a workgroup's LDS histogram into the row's global histogram.
__device__ __forceinline__ void flush_hist(const uint32_t* s_hist, uint32_t* gh) {
  for (int t = threadIdx.x; t < kHistBins; t += blockDim.x) {
    const uint32_t c = s_hist[t];
    if (c) atomicAdd(&gh[t], c);
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
  __shared__ uint32_t s_hist[kHistBins];
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile;
  if (tile0 >= nvis) return;
  for (int t = threadIdx.x; t < kHistBins; t += 256) s_hist[t] = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  constexpr int DI = KS * 32;
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
  __syncthreads();

  const uint16_t* ki = reinterpret_cast<const uint16_t*>(p.ki) + (int64_t)b * p.ki_bs;
  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int64_t tile_end = min(tile0 + (int64_t)p.tile, nvis);
  constexpr int U = 4;  // 16-block groups in flight per wave
  for (int64_t j0 = tile0 + wave * 16; j0 < tile_end; j0 += 4 * 16 * U) {
    bf16x8_t Bv[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + u * 64 + col;
      const bool ok = j < tile_end;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(ki + j * p.ki_rs + s * 32 + grp * 8);
        Bv[u][s] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
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
      const int64_t j = j0 + u * 64 + col;
      if (grp == 0 && j < tile_end) {
        sc[j] = part;
        atomicAdd(&s_hist[score_key(part) >> (32 - kHistBits)], 1u);
      }
    }
  }
  __syncthreads();
  flush_hist(s_hist, p.hist + (int64_t)lr * kHistBins);
}

// ------------------------------------------------------------------ score, fp32 VALU
// One thread per block; the row's indexer queries and weights sit in LDS.
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreP p) {
  __shared__ uint32_t s_hist[kHistBins];
  extern __shared__ float s_q[];  // [heads*dim] then [heads]
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile;
  if (tile0 >= nvis) return;
  const int HD = p.heads * p.dim;
  const float* qi = reinterpret_cast<const float*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
  const float* wi = p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs;
  for (int t = threadIdx.x; t < kHistBins; t += 256) s_hist[t] = 0;
  for (int t = threadIdx.x; t < HD; t += 256) s_q[t] = qi[t];
  for (int t = threadIdx.x; t < p.heads; t += 256) s_q[HD + t] = wi[t];
  __syncthreads();
  const float* ki = reinterpret_cast<const float*>(p.ki) + (int64_t)b * p.ki_bs;
  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int64_t tile_end = min(tile0 + (int64_t)p.tile, nvis);
  for (int64_t j = tile0 + threadIdx.x; j < tile_end; j += 256) {
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
    atomicAdd(&s_hist[score_key(s) >> (32 - kHistBits)], 1u);
  }
  __syncthreads();
  flush_hist(s_hist, p.hist + (int64_t)lr * kHistBins);
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

// ------------------------------------------------------------------ radix helpers
// Given an LDS histogram of nb bins (nb a multiple of 256) and a rank r >= 1, find
// the bin holding the r-th element counted from the top (descending == true) or
// from the bottom; returns the bin and the count strictly before it in that order.
// All 256 threads must call it.
struct RankHit { int bin; uint32_t before; };

__device__ RankHit find_rank(const uint32_t* hist, int nb, uint32_t r, bool descending,
                             uint32_t* s_scan /*[256]*/, RankHit* s_hit) {
  const int t = threadIdx.x;
  const int per = nb / 256;
  uint32_t sum = 0;
  for (int e = 0; e < per; ++e) {
    const int o = t * per + e;
    sum += hist[descending ? nb - 1 - o : o];
  }
  s_scan[t] = sum;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 partial sums
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = t >= off ? s_scan[t - off] : 0u;
    __syncthreads();
    s_scan[t] += v;
    __syncthreads();
  }
  const uint32_t incl = s_scan[t];
  const uint32_t excl = incl - sum;
  if (excl < r && r <= incl) {
    uint32_t run = excl;
    for (int e = 0; e < per; ++e) {
      const int o = t * per + e;
      const int bin = descending ? nb - 1 - o : o;
      const uint32_t c = hist[bin];
      if (run + c >= r) { s_hit->bin = bin; s_hit->before = run; break; }
      run += c;
    }
  }
  __syncthreads();
  const RankHit h = *s_hit;
  __syncthreads();
  return h;
}

// ------------------------------------------------------------------ clear
__global__ void topk_clear_kernel(uint32_t* hist, uint32_t* counts, int64_t nh, int64_t nc) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nh; t += stride) hist[t] = 0;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nc; t += stride) counts[t] = 0;
}

hipError_t launch_topk_clear(const TopkP& p, int nrows, hipStream_t s) {
  const int64_t nh = (int64_t)nrows * kHistBins, nc = (int64_t)nrows * 4;
  const int64_t want = (nh + 255) / 256;
  const int blocks = (int)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(topk_clear_kernel, dim3(blocks), dim3(256), 0, s, const_cast<uint32_t*>(p.hist),
                     p.counts, nh, nc);
  return hipGetLastError();
}

// ------------------------------------------------------------------ filter
constexpr int kFilterSlice = 4096;

__global__ __launch_bounds__(256) void topk_filter_kernel(TopkP p) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_scan[256];
  __shared__ RankHit s_hit;
  __shared__ uint32_t s_sure[kMaxTopk];
  __shared__ uint2 s_cand[kFilterSlice];
  __shared__ uint32_t s_ns, s_nc, s_bs, s_bc;
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  if (nvis <= p.topk) return;                      // everything is selected
  const int64_t start = (int64_t)blockIdx.x * p.slice;
  if (start >= nvis) return;
  const uint32_t* gh = p.hist + (int64_t)lr * kHistBins;
  for (int t = threadIdx.x; t < kHistBins; t += 256) s_hist[t] = gh[t];
  if (threadIdx.x == 0) { s_ns = 0; s_nc = 0; }
  __syncthreads();
  const RankHit h1 = find_rank(s_hist, kHistBins, (uint32_t)p.topk, true, s_scan, &s_hit);
  const uint32_t b1 = (uint32_t)h1.bin;
  const bool overflow = s_hist[b1] > (uint32_t)kCandCap;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.counts[(int64_t)lr * 4 + 2] = b1;
    p.counts[(int64_t)lr * 4 + 3] = h1.before;
  }
  const float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int64_t end = min(start + (int64_t)p.slice, nvis);
  for (int64_t j = start + threadIdx.x; j < end; j += 256) {
    const uint32_t key = score_key(sc[j]);
    const uint32_t bin = key >> (32 - kHistBits);
    if (bin > b1) {
      s_sure[atomicAdd(&s_ns, 1u)] = (uint32_t)j;
    } else if (bin == b1 && !overflow) {
      s_cand[atomicAdd(&s_nc, 1u)] = make_uint2(key, (uint32_t)j);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_bs = s_ns ? atomicAdd(&p.counts[(int64_t)lr * 4 + 0], s_ns) : 0u;
    s_bc = s_nc ? atomicAdd(&p.counts[(int64_t)lr * 4 + 1], s_nc) : 0u;
  }
  __syncthreads();
  uint32_t* gs = p.sure + (int64_t)lr * kMaxTopk;
  uint2* gc = p.cand + (int64_t)lr * kCandCap;
  for (uint32_t t = threadIdx.x; t < s_ns; t += 256) gs[s_bs + t] = s_sure[t];
  for (uint32_t t = threadIdx.x; t < s_nc; t += 256) gc[s_bc + t] = s_cand[t];
}

hipError_t launch_topk_filter(const TopkP& p, int nrows, int nslices, hipStream_t s) {
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)nslices, (unsigned)nrows), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ final
// Candidates of the threshold bin come from the row's candidate list, or, when the
// bin held more than kCandCap elements, from a rescan of the row's scores.
struct CandSrc {
  const uint2* list; const float* sc; uint32_t n; int64_t nvis; uint32_t b1; bool from_list;
  __device__ __forceinline__ int64_t size() const { return from_list ? (int64_t)n : nvis; }
  // returns false when element t is not in the threshold bin
  __device__ __forceinline__ bool get(int64_t t, uint32_t& key, uint32_t& id) const {
    if (from_list) { const uint2 v = list[t]; key = v.x; id = v.y; return true; }
    key = score_key(sc[t]);
    id = (uint32_t)t;
    return (key >> (32 - kHistBits)) == b1;
  }
};

__global__ __launch_bounds__(256) void topk_final_kernel(TopkP p) {
  __shared__ uint32_t s_h[2048];
  __shared__ uint32_t s_scan[256];
  __shared__ RankHit s_hit;
  __shared__ uint32_t s_sel[kMaxTopk];
  __shared__ uint32_t s_n;
  const int lr = blockIdx.x;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int k = p.topk;
  int32_t* out = p.idx + (int64_t)b * p.idx_bs + (int64_t)i * p.idx_rs;
  float* sel = p.sel ? p.sel + (int64_t)b * p.sel_bs + (int64_t)i * p.sel_rs : nullptr;
  const float* sc = p.scores + (int64_t)lr * p.sc_rs;
  if (nvis <= k) {
    for (int t = threadIdx.x; t < k; t += 256) {
      out[t] = t < nvis ? t : -1;
      if (sel) sel[t] = t < nvis ? sc[t] : 0.f;
    }
    return;
  }
  const uint32_t* cnt = p.counts + (int64_t)lr * 4;
  const uint32_t n_sure = cnt[0], n_list = cnt[1], b1 = cnt[2], above1 = cnt[3];
  const uint32_t bin1_total = p.hist[(int64_t)lr * kHistBins + b1];
  CandSrc src{p.cand + (int64_t)lr * kCandCap, sc, n_list, nvis, b1, bin1_total <= (uint32_t)kCandCap};
  const uint32_t r = (uint32_t)k - above1;       // 1 <= r <= bin1_total
  const int64_t ns = src.size();

  // level 2: key bits [19:10]
  for (int t = threadIdx.x; t < 1024; t += 256) s_h[t] = 0;
  __syncthreads();
  for (int64_t t = threadIdx.x; t < ns; t += 256) {
    uint32_t key, id;
    if (src.get(t, key, id)) atomicAdd(&s_h[(key >> 10) & 1023u], 1u);
  }
  __syncthreads();
  const RankHit h2 = find_rank(s_h, 1024, r, true, s_scan, &s_hit);
  const uint32_t r2 = r - h2.before;
  // level 3: key bits [9:0] among keys matching b1:b2
  const uint32_t hi22 = (b1 << 10) | (uint32_t)h2.bin;
  for (int t = threadIdx.x; t < 1024; t += 256) s_h[t] = 0;
  __syncthreads();
  for (int64_t t = threadIdx.x; t < ns; t += 256) {
    uint32_t key, id;
    if (src.get(t, key, id) && (key >> 10) == hi22) atomicAdd(&s_h[key & 1023u], 1u);
  }
  __syncthreads();
  const RankHit h3 = find_rank(s_h, 1024, r2, true, s_scan, &s_hit);
  const uint32_t r3 = r2 - h3.before;             // how many of the ties at T to take
  const uint32_t T = (hi22 << 10) | (uint32_t)h3.bin;
  const uint32_t ties = s_h[h3.bin];
  // ties at T: take the r3 lowest ids -> threshold id by radix on the id, ascending,
  // over bits [31:21], [20:10], [9:0]
  uint32_t id_max = 0xffffffffu;
  if (r3 < ties) {
    uint32_t rr = r3, prefix = 0;
    for (int lvl = 0; lvl < 3; ++lvl) {
      const int shift = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
      const int nbins = lvl == 2 ? 1024 : 2048;
      for (int t = threadIdx.x; t < nbins; t += 256) s_h[t] = 0;
      __syncthreads();
      for (int64_t t = threadIdx.x; t < ns; t += 256) {
        uint32_t key, id;
        if (!src.get(t, key, id) || key != T) continue;
        if (lvl > 0 && (id >> (lvl == 1 ? 21 : 10)) != prefix) continue;
        atomicAdd(&s_h[(id >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
      __syncthreads();
      const RankHit hh = find_rank(s_h, nbins, rr, false, s_scan, &s_hit);
      rr -= hh.before;
      prefix = (prefix << (lvl == 0 ? 0 : (lvl == 1 ? 11 : 10))) | (uint32_t)hh.bin;
    }
    id_max = prefix;  // the r3-th lowest id among the ties
  }
  // gather: sure ids + candidates above T + ties at T with id <= id_max
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  const uint32_t* gs = p.sure + (int64_t)lr * kMaxTopk;
  for (uint32_t t = threadIdx.x; t < n_sure && t < (uint32_t)kMaxTopk; t += 256) {
    const uint32_t slot = atomicAdd(&s_n, 1u);
    if (slot < (uint32_t)kMaxTopk) s_sel[slot] = gs[t];
  }
  for (int64_t t = threadIdx.x; t < ns; t += 256) {
    uint32_t key, id;
    if (!src.get(t, key, id)) continue;
    if (key > T || (key == T && id <= id_max)) {
      const uint32_t slot = atomicAdd(&s_n, 1u);
      if (slot < (uint32_t)kMaxTopk) s_sel[slot] = id;
    }
  }
  __syncthreads();
  // bitonic sort of k ids ascending (padding with UINT_MAX up to a power of two)
  int npow = 1;
  while (npow < k) npow <<= 1;
  for (int t = k + threadIdx.x; t < npow; t += 256) s_sel[t] = 0xffffffffu;
  __syncthreads();
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < npow / 2; t += 256) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint32_t a = s_sel[lo], c = s_sel[hi];
        if ((a > c) == up) { s_sel[lo] = c; s_sel[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int t = threadIdx.x; t < k; t += 256) {
    const uint32_t id = s_sel[t];
    const bool valid = (int64_t)id < nvis;   // always true unless the lists disagree
    out[t] = valid ? (int32_t)id : -1;
    if (sel) sel[t] = valid ? sc[id] : 0.f;
  }
}

hipError_t launch_topk_final(const TopkP& p, int nrows, hipStream_t s) {
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)nrows), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
