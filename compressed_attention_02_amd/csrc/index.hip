// csa_indexer_score + topk_select.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制,
// CSA step 2: a light indexer scores every compressed block for each query token and
// the query keeps its top-k blocks (yage.ai essay on the agentic workload, three-tier
// section: k = 1024 for Pro, 512 for Flash).  Score form fixed by the layer
// configuration: s_j = sum_h w_h * ReLU(qi_h . ki_j).
//
// The keys are the order-preserving uint32 image of the fp32 scores, so "larger key"
// is "larger score"; the result does not depend on launch shape or timing.
//
// score   bf16 / FP8 MFMA 16x16x32 (indexer heads on M, blocks on N) or fp32 VALU,
//         over tiles of 256 blocks.  Every tile leaves a report: the keys of its 8
//         best blocks in id order with their offsets, and a bound, the key of the
//         best block the report leaves out (it bounds every other one).  Decode
//         builds the report in two phases: each 64-block wave keeps its 4 (or 8)
//         best as candidates, then one wave ranks the tile's candidates by counting
//         and keeps the 8 ahead of the rest (bound: the best candidate or wave
//         remainder not kept).  Prefill keeps the tile's exact best 4 (rounds of
//         wave maxima).  The fp32 scores are stored too, for rescans.
// select  one 512-thread workgroup per row, the reports of the row's tiles in its
//         registers.  (1) The exact k-th key T of all the reports: a rank search
//         over a histogram of the live key range (8192 bins, two levels); when the
//         bin holding T has at most 64 keys, those keys are gathered and ranked
//         directly.  (2) If no tile's bound reaches T, the reports hold every key
//         >= T and their top-k is the row's, written in id order.  (3) Otherwise
//         the few tiles whose bound reaches T are rescanned from their stored
//         scores: their keys >= T join the other tiles' reports >= T, and T is
//         searched again in that pool.  Ties at T go to the lower ids; rows with
//         n_vis < k are padded with -1.  Too many rescans, or more tiles than the
//         registers hold, send the row to the same search over all its scores.
//
// Threshold mode (prefill chunks on long contexts, where most tiles hold no pick):
// a first score pass over every 64th tile stores those scores; each row takes
// from them a key theta below its k-th key (the sample's rank 3k n_s / n_vis + 16
// key), which holds for all but rare rows.  The full pass then reports, for every
// tile with at most 8 keys >= theta, exactly those keys (the bound is theta - 1:
// no other key of the tile reaches theta) and stores no scores; only the denser
// tiles store scores and report their exact best 8.  The selection flags a row
// whose k-th key falls below theta (its reports may miss keys); a repair pass
// scores and selects the flagged rows' groups again, exactly.  No global atomics,
// and every buffer a launch reads is written earlier in the same call.
#include "qprep_impl.hpp"
#include "score_impl.hpp"
#include "select_impl.hpp"

namespace v4a {

// ------------------------------------------------------------------ score, bf16 MFMA
// Workgroups of 4 waves (tiles of 256 keys).  With the query prep hosted, the first
// prep_x workgroups of each row prepare that row's attention queries instead
// (dispatched first); the score workgroups follow them.
template <int MT, int KS, int NB, bool FP8>
__global__ __launch_bounds__(256) void score_bf16_kernel(ScoreP p) {
  __shared__ __align__(16) ScoreSmem<4, MT, KS, NB, FP8> sm;
  if ((int)blockIdx.x < p.prep_x) {
    qprep_block(p.prep, p.row0 + blockIdx.y, blockIdx.x);
    return;
  }
  score_block<4, MT, KS, NB, FP8>(p, (int)blockIdx.x - p.prep_x, blockIdx.y, sm);
}

// ------------------------------------------------------------------ score, fp32 VALU
// One thread per block of the tile; the row's indexer queries and weights sit in LDS.
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreP p) {
  extern __shared__ float s_q[];  // [heads*dim] then [heads]
  __shared__ TileStage s_stage;
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
  uint32_t v = 0;
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
    v = score_key(s);
  }
  tile_report_waves(v, j < nvis, 0, p.wave_top, s_stage, p.rep_key + (int64_t)lr * p.key_rs + (int64_t)blockIdx.x * kTileTop,
                    p.rep_info + (int64_t)lr * p.info_rs + blockIdx.x);
}

hipError_t launch_score(int dtype, const ScoreP& p, int nrows, int ntiles, hipStream_t s, int tid) {
  const dim3 grid((unsigned)ntiles, (unsigned)nrows);
  if (dtype == 0) {
    const size_t lds = (size_t)(p.heads * p.dim + p.heads) * sizeof(float);
    V4A_LAUNCH(tid, score_f32_kernel, grid, dim3(256), lds, s, p);
    return hipGetLastError();
  }
  const int mt = p.heads / 16, ks = p.dim / 32;
  ScoreP q = p;
  q.nrows = nrows;
  const dim3 pgrid((unsigned)(p.wgs_per_row + p.prep_x), (unsigned)nrows);
  // a second tile buffer only when workgroups walk several tiles
  const bool two = (int64_t)p.wgs_per_row < ntiles;
  const bool f8 = p.ki_scale != nullptr;
#define V4A_SCORE_CASE(M, K)                                                                             \
  if (mt == M && ks == K) {                                                                              \
    if (f8) {                                                                                            \
      if (two) V4A_LAUNCH(tid, (score_bf16_kernel<M, K, 2, true>), pgrid, dim3(256), 0, s, q);          \
      else V4A_LAUNCH(tid, (score_bf16_kernel<M, K, 1, true>), pgrid, dim3(256), 0, s, q);              \
    } else {                                                                                             \
      if (two) V4A_LAUNCH(tid, (score_bf16_kernel<M, K, 2, false>), pgrid, dim3(256), 0, s, q);         \
      else V4A_LAUNCH(tid, (score_bf16_kernel<M, K, 1, false>), pgrid, dim3(256), 0, s, q);             \
    }                                                                                                    \
    return hipGetLastError();                                                                            \
  }
  V4A_SCORE_CASE(1, 1) V4A_SCORE_CASE(1, 2)
  V4A_SCORE_CASE(2, 1) V4A_SCORE_CASE(2, 2)
  V4A_SCORE_CASE(4, 1) V4A_SCORE_CASE(4, 2)
  V4A_SCORE_CASE(8, 1) V4A_SCORE_CASE(8, 2)
#undef V4A_SCORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_score_rows(const ScoreP& p, int nrows, int ntiles, hipStream_t s, int tid) {
  if (p.heads != 64 || p.dim != 64 || p.ki_scale || p.prep_x != 0 || p.tq % kScoreRowsQ != 0 ||
      p.row0 % kScoreRowsQ != 0 || nrows < 1 || p.wgs_per_row < 1)
    return hipErrorInvalidValue;
  ScoreP q = p;
  q.nrows = nrows;
  // wgs_per_row workgroups per group of kScoreRowsQ queries, each walking tiles
  const dim3 grid((unsigned)std::min(p.wgs_per_row, ntiles), (unsigned)((nrows + kScoreRowsQ - 1) / kScoreRowsQ));
  V4A_LAUNCH(tid, score_rows_kernel, grid, dim3(kScoreRowsQ * 64), 0, s, q);
  return hipGetLastError();
}

// ------------------------------------------------------------------ selection
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectP p) {
  __shared__ SelShared sh;
  select_row(p, blockIdx.x, sh);
}

hipError_t launch_select(const SelectP& p, int nrows, hipStream_t s, int tid) {
  V4A_LAUNCH(tid, select_kernel, dim3((unsigned)nrows), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ threshold
// Threshold mode of the prefill form: from the scores of the sampled tiles (0, S,
// 2S, ...; n_s keys), the r-th largest key with r = 3 k n_s / n_vis + 16, about three
// times the sample's expected share of the row's top-k plus a margin: for keys in
// random order it lies below the row's k-th key by a wide margin, and a row where it
// does not is redone exactly (select_row flags it).  Rows whose sample holds fewer
// than r keys (short rows) get 0, which makes every full tile report exactly.
__global__ __launch_bounds__(kSelThreads) void theta_kernel(SelectP p) {
  __shared__ SelShared sh;
  const int lr = blockIdx.x;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t S = p.sample_stride;
  uint32_t th = 0u;
  if (nvis >= kTile) {
    const int64_t ns_t = ((nvis + kTile - 1) / kTile + S - 1) / S;   // sampled tiles
    const int64_t last = (ns_t - 1) * S;                               // the last one's row tile
    const int64_t n_s = (ns_t - 1) * kTile + min<int64_t>(kTile, nvis - last * kTile);
    const uint64_t r = 3ull * (uint64_t)p.topk * (uint64_t)n_s / (uint64_t)nvis + 16ull;
    if ((uint64_t)n_s >= r) {
      const float* sc = p.scores + (int64_t)lr * p.sc_rs;
      auto each = [&](auto&& f) {
        for (int64_t t = threadIdx.x; t < n_s; t += kSelThreads) {
          const int64_t j = (t / kTile) * S * kTile + t % kTile;
          f(score_key(sc[j]), (uint32_t)j);
        }
      };
      uint32_t rr = (uint32_t)r, n_eq;
      th = rank_search(each, [](uint32_t, uint32_t) { return true; }, [](uint32_t key, uint32_t) { return key; }, rr,
                       true, sh, n_eq);
    }
  }
  if (threadIdx.x == 0) p.theta_out[lr] = th;
}

hipError_t launch_theta(const SelectP& p, int nrows, hipStream_t s, int tid) {
  if (p.sample_stride < 1 || !p.theta_out) return hipErrorInvalidValue;
  V4A_LAUNCH(tid, theta_kernel, dim3((unsigned)nrows), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
