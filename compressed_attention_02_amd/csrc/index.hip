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
//   score   bf16 MFMA 16x16x32 (indexer heads on M, blocks on N) or fp32 VALU over
//           tiles of 256 blocks.  Writes the fp32 scores; each wave (64 consecutive
//           blocks) also reports its 4 best (key, id) pairs and the key of its 5th
//           best, which bounds every key it leaves out.
//   select  one 512-thread workgroup per row.  The k-th largest of the wave maxima
//           bounds the row's k-th key from below (the k-th largest of any subset
//           does), so the reports at or above it (an LDS pool, about k entries)
//           contain the reports' top-k, whose exact k-th key T a rank search over
//           power-of-two slices of the live key range finds (then over the ids, for
//           ties: the lower id wins).  If no wave's bound reaches T, nothing left
//           unreported can beat T and the pool's top-k is the row's.  Otherwise the
//           waves that may hide elements >= T are rescanned into the pool first.
//           Reports come in id order and pools are built by order-preserving
//           compaction, so the k ids come out ascending without a sort.  Too many
//           rescans, an LDS overflow or more than 2048 tiles send the row to the same
//           search over all of its scores.  Rows with n_vis < k are padded with -1.
// Keys are the order-preserving uint32 image of the fp32 scores, so "larger key" is
// "larger score"; the result does not depend on launch shape or timing.
#include "select_impl.hpp"

namespace v4a {

// ------------------------------------------------------------------ score, bf16 MFMA
// S = QI (heads x d_I) . KI^T (d_I x blocks) on v_mfma_f32_16x16x32_bf16.
// Operand layout (wave64): lane l = 16*grp + col.  A (16 heads x 32 dims): lane holds
// head col, 8 dims of group grp; B (32 dims x 16 blocks): lane holds block col, the
// same 8 dims; C (16 heads x 16 blocks): lane holds block col, heads 4*grp + e.
// The dims a lane group carries only have to agree between A and B.
//
// A workgroup walks the tiles blockIdx.x, blockIdx.x + gridDim.x, ... of its row.
// Tile loads are fully coalesced (each wave instruction reads 1 KiB of consecutive
// block rows) into registers one tile ahead, then land in a padded LDS tile from
// which the MFMA operands are read; the indexer queries are staged in LDS once.
template <int MT, int KS>
__global__ __launch_bounds__(256) void score_bf16_kernel(ScoreP p) {
  constexpr int DI = KS * 32;
  constexpr int ROWB = DI * 2 + 16;          // LDS bytes per block row (+16: conflict-free reads)
  constexpr int CPR = DI * 2 / 16;           // 16-byte chunks per block row
  constexpr int LPT = kTile * CPR / 256;     // 16-byte loads per thread per tile
  __shared__ __align__(16) unsigned char sK[kTile * ROWB];
  __shared__ __align__(16) uint16_t sA[MT * 16 * DI];
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = (pos + 1) / p.ratio;
  const int64_t ntile_row = (nvis + kTile - 1) / kTile;
  int64_t tile = blockIdx.x;
  if (tile >= ntile_row) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const uint16_t* ki = reinterpret_cast<const uint16_t*>(p.ki) + (int64_t)b * p.ki_bs;

  uint4 pre[LPT];
  auto fetch = [&](int64_t t) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * 256;
      const int r = e / CPR, c = e - r * CPR;
      const int64_t j = t * kTile + r;
      pre[u] = make_uint4(0, 0, 0, 0);
      if (j < nvis) pre[u] = *reinterpret_cast<const uint4*>(ki + j * p.ki_rs + c * 8);
    }
  };
  fetch(tile);
  {
    const uint4* qi = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.qi) +
                                                     (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs);
    for (int e = tid; e < MT * 16 * DI / 8; e += 256) reinterpret_cast<uint4*>(sA)[e] = qi[e];
  }
  float w[MT][4];
  {
    const float4* wi = reinterpret_cast<const float4*>(p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4 v = wi[mt * 4 + grp];
      w[mt][0] = v.x; w[mt][1] = v.y; w[mt][2] = v.z; w[mt][3] = v.w;
    }
  }
  __syncthreads();
  bf16x8_t A[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      A[mt][s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&sA[(mt * 16 + col) * DI + s * 32 + grp * 8]));

  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  for (; tile < ntile_row; tile += gridDim.x) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * 256;
      const int r = e / CPR, c = e - r * CPR;
      *reinterpret_cast<uint4*>(sK + r * ROWB + c * 16) = pre[u];
    }
    __syncthreads();
    if (tile + gridDim.x < ntile_row) fetch(tile + gridDim.x);
    const int64_t tile0 = tile * kTile;
    float mine = 0.f;       // score of block tile0 + 64*wave + lane after the loop
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = wave * 64 + u * 16 + col;     // block of this lane's column
      float part = 0.f;
      bf16x8_t Bv[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        Bv[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sK + t * ROWB + (s * 4 + grp) * 16));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][s], Bv[s], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(w[mt][e], fmaxf(acc[e], 0.f), part);
      }
      part = col_sum4(part);
      if (grp == u) mine = part;
    }
    const int64_t j = tile0 + wave * 64 + lane;
    if (j < nvis) sc[j] = mine;
    wave_top(j < nvis ? pack_kid(score_key(mine), (uint32_t)j) : 0ull, (uint32_t)(tile0 + wave * 64),
             p.rep_key + (int64_t)lr * p.key_rs + tile * kTileTop + wave * kWaveTop,
             p.rep_info + (int64_t)lr * p.info_rs + tile * 4 + wave);
    __syncthreads();       // sK is rewritten by the next tile
  }
}

// ------------------------------------------------------------------ score, fp32 VALU
// One thread per block of the tile; the row's indexer queries and weights sit in LDS.
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreP p) {
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
  wave_top(v, (uint32_t)(tile0 + (threadIdx.x & ~63)),
           p.rep_key + (int64_t)lr * p.key_rs + (int64_t)blockIdx.x * kTileTop + (threadIdx.x >> 6) * kWaveTop,
           p.rep_info + (int64_t)lr * p.info_rs + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
}

hipError_t launch_score(int dtype, const ScoreP& p, int nrows, int ntiles, hipStream_t s, int tid) {
  const dim3 grid((unsigned)ntiles, (unsigned)nrows);
  if (dtype == 0) {
    const size_t lds = (size_t)(p.heads * p.dim + p.heads) * sizeof(float);
    V4A_LAUNCH(tid, score_f32_kernel, grid, dim3(256), lds, s, p);
    return hipGetLastError();
  }
  const int mt = p.heads / 16, ks = p.dim / 32;
  const dim3 pgrid((unsigned)p.wgs_per_row, (unsigned)nrows);
#define V4A_SCORE_CASE(M, K) \
  if (mt == M && ks == K) { V4A_LAUNCH(tid, (score_bf16_kernel<M, K>), pgrid, dim3(256), 0, s, p); return hipGetLastError(); }
  V4A_SCORE_CASE(1, 1) V4A_SCORE_CASE(1, 2)
  V4A_SCORE_CASE(2, 1) V4A_SCORE_CASE(2, 2)
  V4A_SCORE_CASE(4, 1) V4A_SCORE_CASE(4, 2)
  V4A_SCORE_CASE(8, 1) V4A_SCORE_CASE(8, 2)
#undef V4A_SCORE_CASE
  return hipErrorInvalidValue;
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

}  // namespace v4a
