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
#include "qprep_impl.hpp"
#include "select_impl.hpp"

namespace v4a {

// ------------------------------------------------------------------ score, bf16 MFMA
// S = QI (heads x d_I) . KI^T (d_I x blocks) on v_mfma_f32_16x16x32_bf16.
// Operand layout (wave64): lane l = 16*grp + col.  A (16 heads x 32 dims): lane holds
// head col, 8 dims of group grp; B (32 dims x 16 blocks): lane holds block col, the
// same 8 dims; C (16 heads x 16 blocks): lane holds block col, heads 4*grp + e.
// The dims a lane group carries only have to agree between A and B.
//
// A workgroup (4 waves) walks the tiles x, x + wgs_per_row, ... of its row (x its
// index among the row's score workgroups; with the query prep hosted, the first
// prep_x workgroups of each row prepare the attention queries instead).  A tile of 256 indexer keys goes from HBM straight into LDS (16 bytes per
// lane per load; lane l's piece lands at base + 16 l), unpadded, with the 16-byte
// pieces of row r permuted by XOR with swz_ki(r) so that both the loads and the
// B-fragment reads (16 rows, one piece column) are free of bank conflicts.  QI and
// the head weights stay in registers.  With NB = 2 the next tile loads while the
// current one is scored.  Each wave scores 64 keys: ReLU, w-weighted head sum (row
// swaps across the 4 lane groups), then its top-4 report.
template <int DI> __device__ __forceinline__ int swz_ki(int r) { return DI == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
// FP8 key rows (DI bytes, DI/16 pieces): rows r that share a 256-byte bank offset
// (r mod 256/DI) get distinct piece XORs, so the 8-byte fragment reads of 16 rows
// at one logical piece are free of bank conflicts
template <int DI> __device__ __forceinline__ int swz_k8(int r) { return (r / (256 / DI)) % (DI / 16); }

// 8 FP8 E4M3 codes (bytes of v, low first) -> 8 bf16, exactly (every E4M3 value,
// subnormals and NaN included, is a bf16 value): gfx950's packed conversion with a
// unit scale, two codes per instruction
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint2 v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1),
                                                 __builtin_bit_cast(uint32_t, w2), __builtin_bit_cast(uint32_t, w3)));
}

// FP8: the key rows are FP8 E4M3 codes with one fp32 scale per row; they stay codes
// in LDS (half the bytes), each fragment is decoded to bf16 exactly, and the row's
// scale multiplies its 16 dot products before the ReLU.
template <int MT, int KS, int NB, bool FP8>
__global__ __launch_bounds__(256) void score_bf16_kernel(ScoreP p) {
  constexpr int DI = KS * 32;
  constexpr int ROWB = DI * 2;               // LDS bytes per query row
  constexpr int CPR = DI * 2 / 16;           // 16-byte pieces per query row
  constexpr int RPI = 64 / CPR;              // query rows per wave load
  constexpr int KROWB = FP8 ? DI : DI * 2;   // LDS bytes per key row
  constexpr int KCPR = KROWB / 16;           // 16-byte pieces per key row
  constexpr int KRPI = 64 / KCPR;            // key rows per wave load
  constexpr int IPW = kTile / KRPI / 4;      // loads per wave per tile
  constexpr int QN = MT * 16 / RPI;         // wave loads of the query rows (heads)
  __shared__ __align__(16) unsigned char sK[NB][kTile * KROWB];
  __shared__ __align__(16) unsigned char sQ[MT * 16 * ROWB];
  if ((int)blockIdx.x < p.prep_x) {   // first (dispatched early): the attention queries of row y
    qprep_block(p.prep, p.row0 + blockIdx.y, blockIdx.x);
    return;
  }
  const int lr = blockIdx.y;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = uniform_i64((pos + 1) / p.ratio);
  const int64_t ntile_row = (nvis + kTile - 1) / kTile;
  int64_t tile = (int)blockIdx.x - p.prep_x;
  const int64_t stride = p.wgs_per_row;   // score workgroups of the row
  if (tile >= ntile_row) return;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // key rows in bytes (row strides are in elements: 2 bytes for bf16, 1 for FP8)
  const unsigned char* ki = reinterpret_cast<const unsigned char*>(p.ki) + (int64_t)b * p.ki_bs * (FP8 ? 1 : 2);
  const int64_t ki_rb = p.ki_rs * (FP8 ? 1 : 2);

  // rows past n_vis re-read the last visible row; their scores are dropped
  auto issue = [&](int64_t t, unsigned char* buf) {
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int r0 = (wave * IPW + u) * KRPI;
      const int r = r0 + lane / KCPR;
      const int64_t j = min(t * kTile + r, nvis - 1);
      const int x = FP8 ? swz_k8<DI>(r) : swz_ki<DI>(r);
      lds_load16(ki + j * ki_rb + ((lane % KCPR) ^ x) * 16, lds_addr(buf + r0 * KROWB));
    }
  };
  // the query rows go to LDS once per workgroup (laid out like the key rows), ahead
  // of the first tile; the waves read their fragments from there
  {
    const uint16_t* qi = reinterpret_cast<const uint16_t*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
#pragma unroll
    for (int u = wave; u < QN; u += 4) {
      const int r = u * RPI + lane / CPR;
      lds_load16(qi + r * DI + ((lane % CPR) ^ swz_ki<DI>(r)) * 8, lds_addr(sQ + u * RPI * ROWB));
    }
  }
  float w[MT][4];
  {
    const float* wi = p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 wq = *reinterpret_cast<const f32x4*>(wi + mt * 16 + 4 * grp);
      w[mt][0] = wq[0]; w[mt][1] = wq[1]; w[mt][2] = wq[2]; w[mt][3] = wq[3];
    }
  }
  // the tile loads go out last: the query rows and the weights are the oldest loads
  issue(tile, sK[0]);
  if (NB == 2 && tile + stride < ntile_row) issue(tile + stride, sK[NB - 1]);
  bf16x8_t A[MT][KS];
  bool have_q = false;

  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int kx = swz_ki<DI>(col);          // rows 16u + col of a wave share col's XOR
  const int kx8 = swz_k8<DI>(col);         // (the same holds for the FP8 layout)
  for (int c = 0; tile < ntile_row; tile += stride, ++c) {
    const unsigned char* buf = sK[NB == 2 ? (c & 1) : 0];
    const bool next = NB == 2 && tile + stride < ntile_row;
    if (!have_q) {
      // every wave's share of the query rows is in LDS once the loads issued before
      // the tiles are done (vmcnt counts in issue order); then the query fragments:
      // row mt*16 + col, piece 4s + grp (the rows share col's XOR)
      if (next) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          A[mt][s] = *reinterpret_cast<const bf16x8_t*>(sQ + (mt * 16 + col) * ROWB + (((s * 4 + grp) ^ kx) * 16));
      have_q = true;
    }
    // a wave reads only the key rows it loaded itself, so its own loads are all it
    // waits for (no barrier); the next tile may stay in flight
    if (next) __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int64_t tile0 = tile * kTile;
    float mine = 0.f;       // score of key tile0 + 64*wave + lane after the loop
    float kscale = 1.f;     // FP8: the scale of that key's row (rows past n_vis: the last row's)
    if constexpr (FP8)
      kscale = p.ki_scale[(int64_t)b * p.ks_bs + min(tile0 + wave * 64 + lane, nvis - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = wave * 64 + u * 16 + col;     // key row of this lane's column
      float part = 0.f;
      bf16x8_t Bv[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (FP8)   // elements s*32 + grp*8: piece 2s + grp/2, half grp%2
          Bv[s] = fp8x8_to_bf16(*reinterpret_cast<const uint2*>(buf + t * KROWB + (((2 * s + (grp >> 1)) ^ kx8) * 16) +
                                                                (grp & 1) * 8));
        else
          Bv[s] = *reinterpret_cast<const bf16x8_t*>(buf + t * ROWB + (((s * 4 + grp) ^ kx) * 16));
      }
      // FP8: the scale of this lane's key column (key u*16 + col of the wave)
      const float cs = FP8 ? __shfl(kscale, u * 16 + col) : 1.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][s], Bv[s], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(w[mt][e], fmaxf(FP8 ? acc[e] * cs : acc[e], 0.f), part);
      }
      part = col_sum4(part);
      if (grp == u) mine = part;
    }
    const int64_t j = tile0 + wave * 64 + lane;
    if (j < nvis) sc[j] = mine;
    wave_top(score_key(mine), j < nvis, p.rep_key + (int64_t)lr * p.key_rs + tile * kTileTop + wave * kWaveTop,
             p.rep_info + (int64_t)lr * p.info_rs + tile * 4 + wave);
    // the buffer is reloaded next, each wave into the rows it has just read
    if (NB == 2 && tile + 2 * stride < ntile_row)
      issue(tile + 2 * stride, sK[NB == 2 ? (c & 1) : 0]);
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
  wave_top(v, j < nvis, p.rep_key + (int64_t)lr * p.key_rs + (int64_t)blockIdx.x * kTileTop + (threadIdx.x >> 6) * kWaveTop,
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
