// Device code of the indexer score on MFMA (bf16 or FP8 keys), shared by the score
// kernel of v4attn_index_topk and the decode step's first launch.  The design notes
// are at the top of index.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"
#include "select_impl.hpp"

namespace v4a {

// ------------------------------------------------------------------ score, bf16 MFMA
// S = QI (heads x d_I) . KI^T (d_I x blocks) on v_mfma_f32_16x16x32_bf16.
// Operand layout (wave64): lane l = 16*grp + col.  A (16 heads x 32 dims): lane holds
// head col, 8 dims of group grp; B (32 dims x 16 blocks): lane holds block col, the
// same 8 dims; C (16 heads x 16 blocks): lane holds block col, heads 4*grp + e.
// The dims a lane group carries only have to agree between A and B.
//
// A workgroup of NW waves walks the tiles x, x + wgs_per_row, ... of its row (x its
// index among the row's score workgroups), a tile being 64 * NW indexer keys, 64 per
// wave.  A tile goes from HBM straight into LDS (16 bytes per lane per load; lane
// l's piece lands at base + 16 l), unpadded, with the 16-byte pieces of row r
// permuted by XOR with swz_ki(r) so that both the loads and the B-fragment reads
// (16 rows, one piece column) are free of bank conflicts.  QI and the head weights
// stay in registers.  With NB = 2 the next tile loads while the current one is
// scored.  Each wave scores its 64 keys: ReLU, w-weighted head sum (row swaps across
// the 4 lane groups); the tile's report (its 8 best keys and the bound of the rest)
// comes from the waves' candidates, ranked by one wave.
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
// LDS of a score workgroup
template <int NW, int MT, int KS, int NB, bool FP8>
struct ScoreSmem {
  static constexpr int DI = KS * 32;
  static constexpr int KROWB = FP8 ? DI : DI * 2;   // LDS bytes per key row
  unsigned char sK[NB][64 * NW * KROWB];
  // the query rows until every wave holds its fragments, then the tiles' report
  // candidates (four waves of 64 blocks); a barrier separates the two uses
  union {
    unsigned char sQ[MT * 16 * DI * 2];
    TileStage stage;
  };
};

// Workgroup x (of the row's p.wgs_per_row) of launch row lr.
template <int NW, int MT, int KS, int NB, bool FP8>
__device__ __forceinline__ void score_block(const ScoreP& p, int x, int lr, ScoreSmem<NW, MT, KS, NB, FP8>& sm) {
  static_assert(NW == 4, "a workgroup tile is one report tile of four 64-block waves");
  constexpr int DI = KS * 32;
  constexpr int TILE = 64 * NW;              // keys per workgroup tile
  constexpr int ROWB = DI * 2;               // LDS bytes per query row
  constexpr int CPR = DI * 2 / 16;           // 16-byte pieces per query row
  constexpr int RPI = 64 / CPR;              // query rows per wave load
  constexpr int KROWB = FP8 ? DI : DI * 2;   // LDS bytes per key row
  constexpr int KCPR = KROWB / 16;           // 16-byte pieces per key row
  constexpr int KRPI = 64 / KCPR;            // key rows per wave load
  constexpr int IPW = 64 / KRPI;             // loads per wave per tile (its own 64 rows)
  constexpr int QN = MT * 16 / RPI;         // wave loads of the query rows (heads)
  auto& sK = sm.sK;
  unsigned char* sQ = sm.sQ;
  int b, i;
  int64_t pos;
  row_coords(p.row0 + lr, p.tq, p.pos0, b, i, pos);
  const int64_t nvis = uniform_i64((pos + 1) / p.ratio);
  const int64_t ntile_row = (nvis + TILE - 1) / TILE;
  int64_t tile = x;
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
      const int64_t j = min(t * TILE + r, nvis - 1);
      const int x = FP8 ? swz_k8<DI>(r) : swz_ki<DI>(r);
      lds_load16(ki + j * ki_rb + ((lane % KCPR) ^ x) * 16, lds_addr(buf + r0 * KROWB));
    }
  };
  // the query rows go to LDS once per workgroup (laid out like the key rows), ahead
  // of the first tile; the waves read their fragments from there
  {
    const uint16_t* qi = reinterpret_cast<const uint16_t*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
#pragma unroll
    for (int u = wave; u < QN; u += NW) {
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
      __syncthreads();   // the query rows are read: their LDS holds the wave picks from here on
    }
    // a wave reads only the key rows it loaded itself, so its own loads are all it
    // waits for (no barrier); the next tile may stay in flight
    if (next) __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int64_t tile0 = tile * TILE;
    float mine;             // score of key tile0 + 64*wave + lane after the loop
    float pu[4];            // this lane's part of key group u (keys 16 u .. 16 u + 15 of the wave)
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
      pu[u] = part;
    }
    // sum over the four lane groups, transposed: a row swap (groups 0<->1, 2<->3)
    // leaves even groups the pair sum of key group 2v and odd groups that of 2v+1; a
    // half swap (0<->2, 1<->3) completes group g's key group g (the additions of a
    // row-then-half sum)
    {
      const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[0]), __float_as_uint(pu[1]), false, false);
      const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[2]), __float_as_uint(pu[3]), false, false);
      const float a01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
      const float a23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
      const auto sh = __builtin_amdgcn_permlane32_swap(__float_as_uint(a01), __float_as_uint(a23), false, false);
      mine = __uint_as_float(sh[0]) + __uint_as_float(sh[1]);
    }
    const int64_t j = tile0 + wave * 64 + lane;
    if (j < nvis) sc[j] = mine;
    tile_report_waves(score_key(mine), j < nvis, c & 1, p.wave_top, sm.stage, p.rep_key + (int64_t)lr * p.key_rs + tile * kTileTop,
                      p.rep_info + (int64_t)lr * p.info_rs + tile);
    // the buffer is reloaded next, each wave into the rows it has just read
    if (NB == 2 && tile + 2 * stride < ntile_row)
      issue(tile + 2 * stride, sK[NB == 2 ? (c & 1) : 0]);
  }
}

// ------------------------------------------------------------------ score, several queries
// Prefill chunks: a workgroup of NQ waves takes NQ consecutive query rows of one
// sequence, one per wave (its QI fragments and head weights in registers), and walks
// the 256-key tiles x, x + gridDim.x, ... of the group's visible blocks.  Every tile
// goes to LDS once (double-buffered) and serves all NQ queries, so the indexer keys
// are read once per NQ queries instead of once per query.  A wave scores all 256
// keys of the tile for its query, per 16-key group; lane l ends with the scores of
// keys l, 64 + l, 128 + l and 192 + l, stores them and makes the four 64-block
// reports, in the layout of score_block.  Launch rows lr >= p.nrows (a partial last
// group) load and wait with the others but write nothing.
//
// The ReLU-weighted head sum is taken as s = (sum_h w_h x_h + sum_h w_h |x_h|) / 2
// (max(x, 0) = (x + |x|) / 2, exactly, for any w), x_h = qi_h . k: the second sum is one
// fused multiply-add per head with an absolute-value operand (half the vector work of
// a maximum and a multiply-add), and the first is the single dot product u . k with
// u = sum_h w_h qi_h, formed once per query in fp32 and split into three bf16 parts
// (hi, mid, lo: about 24 significant bits) that fill three rows of a fifth MFMA head
// tile.  The two sums agree with the per-head form to fp32 rounding of terms of the
// size of sum_h w_h |x_h|.
constexpr int kScoreRowsQ = 8;   // query rows per workgroup of score_rows_kernel

__global__ __launch_bounds__(kScoreRowsQ * 64, 4) void score_rows_kernel(ScoreP p) {
  constexpr int NQ = kScoreRowsQ, DI = 64, MT = 4, KS = 2, ROWB = DI * 2, KCPR = ROWB / 16, KRPI = 64 / KCPR;
  constexpr int IPW = kTile / KRPI / NQ;   // tile loads per wave
  __shared__ __align__(16) unsigned char sK[2][kTile * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr0 = blockIdx.y * NQ;                      // the group's first launch row
  const int lr = lr0 + wave;                            // this wave's query
  const bool have = lr < p.nrows;
  const int last = min(lr0 + NQ, p.nrows) - 1;          // the group's last query: most visible blocks
  int b, i, bl, il;
  int64_t pos, pos_l;
  row_coords(p.row0 + (have ? lr : last), p.tq, p.pos0, b, i, pos);
  row_coords(p.row0 + last, p.tq, p.pos0, bl, il, pos_l);
  const int64_t nvis = (pos + 1) / p.ratio;             // this query's
  const int64_t nvis_g = uniform_i64((pos_l + 1) / p.ratio);
  // the tiles walked: every one, or (sampling) 0, S, 2S, ...; tile v of the walk is
  // tile v * S of the row
  const int64_t S = p.sample_stride > 0 ? p.sample_stride : 1;
  const int64_t ntile = ((nvis_g + kTile - 1) / kTile + S - 1) / S;
  int64_t tile = blockIdx.x;
  const int64_t stride = gridDim.x;
  if (tile >= ntile) return;
  if (p.repair) {   // a repair pass: only groups holding a flagged row run
    bool any = false;
#pragma unroll
    for (int q = 0; q < NQ; ++q) any |= lr0 + q < p.nrows && p.repair[lr0 + q] != 0u;
    if (!any) return;
  }
  const unsigned char* ki = reinterpret_cast<const unsigned char*>(p.ki) + (int64_t)bl * p.ki_bs * 2;
  const int64_t ki_rb = p.ki_rs * 2;
  auto issue = [&](int64_t t, unsigned char* buf) {
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int r0 = (wave * IPW + u) * KRPI;
      const int r = r0 + lane / KCPR;
      const int64_t j = min(t * S * kTile + r, nvis_g - 1);
      lds_load16(ki + j * ki_rb + ((lane % KCPR) ^ swz_ki<DI>(r)) * 16, lds_addr(buf + r0 * ROWB));
    }
  };
  // the query's fragments (head mt*16 + col, dims s*32 + grp*8 .. + 8) and weights;
  // U: rows 0, 1, 2 of the fifth head tile are the parts of u = sum_h w_h qi_h, the
  // rest zero (lane (col, grp) holds row col, dims s*32 + grp*8 .. + 8 like A)
  bf16x8_t A[MT][KS], U[KS];
  float w[MT][4];
  {
    const uint16_t* qi = reinterpret_cast<const uint16_t*>(p.qi) + (int64_t)b * p.qi_bs + (int64_t)i * p.qi_rs;
    const float* wi = p.wi + (int64_t)b * p.wi_bs + (int64_t)i * p.wi_rs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        A[mt][s2] = *reinterpret_cast<const bf16x8_t*>(qi + (mt * 16 + col) * DI + s2 * 32 + grp * 8);
      const f32x4 wq = *reinterpret_cast<const f32x4*>(wi + mt * 16 + 4 * grp);
      // the halving of (u.k + sum_h w_h |x_h|) / 2 goes into w and u (exact)
      w[mt][0] = 0.5f * wq[0]; w[mt][1] = 0.5f * wq[1]; w[mt][2] = 0.5f * wq[2]; w[mt][3] = 0.5f * wq[3];
    }
    float u[KS][8];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) u[s2][e] = 0.f;
    for (int h = 0; h < MT * 16; ++h) {   // in head order, the same in every lane of a row
      const float wh = wi[h];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        float q8[8];
        unpack8(*reinterpret_cast<const uint4*>(qi + h * DI + s2 * 32 + grp * 8), q8);
#pragma unroll
        for (int e = 0; e < 8; ++e) u[s2][e] = fmaf(wh, q8[e], u[s2][e]);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float uh = 0.5f * u[s2][e];
        const float hi = bf2f(f2bf(uh));
        const float mid = bf2f(f2bf(uh - hi));
        const float lo = uh - hi - mid;
        // rows 0, 4, 8: the parts land in lane groups 0, 1, 2 (output element 0),
        // which the cross-lane sum of the score adds up
        const float v = col == 0 ? hi : col == 4 ? mid : col == 8 ? lo : 0.f;
        U[s2][e] = (__bf16)v;
      }
  }
  // threshold mode: this query's threshold key
  const uint32_t th = (p.theta && have) ? p.theta[lr] : 0u;
  // (the compiler does not count the tile loads below, so it would wait for them too
  // at the fragments' first use: they are waited for here, before any tile load)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  issue(tile, sK[0]);
  if (tile + stride < ntile) issue(tile + stride, sK[1]);
  float* sc = p.scores + (int64_t)lr * p.sc_rs;
  const int kx = swz_ki<DI>(col);   // rows 16u + col share col's XOR
  for (int c = 0; tile < ntile; tile += stride, ++c) {
    unsigned char* buf = sK[c & 1];
    if (tile + stride < ntile) __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();   // every wave's share of the tile is in LDS
    // lane (col, grp) ends with the score of key 16 u + col for u = 4 q + grp in mine[q]
    float mine[4];
#pragma unroll
    for (int q4 = 0; q4 < kTile / 64; ++q4) {
      float pu[4];   // this lane's part of key group u = 4 q4 + uu
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int t = (4 * q4 + uu) * 16 + col;
        bf16x8_t Bv[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          Bv[s2] = *reinterpret_cast<const bf16x8_t*>(buf + t * ROWB + (((s2 * 4 + grp) ^ kx) * 16));
        f32x4 lin = {0.f, 0.f, 0.f, 0.f};   // a part of u . k / 2 in element 0 of lane groups 0..2
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) lin = __builtin_amdgcn_mfma_f32_16x16x32_bf16(U[s2], Bv[s2], lin, 0, 0, 0);
        float part = lin[0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][s2], Bv[s2], acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) part = fmaf(w[mt][e], fabsf(acc[e]), part);
        }
        pu[uu] = part;
      }
      // sum over the four lane groups, transposed: a row swap (groups 0<->1, 2<->3)
      // pairs the parts of key groups 2v and 2v+1 so that even groups hold 2v's pair
      // sum and odd groups 2v+1's; a half swap (0<->2, 1<->3) then completes group g's
      // key group 4 q4 + g.  The additions are those of a row-then-half sum.
      const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[0]), __float_as_uint(pu[1]), false, false);
      const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[2]), __float_as_uint(pu[3]), false, false);
      const float a01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
      const float a23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
      const auto sh = __builtin_amdgcn_permlane32_swap(__float_as_uint(a01), __float_as_uint(a23), false, false);
      mine[q4] = __uint_as_float(sh[0]) + __uint_as_float(sh[1]);
    }
    if (have) {
      const int64_t rt = tile * S;   // the row's tile
      const int64_t tile0 = rt * kTile;
      uint32_t* keys = p.rep_key + (int64_t)lr * p.key_rs + rt * kTileTop;
      uint4* info = p.rep_info + (int64_t)lr * p.info_rs + rt;
      uint32_t kb[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) kb[blk] = tile0 + 64 * blk + lane < nvis ? score_key(mine[blk]) : 0u;
      auto store = [&]() {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
          if (tile0 + 64 * blk + lane < nvis) sc[tile0 + 64 * blk + lane] = mine[blk];
      };
      if (p.sample_stride > 0) {
        store();   // a sampled tile: its scores are all the threshold needs
      } else if (p.theta) {
        // the keys at or above the row's threshold: when there are at most kTileTop,
        // they are the report, every other key is below the threshold (the bound),
        // and no score is stored; else the exact best kTileTop and the scores
        uint64_t won[4];
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          won[q] = __ballot(kb[q] != 0u && kb[q] >= th);
          c += (uint32_t)__popcll(won[q]);
        }
        if (c <= (uint32_t)kTileTop) {
          tile_emit_few(kb, won, th ? th - 1u : 0u, keys, info);
        } else {
          store();
          uint32_t bound;
          tile_rounds<kTileTop>(kb, won, bound);
          tile_emit(kb, won, bound, keys, info);
        }
      } else {
        store();
        tile_report<kPrefillTileTop>(kb, keys, info);
      }
    }
    __syncthreads();   // every wave is done with this buffer
    if (tile + 2 * stride < ntile) issue(tile + 2 * stride, buf);
  }
}

}  // namespace v4a
