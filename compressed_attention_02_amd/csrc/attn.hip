// sparse_attn_decode (+ the per-query variant used for prefill chunks) and lse_merge.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
// CSA step 3 is multi-query attention over the selected compressed blocks; HCA
// attends densely to every compressed entry; the sliding-window branch adds the
// most recent 128 raw tokens; an optional learnable sink logit joins the softmax
// denominator.  The layer configuration puts all three branches under one softmax.
//
// Each query (row) sees a virtual key list: [CSA picks | HCA entries 0..e_vis-1 |
// raw positions max(0,p-W+1)..p].  The list is cut into splits of keys_per_split
// keys; a workgroup owns one (split, row), walks its keys in chunks of 64 and keeps
// an online softmax per head.  With one split the workgroup writes o and lse
// directly; otherwise it writes (U, m, l) partials that merge_kernel combines in a
// fixed split order (no float atomics: results do not depend on timing).
//
// bf16 path, per chunk of 64 keys (one KV head shared by all H query heads, MQA):
//   * K rows of the chunk go to LDS row-major, V rows transposed (V^T[d][key]);
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: keys on M, 16 heads per wave on N,
//     so a lane ends up with 8 keys of one head and the row statistics need only
//     two cross-lane steps;
//   * O^T += V^T P^T on the same MFMA, P split into bf16 hi + lo parts so that P
//     keeps ~16 significant bits (decode is bandwidth-bound, the second MFMA is
//     free); the keys a lane holds in P^T are exactly the keys it holds in S^T.
// Softmax runs in base 2: logits are pre-multiplied by scale*log2(e); partial m is
// kept in that unit and converted back to natural log for lse.
#include "attn_impl.hpp"
#include "qprep_impl.hpp"

namespace v4a {

// One workgroup of NW waves per (split, row); two workgroups per CU when each wave
// computes one head tile over half the keys (KP = 2; four waves per SIMD), two head
// tiles over half the keys (KP = 2, HT = 2, four waves: two waves per SIMD, up to 256
// registers each), or NW <= 4.  Shared entries of
// D = 512 take most of the LDS (two 64 KB chunk buffers): one workgroup of 8 waves
// per CU, two waves per SIMD, a wave pair per head tile (attend_wide_*).
template <int NW, int HT, int D, int KP>
constexpr int attn_waves_per_eu() {
  return D == 512 ? 2 : (KP == 2 && HT == 2) ? 2 : KP == 2 ? 4 : NW * HT <= 4 ? 2 : 1;
}
template <int NW, int HT, int D, int KP, bool QP, bool SKV, bool F8>
__global__ __launch_bounds__(NW * 64, (attn_waves_per_eu<NW, HT, D, KP>())) void attn_bf16_kernel(AttnP p) {
  __shared__ __align__(16) AttnSmem<D, SKV> sm;
  attn_block<NW, HT, D, KP, QP, SKV, F8>(p, blockIdx.x, blockIdx.y, sm, sm.idx);
}

template <int NW, int HT, int D, int KP, bool SKV, bool F8>
static void launch_bf16(const AttnP& p, dim3 grid, hipStream_t s, int tid) {
  if (p.rope_out) V4A_LAUNCH(tid, (attn_bf16_kernel<NW, HT, D, KP, true, SKV, F8>), grid, dim3(NW * 64), 0, s, p);
  else V4A_LAUNCH(tid, (attn_bf16_kernel<NW, HT, D, KP, false, SKV, F8>), grid, dim3(NW * 64), 0, s, p);
}
// rows of up to 128: bf16 or FP8 caches
template <int NW, int HT, int D, int KP>
static void launch_narrow(const AttnP& p, dim3 grid, hipStream_t s, int tid) {
  if (p.f8) launch_bf16<NW, HT, D, KP, false, true>(p, grid, s, tid);
  else launch_bf16<NW, HT, D, KP, false, false>(p, grid, s, tid);
}

// ------------------------------------------------------------------ fp32 VALU
// One wave per head (heads strided over the 4 waves); a lane scores one key of a
// 64-key chunk, then every lane accumulates its D/64 output columns.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnP p) {
  constexpr int DPL = D / 64;  // output columns per lane
  __shared__ float sQ[4][D];
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / p.tq, i = row - b * p.tq;
  const int64_t pos = p.pos0[b] + i;
  const KeyList L = key_list(p, pos);
  const int64_t k_begin = p.key_lo + (int64_t)split * p.keys_per_split;
  const int64_t k_end = min(min(L.n_keys, p.key_hi), k_begin + (int64_t)p.keys_per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float sl2 = p.scale * kLog2e;

  for (int h0 = 0; h0 < p.heads; h0 += 4) {
    const int head = h0 + wave;
    __syncthreads();
    if (head < p.heads) {
      const float* qrow = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_bs + (int64_t)i * p.q_rs + head * D;
      float qv[DPL], ss = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        qv[e] = qrow[lane + 64 * e];
        ss = fmaf(qv[e], qv[e], ss);
      }
      if (p.q_norm) {  // RMSNorm of the head's query
        const float rq = rsqrtf(wave_sum(ss) / (float)D + p.norm_eps);
#pragma unroll
        for (int e = 0; e < DPL; ++e) qv[e] = qv[e] * rq * p.q_norm[lane + 64 * e];
      }
      if (p.rope) {  // then its rotation at pos: pair partners sit in neighbouring lanes
        const int lo = D - p.rope;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          const float other = __shfl_xor(qv[e], 1);
          const int ch = lane + 64 * e;
          if (ch >= lo) {
            float cs, sn;
            rope_cs((double)pos, (ch - lo) / 2, p.rope, p.rope_lb, cs, sn);
            qv[e] = (ch & 1) ? fmaf(other, sn, qv[e] * cs) : fmaf(-other, sn, qv[e] * cs);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) sQ[wave][lane + 64 * e] = qv[e];
    }
    __syncthreads();
    if (head >= p.heads) continue;
    float m_run = -INFINITY, l_run = 0.f, acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    for (int64_t kc0 = k_begin; kc0 < k_end; kc0 += 64) {
      const int64_t t = kc0 + lane;
      const float *kp, *vp;
      float x = -INFINITY;
      if (t < k_end && key_rows<float>(p, L, b, i, t, kp, vp)) {
        float dot = 0.f;
        for (int c = 0; c < D; c += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(kp + c);
          dot = fmaf(sQ[wave][c], kv.x, dot);
          dot = fmaf(sQ[wave][c + 1], kv.y, dot);
          dot = fmaf(sQ[wave][c + 2], kv.z, dot);
          dot = fmaf(sQ[wave][c + 3], kv.w, dot);
        }
        x = dot * sl2;
      }
      const float m_new = fmaxf(m_run, wave_max(x));
      float alpha = 1.f, pe = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run - m_new);
        pe = exp2f(x - m_new);
      }
      m_run = m_new;
      l_run = l_run * alpha + wave_sum(pe);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
      const int64_t cnt = min<int64_t>(64, k_end - kc0);
      for (int tt = 0; tt < cnt; ++tt) {
        const float pt = __shfl(pe, tt);
        const float *kq, *vq;
        if (pt != 0.f && key_rows<float>(p, L, b, i, kc0 + tt, kq, vq)) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pt, vq[lane + 64 * e], acc[e]);
        }
      }
    }
    if (p.splits_total == 1) {
      float lse;
      const float f = finish_head(m_run, l_run, p.sink, head, &lse);
      const int64_t orow = (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float a = acc[e] * f;
        if (p.rope_out) a = rope_back_pair(p, a, lane + 64 * e, pos);
        store_out1(p.o, p.o_bf16, orow + lane + 64 * e, a);
      }
      if (lane == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
    } else {
      const int64_t slot = ((int64_t)row * p.heads + head) * p.splits_total + p.split_base + split;
#pragma unroll
      for (int e = 0; e < DPL; ++e) p.part_o[slot * D + lane + 64 * e] = acc[e];
      if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_run);
    }
  }
}

// ------------------------------------------------------------------ prefill query tiles
// One workgroup per (query tile, sequence), one per CU.  d = 128: sixteen waves of
// one head tile each (four waves per SIMD); d = 64: eight waves of two.
template <int D, int NW, int HT>
__global__ __launch_bounds__(NW * 64, (NW / 4)) void attn_qtile_kernel(AttnP p) {
  __shared__ __align__(16) QTileSmem<D> sm;
  attn_qtile_block<D, NW, HT>(p, blockIdx.x, blockIdx.y, sm);
}
constexpr int kQTileNW128 = 16, kQTileHT128 = 1;

hipError_t launch_attn_qtile(const AttnP& p, int batch, hipStream_t s, int tid) {
  const int ntq = p.heads / 16;
  if (p.heads % 32 != 0 || ntq < 2 || ntq > 8 || (p.dim != 64 && p.dim != 128) || p.f8 || p.skv ||
      p.splits_total < 2)
    return hipErrorInvalidValue;
  const int nw = p.dim == 64 ? 8 : kQTileNW128, ht = p.dim == 64 ? 2 : kQTileHT128;
  const int wpq = ntq / ht;
  if (wpq < 1 || nw % wpq != 0 || nw / wpq > kMaxQTile) return hipErrorInvalidValue;
  const int qt = nw / wpq;
  const dim3 grid((unsigned)((p.tq + qt - 1) / qt), (unsigned)batch);
  if (p.dim == 64) V4A_LAUNCH(tid, (attn_qtile_kernel<64, 8, 2>), grid, dim3(8 * 64), 0, s, p);
  else V4A_LAUNCH(tid, (attn_qtile_kernel<128, kQTileNW128, kQTileHT128>), grid, dim3(kQTileNW128 * 64), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ query prep
// once per row, when no score launch of the same step carries it (qprep_impl.hpp)
__global__ __launch_bounds__(256) void qprep_kernel(QPrepP p) { qprep_block(p, blockIdx.x, blockIdx.y); }

hipError_t launch_qprep(const QPrepP& p, int nrows, hipStream_t s, int tid) {
  if (p.dim != 64 && p.dim != 128 && p.dim != 512) return hipErrorInvalidValue;
  V4A_LAUNCH(tid, qprep_kernel, dim3((unsigned)nrows, (unsigned)qprep_blocks(p)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge
// One 256-thread workgroup per (row, head, DW output columns): the merge reads every
// partial once, so it is spread over as many workgroups as there are column
// slices to keep all CUs loading; merge_head holds the arithmetic.  DW = 32 by
// default; with few splits a wider slice (64 or 128 columns) still loads all of a
// thread's partials in its first batch and needs fewer, fuller workgroups (not in
// batch-invariant plans, where the width, which sets how the splits are grouped in
// the sum, must not follow the batch).
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 32;          // the narrowest slice; every dim is a multiple
constexpr int kMergeMinWorkgroups = 512;

template <int DW>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnP p) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[kMergeThreads];
  merge_head<kMergeThreads, DW>(p, blockIdx.x, blockIdx.y, blockIdx.z * DW, s_w, s_red);
}

hipError_t launch_attn(int dtype, const AttnP& p, int nrows, hipStream_t s, int tid) {
  if (p.head_groups < 1 || (dtype == 0 && p.head_groups != 1)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.splits * p.head_groups), (unsigned)nrows);
  if (dtype == 0) {
    if (p.dim == 64) V4A_LAUNCH(tid, attn_f32_kernel<64>, grid, dim3(256), 0, s, p);
    else if (p.dim == 128) V4A_LAUNCH(tid, attn_f32_kernel<128>, grid, dim3(256), 0, s, p);
    else V4A_LAUNCH(tid, attn_f32_kernel<512>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int ntile = p.heads / 16 / p.head_groups;   // tiles per workgroup
  if (p.heads % (16 * p.head_groups) != 0 || ntile < 1 || ntile > 8) return hipErrorInvalidValue;
  if (p.dim == 512) {
    // shared entries only: 8 waves, a wave pair per head tile, four tiles per
    // workgroup (more heads come in head groups)
    if (!p.skv || ntile > kWideTiles) return hipErrorInvalidValue;
    if (p.f8) launch_bf16<8, 1, 512, 1, true, true>(p, grid, s, tid);
    else launch_bf16<8, 1, 512, 1, true, false>(p, grid, s, tid);
    return hipGetLastError();
  }
  // 8 waves of 16 heads each: up to 64 heads, two waves per head tile split every
  // chunk's keys in half (four waves per SIMD); exactly four tiles with bf16 caches
  // take four waves of two tiles instead (below); above 64 heads, one wave per head
  // tile (shared entries at d <= 128 arrive with the value pointers aimed at the keys)
  if (ntile == 4 && !p.f8) {
    // four tiles: four waves of two head tiles each, two waves per key half, so a
    // wave's K and V fragment reads from LDS serve two tiles (half the LDS reads of
    // one tile per wave); two workgroups per CU
    if (p.dim == 64) launch_bf16<4, 2, 64, 2, false, false>(p, grid, s, tid);
    else launch_bf16<4, 2, 128, 2, false, false>(p, grid, s, tid);
  } else if (ntile <= 4) {
    if (p.dim == 64) launch_narrow<8, 1, 64, 2>(p, grid, s, tid);
    else launch_narrow<8, 1, 128, 2>(p, grid, s, tid);
  } else {
    if (p.dim == 64) launch_narrow<8, 1, 64, 1>(p, grid, s, tid);
    else launch_narrow<8, 1, 128, 1>(p, grid, s, tid);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnP& p, int nrows, bool fixed_width, hipStream_t s, int tid) {
  if (p.splits_total > kMaxSplits) return hipErrorInvalidValue;
  if (p.dim % kMergeCols != 0 || p.splits_total < 1) return hipErrorInvalidValue;
  const int S = p.splits_total;
  auto fits = [&](int dw) {   // one batch of loads per thread, and enough workgroups
    return !fixed_width && p.dim % dw == 0 && (kMergeThreads / dw) * kMergeBatch >= S &&
           (int64_t)nrows * p.heads * (p.dim / dw) >= kMergeMinWorkgroups;
  };
  const dim3 blk(kMergeThreads);
  if (fits(128)) V4A_LAUNCH(tid, merge_kernel<128>, dim3((unsigned)nrows, (unsigned)p.heads, (unsigned)(p.dim / 128)), blk, 0, s, p);
  else if (fits(64)) V4A_LAUNCH(tid, merge_kernel<64>, dim3((unsigned)nrows, (unsigned)p.heads, (unsigned)(p.dim / 64)), blk, 0, s, p);
  else V4A_LAUNCH(tid, merge_kernel<kMergeCols>, dim3((unsigned)nrows, (unsigned)p.heads, (unsigned)(p.dim / kMergeCols)), blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
