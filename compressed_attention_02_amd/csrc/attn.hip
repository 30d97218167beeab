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
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct KeyList {
  int n_csa;
  int64_t e_vis, w_lo, n_keys;
};

__device__ __forceinline__ KeyList key_list(const AttnP& p, int64_t pos) {
  KeyList L;
  L.n_csa = (p.mask & 1u) ? p.topk : 0;
  L.e_vis = (p.mask & 2u) ? (pos + 1) / p.mh : 0;
  L.w_lo = pos - p.W + 1 > 0 ? pos - p.W + 1 : 0;
  const int64_t n_swa = ((p.mask & 4u) && p.W > 0) ? pos - L.w_lo + 1 : 0;
  L.n_keys = L.n_csa + L.e_vis + n_swa;
  return L;
}

// Row pointers of virtual key t; false for a CSA slot padded with -1.
template <typename T>
__device__ __forceinline__ bool key_rows(const AttnP& p, const KeyList& L, int b, int i, int64_t t,
                                         const T*& kp, const T*& vp) {
  if (t < L.n_csa) {
    const int32_t id = p.idx[(int64_t)b * p.idx_bs + (int64_t)i * p.idx_rs + t];
    if (id < 0) return false;
    kp = reinterpret_cast<const T*>(p.kc) + (int64_t)b * p.kc_bs + (int64_t)id * p.kc_rs;
    vp = reinterpret_cast<const T*>(p.vc) + (int64_t)b * p.vc_bs + (int64_t)id * p.vc_rs;
    return true;
  }
  t -= L.n_csa;
  if (t < L.e_vis) {
    kp = reinterpret_cast<const T*>(p.kh) + (int64_t)b * p.kh_bs + t * p.kh_rs;
    vp = reinterpret_cast<const T*>(p.vh) + (int64_t)b * p.vh_bs + t * p.vh_rs;
    return true;
  }
  t -= L.e_vis;
  const int64_t r = L.w_lo + t - p.raw_start[b];
  kp = reinterpret_cast<const T*>(p.kr) + (int64_t)b * p.kr_bs + r * p.kr_rs;
  vp = reinterpret_cast<const T*>(p.vr) + (int64_t)b * p.vr_bs + r * p.vr_rs;
  return true;
}

// Final normalisation of one head (base-2 running max m, sum l, unnormalised o).
// Returns the factor for o and writes lse (natural log) through *lse_out.
__device__ __forceinline__ float finish_head(float m, float l, const float* sink, int head, float* lse_out) {
  float scale_o = 1.f;
  if (sink) {
    const float z = sink[head] * kLog2e;
    const float mn = fmaxf(m, z);
    const float a = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    l = l * a + exp2f(z - mn);
    scale_o = a;
    m = mn;
  }
  *lse_out = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  return l > 0.f ? scale_o / l : 0.f;
}

// ------------------------------------------------------------------ bf16 MFMA
template <int NW, int D>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnP p) {
  constexpr int NT = NW * 64, CH = kAttnChunk, KS = D / 32, DT = D / 16;
  constexpr int KROW = D + 8;      // bf16 per K row in LDS (+16 B keeps ds_read_b128 conflict-free)
  constexpr int VROW = CH + 8;     // bf16 per V^T row in LDS
  constexpr int C8 = D / 8;        // 16-byte chunks per row
  constexpr int ITEMS = (CH / 2) * C8;          // (key pair, chunk) staging items
  constexpr int LPT = (ITEMS + NT - 1) / NT;
  __shared__ __align__(16) uint16_t sK[CH * KROW];
  __shared__ __align__(16) uint16_t sV[D * VROW];
  __shared__ int sOK[CH];

  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / p.tq, i = row - b * p.tq;
  const int64_t pos = p.pos0[b] + i;
  const KeyList L = key_list(p, pos);
  const int64_t k_begin = p.key_lo + (int64_t)split * p.keys_per_split;
  const int64_t k_end = min(min(L.n_keys, p.key_hi), k_begin + (int64_t)p.keys_per_split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int head = wave * 16 + col;
  const float sl2 = p.scale * kLog2e;

  uint4 pk[LPT][2], pv[LPT][2];
  int pok[LPT][2];
  auto fetch = [&](int64_t kc0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * NT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pk[u][h] = make_uint4(0, 0, 0, 0);
        pv[u][h] = make_uint4(0, 0, 0, 0);
        pok[u][h] = 0;
      }
      if (e < ITEMS) {
        const int kp2 = e / C8, c8 = e - kp2 * C8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t t = kc0 + 2 * kp2 + h;
          const uint16_t *kp, *vp;
          if (t < k_end && key_rows<uint16_t>(p, L, b, i, t, kp, vp)) {
            pk[u][h] = *reinterpret_cast<const uint4*>(kp + c8 * 8);
            pv[u][h] = *reinterpret_cast<const uint4*>(vp + c8 * 8);
            pok[u][h] = 1;
          }
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * NT;
      if (e < ITEMS) {
        const int kp2 = e / C8, c8 = e - kp2 * C8;
        const int key = 2 * kp2;
        *reinterpret_cast<uint4*>(&sK[key * KROW + c8 * 8]) = pk[u][0];
        *reinterpret_cast<uint4*>(&sK[(key + 1) * KROW + c8 * 8]) = pk[u][1];
        // V^T[d][key..key+1]: one 32-bit word per dim holds the pair
        const uint32_t a[4] = {pv[u][0].x, pv[u][0].y, pv[u][0].z, pv[u][0].w};
        const uint32_t c[4] = {pv[u][1].x, pv[u][1].y, pv[u][1].z, pv[u][1].w};
        uint32_t* vt = reinterpret_cast<uint32_t*>(&sV[(c8 * 8) * VROW + key]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vt[(2 * q) * (VROW / 2)] = (a[q] & 0xffffu) | (c[q] << 16);
          vt[(2 * q + 1) * (VROW / 2)] = (a[q] >> 16) | (c[q] & 0xffff0000u);
        }
        if (c8 == 0) { sOK[key] = pok[u][0]; sOK[key + 1] = pok[u][1]; }
      }
    }
  };

  if (k_begin < k_end) fetch(k_begin);
  bf16x8_t Qb[KS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bs +
                           (int64_t)i * p.q_rs + head * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      Qb[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + s * 32 + grp * 8));
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t kc0 = k_begin; kc0 < k_end; kc0 += CH) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kc0 + CH < k_end) fetch(kc0 + CH);

    // S^T for 4 tiles of 16 keys: lane holds head col, keys 16*kt + 4*grp + e
    f32x4 S[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t A = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&sK[(16 * kt + col) * KROW + s * 32 + grp * 8]));
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qb[s], S[kt], 0, 0, 0);
      }
    }
    float x[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * kt + e] = sOK[16 * kt + 4 * grp + e] ? S[kt][e] * sl2 : -INFINITY;
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) cm = fmaxf(cm, x[e]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float m_new = fmaxf(m_run, cm);
    float alpha = 1.f, pe[16];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 16; ++e) pe[e] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 16; ++e) pe[e] = exp2f(x[e] - m_new);
    }
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += pe[e];
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // P^T operand of keys 32kk + {4grp+e, 16+4grp+e}: tiles 2kk and 2kk+1
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = bf2f(f2bf(pe[8 * kk + e]));
        hi[4 + e] = bf2f(f2bf(pe[8 * kk + 4 + e]));
        lo[e] = pe[8 * kk + e] - hi[e];
        lo[4 + e] = pe[8 * kk + 4 + e] - hi[4 + e];
      }
      const bf16x8_t Bhi = __builtin_bit_cast(bf16x8_t, pack8(hi));
      const bf16x8_t Blo = __builtin_bit_cast(bf16x8_t, pack8(lo));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = &sV[(dt * 16 + col) * VROW + 32 * kk];
        const uint2 a0 = *reinterpret_cast<const uint2*>(vr + 4 * grp);
        const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 16 + 4 * grp);
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bhi, O[dt], 0, 0, 0);
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Blo, O[dt], 0, 0, 0);
      }
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  if (p.splits_total == 1) {
    float lse;
    const float f = finish_head(m_run, l_run, p.sink, head, &lse);
    float* orow = p.o + (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(orow + dt * 16 + 4 * grp) =
          make_float4(O[dt][0] * f, O[dt][1] * f, O[dt][2] * f, O[dt][3] * f);
    if (grp == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
  } else {
    const int64_t slot = ((int64_t)row * p.splits_total + p.split_base + split) * p.heads + head;
    float* po = p.part_o + slot * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16 + 4 * grp) = make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
    if (grp == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_run);
  }
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
      for (int c = lane; c < D; c += 64) sQ[wave][c] = qrow[c];
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
      float* orow = p.o + (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = acc[e] * f;
      if (lane == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
    } else {
      const int64_t slot = ((int64_t)row * p.splits_total + p.split_base + split) * p.heads + head;
#pragma unroll
      for (int e = 0; e < DPL; ++e) p.part_o[slot * D + lane + 64 * e] = acc[e];
      if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_run);
    }
  }
}

// ------------------------------------------------------------------ merge
// One 1024-thread workgroup per (row, head).  Split weights go to LDS; the weighted
// sum over splits is spread over 1024/D thread groups, each with four independent
// accumulators so that its loads are in flight together, and combined in LDS in a
// fixed order, so the result does not depend on timing.
constexpr int kMergeThreads = 1024;
constexpr int kMaxSplits = 1024;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnP p) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[kMergeThreads];
  const int row = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int b = row / p.tq, i = row - b * p.tq;
  const int S = p.splits_total, D = p.dim;
  const float* ml = p.part_ml + ((int64_t)row * S * p.heads + head) * 2;
  const int64_t ml_step = (int64_t)p.heads * 2;
  float ms = -INFINITY, ls = 0.f;
  if (tid < S) {
    const float2 v = *reinterpret_cast<const float2*>(ml + tid * ml_step);
    ms = v.x;
    ls = v.y;
  }
  // 1) global max of the split maxima (S <= kMergeThreads: one split per thread)
  float mx = wave_max(ms);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  float M = s_red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();
  // 2) split weights and the total sum
  const float wgt = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
  if (tid < S) s_w[tid] = wgt;
  float part = wave_sum(wgt * ls);
  if ((tid & 63) == 0) s_red[tid >> 6] = part;
  __syncthreads();
  float l = 0.f;
  for (int w = 0; w < kMergeThreads / 64; ++w) l += s_red[w];
  __syncthreads();
  // 3) weighted sum of the partial outputs: thread (g, c) takes splits g, g+G, ...
  const int G = kMergeThreads / D;
  const int c = tid % D, g = tid / D;
  const float* po = p.part_o + ((int64_t)row * S * p.heads + head) * D + c;
  const int64_t po_step = (int64_t)p.heads * D;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int s = g;
  for (; s + 3 * G < S; s += 4 * G) {
    a0 = fmaf(s_w[s], po[s * po_step], a0);
    a1 = fmaf(s_w[s + G], po[(s + G) * po_step], a1);
    a2 = fmaf(s_w[s + 2 * G], po[(s + 2 * G) * po_step], a2);
    a3 = fmaf(s_w[s + 3 * G], po[(s + 3 * G) * po_step], a3);
  }
  for (; s < S; s += G) a0 = fmaf(s_w[s], po[s * po_step], a0);
  s_red[tid] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (g == 0) {
    float acc = s_red[c];
    for (int gg = 1; gg < G; ++gg) acc += s_red[gg * D + c];
    float lse;
    const float f = finish_head(M, l, p.sink, head, &lse);
    p.o[(int64_t)b * p.o_bs + (int64_t)i * p.o_rs + (int64_t)head * D + c] = acc * f;
    if (c == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
  }
}

hipError_t launch_attn(int dtype, const AttnP& p, int nrows, hipStream_t s) {
  const dim3 grid((unsigned)p.splits, (unsigned)nrows);
  if (dtype == 0) {
    if (p.dim == 64) hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int nw = p.heads / 16;
#define V4A_ATTN_CASE(W)                                                                              \
  if (nw == W) {                                                                                      \
    if (p.dim == 64) hipLaunchKernelGGL((attn_bf16_kernel<W, 64>), grid, dim3(W * 64), 0, s, p);      \
    else hipLaunchKernelGGL((attn_bf16_kernel<W, 128>), grid, dim3(W * 64), 0, s, p);                 \
    return hipGetLastError();                                                                         \
  }
  V4A_ATTN_CASE(1) V4A_ATTN_CASE(2) V4A_ATTN_CASE(3) V4A_ATTN_CASE(4)
  V4A_ATTN_CASE(5) V4A_ATTN_CASE(6) V4A_ATTN_CASE(7) V4A_ATTN_CASE(8)
#undef V4A_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnP& p, int nrows, hipStream_t s) {
  if (p.splits_total > kMaxSplits) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nrows, (unsigned)p.heads), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
