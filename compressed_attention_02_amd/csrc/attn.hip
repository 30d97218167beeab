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
// keys; a workgroup owns one (split, row), walks its keys in chunks of 32 and keeps
// an online softmax per head.  With one split the workgroup writes o and lse
// directly; otherwise it writes (U, m, l) partials that merge_kernel combines in a
// fixed split order (no float atomics: results do not depend on timing).
//
// bf16 path, per chunk (one KV head shared by all H query heads, MQA):
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
  constexpr int LPT = (CH * C8 + NT - 1) / NT;
  __shared__ __align__(16) uint16_t sK[CH * KROW];
  __shared__ __align__(16) uint16_t sV[D * VROW];
  __shared__ int sOK[CH];

  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / p.tq, i = row - b * p.tq;
  const int64_t pos = p.pos0[b] + i;
  const KeyList L = key_list(p, pos);
  const int64_t k_begin = (int64_t)split * p.keys_per_split;
  const int64_t k_end = min(L.n_keys, k_begin + (int64_t)p.keys_per_split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int head = wave * 16 + col;
  const float sl2 = p.scale * kLog2e;

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

  uint4 pk[LPT], pv[LPT];
  int pok[LPT];
  auto fetch = [&](int64_t kc0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * NT;
      pk[u] = make_uint4(0, 0, 0, 0);
      pv[u] = make_uint4(0, 0, 0, 0);
      pok[u] = 0;
      if (e < CH * C8) {
        const int key = e / C8, c8 = e - key * C8;
        const int64_t t = kc0 + key;
        const uint16_t *kp, *vp;
        if (t < k_end && key_rows<uint16_t>(p, L, b, i, t, kp, vp)) {
          pk[u] = *reinterpret_cast<const uint4*>(kp + c8 * 8);
          pv[u] = *reinterpret_cast<const uint4*>(vp + c8 * 8);
          pok[u] = 1;
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int e = tid + u * NT;
      if (e < CH * C8) {
        const int key = e / C8, c8 = e - key * C8;
        *reinterpret_cast<uint4*>(&sK[key * KROW + c8 * 8]) = pk[u];
        uint16_t* vt = &sV[(c8 * 8) * VROW + key];
        vt[0 * VROW] = (uint16_t)(pv[u].x & 0xffffu);
        vt[1 * VROW] = (uint16_t)(pv[u].x >> 16);
        vt[2 * VROW] = (uint16_t)(pv[u].y & 0xffffu);
        vt[3 * VROW] = (uint16_t)(pv[u].y >> 16);
        vt[4 * VROW] = (uint16_t)(pv[u].z & 0xffffu);
        vt[5 * VROW] = (uint16_t)(pv[u].z >> 16);
        vt[6 * VROW] = (uint16_t)(pv[u].w & 0xffffu);
        vt[7 * VROW] = (uint16_t)(pv[u].w >> 16);
        if (c8 == 0) sOK[key] = pok[u];
      }
    }
  };

  if (k_begin < k_end) fetch(k_begin);
  for (int64_t kc0 = k_begin; kc0 < k_end; kc0 += CH) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kc0 + CH < k_end) fetch(kc0 + CH);

    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&sK[col * KROW + s * 32 + grp * 8]));
      const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&sK[(16 + col) * KROW + s * 32 + grp * 8]));
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Qb[s], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Qb[s], S1, 0, 0, 0);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = sOK[4 * grp + e] ? S0[e] * sl2 : -INFINITY;
      x[4 + e] = sOK[16 + 4 * grp + e] ? S1[e] * sl2 : -INFINITY;
    }
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float m_new = fmaxf(m_run, cm);
    float alpha = 1.f, pe[8];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = exp2f(x[e] - m_new);
    }
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ps += pe[e];
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = bf2f(f2bf(pe[e]));
      lo[e] = pe[e] - hi[e];
    }
    const bf16x8_t Bhi = __builtin_bit_cast(bf16x8_t, pack8(hi));
    const bf16x8_t Blo = __builtin_bit_cast(bf16x8_t, pack8(lo));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vr = &sV[(dt * 16 + col) * VROW];
      const uint2 a0 = *reinterpret_cast<const uint2*>(vr + 4 * grp);
      const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 16 + 4 * grp);
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bhi, O[dt], 0, 0, 0);
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Blo, O[dt], 0, 0, 0);
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  if (p.splits == 1) {
    float lse;
    const float f = finish_head(m_run, l_run, p.sink, head, &lse);
    float* orow = p.o + (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(orow + dt * 16 + 4 * grp) =
          make_float4(O[dt][0] * f, O[dt][1] * f, O[dt][2] * f, O[dt][3] * f);
    if (grp == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
  } else {
    const int64_t slot = ((int64_t)row * p.splits + split) * p.heads + head;
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
  const int64_t k_begin = (int64_t)split * p.keys_per_split;
  const int64_t k_end = min(L.n_keys, k_begin + (int64_t)p.keys_per_split);
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
    if (p.splits == 1) {
      float lse;
      const float f = finish_head(m_run, l_run, p.sink, head, &lse);
      float* orow = p.o + (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = acc[e] * f;
      if (lane == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
    } else {
      const int64_t slot = ((int64_t)row * p.splits + split) * p.heads + head;
#pragma unroll
      for (int e = 0; e < DPL; ++e) p.part_o[slot * D + lane + 64 * e] = acc[e];
      if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_run);
    }
  }
}

// ------------------------------------------------------------------ merge
// One workgroup per (row, head), one thread per output column; splits are merged
// in index order.
__global__ void merge_kernel(AttnP p) {
  const int row = blockIdx.x, head = blockIdx.y, c = threadIdx.x;
  const int b = row / p.tq, i = row - b * p.tq;
  const int S = p.splits;
  const float* ml = p.part_ml + ((int64_t)row * S * p.heads + head) * 2;
  const float* po = p.part_o + ((int64_t)row * S * p.heads + head) * p.dim + c;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(int64_t)s * p.heads * 2]);
  float l = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = ml[(int64_t)s * p.heads * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      l = fmaf(w, ml[(int64_t)s * p.heads * 2 + 1], l);
      acc = fmaf(w, po[(int64_t)s * p.heads * p.dim], acc);
    }
  }
  float lse;
  const float f = finish_head(M, l, p.sink, head, &lse);
  p.o[(int64_t)b * p.o_bs + (int64_t)i * p.o_rs + (int64_t)head * p.dim + c] = acc * f;
  if (c == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
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
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nrows, (unsigned)p.heads), dim3((unsigned)p.dim), 0, s, p);
  return hipGetLastError();
}

}  // namespace v4a
