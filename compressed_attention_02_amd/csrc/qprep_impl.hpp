// Query prep: [QbitAI] "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制,
// the Q/KV normalization and partial RoPE paragraphs.  Each head's query is
// RMS-normalised with the gain, then its last R channels rotated at the row's
// position, in fp32 from the bf16 input and rounded to bf16 once.  A thread holds
// 8 consecutive channels of one head (rotation pairs stay inside it); the D/8
// threads of a head are neighbouring lanes and add their squares by butterfly.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

// 8-channel group g (of heads * D/8) of row `row`; every lane of the wave calls it
template <int D>
__device__ __forceinline__ void qprep_group(const QPrepP& p, int row, int g) {
  constexpr int GS = D / 8;   // threads per head
  const int b = row / p.tq, i = row - b * p.tq;
  const bool ok = g < p.heads * GS;
  const int part = g % GS;
  float x[8];
  if (ok) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bs + (int64_t)i * p.q_rs + g * 8;
    unpack8(*reinterpret_cast<const uint4*>(src), x);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  }
  if (p.gain) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
    for (int m = 1; m < GS; m <<= 1) ss += __shfl_xor(ss, m);
    const float rq = rsqrtf(ss / (float)D + p.eps);
    if (ok) {
      const float4 g0 = *reinterpret_cast<const float4*>(p.gain + part * 8);
      const float4 g1 = *reinterpret_cast<const float4*>(p.gain + part * 8 + 4);
      const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * rq * gs[e];
    }
  }
  if (!ok) return;
  if (p.rope) {
    const int64_t pos = p.pos0[b] + i;
    const int lo = D - p.rope;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int ch = part * 8 + 2 * k2;
      if (ch < lo) continue;
      float cs, sn;
      rope_cs((double)pos, (ch - lo) / 2, p.rope, p.rope_lb, cs, sn);
      rot2(x[2 * k2], x[2 * k2 + 1], cs, sn, false);
    }
  }
  *reinterpret_cast<uint4*>(p.out + (int64_t)row * p.heads * D + g * 8) = pack8(x);
}

// block `blk` (256 threads) of the prep of row `row`, any supported D
__device__ __forceinline__ void qprep_block(const QPrepP& p, int row, int blk) {
  const int g = blk * 256 + (int)threadIdx.x;
  if (p.dim == 64) qprep_group<64>(p, row, g);
  else if (p.dim == 128) qprep_group<128>(p, row, g);
  else qprep_group<512>(p, row, g);
}

}  // namespace v4a
