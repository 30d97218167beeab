// kv_compress: pool every complete block of r raw tokens into one entry.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
// CSA step 1 merges every m tokens' KV entries into one with learned, attention-like
// weights; HCA does the same with m' = 128 and no overlap.  The weights are the
// softmax of one fp32 logit per raw token over its block, shared by K and V.
//
// Pure HBM streaming: each raw K/V row is read once, each output row written once.
// Thread layout: a row of d elements is CH 16-byte chunks; G threads ("row groups")
// share one block's r rows (rows g, g+G, ...), so a ratio-128 block keeps 256
// threads busy and a ratio-4 block 64.  Row groups are combined in LDS.
//
// Optional RMSNorm of the entries ([QbitAI] 混合注意力机制, Q/KV normalization:
// KV entries are normalised before core attention): with a gain g the stored entry
// is g * y / sqrt(mean(y^2) + eps).  Optional partial RoPE (the partial RoPE
// paragraph of the same section): raw rows are rotated at their own positions; the
// entry is pooled and normalised in the unrotated frame and stored rotated at the
// position of its block's last token.  Optional FP8 entries ([wiki] quantization and
// deployment section: FP8 KV caches): one fp32 scale max|y| / 448 per entry and the
// E4M3 codes of y / scale, nearest with ties to even.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* o) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ static void store(float* p, const float* o) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
};
template <> struct Chunk<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* o) { unpack8(*reinterpret_cast<const uint4*>(p), o); }
  __device__ static void store(uint16_t* p, const float* o) { *reinterpret_cast<uint4*>(p) = pack8(o); }
};

// Partial RoPE table of the in-block offsets: (cos, sin) of u * theta_i for u < r
constexpr int kRopeTab = 4096;

// HV: the block has V rows too (else the entries are shared K = V: K alone is pooled)
// The E4M3 code of x, |x| <= 448 (larger magnitudes are taken as 448): the nearest
// finite E4M3 value, ties to the even code.  Below 2^-6 the values are the multiples
// of 2^-9 (codes 0..8, 8 being 2^-6 itself); above, the fp32 mantissa is rounded to 3
// bits (nearest, ties to even: add 2^19 - 1 plus the lowest kept bit, carrying into
// the exponent), and the exponent is rebased from bias 127 to bias 7.
__device__ __forceinline__ uint32_t e4m3_nearest(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t m;
  if (a < 0.015625f) {
    m = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    m = ((bits + 0x7FFFFu + ((bits >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return sign | m;
}

template <typename T, bool ROPE, bool HV, bool F8O>
__global__ __launch_bounds__(256) void compress_kernel(CompressP p) {
  constexpr int N = Chunk<T>::N;
  __shared__ float s_max[256];
  __shared__ float s_acc[256][2 * N + 1];
  __shared__ float2 s_cs[ROPE ? kRopeTab : 1];

  const int tid = threadIdx.x;
  const int per_block = p.ch * p.g;
  const int slot = tid / per_block;
  const int rem = tid - slot * per_block;
  const int g = rem / p.ch;
  const int c = rem - g * p.ch;
  const int b = blockIdx.y;
  const int64_t jb = (int64_t)blockIdx.x * p.bpw + slot;
  const bool active = slot < p.bpw && jb < p.nb;
  const int64_t j = p.t0 / p.r + jb;                       // absolute block id
  const int64_t row0 = j * p.r - p.raw_start[b];           // raw row of its first token

  const float* lg = p.logits + (int64_t)b * p.lg_bs + row0;
  float mx = -INFINITY;
  if (active)
    for (int u = g; u < p.r; u += p.g) mx = fmaxf(mx, lg[u]);
  s_max[tid] = mx;
  const int R = ROPE ? p.rope : 0, hr = R / 2, lo = p.d - R;
  if (R)
    for (int t = tid; t < p.r * hr; t += 256) {
      float cs, sn;
      rope_cs((double)(t / hr), t % hr, R, p.rope_lb, cs, sn);
      s_cs[t] = make_float2(cs, sn);
    }
  __syncthreads();
  if (active)
    for (int gg = 0; gg < p.g; ++gg) mx = fmaxf(mx, s_max[slot * per_block + gg * p.ch + c]);

  float ak[N], av[N], ws = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) { ak[e] = 0.f; av[e] = 0.f; }
  if (active) {
    const T* kr = reinterpret_cast<const T*>(p.k_raw) + (int64_t)b * p.kr_bs + row0 * p.kr_rs + c * N;
    const T* vr = reinterpret_cast<const T*>(p.v_raw) + (int64_t)b * p.vr_bs + row0 * p.vr_rs + c * N;
#pragma unroll 4
    for (int u = g; u < p.r; u += p.g) {
      const float w = __expf(lg[u] - mx);
      float xk[N], xv[N];
      Chunk<T>::load(kr + (int64_t)u * p.kr_rs, xk);
      if (HV) Chunk<T>::load(vr + (int64_t)u * p.vr_rs, xv);
      if (R) {
        // raw rows are rotated at their positions j*r + u: undo the in-block part u
        // here, the block part j*r once on the pooled entry
#pragma unroll
        for (int k2 = 0; k2 < N / 2; ++k2) {
          const int e0 = c * N + 2 * k2;
          if (e0 < lo) continue;
          const float2 cs = s_cs[u * hr + (e0 - lo) / 2];
          rot2(xk[2 * k2], xk[2 * k2 + 1], cs.x, cs.y, true);
          if (HV && p.rope_v) rot2(xv[2 * k2], xv[2 * k2 + 1], cs.x, cs.y, true);
        }
      }
      ws += w;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        ak[e] = fmaf(w, xk[e], ak[e]);
        if (HV) av[e] = fmaf(w, xv[e], av[e]);
      }
    }
  }
  if (p.g > 1) {
#pragma unroll
    for (int e = 0; e < N; ++e) { s_acc[tid][e] = ak[e]; s_acc[tid][N + e] = av[e]; }
    s_acc[tid][2 * N] = ws;
    __syncthreads();
    if (active && g == 0) {
      for (int gg = 1; gg < p.g; ++gg) {
        const float* o = s_acc[slot * per_block + gg * p.ch + c];
#pragma unroll
        for (int e = 0; e < N; ++e) { ak[e] += o[e]; av[e] += o[N + e]; }
        ws += o[2 * N];
      }
    }
  }
  float kss = 0.f, vss = 0.f;
  if (active && g == 0) {
    const float inv = 1.0f / ws;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      ak[e] *= inv;
      av[e] *= inv;
    }
    if (R) {  // into the unrotated frame: undo the block's base rotation j*r
#pragma unroll
      for (int k2 = 0; k2 < N / 2; ++k2) {
        const int e0 = c * N + 2 * k2;
        if (e0 < lo) continue;
        float cs, sn;
        rope_cs((double)(j * p.r), (e0 - lo) / 2, R, p.rope_lb, cs, sn);
        rot2(ak[2 * k2], ak[2 * k2 + 1], cs, sn, true);
        if (HV && p.rope_v) rot2(av[2 * k2], av[2 * k2 + 1], cs, sn, true);
      }
    }
#pragma unroll
    for (int e = 0; e < N; ++e) {
      kss = fmaf(ak[e], ak[e], kss);
      vss = fmaf(av[e], av[e], vss);
    }
  }
  if (p.gk || p.gv) {
    // RMSNorm of the entry: the row's ch chunk threads add their squares in LDS,
    // in chunk order
    __syncthreads();
    s_acc[tid][0] = kss;
    s_acc[tid][1] = vss;
    __syncthreads();
    if (active && g == 0) {
      float sk = 0.f, sv = 0.f;
      for (int cc = 0; cc < p.ch; ++cc) {
        sk += s_acc[slot * per_block + cc][0];
        sv += s_acc[slot * per_block + cc][1];
      }
      const float rk = rsqrtf(sk / (float)p.d + p.eps), rv = rsqrtf(sv / (float)p.d + p.eps);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        if (p.gk) ak[e] = ak[e] * rk * p.gk[c * N + e];
        if (HV && p.gv) av[e] = av[e] * rv * p.gv[c * N + e];
      }
    }
  }
  if (active && g == 0 && R) {  // the entry's own rotation, at its block's last position
#pragma unroll
    for (int k2 = 0; k2 < N / 2; ++k2) {
      const int e0 = c * N + 2 * k2;
      if (e0 < lo) continue;
      float cs, sn;
      rope_cs((double)((j + 1) * p.r - 1), (e0 - lo) / 2, R, p.rope_lb, cs, sn);
      rot2(ak[2 * k2], ak[2 * k2 + 1], cs, sn, false);
      if (HV && p.rope_v) rot2(av[2 * k2], av[2 * k2 + 1], cs, sn, false);
    }
  }
  if constexpr (F8O) {
    // FP8 entries: the row's scale s = max |y| / 448 (its ch chunk threads meet in
    // LDS, in chunk order), then the codes of y / s and, from chunk thread 0, s
    float mk = 0.f, mv = 0.f;
    if (active && g == 0) {
#pragma unroll
      for (int e = 0; e < N; ++e) {
        mk = fmaxf(mk, fabsf(ak[e]));
        if (HV) mv = fmaxf(mv, fabsf(av[e]));
      }
    }
    __syncthreads();   // the combine or the norm above may still read s_acc
    s_acc[tid][0] = mk;
    s_acc[tid][1] = mv;
    __syncthreads();
    if (active && g == 0) {
      for (int cc = 0; cc < p.ch; ++cc) {
        mk = fmaxf(mk, s_acc[slot * per_block + cc][0]);
        mv = fmaxf(mv, s_acc[slot * per_block + cc][1]);
      }
      const float sk = mk / 448.f, sv = mv / 448.f;
      uint32_t wk[N / 4], wv[N / 4];
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        wk[q] = 0u;
        wv[q] = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[q] |= e4m3_nearest(sk > 0.f ? ak[4 * q + e] / sk : 0.f) << (8 * e);
          if (HV) wv[q] |= e4m3_nearest(sv > 0.f ? av[4 * q + e] / sv : 0.f) << (8 * e);
        }
      }
      unsigned char* ko = reinterpret_cast<unsigned char*>(p.k_out) + (int64_t)b * p.ko_bs + j * p.ko_rs + c * N;
      unsigned char* vo = reinterpret_cast<unsigned char*>(p.v_out) + (int64_t)b * p.vo_bs + j * p.vo_rs + c * N;
      if constexpr (N == 8) {
        *reinterpret_cast<uint2*>(ko) = make_uint2(wk[0], wk[1]);
        if (HV) *reinterpret_cast<uint2*>(vo) = make_uint2(wv[0], wv[1]);
      } else {
        *reinterpret_cast<uint32_t*>(ko) = wk[0];
        if (HV) *reinterpret_cast<uint32_t*>(vo) = wv[0];
      }
      if (c == 0) {
        p.ks_out[(int64_t)b * p.kso_bs + j] = sk;
        if (HV) p.vs_out[(int64_t)b * p.vso_bs + j] = sv;
      }
    }
  } else if (active && g == 0) {
    T* ko = reinterpret_cast<T*>(p.k_out) + (int64_t)b * p.ko_bs + j * p.ko_rs + c * N;
    T* vo = reinterpret_cast<T*>(p.v_out) + (int64_t)b * p.vo_bs + j * p.vo_rs + c * N;
    Chunk<T>::store(ko, ak);
    if (HV) Chunk<T>::store(vo, av);
  }
}

template <typename T, bool HV, bool F8O>
static void launch_variant(const CompressP& p, dim3 grid, hipStream_t s, int tid) {
  if (p.rope) V4A_LAUNCH(tid, (compress_kernel<T, true, HV, F8O>), grid, dim3(256), 0, s, p);
  else V4A_LAUNCH(tid, (compress_kernel<T, false, HV, F8O>), grid, dim3(256), 0, s, p);
}

template <typename T, bool HV>
static void launch_out(const CompressP& p, dim3 grid, hipStream_t s, int tid) {
  if (p.f8out) launch_variant<T, HV, true>(p, grid, s, tid);
  else launch_variant<T, HV, false>(p, grid, s, tid);
}

hipError_t launch_compress(int dtype, const CompressP& p, int batch, hipStream_t s, int tid) {
  const dim3 grid((unsigned)((p.nb + p.bpw - 1) / p.bpw), (unsigned)batch);
  const bool hv = p.v_raw != nullptr;
  if (dtype == 0) {
    if (hv) launch_out<float, true>(p, grid, s, tid);
    else launch_out<float, false>(p, grid, s, tid);
  } else {
    if (hv) launch_out<uint16_t, true>(p, grid, s, tid);
    else launch_out<uint16_t, false>(p, grid, s, tid);
  }
  return hipGetLastError();
}

}  // namespace v4a
