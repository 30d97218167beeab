// Device helpers shared by the v4attn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v4a {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte load unit (a native vector, not HIP's uint4 struct, so copies stay in registers)

constexpr int kWave = 64;

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// unpack 8 bf16 held in a uint4 into fp32
__device__ __forceinline__ void unpack8(const uint4 v, float* o) {
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
  o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 r;
  r.x = f2bf(f[0]) | (f2bf(f[1]) << 16);
  r.y = f2bf(f[2]) | (f2bf(f[3]) << 16);
  r.z = f2bf(f[4]) | (f2bf(f[5]) << 16);
  r.w = f2bf(f[6]) | (f2bf(f[7]) << 16);
  return r;
}

// Output stores: o is fp32, or bf16 rounded to nearest even (element offset off)
__device__ __forceinline__ void store_out4(void* o, bool bf16, int64_t off, float a, float b, float c, float d) {
  if (bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(o) + off) =
        make_uint2(f2bf(a) | (f2bf(b) << 16), f2bf(c) | (f2bf(d) << 16));
  else
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(o) + off) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store_out1(void* o, bool bf16, int64_t off, float a) {
  if (bf16) reinterpret_cast<uint16_t*>(o)[off] = (uint16_t)f2bf(a);
  else reinterpret_cast<float*>(o)[off] = a;
}

// ---- order-preserving key of an fp32 score ---------------------------------
// Larger float -> larger unsigned key.  -0 is folded onto +0 so the two compare
// equal, as they do as floats.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---- wave-level scans and reductions on DPP ---------------------------------
// All cross-lane steps below are DPP moves (quad swaps, row shifts, row mirrors,
// row_bcast15/31) plus one readlane: no LDS round trips, and a fixed combination
// order, so every lane of every run sees the same bits.
template <int CTRL, int ROWMASK = 0xF, int BANKMASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROWMASK, BANKMASK, BOUND_ZERO);
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  uint32_t s = v + dpp_u32<0x111, 0xF, 0xF, true>(0, v);   // row_shr:1
  s += dpp_u32<0x112, 0xF, 0xF, true>(0, v);                // row_shr:2
  s += dpp_u32<0x113, 0xF, 0xF, true>(0, v);                // row_shr:3
  s += dpp_u32<0x114, 0xF, 0xE, true>(0, s);                // row_shr:4 into banks 1-3
  s += dpp_u32<0x118, 0xF, 0xC, true>(0, s);                // row_shr:8 into banks 2-3
  s += dpp_u32<0x142, 0xA>(0, s);                           // row_bcast:15 into rows 1, 3
  s += dpp_u32<0x143, 0xC>(0, s);                           // row_bcast:31 into rows 2, 3
  return s;
}

// Reduction with an associative, commutative op whose identity is `id` (rows the
// row_bcast steps leave out contribute `id`); the result is wave-uniform.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op, uint32_t id) {
  v = op(v, dpp_u32<0xB1>(id, v));        // quad_perm [1,0,3,2]
  v = op(v, dpp_u32<0x4E>(id, v));        // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0x141>(id, v));       // row_half_mirror
  v = op(v, dpp_u32<0x140>(id, v));       // row_mirror
  v = op(v, dpp_u32<0x142, 0xA>(id, v));  // row_bcast:15 into rows 1, 3
  v = op(v, dpp_u32<0x143, 0xC>(id, v));  // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u32(
      __float_as_uint(v),
      [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); },
      0xff800000u));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce_u32(
      __float_as_uint(v),
      [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); }, 0u));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; }, 0xffffffffu);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; }, 0u);
}

// Reductions over the four lanes that share lane % 16 (the four 16-lane rows of a
// wave), e.g. the four row groups of one MFMA output column; every lane gets the
// result.  Two row-swap steps (permlane16 and permlane32 swaps), no LDS.
__device__ __forceinline__ float col_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
__device__ __forceinline__ float col_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// A value every lane holds the same copy of, moved to scalar registers so that the
// compiler treats what derives from it as uniform (scalar branches and address
// arithmetic instead of per-lane ones).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One 16-byte-per-lane load from global memory straight into LDS: lane l's bytes
// land at LDS address lds + 16 l (lds wave-uniform).  Written as inline asm so that
// the compiler's wait insertion does not treat every later LDS read as depending
// on it; the code that consumes the data waits for it explicitly (s_waitcnt on
// the vector-memory counter, then a workgroup barrier).  The instruction has no
// register result, and the compiler's own waits can only get stricter for not
// counting it, since vector-memory loads complete in issue order.
// s_waitcnt immediate for vmcnt(n) (gfx9: low 4 bits at [3:0], high 2 at [15:14]),
// every other counter left alone
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

__device__ __forceinline__ void lds_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// The 4-byte form: lane l's word lands at lds + 4 l.
__device__ __forceinline__ void lds_load4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Partial RoPE: cos and sin of the angle pos * 2^(-2i/R * lb) of channel pair i
// (lb = log2 of the base).  The angle is formed in fp64 and reduced there to
// r = a - k pi/2 with |r| <= pi/4 (positions in the millions keep their phase to
// ~1e-10 rad); sin r and cos r are their Taylor series through r^9 and r^10
// (truncation below 2e-9 on that interval) in fp32, and the quadrant k mod 4
// swaps and negates them.  No library sincos: its large-argument path keeps
// per-lane arrays in scratch memory even when the argument is small.
__device__ __forceinline__ void rope_cs(double pos, int i, int R, double lb, float& c, float& s) {
  constexpr double kHalfPi = 1.5707963267948966, kTwoOverPi = 0.6366197723675814;
  const double th = exp2(-2.0 * (double)i / (double)R * lb);
  const double a = pos * th;
  const double k = rint(a * kTwoOverPi);
  const float r = (float)(a - k * kHalfPi);
  const float r2 = r * r;
  const float ps = r * (1.f - r2 * (1.f / 6.f - r2 * (1.f / 120.f - r2 * (1.f / 5040.f - r2 * (1.f / 362880.f)))));
  const float pc = 1.f - r2 * (0.5f - r2 * (1.f / 24.f - r2 * (1.f / 720.f - r2 * (1.f / 40320.f - r2 * (1.f / 3628800.f)))));
  const int q = (int)((long long)k & 3);
  s = q == 0 ? ps : q == 1 ? pc : q == 2 ? -ps : -pc;
  c = q == 0 ? pc : q == 1 ? -ps : q == 2 ? -pc : ps;
}
// (x, y) turned by the angle whose cos and sin are (c, s); by its opposite with neg
__device__ __forceinline__ void rot2(float& x, float& y, float c, float s, bool neg) {
  const float sn = neg ? -s : s;
  const float nx = x * c - y * sn, ny = x * sn + y * c;
  x = nx;
  y = ny;
}
// exp(x) with -inf -> 0
__device__ __forceinline__ float fexp(float x) { return __expf(x); }

}  // namespace v4a
