// Device code of the bf16 decode/prefill attention, shared by the attention kernel
// and the combined selection + attention kernel of the decode step.  The design
// notes are at the top of attn.hip.
#pragma once
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

// Output channel ch of a query at pos, turned back by -pos when it lies in the
// rotated part: its pair partner is the neighbouring lane (ch ^ 1 sits in lane ^ 1),
// so every lane of the wave must call this together.
__device__ __forceinline__ float rope_back_pair(const AttnP& p, float a, int ch, int64_t pos) {
  const float other = __shfl_xor(a, 1);
  const int lo = p.dim - p.rope;
  if (ch < lo) return a;
  float cs, sn;
  rope_cs((double)pos, (ch - lo) / 2, p.rope, p.rope_lb, cs, sn);
  // x' = x c + y s, y' = -x s + y c (the rotation by -angle)
  return (ch & 1) ? fmaf(-other, sn, a * cs) : fmaf(other, sn, a * cs);
}

// ------------------------------------------------------------------ merge
// Combination of the split partials of one (row, head) (U_s, m_s, l_s), m in base 2: weights exp2(m_s - max m), o = sum w_s U_s
// / sum w_s l_s, for output columns [d0, d0 + DW).  NT threads; the statistics are
// spread over the threads (kMaxSplits / NT each), the weighted sum over NT/DW thread
// groups, each summing its splits in ascending order, and the groups are combined
// in LDS in a fixed order, so the result does not depend on timing.  s_w holds
// kMaxSplits floats, s_red NT.
constexpr int kMaxSplits = 1024;
constexpr int kMergeBatch = 16;

template <int NT, int DW>
__device__ __forceinline__ void merge_head(const AttnP& p, int row, int head, int d0, float* s_w, float* s_red) {
  constexpr int G = NT / DW, NWV = NT / 64, KST = kMaxSplits / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row / p.tq, i = row - b * p.tq;
  const int S = p.splits_total, D = p.dim;
  const float* ml = p.part_ml + ((int64_t)row * p.heads + head) * S * 2;
  const int c = tid % DW, g = tid / DW;
  const float* po = p.part_o + ((int64_t)row * p.heads + head) * S * D + d0 + c;
  // this thread's first kMergeBatch partial values load together with the statistics
  float v[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) v[u] = po[(int64_t)min(g + u * G, S - 1) * D];
  float ms[KST], ls[KST];
#pragma unroll
  for (int u = 0; u < KST; ++u) {
    const int t = tid + u * NT;
    const float2 m2 = *reinterpret_cast<const float2*>(ml + (int64_t)min(t, S - 1) * 2);
    ms[u] = t < S ? m2.x : -INFINITY;
    ls[u] = t < S ? m2.y : 0.f;
  }
  // 1) global max of the split maxima
  float mx = ms[0];
#pragma unroll
  for (int u = 1; u < KST; ++u) mx = fmaxf(mx, ms[u]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();
  // 2) split weights and the total sum (per thread in u order, then waves in order)
  float part = 0.f;
#pragma unroll
  for (int u = 0; u < KST; ++u) {
    const int t = tid + u * NT;
    const float wgt = (M == -INFINITY || ms[u] == -INFINITY) ? 0.f : exp2f(ms[u] - M);
    if (t < S) s_w[t] = wgt;
    part += wgt * ls[u];
  }
  part = wave_sum(part);
  if (lane == 0) s_red[wave] = part;
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) l += s_red[w];
  __syncthreads();
  // 3) weighted sum of the partial outputs
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)
    if (g + u * G < S) acc = fmaf(s_w[g + u * G], v[u], acc);
  for (int s0 = g + G * kMergeBatch; s0 < S; s0 += G * kMergeBatch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = po[(int64_t)min(s0 + u * G, S - 1) * D];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (s0 + u * G < S) acc = fmaf(s_w[s0 + u * G], v[u], acc);
  }
  s_red[tid] = acc;
  __syncthreads();
  if (g == 0) {
    float a = s_red[c];
    for (int gg = 1; gg < G; ++gg) a += s_red[gg * DW + c];
    float lse;
    const float f = finish_head(M, l, p.sink, head, &lse);
    a *= f;
    if (p.rope_out) a = rope_back_pair(p, a, d0 + c, p.pos0[b] + i);
    store_out1(p.o, p.o_bf16, (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + (int64_t)head * D + d0 + c, a);
    if (c == 0 && d0 == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
  }
}

// ------------------------------------------------------------------ bf16 MFMA
// Where the keys of one row come from.  Virtual key t < n_csa is CSA pick t (its
// id read from the split's copy of the idx row in LDS), t < hca_end is HCA entry
// t - n_csa, anything later is raw row t + raw_off.  Keys the row does not have
// (past the split's end, padded CSA slots) read the row's query instead, which is
// always valid memory, and are masked out, so every load is unconditional and no
// load waits on another.
struct RowKeys {
  const uint16_t *kc, *vc, *kh, *vh, *kr, *vr, *fallback;  // the row's sequence
  int64_t kc_rs, vc_rs, kh_rs, vh_rs, kr_rs, vr_rs;        // row strides (elements)
  int64_t n_csa, hca_end, raw_off, k_begin, k_end;
  // FP8 caches: the row's scales (one per cache row); the code tables are the
  // pointers above taken as bytes
  const float *kcs, *vcs, *khs, *vhs, *krs, *vrs;
};


constexpr float kLazyRescale = 8.f; // running max moves only when exceeded by 2^8
constexpr int kWideGroup = 4;        // fragment steps per scheduling group of rows wider than 128

// Source rows of key t in the general case (a chunk that straddles branches or
// the end of the split): selects only.
__device__ __forceinline__ void key_src_any(const RowKeys& R, const int* s_idx, int64_t t, const uint16_t*& kp,
                                            const uint16_t*& vp, bool& ok) {
  const bool in = t < R.k_end;
  const bool csa = t < R.n_csa, hca = t < R.hca_end;
  const int64_t j = t - R.k_begin;
  const int id = s_idx[j < 0 ? 0 : (j >= kMaxTopk ? kMaxTopk - 1 : j)];
  ok = in && (!csa || id >= 0);
  const int64_t rc = id, rh = t - R.n_csa, rr = t + R.raw_off;
  const int64_t r = ok ? (csa ? rc : (hca ? rh : rr)) : 0;
  const int64_t kcs = R.kc_rs, khs = R.kh_rs, krs = R.kr_rs, vcs = R.vc_rs, vhs = R.vh_rs, vrs = R.vr_rs;
  const int64_t ks = csa ? kcs : (hca ? khs : krs);
  const int64_t vs = csa ? vcs : (hca ? vhs : vrs);
  const uint16_t *kc = R.kc, *kh = R.kh, *kr = R.kr, *vc = R.vc, *vh = R.vh, *vr = R.vr, *fb = R.fallback;
  const uint16_t* kb = ok ? (csa ? kc : (hca ? kh : kr)) : fb;
  const uint16_t* vb = ok ? (csa ? vc : (hca ? vh : vr)) : fb;
  kp = kb + r * ks;
  vp = vb + r * vs;
}

// LDS layout of a chunk: K and V rows of D bf16 each, unpadded, with the 16-byte
// pieces of row r permuted by XOR with swz_k(r) / swz_v(r).  The permutations make
// the three access patterns free of bank conflicts: the direct global->LDS loads
// (a wave writes 1 KB contiguously), the K fragment reads (16 rows, one piece
// column) and the transposing V reads (4 rows x 2 pieces per 16 lanes).  At
// D = 512 the entries are shared (one buffer is read both ways), so one XOR serves
// both: 2(r mod 8) + bit 3 of r is distinct over 16 rows (K reads) and keeps piece
// pairs together with distinct pair slots over each 8 rows (V reads).
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D == 512 ? (2 * (r & 7) | ((r >> 3) & 1)) : D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D == 512 ? swz_k<512>(r) : D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// Rows wider than 128 are kept as D / 128 stacked sub-buffers of 128 columns
// (column group g of row r at (g * kAttnChunk + r) * 128), so that every sub-row is
// 256 bytes like a d = 128 row: a load instruction then moves 4 rows of one group
// (per-lane row addresses) and the XOR permutes 16 pieces.
template <int D> constexpr int sub_cols() { return D > 128 ? 128 : D; }
// element offset of 16-byte piece p of chunk row r in that layout
template <int D> __device__ __forceinline__ int chunk_off(int r, int p, int x) {
  constexpr int PS = sub_cols<D>() / 8;
  return ((p / PS) * kAttnChunk + r) * sub_cols<D>() + ((p % PS) ^ x) * 8;
}


// row r of a table at base with row stride rs (elements): 32 x 32 -> 64-bit product
__device__ __forceinline__ const uint16_t* row_ptr(const uint16_t* base, uint32_t r, int64_t rs) {
  return base + (uint64_t)r * (uint32_t)rs;
}

// Issues the loads of the chunk at virtual key kc0 straight into LDS (sK, sV) and
// writes its mask (sBias[key] = 0 or -inf).  Each wave moves 64 lanes x 16 bytes
// per instruction: RPI rows of one column group; lane l's piece lands at LDS base
// + 16 l, so the lane loads the global piece that the XOR layout puts there.  A
// lane's row address serves all column groups.  wave is uniform.
template <int NW, int D, bool SKV>
__device__ __forceinline__ void issue_chunk(const RowKeys& R, const int* s_idx, int64_t kc0, uint16_t* sK,
                                            uint16_t* sV, float* sBias, int wave, int lane) {
  constexpr int SUB = sub_cols<D>(), NG = D / SUB;
  constexpr int PS = SUB / 8;                     // 16-byte pieces per sub-row
  constexpr int RPI = 64 / PS;                    // rows per wave instruction
  constexpr int RBW = kAttnChunk / RPI / NW;      // row blocks per wave (NG instructions each)
  static_assert(RBW * RPI * NW == kAttnChunk, "rows must divide over the waves");
  const int prow = lane / PS, ppiece = lane % PS;
  // chunks wholly inside one branch (the common case) take a plain address
  const bool whole = kc0 + kAttnChunk <= R.k_end;
  const bool all_h = whole && kc0 >= R.n_csa && kc0 + kAttnChunk <= R.hca_end;
  const bool all_r = whole && kc0 >= R.hca_end;
  const bool all_c = whole && kc0 + kAttnChunk <= R.n_csa;
  const uint16_t *kb = R.kh, *vb = R.vh;
  int64_t ks = R.kh_rs, vs = R.vh_rs;
  if (all_r) { kb = R.kr + (kc0 + R.raw_off) * R.kr_rs; vb = R.vr + (kc0 + R.raw_off) * R.vr_rs; ks = R.kr_rs; vs = R.vr_rs; }
  else if (all_h) { kb = R.kh + (kc0 - R.n_csa) * R.kh_rs; vb = R.vh + (kc0 - R.n_csa) * R.vh_rs; }
#pragma unroll
  for (int u = 0; u < RBW; ++u) {
    const int r0 = (wave * RBW + u) * RPI;    // first row of this block (uniform)
    const int r = r0 + prow;
    const uint16_t *kp, *vp;
    bool ok = true;
    if (all_h || all_r) {
      kp = row_ptr(kb, r, ks);
      vp = row_ptr(vb, r, vs);
    } else if (all_c) {
      const int id = s_idx[kc0 - R.k_begin + r];
      ok = id >= 0;
      kp = row_ptr(ok ? R.kc : R.fallback, ok ? id : 0, R.kc_rs);
      vp = row_ptr(ok ? R.vc : R.fallback, ok ? id : 0, R.vc_rs);
    } else {
      key_src_any(R, s_idx, kc0 + r, kp, vp, ok);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      lds_load16(kp + (g * PS + (ppiece ^ swz_k<D>(r))) * 8, lds_addr(sK + (g * kAttnChunk + r0) * SUB));
      if constexpr (!SKV)
        lds_load16(vp + (g * PS + (ppiece ^ swz_v<D>(r))) * 8, lds_addr(sV + (g * kAttnChunk + r0) * SUB));
    }
    if (ppiece == 0) sBias[r] = ok ? 0.f : -INFINITY;
  }
}

// FP8 caches: where virtual key t's codes (bytes) and scales live; !ok keys read
// the row's query bytes and a fallback scale word, always valid memory.
__device__ __forceinline__ void key_src_f8(const RowKeys& R, const int* s_idx, int64_t t, bool want_v,
                                           const unsigned char*& code, const float*& scale, bool& ok) {
  const bool in = t < R.k_end;
  const bool csa = t < R.n_csa, hca = t < R.hca_end;
  const int64_t j = t - R.k_begin;
  const int id = csa ? s_idx[j < 0 ? 0 : (j >= kMaxTopk ? kMaxTopk - 1 : j)] : 0;
  ok = in && (!csa || id >= 0);
  const int64_t r = ok ? (csa ? (int64_t)id : (hca ? t - R.n_csa : t + R.raw_off)) : 0;
  const uint16_t* base = want_v ? (csa ? R.vc : (hca ? R.vh : R.vr)) : (csa ? R.kc : (hca ? R.kh : R.kr));
  const int64_t rs = want_v ? (csa ? R.vc_rs : (hca ? R.vh_rs : R.vr_rs)) : (csa ? R.kc_rs : (hca ? R.kh_rs : R.kr_rs));
  const float* sb = want_v ? (csa ? R.vcs : (hca ? R.vhs : R.vrs)) : (csa ? R.kcs : (hca ? R.khs : R.krs));
  code = ok ? reinterpret_cast<const unsigned char*>(base) + r * rs : reinterpret_cast<const unsigned char*>(R.fallback);
  scale = ok ? sb + r : reinterpret_cast<const float*>(R.fallback);
}

// Issues the loads of the FP8 chunk at virtual key kc0 into the staging buffers
// (codes row-major, D bytes per row: lane l's 16 codes land at base + 16 l), the
// rows' K and V scales (waves 0 and 1, lane l = row l, 4 bytes each) and writes the
// mask.  Everything lands in LDS by direct loads; the caller waits for vmcnt(0).
template <int NW, int D>
__device__ __forceinline__ void issue_chunk_f8(const RowKeys& R, const int* s_idx, int64_t kc0, unsigned char* sKc,
                                               unsigned char* sVc, float* sBias, float* sKs, float* sVs, int wave,
                                               int lane) {
  constexpr int PS = D / 16;              // 16-code pieces per row
  constexpr int RPI = 64 / PS;            // rows per wave instruction
  constexpr int NI = kAttnChunk / RPI;    // instructions per chunk, for K and for V
  const int prow = lane / PS, ppiece = lane % PS;
  for (int u = wave; u < NI; u += NW) {
    const int r = u * RPI + prow;
    const unsigned char *kp, *vp;
    const float *ks, *vs;
    bool ok;
    key_src_f8(R, s_idx, kc0 + r, false, kp, ks, ok);
    key_src_f8(R, s_idx, kc0 + r, true, vp, vs, ok);
    lds_load16(kp + ppiece * 16, lds_addr(sKc + u * RPI * D));
    lds_load16(vp + ppiece * 16, lds_addr(sVc + u * RPI * D));
    if (ppiece == 0) sBias[r] = ok ? 0.f : -INFINITY;
  }
  if (wave < 2) {
    const unsigned char* cp;
    const float* sp;
    bool ok;
    key_src_f8(R, s_idx, kc0 + lane, wave == 1, cp, sp, ok);
    lds_load4(sp, lds_addr(wave == 0 ? sKs : sVs));
  }
}

// FP8 shared entries (every row its own value, one scale per row serving as the
// key's and the value's): the chunk's codes into staging (row-major, D bytes per
// row), the rows' scales into sKs (wave 0, lane l = row l) and the mask.
template <int NW, int D>
__device__ __forceinline__ void issue_chunk_f8_shared(const RowKeys& R, const int* s_idx, int64_t kc0,
                                                      unsigned char* sKc, float* sBias, float* sKs, int wave,
                                                      int lane) {
  constexpr int PS = D / 16;              // 16-code pieces per row
  constexpr int RPI = 64 / PS;            // rows per wave instruction
  constexpr int NI = kAttnChunk / RPI;    // instructions per chunk
  const int prow = lane / PS, ppiece = lane % PS;
  for (int u = wave; u < NI; u += NW) {
    const int r = u * RPI + prow;
    const unsigned char* kp;
    const float* ks;
    bool ok;
    key_src_f8(R, s_idx, kc0 + r, false, kp, ks, ok);
    lds_load16(kp + ppiece * 16, lds_addr(sKc + u * RPI * D));
    if (ppiece == 0) sBias[r] = ok ? 0.f : -INFINITY;
  }
  if (wave == 0) {
    const unsigned char* cp;
    const float* sp;
    bool ok;
    key_src_f8(R, s_idx, kc0 + lane, false, cp, sp, ok);
    lds_load4(sp, lds_addr(sKs));
  }
}

// Staged FP8 codes -> the bf16 chunk layout (K with swz_k, V with swz_v), exactly:
// thread item x takes 16 codes of one row (one staging piece) and writes two bf16
// pieces.  Masked rows (sBias -inf) become zeros: their staged bytes are the query
// row's, which may hold NaN codes, and a NaN times a zero weight would still reach
// the sums.
template <int NT, int D, bool KONLY = false>
__device__ __forceinline__ void convert_chunk_f8(const unsigned char* sKc, const unsigned char* sVc, uint16_t* sK,
                                                 uint16_t* sV, const float* sBias) {
  constexpr int PS = D / 16;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  for (int x = threadIdx.x; x < (KONLY ? 1 : 2) * kAttnChunk * PS; x += NT) {
    const bool v = !KONLY && x >= kAttnChunk * PS;
    const int y = v ? x - kAttnChunk * PS : x;
    const int r = y / PS, pc = y % PS;
    uint4 c = *reinterpret_cast<const uint4*>((v ? sVc : sKc) + r * D + pc * 16);
    if (sBias[r] != 0.f) c = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[k], 1.0f, false));
      w[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[k], 1.0f, true));
    }
    uint16_t* dst = v ? sV : sK;
    const int x0 = v ? swz_v<D>(r) : swz_k<D>(r);
    *reinterpret_cast<uint4*>(dst + chunk_off<D>(r, 2 * pc, x0)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + chunk_off<D>(r, 2 * pc + 1, x0)) = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// S^T = K Q^T, online softmax and O^T += V^T P^T for one chunk of kAttnChunk keys
// in LDS, for HT tiles of 16 heads.
//   * S^T: keys on M, heads on N; lane (col, grp) ends up with head col and keys
//     16*kt + 4*grp + e of the chunk; each K fragment feeds all HT tiles.
//   * P^T operand of 32 keys holds keys {4grp+e, 16+4grp+e}; the matching V^T
//     fragment comes from two transposing LDS reads (ds_read_b64_tr_b16), each of
//     which hands lane j of a 16-lane group V[key0+e][d0+j], e = 0..3, when lane s
//     of the group points at V[key0 + s/4][d0 + 4*(s%4)].
//   * P is split into bf16 hi + lo parts (hardware round-to-nearest conversion),
//     so P keeps ~16 significant bits.
//   * The running max m only moves when a chunk max exceeds it by more than
//     kLazyRescale (base 2); until then exp2(x - m) <= 2^8 and O, l need no
//     rescaling.  (m, l, O) stay consistent, which is all that finishing and
//     merging need.
// With F8, sKs / sVs hold the chunk's key and value scales: a key's scale joins its
// logit, a value's its weight in the product (not the denominator l).
template <int D, int HT, int KP, bool F8 = false>
__device__ __forceinline__ void attend_chunk(const uint16_t* sK, const uint16_t* sV, const float* sBias,
                                             const bf16x8_t (&Qb)[HT][D / 32], f32x4 (&O)[HT][D / 16],
                                             float (&m_run)[HT], float (&l_run)[HT], float sl2, int col, int grp,
                                             int kh, const float* sKs = nullptr, const float* sVs = nullptr) {
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int NKT = 4 / KP;     // tiles of 16 keys of this wave: its part kh of the chunk
  f32x4 S[HT][NKT];
  // K fragment: row 16kt + col, piece 4s + grp; the row's XOR does not depend on kt
  const int kr0 = col + 16 * NKT * kh;
  const int kx = swz_k<D>(col);
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int t = 0; t < HT; ++t) S[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  static_assert(D <= 128, "rows wider than 128 take attend_wide_*");
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(sK + chunk_off<D>(kr0 + 16 * kt, 4 * s + grp, kx));
#pragma unroll
      for (int t = 0; t < HT; ++t) S[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qb[t][s], S[t][kt], 0, 0, 0);
    }
  // logits in base 2 (masked keys -inf), in place
  float cm[HT];
  bool need = false;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const f32x4 bias = *reinterpret_cast<const f32x4*>(&sBias[16 * (NKT * kh + kt) + 4 * grp]);
    f32x4 ksl = {sl2, sl2, sl2, sl2};
    if constexpr (F8) {   // masked keys' scale words are whatever the fallback holds: zero them
      ksl = *reinterpret_cast<const f32x4*>(&sKs[16 * (NKT * kh + kt) + 4 * grp]) * sl2;
#pragma unroll
      for (int e = 0; e < 4; ++e) ksl[e] = bias[e] == 0.f ? ksl[e] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[t][kt][e] = fmaf(S[t][kt][e], ksl[e], bias[e]);
  }
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    float c = fmaxf(fmaxf(S[t][0][0], S[t][0][1]), fmaxf(S[t][0][2], S[t][0][3]));
#pragma unroll
    for (int kt = 1; kt < NKT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) c = fmaxf(c, S[t][kt][e]);
    cm[t] = col_max4(c);
    need = need || (cm[t] > m_run[t] + kLazyRescale);
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      const bool up = cm[t] > m_run[t] + kLazyRescale;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run[t] - cm[t]) : 1.f;
      m_run[t] = up ? cm[t] : m_run[t];
      l_run[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[t][dt] *= alpha;
    }
  }
  float mu[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) mu[t] = m_run[t] == -INFINITY ? 0.f : m_run[t];

  typedef short v4i16 __attribute__((ext_vector_type(4)));
  // V^T fragment: rows 32kk + 4grp + col/4 (+16), piece 2dt + (col%4)/2, half col%2;
  // the rows' XOR does not depend on kk
  const int vr = 4 * grp + (col >> 2);
  const int vx = swz_v<D>(vr);
  const uint16_t* vb = sV + (col & 1) * 4;
#pragma unroll
  for (int k2 = 0; k2 < 2 / KP; ++k2) {
    const int kk = (2 / KP) * kh + k2;   // 32-key half of the chunk
    // P^T of keys 32kk + {4grp+e, 16+4grp+e} (tiles 2kk, 2kk+1) as bf16 hi + lo
    float vsc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vsc[e] = F8 ? sVs[32 * kk + 16 * (e >> 2) + 4 * grp + (e & 3)] : 1.f;
    bf16x8_t Bhi[HT], Blo[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = __builtin_amdgcn_exp2f(S[t][2 * k2 + (e >> 2)][e & 3] - mu[t]);
        ps += v;
        const float pv = F8 ? (v > 0.f ? v * vsc[e] : 0.f) : v;   // (masked keys: v = 0)
        const __bf16 h = (__bf16)pv;
        Bhi[t][e] = h;
        Blo[t][e] = (__bf16)(pv - (float)h);
      }
      l_run[t] += ps;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* v0 = vb + chunk_off<D>(vr + 32 * kk, 2 * dt + ((col & 3) >> 1), vx);
      const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(v0));
      const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(v0 + 16 * sub_cols<D>()));
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        O[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bhi[t], O[t][dt], 0, 0, 0);
        O[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Blo[t], O[t][dt], 0, 0, 0);
      }
    }
  }
}

// The chunk pipeline of one split, double-buffered in LDS: the loads of chunk c + 1
// are in flight while chunk c is computed.  The waits count the direct loads (2 *
// IPW per lane per chunk) that may stay outstanding; everything issued before the
// first chunk (q, ids) is older and therefore settled by the first wait.
template <int NW, int D, int HT, int KP, bool SKV>
__device__ __forceinline__ void run_chunks(const RowKeys& R, const int* s_idx, uint16_t* K0, uint16_t* V0, float* B0,
                                           uint16_t* K1, uint16_t* V1, float* B1, int64_t nch, bool active,
                                           const bf16x8_t (&Qb)[HT][D / 32], f32x4 (&O)[HT][D / 16],
                                           float (&m_run)[HT], float (&l_run)[HT], float sl2, int wave, int lane,
                                           int kh) {
  constexpr int CH = kAttnChunk;
  constexpr int IPW = CH * (D / 8) / 64 / NW;     // direct loads per wave per chunk, for K and for V
  constexpr int LPW = SKV ? IPW : 2 * IPW;        // all of a chunk's loads per wave
  const int col = lane & 15, grp = lane >> 4;
  if (nch > 0) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin, K0, V0, B0, wave, lane);
  if (nch > 1) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin + CH, K1, V1, B1, wave, lane);
  // chunk c is computed while chunk c + 1 (if any) loads; the wait before chunk c
  // leaves only chunk c + 1's loads outstanding, so the last chunk waits for all.
  // One body for both buffers (the buffer is a uniform base): the per-lane LDS
  // offsets are kept once, not once per buffer.
  for (int64_t c = 0; c < nch; ++c) {
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    const bool odd = (c & 1) != 0;
    uint16_t* Kc = odd ? K1 : K0;
    uint16_t* Vc = odd ? V1 : V0;
    float* Bc = odd ? B1 : B0;
    if (active) attend_chunk<D, HT, KP>(Kc, Vc, Bc, Qb, O, m_run, l_run, sl2, col, grp, kh);
    __syncthreads();
    if (c + 2 < nch) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin + (c + 2) * CH, Kc, Vc, Bc, wave, lane);
  }
}

// Loads that issue_chunk_f8 (shared: issue_chunk_f8_shared) gives wave `wave` for
// one chunk: its code pieces (K and V, or K alone) and its scale word.
template <int NW, int D, bool SHARED>
__device__ __forceinline__ int f8_chunk_loads(int wave) {
  constexpr int PS = D / 16, RPI = 64 / PS, NI = kAttnChunk / RPI;
  const int nu = wave < NI ? (NI - 1 - wave) / NW + 1 : 0;
  return SHARED ? nu + (wave == 0 ? 1 : 0) : 2 * nu + (wave < 2 ? 1 : 0);
}
// Waits until at most n (wave-uniform) of the wave's vector memory operations are
// outstanding; n above 7 waits for 7.
__device__ __forceinline__ void wait_vm_at_most(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
  }
}

// The chunk pipeline of FP8 caches: two staging halves of codes and one bf16 chunk
// buffer.  Chunks 0 and 1 are issued together; chunk c lands in staging half c & 1,
// is converted into the bf16 layout and computed while chunk c + 1 is in flight, and
// chunk c + 2 is issued into its half once it is done (the mask and scale arrays
// alternate by chunk parity as well).
template <int NW, int D, int HT, int KP>
__device__ __forceinline__ void run_chunks_f8(const RowKeys& R, const int* s_idx, uint16_t* sK, uint16_t* sV,
                                              unsigned char* sKc, unsigned char* sVc, float* B0, float* B1,
                                              float* sS, int64_t nch, bool active, const bf16x8_t (&Qb)[HT][D / 32],
                                              f32x4 (&O)[HT][D / 16], float (&m_run)[HT], float (&l_run)[HT],
                                              float sl2, int wave, int lane, int kh) {
  constexpr int CH = kAttnChunk, SB = kAttnChunk * D;   // staging bytes per chunk (K codes; V codes)
  const int col = lane & 15, grp = lane >> 4;
  const int nl = f8_chunk_loads<NW, D, false>(wave);
  // sS: [parity][K, V][64] scales
  auto issue = [&](int64_t c) {
    const int par = __builtin_amdgcn_readfirstlane((int)(c & 1));   // (the staging address must be scalar)
    issue_chunk_f8<NW, D>(R, s_idx, R.k_begin + c * CH, sKc + par * SB, sVc + par * SB, par ? B1 : B0,
                          sS + par * 2 * CH, sS + par * 2 * CH + CH, wave, lane);
  };
  if (nch > 0) issue(0);
  if (nch > 1) issue(1);
  for (int64_t c = 0; c < nch; ++c) {
    const int par = (int)(c & 1);
    wait_vm_at_most(c + 1 < nch ? nl : 0);   // chunk c landed (chunk c + 1 may be in flight)
    __syncthreads();
    convert_chunk_f8<NW * 64, D>(sKc + par * SB, sVc + par * SB, sK, sV, par ? B1 : B0);
    __syncthreads();
    if (active)
      attend_chunk<D, HT, KP, true>(sK, sV, par ? B1 : B0, Qb, O, m_run, l_run, sl2, col, grp, kh,
                                    sS + par * 2 * CH, sS + par * 2 * CH + CH);
    __syncthreads();
    if (c + 2 < nch) issue(c + 2);
  }
}

// ---- rows wider than 128 (d = 512 shared entries): one 16-head tile per wave
// pair.  A tile's O^T alone would take 128 of a lane's registers and its queries
// 64 more, which leaves none to keep LDS reads in flight; so the pair (lt, hh),
// hh = 0, 1, splits the chunk: wave hh scores key tiles 2hh, 2hh+1 over all of d
// (attend_wide_scores) and hands them to its partner through LDS; after a barrier
// both hold the chunk's 64 logits per head, take the same softmax steps on the
// same values, and wave hh accumulates columns [hh d/2, (hh+1) d/2) of O^T
// (attend_wide_pv).  m and l are computed twice, identically.

// logits (base 2, masked) of key tiles kt0 .. kt0 + NJ - 1 of the chunk over all of d
template <int D, int NJ, bool F8 = false>
__device__ __forceinline__ void wide_logits(const uint16_t* sK, const float* sBias, const bf16x8_t (&Qb)[1][D / 32],
                                            float sl2, int kt0, int lane, f32x4 (&S)[NJ], const float* sKs = nullptr) {
  constexpr int KS = D / 32;
  const int col = lane & 15, grp = lane >> 4;
  const int kx = swz_k<D>(col);
#pragma unroll
  for (int j = 0; j < NJ; ++j) S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two independent chains, software-pipelined by groups of kWideGroup steps: the
  // fragment reads of group g + 1 are issued before the products of group g, and a
  // scheduling fence closes each group, so a group's reads land while the
  // previous group computes and no more than two groups are in registers
  constexpr int G = kWideGroup * 2 / NJ, NGR = KS / G;
  static_assert(KS % G == 0, "whole groups");
  bf16x8_t A[2][G][NJ];
  auto fetch = [&](int g, bf16x8_t (&buf)[G][NJ]) {
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        buf[u][j] = *reinterpret_cast<const bf16x8_t*>(sK + chunk_off<D>(16 * (kt0 + j) + col, 4 * (g * G + u) + grp, kx));
  };
  fetch(0, A[0]);
#pragma unroll
  for (int g = 0; g < NGR; ++g) {
    if (g + 1 < NGR) fetch(g + 1, A[(g + 1) & 1]);
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        S[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g & 1][u][j], Qb[0][g * G + u], S[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const f32x4 bias = *reinterpret_cast<const f32x4*>(&sBias[16 * (kt0 + j) + 4 * grp]);
    f32x4 ksl = {sl2, sl2, sl2, sl2};
    if constexpr (F8) {   // the rows' scales; masked keys' scale words are whatever the fallback holds
      ksl = *reinterpret_cast<const f32x4*>(&sKs[16 * (kt0 + j) + 4 * grp]) * sl2;
#pragma unroll
      for (int e = 0; e < 4; ++e) ksl[e] = bias[e] == 0.f ? ksl[e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) S[j][e] = fmaf(S[j][e], ksl[e], bias[e]);
  }
}

// the pair's hand-over: wave hh scores key tiles 2hh, 2hh + 1 into sX
template <int D, bool F8 = false>
__device__ __forceinline__ void attend_wide_scores(const uint16_t* sK, const float* sBias, float* sX,
                                                   const bf16x8_t (&Qb)[1][D / 32], float sl2, int lt, int hh,
                                                   int lane, const float* sKs = nullptr) {
  f32x4 S[2];
  wide_logits<D, 2, F8>(sK, sBias, Qb, sl2, 2 * hh, lane, S, sKs);
#pragma unroll
  for (int j = 0; j < 2; ++j) reinterpret_cast<f32x4*>(sX)[(lt * 4 + 2 * hh + j) * 64 + lane] = S[j];
}

// softmax of the chunk's logits S (4 key tiles) and this wave's half of O^T += V^T P^T
// (F8: sVs holds the rows' scales, which weight the values in the product, not l)
template <int D, bool F8 = false>
__device__ __forceinline__ void attend_wide_pv(const uint16_t* sV, const f32x4 (&S)[4], f32x4 (&O)[1][D / 32],
                                               float (&m_run)[1], float (&l_run)[1], int hh, int lane,
                                               const float* sVs = nullptr) {
  constexpr int DH = D / 32;   // 16-column tiles of this wave's half
  const int col = lane & 15, grp = lane >> 4;
  float c = fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3]));
#pragma unroll
  for (int kt = 1; kt < 4; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) c = fmaxf(c, S[kt][e]);
  const float cm = col_max4(c);
  if (__builtin_amdgcn_ballot_w64(cm > m_run[0] + kLazyRescale)) {
    const bool up = cm > m_run[0] + kLazyRescale;
    const float alpha = up ? __builtin_amdgcn_exp2f(m_run[0] - cm) : 1.f;
    m_run[0] = up ? cm : m_run[0];
    l_run[0] *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH; ++dt) O[0][dt] *= alpha;
  }
  const float mu = m_run[0] == -INFINITY ? 0.f : m_run[0];
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int vr = 4 * grp + (col >> 2);
  const int vx = swz_v<D>(vr);
  const uint16_t* vb = sV + (col & 1) * 4;
  // P^T of both 32-key halves first, then the products, pipelined like the
  // scores: the V^T fragments of group g + 1 (over (kk, dt)) are read before the
  // products of group g
  bf16x8_t Bhi[2], Blo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = __builtin_amdgcn_exp2f(S[2 * kk + (e >> 2)][e & 3] - mu);
      ps += v;
      // (masked keys: v = 0, and their scale words are never multiplied)
      const float pv = F8 ? (v > 0.f ? v * sVs[32 * kk + 16 * (e >> 2) + 4 * grp + (e & 3)] : 0.f) : v;
      const __bf16 h = (__bf16)pv;
      Bhi[kk][e] = h;
      Blo[kk][e] = (__bf16)(pv - (float)h);
    }
    l_run[0] += ps;
  }
  constexpr int G = kWideGroup, NGR = 2 * DH / G;   // groups over (kk, dt), kk outer
  static_assert(DH % G == 0, "whole groups");
  bf16x8_t A[2][G];
  auto fetch = [&](int g, bf16x8_t (&buf)[G]) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int kk = (g * G + u) / DH, dt = (g * G + u) % DH;
      const uint16_t* v0 = vb + chunk_off<D>(vr + 32 * kk, 2 * (hh * DH + dt) + ((col & 3) >> 1), vx);
      const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(v0));
      const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(v0 + 16 * sub_cols<D>()));
      buf[u] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  fetch(0, A[0]);
#pragma unroll
  for (int g = 0; g < NGR; ++g) {
    if (g + 1 < NGR) fetch(g + 1, A[(g + 1) & 1]);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int kk = (g * G + u) / DH, dt = (g * G + u) % DH;
      O[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g & 1][u], Bhi[kk], O[0][dt], 0, 0, 0);
      O[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g & 1][u], Blo[kk], O[0][dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The chunk pipeline of the wide rows: as run_chunks, with the pair's hand-over
// between the scores and the products (one more barrier per chunk).
template <int NW, int D, bool SKV>
__device__ __forceinline__ void run_chunks_wide(const RowKeys& R, const int* s_idx, uint16_t* K0, uint16_t* V0,
                                                float* B0, uint16_t* K1, uint16_t* V1, float* B1, float* sX,
                                                int64_t nch, bool active, const bf16x8_t (&Qb)[1][D / 32],
                                                f32x4 (&O)[1][D / 32], float (&m_run)[1], float (&l_run)[1],
                                                float sl2, int wave, int lane, int lt, int hh) {
  constexpr int CH = kAttnChunk;
  constexpr int IPW = CH * (D / 8) / 64 / NW;
  constexpr int LPW = SKV ? IPW : 2 * IPW;
  if (nch > 0) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin, K0, V0, B0, wave, lane);
  if (nch > 1) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin + CH, K1, V1, B1, wave, lane);
  for (int64_t c = 0; c < nch; ++c) {
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    const bool odd = (c & 1) != 0;
    uint16_t* Kc = odd ? K1 : K0;
    uint16_t* Vc = odd ? V1 : V0;
    float* Bc = odd ? B1 : B0;
    // (each wave scoring the whole chunk itself, without the hand-over, measured
    // slower: 33% more products for one barrier less)
    if (active) attend_wide_scores<D>(Kc, Bc, sX, Qb, sl2, lt, hh, lane);
    __syncthreads();
    if (active) {
      f32x4 S[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) S[kt] = reinterpret_cast<const f32x4*>(sX)[(lt * 4 + kt) * 64 + lane];
      attend_wide_pv<D>(Vc, S, O, m_run, l_run, hh, lane);
    }
    __syncthreads();
    if (c + 2 < nch) issue_chunk<NW, D, SKV>(R, s_idx, R.k_begin + (c + 2) * CH, Kc, Vc, Bc, wave, lane);
  }
}

// The chunk pipeline of FP8 shared rows of 512, as run_chunks_f8: two staging halves
// in the second chunk buffer's space (32 KB of codes each), converted into the first;
// chunks 0 and 1 go out together, chunk c + 2 once chunk c is done.
template <int NW, int D>
__device__ __forceinline__ void run_chunks_wide_f8(const RowKeys& R, const int* s_idx, uint16_t* sK,
                                                   unsigned char* sKc, float* B0, float* B1, float* sS, float* sX,
                                                   int64_t nch, bool active, const bf16x8_t (&Qb)[1][D / 32],
                                                   f32x4 (&O)[1][D / 32], float (&m_run)[1], float (&l_run)[1],
                                                   float sl2, int wave, int lane, int lt, int hh) {
  constexpr int CH = kAttnChunk, SB = kAttnChunk * D;   // staging bytes per chunk
  const int nl = f8_chunk_loads<NW, D, true>(wave);
  auto issue = [&](int64_t c) {
    const int par = __builtin_amdgcn_readfirstlane((int)(c & 1));   // (the staging address must be scalar)
    issue_chunk_f8_shared<NW, D>(R, s_idx, R.k_begin + c * CH, sKc + par * SB, par ? B1 : B0, sS + par * CH, wave,
                                 lane);
  };
  if (nch > 0) issue(0);
  if (nch > 1) issue(1);
  for (int64_t c = 0; c < nch; ++c) {
    const int par = (int)(c & 1);
    float* Bc = par ? B1 : B0;
    const float* Sc = sS + par * CH;
    wait_vm_at_most(c + 1 < nch ? nl : 0);   // chunk c landed (chunk c + 1 may be in flight)
    __syncthreads();
    convert_chunk_f8<NW * 64, D, true>(sKc + par * SB, sKc + par * SB, sK, sK, Bc);
    __syncthreads();
    if (active) attend_wide_scores<D, true>(sK, Bc, sX, Qb, sl2, lt, hh, lane, Sc);
    __syncthreads();
    if (active) {
      f32x4 S[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) S[kt] = reinterpret_cast<const f32x4*>(sX)[(lt * 4 + kt) * 64 + lane];
      attend_wide_pv<D, true>(sK, S, O, m_run, l_run, hh, lane, Sc);
    }
    __syncthreads();
    if (c + 2 < nch) issue(c + 2);
  }
}

// LDS of one attention workgroup: two chunk buffers (K, V, mask; shared entries
// (SKV) keep one row that serves as both); AttnSmem adds the split's CSA ids.
template <int D, bool SKV = false>
struct AttnBuf {
  static constexpr int kRows = kAttnChunk * D;
  union {
    uint16_t buf[(SKV ? 2 : 4) * kRows];
    // after the last chunk: the state (O, m, l) one key half hands to the other,
    // per lane of 4 waves (rows up to 128)
    float C[D > 128 ? 1 : 4 * 64 * (D / 4 + 2)];
  };
  // wide rows: the logits a wave pair hands over, [tile][key tile][lane] x 4
  float X[D > 128 ? kWideTiles * 4 * 64 * 4 : 1];
  float B0[kAttnChunk], B1[kAttnChunk];
  float S8[4 * kAttnChunk];   // FP8 caches: [parity][K, V] row scales of a chunk
  __device__ uint16_t* K0() { return buf; }
  __device__ uint16_t* K1() { return buf + kRows; }
  __device__ uint16_t* V0() { return SKV ? buf : buf + 2 * kRows; }
  __device__ uint16_t* V1() { return SKV ? buf + kRows : buf + 3 * kRows; }
};
template <int D, bool SKV = false>
struct AttnSmem : AttnBuf<D, SKV> {
  int idx[kMaxTopk];
};

// The work of one workgroup of NW waves on (split, row).  With KP = 1, wave w computes
// head tiles w, w + NW, ... (HT of them); with KP = 2, waves w and w + NW/2 share
// head tiles w, w + NW/2, ... (HT of them) and take one half of every chunk's keys
// each, and combine their softmax states through LDS at the end.  With head_groups > 1 the
// launch's x index is split * head_groups + group and the workgroup takes only the
// group's head tiles (fewer queries read and partials written per workgroup).  A
// tile past the group's is computed on a copy of the group's first tile's queries
// and not written.  All waves load.
// Chunks are double-buffered in LDS: the loads of chunk c + 1 are in flight while
// chunk c is computed.
// QP: the output is rotated back at -pos (the query arrives normalised and rotated
// from launch_qprep); without it the kernel carries none of that code.  SKV: every
// entry is its own value (shared K = V rows, loaded once).
// s_idx: the LDS array of the split's CSA ids (the split's slot t at s_idx[t]); with
// ids_ready the caller has filled it already (and synchronised), else they are
// loaded from p.idx here.
template <int NW, int HT, int D, int KP, bool QP = false, bool SKV = false, bool F8 = false>
__device__ __forceinline__ void attn_block(const AttnP& p, int xs, int row, AttnBuf<D, SKV>& sm, int* s_idx,
                                           bool ids_ready = false) {
  static_assert(!F8 || (!SKV && D <= 128) || (SKV && D == 512),
                "FP8 caches: separate K and V rows of up to 128, or shared rows of 512");
  static_assert(KP == 1 || (KP == 2 && NW % 2 == 0 && (NW / 2) * HT <= 4),
                "key halves pair waves on their head tiles; the combine buffer holds 4 (wave, tile) states");
  constexpr bool WIDE = D > 128;   // wave pairs per head tile (attend_wide_*)
  static_assert(!WIDE || (NW == 8 && HT == 1 && KP == 1), "wide rows: 8 waves, one tile per pair");
  // xs = split * head_groups + group: the workgroup takes group's head tiles
  const int hgn = p.head_groups, split = xs / hgn, hgi = xs - split * hgn;
  constexpr int TW = WIDE ? kWideTiles : NW / KP;   // head tiles of one pass
  constexpr int NT = NW * 64, CH = kAttnChunk, KS = D / 32, DT = D / 16;
  const int b = row / p.tq, i = row - b * p.tq;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntg = p.heads / 16 / hgn;   // head tiles of the group
  const float sl2 = p.scale * kLog2e;

  // Independent loads first, all in flight together: the position, the raw
  // window's start, q and the split's CSA ids (their range does not depend on the
  // position: slots past the row's visible blocks hold -1).
  const int64_t pos_ld = p.pos0[b];
  const int64_t raw_ld = (p.mask & 4u) ? p.raw_start[b] : 0;
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bs + (int64_t)i * p.q_rs;
  int tile[HT];
  bool tv[HT];   // the wave's tile t exists in the group
  bf16x8_t Qb[HT][KS];
  const int kh = (KP == 2 || WIDE) ? wave / TW : 0;   // key half, or the pair's half of a wide row
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int lt = wave % TW + TW * t;
    tv[t] = lt < ntg;
    tile[t] = hgi * ntg + (tv[t] ? lt : 0);
    const int tq = tile[t];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      Qb[t][s] = *reinterpret_cast<const bf16x8_t*>(qrow + (tq * 16 + col) * D + s * 32 + grp * 8);
  }
  const int64_t k_begin = p.key_lo + (int64_t)split * p.keys_per_split;
  const int64_t n_csa = (p.mask & 1u) ? p.topk : 0;
  const int64_t n_idx = min(min(n_csa, p.key_hi), k_begin + (int64_t)p.keys_per_split) - k_begin;
  const int32_t* ip = p.idx + (int64_t)b * p.idx_bs + (int64_t)i * p.idx_rs + k_begin;
  constexpr int IDX_PER = kMaxTopk / NT;  // ids per thread: n_idx <= topk <= kMaxTopk
  int ids[IDX_PER];
  if (!ids_ready && n_idx > 0) {
#pragma unroll
    for (int u = 0; u < IDX_PER; ++u) ids[u] = ip[min((int64_t)(u * NT + tid), n_idx - 1)];
  }

  const int64_t pos = uniform_i64(pos_ld + i);
  const int64_t raw0 = uniform_i64(raw_ld);
  const KeyList L = key_list(p, pos);
  RowKeys R;
  R.k_begin = k_begin;
  R.k_end = min(min(L.n_keys, p.key_hi), R.k_begin + (int64_t)p.keys_per_split);
  R.n_csa = L.n_csa;
  R.hca_end = L.n_csa + L.e_vis;
  R.raw_off = L.w_lo - R.hca_end - raw0;
  R.fallback = qrow;
  R.kc = (p.mask & 1u) ? reinterpret_cast<const uint16_t*>(p.kc) + (int64_t)b * p.kc_bs : qrow;
  R.vc = (p.mask & 1u) ? reinterpret_cast<const uint16_t*>(p.vc) + (int64_t)b * p.vc_bs : qrow;
  R.kh = (p.mask & 2u) ? reinterpret_cast<const uint16_t*>(p.kh) + (int64_t)b * p.kh_bs : qrow;
  R.vh = (p.mask & 2u) ? reinterpret_cast<const uint16_t*>(p.vh) + (int64_t)b * p.vh_bs : qrow;
  R.kr = (p.mask & 4u) ? reinterpret_cast<const uint16_t*>(p.kr) + (int64_t)b * p.kr_bs : qrow;
  R.vr = (p.mask & 4u) ? reinterpret_cast<const uint16_t*>(p.vr) + (int64_t)b * p.vr_bs : qrow;
  R.kc_rs = p.kc_rs; R.vc_rs = p.vc_rs; R.kh_rs = p.kh_rs; R.vh_rs = p.vh_rs; R.kr_rs = p.kr_rs; R.vr_rs = p.vr_rs;
  if constexpr (F8) {
    // codes are bytes (strides in elements = bytes); scales one fp32 per cache row
    auto bytes = [&](const void* t, int64_t bs, bool on) {
      return on ? reinterpret_cast<const uint16_t*>(reinterpret_cast<const unsigned char*>(t) + (int64_t)b * bs) : qrow;
    };
    R.kc = bytes(p.kc, p.kc_bs, p.mask & 1u);
    R.kh = bytes(p.kh, p.kh_bs, p.mask & 2u);
    R.kr = bytes(p.kr, p.kr_bs, p.mask & 4u);
    const float* fb = reinterpret_cast<const float*>(qrow);
    R.kcs = (p.mask & 1u) ? p.kcs + (int64_t)b * p.kcs_bs : fb;
    R.khs = (p.mask & 2u) ? p.khs + (int64_t)b * p.khs_bs : fb;
    R.krs = (p.mask & 4u) ? p.krs + (int64_t)b * p.krs_bs : fb;
    if constexpr (SKV) {   // every row its own value: the value tables are the key tables
      R.vc = R.kc; R.vh = R.kh; R.vr = R.kr;
      R.vcs = R.kcs; R.vhs = R.khs; R.vrs = R.krs;
    } else {
      R.vc = bytes(p.vc, p.vc_bs, p.mask & 1u);
      R.vh = bytes(p.vh, p.vh_bs, p.mask & 2u);
      R.vr = bytes(p.vr, p.vr_bs, p.mask & 4u);
      R.vcs = (p.mask & 1u) ? p.vcs + (int64_t)b * p.vcs_bs : fb;
      R.vhs = (p.mask & 2u) ? p.vhs + (int64_t)b * p.vhs_bs : fb;
      R.vrs = (p.mask & 4u) ? p.vrs + (int64_t)b * p.vrs_bs : fb;
    }
  }
  if (!ids_ready && n_idx > 0) {
#pragma unroll
    for (int u = 0; u < IDX_PER; ++u)
      if (u * NT + tid < n_idx) s_idx[u * NT + tid] = ids[u];
    __syncthreads();
  }

  // the 16-column tiles of O^T this wave holds (a wide row's pair splits them) and
  // the first one's index
  constexpr int DTW = WIDE ? DT / 2 : DT;
  const int dt0 = WIDE ? kh * DTW : 0;
  float m_run[HT], l_run[HT];
  f32x4 O[HT][DTW];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) O[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t nch = R.k_end > R.k_begin ? (R.k_end - R.k_begin + CH - 1) / CH : 0;
  if constexpr (F8 && WIDE)
    run_chunks_wide_f8<NW, D>(R, s_idx, sm.K0(), reinterpret_cast<unsigned char*>(sm.K1()), sm.B0, sm.B1, sm.S8, sm.X,
                              nch, tv[0], Qb, O, m_run, l_run, sl2, wave, lane, wave % TW, kh);
  else if constexpr (F8)
    run_chunks_f8<NW, D, HT, KP>(R, s_idx, sm.K0(), sm.V0(), reinterpret_cast<unsigned char*>(sm.K1()),
                                 reinterpret_cast<unsigned char*>(sm.V1()), sm.B0, sm.B1, sm.S8, nch, tv[0], Qb, O,
                                 m_run, l_run, sl2, wave, lane, kh);
  else if constexpr (WIDE)
    run_chunks_wide<NW, D, SKV>(R, s_idx, sm.K0(), sm.V0(), sm.B0, sm.K1(), sm.V1(), sm.B1, sm.X, nch, tv[0], Qb,
                                O, m_run, l_run, sl2, wave, lane, wave % TW, kh);
  else
    run_chunks<NW, D, HT, KP, SKV>(R, s_idx, sm.K0(), sm.V0(), sm.B0, sm.K1(), sm.V1(), sm.B1, nch, tv[0], Qb, O,
                                   m_run, l_run, sl2, wave, lane, kh);

  if constexpr (KP == 2) {
    // the second key half hands (O, m, l) of each of its tiles to the first through
    // LDS; the chunk buffers are free (every chunk's reads ended at a barrier, no
    // load in flight)
    f32x4* sO = reinterpret_cast<f32x4*>(sm.C);
    float* sM = sm.C + 4 * 64 * (D / 4);
    constexpr int NS = TW * HT * 64;   // (wave, tile) state slots
    if (kh == 1) {
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        const int slot = (t * TW + wave % TW) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) sO[dt * NS + slot] = O[t][dt];
        sM[slot] = m_run[t];
        sM[NS + slot] = l_run[t];
      }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        const int slot = (t * TW + wave % TW) * 64 + lane;
        const float m1 = sM[slot], l1 = sM[NS + slot];
        const float m = fmaxf(m_run[t], m1);
        const float a0 = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - m);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
        m_run[t] = m;
        l_run[t] = l_run[t] * a0 + l1 * a1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[t][dt] = O[t][dt] * a0 + sO[dt * NS + slot] * a1;
      }
    }
  }

#pragma unroll
  for (int t = 0; t < HT; ++t) {
    if (!tv[t] || (KP == 2 && kh != 0)) continue;
    const bool stats = !WIDE || kh == 0;   // one wave of a wide pair writes lse / (m, l)
    const int head = tile[t] * 16 + col;
    const float l = col_sum4(l_run[t]);
    if (p.splits_total == 1) {
      float lse;
      const float f = finish_head(m_run[t], l, p.sink, head, &lse);
      const int64_t orow = (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        float ov[4] = {O[t][dt][0] * f, O[t][dt][1] * f, O[t][dt][2] * f, O[t][dt][3] * f};
        if (QP && p.rope_out) {  // back at -pos: channels (dt0+dt)*16 + 4*grp + e, pairs inside the lane
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int e0 = (dt0 + dt) * 16 + 4 * grp + 2 * k2;
            if (e0 < D - p.rope) continue;
            float cs, sn;
            rope_cs((double)pos, (e0 - (D - p.rope)) / 2, p.rope, p.rope_lb, cs, sn);
            rot2(ov[2 * k2], ov[2 * k2 + 1], cs, sn, true);
          }
        }
        store_out4(p.o, p.o_bf16, orow + (dt0 + dt) * 16 + 4 * grp, ov[0], ov[1], ov[2], ov[3]);
      }
      if (stats && grp == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
    } else {
      const int64_t slot = ((int64_t)row * p.heads + head) * p.splits_total + p.split_base + split;
      float* po = p.part_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
        *reinterpret_cast<float4*>(po + (dt0 + dt) * 16 + 4 * grp) =
            make_float4(O[t][dt][0], O[t][dt][1], O[t][dt][2], O[t][dt][3]);
      if (stats && grp == 0)
        *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run[t], l);
    }
  }
}

// ------------------------------------------------------------------ prefill query tiles
// [QbitAI] 混合注意力机制, HCA and window paragraphs: inside a prefill chunk the HCA
// entries and raw window rows one query sees are, up to the causal edge, the ones its
// neighbours see.  A workgroup of NW waves of HT head tiles each takes
// QT = 16 NW HT / H consecutive queries of one sequence and streams the union of
// their keys, HCA entries [0, e_vis(last)) then raw positions [w_lo(first), p(last)],
// through LDS once for all of them; each query masks what it does not see (the
// causal HCA edge, its own window bounds).  So every key row is read from L2 once
// per QT queries instead of once per query.  The CSA picks differ per query and are
// attended per row by the launch before this one, which leaves each row's partial
// (O, m, l) in split slot 0; this kernel joins it to its own state and writes the
// row's o and lse.  Rows past tq in a sequence's last tile are computed on the last
// row's queries and not written.
constexpr int kMaxQTile = 8;

template <int D>
struct QTileSmem {
  uint16_t buf[4 * kAttnChunk * D];           // K0, K1, V0, V1
  float bias[2][kMaxQTile][kAttnChunk];       // [chunk parity][query][key]
  __device__ uint16_t* K(int c) { return buf + c * kAttnChunk * D; }
  __device__ uint16_t* V(int c) { return buf + (2 + c) * kAttnChunk * D; }
};

// the tile's union key list and one query's view of it
struct QTileKeys {
  const uint16_t *kh, *vh, *kr, *vr, *fallback;
  int64_t kh_rs, vh_rs, kr_rs, vr_rs;
  int64_t n_h, n_u, w_lo0, raw0;     // HCA entries, all keys, first window position, raw_start
  // query q (absent ones mirror the last present one) sees HCA entries [0, evis[q])
  // and window keys with t - n_h in (hi[q] - W, hi[q]]
  int evis[kMaxQTile], hi[kMaxQTile];
  int W, qt;
};

// Loads chunk kc0 of the union list into (sK, sV) and writes every query's mask.
template <int D, int NW>
__device__ __forceinline__ void issue_qchunk(const QTileKeys& T, int64_t kc0, uint16_t* sK, uint16_t* sV,
                                             float (*bias)[kAttnChunk], int wave, int lane) {
  constexpr int PS = D / 8, RPI = 64 / PS, RBW = kAttnChunk / RPI / NW;
  static_assert(D <= 128 && RBW >= 1 && RBW * RPI * NW == kAttnChunk, "rows of up to 128, spread over the waves");
  const int prow = lane / PS, ppiece = lane % PS;
#pragma unroll
  for (int u = 0; u < RBW; ++u) {
    const int r0 = (wave * RBW + u) * RPI;
    const int r = r0 + prow;
    const int64_t t = kc0 + r;
    const bool in_h = t < T.n_h, in_w = !in_h && t < T.n_u;
    const int64_t pt = T.w_lo0 + (t - T.n_h);          // window keys: their position
    const uint16_t* kp = in_h ? row_ptr(T.kh, (uint32_t)t, T.kh_rs)
                              : in_w ? row_ptr(T.kr, (uint32_t)(pt - T.raw0), T.kr_rs) : T.fallback;
    const uint16_t* vp = in_h ? row_ptr(T.vh, (uint32_t)t, T.vh_rs)
                              : in_w ? row_ptr(T.vr, (uint32_t)(pt - T.raw0), T.vr_rs) : T.fallback;
    lds_load16(kp + (ppiece ^ swz_k<D>(r)) * 8, lds_addr(sK + r0 * D));
    lds_load16(vp + (ppiece ^ swz_v<D>(r)) * 8, lds_addr(sV + r0 * D));
    if (ppiece == 0) {
      const int tw = (int)(t - T.n_h);
#pragma unroll
      for (int q = 0; q < kMaxQTile; ++q) {
        if (q >= T.qt) break;
        const bool ok = in_h ? t < T.evis[q] : in_w && tw <= T.hi[q] && tw > T.hi[q] - T.W;
        bias[q][r] = ok ? 0.f : -INFINITY;
      }
    }
  }
}

template <int D, int NW, int HT>
__device__ __forceinline__ void attn_qtile_block(const AttnP& p, int tile, int b, QTileSmem<D>& sm) {
  constexpr int KS = D / 32, DT = D / 16, CH = kAttnChunk;
  constexpr int LPW = 2 * (CH * (D / 8) / 64 / NW);   // a chunk's direct loads per wave (K and V)
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntq = p.heads / 16;                 // head tiles per query
  const int wpq = ntq / HT;                     // waves per query
  const int QT = NW / wpq;                      // queries per workgroup tile
  const int q = wave / wpq, t0 = (wave % wpq) * HT;
  const int i0 = tile * QT;
  const int nq = min(QT, p.tq - i0);            // queries of this tile that exist
  const int i = i0 + min(q, nq - 1);            // the row this wave computes
  const int64_t pos_ld = p.pos0[b];
  const int64_t raw_ld = (p.mask & 4u) ? p.raw_start[b] : 0;
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bs + (int64_t)i * p.q_rs;
  bf16x8_t Qb[HT][KS];
#pragma unroll
  for (int t = 0; t < HT; ++t)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      Qb[t][s2] = *reinterpret_cast<const bf16x8_t*>(qrow + ((t0 + t) * 16 + col) * D + s2 * 32 + grp * 8);

  QTileKeys T;
  const int64_t pos0 = uniform_i64(pos_ld) + i0;
  T.qt = QT;
  T.W = ((p.mask & 4u) && p.W > 0) ? p.W : 0;
  const int64_t p_last = pos0 + nq - 1;
  T.n_h = (p.mask & 2u) ? (p_last + 1) / p.mh : 0;
  T.w_lo0 = pos0 - T.W + 1 > 0 ? pos0 - T.W + 1 : 0;
#pragma unroll
  for (int qq = 0; qq < kMaxQTile; ++qq) {
    const int64_t pq = pos0 + min(qq, nq - 1);
    T.evis[qq] = (p.mask & 2u) ? (int)((pq + 1) / p.mh) : 0;
    T.hi[qq] = (int)(pq - T.w_lo0);
  }
  T.n_u = T.n_h + (T.W > 0 ? p_last - T.w_lo0 + 1 : 0);
  T.raw0 = uniform_i64(raw_ld);
  T.fallback = qrow;
  T.kh = (p.mask & 2u) ? reinterpret_cast<const uint16_t*>(p.kh) + (int64_t)b * p.kh_bs : qrow;
  T.vh = (p.mask & 2u) ? reinterpret_cast<const uint16_t*>(p.vh) + (int64_t)b * p.vh_bs : qrow;
  T.kr = (p.mask & 4u) ? reinterpret_cast<const uint16_t*>(p.kr) + (int64_t)b * p.kr_bs : qrow;
  T.vr = (p.mask & 4u) ? reinterpret_cast<const uint16_t*>(p.vr) + (int64_t)b * p.vr_bs : qrow;
  T.kh_rs = p.kh_rs; T.vh_rs = p.vh_rs; T.kr_rs = p.kr_rs; T.vr_rs = p.vr_rs;

  const float sl2 = p.scale * kLog2e;
  float m_run[HT], l_run[HT];
  f32x4 O[HT][DT];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int64_t nch = (T.n_u + CH - 1) / CH;
  if (nch > 0) issue_qchunk<D, NW>(T, 0, sm.K(0), sm.V(0), sm.bias[0], wave, lane);
  if (nch > 1) issue_qchunk<D, NW>(T, CH, sm.K(1), sm.V(1), sm.bias[1], wave, lane);
  for (int64_t c = 0; c < nch; ++c) {
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    const int par = (int)(c & 1);
    attend_chunk<D, HT, 1>(sm.K(par), sm.V(par), sm.bias[par][q], Qb, O, m_run, l_run, sl2, col, grp, 0);
    __syncthreads();
    if (c + 2 < nch) issue_qchunk<D, NW>(T, (c + 2) * CH, sm.K(par), sm.V(par), sm.bias[par], wave, lane);
  }
  if (q >= nq) return;
  // the row's CSA partial (slot 0, written by the launch before this one) joins this
  // state, and the row's output is written here: o, lse (no merge launch)
  const int64_t row = (int64_t)b * p.tq + i;
  const int64_t pos = pos0 + q;
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int head = (t0 + t) * 16 + col;
    const int64_t slot = (row * p.heads + head) * p.splits_total;
    const float2 mlc = *reinterpret_cast<const float2*>(p.part_ml + slot * 2);
    const float* pc = p.part_o + slot * D;
    const float m = fmaxf(m_run[t], mlc.x);
    const float a = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - m);
    const float ac = mlc.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mlc.x - m);
    const float l = col_sum4(l_run[t]) * a + mlc.y * ac;
    float lse;
    const float f = finish_head(m, l, p.sink, head, &lse);
    const int64_t orow = (int64_t)b * p.o_bs + (int64_t)i * p.o_rs + head * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float4 oc = *reinterpret_cast<const float4*>(pc + dt * 16 + 4 * grp);
      float ov[4] = {(O[t][dt][0] * a + oc.x * ac) * f, (O[t][dt][1] * a + oc.y * ac) * f,
                     (O[t][dt][2] * a + oc.z * ac) * f, (O[t][dt][3] * a + oc.w * ac) * f};
      if (p.rope_out) {  // back at -pos: channels dt*16 + 4*grp + e, pairs inside the lane
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int e0 = dt * 16 + 4 * grp + 2 * k2;
          if (e0 < D - p.rope) continue;
          float cs, sn;
          rope_cs((double)pos, (e0 - (D - p.rope)) / 2, p.rope, p.rope_lb, cs, sn);
          rot2(ov[2 * k2], ov[2 * k2 + 1], cs, sn, true);
        }
      }
      store_out4(p.o, p.o_bf16, orow + dt * 16 + 4 * grp, ov[0], ov[1], ov[2], ov[3]);
    }
    if (grp == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)i * p.lse_rs + head] = lse;
  }
}

}  // namespace v4a
