// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v4a {

// ---------------------------------------------------------------- compress
struct CompressP {
  const void* k_raw; const void* v_raw; const float* logits;
  void* k_out; void* v_out;
  const int64_t* raw_start;
  int64_t kr_bs, kr_rs, vr_bs, vr_rs, lg_bs;
  int64_t ko_bs, ko_rs, vo_bs, vo_rs;
  int64_t t0;     // first position (multiple of r)
  int64_t nb;     // blocks to write
  int r, d;
  int ch;         // 16-byte chunks per row
  int g;          // row groups per block (threads sharing one block's rows)
  int bpw;        // blocks per workgroup
};
hipError_t launch_compress(int dtype, const CompressP& p, int batch, hipStream_t s);

// ---------------------------------------------------------------- indexer
constexpr int kHistBits = 12;                 // first radix level: top 12 key bits
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = 16384;               // per-row candidate list capacity
constexpr int kMaxTopk = 2048;

struct ScoreP {
  const void* qi; const float* wi; const void* ki;
  const int64_t* pos0;
  float* scores;      // [rows][sc_rs]
  uint32_t* hist;     // [rows][kHistBins]
  int64_t qi_bs, qi_rs, wi_bs, wi_rs, ki_bs, ki_rs, sc_rs;
  int tq, row0;       // launch covers global rows row0 + blockIdx.y; row = b*tq + i
  int heads, dim, ratio, topk;
  int tile;           // blocks per workgroup
};
hipError_t launch_score(int dtype, const ScoreP& p, int nrows, int ntiles, hipStream_t s);

struct TopkP {
  const float* scores; const uint32_t* hist;
  uint32_t* sure;     // [rows][kMaxTopk] ids above the threshold bin
  uint2* cand;        // [rows][kCandCap] (key, id) in the threshold bin
  uint32_t* counts;   // [rows][4]: n_sure, n_cand
  const int64_t* pos0;
  int32_t* idx; int64_t idx_bs, idx_rs;
  float* sel; int64_t sel_bs, sel_rs;
  int64_t sc_rs;
  int tq, row0, ratio, topk;
  int slice;          // scores per filter workgroup
};
hipError_t launch_topk_clear(const TopkP& p, int nrows, hipStream_t s);
hipError_t launch_topk_filter(const TopkP& p, int nrows, int nslices, hipStream_t s);
hipError_t launch_topk_final(const TopkP& p, int nrows, hipStream_t s);

// ---------------------------------------------------------------- attention
constexpr int kAttnChunk = 32;  // keys per inner chunk of the attention kernels

struct AttnP {
  const void* q; int64_t q_bs, q_rs;
  const int32_t* idx; int64_t idx_bs, idx_rs;
  const void* kc; const void* vc; int64_t kc_bs, kc_rs, vc_bs, vc_rs;
  const void* kh; const void* vh; int64_t kh_bs, kh_rs, vh_bs, vh_rs;
  const void* kr; const void* vr; int64_t kr_bs, kr_rs, vr_bs, vr_rs;
  const int64_t* raw_start; const int64_t* pos0; const float* sink;
  float* o; int64_t o_bs, o_rs;
  float* lse; int64_t lse_bs, lse_rs;
  float* part_o;   // [rows][splits][H][d]
  float* part_ml;  // [rows][splits][H][2]
  int tq, heads, dim;
  uint32_t mask;
  int m, mh, W, topk;
  float scale;     // already resolved (never 0)
  int splits, keys_per_split;
};
hipError_t launch_attn(int dtype, const AttnP& p, int nrows, hipStream_t s);
hipError_t launch_merge(const AttnP& p, int nrows, hipStream_t s);

// ---------------------------------------------------------------- timing hooks
void timing_before(int kernel, hipStream_t s);
void timing_after(int kernel, hipStream_t s);

}  // namespace v4a
