// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_ext.h>
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
  const float* gk; const float* gv; float eps;  // RMSNorm gains of the entries (null: none)
  int rope;            // rotated channels R (0: off), the last R of each row
  int rope_v;          // raw V rows are rotated too
  double rope_lb;      // log2 of the RoPE base
  int f8out;           // entries stored as FP8 E4M3 codes (k_out / v_out bytes) with fp32 row scales
  float* ks_out; float* vs_out; int64_t kso_bs, vso_bs;
};
hipError_t launch_compress(int dtype, const CompressP& p, int batch, hipStream_t s, int tid);

// ---------------------------------------------------------------- indexer
constexpr int kTile = 256;        // blocks per score tile
constexpr int kWaveTop = 4;       // (key, id) pairs each 64-block wave picks
constexpr int kTileTop = 8;       // (key, id) slots of a tile report
constexpr int kPrefillTileTop = 4;  // slots the prefill score kernel fills (the rest are empty)
constexpr int kPoolCap = 4096;    // candidate pool of the per-row selection (LDS)
constexpr int kMaxTopk = 2048;
constexpr int kSelThreads = 512;

// Query prep (bf16): [QbitAI] 混合注意力机制, Q/KV normalization and partial RoPE.
// Row r = b * tq + i of q is RMS-normalised with gain (if any) and its last `rope`
// channels rotated at pos0[b] + i; out [rows][heads][dim] bf16.
struct QPrepP {
  const void* q; int64_t q_bs, q_rs;
  const float* gain; float eps;
  int rope; double rope_lb;
  int heads, dim, tq;
  const int64_t* pos0;
  uint16_t* out;
};
hipError_t launch_qprep(const QPrepP& p, int nrows, hipStream_t s, int tid);
// 256-thread blocks of the query prep of one row
inline int qprep_blocks(const QPrepP& p) { return (p.heads * (p.dim / 8) + 255) / 256; }

struct ScoreP {
  const void* qi; const float* wi; const void* ki;
  const float* ki_scale; int64_t ks_bs;   // FP8 keys: one scale per row (null: bf16 keys)
  const int64_t* pos0;
  float* scores;      // [rows][sc_rs]
  uint32_t* rep_key;  // [rows][key_rs]: per tile, the keys of its kTileTop best, in id order
  uint4* rep_info;    // [rows][info_rs]: per tile, (offsets 0-3, offsets 4-7 as 8-bit fields, bound key, 0)
  int64_t qi_bs, qi_rs, wi_bs, wi_rs, ki_bs, ki_rs, sc_rs, key_rs, info_rs;
  int tq, row0;       // launch covers global rows row0 + blockIdx.y; row = b*tq + i
  int heads, dim, ratio;
  int wgs_per_row;    // bf16 kernel: workgroups per row group, each walking tiles with that stride
  int wave_top;       // decode forms: candidates per 64-block wave of a tile report (4 or kTileTop)
  // prefill form only:
  int sample_stride;      // > 0: score tiles 0, s, 2s, ... only and store their scores (no reports)
  const uint32_t* theta;  // [launch rows]: threshold mode, per row a key that bounds the row's k-th
                          // from below (null: exact reports of kPrefillTileTop and every score stored)
  const uint32_t* repair; // [launch rows]: only workgroups with a flagged row run (null: all)
  int nrows;          // rows of the launch (set by launch_score)
  // bf16 kernel: workgroups x < prep_x of row y prepare that row's attention queries
  // instead (0: none); the score workgroups follow them
  QPrepP prep; int prep_x;
};
hipError_t launch_score(int dtype, const ScoreP& p, int nrows, int ntiles, hipStream_t s, int tid);
// Prefill form (bf16 64 x 64 indexer, tq a multiple of 8, row0 too): workgroups of 8
// query rows, each key tile read once for the 8; p.wgs_per_row workgroups per group
// of 8 rows, walking the tiles (at most ntiles).  Same outputs as launch_score.
hipError_t launch_score_rows(const ScoreP& p, int nrows, int ntiles, hipStream_t s, int tid);

struct SelectP {
  const float* scores; const uint32_t* rep_key; const uint4* rep_info;
  const int64_t* pos0;
  int32_t* idx; int64_t idx_bs, idx_rs;
  float* sel; int64_t sel_bs, sel_rs;
  int64_t sc_rs, key_rs, info_rs;
  int tq, row0, ratio, topk;
  int ntiles_cap;     // score tiles of the longest row (pos_max): bounds the report loads
  int rep_top;        // report slots per tile that the score kernel fills (kTileTop or kPrefillTileTop)
  // prefill threshold mode:
  const uint32_t* theta;  // [launch rows]: the rows' thresholds (null: exact reports)
  uint32_t* flag;         // [launch rows]: set to 1 where a row has to be redone exactly, else 0
  const uint32_t* repair; // [launch rows]: only flagged rows are selected (null: all)
  int sample_stride;      // theta_kernel: the sampled tiles (0, s, 2s, ...)
  uint32_t* theta_out;    // theta_kernel: [launch rows]
};
hipError_t launch_select(const SelectP& p, int nrows, hipStream_t s, int tid);
// Per row, a threshold key from the scores of the sampled tiles: the r-th largest
// with r = 3 k n_s / n_vis + 16 (n_s sampled keys), or 0 when the sample holds fewer.
hipError_t launch_theta(const SelectP& p, int nrows, hipStream_t s, int tid);

// ---------------------------------------------------------------- attention
constexpr int kAttnChunk = 64;  // keys per inner chunk of the attention kernels
constexpr int kWideTiles = 4;   // 16-head tiles per workgroup for rows wider than 128 (a wave pair each)
constexpr int kAttnMaxSplits = 1024;

struct AttnP {
  const void* q; int64_t q_bs, q_rs;
  const int32_t* idx; int64_t idx_bs, idx_rs;
  const void* kc; const void* vc; int64_t kc_bs, kc_rs, vc_bs, vc_rs;
  const void* kh; const void* vh; int64_t kh_bs, kh_rs, vh_bs, vh_rs;
  const void* kr; const void* vr; int64_t kr_bs, kr_rs, vr_bs, vr_rs;
  const int64_t* raw_start; const int64_t* pos0; const float* sink;
  void* o; int64_t o_bs, o_rs;   // o: fp32, or bf16 (round to nearest even) with o_bf16
  int o_bf16;
  float* lse; int64_t lse_bs, lse_rs;
  float* part_o;   // [rows][H][splits][d]: one head's splits contiguous for the merge
  float* part_ml;  // [rows][H][splits][2]
  int tq, heads, dim;
  uint32_t mask;
  int m, mh, W, topk;
  float scale;     // already resolved (never 0)
  const float* q_norm; float norm_eps;  // RMSNorm gain of the queries (null: none)
  int rope; int rope_out; double rope_lb;  // query rotation (R channels), output rotation at -p
  int skv;             // shared entries: the value rows are the key rows (vc/vh/vr alias kc/kh/kr)
  // FP8 caches (f8): every cache holds FP8 E4M3 codes; the row scales, [batch][rows]
  int f8;
  const float *kcs, *vcs, *khs, *vhs, *krs, *vrs;
  int64_t kcs_bs, vcs_bs, khs_bs, vhs_bs, krs_bs, vrs_bs;
  // this launch covers the virtual keys [key_lo, key_hi) of every row, cut into
  // `splits` splits of keys_per_split keys; its partials go to slots
  // split_base .. split_base + splits - 1 of splits_total per row.  With
  // splits_total == 1 the launch writes o and lse directly.
  int64_t key_lo, key_hi;
  int splits, keys_per_split, split_base, splits_total;
  // bf16 launches: heads split into head_groups groups of whole 16-head tiles, one
  // workgroup per (split, group); 1 = every workgroup takes all heads
  int head_groups;
};
hipError_t launch_attn(int dtype, const AttnP& p, int nrows, hipStream_t s, int tid);

// Prefill (tq > 1, bf16, d <= 128, separate K and V): the HCA entries and the window
// of 256 / H consecutive queries per workgroup, streamed once for all of them; each
// row's CSA partial in split slot 0 of p.splits_total (>= 2) joins the result, and
// the rows' o and lse are written.  Grid: (ceil(tq / (256 / H)), batch).
hipError_t launch_attn_qtile(const AttnP& p, int batch, hipStream_t s, int tid);

// fixed_width: always 32 output columns per workgroup (batch-invariant plans: the
// width sets how the splits are grouped in the sum)
hipError_t launch_merge(const AttnP& p, int nrows, bool fixed_width, hipStream_t s, int tid);

// selection of rows [0, n_sel) of sp and bf16 attention of ap ((splits x head
// groups x n_rows) workgroups) in one launch
hipError_t launch_select_attn(const SelectP& sp, int n_sel, const AttnP& ap, int n_rows, hipStream_t s, int tid);

// ---------------------------------------------------------------- HBM read probe
// reads bytes (a multiple of 16) of buf once; sink holds workgroups * 4 words
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s, int tid);

// ---------------------------------------------------------------- timing hooks
// The next (start, stop) event pair of kernel id `tid` while timing is enabled for
// it, else two nulls.  They are recorded on the launch stream right before and right
// after the launch, so they bracket the kernel and its dispatch.  (Events that the
// dispatch packet records itself were tried first: they lengthened the kernel they
// timed by about 2 us and the step by about 0.5 us more than these do.)
void timing_events(int tid, hipEvent_t* start, hipEvent_t* stop);

#define V4A_LAUNCH(TID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                               \
  do {                                                                                        \
    hipEvent_t v4a_e0_, v4a_e1_;                                                              \
    ::v4a::timing_events(TID, &v4a_e0_, &v4a_e1_);                                            \
    if (v4a_e0_) (void)hipEventRecord(v4a_e0_, STREAM);                                        \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                      \
    if (v4a_e1_) (void)hipEventRecord(v4a_e1_, STREAM);                                        \
  } while (0)

}  // namespace v4a
