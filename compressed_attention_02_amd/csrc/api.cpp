// C-ABI entry points of libv4attn: host-side validation, launch planning,
// workspace layout and kernel-timing hooks.  Every argument is checked before the
// first HIP call so that errors are reported synchronously and nothing is enqueued
// on failure.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/v4attn.h"
#include "kernels.hpp"

using namespace v4a;

namespace {

thread_local std::string g_err;

v4a_status fail(v4a_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

v4a_status ok() {
  g_err.clear();
  return V4A_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dtype) { return dtype == V4A_FP8_E4M3 ? 1 : dtype == V4A_BF16 ? 2 : 4; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Compute-unit count of the current device; 256 (MI355X) if it cannot be queried.
int cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return 256; }
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

// Checks a tensor: non-NULL, 16-byte aligned, strides multiples of 16 bytes and row
// stride >= min_row elements.  batch_stride is only used when batch > 1.
v4a_status check_tensor(const char* name, const v4a_tensor& t, int dtype, int64_t min_row, int batch,
                        size_t align = 16) {
  const int64_t es = (int64_t)esize(dtype);
  if (!t.ptr) return fail(V4A_EINVAL, "%s: NULL pointer", name);
  if (!aligned(t.ptr, align)) return fail(V4A_EINVAL, "%s: pointer not %zu-byte aligned", name, align);
  if (t.row_stride < min_row) return fail(V4A_EINVAL, "%s: row_stride %lld < %lld", name, (long long)t.row_stride, (long long)min_row);
  if (align >= 16 && (t.row_stride * es) % 16 != 0) return fail(V4A_EINVAL, "%s: row_stride not a multiple of 16 bytes", name);
  if (batch > 1) {
    if (t.batch_stride <= 0) return fail(V4A_EINVAL, "%s: batch_stride must be positive", name);
    if (align >= 16 && (t.batch_stride * es) % 16 != 0) return fail(V4A_EINVAL, "%s: batch_stride not a multiple of 16 bytes", name);
  }
  return V4A_OK;
}

#define V4A_TRY(expr)              \
  do {                             \
    const v4a_status _s = (expr);  \
    if (_s != V4A_OK) return _s;   \
  } while (0)

v4a_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(V4A_EHIP, "%s: %s", what, hipGetErrorString(e));
  return V4A_OK;
}

// ---------------------------------------------------------------- timing hooks
struct Timing {
  std::vector<hipEvent_t> start, stop;
  int cap = 0, used = 0;
};
std::mutex g_tmu;
Timing g_timing[V4A_K_COUNT];

const char* kKernelNames[V4A_K_COUNT] = {"compress", "index_score", "topk_select", "attn", "merge",
                                          "prefill", "select_attn", "qprep", "read_probe"};

// ---------------------------------------------------------------- plans
// Threshold mode (prefill form): every kThetaStride-th tile is scored first, and a
// per-row threshold from those scores lets most tiles report without rounds and
// store no scores; it needs rows of at least kThetaMinTiles tiles.
constexpr int64_t kThetaStride = 64;
constexpr int64_t kThetaMinTiles = 256;
// workspace bytes of scores and tile reports for one chunk of index rows
constexpr int64_t kScoreBudget = (int64_t)8 << 30;

struct IndexPlan {
  int64_t rows, n_cap, sc_rs, ntiles, key_rs, info_rs, chunk_rows;
  size_t off_keys, off_info, off_theta, off_flag, ws_bytes;
  bool multi;   // score in workgroups of 8 query rows (prefill chunks of a 64 x 64 bf16 indexer)
  bool theta;   // multi, in threshold mode
};

IndexPlan plan_index(const v4a_index_args* a) {
  IndexPlan P{};
  P.rows = (int64_t)a->batch * a->tq;
  P.n_cap = (a->pos_max + 1) / a->ratio;
  P.sc_rs = round_up(std::max<int64_t>(P.n_cap, 1), 64);
  P.ntiles = std::max<int64_t>(1, cdiv(P.n_cap, kTile));
  P.key_rs = round_up(P.ntiles * kTileTop, 64);
  P.info_rs = round_up(P.ntiles, 16);
  // rows are processed in chunks whose scores fit in kScoreBudget (a prefill chunk of
  // 4096 queries at 1M context takes 4.5 GB, one chunk: each chunk's launches, the
  // threshold mode's six among them, are paid once)
  const int64_t row_bytes = P.sc_rs * 4 + P.key_rs * 4 + P.info_rs * 16;
  P.chunk_rows = std::max<int64_t>(1, std::min<int64_t>(P.rows, kScoreBudget / row_bytes));
  // queries in groups of 8 share each key tile: a chunk of rows holds whole groups
  P.multi = a->dtype == V4A_BF16 && a->heads == 64 && a->dim == 64 && a->ki_dtype != V4A_FP8_E4M3 &&
            a->tq % 8 == 0 && P.chunk_rows >= 8;
  if (P.multi) P.chunk_rows -= P.chunk_rows % 8;

  // (not when the selected scores are asked for: most tiles store none)
  P.theta = P.multi && P.ntiles >= kThetaMinTiles && !a->sel_scores.ptr;

  P.off_keys = (size_t)round_up(P.chunk_rows * P.sc_rs * 4, 256);
  P.off_info = P.off_keys + (size_t)round_up(P.chunk_rows * P.key_rs * 4, 256);
  P.off_theta = P.off_info + (size_t)round_up(P.chunk_rows * P.info_rs * 16, 256);
  P.off_flag = P.off_theta + (size_t)round_up(P.chunk_rows * 4, 256);
  P.ws_bytes = P.theta ? P.off_flag + (size_t)round_up(P.chunk_rows * 4, 256) : P.off_theta;
  return P;
}

struct AttnPlan {
  int64_t rows, n_keys, splits, kps;
  size_t off_q, ws_bytes;   // off_q: prepared bf16 queries (when qprep), after the partials
  bool fits;                // the split count stays within what the merge takes
  bool qtile;               // prefill: CSA picks per row (slot 0) + HCA/window per query tile (slot 1)
};

// Prefill chunks whose queries share HCA entries and window rows: bf16, rows of up to
// 128 with separate K and V, 32 to 128 heads (two 16-head tiles per wave, 256 / H
// queries per workgroup), the CSA branch and at least one of the others on, no
// batch-invariant plan (a tile's chunking depends on its neighbours' positions).
bool qtile_ok(const v4a_attn_args* a, bool prefill) {
  const int ntq = a->heads / 16;
  return prefill && a->tq > 1 && a->dtype == V4A_BF16 && a->dim <= 128 && !(a->flags & V4A_SHARED_KV) &&
         a->kv_dtype != V4A_FP8_E4M3 && !(a->flags & V4A_BATCH_INVARIANT) && a->heads % 32 == 0 && ntq >= 2 &&
         ntq <= 8 && (a->branch_mask & V4A_CSA) && (a->branch_mask & (V4A_HCA | V4A_SWA));
}

// bf16 queries with a norm gain or a rotation are prepared once per row
// (launch_qprep) into the workspace: rows * heads * dim bf16
bool needs_qprep(const v4a_attn_args* a) { return a->dtype == V4A_BF16 && (a->q_norm || a->rope_dims > 0); }
size_t add_qprep(const v4a_attn_args* a, int64_t rows, size_t& ws_bytes) {
  if (!needs_qprep(a)) return 0;
  const size_t off = (size_t)round_up((int64_t)ws_bytes, 256);
  ws_bytes = off + (size_t)rows * a->heads * a->dim * 2;
  return off;
}

QPrepP qprep_params(const v4a_attn_args* a, const AttnP& p, void* ws, size_t off_q) {
  QPrepP q{};
  q.q = a->q.ptr; q.q_bs = a->q.batch_stride; q.q_rs = a->q.row_stride;
  q.gain = a->q_norm; q.eps = a->norm_eps;
  q.rope = a->rope_dims; q.rope_lb = p.rope_lb;
  q.heads = a->heads; q.dim = a->dim; q.tq = a->tq; q.pos0 = a->pos0;
  q.out = (uint16_t*)((char*)ws + off_q);
  return q;
}

// Points p at the prepared queries (when the queries need it); with launch, also
// launches the prep (else a score launch of the step carries it).
v4a_status prep_queries(const v4a_attn_args* a, AttnP& p, int64_t rows, void* ws, size_t off_q, hipStream_t s,
                        bool launch) {
  if (!needs_qprep(a)) return V4A_OK;
  const QPrepP q = qprep_params(a, p, ws, off_q);
  if (launch) V4A_TRY(hip_check(launch_qprep(q, (int)rows, s, V4A_K_QPREP), "query prep launch"));
  p.q = q.out;
  p.q_rs = (int64_t)a->heads * a->dim;
  p.q_bs = (int64_t)a->tq * p.q_rs;
  p.q_norm = nullptr;
  return V4A_OK;
}

// Splits of the virtual key list: enough (split, row) workgroups to cover the
// chip twice, but at least kMinKeysPerSplit keys each, since every split writes a
// partial of heads * (dim + 2) floats that the merge reads back.
constexpr int64_t kMinKeysPerSplit = 128;
// keys per split of the batch-invariant plans
constexpr int64_t kInvariantKeysPerSplit = 256;

AttnPlan plan_attn(const v4a_attn_args* a, bool prefill = false) {
  AttnPlan P{};
  P.rows = (int64_t)a->batch * a->tq;
  if (qtile_ok(a, prefill)) {
    P.qtile = true;
    P.n_keys = a->topk;
    P.splits = 2;   // slot 0 holds the CSA partial; the query-tile kernel writes o itself
    P.kps = round_up(std::max<int64_t>(a->topk, 1), kAttnChunk);
    P.ws_bytes = (size_t)(P.rows * P.splits * a->heads) * (size_t)(a->dim + 2) * 4 + 256;
    P.off_q = add_qprep(a, P.rows, P.ws_bytes);
    P.fits = true;
    return P;
  }
  const int64_t pmax = a->pos_max;
  P.n_keys = ((a->branch_mask & V4A_CSA) ? a->topk : 0) + ((a->branch_mask & V4A_HCA) ? (pmax + 1) / a->hca_ratio : 0) +
             ((a->branch_mask & V4A_SWA) ? std::min<int64_t>(a->window, pmax + 1) : 0);
  const int64_t target = 2 * (int64_t)cu_count();
  P.splits = 1;
  if (a->flags & V4A_BATCH_INVARIANT) {
    // fixed split size: a query's splits cover the same keys whatever the batch and
    // pos_max (splits past its keys are empty and add exact zeros in the merge)
    P.kps = kInvariantKeysPerSplit;
    P.splits = cdiv(std::max<int64_t>(P.n_keys, 1), P.kps);
    if (P.splits == 1) P.splits = 2;  // the merge's rounding, not the direct write's
  } else if (P.rows < target && P.n_keys > kMinKeysPerSplit) {
    const int64_t per_row = cdiv(target, P.rows);
    P.kps = round_up(cdiv(P.n_keys, per_row), kAttnChunk);
    P.kps = std::max<int64_t>(P.kps, kMinKeysPerSplit);
    P.kps = std::max<int64_t>(P.kps, round_up(cdiv(P.n_keys, kAttnMaxSplits), kAttnChunk));
    P.splits = cdiv(P.n_keys, P.kps);
  }
  if (P.splits <= 1) {
    P.splits = 1;
    P.kps = round_up(std::max<int64_t>(P.n_keys, 1), kAttnChunk);
    P.ws_bytes = 0;
  } else {
    P.ws_bytes = (size_t)(P.rows * P.splits * a->heads) * (size_t)(a->dim + 2) * 4 + 256;
  }
  P.off_q = add_qprep(a, P.rows, P.ws_bytes);
  P.fits = P.splits <= kAttnMaxSplits;
  return P;
}

// ---------------------------------------------------------------- validation
// A row-scale table of FP8 caches: fp32 [batch][rows], one word per row.
v4a_status check_scale(const char* name, const v4a_tensor& t, int batch) {
  if (!t.ptr || !aligned(t.ptr, 4)) return fail(V4A_EINVAL, "%s: NULL or not 4-byte aligned", name);
  if (t.row_stride != 1) return fail(V4A_EINVAL, "%s: row_stride must be 1", name);
  if (batch > 1 && t.batch_stride <= 0) return fail(V4A_EINVAL, "%s: batch_stride must be positive", name);
  return V4A_OK;
}

v4a_status validate_compress(const v4a_compress_args* a) {
  if (!a) return fail(V4A_EINVAL, "args is NULL");
  if (a->abi_version != V4ATTN_ABI_VERSION) return fail(V4A_EINVAL, "abi_version %u != %u", a->abi_version, V4ATTN_ABI_VERSION);
  if (a->dtype != V4A_F32 && a->dtype != V4A_BF16) return fail(V4A_EINVAL, "dtype %d unknown", a->dtype);
  if (a->batch < 0) return fail(V4A_EINVAL, "batch < 0");
  if (a->ratio < 1) return fail(V4A_EINVAL, "ratio must be >= 1");
  if (a->t0 < 0 || a->n < 0) return fail(V4A_EINVAL, "t0 and n must be >= 0");
  if (a->t0 % a->ratio != 0) return fail(V4A_EINVAL, "t0 (%lld) must be a multiple of ratio (%d)", (long long)a->t0, a->ratio);
  if (a->dim < 1) return fail(V4A_EINVAL, "dim must be >= 1");
  if ((a->dim * esize(a->dtype)) % 16 != 0 || a->dim > 512)
    return fail(V4A_ENOTSUP, "dim %d: rows must be a multiple of 16 bytes and dim <= 512", a->dim);
  if (a->rope_dims < 0 || a->rope_dims % 2 != 0 || a->rope_dims > a->dim)
    return fail(V4A_EINVAL, "rope_dims must be even and in [0, dim]");
  if (a->rope_dims > 0 && !(a->rope_base > 0.f && std::isfinite(a->rope_base)))
    return fail(V4A_EINVAL, "rope_base must be finite and > 0");
  if (a->rope_flags & ~V4A_ROPE_V) return fail(V4A_EINVAL, "unknown rope_flags 0x%x", a->rope_flags);
  if ((int64_t)a->ratio * (a->rope_dims / 2) > 4096)
    return fail(V4A_ENOTSUP, "rope: ratio * rope_dims / 2 must be <= 4096");
  if ((a->norm_k || a->norm_v) && !(a->norm_eps >= 0.f && std::isfinite(a->norm_eps)))
    return fail(V4A_EINVAL, "norm_eps must be finite and >= 0");
  if ((a->norm_k && !aligned(a->norm_k, 4)) || (a->norm_v && !aligned(a->norm_v, 4)))
    return fail(V4A_EINVAL, "norm gains must be 4-byte aligned");
  const bool hv = a->v_raw.ptr || a->v_out.ptr;   // else shared K = V entries: K alone
  if (hv && !(a->v_raw.ptr && a->v_out.ptr)) return fail(V4A_EINVAL, "v_raw and v_out must both be set or both be NULL");
  if (!hv && (a->norm_v || (a->rope_flags & V4A_ROPE_V)))
    return fail(V4A_EINVAL, "K-only compression: norm_v must be NULL and rope_flags 0");
  if (a->out_dtype != 0 && a->out_dtype != a->dtype && a->out_dtype != V4A_FP8_E4M3)
    return fail(V4A_EINVAL, "out_dtype %d: 0, dtype or V4A_FP8_E4M3", a->out_dtype);
  const bool f8 = a->out_dtype == V4A_FP8_E4M3;
  if (!f8 && (a->k_scale.ptr || a->v_scale.ptr)) return fail(V4A_EINVAL, "k_scale / v_scale are for an FP8 output only");
  if (f8 && a->dim % 16 != 0) return fail(V4A_ENOTSUP, "FP8 entries: dim must be a multiple of 16");
  if (f8 && !hv && a->v_scale.ptr) return fail(V4A_EINVAL, "K-only compression: v_scale must be NULL");
  if (a->batch == 0 || a->n / a->ratio == 0) return V4A_OK;
  if (!a->raw_start) return fail(V4A_EINVAL, "raw_start is NULL");
  const int odt = f8 ? V4A_FP8_E4M3 : a->dtype;
  V4A_TRY(check_tensor("k_raw", a->k_raw, a->dtype, a->dim, a->batch));
  V4A_TRY(check_tensor("k_out", a->k_out, odt, a->dim, a->batch));
  if (hv) {
    V4A_TRY(check_tensor("v_raw", a->v_raw, a->dtype, a->dim, a->batch));
    V4A_TRY(check_tensor("v_out", a->v_out, odt, a->dim, a->batch));
  }
  if (f8) {
    V4A_TRY(check_tensor("k_scale", a->k_scale, V4A_F32, 1, a->batch, 4));
    if (a->k_scale.row_stride != 1) return fail(V4A_EINVAL, "k_scale: row_stride must be 1");
    if (hv) {
      V4A_TRY(check_tensor("v_scale", a->v_scale, V4A_F32, 1, a->batch, 4));
      if (a->v_scale.row_stride != 1) return fail(V4A_EINVAL, "v_scale: row_stride must be 1");
    }
  }
  if (!a->logits.ptr) return fail(V4A_EINVAL, "logits: NULL pointer");
  if (!aligned(a->logits.ptr, 4)) return fail(V4A_EINVAL, "logits: pointer not 4-byte aligned");
  if (a->logits.row_stride != 1) return fail(V4A_EINVAL, "logits: row_stride must be 1");
  if (a->batch > 1 && a->logits.batch_stride <= 0) return fail(V4A_EINVAL, "logits: batch_stride must be positive");
  return V4A_OK;
}

v4a_status validate_index(const v4a_index_args* a) {
  if (!a) return fail(V4A_EINVAL, "args is NULL");
  if (a->abi_version != V4ATTN_ABI_VERSION) return fail(V4A_EINVAL, "abi_version %u != %u", a->abi_version, V4ATTN_ABI_VERSION);
  if (a->dtype != V4A_F32 && a->dtype != V4A_BF16) return fail(V4A_EINVAL, "dtype %d unknown", a->dtype);
  if (a->batch < 0) return fail(V4A_EINVAL, "batch < 0");
  if (a->tq < 1) return fail(V4A_EINVAL, "tq must be >= 1");
  if (a->heads < 1 || a->dim < 1) return fail(V4A_EINVAL, "heads and dim must be >= 1");
  if (a->ratio < 1) return fail(V4A_EINVAL, "ratio must be >= 1");
  if (a->topk < 1) return fail(V4A_EINVAL, "topk must be >= 1");
  if (a->topk > kMaxTopk) return fail(V4A_ENOTSUP, "topk %d > %d", a->topk, kMaxTopk);
  if (a->pos_max < 0) return fail(V4A_EINVAL, "pos_max must be >= 0");
  if (a->pos_max < (int64_t)a->tq - 1) return fail(V4A_EINVAL, "pos_max must be >= tq - 1");
  if ((a->pos_max + 1) / a->ratio >= ((int64_t)1 << 31) - 1) return fail(V4A_ENOTSUP, "more than 2^31 - 2 blocks");
  if (a->dtype == V4A_BF16) {
    if (!(a->heads == 16 || a->heads == 32 || a->heads == 64 || a->heads == 128))
      return fail(V4A_ENOTSUP, "bf16 indexer: heads must be 16, 32, 64 or 128");
    if (!(a->dim == 32 || a->dim == 64)) return fail(V4A_ENOTSUP, "bf16 indexer: dim must be 32 or 64");
  } else {
    if (a->dim % 4 != 0) return fail(V4A_ENOTSUP, "fp32 indexer: dim must be a multiple of 4");
    if ((int64_t)a->heads * a->dim + a->heads > 16384) return fail(V4A_ENOTSUP, "fp32 indexer: heads*dim too large");
  }
  const int kdt = a->ki_dtype == 0 ? a->dtype : a->ki_dtype;
  if (kdt != a->dtype && !(kdt == V4A_FP8_E4M3 && a->dtype == V4A_BF16))
    return fail(V4A_EINVAL, "ki_dtype %d: 0, dtype, or FP8_E4M3 with a bf16 indexer", a->ki_dtype);
  if (a->batch == 0) return V4A_OK;
  if (!a->pos0) return fail(V4A_EINVAL, "pos0 is NULL");
  V4A_TRY(check_tensor("qi", a->qi, a->dtype, (int64_t)a->heads * a->dim, a->batch));
  V4A_TRY(check_tensor("ki", a->ki, kdt, a->dim, a->batch));
  if (kdt == V4A_FP8_E4M3) {
    if (!a->ki_scale.ptr || !aligned(a->ki_scale.ptr, 4)) return fail(V4A_EINVAL, "ki_scale: NULL or not 4-byte aligned");
    if (a->ki_scale.row_stride != 1) return fail(V4A_EINVAL, "ki_scale: row_stride must be 1");
    if (a->batch > 1 && a->ki_scale.batch_stride <= 0) return fail(V4A_EINVAL, "ki_scale: batch_stride must be positive");
  }
  if (!a->wi.ptr || !aligned(a->wi.ptr, 4)) return fail(V4A_EINVAL, "wi: NULL or not 4-byte aligned");
  if (a->wi.row_stride < a->heads) return fail(V4A_EINVAL, "wi: row_stride < heads");
  if (a->batch > 1 && a->wi.batch_stride <= 0) return fail(V4A_EINVAL, "wi: batch_stride must be positive");
  if (!a->idx.ptr || !aligned(a->idx.ptr, 4)) return fail(V4A_EINVAL, "idx: NULL or not 4-byte aligned");
  if (a->idx.row_stride < a->topk) return fail(V4A_EINVAL, "idx: row_stride < topk");
  if (a->sel_scores.ptr) {
    if (!aligned(a->sel_scores.ptr, 4)) return fail(V4A_EINVAL, "sel_scores: not 4-byte aligned");
    if (a->sel_scores.row_stride < a->topk) return fail(V4A_EINVAL, "sel_scores: row_stride < topk");
  }
  return V4A_OK;
}

v4a_status validate_attn(const v4a_attn_args* a, bool prefill) {
  if (!a) return fail(V4A_EINVAL, "args is NULL");
  if (a->abi_version != V4ATTN_ABI_VERSION) return fail(V4A_EINVAL, "abi_version %u != %u", a->abi_version, V4ATTN_ABI_VERSION);
  if (a->dtype != V4A_F32 && a->dtype != V4A_BF16) return fail(V4A_EINVAL, "dtype %d unknown", a->dtype);
  if (a->out_dtype != V4A_F32 && a->out_dtype != V4A_BF16) return fail(V4A_EINVAL, "out_dtype must be F32 or BF16");
  if (a->batch < 0) return fail(V4A_EINVAL, "batch < 0");
  if (prefill ? a->tq < 1 : a->tq != 1) return fail(V4A_EINVAL, prefill ? "tq must be >= 1" : "decode needs tq == 1");
  if (a->heads < 1 || a->heads > 128) return fail(V4A_ENOTSUP, "heads must be in 1..128");
  if (a->dtype == V4A_BF16 && a->heads % 16 != 0) return fail(V4A_ENOTSUP, "bf16 attention: heads must be a multiple of 16");
  const bool skv = (a->flags & V4A_SHARED_KV) != 0;
  if (a->dim != 64 && a->dim != 128 && a->dim != 512) return fail(V4A_ENOTSUP, "dim must be 64, 128 or 512");
  if (a->dim == 512 && a->dtype == V4A_BF16 && !skv)
    return fail(V4A_ENOTSUP, "bf16 attention at dim 512 needs V4A_SHARED_KV");
  const int kvt = a->kv_dtype == 0 ? a->dtype : a->kv_dtype;   // type of the caches
  const bool f8 = kvt == V4A_FP8_E4M3;
  if (kvt != a->dtype && !(f8 && a->dtype == V4A_BF16))
    return fail(V4A_EINVAL, "kv_dtype %d: 0, dtype, or FP8_E4M3 with bf16 attention", a->kv_dtype);
  if (f8 && !(a->dim <= 128 && !skv) && !(a->dim == 512 && skv))
    return fail(V4A_ENOTSUP, "FP8 caches: separate K and V rows of dim <= 128, or shared entries (V4A_SHARED_KV) of 512");
  if (f8 && skv && (a->vc_scale.ptr || a->vh_scale.ptr || a->vr_scale.ptr))
    return fail(V4A_EINVAL, "V4A_SHARED_KV: vc_scale, vh_scale and vr_scale must be NULL (the key rows' scales serve)");
  if (a->branch_mask == 0 || a->branch_mask > 7) return fail(V4A_EINVAL, "branch_mask must be a non-empty subset of CSA|HCA|SWA");
  if (a->csa_ratio < 1 || a->hca_ratio < 1) return fail(V4A_EINVAL, "compression ratios must be >= 1");
  if (a->window < 0) return fail(V4A_EINVAL, "window must be >= 0");
  if (a->flags & ~(V4A_BATCH_INVARIANT | V4A_ROPE_OUTPUT | V4A_SHARED_KV))
    return fail(V4A_EINVAL, "unknown flags 0x%x", a->flags);
  if (skv && (a->vc.ptr || a->vh.ptr || a->v_raw.ptr))
    return fail(V4A_EINVAL, "V4A_SHARED_KV: vc, vh and v_raw must be NULL (the key rows are the values)");
  if (a->rope_dims < 0 || a->rope_dims % 2 != 0 || a->rope_dims > a->dim)
    return fail(V4A_EINVAL, "rope_dims must be even and in [0, dim]");
  if (a->rope_dims > 0 && !(a->rope_base > 0.f && std::isfinite(a->rope_base)))
    return fail(V4A_EINVAL, "rope_base must be finite and > 0");
  if ((a->flags & V4A_ROPE_OUTPUT) && a->rope_dims == 0) return fail(V4A_EINVAL, "V4A_ROPE_OUTPUT needs rope_dims > 0");
  if (a->q_norm && !(a->norm_eps >= 0.f && std::isfinite(a->norm_eps)))
    return fail(V4A_EINVAL, "norm_eps must be finite and >= 0");
  if (a->q_norm && !aligned(a->q_norm, 16)) return fail(V4A_EINVAL, "q_norm must be 16-byte aligned");
  if (a->branch_mask & V4A_CSA) {
    if (a->topk < 1) return fail(V4A_EINVAL, "topk must be >= 1");
    if (a->topk > kMaxTopk) return fail(V4A_ENOTSUP, "topk %d > %d", a->topk, kMaxTopk);
  }
  if (!std::isfinite(a->scale)) return fail(V4A_EINVAL, "scale must be finite");
  if (a->pos_max < 0 || a->pos_max < (int64_t)a->tq - 1) return fail(V4A_EINVAL, "pos_max must be >= tq - 1 >= 0");
  if (a->batch == 0) return V4A_OK;
  if (!a->pos0) return fail(V4A_EINVAL, "pos0 is NULL");
  const int64_t hd = (int64_t)a->heads * a->dim;
  const int bq = a->batch;
  V4A_TRY(check_tensor("q", a->q, a->dtype, hd, bq));
  V4A_TRY(check_tensor("o", a->o, a->out_dtype, hd, bq));
  if (a->lse.ptr) {
    if (!aligned(a->lse.ptr, 4)) return fail(V4A_EINVAL, "lse: not 4-byte aligned");
    if (a->lse.row_stride < a->heads) return fail(V4A_EINVAL, "lse: row_stride < heads");
  }
  if (a->branch_mask & V4A_CSA) {
    if (!a->idx.ptr || !aligned(a->idx.ptr, 4)) return fail(V4A_EINVAL, "idx: NULL or not 4-byte aligned");
    if (a->idx.row_stride < a->topk) return fail(V4A_EINVAL, "idx: row_stride < topk");
    V4A_TRY(check_tensor("kc", a->kc, kvt, a->dim, bq));
    if (!skv) V4A_TRY(check_tensor("vc", a->vc, kvt, a->dim, bq));
    if (f8) { V4A_TRY(check_scale("kc_scale", a->kc_scale, bq)); if (!skv) V4A_TRY(check_scale("vc_scale", a->vc_scale, bq)); }
  }
  if (a->branch_mask & V4A_HCA) {
    V4A_TRY(check_tensor("kh", a->kh, kvt, a->dim, bq));
    if (!skv) V4A_TRY(check_tensor("vh", a->vh, kvt, a->dim, bq));
    if (f8) { V4A_TRY(check_scale("kh_scale", a->kh_scale, bq)); if (!skv) V4A_TRY(check_scale("vh_scale", a->vh_scale, bq)); }
  }
  if ((a->branch_mask & V4A_SWA) && a->window > 0) {
    V4A_TRY(check_tensor("k_raw", a->k_raw, kvt, a->dim, bq));
    if (!skv) V4A_TRY(check_tensor("v_raw", a->v_raw, kvt, a->dim, bq));
    if (f8) { V4A_TRY(check_scale("kr_scale", a->kr_scale, bq)); if (!skv) V4A_TRY(check_scale("vr_scale", a->vr_scale, bq)); }
    if (!a->raw_start) return fail(V4A_EINVAL, "raw_start is NULL");
  }
  if (a->sink && !aligned(a->sink, 4)) return fail(V4A_EINVAL, "sink: not 4-byte aligned");
  // the kernels form cache row offsets from 32-bit row strides
  const v4a_tensor* caches[] = {&a->kc, &a->vc, &a->kh, &a->vh, &a->k_raw, &a->v_raw};
  for (const v4a_tensor* t : caches)
    if (t->ptr && t->row_stride > INT32_MAX) return fail(V4A_ENOTSUP, "cache row strides must be < 2^31 elements");
  return V4A_OK;
}

v4a_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return V4A_OK;
  if (!ws) return fail(V4A_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned(ws, 256)) return fail(V4A_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(V4A_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return V4A_OK;
}

// Fewest head groups the attention kernel needs: bf16 rows of 512 take at most
// kWideTiles 16-head tiles per workgroup (a wave pair each); otherwise one.
int min_head_groups(const v4a_attn_args* a) {
  if (a->dtype != V4A_BF16 || a->dim <= 128) return 1;
  const int ntile = std::max(1, a->heads / 16);
  int hg = (ntile + kWideTiles - 1) / kWideTiles;
  while (ntile % hg != 0) ++hg;
  return hg;
}

AttnP make_attn_params(const v4a_attn_args* a, const AttnPlan& P, void* ws) {
  AttnP p{};
  p.head_groups = min_head_groups(a);
  p.q = a->q.ptr; p.q_bs = a->q.batch_stride; p.q_rs = a->q.row_stride;
  p.idx = (const int32_t*)a->idx.ptr; p.idx_bs = a->idx.batch_stride; p.idx_rs = a->idx.row_stride;
  p.kc = a->kc.ptr; p.kc_bs = a->kc.batch_stride; p.kc_rs = a->kc.row_stride;
  p.vc = a->vc.ptr; p.vc_bs = a->vc.batch_stride; p.vc_rs = a->vc.row_stride;
  p.kh = a->kh.ptr; p.kh_bs = a->kh.batch_stride; p.kh_rs = a->kh.row_stride;
  p.vh = a->vh.ptr; p.vh_bs = a->vh.batch_stride; p.vh_rs = a->vh.row_stride;
  p.kr = a->k_raw.ptr; p.kr_bs = a->k_raw.batch_stride; p.kr_rs = a->k_raw.row_stride;
  p.vr = a->v_raw.ptr; p.vr_bs = a->v_raw.batch_stride; p.vr_rs = a->v_raw.row_stride;
  p.skv = (a->flags & V4A_SHARED_KV) != 0;
  p.f8 = a->kv_dtype == V4A_FP8_E4M3;
  if (p.f8) {
    p.kcs = (const float*)a->kc_scale.ptr; p.kcs_bs = a->kc_scale.batch_stride;
    p.vcs = (const float*)a->vc_scale.ptr; p.vcs_bs = a->vc_scale.batch_stride;
    p.khs = (const float*)a->kh_scale.ptr; p.khs_bs = a->kh_scale.batch_stride;
    p.vhs = (const float*)a->vh_scale.ptr; p.vhs_bs = a->vh_scale.batch_stride;
    p.krs = (const float*)a->kr_scale.ptr; p.krs_bs = a->kr_scale.batch_stride;
    p.vrs = (const float*)a->vr_scale.ptr; p.vrs_bs = a->vr_scale.batch_stride;
  }
  if (p.skv) {  // every entry is its own value
    p.vc = p.kc; p.vc_bs = p.kc_bs; p.vc_rs = p.kc_rs;
    p.vh = p.kh; p.vh_bs = p.kh_bs; p.vh_rs = p.kh_rs;
    p.vr = p.kr; p.vr_bs = p.kr_bs; p.vr_rs = p.kr_rs;
  }
  p.raw_start = a->raw_start; p.pos0 = a->pos0; p.sink = a->sink;
  p.o = a->o.ptr; p.o_bs = a->o.batch_stride; p.o_rs = a->o.row_stride;
  p.o_bf16 = a->out_dtype == V4A_BF16;
  p.lse = (float*)a->lse.ptr; p.lse_bs = a->lse.batch_stride; p.lse_rs = a->lse.row_stride;
  p.tq = a->tq; p.heads = a->heads; p.dim = a->dim;
  p.mask = a->branch_mask;
  if (!(a->window > 0)) p.mask &= ~V4A_SWA;
  p.m = a->csa_ratio; p.mh = a->hca_ratio; p.W = a->window; p.topk = a->topk;
  p.scale = a->scale != 0.f ? a->scale : 1.0f / std::sqrt((float)a->dim);
  p.q_norm = a->q_norm; p.norm_eps = a->norm_eps;
  p.rope = a->rope_dims; p.rope_out = (a->flags & V4A_ROPE_OUTPUT) != 0;
  p.rope_lb = a->rope_dims > 0 ? std::log2((double)a->rope_base) : 0.0;
  p.key_lo = 0; p.key_hi = INT64_MAX;
  p.splits = (int)P.splits; p.keys_per_split = (int)P.kps;
  p.split_base = 0; p.splits_total = (int)P.splits;
  if (P.splits > 1) {
    p.part_o = (float*)ws;
    p.part_ml = p.part_o + (size_t)P.rows * P.splits * a->heads * a->dim;
  }
  return p;
}

v4a_status run_attn(const v4a_attn_args* a, void* ws, size_t ws_bytes, hipStream_t s, bool prefill) {
  V4A_TRY(validate_attn(a, prefill));
  if (a->batch == 0) return ok();
  const AttnPlan P = plan_attn(a, prefill);
  if (!P.fits)
    return fail(V4A_ENOTSUP, "%lld key splits per query exceed the merge's %d (batch-invariant plans split every 256 keys)",
                (long long)P.splits, kAttnMaxSplits);
  if (P.rows > 65535 * 1024LL) return fail(V4A_ENOTSUP, "launch too large");
  V4A_TRY(check_ws(ws, ws_bytes, P.ws_bytes));
  AttnP p = make_attn_params(a, P, ws);
  V4A_TRY(prep_queries(a, p, P.rows, ws, P.off_q, s, true));
  const int kid = prefill ? V4A_K_PREFILL : V4A_K_ATTN;
  if (P.qtile) {
    // the CSA picks of every row in one split (partials in slot 0 of 2), then the HCA
    // entries and the window per query tile, which join that partial and write o
    AttnP csa = p, rest = p;
    csa.key_lo = 0;
    csa.key_hi = a->topk;
    csa.splits = 1;
    rest.split_base = 1;
    V4A_TRY(hip_check(launch_attn(a->dtype, csa, (int)P.rows, s, kid), "attention launch"));
    V4A_TRY(hip_check(launch_attn_qtile(rest, a->batch, s, kid), "query-tile attention launch"));
  } else {
    V4A_TRY(hip_check(launch_attn(a->dtype, p, (int)P.rows, s, kid), "attention launch"));
  }
  if (P.splits > 1 && !P.qtile) {
    const bool inv = (a->flags & V4A_BATCH_INVARIANT) != 0;
    V4A_TRY(hip_check(launch_merge(p, (int)P.rows, inv, s, V4A_K_MERGE), "merge launch"));
  }
  return ok();
}

// Launch parameters of v4attn_index_topk (arguments validated, workspace checked).
struct IndexLaunch {
  IndexPlan P;
  ScoreP sp;
  SelectP tp;
};

IndexLaunch index_launch(const v4a_index_args* a, void* ws) {
  IndexLaunch L{};
  const IndexPlan& P = L.P = plan_index(a);
  char* base = (char*)ws;
  ScoreP& sp = L.sp;
  sp.qi = a->qi.ptr; sp.wi = (const float*)a->wi.ptr; sp.ki = a->ki.ptr; sp.pos0 = a->pos0;
  if (a->ki_dtype == V4A_FP8_E4M3) {
    sp.ki_scale = (const float*)a->ki_scale.ptr;
    sp.ks_bs = a->ki_scale.batch_stride;
  }
  sp.scores = (float*)base;
  sp.rep_key = (uint32_t*)(base + P.off_keys);
  sp.rep_info = (uint4*)(base + P.off_info);
  sp.key_rs = P.key_rs;
  sp.info_rs = P.info_rs;
  sp.qi_bs = a->qi.batch_stride; sp.qi_rs = a->qi.row_stride;
  sp.wi_bs = a->wi.batch_stride; sp.wi_rs = a->wi.row_stride;
  sp.ki_bs = a->ki.batch_stride; sp.ki_rs = a->ki.row_stride;
  sp.sc_rs = P.sc_rs;
  sp.tq = a->tq; sp.heads = a->heads; sp.dim = a->dim; sp.ratio = a->ratio;
  // enough workgroups to cover the chip about eight times; a row with more tiles
  // than its share has each workgroup walk several of them
  const int64_t per_row = cdiv(8 * (int64_t)cu_count(), std::min<int64_t>(P.rows, P.chunk_rows));
  sp.wgs_per_row = (int)std::max<int64_t>(1, std::min<int64_t>(P.ntiles, per_row));
  // a 64-block wave of a decode tile report offers 4 candidates when it holds about a
  // quarter of a pick or less (more than 4 of the row's top-k in one wave is then
  // rare, and only costs a rescan), else kTileTop
  const int64_t nvis_max = (a->pos_max + 1) / a->ratio;
  sp.wave_top = (int64_t)a->topk * 64 * 4 <= std::max<int64_t>(nvis_max, 1) ? 4 : kTileTop;
  SelectP& tp = L.tp;
  tp.scores = sp.scores; tp.rep_key = sp.rep_key; tp.rep_info = sp.rep_info; tp.pos0 = a->pos0;
  tp.idx = (int32_t*)a->idx.ptr; tp.idx_bs = a->idx.batch_stride; tp.idx_rs = a->idx.row_stride;
  tp.sel = (float*)a->sel_scores.ptr; tp.sel_bs = a->sel_scores.batch_stride; tp.sel_rs = a->sel_scores.row_stride;
  tp.sc_rs = P.sc_rs; tp.key_rs = P.key_rs; tp.info_rs = P.info_rs; tp.tq = a->tq; tp.ratio = a->ratio; tp.topk = a->topk;
  tp.ntiles_cap = (int)P.ntiles;
  tp.rep_top = P.multi ? kPrefillTileTop : kTileTop;
  return L;
}

v4a_status score_row_chunk(const v4a_index_args* a, IndexLaunch& L, int64_t r0, int nr, hipStream_t stream) {
  L.sp.row0 = (int)r0;
  L.tp.row0 = (int)r0;
  if (L.P.multi) {
    // enough workgroups to cover the chip about four times, each walking tiles
    ScoreP sp = L.sp;
    const int64_t groups = cdiv(nr, 8);
    sp.wgs_per_row = (int)std::max<int64_t>(1, std::min<int64_t>(L.P.ntiles, cdiv(4 * (int64_t)cu_count(), groups)));
    V4A_TRY(hip_check(launch_score_rows(sp, nr, (int)L.P.ntiles, stream, V4A_K_INDEX_SCORE), "index score launch"));
    return V4A_OK;
  }
  V4A_TRY(hip_check(launch_score(a->dtype, L.sp, nr, (int)L.P.ntiles, stream, V4A_K_INDEX_SCORE), "index score launch"));
  return V4A_OK;
}

// Threshold mode for a group of rows: (1) the sampled tiles' scores, (2) each row's
// threshold from them, (3) every tile, reporting its keys at or above the threshold
// when there are at most kTileTop (else its exact best and its scores), (4) the
// selection, which flags rows whose k-th key falls below their threshold, (5, 6) the
// exact score and selection of the flagged rows' groups only.
v4a_status theta_row_chunk(IndexLaunch& L, void* ws, int64_t r0, int nr, hipStream_t stream) {
  ScoreP sp = L.sp;
  SelectP tp = L.tp;
  sp.row0 = tp.row0 = (int)r0;
  uint32_t* theta = (uint32_t*)((char*)ws + L.P.off_theta);
  uint32_t* flag = (uint32_t*)((char*)ws + L.P.off_flag);
  const int64_t groups = cdiv(nr, 8);
  // workgroups per group: the chip about eight times over (a 4096-query chunk: 2048
  // workgroups in four rounds of two per CU; 10.41 against 10.47 ms per chunk with half
  // as many, 10.53 and 10.82 with two and four times as many)
  auto wgs = [&](int64_t walk) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(walk, cdiv(8 * (int64_t)cu_count(), groups)));
  };
  const int64_t nsamp = cdiv(L.P.ntiles, kThetaStride);
  ScoreP s1 = sp;
  s1.sample_stride = (int)kThetaStride;
  s1.wgs_per_row = wgs(nsamp);
  V4A_TRY(hip_check(launch_score_rows(s1, nr, (int)nsamp, stream, V4A_K_INDEX_SCORE), "index sample launch"));
  SelectP t2 = tp;
  t2.sample_stride = (int)kThetaStride;
  t2.theta_out = theta;
  V4A_TRY(hip_check(launch_theta(t2, nr, stream, V4A_K_TOPK_SELECT), "threshold launch"));
  ScoreP s3 = sp;
  s3.theta = theta;
  s3.wgs_per_row = wgs(L.P.ntiles);
  V4A_TRY(hip_check(launch_score_rows(s3, nr, (int)L.P.ntiles, stream, V4A_K_INDEX_SCORE), "index score launch"));
  SelectP t4 = tp;
  t4.theta = theta;
  t4.flag = flag;
  t4.rep_top = kTileTop;
  V4A_TRY(hip_check(launch_select(t4, nr, stream, V4A_K_TOPK_SELECT), "top-k select launch"));
  ScoreP s5 = sp;
  s5.repair = flag;
  s5.wgs_per_row = wgs(L.P.ntiles);
  V4A_TRY(hip_check(launch_score_rows(s5, nr, (int)L.P.ntiles, stream, V4A_K_INDEX_SCORE), "index repair launch"));
  SelectP t6 = tp;
  t6.repair = flag;
  V4A_TRY(hip_check(launch_select(t6, nr, stream, V4A_K_TOPK_SELECT), "top-k repair launch"));
  return V4A_OK;
}

// Scores and selection of v4attn_index_topk on stream (arguments validated).
v4a_status run_index(const v4a_index_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  V4A_TRY(check_ws(ws, ws_bytes, plan_index(a).ws_bytes));   // before any pointer into ws is formed
  IndexLaunch L = index_launch(a, ws);
  for (int64_t r0 = 0; r0 < L.P.rows; r0 += L.P.chunk_rows) {
    const int nr = (int)std::min<int64_t>(L.P.chunk_rows, L.P.rows - r0);
    if (L.P.theta) {
      V4A_TRY(theta_row_chunk(L, ws, r0, nr, stream));
      continue;
    }
    V4A_TRY(score_row_chunk(a, L, r0, nr, stream));
    V4A_TRY(hip_check(launch_select(L.tp, nr, stream, V4A_K_TOPK_SELECT), "top-k select launch"));
  }
  return ok();
}

// ---------------------------------------------------------------- fused decode step
// Key list of a decode row = [CSA picks | HCA entries + window].  The second part
// does not depend on the selection: its splits of kps_rest keys are workgroups of
// the selection's own launch, attended while the selection runs; the CSA picks are
// attended afterwards in one-chunk splits (they sit on the critical path).  Both
// write partials into one [rows][s_rest + s_csa] table, merged once.
struct StepPlan {
  bool csa;
  IndexPlan ix;
  int64_t rows, n_rest, kps_rest, s_rest, s_csa, s_total;
  int hg_rest;   // head groups of the rest's launch (0: the attention's default)
  size_t off_attn, off_q, ws_bytes;
  bool fits;   // the split count stays within what the merge takes
};

StepPlan plan_step(const v4a_index_args* ix, const v4a_attn_args* a) {
  StepPlan P{};
  P.csa = (a->branch_mask & V4A_CSA) != 0;
  P.rows = a->batch;
  const int64_t pmax = a->pos_max;
  P.n_rest = ((a->branch_mask & V4A_HCA) ? (pmax + 1) / a->hca_ratio : 0) +
             ((a->branch_mask & V4A_SWA) && a->window > 0 ? std::min<int64_t>(a->window, pmax + 1) : 0);
  P.s_csa = P.csa ? cdiv(a->topk, kAttnChunk) : 0;
  const bool inv = (a->flags & V4A_BATCH_INVARIANT) != 0;
  if (P.n_rest > 0 && inv) {
    P.kps_rest = kInvariantKeysPerSplit;
    P.s_rest = cdiv(P.n_rest, P.kps_rest);
  } else if (P.n_rest > 0) {
    int64_t per_row = cdiv(2 * (int64_t)cu_count(), P.rows);
    // shared bf16 rows of 512 (one workgroup per CU): workgroups of two head tiles,
    // half what one takes at most, so each reads every chunk from LDS for fewer tiles
    // and writes fewer partials (heads * 514 floats a split: 131 KB at 64 heads), and
    // about one split per CU and head group (a 128-head step at 1M context: 51.0
    // against 52.1 us; with FP8 rows the extra rows each CU then loads cost more than
    // that saves: 71.5 against 67.4 us)
    const int ntile = std::max(1, a->heads / 16);
    if (a->dtype == V4A_BF16 && a->dim == 512 && a->kv_dtype != V4A_FP8_E4M3 && ntile % 2 == 0 && ntile >= 4) {
      P.hg_rest = ntile / 2;
      per_row = std::max<int64_t>(1, (int64_t)cu_count() / (P.rows * P.hg_rest));
    }
    P.kps_rest = std::max<int64_t>(round_up(cdiv(P.n_rest, per_row), kAttnChunk), kMinKeysPerSplit);
    P.kps_rest = std::max<int64_t>(P.kps_rest, round_up(cdiv(P.n_rest, kAttnMaxSplits - P.s_csa), kAttnChunk));
    P.s_rest = cdiv(P.n_rest, P.kps_rest);
  }
  if (P.s_rest + P.s_csa == 0) {  // no key at all: one empty split writes o = 0 (or the sink alone)
    P.s_rest = 1;
    P.kps_rest = kAttnChunk;
  }
  P.s_total = P.s_rest + P.s_csa;
  P.fits = P.s_total <= kAttnMaxSplits;
  if (P.csa) P.ix = plan_index(ix);
  P.off_attn = P.csa ? (size_t)round_up((int64_t)P.ix.ws_bytes, 256) : 0;
  P.ws_bytes = P.off_attn;
  if (P.s_total > 1) P.ws_bytes += (size_t)(P.rows * P.s_total * a->heads) * (size_t)(a->dim + 2) * 4 + 256;
  P.off_q = add_qprep(a, P.rows, P.ws_bytes);
  return P;
}

v4a_status validate_step(const v4a_index_args* ix, const v4a_attn_args* a) {
  V4A_TRY(validate_attn(a, false));
  if (!(a->branch_mask & V4A_CSA)) return V4A_OK;
  if (!ix) return fail(V4A_EINVAL, "index arguments are NULL but the CSA branch is on");
  V4A_TRY(validate_index(ix));
  if (ix->tq != 1) return fail(V4A_EINVAL, "index: tq must be 1 for a decode step");
  if (ix->batch != a->batch || ix->pos0 != a->pos0 || ix->pos_max != a->pos_max)
    return fail(V4A_EINVAL, "index and attention disagree on batch, pos0 or pos_max");
  if (ix->topk != a->topk || ix->ratio != a->csa_ratio)
    return fail(V4A_EINVAL, "index and attention disagree on topk or the CSA ratio");
  if (ix->idx.ptr != a->idx.ptr || ix->idx.row_stride != a->idx.row_stride ||
      (a->batch > 1 && ix->idx.batch_stride != a->idx.batch_stride))
    return fail(V4A_EINVAL, "index and attention must name the same idx buffer with the same strides");
  return V4A_OK;
}

v4a_status run_step(const v4a_index_args* ix, const v4a_attn_args* a, void* ws, size_t ws_bytes, hipStream_t s) {
  V4A_TRY(validate_step(ix, a));
  if (a->batch == 0) return ok();
  const StepPlan P = plan_step(ix, a);
  if (!P.fits)
    return fail(V4A_ENOTSUP, "%lld key splits per query exceed the merge's %d (batch-invariant plans split every 256 keys)",
                (long long)P.s_total, kAttnMaxSplits);
  if (P.rows > 65535 * 1024LL) return fail(V4A_ENOTSUP, "launch too large");
  V4A_TRY(check_ws(ws, ws_bytes, P.ws_bytes));
  AttnPlan AP{};
  AP.rows = P.rows;
  AP.splits = P.s_total;
  AttnP p = make_attn_params(a, AP, nullptr);
  p.splits_total = (int)P.s_total;
  if (P.s_total > 1) {
    p.part_o = (float*)((char*)ws + P.off_attn);
    p.part_ml = p.part_o + (size_t)P.rows * P.s_total * a->heads * a->dim;
  }
  // the selection's launch hosts the rest of the rows' attention when the rows fit
  // one score pass and the attention is bf16; the score launch before it then
  // carries the query prep too
  const bool combined = P.csa && a->dtype == V4A_BF16 && P.s_rest > 0 && P.ix.chunk_rows >= P.ix.rows;
  V4A_TRY(prep_queries(a, p, P.rows, ws, P.off_q, s, !combined));
  // batch-invariant plans put the CSA slots first, so that the rest's split count
  // (from pos_max) only appends empty slots at the end of the merge order
  const bool inv = (a->flags & V4A_BATCH_INVARIANT) != 0;
  AttnP rest = p, csa = p;
  rest.key_lo = P.csa ? a->topk : 0;
  rest.key_hi = INT64_MAX;
  rest.splits = (int)P.s_rest;
  rest.keys_per_split = (int)P.kps_rest;
  if (P.hg_rest > 0) rest.head_groups = P.hg_rest;
  rest.split_base = inv ? (int)P.s_csa : 0;
  csa.key_lo = 0;
  csa.key_hi = a->topk;
  csa.splits = (int)P.s_csa;
  csa.keys_per_split = kAttnChunk;
  csa.split_base = inv ? 0 : (int)P.s_rest;
  // the picks' launch is short and on the critical path: head groups cut the queries
  // each workgroup reads and the partials it writes; the smallest groups (one 16-head
  // tile) while the launch stays within half a workgroup per CU (measured: batch 1 at
  // 128 heads keeps one-tile groups, 128 workgroups; batch 8 at 64 heads takes groups of
  // four tiles, 128 workgroups: 40.75 against 41.3 us per step with two-tile groups)
  if (a->dtype == V4A_BF16 && P.s_csa > 0) {
    const int ntile = std::max(1, a->heads / 16);
    const int hmin = min_head_groups(a);
    int hg = ntile;
    while (!inv && hg > hmin && (ntile % hg != 0 || P.rows * P.s_csa * hg > cu_count() / 2)) --hg;
    csa.head_groups = hg;
  }
  // the rest's launch also hosts the selection: with eight or more head tiles its
  // workgroups take half of them each, so that the rest's attention (every chunk
  // read from LDS once per head tile) ends with the selection rather than after it
  if (combined && a->dim <= 128 && a->heads >= 128 && (a->heads / 16) % 2 == 0) rest.head_groups = 2;

  auto attend = [&](const AttnP& ap) -> v4a_status {
    V4A_TRY(hip_check(launch_attn(a->dtype, ap, (int)P.rows, s, V4A_K_ATTN), "attention launch"));
    return V4A_OK;
  };
  if (P.csa) {
    if (combined) {
      // selection and the selection-independent attention share one launch
      IndexLaunch IL = index_launch(ix, ws);
      if (needs_qprep(a)) {
        IL.sp.prep = qprep_params(a, p, ws, P.off_q);
        IL.sp.prep_x = qprep_blocks(IL.sp.prep);
      }
      V4A_TRY(score_row_chunk(ix, IL, 0, (int)IL.P.rows, s));
      V4A_TRY(hip_check(launch_select_attn(IL.tp, (int)IL.P.rows, rest, (int)P.rows, s, V4A_K_SELECT_ATTN),
                        "select+attention launch"));
    } else {
      V4A_TRY(run_index(ix, ws, P.ix.ws_bytes, s));
      if (P.s_rest > 0) V4A_TRY(attend(rest));
    }
    V4A_TRY(attend(csa));
  } else {
    V4A_TRY(attend(rest));
  }
  if (P.s_total > 1) {
    V4A_TRY(hip_check(launch_merge(p, (int)P.rows, inv, s, V4A_K_MERGE), "merge launch"));
  }
  return ok();
}

}  // namespace

// ---------------------------------------------------------------- static scratch
// The workspace of v4attn_decode_step_noalloc: one array per device, held from the
// library's load until the process ends.  In host code its name is only a symbol;
// its device address (per device) comes from hipGetSymbolAddress, taken once per
// device with that device current, and is what the kernels get.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
v4a_status scratch_ptr(void** out) {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = 0;
  V4A_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  std::lock_guard<std::mutex> lk(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    V4A_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(V4A_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return V4A_OK;
}
}  // namespace

// ---------------------------------------------------------------- timing (namespace v4a)
namespace v4a {
void timing_events(int k, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (k < 0 || k >= V4A_K_COUNT) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  Timing& t = g_timing[k];
  if (t.used < t.cap) {
    *start = t.start[t.used];
    *stop = t.stop[t.used++];
  }
}
}  // namespace v4a

// ---------------------------------------------------------------- C ABI
extern "C" {

uint32_t v4attn_abi_version(void) { return V4ATTN_ABI_VERSION; }

const char* v4attn_status_string(v4a_status s) {
  switch (s) {
    case V4A_OK: return "ok";
    case V4A_EINVAL: return "invalid argument";
    case V4A_ENOTSUP: return "unsupported shape or combination";
    case V4A_EWORKSPACE: return "workspace missing or too small";
    case V4A_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* v4attn_last_error(void) { return g_err.c_str(); }

const char* v4attn_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < V4A_K_COUNT) ? kKernelNames[kernel] : "";
}

v4a_status v4attn_compress(const v4a_compress_args* a, hipStream_t stream) {
  V4A_TRY(validate_compress(a));
  const int64_t nb = a->n / a->ratio;
  if (a->batch == 0 || nb == 0) return ok();
  CompressP p{};
  p.k_raw = a->k_raw.ptr; p.v_raw = a->v_raw.ptr; p.logits = (const float*)a->logits.ptr;
  p.k_out = a->k_out.ptr; p.v_out = a->v_out.ptr; p.raw_start = a->raw_start;
  p.kr_bs = a->k_raw.batch_stride; p.kr_rs = a->k_raw.row_stride;
  p.vr_bs = a->v_raw.batch_stride; p.vr_rs = a->v_raw.row_stride;
  p.lg_bs = a->logits.batch_stride;
  p.ko_bs = a->k_out.batch_stride; p.ko_rs = a->k_out.row_stride;
  p.vo_bs = a->v_out.batch_stride; p.vo_rs = a->v_out.row_stride;
  p.t0 = a->t0; p.nb = nb; p.r = a->ratio; p.d = a->dim;
  p.ch = (int)(a->dim * esize(a->dtype) / 16);
  p.g = std::max(1, std::min(a->ratio, 256 / p.ch));
  p.bpw = std::max(1, 256 / (p.ch * p.g));
  p.gk = a->norm_k; p.gv = a->norm_v; p.eps = a->norm_eps;
  p.rope = a->rope_dims; p.rope_v = (a->rope_flags & V4A_ROPE_V) != 0;
  p.rope_lb = a->rope_dims > 0 ? std::log2((double)a->rope_base) : 0.0;
  p.f8out = a->out_dtype == V4A_FP8_E4M3;
  p.ks_out = (float*)a->k_scale.ptr; p.vs_out = (float*)a->v_scale.ptr;
  p.kso_bs = a->k_scale.batch_stride; p.vso_bs = a->v_scale.batch_stride;
  if (cdiv(nb, p.bpw) > INT32_MAX || a->batch > 65535) return fail(V4A_ENOTSUP, "launch too large");
  V4A_TRY(hip_check(launch_compress(a->dtype, p, a->batch, stream, V4A_K_COMPRESS), "compress launch"));
  return ok();
}

size_t v4attn_index_topk_workspace(const v4a_index_args* a) {
  if (validate_index(a) != V4A_OK || a->batch == 0) return 0;
  return plan_index(a).ws_bytes;
}

v4a_status v4attn_index_topk(const v4a_index_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  V4A_TRY(validate_index(a));
  return run_index(a, ws, ws_bytes, stream);
}

size_t v4attn_decode_workspace(const v4a_attn_args* a) {
  if (validate_attn(a, false) != V4A_OK || a->batch == 0) return 0;
  const AttnPlan P = plan_attn(a);
  return P.fits ? P.ws_bytes : 0;
}

v4a_status v4attn_decode(const v4a_attn_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_attn(a, ws, ws_bytes, stream, false);
}

size_t v4attn_decode_step_workspace(const v4a_index_args* ix, const v4a_attn_args* a) {
  if (validate_step(ix, a) != V4A_OK || a->batch == 0) return 0;
  const StepPlan P = plan_step(ix, a);
  return P.fits ? P.ws_bytes : 0;
}

v4a_status v4attn_decode_step(const v4a_index_args* ix, const v4a_attn_args* a, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  return run_step(ix, a, ws, ws_bytes, stream);
}

v4a_status v4attn_decode_step_noalloc(const v4a_index_args* ix, const v4a_attn_args* a, hipStream_t stream) {
  V4A_TRY(validate_step(ix, a));
  if (a->batch == 0) return ok();
  const StepPlan P = plan_step(ix, a);
  if (P.fits && P.ws_bytes > kScratchBytes)
    return fail(V4A_ENOTSUP, "the step needs %zu bytes of scratch, more than the %zu this entry point holds",
                P.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  V4A_TRY(scratch_ptr(&ws));
  return run_step(ix, a, ws, kScratchBytes, stream);
}

size_t v4attn_prefill_chunk_workspace(const v4a_attn_args* a) {
  if (validate_attn(a, true) != V4A_OK || a->batch == 0) return 0;
  const AttnPlan P = plan_attn(a, true);
  return P.fits ? P.ws_bytes : 0;
}

size_t v4attn_workspace_size(int op, const void* args) {
  if (!args) return 0;
  switch (op) {
    case V4A_OP_COMPRESS: return 0;
    case V4A_OP_INDEX_TOPK: return v4attn_index_topk_workspace(static_cast<const v4a_index_args*>(args));
    case V4A_OP_DECODE: return v4attn_decode_workspace(static_cast<const v4a_attn_args*>(args));
    case V4A_OP_PREFILL_CHUNK: return v4attn_prefill_chunk_workspace(static_cast<const v4a_attn_args*>(args));
    case V4A_OP_DECODE_STEP: {
      const v4a_step_args* st = static_cast<const v4a_step_args*>(args);
      return v4attn_decode_step_workspace(st->index, st->attn);
    }
  }
  return 0;
}

v4a_status v4attn_prefill_chunk(const v4a_attn_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_attn(a, ws, ws_bytes, stream, true);
}

v4a_status v4attn_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4)) return fail(V4A_EINVAL, "buf / sink NULL or misaligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(V4A_EINVAL, "bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(V4A_EINVAL, "workgroups out of range");
  V4A_TRY(hip_check(launch_read_probe(buf, bytes, sink, workgroups, stream, V4A_K_READ_PROBE), "read probe launch"));
  return ok();
}

v4a_status v4attn_timing_enable(int kernel, int max_launches) {
  if (kernel < 0 || kernel >= V4A_K_COUNT) return fail(V4A_EINVAL, "unknown kernel id %d", kernel);
  if (max_launches < 0 || max_launches > (1 << 20)) return fail(V4A_EINVAL, "max_launches out of range");
  std::lock_guard<std::mutex> lk(g_tmu);
  Timing& t = g_timing[kernel];
  for (hipEvent_t e : t.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t.stop) (void)hipEventDestroy(e);
  t.start.assign(max_launches, nullptr);
  t.stop.assign(max_launches, nullptr);
  t.cap = 0;
  t.used = 0;
  for (int n = 0; n < max_launches; ++n) {
    if (hipEventCreate(&t.start[n]) != hipSuccess || hipEventCreate(&t.stop[n]) != hipSuccess)
      return fail(V4A_EHIP, "hipEventCreate failed");
    t.cap = n + 1;
  }
  return ok();
}

int v4attn_timing_read(int kernel, float* ms, int cap) {
  if (kernel < 0 || kernel >= V4A_K_COUNT || (cap > 0 && !ms)) return -1;
  std::lock_guard<std::mutex> lk(g_tmu);
  Timing& t = g_timing[kernel];
  const int n = std::min(t.used, cap);
  for (int k = 0; k < n; ++k) {
    if (hipEventSynchronize(t.stop[k]) != hipSuccess) return -1;
    float v = 0.f;
    if (hipEventElapsedTime(&v, t.start[k], t.stop[k]) != hipSuccess) return -1;
    ms[k] = v;
  }
  return n;
}

void v4attn_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (Timing& t : g_timing) {
    for (hipEvent_t e : t.start) (void)hipEventDestroy(e);
    for (hipEvent_t e : t.stop) (void)hipEventDestroy(e);
    t.start.clear();
    t.stop.clear();
    t.cap = t.used = 0;
  }
}

}  // extern "C"
