/*
 * v4attn — hybrid compressed attention (CSA + HCA + sliding window) for AMD
 * MI355X (gfx950).  C ABI.
 *
 * The layer, as the source pages describe it:
 *   [QbitAI]  "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
 *             CSA merges every m tokens' KV entries into one with learned,
 *             attention-like weights (step 1), scores every compressed block per
 *             query token with a light indexer and keeps the top-k (step 2), runs
 *             multi-query attention over the kept blocks (step 3); HCA merges every
 *             m' = 128 tokens without overlap and attends densely to all entries;
 *             a sliding-window branch over the most recent 128 raw tokens makes up
 *             for the strict causality of compressed blocks; a learnable sink
 *             logit may sit in the softmax denominator.
 *   [yage]    yage.ai essay on V4's agentic workload, section on the three tiers:
 *             k = 1024 (Pro) / 512 (Flash), window 128, all three views per query.
 *   [wiki]    aperture-daq wiki "DeepSeek-V4 Preview", CSA/HCA dual-track section:
 *             4:1 and 128:1 compression, MQA with one shared KV head.
 * The choices the pages leave open are fixed as follows (one softmax over all
 * three branches, scale 1/sqrt(d) by default; pooling = softmax over one fp32 logit
 * per raw token inside each non-overlapping block, shared by K and V; a block is
 * visible to a query at p iff it is complete, (j+1)*r-1 <= p; indexer score
 * s_j = sum_h w_h * ReLU(qi_h . ki_j); top-k ties go to the lower block id; the
 * window is positions [p-W+1, p], the query's own token included).
 *
 * Conventions for every call
 * --------------------------
 *  * Positions are absolute token positions, 0-based.  Compressed rows are
 *    indexed by absolute block id (row j of a ratio-r cache pools positions
 *    [j*r, (j+1)*r)).  Raw K/V rows are indexed by position - raw_start[b].
 *  * A v4a_tensor is a device pointer plus element strides between sequences
 *    (batch_stride) and between rows (row_stride); the innermost dimension is
 *    contiguous.  Pointers must be 16-byte aligned and strides multiples of 16
 *    bytes (8 bf16 / 4 fp32 elements) except where a field says otherwise.
 *  * All pointers are device pointers unless the field says "host".
 *  * Ownership: the caller owns every buffer, including the workspace whose
 *    size v4attn_workspace_size() (or the matching *_workspace() function)
 *    returns.  The library allocates
 *    no device memory, keeps no pointer after a call returns, and holds no state
 *    between calls except a per-device property cache and the optional kernel
 *    timing events (v4attn_timing_*).
 *  * Calls are asynchronous and ordered on the given stream.  Every argument is
 *    validated on the host before any HIP call; on error nothing is launched and
 *    v4attn_last_error() (thread-local) describes the problem.  Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  * Preconditions that are not checked (device data): selected ids are unique
 *    and < n_vis of their query, or -1; caches hold every row a query may read;
 *    raw rows cover the window and the compressed span.
 */
#ifndef V4ATTN_H
#define V4ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define V4ATTN_ABI_VERSION 8u

typedef enum v4a_status {
  V4A_OK = 0,
  V4A_EINVAL = 1,      /* bad argument (NULL, range, alignment, stride, dtype)   */
  V4A_ENOTSUP = 2,     /* valid but unsupported shape or combination            */
  V4A_EWORKSPACE = 3,  /* workspace missing or smaller than *_workspace()      */
  V4A_EHIP = 4         /* a HIP runtime call failed at enqueue                  */
} v4a_status;

/* V4A_FP8_E4M3: v4a_index_args.ki_dtype only (cache rows of FP8 codes with one
 * fp32 scale per row) */
typedef enum v4a_dtype { V4A_F32 = 0, V4A_BF16 = 1, V4A_FP8_E4M3 = 2 } v4a_dtype;

/* branch_mask bits */
#define V4A_CSA 1u
#define V4A_HCA 2u
#define V4A_SWA 4u

typedef struct v4a_tensor {
  void* ptr;
  int64_t batch_stride; /* elements */
  int64_t row_stride;   /* elements */
} v4a_tensor;

/* ---------------------------------------------------------------------------
 * v4attn_compress — pool raw K and V into compressed entries.
 * [QbitAI] 混合注意力机制, CSA step 1 and the HCA paragraph (no overlap).
 * For every complete block j of ratio r inside [t0, t0+n):
 *   w_t = softmax over the block of logits[t];  out_j = sum_t w_t * x_t
 * for x = k_raw and x = v_raw with the same weights.  floor(n/r) blocks
 * (ids t0/r .. t0/r + floor(n/r) - 1) are written to k_out / v_out; a partial
 * tail of fewer than r tokens is left alone (it is the "state" a later call
 * compresses once its block is complete).  Accumulation is fp32; a bf16 store
 * rounds to nearest even.
 *   dtype        F32 or BF16: type of k_raw, v_raw, k_out, v_out
 *   dim          d, a multiple of 16 up to 256 (row size a multiple of 16 bytes)
 *   ratio        r >= 1
 *   t0, n        host; t0 >= 0 is a multiple of r, n >= 0; the same for all sequences
 *   raw_start    [batch] int64: position of raw row 0 of each sequence
 *   k_raw/v_raw  [batch][T_raw][d]; v_raw.ptr and v_out.ptr both NULL pools K
 *                alone (shared K = V entries: [QbitAI] 混合注意力机制, the partial
 *                RoPE paragraph, and [wiki] shared-KV MQA); norm_v must then be
 *                NULL and rope_flags 0
 *   logits       fp32 [batch][T_raw], row_stride must be 1, no alignment needed
 *   k_out/v_out  [batch][N_cap][d] indexed by absolute block id
 *   norm_k/norm_v  fp32 [d] RMSNorm gains or NULL.  [QbitAI] 混合注意力机制,
 *                the Q/KV normalization paragraph: KV entries are RMS-normalised
 *                before core attention; with a gain the pooled entry y is
 *                stored as g * y / sqrt(mean(y^2) + norm_eps) (fp32, then the
 *                store rounding).  norm_eps >= 0, finite.
 *   rope_dims    R, even, 0 <= R <= d (0: off).  [QbitAI] 混合注意力机制, the
 *                partial RoPE paragraph: the last 64 channels of the KV entries
 *                carry a rotary position encoding.  Raw K rows (and raw V rows
 *                when rope_flags & V4A_ROPE_V) are taken as rotated at their own
 *                positions t: channel pairs (d-R+2i, d-R+2i+1) turned by
 *                t * rope_base^(-2i/R).  The entry is pooled in the unrotated
 *                frame, normalised there, and stored rotated at the position of
 *                its block's last token, (j+1)*r - 1.  Angles are reduced in
 *                fp64.  rope_base > 0, finite.
 *   out_dtype    0 (entries stored in dtype) or V4A_FP8_E4M3: FP8 caches
 *                ([wiki] the quantization and deployment section: FP8 KV caches;
 *                the pages give no scale rule).  Each stored entry y (fp32, after
 *                the pooling, the norm and the rotation) becomes one fp32 scale
 *                s = max_c |y_c| / 448 and the E4M3 codes of y / s, each the
 *                nearest finite E4M3 value, ties to the even code; an all-zero
 *                entry gets s = 0 and zero codes.  k_out / v_out then hold uint8
 *                codes [batch][N_cap][d] (strides in bytes, rows 16-byte
 *                aligned, dim a multiple of 16) and k_scale / v_scale the fp32
 *                scales [batch][N_cap] (row_stride 1): the layout the attention
 *                reads with kv_dtype V4A_FP8_E4M3 (value = s * decode(code)).
 *   k_scale/v_scale  fp32 row scales of an FP8 output; v_scale set iff v_out
 *                is; both NULL unless out_dtype is V4A_FP8_E4M3
 * ------------------------------------------------------------------------- */
typedef struct v4a_compress_args {
  uint32_t abi_version;
  int32_t dtype;
  int32_t batch;
  int32_t dim;
  int32_t ratio;
  int32_t reserved0;
  int64_t t0;
  int64_t n;
  const int64_t* raw_start;
  v4a_tensor k_raw, v_raw;
  v4a_tensor logits;
  v4a_tensor k_out, v_out;
  const float* norm_k;
  const float* norm_v;
  float norm_eps;
  int32_t rope_dims;
  float rope_base;
  uint32_t rope_flags;  /* V4A_ROPE_V or 0 */
  int32_t out_dtype;    /* 0 (= dtype) or V4A_FP8_E4M3 */
  int32_t reserved1;
  v4a_tensor k_scale, v_scale;
} v4a_compress_args;

v4a_status v4attn_compress(const v4a_compress_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * v4attn_index_topk — lightning-indexer scores and per-query top-k.
 * [QbitAI] 混合注意力机制, CSA step 2; [yage] three tiers (k = 1024 / 512).
 * For query token i of sequence b at position p = pos0[b] + i and every
 * visible block j < n_vis = floor((p+1)/m):
 *   s_j = sum_h wi[h] * max(0, qi[h] . ki[j])          (fp32 accumulation)
 * idx[b][i] receives the k_eff = min(k, n_vis) ids with the largest s_j (ties
 * to the lower id), sorted ascending, then -1 up to k.  sel_scores (optional)
 * receives s of each written id (0 for padding).
 *   dtype        F32 or BF16: type of qi and ki
 *   heads, dim   H_I and d_I; BF16 needs heads in {16, 32, 64, 128} and
 *                d_I in {32, 64}; F32 needs d_I % 4 == 0 and H_I*(d_I+1) <= 16384
 *   ratio        m >= 1
 *   topk         1 <= k <= 2048
 *   pos0         [batch] int64; pos_max (host) >= pos0[b] + tq - 1 for all b
 *   qi           [batch][tq][H_I][d_I] (row = query token, heads contiguous)
 *   wi           fp32 [batch][tq][H_I] (row = query token); weights should be
 *                >= 0 (the ReLU form assumes it; not checked)
 *   ki           [batch][N_cap][d_I] (row = block id), of type ki_dtype
 *   ki_dtype     0 (the same as dtype) or, with dtype BF16, V4A_FP8_E4M3:
 *                ki holds FP8 E4M3 codes (bytes: sign, 4 exponent bits with
 *                bias 7, 3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN)
 *                and row j of block b stands for ki_scale[b][j] * decode(code),
 *                so the score is s_j = sum_h wi[h] * max(0, ki_scale[b][j] *
 *                (qi[h] . decode(ki[j]))).  [wiki] the quantization and
 *                deployment section (attention kept in FP8, FP8 KV caches); the
 *                E4M3 format and the per-row scale are readings.
 *   ki_scale     fp32 [batch][N_cap], row_stride 1 (ki_dtype FP8 only)
 *   idx          int32 out [batch][tq][k] (row = query token), row_stride >= k
 *   sel_scores   fp32 out, same layout as idx, or ptr == NULL
 * Workspace: v4attn_index_topk_workspace(args) bytes: per query row about
 * 4 * N_cap + 48 * N_cap / 256 bytes of scores and tile reports, for as many
 * rows as fit in 8 GiB at once (larger calls take their rows in groups of that
 * size).  A 4096-query prefill chunk at 1M context needs 4.5 GB, a decode step
 * at 1M context 1.1 MB per row.
 * ------------------------------------------------------------------------- */
typedef struct v4a_index_args {
  uint32_t abi_version;
  int32_t dtype;
  int32_t batch;
  int32_t tq;
  int32_t heads;
  int32_t dim;
  int32_t ratio;
  int32_t topk;
  const int64_t* pos0;
  int64_t pos_max;
  v4a_tensor qi, wi, ki;
  v4a_tensor idx;
  v4a_tensor sel_scores;
  int32_t ki_dtype;     /* 0 (= dtype) or V4A_FP8_E4M3 */
  int32_t reserved0;
  v4a_tensor ki_scale;
} v4a_index_args;

size_t v4attn_index_topk_workspace(const v4a_index_args* args);
v4a_status v4attn_index_topk(const v4a_index_args* args, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * v4attn_decode / v4attn_prefill_chunk — one softmax per query and head over
 *   CSA: rows idx[b][i][*] >= 0 of kc/vc            [QbitAI] CSA step 3
 *   HCA: rows 0 .. floor((p+1)/m')-1 of kh/vh       [QbitAI] HCA paragraph
 *   SWA: raw positions max(0, p-W+1) .. p           [QbitAI] window paragraph
 * with p = pos0[b] + i.  All query heads share the one KV head (MQA).
 *   l = scale * q_h . k ;  o_h = sum e^(l-M) v / Z ;  lse_h = M + ln Z,
 *   Z = sum e^(l-M) (+ e^(sink_h - M) when sink != NULL).
 * A query with no key and no sink gets o = 0, lse = -inf.  Disabled branches
 * (branch_mask) contribute nothing and their pointers may be NULL.
 *   dtype        F32 or BF16: q and every cache; BF16 needs heads % 16 == 0
 *   out_dtype    F32 or BF16: the type of o (bf16 rounds the fp32 result to
 *                nearest even); lse is always fp32
 *   tq           query tokens per sequence: 1 for v4attn_decode, >= 1 for
 *                v4attn_prefill_chunk
 *   heads, dim   H <= 128; d = 64, 128 or 512 (bf16 at 512: V4A_SHARED_KV only)
 *   csa_ratio, hca_ratio, window   m, m' >= 1; W >= 0
 *   topk         k, the row length of idx (CSA only), 1..2048
 *   scale        softmax scale; 0 selects 1/sqrt(d)
 *   pos0         [batch] int64; pos_max (host) >= pos0[b] + tq - 1 for all b
 *   q            [batch][tq][H][d] (row = query token, heads contiguous)
 *   idx          int32 [batch][tq][k], as written by v4attn_index_topk
 *   kc, vc       [batch][N_cap][d]; kh, vh [batch][E_cap][d] (vc, vh, v_raw
 *                NULL with V4A_SHARED_KV)
 *   k_raw, v_raw [batch][T_raw][d]; raw_start [batch] int64
 *   sink         fp32 [H] or NULL
 *   o            out [batch][tq][H][d] (row = query token), of type out_dtype
 *   lse          fp32 out [batch][tq][H] (row = query token) or ptr == NULL
 *   q_norm       fp32 [d], 16-byte aligned: RMSNorm gain for every head's query, or NULL:
 *                q_h is used as g * q_h / sqrt(mean(q_h^2) + norm_eps) ([QbitAI]
 *                混合注意力机制, Q/KV normalization); the bf16 path rounds the
 *                normalised query to bf16.  norm_eps >= 0, finite.
 *   rope_dims    R, even, 0 <= R <= d (0: off): the query (after q_norm) is
 *                rotated at its position p like the entries (see
 *                v4attn_compress); rope_base > 0, finite.  The caches hold
 *                entries already rotated (compress, and the caller's raw rows).
 *   kv_dtype     0 (the caches have type dtype) or, with dtype BF16, d <= 128
 *                and no V4A_SHARED_KV, V4A_FP8_E4M3: every enabled cache (kc,
 *                vc, kh, vh, k_raw, v_raw) holds FP8 E4M3 codes (as in
 *                v4attn_index_topk) and its row r stands for scale[b][r] *
 *                decode(code), the scale from the matching *_scale tensor (fp32
 *                [batch][rows], row_stride 1).  Keys enter the logit and values
 *                the output with their scale; the query stays bf16.  [wiki] the
 *                quantization and deployment section (FP8 KV caches).
 *   flags        V4A_ROPE_OUTPUT (with rope_dims): o's last R channels are
 *                rotated at -p.
 *                V4A_BATCH_INVARIANT: a query's o and lse (and, through
 *                v4attn_decode_step, its idx) depend only on its own sequence's
 *                inputs, bit for bit, not on the other sequences of the batch
 *                nor on pos_max.  Key splits then have a fixed size (256 keys;
 *                64 for the CSA picks of v4attn_decode_step) and the CSA picks'
 *                attention takes one 16-head tile per workgroup.  A query may
 *                then have at most 1024 splits (about 262k keys): larger
 *                pos_max / hca_ratio give V4A_ENOTSUP before anything is
 *                enqueued, and a zero workspace size.
 *                V4A_SHARED_KV: every entry is its own value (v = k in the
 *                formula above), read once; vc, vh and v_raw must be NULL.
 *                [QbitAI] 混合注意力机制, the partial RoPE paragraph (the KV
 *                entries serve as keys and values) and CSA step 4 (head
 *                dimension c = 512); [wiki] shared-KV MQA.  With RoPE the values
 *                carry the rotation too, which V4A_ROPE_OUTPUT takes back out.
 *                Other bits: V4A_EINVAL.
 * The caller appends the query's own K/V to the raw buffers, and for a prefill
 * chunk runs v4attn_compress over the chunk first.
 * Workspace: v4attn_decode_workspace / v4attn_prefill_chunk_workspace.
 * ------------------------------------------------------------------------- */
/* [wiki] the batch-invariance material: results that must not change with
 * the batch a request is served in. */
#define V4A_BATCH_INVARIANT 1u
/* [QbitAI] 混合注意力机制, partial RoPE paragraph: the KV entries are the values
 * too, so the output would carry absolute positions; V4A_ROPE_OUTPUT rotates o
 * at -p (its last rope_dims channels) to keep relative ones only. */
#define V4A_ROPE_OUTPUT 2u
/* v4a_compress_args.rope_flags: raw V rows are rotated too. */
#define V4A_ROPE_V 1u
/* [QbitAI] 混合注意力机制 (the KV entries serve as keys and values; c = 512) and
 * [wiki] shared-KV MQA: the key rows are the values, loaded once. */
#define V4A_SHARED_KV 4u

typedef struct v4a_attn_args {
  uint32_t abi_version;
  int32_t dtype;
  int32_t out_dtype;
  int32_t batch;
  int32_t tq;
  int32_t heads;
  int32_t dim;
  uint32_t branch_mask;
  int32_t csa_ratio;
  int32_t hca_ratio;
  int32_t window;
  int32_t topk;
  float scale;
  uint32_t flags;      /* V4A_BATCH_INVARIANT or 0 */
  const int64_t* pos0;
  int64_t pos_max;
  v4a_tensor q;
  v4a_tensor idx;
  v4a_tensor kc, vc, kh, vh, k_raw, v_raw;
  const int64_t* raw_start;
  const float* sink;
  v4a_tensor o;
  v4a_tensor lse;
  const float* q_norm;
  float norm_eps;
  int32_t rope_dims;
  float rope_base;
  int32_t reserved1;
  int32_t kv_dtype;     /* 0 (= dtype) or V4A_FP8_E4M3 */
  int32_t reserved2;
  v4a_tensor kc_scale, vc_scale, kh_scale, vh_scale, kr_scale, vr_scale;
} v4a_attn_args;

size_t v4attn_decode_workspace(const v4a_attn_args* args);
v4a_status v4attn_decode(const v4a_attn_args* args, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

size_t v4attn_prefill_chunk_workspace(const v4a_attn_args* args);
v4a_status v4attn_prefill_chunk(const v4a_attn_args* args, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * v4attn_decode_step — one decode step of the layer: v4attn_index_topk then
 * v4attn_decode, with the same results (idx bit for bit; o and lse up to
 * rounding, as the key list is split differently).
 * [QbitAI] 混合注意力机制: the HCA and window branches do not depend on the
 * CSA selection, so with a bf16 attention they are attended by the other
 * workgroups of the launch that runs the top-k selection (which needs one
 * workgroup per query row); the CSA keys are attended once the selection is
 * done, and one merge combines both.  Everything runs on `stream`, in order;
 * no workgroup ever waits for another.
 *   index   arguments of v4attn_index_topk with tq == 1; its idx is read by
 *           the attention.  Ignored (may be NULL) when attn has no CSA branch.
 *   attn    arguments of v4attn_decode.  With CSA: batch, pos0 and pos_max
 *           equal index's, topk == index->topk, csa_ratio == index->ratio,
 *           and idx names the same buffer with the same strides.
 * Errors: as the two calls, plus V4A_EINVAL when index and attn disagree.
 * Workspace: v4attn_decode_step_workspace(index, attn) bytes (0 when the
 * arguments are invalid), 256-byte aligned, owned by the caller and not used
 * after the work enqueued on stream completes.
 * ------------------------------------------------------------------------- */
size_t v4attn_decode_step_workspace(const v4a_index_args* index,
                                    const v4a_attn_args* attn);
v4a_status v4attn_decode_step(const v4a_index_args* index,
                              const v4a_attn_args* attn, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * v4attn_decode_step_noalloc — v4attn_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same launches and results as
 * v4attn_decode_step, bit for bit, with the workspace taken from a 64 MiB array
 * the library holds in each device's memory (from its first use on that device
 * until the process ends) instead of from the caller.  The call allocates and
 * frees nothing.  Calls that need more than 64 MiB of workspace (what
 * v4attn_decode_step_workspace returns) get V4A_ENOTSUP, before anything is
 * enqueued.  Every call on a device shares that device's array and leaves its
 * contents behind; no kernel expects it to hold anything on entry.  Calls whose
 * work may overlap on one device (different streams, or different threads
 * without ordering) race on the array and must not be issued.  Otherwise the
 * arguments, errors and ordering are those of v4attn_decode_step.
 * ------------------------------------------------------------------------- */
v4a_status v4attn_decode_step_noalloc(const v4a_index_args* index, const v4a_attn_args* attn, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * v4attn_workspace_size — workspace bytes of one call, by operation.
 *   op    V4A_OP_*; args points to that operation's arguments:
 *         V4A_OP_COMPRESS      v4a_compress_args   (always 0: no workspace)
 *         V4A_OP_INDEX_TOPK    v4a_index_args
 *         V4A_OP_DECODE        v4a_attn_args
 *         V4A_OP_PREFILL_CHUNK v4a_attn_args
 *         V4A_OP_DECODE_STEP   v4a_step_args (the pair v4attn_decode_step takes)
 * Returns 0 for invalid or unsupported arguments, an unknown op or args NULL
 * (the call itself then reports why), and for calls that need no workspace.  The
 * buffer must be 256-byte aligned.  The same as the per-operation
 * *_workspace() functions, which stay for callers that prefer them.
 * ------------------------------------------------------------------------- */
enum {
  V4A_OP_COMPRESS = 0,
  V4A_OP_INDEX_TOPK = 1,
  V4A_OP_DECODE = 2,
  V4A_OP_PREFILL_CHUNK = 3,
  V4A_OP_DECODE_STEP = 4
};
typedef struct v4a_step_args {
  const v4a_index_args* index;   /* may be NULL without the CSA branch */
  const v4a_attn_args* attn;
} v4a_step_args;
size_t v4attn_workspace_size(int op, const void* args);

/* ---------------------------------------------------------------------------
 * Status, version, diagnostics.
 * ------------------------------------------------------------------------- */
const char* v4attn_status_string(v4a_status s);
/* Thread-local text of the last error raised by this thread ("" if none). */
const char* v4attn_last_error(void);
uint32_t v4attn_abi_version(void);

/* ---------------------------------------------------------------------------
 * Kernel timing for benchmarks.  v4attn_timing_enable(kernel, n) makes the
 * library bracket each of the next n launches of that kernel with a pair of
 * events recorded on the launch stream right before and right after it (so
 * the interval holds the kernel and its dispatch; events created here, kept
 * until v4attn_timing_reset).  v4attn_timing_read waits for the recorded events and
 * writes up to cap per-launch durations in milliseconds; it returns the count,
 * or -1 on error.  kernel: one of the V4A_K_* ids.
 * ------------------------------------------------------------------------- */
enum {
  V4A_K_COMPRESS = 0,
  V4A_K_INDEX_SCORE = 1,
  V4A_K_TOPK_SELECT = 2,
  V4A_K_ATTN = 3,
  V4A_K_MERGE = 4,
  V4A_K_PREFILL = 5,
  V4A_K_SELECT_ATTN = 6, /* v4attn_decode_step: selection + HCA/window attention */
  V4A_K_QPREP = 7,       /* bf16 queries normalised / rotated once per row */
  V4A_K_READ_PROBE = 8,  /* v4attn_read_probe */
  V4A_K_COUNT = 9
};
v4a_status v4attn_timing_enable(int kernel, int max_launches);
/* HBM read probe for benchmarks: reads `bytes` (a positive multiple of 16) of the
 * device buffer `buf` (16-byte aligned) once with `workgroups` workgroups of 256
 * threads (16-byte loads at a grid stride), and writes workgroups * 4 words of
 * xor-folded data to `sink` so that no load is dropped.  Timed through
 * V4A_K_READ_PROBE like the kernels above; it gives the streaming rate this GPU
 * reaches, the ceiling the layer's kernels are compared with. */
v4a_status v4attn_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);
int v4attn_timing_read(int kernel, float* ms, int cap);
void v4attn_timing_reset(void);
const char* v4attn_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* V4ATTN_H */
