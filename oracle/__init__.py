"""fp64 CPU oracle of the hybrid compressed-attention layer (CSA + HCA + SWA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this package: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from it; the only thing both sides share is the seeded input generator
(``synth``), which holds none of the method's arithmetic.

Every function is the plain definition, in NumPy fp64, with no blocking, fusion or
reordering beyond what the definition states.  Sources (cited by page title and
section; the pages fix the structure, the layer configuration fixes the choices
they leave open):

* [QbitAI] "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
  CSA step 1 (every m tokens' KV entries are merged into one by learned,
  attention-like weights), step 2 (a light indexer scores every compressed block
  per query token, top-k kept), step 3 (multi-query attention over the selected
  blocks); HCA (m' = 128, no overlap, dense attention over every compressed entry);
  the sliding-window branch over the most recent 128 uncompressed tokens, added
  because compressed attention is strictly causal; the learnable sink logit in the
  softmax denominator.
* [yage] yage.ai essay on V4's agentic workload, section on the three tiers: HCA,
  CSA with k = 1024 (Pro) / 512 (Flash), and a 128-token window, read together.
* [wiki] aperture-daq wiki "DeepSeek-V4 Preview", section on the CSA/HCA dual track:
  4:1 and 128:1 compression, shared-KV MQA.

Readings taken where the pages are silent (each one is listed in the design doc):
pooling = softmax-weighted sum inside each non-overlapping block with one fp32
logit per raw token per branch, shared by K and V; a block is visible to a query at
p iff it is complete, (j+1)*r - 1 <= p; indexer score = sum_h w_h*ReLU(qi_h . ki_j)
with no scale; top-k ties go to the lower block id, k_eff = min(k, n_vis), ids
sorted ascending and padded with -1; the window is positions [p-W+1, p], the query's
own token included; the three branches share one softmax with scale 1/sqrt(d); no
de-duplication between branches.

Every function here is pinned by tests under ``tests/`` against brute force,
closed forms and library routines; nothing in it is "parity unpinned" except the
absolute output values a trained V4 layer would give, which need weights that do
not exist here.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "as_f64", "compress", "index_scores", "topk_select", "attend",
    "decode_keyset", "decode_query", "prefill", "lse_merge", "n_visible", "rms_norm",
    "rope", "compress_entries", "fp8_e4m3_decode", "fp8_rows", "fp8_e4m3_encode", "fp8_quantize_rows",
]


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 stored bits are the high half of an
    IEEE binary32 word whose low half is zero."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def as_f64(arr, dtype: str) -> np.ndarray:
    """fp64 value of a stored tensor; dtype is "bf16" (uint16 bits) or "f32"."""
    if dtype == "bf16":
        return bf16_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def n_visible(p: int, r: int) -> int:
    """Number of compressed entries of ratio r a query at position p may use.
    [QbitAI] 混合注意力机制, sliding-window paragraph: compressed attention is
    strictly causal, so only complete blocks count: block j is visible iff
    (j+1)*r - 1 <= p."""
    return (p + 1) // r


def compress(x_raw: np.ndarray, logits: np.ndarray, raw_start: int, t0: int, n: int,
             r: int) -> tuple[np.ndarray, np.ndarray]:
    """Pool the complete blocks of ratio r inside [t0, t0+n) of one sequence.

    [QbitAI] 混合注意力机制, CSA step 1 and the HCA paragraph (no overlap): block j
    covers positions [j*r, (j+1)*r); its weights are the softmax of the block's
    pooling logits and the compressed entry is the weighted sum of its rows.

    x_raw: [T_raw, d] fp64, row t - raw_start holds position t; logits: [T_raw].
    Returns (block ids [nb], rows [nb, d]) for the floor(n/r) complete blocks.
    """
    if t0 % r != 0:
        raise ValueError("t0 must start a block")
    nb = n // r
    ids = np.arange(t0 // r, t0 // r + nb, dtype=np.int64)
    out = np.zeros((nb, x_raw.shape[1]), dtype=np.float64)
    for bi, j in enumerate(ids):
        lo = j * r - raw_start
        z = np.asarray(logits[lo:lo + r], dtype=np.float64)
        e = np.exp(z - z.max())
        w = e / e.sum()
        out[bi] = w @ x_raw[lo:lo + r]
    return ids, out


def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """RMSNorm along the last axis: x / sqrt(mean(x^2) + eps) * gain.

    [QbitAI] 混合注意力机制, the Q/KV normalization paragraph: before core attention
    both the queries and the KV entries are RMS-normalised (to keep the logits from
    blowing up).  The gain is one value per channel of the last axis.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope(x: np.ndarray, pos, dims: int, base: float) -> np.ndarray:
    """Partial rotary position encoding of the last ``dims`` channels at ``pos``.

    [QbitAI] 混合注意力机制, the partial RoPE paragraph: only the last 64 channels of
    the queries and KV entries are rotated, the rest are left alone.  The rotation
    itself is the usual one (the pages name it, not its form): channel pairs
    (2j, 2j+1) of the rotated part turn by the angle pos * base^(-2j/dims).
    ``pos`` is a scalar or one position per row of x.
    """
    x = np.array(x, dtype=np.float64)
    if dims == 0:
        return x
    d = x.shape[-1]
    lo = d - dims
    j = np.arange(dims // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / dims)
    ang = np.multiply.outer(np.asarray(pos, dtype=np.float64), theta)
    c, s_ = np.cos(ang), np.sin(ang)
    a, b = x[..., lo::2].copy(), x[..., lo + 1::2].copy()
    x[..., lo::2] = a * c - b * s_
    x[..., lo + 1::2] = a * s_ + b * c
    return x


def compress_entries(x_raw, logits, raw_start, t0, n, r, *, gain=None, eps=1e-6, rope_dims=0, rope_base=1e4):
    """Compressed entries with the layer's pre-attention operations.

    Raw rows hold per-token entries already rotated at their own positions (the form
    the window branch attends to).  An entry is pooled in the unrotated frame, then
    RMS-normalised (``rms_norm``, with a gain) and rotated at the position of its
    block's last token, (j+1)*r - 1 (a reading: the pages give entries a position
    but not which one).  Returns (block ids, rows) like ``compress``.
    """
    x = np.asarray(x_raw, dtype=np.float64)
    if rope_dims:
        x = rope(x, -(raw_start + np.arange(x.shape[0])), rope_dims, rope_base)
    ids, out = compress(x, logits, raw_start, t0, n, r)
    if gain is not None:
        out = rms_norm(out, gain, eps)
    if rope_dims:
        out = rope(out, (ids + 1) * r - 1, rope_dims, rope_base)
    return ids, out


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of FP8 E4M3 codes (one sign bit, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 is subnormal, m * 2^-9; the all-ones exponent and
    mantissa is NaN; no infinities), exactly, in fp64.

    [wiki] the quantization and deployment section: the checkpoint keeps attention
    in FP8, and FP8 KV caches serve long contexts.  The pages name the format only
    as FP8; E4M3 is a reading, and so is the cache layout: a row holds codes plus
    one fp32 scale, value = scale * decode(code).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def fp8_rows(codes, scales) -> np.ndarray:
    """Rows of an FP8 cache: scale[j] * decode(codes[j])."""
    return fp8_e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def fp8_e4m3_encode(x) -> np.ndarray:
    """The E4M3 code whose value is nearest to each x (|x| <= 448), and of two equally
    near the one with an even mantissa (last code bit 0): round to nearest even,
    taken as a search over the 127 finite magnitudes that ``fp8_e4m3_decode``
    defines.  The sign bit is x's own (so -0.0 gives 0x80).

    [wiki] the quantization and deployment section (FP8 caches); writing a cache row
    in FP8 is the inverse of reading it, and nearest-even rounding is a reading.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0) or np.any(np.isnan(a)):
        raise ValueError("E4M3 encoding takes finite |x| <= 448")
    mags = fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0..126, ascending
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == mags[hi], hi, pick)
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fp8_quantize_rows(rows) -> tuple[np.ndarray, np.ndarray]:
    """Rows as an FP8 cache stores them: per row the scale max|row| / 448 (the row's
    largest magnitude lands on the largest finite E4M3 value) and the codes of
    row / scale; a row of zeros gets scale 0 and zero codes.  Returns (codes
    [..., d] uint8, scales [...] fp64); ``fp8_rows`` reads them back.

    The pages give no scale rule for their FP8 caches; one scale per row at its
    maximum magnitude is the reading taken.
    """
    x = np.asarray(rows, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale = amax / 448.0
    safe = np.where(scale > 0, scale, 1.0)
    codes = fp8_e4m3_encode(np.clip(x / safe[..., None], -448.0, 448.0))
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def index_scores(qi: np.ndarray, wi: np.ndarray, ki: np.ndarray) -> np.ndarray:
    """Indexer score of every given compressed block for one query token.

    [QbitAI] 混合注意力机制, CSA step 2: a lightweight indexer relates the query to
    each compressed block.  The configuration fixes the form: a ReLU-weighted sum
    over indexer heads, s_j = sum_h w_h * max(0, qi_h . ki_j).

    qi: [H_I, d_I], wi: [H_I], ki: [n, d_I] -> s: [n].
    """
    dots = ki @ qi.T                     # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(wi, dtype=np.float64)


def topk_select(s: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest scores, ties to the lower id, sorted ascending, padded
    with -1 to length k when fewer than k blocks are visible.

    [QbitAI] 混合注意力机制, CSA step 2 (top-k of the indexer scores); [yage] three
    tiers (k = 1024 Pro, 512 Flash).
    """
    n = s.shape[0]
    k_eff = min(k, n)
    order = np.lexsort((np.arange(n), -s))      # primary: score descending; then id
    sel = np.sort(order[:k_eff]).astype(np.int64)
    return np.concatenate([sel, np.full(k - k_eff, -1, dtype=np.int64)])


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
           sink: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """One softmax per head over a key multiset; returns (o [H, d], lse [H]).

    [QbitAI] 混合注意力机制: core attention is multi-query attention (one shared KV
    head); the sink paragraph adds a learnable logit to the denominator only.
    With no key and no sink: o = 0, lse = -inf.

    q: [H, d], keys/values: [n, d], sink: [H] or None.
    """
    H, d = q.shape
    if keys.shape[0] == 0:
        o = np.zeros((H, values.shape[1] if values.ndim == 2 else d))
        lse = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64).copy()
        return o, lse
    logits = scale * (q @ keys.T)                # [H, n]
    M = logits.max(axis=1)
    if sink is not None:
        M = np.maximum(M, np.asarray(sink, dtype=np.float64))
    e = np.exp(logits - M[:, None])
    Z = e.sum(axis=1)
    if sink is not None:
        Z = Z + np.exp(np.asarray(sink, dtype=np.float64) - M)
    o = (e @ values) / Z[:, None]
    return o, M + np.log(Z)


def decode_keyset(p: int, *, branches: int, m: int, m_hca: int, window: int,
                  idx=None, kc=None, vc=None, kh=None, vh=None,
                  k_raw=None, v_raw=None, raw_start: int = 0):
    """Keys and values one query at position p attends to, per branch.

    CSA: the compressed rows named by the selected ids (only ids >= 0);
    HCA: every visible compressed entry 0..e_vis-1 ([QbitAI] HCA paragraph);
    SWA: raw positions max(0, p-W+1)..p ([QbitAI] sliding-window paragraph;
    [yage] the 128-token window).  Returns {"csa": (K, V), "hca": ..., "swa": ...}
    with only the enabled branches.  A branch given without values (vc, vh or v_raw
    None) has shared entries: each one is its own value ([QbitAI] 混合注意力机制, the
    partial RoPE paragraph: the KV entries serve as keys and as values; [wiki]
    shared-KV MQA).
    """
    vc = kc if vc is None else vc
    vh = kh if vh is None else vh
    v_raw = k_raw if v_raw is None else v_raw
    out = {}
    if branches & 1:
        sel = np.asarray(idx, dtype=np.int64)
        sel = sel[sel >= 0]
        if sel.size and sel.max() >= n_visible(p, m):
            raise ValueError("selected block not visible to the query")
        out["csa"] = (kc[sel], vc[sel])
    if branches & 2:
        e_vis = n_visible(p, m_hca)
        out["hca"] = (kh[:e_vis], vh[:e_vis])
    if branches & 4:
        lo = max(0, p - window + 1)
        out["swa"] = (k_raw[lo - raw_start:p + 1 - raw_start], v_raw[lo - raw_start:p + 1 - raw_start])
    return out


def decode_query(q: np.ndarray, p: int, scale: float | None = None, sink=None, q_norm=None,
                 norm_eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 1e4, rope_out: bool = False,
                 **ks):
    """Attention output of one query token: every enabled branch feeds one softmax.

    The configuration fixes the single softmax across CSA, HCA and SWA; [yage]
    three tiers describe the three views (far coarse, relevant blocks fine, recent
    tokens in full) of one query.  With a gain q_norm, each head's query is
    RMS-normalised first (``rms_norm``); with rope_dims it is then rotated at p
    (``rope``).  rope_out rotates the output at -p: [QbitAI] 混合注意力机制, the
    partial RoPE paragraph, since the KV entries are the values too, the output
    would carry absolute positions, and the rotation at -p leaves relative ones.
    """
    d = q.shape[1]
    if q_norm is not None:
        q = rms_norm(q, q_norm, norm_eps)
    if rope_dims:
        q = rope(q, p, rope_dims, rope_base)
    scale = 1.0 / math.sqrt(d) if scale is None or scale == 0.0 else scale
    parts = decode_keyset(p, **ks)
    if parts:
        K = np.concatenate([kv[0] for kv in parts.values()], axis=0)
        V = np.concatenate([kv[1] for kv in parts.values()], axis=0)
    else:
        K = np.zeros((0, d))
        V = np.zeros((0, d))
    o, lse = attend(q, K, V, scale, sink)
    if rope_out and rope_dims:
        o = rope(o, -p, rope_dims, rope_base)
    return o, lse


def prefill(q, pos0: int, idx, *, rows=None, scale=None, sink=None, raw_start: int = 0, q_norm=None,
            norm_eps=1e-6, rope_dims=0, rope_base=1e4, rope_out=False, **caches):
    """Chunked prefill of one sequence: row i is the query at p = pos0 + i and is the
    decode of that query over the caches after the chunk has been compressed.
    q [Tq, H, d], idx [Tq, k]; ``rows`` restricts the rows computed."""
    rows = range(q.shape[0]) if rows is None else rows
    os_, ls_ = [], []
    for i in rows:
        o, lse = decode_query(q[i], pos0 + i, scale=scale, sink=sink, q_norm=q_norm, norm_eps=norm_eps,
                              rope_dims=rope_dims, rope_base=rope_base, rope_out=rope_out,
                              idx=None if idx is None else idx[i], raw_start=raw_start, **caches)
        os_.append(o)
        ls_.append(lse)
    return np.stack(os_), np.stack(ls_)


def lse_merge(parts):
    """Merge softmax results over disjoint key sets: parts is a list of (o, lse) of
    equal shapes.  A part with lse = -inf contributes nothing."""
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])
    M = lses.max(axis=0)
    Mf = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lses - Mf)
    Z = w.sum(axis=0)
    o = sum(w[i][..., None] * parts[i][0] for i in range(len(parts)))
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(Z[..., None] > 0, o / np.where(Z > 0, Z, 1.0)[..., None], 0.0)
        lse = np.where(Z > 0, Mf + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    return o, lse
