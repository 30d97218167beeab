"""Seeded synthetic inputs for the hybrid compressed-attention layer.

Both the fp64 CPU oracle's tests and the HIP path draw their inputs from here, so
this module holds none of the method's arithmetic: it only draws random numbers,
rounds them to the storage type and plants a few high-relevance blocks.

Recipe (the same for every configuration):
  * generator: numpy PCG64, seeded with ``cfg.seed`` through a SeedSequence that is
    spawned into one child stream per tensor, in the fixed order of ``_STREAMS``;
  * Q, K, V, indexer q/k and the directly generated compressed caches are N(0,1),
    drawn in fp64 and rounded to the configuration's type (fp32: numpy's
    round-to-nearest-even cast; bf16: fp64 -> fp32 -> bf16, each step RNE).  The
    stored bit patterns are the canonical inputs;
  * pooling logits (one per raw token per branch) are N(0,1) fp32; indexer head
    weights are U(0,1) fp32;
  * planted needles (CSA blocks every query should select): indexer key
    KI_j <- g_j + 3*sqrt(d_I)*u with u the unit vector of sum_h w_h*QI_h of that
    sequence's query (for a prefill chunk, of the chunk-shared part of the indexer
    queries); where the CSA cache is drawn directly, Kc_j <- g + 3*unit(mean_h q_h);
  * for a prefill chunk the indexer queries are QI = sqrt(1-rho^2)*g + rho*s_h with
    s_h shared across the chunk, which keeps every marginal N(0,1);
  * raw K/V exist only for the positions the step touches (window + compressed
    span); the 1M-token history is never materialised, its compressed caches are
    drawn directly.  Caches hold at least one row even when no entry is visible;
  * a ragged batch (decode without compression) puts sequence b's query at
    pos - pos_back[b]; caches are sized for the longest sequence, raw buffers
    start at each sequence's own window;
  * shared K = V configurations draw no V tensor (each entry is its own value);
    with a query RMSNorm its per-channel gain is U(0.5, 1.5) fp32;
  * FP8 indexer keys: each drawn row (needles planted as above) gets the scale
    max|row| / 448 (1 for an all-zero row), stored in fp32, and its codes are
    torch's round-to-nearest-even cast of row / scale to float8_e4m3fn; FP8 K/V
    caches the same, each cache row from its N(0,1) draw (needle nudges included).
"""
from __future__ import annotations

import numpy as np

from .configs import C1, C2, C3, C4, C5, C6, C7, C8, C9, CONFIGS, CSA, HCA, SWA, LayerConfig  # noqa: F401

# appending a stream leaves the earlier ones' draws unchanged
_STREAMS = ("q", "qi", "wi", "ki", "kc", "vc", "kh", "vh", "k_raw", "v_raw",
            "logit_csa", "logit_hca", "needles", "shared", "gq")


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _load(stored: np.ndarray, dtype: str) -> np.ndarray:
    return (bf16_bits_to_f32(stored) if dtype == "bf16" else stored).astype(np.float64)


def _fp8_rows(x64: np.ndarray):
    """FP8 E4M3 codes (uint8) and fp32 per-row scales of the rows of x (last axis)."""
    import torch
    amax = np.abs(x64).max(axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    y = torch.from_numpy(x64 / scale.astype(np.float64)[..., None])
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _store(rng.standard_normal(shape), dtype)


def generate(cfg: LayerConfig, seed: int | None = None) -> dict:
    """Draw one input set for ``cfg``.  Returns a dict of numpy arrays; bf16 tensors
    are uint16 bit patterns, fp32 tensors float32, positions int64."""
    seed = cfg.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    rngs = dict(zip(_STREAMS, (np.random.Generator(np.random.PCG64(s))
                               for s in ss.spawn(len(_STREAMS)))))
    B, Tq, H, d = cfg.batch, cfg.tq, cfg.heads, cfg.dim
    HI, dI = cfg.idx_heads, cfg.idx_dim
    if cfg.pos_back and (cfg.compress != "none" or Tq != 1 or min(cfg.pos_back) < 0):
        raise ValueError("ragged positions: decode steps without compression, pos_back >= 0")
    out: dict = {}
    out["pos"] = np.array([cfg.seq_pos(b) for b in range(B)], dtype=np.int64)
    out["raw_start"] = np.array([cfg.seq_raw_start(b) for b in range(B)], dtype=np.int64)
    out["q"] = _normal(rngs["q"], (B, Tq, H, d), cfg.dtype)

    use_csa = bool(cfg.branches & CSA)
    use_hca = bool(cfg.branches & HCA)
    if use_csa:
        if cfg.rho > 0.0:
            g = rngs["qi"].standard_normal((B, Tq, HI, dI))
            shared = rngs["shared"].standard_normal((B, 1, HI, dI))
            qi64 = np.sqrt(1.0 - cfg.rho ** 2) * g + cfg.rho * shared
        else:
            shared = None
            qi64 = rngs["qi"].standard_normal((B, Tq, HI, dI))
        out["qi"] = _store(qi64, cfg.dtype)
        out["wi"] = rngs["wi"].uniform(0.0, 1.0, (B, Tq, HI)).astype(np.float32)
        ki = rngs["ki"].standard_normal((B, max(cfg.n_cap, 1), dI))
        needles = np.zeros((B, cfg.needles), dtype=np.int64)
        # needles are planted among the blocks every query of the sequence can see
        for b in range(B):
            if cfg.needles == 0:
                break
            first_vis = (cfg.seq_pos(b) + 1) // cfg.m
            needles[b] = np.sort(rngs["needles"].choice(first_vis, cfg.needles, replace=False))
            if shared is not None:
                wbar = out["wi"][b].astype(np.float64).mean(axis=0)
                u = (wbar[:, None] * shared[b, 0]).sum(axis=0)
            else:
                u = (out["wi"][b, 0].astype(np.float64)[:, None] * _load(out["qi"][b, 0], cfg.dtype)).sum(axis=0)
            u /= np.linalg.norm(u)
            ki[b, needles[b]] += 3.0 * np.sqrt(dI) * u
        if cfg.ki_fp8:
            out["ki"], out["ki_scale"] = _fp8_rows(ki)
        else:
            out["ki"] = _store(ki, cfg.dtype)
        out["needles"] = needles
        kc = rngs["kc"].standard_normal((B, max(cfg.n_cap, 1), d))
        vc = None if cfg.shared_kv else rngs["vc"].standard_normal((B, max(cfg.n_cap, 1), d))
        if cfg.compress == "none" and cfg.needles:
            for b in range(B):
                qm = _load(out["q"][b, 0], cfg.dtype).mean(axis=0)
                kc[b, needles[b]] += 3.0 * qm / np.linalg.norm(qm)
        if cfg.kv_fp8:
            out["kc"], out["kc_scale"] = _fp8_rows(kc)
            if not cfg.shared_kv:
                out["vc"], out["vc_scale"] = _fp8_rows(vc)
        else:
            out["kc"] = _store(kc, cfg.dtype)
            if not cfg.shared_kv:
                out["vc"] = _store(vc, cfg.dtype)
    def cache(name, shape):
        if cfg.kv_fp8:
            out[name], out[name + "_scale"] = _fp8_rows(rngs[name].standard_normal(shape))
        else:
            out[name] = _normal(rngs[name], shape, cfg.dtype)
    if use_hca:
        cache("kh", (B, max(cfg.e_cap, 1), d))
        if not cfg.shared_kv:
            cache("vh", (B, max(cfg.e_cap, 1), d))
    cache("k_raw", (B, cfg.raw_rows, d))
    if not cfg.shared_kv:
        cache("v_raw", (B, cfg.raw_rows, d))
    if cfg.q_norm:
        out["gq"] = rngs["gq"].uniform(0.5, 1.5, d).astype(np.float32)
    if cfg.compress != "none":
        out["logit_csa"] = rngs["logit_csa"].standard_normal((B, cfg.raw_rows)).astype(np.float32)
        out["logit_hca"] = rngs["logit_hca"].standard_normal((B, cfg.raw_rows)).astype(np.float32)
    return out


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored inputs (bf16 bit patterns or fp32)."""
    return _load(arr, dtype)
