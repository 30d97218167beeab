"""Layer configurations of the hybrid compressed-attention layer.

A configuration fixes every concrete choice the source pages leave open: the
arithmetic type, batch, query position, head counts and sizes, the two
compression ratios (CSA m, HCA m'), the indexer shape, top-k and the sliding
window, which branches are on, how many planted needles the inputs carry and
what the timed step compresses.

Pages (the structure only): QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开",
section 混合注意力机制 (CSA steps, HCA m' = 128, the 128-token window); yage.ai essay on
V4's agentic workload, section on the three tiers (k = 1024 Pro / 512 Flash, W = 128);
aperture-daq wiki "DeepSeek-V4 Preview", section on the CSA/HCA dual track (4:1 and 128:1).

This module holds no arithmetic of the method; it only describes shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

CSA = 1
HCA = 2
SWA = 4


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str            # "f32" or "bf16": type of Q, K, V, indexer q/k and caches
    batch: int            # B sequences
    pos: int              # absolute position of the (first) query token
    tq: int               # query tokens per sequence (1 = decode)
    heads: int            # H query heads
    dim: int              # d, head dim of Q and of the single shared KV head
    idx_heads: int        # H_I indexer heads
    idx_dim: int          # d_I indexer head dim
    m: int                # CSA compression ratio
    topk: int             # k selected CSA blocks per query
    m_hca: int            # HCA compression ratio m'
    window: int           # W raw tokens in the sliding window
    branches: int         # bit mask of CSA | HCA | SWA
    needles: int          # planted high-relevance CSA blocks per sequence
    compress: str         # which compression the step runs: "all", "hca_newest", "chunk", "none"
    compress_tokens: int  # tokens compressed by the step (for "hca_newest"/"chunk")
    seed: int
    timed: str            # what one timed step covers
    rho: float = 0.0      # shared-relevance mix of indexer queries (prefill only)
    shared_kv: bool = False  # one tensor per branch: every entry is its own value
    rope_dims: int = 0    # partial RoPE on the last rope_dims channels (0: off)
    q_norm: bool = False  # RMSNorm of each head's query with a synthetic gain
    ki_fp8: bool = False  # indexer keys stored as FP8 E4M3 codes with one fp32 scale per row
    kv_fp8: bool = False  # every K/V cache stored the same way (caches drawn directly)
    # ragged batch (decode steps without compression): sequence b's query sits at
    # pos - pos_back[b % len(pos_back)] instead of pos; () keeps every query at pos
    pos_back: tuple = ()

    # ---- derived shape helpers (pure bookkeeping, no method arithmetic) ----
    @property
    def last_pos(self) -> int:
        return self.pos + self.tq - 1

    @property
    def n_cap(self) -> int:
        """Rows allocated in the CSA caches (indexer keys, Kc, Vc): every block that
        any query of the step can see."""
        return (self.last_pos + 1) // self.m

    @property
    def e_cap(self) -> int:
        return (self.last_pos + 1) // self.m_hca

    def seq_pos(self, b: int) -> int:
        """Position of sequence b's (first) query."""
        return self.pos - (self.pos_back[b % len(self.pos_back)] if self.pos_back else 0)

    def seq_raw_start(self, b: int) -> int:
        """Absolute position of raw row 0 of sequence b (its own window start in a
        ragged batch; raw_start otherwise)."""
        if not self.pos_back:
            return self.raw_start
        return max(0, self.seq_pos(b) - self.window + 1)

    @property
    def raw_start(self) -> int:
        """Absolute position of raw row 0 of each sequence's raw K/V buffer."""
        lo = max(0, self.pos - self.window + 1)
        if self.compress == "all":
            lo = 0
        elif self.compress in ("hca_newest", "chunk"):
            lo = min(lo, self.compress_t0)
        return lo

    @property
    def raw_rows(self) -> int:
        return self.last_pos + 1 - self.raw_start

    @property
    def compress_t0(self) -> int:
        if self.compress == "all":
            return 0
        if self.compress == "hca_newest":
            return self.pos - self.compress_tokens
        if self.compress == "chunk":
            return self.pos
        return self.pos

    def small(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five configurations.  Positions are 0-based: a context of N tokens is
# positions 0..N-1 and the query sits at N with its own K/V appended there.
C1 = LayerConfig(
    name="c1_tiny_f32", dtype="f32", batch=1, pos=4096, tq=1, heads=8, dim=64,
    idx_heads=4, idx_dim=32, m=4, topk=64, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=8, compress="all", compress_tokens=4096,
    seed=20260001, timed="compress + index_topk + decode")

C2 = LayerConfig(
    name="c2_flash_decode_b8_128k", dtype="bf16", batch=8, pos=131072, tq=1, heads=64,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=512, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=32, compress="none", compress_tokens=0,
    seed=20260002, timed="index_topk + decode")

C3 = LayerConfig(
    name="c3_pro_decode_b1_1m", dtype="bf16", batch=1, pos=1048576, tq=1, heads=128,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="none", compress_tokens=0,
    seed=20260003, timed="index_topk + decode")

C4 = LayerConfig(
    name="c4_hca_decode_b16_1m", dtype="bf16", batch=16, pos=1048576, tq=1, heads=64,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=0, m_hca=128, window=128,
    branches=HCA | SWA, needles=0, compress="hca_newest", compress_tokens=4096,
    seed=20260004, timed="compress(HCA, newest 4096) + decode")

C5 = LayerConfig(
    name="c5_prefill_4096_on_1m", dtype="bf16", batch=1, pos=1048576, tq=4096, heads=64,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="chunk", compress_tokens=4096,
    seed=20260005, timed="compress(chunk) + index_topk(4096) + prefill", rho=0.5)

# The pages' own layer shape: shared K = V entries of c = 512 ([QbitAI] 混合注意力机制,
# CSA step 4 and the partial RoPE paragraph; [wiki] shared-KV MQA), RoPE on the last
# 64 channels, RMS-normalised queries, Pro's 128 heads and k = 1024 at 1M context.
C6 = LayerConfig(
    name="c6_shared_kv_c512_decode_b1_1m", dtype="bf16", batch=1, pos=1048576, tq=1, heads=128,
    dim=512, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="none", compress_tokens=0,
    seed=20260006, timed="index_topk + decode", shared_kv=True, rope_dims=64, q_norm=True)

# C3 with the indexer keys (the step's largest stream) kept in FP8 ([wiki]
# quantization and deployment section: attention in FP8, FP8 caches).
C7 = LayerConfig(
    name="c7_fp8_indexer_decode_b1_1m", dtype="bf16", batch=1, pos=1048576, tq=1, heads=128,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="none", compress_tokens=0,
    seed=20260007, timed="index_topk + decode", ki_fp8=True)

# C7 with every K/V cache in FP8 as well (compressed CSA and HCA entries and the
# window's raw rows).
C8 = LayerConfig(
    name="c8_fp8_caches_decode_b1_1m", dtype="bf16", batch=1, pos=1048576, tq=1, heads=128,
    dim=128, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="none", compress_tokens=0,
    seed=20260008, timed="index_topk + decode", ki_fp8=True, kv_fp8=True)

# The pages' layer shape (C6) with its caches in FP8 as well: the indexer keys and the
# shared entries of 512, each row one scale that serves it as key and as value.
C9 = LayerConfig(
    name="c9_shared_kv_c512_fp8_decode_b1_1m", dtype="bf16", batch=1, pos=1048576, tq=1, heads=128,
    dim=512, idx_heads=64, idx_dim=64, m=4, topk=1024, m_hca=128, window=128,
    branches=CSA | HCA | SWA, needles=64, compress="none", compress_tokens=0,
    seed=20260009, timed="index_topk + decode", shared_kv=True, rope_dims=64, q_norm=True, ki_fp8=True,
    kv_fp8=True)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C6, C7, C8, C9)}
