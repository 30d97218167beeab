"""One step of the hybrid compressed-attention layer on device-resident tensors.

``LayerStep`` strings the four C entry points together in the order a decode or
prefill step needs them (compress the newly complete blocks, score and select CSA
blocks, attend) and keeps the workspaces between calls.  It adds no arithmetic:
everything runs in libv4attn's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import CSA, HCA, SWA, CompressCall, DecodeStepCall, decode, index_topk, prefill_chunk


def to_device(arrays: dict, device="cuda") -> dict:
    """Upload numpy inputs: uint16 arrays are bf16 bit patterns, float32 stays fp32,
    int64 stays int64."""
    import torch
    out = {}
    for k, v in arrays.items():
        if not isinstance(v, np.ndarray):
            continue
        if v.dtype == np.uint16:
            t = torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        out[k] = t
    return out


@dataclass
class LayerShape:
    heads: int
    dim: int
    idx_heads: int
    idx_dim: int
    m: int
    m_hca: int
    window: int
    topk: int
    branches: int
    compress: str          # "all", "hca_newest", "chunk" or "none"
    compress_t0: int
    pos: int               # position of the first query of the step
    tq: int
    shared_kv: bool = False  # every entry is its own value (no V tensors)
    rope_dims: int = 0       # partial RoPE of the query, output rotated back
    rope_base: float = 1e4
    q_norm: bool = False     # RMSNorm of the queries with the gain t["gq"]
    norm_eps: float = 1e-6
    batch_invariant: bool = False  # V4A_BATCH_INVARIANT split plans
    out_bf16: bool = False         # o stored in bf16 (round to nearest even) instead of fp32

    @classmethod
    def of(cls, cfg) -> "LayerShape":
        return cls(cfg.heads, cfg.dim, cfg.idx_heads, cfg.idx_dim, cfg.m, cfg.m_hca, cfg.window,
                   max(cfg.topk, 1), cfg.branches, cfg.compress, cfg.compress_t0, cfg.pos, cfg.tq,
                   shared_kv=cfg.shared_kv, rope_dims=cfg.rope_dims, q_norm=cfg.q_norm)


class LayerStep:
    """Buffers of one step: ``t`` holds the device tensors (inputs and caches, as
    produced by ``to_device``); outputs ``o``/``lse``/``idx`` are allocated here."""

    def __init__(self, shape: LayerShape, t: dict):
        import torch
        self.s = shape
        self.t = t
        B = t["q"].shape[0]
        dev = t["q"].device
        self.B = B
        self.pos_max = shape.pos + shape.tq - 1
        self.o = torch.empty((B, shape.tq, shape.heads, shape.dim),
                             dtype=torch.bfloat16 if shape.out_bf16 else torch.float32, device=dev)
        self.lse = torch.empty((B, shape.tq, shape.heads), dtype=torch.float32, device=dev)
        self.idx = torch.full((B, shape.tq, shape.topk), -1, dtype=torch.int32, device=dev)
        self.ws_index = None
        self.ws_attn = None

    # -- stages -------------------------------------------------------------
    def run_compress(self, stream=None):
        """The step's compress calls (CSA then HCA), marshalled on first use."""
        if getattr(self, "_compress_calls", None) is None:
            self._compress_calls = self._make_compress_calls()
        for call in self._compress_calls:
            call(stream)

    def _make_compress_calls(self):
        s, t = self.s, self.t
        if s.compress == "none":
            return []
        n = self.pos_max + 1 - s.compress_t0
        # with RoPE, raw rows arrive rotated at their positions and entries are stored
        # rotated at their block's last one (shared entries: the values are the keys)
        kw = dict(t0=s.compress_t0, n=n, rope_dims=s.rope_dims, rope_base=s.rope_base)
        calls = []
        if s.branches & CSA and s.compress in ("all", "chunk"):
            calls.append(CompressCall(t["k_raw"], t.get("v_raw"), t["logit_csa"], t["raw_start"], t["kc"],
                                      t.get("vc"), ratio=s.m, **kw))
        if s.branches & HCA:
            calls.append(CompressCall(t["k_raw"], t.get("v_raw"), t["logit_hca"], t["raw_start"], t["kh"],
                                      t.get("vh"), ratio=s.m_hca, **kw))
        return calls

    def run_index(self, stream=None):
        s, t = self.s, self.t
        if not s.branches & CSA:
            return
        self.ws_index = index_topk(t["qi"], t["wi"], t["ki"], t["pos"], self.idx, ratio=s.m, topk=s.topk,
                                   pos_max=self.pos_max, workspace=self.ws_index, stream=stream,
                                   ki_scale=t.get("ki_scale"))

    def attn_kwargs(self):
        s, t = self.s, self.t
        return dict(lse=self.lse, idx=self.idx if s.branches & CSA else None, kc=t.get("kc"), vc=t.get("vc"),
                    kh=t.get("kh"), vh=t.get("vh"), k_raw=t.get("k_raw"), v_raw=t.get("v_raw"),
                    raw_start=t.get("raw_start"), branch_mask=s.branches, csa_ratio=s.m,
                    hca_ratio=s.m_hca, window=s.window, topk=s.topk, pos_max=self.pos_max,
                    shared_kv=s.shared_kv, rope_dims=s.rope_dims, rope_base=s.rope_base,
                    rope_out=s.rope_dims > 0, q_norm=t.get("gq") if s.q_norm else None, norm_eps=s.norm_eps,
                    batch_invariant=s.batch_invariant,
                    kc_scale=t.get("kc_scale"), vc_scale=t.get("vc_scale"), kh_scale=t.get("kh_scale"),
                    vh_scale=t.get("vh_scale"), kr_scale=t.get("k_raw_scale"), vr_scale=t.get("v_raw_scale"))

    def run_attn(self, stream=None):
        fn = decode if self.s.tq == 1 else prefill_chunk
        self.ws_attn = fn(self.t["q"], self.t["pos"], self.o, workspace=self.ws_attn, stream=stream,
                          **self.attn_kwargs())

    def run_decode_step(self, stream=None):
        """index_topk + decode as one v4attn_decode_step (decode only); the call's
        arguments are marshalled on first use (or by prepare()) and reused."""
        self.prepare()
        self._step_call(stream)

    def prepare(self):
        """Marshal the step's calls (compress, decode step) without launching anything."""
        if getattr(self, "_compress_calls", None) is None:
            self._compress_calls = self._make_compress_calls()
        if getattr(self, "_step_call", None) is None:
            s, t = self.s, self.t
            kw = self.attn_kwargs()
            for k in ("idx", "csa_ratio", "topk", "pos_max"):
                kw.pop(k)
            csa = bool(s.branches & CSA)
            if t.get("ki_scale") is not None:
                kw["ki_scale"] = t["ki_scale"]
            self._step_call = DecodeStepCall(t["qi"] if csa else None, t.get("wi"), t.get("ki"), t["q"], t["pos"],
                                             self.o, self.idx, ratio=s.m, topk=s.topk, pos_max=self.pos_max,
                                             workspace=getattr(self, "ws_step", None), **kw)
            self.ws_step = self._step_call.workspace

    def step(self, stream=None, fused=True):
        """The whole hot path of one step: compress (if the step compresses),
        index_topk (if CSA is on), attention.  A decode step with fused=True runs
        the last two as one v4attn_decode_step."""
        self.run_compress(stream)
        if fused and self.s.tq == 1:
            self.run_decode_step(stream)
            return
        self.run_index(stream)
        self.run_attn(stream)
