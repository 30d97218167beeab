"""Python binding of libv4attn (hybrid CSA + HCA + sliding-window attention, gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libv4attn.so``; PyTorch supplies device memory and the current stream.  The
functions mirror the C entry points of ``include/v4attn.h`` by name:

    compress        -> v4attn_compress
    index_topk      -> v4attn_index_topk
    decode          -> v4attn_decode
    prefill_chunk   -> v4attn_prefill_chunk

Tensor layouts (torch tensors on the GPU, innermost dimension contiguous):
    raw K/V       [B, T_raw, d]      row t holds position raw_start[b] + t
    pool logits   [B, T_raw]         fp32
    caches        [B, rows, d]       row = absolute block / entry id
    qi            [B, Tq, H_I, d_I]; wi [B, Tq, H_I] fp32; ki [B, N_cap, d_I]
    idx           [B, Tq, k] int32 (decode: [B, 1, k])
    q, o          [B, Tq, H, d] (o fp32);  lse [B, Tq, H] fp32
    pos0, raw_start  [B] int64
There is no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# V4ATTN_LIB names another build of the same library (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("V4ATTN_LIB") or os.path.join(PKG_DIR, "libv4attn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
CSA, HCA, SWA = 1, 2, 4
BATCH_INVARIANT = 1   # v4a_attn_args.flags
ROPE_OUTPUT = 2       # v4a_attn_args.flags
SHARED_KV = 4         # v4a_attn_args.flags
ROPE_V = 1            # v4a_compress_args.rope_flags
ABI_VERSION = 8
OP_COMPRESS, OP_INDEX_TOPK, OP_DECODE, OP_PREFILL_CHUNK, OP_DECODE_STEP = 0, 1, 2, 3, 4
KERNELS = {"compress": 0, "index_score": 1, "topk_select": 2, "attn": 3, "merge": 4, "prefill": 5,
           "select_attn": 6, "qprep": 7, "read_probe": 8}


class V4AttnError(RuntimeError):
    pass


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("batch_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class CompressArgs(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("ratio", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("t0", ctypes.c_int64), ("n", ctypes.c_int64), ("raw_start", ctypes.c_void_p),
                ("k_raw", Tensor), ("v_raw", Tensor), ("logits", Tensor), ("k_out", Tensor),
                ("v_out", Tensor), ("norm_k", ctypes.c_void_p), ("norm_v", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("rope_dims", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rope_flags", ctypes.c_uint32), ("out_dtype", ctypes.c_int32), ("reserved1", ctypes.c_int32),
                ("k_scale", Tensor), ("v_scale", Tensor)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("tq", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("ratio", ctypes.c_int32), ("topk", ctypes.c_int32), ("pos0", ctypes.c_void_p),
                ("pos_max", ctypes.c_int64), ("qi", Tensor), ("wi", Tensor), ("ki", Tensor),
                ("idx", Tensor), ("sel_scores", Tensor), ("ki_dtype", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("ki_scale", Tensor)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("tq", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("branch_mask", ctypes.c_uint32), ("csa_ratio", ctypes.c_int32),
                ("hca_ratio", ctypes.c_int32), ("window", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32), ("pos0", ctypes.c_void_p),
                ("pos_max", ctypes.c_int64), ("q", Tensor), ("idx", Tensor), ("kc", Tensor),
                ("vc", Tensor), ("kh", Tensor), ("vh", Tensor), ("k_raw", Tensor), ("v_raw", Tensor),
                ("raw_start", ctypes.c_void_p), ("sink", ctypes.c_void_p), ("o", Tensor), ("lse", Tensor),
                ("q_norm", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("rope_dims", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("reserved1", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("reserved2", ctypes.c_int32), ("kc_scale", Tensor), ("vc_scale", Tensor), ("kh_scale", Tensor),
                ("vh_scale", Tensor), ("kr_scale", Tensor), ("vr_scale", Tensor)]


class StepArgs(ctypes.Structure):
    _fields_ = [("index", ctypes.c_void_p), ("attn", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libv4attn.so (built by ``compressed_attention_02_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise V4AttnError(f"{LIB_PATH} is missing: build it with `python -m compressed_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.v4attn_compress.argtypes = [ctypes.POINTER(CompressArgs), ctypes.c_void_p]
        L.v4attn_index_topk.argtypes = [ctypes.POINTER(IndexArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.v4attn_index_topk_workspace.argtypes = [ctypes.POINTER(IndexArgs)]
        L.v4attn_index_topk_workspace.restype = ctypes.c_size_t
        for name in ("v4attn_decode", "v4attn_prefill_chunk"):
            getattr(L, name).argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        for name in ("v4attn_decode_workspace", "v4attn_prefill_chunk_workspace"):
            getattr(L, name).argtypes = [ctypes.POINTER(AttnArgs)]
            getattr(L, name).restype = ctypes.c_size_t
        L.v4attn_decode_step.argtypes = [ctypes.POINTER(IndexArgs), ctypes.POINTER(AttnArgs), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
        L.v4attn_decode_step_noalloc.argtypes = [ctypes.POINTER(IndexArgs), ctypes.POINTER(AttnArgs), ctypes.c_void_p]
        L.v4attn_decode_step_noalloc.restype = ctypes.c_int
        L.v4attn_decode_step_workspace.argtypes = [ctypes.POINTER(IndexArgs), ctypes.POINTER(AttnArgs)]
        L.v4attn_decode_step_workspace.restype = ctypes.c_size_t
        L.v4attn_workspace_size.argtypes = [ctypes.c_int, ctypes.c_void_p]
        L.v4attn_workspace_size.restype = ctypes.c_size_t
        for name in ("v4attn_compress", "v4attn_index_topk", "v4attn_decode", "v4attn_prefill_chunk",
                     "v4attn_decode_step", "v4attn_timing_enable"):
            getattr(L, name).restype = ctypes.c_int
        L.v4attn_status_string.argtypes = [ctypes.c_int]
        L.v4attn_status_string.restype = ctypes.c_char_p
        L.v4attn_last_error.restype = ctypes.c_char_p
        L.v4attn_abi_version.restype = ctypes.c_uint32
        L.v4attn_kernel_name.argtypes = [ctypes.c_int]
        L.v4attn_kernel_name.restype = ctypes.c_char_p
        L.v4attn_timing_enable.argtypes = [ctypes.c_int, ctypes.c_int]
        L.v4attn_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.v4attn_timing_read.restype = ctypes.c_int
        L.v4attn_timing_reset.restype = None
        L.v4attn_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.v4attn_read_probe.restype = ctypes.c_int
        if L.v4attn_abi_version() != ABI_VERSION:
            raise V4AttnError("libv4attn ABI version mismatch")
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise V4AttnError(f"{L.v4attn_status_string(status).decode()}: {L.v4attn_last_error().decode()}")


# ---------------------------------------------------------------- marshalling helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise V4AttnError(f"unsupported dtype {t.dtype}")


def _tensor(t, rows_dim: int = 1) -> Tensor:
    """Descriptor of a [B, rows, ...] tensor: strides of dims 0 and rows_dim; the dims
    after rows_dim must be packed."""
    if t is None:
        return Tensor(None, 0, 0)
    shape, st = t.shape, t.stride()
    packed = 1
    for dim in range(t.dim() - 1, rows_dim, -1):
        if st[dim] != packed:
            raise V4AttnError(f"tensor of shape {tuple(shape)} is not packed after dim {rows_dim}")
        packed *= shape[dim]
    return Tensor(t.data_ptr(), st[0], st[rows_dim] if t.dim() > rows_dim else 0)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_ws(nbytes: int, device):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


# ---------------------------------------------------------------- entry points
def compress_args(k_raw, v_raw, logits, raw_start, k_out, v_out, *, t0: int, n: int, ratio: int,
                  norm_k=None, norm_v=None, norm_eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 1e4,
                  rope_v: bool = False, k_scale=None, v_scale=None) -> CompressArgs:
    """k_out / v_out as uint8 receive the entries as FP8 E4M3 codes, with their fp32
    row scales in k_scale / v_scale [B, N_cap]."""
    import torch
    fp8 = k_out is not None and k_out.dtype == torch.uint8
    return CompressArgs(ABI_VERSION, _dtype_code(k_raw), k_raw.shape[0], k_raw.shape[-1], ratio, 0, t0, n,
                        _ptr(raw_start), _tensor(k_raw), _tensor(v_raw), _tensor(logits), _tensor(k_out),
                        _tensor(v_out), _ptr(norm_k), _ptr(norm_v), norm_eps, rope_dims, rope_base,
                        ROPE_V if rope_v else 0, FP8_E4M3 if fp8 else 0, 0, _tensor(k_scale), _tensor(v_scale))


def compress(k_raw, v_raw, logits, raw_start, k_out, v_out, *, t0: int, n: int, ratio: int, stream=None,
             norm_k=None, norm_v=None, norm_eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 1e4,
             rope_v: bool = False, k_scale=None, v_scale=None):
    """v4attn_compress: pool the complete ratio-blocks of [t0, t0+n) into k_out/v_out
    (RMS-normalised with the fp32 gains norm_k / norm_v when given; with rope_dims,
    raw rows are rotated at their positions and entries at their block's last one).
    v_raw and v_out None: shared K = V entries, K alone is pooled.  uint8 k_out / v_out:
    FP8 E4M3 entries with fp32 row scales in k_scale / v_scale."""
    a = compress_args(k_raw, v_raw, logits, raw_start, k_out, v_out, t0=t0, n=n, ratio=ratio, norm_k=norm_k,
                      norm_v=norm_v, norm_eps=norm_eps, rope_dims=rope_dims, rope_base=rope_base, rope_v=rope_v,
                      k_scale=k_scale, v_scale=v_scale)
    _check(lib().v4attn_compress(ctypes.byref(a), _stream(stream)))


class CompressCall:
    """A v4attn_compress call whose arguments are marshalled once (same keywords as
    compress); repeated calls on the same tensors pay only the C call."""

    def __init__(self, k_raw, v_raw, logits, raw_start, k_out, v_out, **kw):
        self._a = compress_args(k_raw, v_raw, logits, raw_start, k_out, v_out, **kw)
        self._ref = ctypes.byref(self._a)
        self._keep = (k_raw, v_raw, logits, raw_start, k_out, v_out, kw.get("norm_k"), kw.get("norm_v"),
                      kw.get("k_scale"), kw.get("v_scale"))
        self._fn = lib().v4attn_compress

    def __call__(self, stream=None):
        _check(self._fn(self._ref, _stream(stream)))


def index_args(qi, wi, ki, pos0, idx, *, ratio, topk, pos_max, sel_scores=None, ki_scale=None) -> IndexArgs:
    """ki as uint8 holds FP8 E4M3 codes, with ki_scale fp32 [B, N_cap] (one scale per row)."""
    import torch
    B, Tq, HI, dI = qi.shape
    fp8 = ki is not None and ki.dtype == torch.uint8
    return IndexArgs(ABI_VERSION, _dtype_code(qi), B, Tq, HI, dI, ratio, topk, _ptr(pos0), pos_max,
                     _tensor(qi), _tensor(wi), _tensor(ki), _tensor(idx), _tensor(sel_scores),
                     FP8_E4M3 if fp8 else 0, 0, _tensor(ki_scale))


def index_topk_workspace(qi, wi, ki, pos0, idx, *, ratio, topk, pos_max, ki_scale=None) -> int:
    a = index_args(qi, wi, ki, pos0, idx, ratio=ratio, topk=topk, pos_max=pos_max, ki_scale=ki_scale)
    return int(lib().v4attn_index_topk_workspace(ctypes.byref(a)))


def index_topk(qi, wi, ki, pos0, idx, *, ratio: int, topk: int, pos_max: int, sel_scores=None,
               workspace=None, stream=None, ki_scale=None):
    """v4attn_index_topk: indexer scores and per-query top-k ids into idx [B, Tq, k]."""
    a = index_args(qi, wi, ki, pos0, idx, ratio=ratio, topk=topk, pos_max=pos_max, sel_scores=sel_scores,
                   ki_scale=ki_scale)
    if workspace is None:
        workspace = _alloc_ws(int(lib().v4attn_index_topk_workspace(ctypes.byref(a))), qi.device)
    p, n = _ws_ptr(workspace)
    _check(lib().v4attn_index_topk(ctypes.byref(a), p, n, _stream(stream)))
    return workspace


def attn_args(q, pos0, o, *, lse=None, idx=None, kc=None, vc=None, kh=None, vh=None, k_raw=None,
              v_raw=None, raw_start=None, branch_mask=CSA | HCA | SWA, csa_ratio=4, hca_ratio=128,
              window=128, topk=1, pos_max=None, scale=0.0, sink=None, batch_invariant=False,
              q_norm=None, norm_eps=1e-6, rope_dims=0, rope_base=1e4, rope_out=False,
              shared_kv=False, kc_scale=None, vc_scale=None, kh_scale=None, vh_scale=None, kr_scale=None,
              vr_scale=None) -> AttnArgs:
    """Caches given as uint8 hold FP8 E4M3 codes; each then comes with its fp32 [B, rows]
    *_scale (one scale per row).  o may be fp32 or bf16 (out_dtype follows it)."""
    import torch
    B, Tq, H, d = q.shape
    if pos_max is None:
        raise V4AttnError("pos_max (host upper bound of the query positions) is required")
    fp8 = any(t is not None and t.dtype == torch.uint8 for t in (kc, vc, kh, vh, k_raw, v_raw))
    return AttnArgs(ABI_VERSION, _dtype_code(q), _dtype_code(o), B, Tq, H, d, branch_mask, csa_ratio, hca_ratio,
                    window, topk, scale,
                    (BATCH_INVARIANT if batch_invariant else 0) | (ROPE_OUTPUT if rope_out else 0) |
                    (SHARED_KV if shared_kv else 0),
                    _ptr(pos0), pos_max, _tensor(q), _tensor(idx), _tensor(kc),
                    _tensor(vc), _tensor(kh), _tensor(vh), _tensor(k_raw), _tensor(v_raw),
                    _ptr(raw_start), _ptr(sink), _tensor(o), _tensor(lse), _ptr(q_norm), norm_eps, rope_dims,
                    rope_base, 0, FP8_E4M3 if fp8 else 0, 0, _tensor(kc_scale), _tensor(vc_scale),
                    _tensor(kh_scale), _tensor(vh_scale), _tensor(kr_scale), _tensor(vr_scale))


def _run_attn(fn, wsfn, q, pos0, o, workspace, stream, kw):
    a = attn_args(q, pos0, o, **kw)
    if workspace is None:
        workspace = _alloc_ws(int(getattr(lib(), wsfn)(ctypes.byref(a))), q.device)
    p, n = _ws_ptr(workspace)
    _check(getattr(lib(), fn)(ctypes.byref(a), p, n, _stream(stream)))
    return workspace


def decode_workspace(q, pos0, o, **kw) -> int:
    return int(lib().v4attn_decode_workspace(ctypes.byref(attn_args(q, pos0, o, **kw))))


def decode(q, pos0, o, *, workspace=None, stream=None, **kw):
    """v4attn_decode: one query token per sequence (q [B, 1, H, d]); fills o and lse."""
    return _run_attn("v4attn_decode", "v4attn_decode_workspace", q, pos0, o, workspace, stream, kw)


def prefill_chunk(q, pos0, o, *, workspace=None, stream=None, **kw):
    """v4attn_prefill_chunk: Tq causal queries per sequence at pos0[b] + i."""
    return _run_attn("v4attn_prefill_chunk", "v4attn_prefill_chunk_workspace", q, pos0, o, workspace, stream, kw)


def _step_args(qi, wi, ki, q, pos0, o, idx, ratio, topk, pos_max, attn_kw):
    attn_kw = dict(attn_kw)
    ki_scale = attn_kw.pop("ki_scale", None)
    ia = None
    if qi is not None:
        ia = index_args(qi, wi, ki, pos0, idx, ratio=ratio, topk=topk, pos_max=pos_max, ki_scale=ki_scale)
    aa = attn_args(q, pos0, o, idx=idx, csa_ratio=ratio, topk=topk, pos_max=pos_max, **attn_kw)
    return (ctypes.byref(ia) if ia is not None else None), ctypes.byref(aa)


def decode_step_workspace(qi, wi, ki, q, pos0, o, idx, *, ratio, topk, pos_max, **attn_kw) -> int:
    ia, aa = _step_args(qi, wi, ki, q, pos0, o, idx, ratio, topk, pos_max, attn_kw)
    return int(lib().v4attn_decode_step_workspace(ia, aa))


def decode_step(qi, wi, ki, q, pos0, o, idx, *, ratio: int, topk: int, pos_max: int, workspace=None,
                stream=None, **attn_kw):
    """v4attn_decode_step: index_topk (into idx) and decode in one call; the HCA and window
    attention overlaps the indexer.  qi/wi/ki may be None when branch_mask has no CSA."""
    ia, aa = _step_args(qi, wi, ki, q, pos0, o, idx, ratio, topk, pos_max, attn_kw)
    if workspace is None:
        workspace = _alloc_ws(int(lib().v4attn_decode_step_workspace(ia, aa)), q.device)
    p, n = _ws_ptr(workspace)
    _check(lib().v4attn_decode_step(ia, aa, p, n, _stream(stream)))
    return workspace


def decode_step_noalloc(qi, wi, ki, q, pos0, o, idx, *, ratio: int, topk: int, pos_max: int, stream=None,
                        **attn_kw):
    """v4attn_decode_step_noalloc: decode_step with the library's own static scratch
    as workspace (nothing allocated; calls on one device must not overlap)."""
    ia, aa = _step_args(qi, wi, ki, q, pos0, o, idx, ratio, topk, pos_max, attn_kw)
    _check(lib().v4attn_decode_step_noalloc(ia, aa, _stream(stream)))


class DecodeStepCall:
    """A v4attn_decode_step call whose arguments are marshalled once: repeated calls on
    the same tensors (a serving loop, a benchmark) pay only the C call."""

    def __init__(self, qi, wi, ki, q, pos0, o, idx, *, ratio: int, topk: int, pos_max: int, workspace=None,
                 **attn_kw):
        ia, aa = _step_args(qi, wi, ki, q, pos0, o, idx, ratio, topk, pos_max, attn_kw)
        self._keep = (ia, aa)
        if workspace is None:
            workspace = _alloc_ws(int(lib().v4attn_decode_step_workspace(ia, aa)), q.device)
        self.workspace = workspace
        self._ws = _ws_ptr(workspace)
        self._fn = lib().v4attn_decode_step

    def __call__(self, stream=None):
        _check(self._fn(self._keep[0], self._keep[1], self._ws[0], self._ws[1], _stream(stream)))


def workspace_size(op: int, args) -> int:
    """v4attn_workspace_size: workspace bytes of an operation (OP_*) for its marshalled
    arguments (CompressArgs, IndexArgs, AttnArgs, or StepArgs for OP_DECODE_STEP)."""
    return int(lib().v4attn_workspace_size(int(op), ctypes.byref(args)))


# ---------------------------------------------------------------- kernel timing
def timing_enable(kernel: str, max_launches: int) -> None:
    _check(lib().v4attn_timing_enable(KERNELS[kernel], max_launches))


def timing_read(kernel: str, cap: int = 1 << 16) -> list:
    buf = (ctypes.c_float * cap)()
    n = lib().v4attn_timing_read(KERNELS[kernel], buf, cap)
    if n < 0:
        raise V4AttnError("v4attn_timing_read failed")
    return [buf[i] for i in range(n)]


def timing_reset() -> None:
    lib().v4attn_timing_reset()


def read_probe(buf, sink, workgroups: int, stream=None) -> None:
    """v4attn_read_probe: read the device tensor buf once (HBM read-rate probe)."""
    _check(lib().v4attn_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), int(workgroups),
                                   _stream(stream)))
