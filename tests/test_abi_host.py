"""C-ABI library: loads, exports every declared symbol, validates on the host.

No GPU needed.  Validation-failure calls use fake, aligned, never-dereferenced
pointers: the library must reject them before any HIP call.  Calls with valid
arguments are only made when no GPU is visible (they must then fail with EHIP).
"""
import ctypes
import os
import re

import pytest

import compressed_attention_02_amd as V

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "v4attn.h")
EINVAL, ENOTSUP, EWORKSPACE, EHIP = 1, 2, 3, 4
FAKE = 0x7f0000000000          # 256-byte aligned, never dereferenced


def _declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(v4attn_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = V.lib()
    names = _declared()
    assert len(names) >= 13
    assert "v4attn_workspace_size" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.v4attn_abi_version() == V.ABI_VERSION == 8
    assert L.v4attn_status_string(0) == b"ok"
    assert L.v4attn_kernel_name(1) == b"index_score"


def _T(p=FAKE, bs=0, rs=0):
    return V.Tensor(p, bs, rs)


def good_compress(**kw):
    a = V.CompressArgs(V.ABI_VERSION, V.BF16, 2, 128, 4, 0, 0, 4096, FAKE,
                       _T(rs=128, bs=128 * 5000), _T(rs=128, bs=128 * 5000), _T(rs=1, bs=5000),
                       _T(rs=128, bs=128 * 1024), _T(rs=128, bs=128 * 1024))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def good_index(**kw):
    a = V.IndexArgs(V.ABI_VERSION, V.BF16, 2, 1, 64, 64, 4, 512, FAKE, 131072,
                    _T(bs=4096, rs=4096), _T(bs=64, rs=64), _T(bs=64 * 32768, rs=64),
                    _T(bs=512, rs=512), _T(None))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def good_attn(**kw):
    T = _T
    a = V.AttnArgs(V.ABI_VERSION, V.BF16, V.F32, 2, 1, 64, 128, 7, 4, 128, 128, 512, 0.0, 0, FAKE, 131072,
                   T(bs=8192, rs=8192), T(bs=512, rs=512), T(bs=128 * 32768, rs=128),
                   T(bs=128 * 32768, rs=128), T(bs=128 * 1024, rs=128), T(bs=128 * 1024, rs=128),
                   T(bs=128 * 128, rs=128), T(bs=128 * 128, rs=128), FAKE, None,
                   T(bs=8192, rs=8192), T(bs=64, rs=64))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _st(fn, a, *extra):
    r = fn(ctypes.byref(a), *extra)
    return r, V.lib().v4attn_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 1, EINVAL), ("dtype", 7, EINVAL), ("ratio", 0, EINVAL), ("t0", 6, EINVAL),
    ("n", -1, EINVAL), ("dim", 100, ENOTSUP), ("raw_start", None, EINVAL),
])
def test_compress_rejects(field, value, code):
    r, msg = _st(V.lib().v4attn_compress, good_compress(**{field: value}), None)
    assert r == code and msg


def test_compress_rejects_tensors():
    L = V.lib()
    assert _st(L.v4attn_compress, good_compress(k_raw=_T(None, 640000, 128)), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(v_out=_T(FAKE + 8, 131072, 128)), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(k_out=_T(FAKE, 131072, 100)), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(logits=_T(FAKE, 5000, 2)), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(k_raw=_T(FAKE, 0, 128)), None)[0] == EINVAL
    # nothing to do is not an error, even with NULL buffers
    assert _st(L.v4attn_compress, good_compress(n=3, k_raw=_T(None)), None)[0] == 0
    assert _st(L.v4attn_compress, good_compress(batch=0), None)[0] == 0


def test_compress_rejects_fp8_output():
    L = V.lib()
    ks = _T(FAKE, 1024, 1)
    f8 = dict(out_dtype=V.FP8_E4M3, k_out=_T(FAKE, 128 * 1024, 128), v_out=_T(FAKE, 128 * 1024, 128))
    assert _st(L.v4attn_compress, good_compress(out_dtype=7), None)[0] == EINVAL
    # scales belong to an FP8 output only
    assert _st(L.v4attn_compress, good_compress(k_scale=ks), None)[0] == EINVAL
    # an FP8 output needs its scales: present, 4-byte aligned, one per row (row_stride 1)
    assert _st(L.v4attn_compress, good_compress(**f8), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(**f8, k_scale=ks), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(**f8, k_scale=ks, v_scale=_T(FAKE, 1024, 2)), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(**f8, k_scale=_T(FAKE + 2, 1024, 1), v_scale=ks), None)[0] == EINVAL
    # code rows of 16-byte multiples: dim a multiple of 16, row_stride a multiple of 16 bytes
    assert _st(L.v4attn_compress, good_compress(**f8, dim=120, k_scale=ks, v_scale=ks), None)[0] == ENOTSUP
    bad_rows = dict(f8, k_out=_T(FAKE, 128 * 1024, 136))
    assert _st(L.v4attn_compress, good_compress(**bad_rows, k_scale=ks, v_scale=ks), None)[0] == EINVAL
    # K-only pooling takes no v_scale
    konly = dict(f8, v_out=_T(None))
    assert _st(L.v4attn_compress, good_compress(**konly, v_raw=_T(None), k_scale=ks, v_scale=ks), None)[0] == EINVAL


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 0, EINVAL), ("tq", 0, EINVAL), ("topk", 0, EINVAL), ("topk", 4096, ENOTSUP),
    ("heads", 48, ENOTSUP), ("dim", 48, ENOTSUP), ("ratio", 0, EINVAL), ("pos_max", -1, EINVAL),
    ("pos0", None, EINVAL),
])
def test_index_rejects(field, value, code):
    L = V.lib()
    r, msg = _st(L.v4attn_index_topk, good_index(**{field: value}), None, 0, None)
    assert r == code and msg


def test_index_rejects_tensors_and_workspace():
    L = V.lib()
    f = L.v4attn_index_topk
    assert _st(f, good_index(idx=_T(FAKE, 512, 100)), None, 0, None)[0] == EINVAL
    assert _st(f, good_index(qi=_T(FAKE + 4, 4096, 4096)), None, 0, None)[0] == EINVAL
    assert _st(f, good_index(ki=_T(FAKE, 64 * 32768, 32)), None, 0, None)[0] == EINVAL
    a = good_index()
    need = L.v4attn_index_topk_workspace(ctypes.byref(a))
    assert need > 2 * 32768 * 4
    assert _st(f, a, None, 0, None)[0] == EWORKSPACE
    assert _st(f, a, FAKE, need - 1, None)[0] == EWORKSPACE
    assert _st(f, a, FAKE + 16, need, None)[0] == EWORKSPACE
    # f32 indexer shapes: any head count, dim a multiple of 4
    a = good_index(dtype=V.F32, heads=4, dim=32, qi=_T(bs=128, rs=128), ki=_T(bs=32 * 32768, rs=32))
    assert L.v4attn_index_topk_workspace(ctypes.byref(a)) > 0


@pytest.mark.parametrize("field,value,code", [
    ("out_dtype", 2, EINVAL), ("tq", 2, EINVAL), ("heads", 40, ENOTSUP), ("dim", 96, ENOTSUP),
    ("branch_mask", 0, EINVAL), ("branch_mask", 9, EINVAL), ("csa_ratio", 0, EINVAL),
    ("window", -1, EINVAL), ("topk", 0, EINVAL), ("topk", 3000, ENOTSUP), ("scale", float("nan"), EINVAL),
    ("pos0", None, EINVAL), ("raw_start", None, EINVAL), ("sink", FAKE + 2, EINVAL),
])
def test_decode_rejects(field, value, code):
    L = V.lib()
    r, msg = _st(L.v4attn_decode, good_attn(**{field: value}), None, 0, None)
    assert r == code and msg


def test_decode_rejects_branch_pointers():
    L = V.lib()
    f = L.v4attn_decode
    assert _st(f, good_attn(kc=_T(None)), None, 0, None)[0] == EINVAL
    assert _st(f, good_attn(kh=_T(None)), None, 0, None)[0] == EINVAL
    assert _st(f, good_attn(idx=_T(None)), None, 0, None)[0] == EINVAL
    assert _st(f, good_attn(o=_T(FAKE, 8192, 8000)), None, 0, None)[0] == EINVAL
    # disabled branches may be NULL: HCA+SWA only
    a = good_attn(branch_mask=6, kc=_T(None), vc=_T(None), idx=_T(None))
    assert V.lib().v4attn_decode_workspace(ctypes.byref(a)) >= 0
    # prefill accepts tq > 1, decode does not
    a = good_attn(tq=16, q=_T(bs=16 * 8192, rs=8192), o=_T(bs=16 * 8192, rs=8192))
    assert _st(L.v4attn_decode, a, None, 0, None)[0] == EINVAL
    assert _st(L.v4attn_prefill_chunk, good_attn(tq=0), None, 0, None)[0] == EINVAL


def test_decode_workspace_and_split_plan():
    L = V.lib()
    a = good_attn()
    need = L.v4attn_decode_workspace(ctypes.byref(a))
    # two sequences, 512 + 1024 + 128 keys each: the keys are split across workgroups
    assert need > 0
    assert _st(L.v4attn_decode, a, None, 0, None)[0] == EWORKSPACE


def test_timing_api_validates():
    L = V.lib()
    assert L.v4attn_timing_enable(99, 1) == EINVAL
    assert L.v4attn_timing_read(99, None, 0) == -1
    L.v4attn_timing_reset()


def test_valid_call_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this checks the no-device path only")
    r, msg = _st(V.lib().v4attn_compress, good_compress(), None)
    assert r == EHIP and msg


def _step(ix, a, ws=None, n=0):
    L = V.lib()
    r = L.v4attn_decode_step(ctypes.byref(ix) if ix is not None else None, ctypes.byref(a), ws, n, None)
    return r, L.v4attn_last_error().decode()


@pytest.mark.parametrize("ix_kw,a_kw", [
    (dict(topk=256), {}), (dict(ratio=8), {}), (dict(pos_max=131073), {}), (dict(tq=2), {}),
    (dict(idx=_T(FAKE + 256, 512, 512)), {}), (dict(idx=_T(FAKE, 512, 1024)), {}), (dict(batch=1), {}),
    ({}, dict(tq=2)), ({}, dict(topk=0)),
])
def test_decode_step_rejects_mismatch(ix_kw, a_kw):
    r, msg = _step(good_index(**ix_kw), good_attn(**a_kw))
    assert r == EINVAL and msg


def test_decode_step_workspace_and_null_index():
    L = V.lib()
    ix, a = good_index(), good_attn()
    need = L.v4attn_decode_step_workspace(ctypes.byref(ix), ctypes.byref(a))
    # the indexer's workspace plus the attention partials of both launches
    assert need > L.v4attn_index_topk_workspace(ctypes.byref(ix))
    assert _step(ix, a)[0] == EWORKSPACE
    assert _step(ix, a, FAKE + 16, need)[0] == EWORKSPACE
    # the CSA branch needs the indexer's arguments; without it they may be NULL
    assert _step(None, a)[0] == EINVAL
    assert L.v4attn_decode_step_workspace(None, ctypes.byref(a)) == 0
    b = good_attn(branch_mask=6, kc=_T(None), vc=_T(None), idx=_T(None))
    assert L.v4attn_decode_step_workspace(None, ctypes.byref(b)) > 0
    # invalid arguments report no workspace
    assert L.v4attn_decode_step_workspace(ctypes.byref(good_index(topk=256)), ctypes.byref(a)) == 0


def test_attention_rejects_huge_row_strides():
    big = 1 << 31
    r, msg = _st(V.lib().v4attn_decode, good_attn(kh=_T(FAKE, big * 4, big)), None, 0, None)
    assert r == ENOTSUP and msg


def test_workspace_size_by_operation():
    # v4attn_workspace_size dispatches to the per-operation sizes
    L = V.lib()
    ix, a = good_index(), good_attn()
    ws = lambda op, x: V.workspace_size(op, x)
    assert ws(V.OP_COMPRESS, good_compress()) == 0
    assert ws(V.OP_INDEX_TOPK, ix) == L.v4attn_index_topk_workspace(ctypes.byref(ix)) > 0
    assert ws(V.OP_DECODE, a) == L.v4attn_decode_workspace(ctypes.byref(a)) > 0
    assert ws(V.OP_PREFILL_CHUNK, a) == L.v4attn_prefill_chunk_workspace(ctypes.byref(a)) > 0
    st = V.StepArgs(ctypes.addressof(ix), ctypes.addressof(a))
    assert ws(V.OP_DECODE_STEP, st) == L.v4attn_decode_step_workspace(ctypes.byref(ix), ctypes.byref(a)) > 0
    b = good_attn(branch_mask=6, kc=_T(None), vc=_T(None), idx=_T(None))
    assert ws(V.OP_DECODE_STEP, V.StepArgs(None, ctypes.addressof(b))) > 0
    assert ws(99, a) == 0
    assert L.v4attn_workspace_size(V.OP_DECODE, None) == 0
    assert ws(V.OP_DECODE, good_attn(dtype=9)) == 0


def test_bf16_output_is_accepted_and_checked():
    # out_dtype BF16: o holds bf16 (strides in bf16 elements, 16-byte multiples)
    L = V.lib()
    a = good_attn(out_dtype=V.BF16)
    assert L.v4attn_decode_workspace(ctypes.byref(a)) > 0
    assert _st(L.v4attn_decode, a, None, 0, None)[0] == EWORKSPACE   # past validation
    r, msg = _st(L.v4attn_decode, good_attn(out_dtype=V.BF16, o=_T(FAKE, 8192 + 4, 8192)), None, 0, None)
    assert r == EINVAL and "o" in msg
    r, msg = _st(L.v4attn_decode, good_attn(out_dtype=3), None, 0, None)
    assert r == EINVAL and "out_dtype" in msg


def test_batch_invariant_split_limit_is_rejected_before_launch():
    # batch-invariant plans split every 256 keys and the merge takes at most 1024
    # splits: hca_ratio 1 at pos_max 300000 needs about 1173 splits.  The call must
    # fail with ENOTSUP before anything is enqueued, and the workspace queries say 0.
    L = V.lib()
    a = good_attn(flags=V.BATCH_INVARIANT, hca_ratio=1, pos_max=300000)
    ix = good_index(pos_max=300000)
    assert L.v4attn_decode_workspace(ctypes.byref(a)) == 0
    assert L.v4attn_prefill_chunk_workspace(ctypes.byref(a)) == 0
    assert L.v4attn_decode_step_workspace(ctypes.byref(ix), ctypes.byref(a)) == 0
    r, msg = _st(L.v4attn_decode, a, FAKE, 1 << 40, None)
    assert r == ENOTSUP and "splits" in msg
    r, msg = _step(ix, a, FAKE, 1 << 40)
    assert r == ENOTSUP and "splits" in msg
    # the same shape without the flag is planned with longer splits
    b = good_attn(hca_ratio=1, pos_max=300000)
    assert L.v4attn_decode_workspace(ctypes.byref(b)) > 0
    assert L.v4attn_decode_step_workspace(ctypes.byref(ix), ctypes.byref(b)) > 0


def test_attention_rejects_unknown_flags():
    r, msg = _st(V.lib().v4attn_decode, good_attn(flags=8), None, 0, None)
    assert r == EINVAL and "flags" in msg


def test_shared_kv_argument_checks():
    L = V.lib()
    # shared entries: the value tensors must be absent
    r, msg = _st(L.v4attn_decode, good_attn(flags=V.SHARED_KV), None, 0, None)
    assert r == EINVAL and "SHARED_KV" in msg
    none = V.Tensor(None, 0, 0)
    ok = good_attn(flags=V.SHARED_KV, vc=none, vh=none, v_raw=none)
    assert L.v4attn_decode_workspace(ctypes.byref(ok)) > 0
    # bf16 rows of 512 only as shared entries; 256 is no supported size
    assert _st(L.v4attn_decode, good_attn(dim=512), None, 0, None)[0] == ENOTSUP
    assert _st(L.v4attn_decode, good_attn(dim=256, flags=V.SHARED_KV, vc=none, vh=none, v_raw=none),
               None, 0, None)[0] == ENOTSUP
    wide = dict(dim=512, flags=V.SHARED_KV, vc=none, vh=none, v_raw=none, q=_T(bs=32768, rs=32768),
                o=_T(bs=32768, rs=32768), kc=_T(bs=512 * 32768, rs=512), kh=_T(bs=512 * 1024, rs=512),
                k_raw=_T(bs=512 * 128, rs=512))
    assert L.v4attn_decode_workspace(ctypes.byref(good_attn(**wide))) > 0
    assert L.v4attn_decode_workspace(ctypes.byref(good_attn(**dict(wide, dtype=V.F32)))) > 0
    # K-only compression: v_raw and v_out both absent, and then no V gain or V rotation
    assert _st(L.v4attn_compress, good_compress(v_out=none), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(v_raw=none, v_out=none, norm_v=FAKE), None)[0] == EINVAL
    assert _st(L.v4attn_compress, good_compress(v_raw=none, v_out=none, rope_dims=64, rope_base=1e4,
                                                rope_flags=V.ROPE_V), None)[0] == EINVAL


@pytest.mark.parametrize("field,value", [("rope_dims", 3), ("rope_dims", 130), ("rope_dims", -2), ("rope_base", 0.0)])
def test_rope_argument_checks(field, value):
    kw = {field: value}
    if field == "rope_base":
        kw["rope_dims"] = 64
    r, msg = _st(V.lib().v4attn_decode, good_attn(**kw), None, 0, None)
    assert r == EINVAL and "rope" in msg
    assert _st(V.lib().v4attn_decode, good_attn(flags=2), None, 0, None)[0] == EINVAL   # output rotation needs R
    rc, msg = _st(V.lib().v4attn_compress, good_compress(**kw), None)
    assert rc == EINVAL and "rope" in msg
    assert _st(V.lib().v4attn_compress, good_compress(rope_dims=64, rope_base=1e4, rope_flags=4), None)[0] == EINVAL
    assert _st(V.lib().v4attn_compress, good_compress(rope_dims=128, rope_base=1e4, ratio=128), None)[0] == ENOTSUP


def test_fp8_key_argument_checks():
    L = V.lib()
    f = L.v4attn_index_topk
    # FP8 keys need a bf16 indexer and a scale tensor with unit row stride
    r, msg = _st(f, good_index(ki_dtype=V.FP8_E4M3), None, 0, None)
    assert r == EINVAL and "ki_scale" in msg
    assert _st(f, good_index(ki_dtype=V.FP8_E4M3, dtype=V.F32), None, 0, None)[0] == EINVAL
    assert _st(f, good_index(ki_dtype=7), None, 0, None)[0] == EINVAL
    fp8 = dict(ki_dtype=V.FP8_E4M3, ki=_T(bs=64 * 32768, rs=64), ki_scale=_T(bs=32768, rs=1))
    assert L.v4attn_index_topk_workspace(ctypes.byref(good_index(**fp8))) > 0
    assert _st(f, good_index(**dict(fp8, ki_scale=_T(bs=32768, rs=2))), None, 0, None)[0] == EINVAL


def test_fp8_cache_argument_checks():
    L = V.lib()
    none = V.Tensor(None, 0, 0)
    f8 = dict(kv_dtype=V.FP8_E4M3, kc=_T(bs=128 * 32768, rs=128), vc=_T(bs=128 * 32768, rs=128),
              kh=_T(bs=128 * 1024, rs=128), vh=_T(bs=128 * 1024, rs=128), k_raw=_T(bs=128 * 128, rs=128),
              v_raw=_T(bs=128 * 128, rs=128))
    scales = {n: _T(bs=32768, rs=1) for n in ("kc_scale", "vc_scale", "kh_scale", "vh_scale", "kr_scale", "vr_scale")}
    assert L.v4attn_decode_workspace(ctypes.byref(good_attn(**f8, **scales))) > 0
    r, msg = _st(L.v4attn_decode, good_attn(**f8), None, 0, None)
    assert r == EINVAL and "scale" in msg
    assert _st(L.v4attn_decode, good_attn(**f8, **dict(scales, kh_scale=_T(bs=1024, rs=4))), None, 0, None)[0] == EINVAL
    assert _st(L.v4attn_decode, good_attn(**f8, **scales, dtype=V.F32), None, 0, None)[0] == EINVAL
    r, msg = _st(L.v4attn_decode, good_attn(**dict(f8, flags=V.SHARED_KV, vc=none, vh=none, v_raw=none), **scales),
                 None, 0, None)
    assert r == ENOTSUP
    # shared entries of 512 in FP8: the key rows' scales serve as the values' too
    s512 = dict(kv_dtype=V.FP8_E4M3, dim=512, flags=V.SHARED_KV, q=_T(bs=64 * 512, rs=64 * 512),
                o=_T(bs=64 * 512, rs=64 * 512), kc=_T(bs=512 * 32768, rs=512), vc=none,
                kh=_T(bs=512 * 1024, rs=512), vh=none, k_raw=_T(bs=512 * 128, rs=512), v_raw=none)
    kscales = {n: _T(bs=32768, rs=1) for n in ("kc_scale", "kh_scale", "kr_scale")}
    assert L.v4attn_decode_workspace(ctypes.byref(good_attn(**s512, **kscales))) > 0
    r, msg = _st(L.v4attn_decode, good_attn(**s512, **kscales, vh_scale=_T(bs=32768, rs=1)), None, 0, None)
    assert r == EINVAL and "vc_scale" in msg
    r, msg = _st(L.v4attn_decode, good_attn(**dict(s512, kv_dtype=0)), None, 0, None)   # bf16 rows of 512 still fine
    assert r != ENOTSUP


def test_noalloc_step_validates_before_touching_the_device():
    # invalid arguments are rejected on the host; a step whose workspace exceeds the
    # 64 MiB static scratch gets ENOTSUP before any HIP call
    L = V.lib()
    r = L.v4attn_decode_step_noalloc(ctypes.byref(good_index(topk=256)), ctypes.byref(good_attn()), None)
    assert r == EINVAL
    a = good_attn(pos_max=1 << 26)      # 2^24 visible blocks: 64 MiB of scores per row
    ix = good_index(pos_max=1 << 26)
    assert L.v4attn_decode_step_workspace(ctypes.byref(ix), ctypes.byref(a)) > 64 << 20
    r = L.v4attn_decode_step_noalloc(ctypes.byref(ix), ctypes.byref(a), None)
    assert r == ENOTSUP and "scratch" in L.v4attn_last_error().decode()


def test_index_workspace_row_groups():
    # scores and tile reports of about 1.1 MB a row at 1M context, taken in groups of
    # rows within 8 GiB: a 4096-query chunk is one group, an 8192-query chunk two, so
    # its workspace holds fewer rows than the chunk has
    L = V.lib()
    per_row = 262144 * 4 + 1024 * (8 * 4 + 16)   # fp32 scores + 8 report keys and an info word a tile
    w4 = L.v4attn_index_topk_workspace(ctypes.byref(good_index(batch=1, tq=4096, pos_max=1048576 + 4095)))
    w8 = L.v4attn_index_topk_workspace(ctypes.byref(good_index(batch=1, tq=8192, pos_max=1048576 + 8191)))
    assert 4096 * per_row <= w4 < 4200 * per_row
    assert w8 <= 8 << 30
    assert 4096 * per_row < w8 < 8192 * per_row
