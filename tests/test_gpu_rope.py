"""Partial RoPE ([QbitAI] 混合注意力机制, the partial RoPE paragraph) against the fp64
oracle: compressed entries pooled in the unrotated frame and rotated at their block's
last position, the query rotated at p, and the output rotated back at -p."""
import numpy as np
import pytest
import torch

import compressed_attention_02_amd as V
import oracle as O
import synth
from synth import configs as C
from compressed_attention_02_amd.layer import to_device
from tests.gpu_harness import Run, assert_close_store, dev_to_np, sample_rows

pytestmark = pytest.mark.gpu
R, BASE, EPS = 64, 10000.0, 1e-5


def _gain(d, seed):
    return np.random.default_rng(seed).uniform(0.5, 1.5, d).astype(np.float32)


@pytest.mark.parametrize("base,ratio_name,rope_v,norm", [
    ("c4", "m_hca", True, True), ("c4", "m_hca", False, False), ("c1", "m", True, False), ("c1", "m_hca", False, True)])
def test_compress_entry_rope(base, ratio_name, rope_v, norm):
    cfg = (C.C4.small(name="rp4", batch=2, pos=4096 + 77, compress_tokens=1024 + 77) if base == "c4"
           else C.C1.small(name="rp1", batch=2, pos=999, dim=128, compress_tokens=1000))
    g = synth.generate(cfg)
    t = to_device(g)
    r = getattr(cfg, ratio_name)
    lg = "logit_hca" if ratio_name == "m_hca" else "logit_csa"
    t0 = cfg.compress_t0 - cfg.compress_t0 % r
    n = cfg.last_pos + 1 - t0
    kn, vn = ("kh", "vh") if ratio_name == "m_hca" else ("kc", "vc")
    ok, ov = torch.zeros_like(t[kn]), torch.zeros_like(t[vn])
    gk, gv = _gain(cfg.dim, 5), _gain(cfg.dim, 6)
    kw = dict(norm_k=torch.from_numpy(gk).cuda(), norm_v=torch.from_numpy(gv).cuda(), norm_eps=EPS) if norm else {}
    print(f"[case] compress rope {base} r={r} rope_v={rope_v} norm={norm}", flush=True)
    V.compress(t["k_raw"], t["v_raw"], t[lg], t["raw_start"], ok, ov, t0=t0, n=n, ratio=r, rope_dims=R,
               rope_base=BASE, rope_v=rope_v, **kw)
    torch.cuda.synchronize()
    kr, vr = O.as_f64(g["k_raw"], cfg.dtype), O.as_f64(g["v_raw"], cfg.dtype)
    gok, gov = O.as_f64(dev_to_np(ok), cfg.dtype), O.as_f64(dev_to_np(ov), cfg.dtype)
    for b in range(cfg.batch):
        rs = int(g["raw_start"][b])
        ids, ck = O.compress_entries(kr[b], g[lg][b], rs, t0, n, r, gain=gk if norm else None, eps=EPS,
                                     rope_dims=R, rope_base=BASE)
        _, cv = O.compress_entries(vr[b], g[lg][b], rs, t0, n, r, gain=gv if norm else None, eps=EPS,
                                   rope_dims=R if rope_v else 0, rope_base=BASE)
        assert_close_store(gok[b, ids], ck, cfg.dtype, f"compress k b={b}")
        assert_close_store(gov[b, ids], cv, cfg.dtype, f"compress v b={b}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
@pytest.mark.parametrize("entry", ["decode", "decode_step"])
@pytest.mark.parametrize("rope_out,norm", [(True, True), (False, False)])
def test_query_and_output_rope_decode(name, entry, rope_out, norm):
    cfg = {"c1": C.C1.small(name="rq1", dim=128), "c2": C.C2.small(name="rq2", batch=3, pos=16389, needles=8),
           "c3": C.C3.small(name="rq3", pos=65539, needles=16)}[name]
    r = Run(cfg).run()
    gq = _gain(cfg.dim, 7)
    kw = r.step.attn_kwargs()
    kw.update(rope_dims=R, rope_base=BASE, rope_out=rope_out)
    if norm:
        kw.update(q_norm=torch.from_numpy(gq).cuda(), norm_eps=EPS)
    print(f"[case] rope {name} {entry} out={rope_out} norm={norm}", flush=True)
    if entry == "decode":
        V.decode(r.t["q"], r.t["pos"], r.step.o, **kw)
    else:
        for k in ("idx", "csa_ratio", "topk", "pos_max"):
            kw.pop(k)
        V.decode_step(r.t["qi"], r.t["wi"], r.t["ki"], r.t["q"], r.t["pos"], r.step.o, r.step.idx, ratio=cfg.m,
                      topk=cfg.topk, pos_max=r.step.pos_max, **kw)
    torch.cuda.synchronize()
    r.check_topk()
    r.check_attn(q_norm=gq if norm else None, norm_eps=EPS, rope_dims=R, rope_base=BASE, rope_out=rope_out)


def test_query_and_output_rope_prefill():
    cfg = C.C5.small(name="rq5", pos=8192, tq=320, needles=8)
    r = Run(cfg).run()
    gq = _gain(cfg.dim, 8)
    kw = r.step.attn_kwargs()
    kw.update(q_norm=torch.from_numpy(gq).cuda(), norm_eps=EPS, rope_dims=R, rope_base=BASE, rope_out=True)
    print("[case] rope prefill", flush=True)
    V.prefill_chunk(r.t["q"], r.t["pos"], r.step.o, **kw)
    torch.cuda.synchronize()
    r.check_attn(rows=sample_rows(cfg), q_norm=gq, norm_eps=EPS, rope_dims=R, rope_base=BASE, rope_out=True)


def test_query_prep_in_score_launch_with_walking_workgroups():
    # the decode step hosts the query prep in its score launch; with many rows each
    # score workgroup walks several indexer tiles (20 rows x 128 tiles here), which
    # the prep workgroups must not disturb
    cfg = C.C2.small(name="rq2w", batch=20, pos=131077, needles=8)
    r = Run(cfg).run()
    gq = _gain(cfg.dim, 9)
    kw = r.step.attn_kwargs()
    for k in ("idx", "csa_ratio", "topk", "pos_max"):
        kw.pop(k)
    kw.update(rope_dims=R, rope_base=BASE, rope_out=True, q_norm=torch.from_numpy(gq).cuda(), norm_eps=EPS)
    print("[case] rope decode_step 20 rows", flush=True)
    V.decode_step(r.t["qi"], r.t["wi"], r.t["ki"], r.t["q"], r.t["pos"], r.step.o, r.step.idx, ratio=cfg.m,
                  topk=cfg.topk, pos_max=r.step.pos_max, **kw)
    torch.cuda.synchronize()
    r.check_topk()
    r.check_attn(q_norm=gq, norm_eps=EPS, rope_dims=R, rope_base=BASE, rope_out=True)
