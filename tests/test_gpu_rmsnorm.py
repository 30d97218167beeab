"""RMSNorm of the queries and of the compressed KV entries ([QbitAI] 混合注意力机制,
the Q/KV normalization paragraph) against the fp64 oracle: compress with gains for K
and V, and every attention entry point with a query gain."""
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
EPS = 1e-5


def _gain(d, seed):
    return np.random.default_rng(seed).uniform(0.5, 1.5, d).astype(np.float32)


@pytest.mark.parametrize("base,ratio_name", [("c4", "m_hca"), ("c1", "m"), ("c1", "m_hca")])
def test_compress_entry_rmsnorm(base, ratio_name):
    cfg = (C.C4.small(name="nrm4", batch=2, pos=4096 + 77, compress_tokens=1024 + 77) if base == "c4"
           else C.C1.small(name="nrm1", batch=2, pos=999, compress_tokens=1000))
    g = synth.generate(cfg)
    t = to_device(g)
    r = getattr(cfg, ratio_name)
    lg = "logit_hca" if ratio_name == "m_hca" else "logit_csa"
    t0 = cfg.compress_t0 - cfg.compress_t0 % r
    n = cfg.last_pos + 1 - t0
    kn, vn = ("kh", "vh") if ratio_name == "m_hca" else ("kc", "vc")
    ok, ov = torch.zeros_like(t[kn]), torch.zeros_like(t[vn])
    gk, gv = _gain(cfg.dim, 1), _gain(cfg.dim, 2)
    print(f"[case] compress rmsnorm {base} r={r}", flush=True)
    V.compress(t["k_raw"], t["v_raw"], t[lg], t["raw_start"], ok, ov, t0=t0, n=n, ratio=r,
               norm_k=torch.from_numpy(gk).cuda(), norm_v=torch.from_numpy(gv).cuda(), norm_eps=EPS)
    torch.cuda.synchronize()
    kr, vr = O.as_f64(g["k_raw"], cfg.dtype), O.as_f64(g["v_raw"], cfg.dtype)
    gok, gov = O.as_f64(dev_to_np(ok), cfg.dtype), O.as_f64(dev_to_np(ov), cfg.dtype)
    for b in range(cfg.batch):
        rs = int(g["raw_start"][b])
        ids, ck = O.compress(kr[b], g[lg][b], rs, t0, n, r)
        _, cv = O.compress(vr[b], g[lg][b], rs, t0, n, r)
        assert_close_store(gok[b, ids], O.rms_norm(ck, gk, EPS), cfg.dtype, f"compress k b={b}")
        assert_close_store(gov[b, ids], O.rms_norm(cv, gv, EPS), cfg.dtype, f"compress v b={b}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
@pytest.mark.parametrize("entry", ["decode", "decode_step"])
def test_query_rmsnorm_decode(name, entry):
    cfg = {"c1": C.C1, "c2": C.C2.small(name="qn2", batch=3, pos=16389, needles=8),
           "c3": C.C3.small(name="qn3", pos=65539, needles=16)}[name]
    r = Run(cfg).run()
    gq = _gain(cfg.dim, 3)
    kw = r.step.attn_kwargs()
    kw.update(q_norm=torch.from_numpy(gq).cuda(), norm_eps=EPS)
    print(f"[case] query rmsnorm {name} {entry}", flush=True)
    if entry == "decode":
        V.decode(r.t["q"], r.t["pos"], r.step.o, **kw)
    else:
        for k in ("idx", "csa_ratio", "topk", "pos_max"):
            kw.pop(k)
        V.decode_step(r.t["qi"], r.t["wi"], r.t["ki"], r.t["q"], r.t["pos"], r.step.o, r.step.idx, ratio=cfg.m,
                      topk=cfg.topk, pos_max=r.step.pos_max, **kw)
    torch.cuda.synchronize()
    r.check_topk()
    r.check_attn(q_norm=gq, norm_eps=EPS)


def test_query_rmsnorm_prefill():
    cfg = C.C5.small(name="qn5", pos=8192, tq=320, needles=8)
    r = Run(cfg).run()
    gq = _gain(cfg.dim, 4)
    kw = r.step.attn_kwargs()
    kw.update(q_norm=torch.from_numpy(gq).cuda(), norm_eps=EPS)
    print("[case] query rmsnorm prefill", flush=True)
    V.prefill_chunk(r.t["q"], r.t["pos"], r.step.o, **kw)
    torch.cuda.synchronize()
    r.check_attn(rows=sample_rows(cfg), q_norm=gq, norm_eps=EPS)
