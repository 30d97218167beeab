"""Shared K = V entries ([QbitAI] 混合注意力机制: the KV entries serve as keys and as
values, head dimension c = 512, RoPE on the last 64 channels with the output rotated
back; [wiki] shared-KV MQA) against the fp64 oracle, through the C ABI.

The oracle attends with each entry as its own value (no V tensor exists); the GPU
reads each row once.  Rows of 512 run one 16-head tile per wave, two waves per
tile on the halves of every chunk up to 64 heads, so the cases cover 16, 64, 80
(idle waves) and 128 heads, every branch subset, the sink, prefill rows and the
decode step, plus the fp32 path and the d = 128 aliasing path.
"""
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
R, BASE, EPS = 64, 10000.0, 1e-6


def _c6(**kw):
    base = dict(name="sk6", pos=70003, needles=8)
    base.update(kw)
    return C.C6.small(**base)


@pytest.mark.parametrize("heads,batch,branches", [
    (128, 1, 7), (64, 3, 7), (16, 2, 7), (80, 2, 7), (128, 2, 1), (64, 2, 6), (128, 1, 4)])
@pytest.mark.parametrize("fused", [False, True], ids=["stages", "decode_step"])
def test_shared_kv_decode(heads, batch, branches, fused):
    cfg = _c6(heads=heads, batch=batch, branches=branches, needles=8 if branches & 1 else 0,
              topk=1024 if branches & 1 else 0)
    print(f"[case] shared-kv decode H={heads} B={batch} br={branches} fused={fused}", flush=True)
    Run(cfg).run(fused=fused).check_all()


@pytest.mark.parametrize("rope,norm", [(False, False), (True, False), (False, True)])
def test_shared_kv_decode_options(rope, norm):
    cfg = _c6(name="sk6o", heads=64, batch=2, rope_dims=R if rope else 0, q_norm=norm)
    print(f"[case] shared-kv options rope={rope} norm={norm}", flush=True)
    Run(cfg).run().check_all()


def test_shared_kv_sink_and_short_history():
    # fewer visible blocks than k, a history shorter than the window's reach, a sink
    cfg = _c6(name="sk6s", pos=300, heads=64, needles=4, topk=512)
    r = Run(cfg).run()
    sink = np.linspace(-1.0, 2.0, cfg.heads).astype(np.float32)
    kw = r.step.attn_kwargs()
    kw["sink"] = torch.from_numpy(sink).cuda()
    print("[case] shared-kv sink", flush=True)
    V.decode(r.t["q"], r.t["pos"], r.step.o, **kw)
    torch.cuda.synchronize()
    ro, rl = r.oracle_attn(sink=sink.astype(np.float64))
    from tests.gpu_harness import assert_close
    assert_close(dev_to_np(r.step.o)[:, 0], ro.reshape(cfg.batch, cfg.heads, cfg.dim), "bf16", "o")
    assert_close(dev_to_np(r.step.lse)[:, 0], rl.reshape(cfg.batch, cfg.heads), "bf16", "lse")


def test_shared_kv_prefill_rows():
    cfg = C.C5.small(name="sk5", pos=8192, tq=320, needles=8, dim=512, shared_kv=True, rope_dims=R,
                     q_norm=True)
    print("[case] shared-kv prefill", flush=True)
    Run(cfg).run().check_all(rows=sample_rows(cfg))


def test_shared_kv_f32_and_d128_alias():
    print("[case] shared-kv f32 d=512", flush=True)
    Run(C.C1.small(name="sk1", dim=512, shared_kv=True, rope_dims=R, q_norm=True)).run().check_all()
    print("[case] shared-kv bf16 d=128", flush=True)
    Run(C.C2.small(name="sk2", batch=2, pos=16389, needles=8, shared_kv=True, rope_dims=R,
                   q_norm=True)).run(fused=True).check_all()


@pytest.mark.parametrize("dtype,ratio,norm", [("bf16", 4, True), ("bf16", 128, False), ("f32", 128, True)])
def test_k_only_compress(dtype, ratio, norm):
    cfg = (C.C4.small(name="skc", batch=2, pos=4096 + 77, compress_tokens=1024 + 77, dim=512, shared_kv=True)
           if dtype == "bf16" else C.C1.small(name="skc1", batch=2, pos=999, dim=512, compress_tokens=1000,
                                               shared_kv=True))
    g = synth.generate(cfg)
    t = to_device(g)
    lg = "logit_hca"
    t0 = cfg.compress_t0 - cfg.compress_t0 % ratio
    n = cfg.last_pos + 1 - t0
    rows = (cfg.last_pos + 1) // ratio
    out = torch.zeros((cfg.batch, rows, cfg.dim), dtype=t["k_raw"].dtype, device="cuda")
    gk = np.random.default_rng(9).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
    kw = dict(norm_k=torch.from_numpy(gk).cuda(), norm_eps=EPS) if norm else {}
    print(f"[case] k-only compress {dtype} r={ratio} norm={norm}", flush=True)
    V.compress(t["k_raw"], None, t[lg], t["raw_start"], out, None, t0=t0, n=n, ratio=ratio, rope_dims=R,
               rope_base=BASE, **kw)
    torch.cuda.synchronize()
    kr = O.as_f64(g["k_raw"], cfg.dtype)
    got = O.as_f64(dev_to_np(out), cfg.dtype)
    for b in range(cfg.batch):
        ids, ref = O.compress_entries(kr[b], g[lg][b], int(g["raw_start"][b]), t0, n, ratio,
                                      gain=gk if norm else None, eps=EPS, rope_dims=R, rope_base=BASE)
        assert_close_store(got[b, ids], ref, cfg.dtype, f"k-only compress b={b}")


def test_full_c6_decode_step():
    # the pages' layer shape at 1M context, in the launch configuration bench.py times
    cfg = C.C6
    print("[case] full c6", flush=True)
    r = Run(cfg).run(fused=True).check_all()
    idx = dev_to_np(r.step.idx)
    assert set(r.g["needles"][0].tolist()) <= set(idx[0, 0].tolist())
