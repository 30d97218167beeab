"""FP8 E4M3 indexer keys ([wiki] the quantization and deployment section: attention
kept in FP8, FP8 caches) against the fp64 oracle, through the C ABI.

Key rows are codes plus one fp32 scale; the oracle decodes every code exactly
(oracle.fp8_e4m3_decode, pinned to torch's float8_e4m3fn) and scores the scaled
rows; the GPU keeps the codes in LDS, decodes each fragment to bf16 and scales the
dot products before the ReLU.  Top-k sets must match outside the tie band, in the
stage-by-stage path, the decode step, prefill rows and launches whose workgroups
walk several tiles; the codes cover every non-NaN value, subnormals and zero rows.
"""
import numpy as np
import pytest
import torch

from synth import configs as C
import synth
from tests.gpu_harness import Run, dev_to_np, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,pos,fused", [(1, 70003, False), (1, 70003, True), (3, 40961, True),
                                              (20, 131077, True)])
def test_fp8_keys_decode(batch, pos, fused):
    cfg = C.C7.small(name="f8d", batch=batch, pos=pos, needles=8, heads=64)
    print(f"[case] fp8 decode B={batch} pos={pos} fused={fused}", flush=True)
    r = Run(cfg).run(fused=fused).check_all()
    idx = dev_to_np(r.step.idx)
    for b in range(batch):
        assert set(r.g["needles"][b].tolist()) <= set(idx[b, 0].tolist())


def test_fp8_keys_prefill_rows():
    cfg = C.C5.small(name="f85", pos=8192, tq=320, needles=8, ki_fp8=True)
    print("[case] fp8 prefill", flush=True)
    Run(cfg).run().check_all(rows=sample_rows(cfg))


def test_fp8_every_code_subnormals_zero_rows_and_signs():
    # rows built from all 254 non-NaN codes (in a seeded order), some all-zero rows,
    # some scales negative (the definition scales before the ReLU) or zero
    cfg = C.C7.small(name="f8c", pos=20483, needles=0, heads=64, topk=512)
    g = synth.generate(cfg)
    rng = np.random.default_rng(47)
    n, d = g["ki"].shape[1], g["ki"].shape[2]
    pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    g["ki"][0] = rng.choice(pool, size=(n, d))
    g["ki"][0, ::97] = 0
    sc = rng.uniform(0.001, 0.05, n).astype(np.float32)
    sc[::31] *= -1
    sc[::53] = 0
    g["ki_scale"][0] = sc
    print("[case] fp8 codes", flush=True)
    Run(cfg, gen=g).run(fused=True).check_all()


def test_full_c7_decode_step():
    cfg = C.C7
    print("[case] full c7", flush=True)
    r = Run(cfg).run(fused=True).check_all()
    idx = dev_to_np(r.step.idx)
    assert set(r.g["needles"][0].tolist()) <= set(idx[0, 0].tolist())


# ---- FP8 K/V caches (every branch): codes staged in LDS, converted to the bf16
# chunk layout, key scales in the logits, value scales in the product weights
@pytest.mark.parametrize("heads,batch,fused", [(128, 1, False), (128, 1, True), (64, 3, True), (16, 2, False)])
def test_fp8_caches_decode(heads, batch, fused):
    cfg = C.C8.small(name="f8kv", heads=heads, batch=batch, pos=70003, needles=8)
    print(f"[case] fp8 caches H={heads} B={batch} fused={fused}", flush=True)
    Run(cfg).run(fused=fused).check_all()


def test_fp8_caches_prefill_rows():
    cfg = C.C5.small(name="f8kv5", pos=8192, tq=320, needles=8, compress="none", ki_fp8=True, kv_fp8=True)
    print("[case] fp8 caches prefill", flush=True)
    Run(cfg).run().check_all(rows=sample_rows(cfg))


def test_fp8_caches_every_code_and_signs():
    cfg = C.C8.small(name="f8kvc", pos=20483, needles=0, heads=64, topk=512)
    g = synth.generate(cfg)
    rng = np.random.default_rng(48)
    pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for nm in ("kc", "vc", "kh", "vh", "k_raw", "v_raw"):
        g[nm][...] = rng.choice(pool, size=g[nm].shape)
        sc = rng.uniform(0.001, 0.01, g[nm + "_scale"].shape).astype(np.float32)
        sc[..., ::29] *= -1
        sc[..., ::41] = 0
        g[nm + "_scale"][...] = sc
    print("[case] fp8 caches codes", flush=True)
    Run(cfg, gen=g).run(fused=True).check_all()


def test_full_c8_decode_step():
    print("[case] full c8", flush=True)
    r = Run(C.C8).run(fused=True).check_all()
    idx = dev_to_np(r.step.idx)
    assert set(r.g["needles"][0].tolist()) <= set(idx[0, 0].tolist())


@pytest.mark.parametrize("fused", [False, True], ids=["stages", "decode_step"])
def test_fp8_caches_with_query_prep_and_output_rotation(fused):
    # FP8 keys and caches under the query RMSNorm, partial RoPE and the output rotation
    cfg = C.C8.small(name="f8r", heads=64, batch=2, pos=70003, needles=8, rope_dims=64, q_norm=True)
    print(f"[case] fp8 caches + rope/norm fused={fused}", flush=True)
    Run(cfg).run(fused=fused).check_all()


def test_fp8_caches_and_shared_rows_batch_invariant_mode():
    # the batch-invariant split plan over FP8 caches, over shared rows of 512, and both
    import compressed_attention_02_amd as V
    for cfg in (C.C8.small(name="f8i", heads=64, batch=3, pos=40961, needles=8),
                C.C6.small(name="s6i", heads=64, batch=2, pos=40961, needles=8),
                C.C9.small(name="f8si", heads=64, batch=2, pos=40961, needles=8)):
        r = Run(cfg).run()
        kw = r.step.attn_kwargs()
        if cfg.ki_fp8:
            kw["ki_scale"] = r.t["ki_scale"]
        for k in ("idx", "csa_ratio", "topk", "pos_max"):
            kw.pop(k)
        kw["batch_invariant"] = True
        print(f"[case] invariant mode {cfg.name}", flush=True)
        V.decode_step(r.t["qi"], r.t["wi"], r.t["ki"], r.t["q"], r.t["pos"], r.step.o, r.step.idx, ratio=cfg.m,
                      topk=cfg.topk, pos_max=r.step.pos_max, **kw)
        torch.cuda.synchronize()
        r.check_topk()
        r.check_attn()


# ---- FP8 shared entries of 512 (the pages' layer with FP8 caches): a row's codes
# serve as its key and its value, one scale per row in both roles; each chunk's
# codes are staged and converted in LDS for the wave-pair scoring of wide rows
@pytest.mark.parametrize("heads,batch,branches,fused", [
    (128, 1, 7, False), (128, 1, 7, True), (64, 3, 7, True), (16, 2, 7, False), (128, 2, 6, True), (64, 1, 4, False)])
def test_fp8_shared_rows_decode(heads, batch, branches, fused):
    cfg = C.C9.small(name="f8s", heads=heads, batch=batch, pos=70003, branches=branches,
                     needles=8 if branches & 1 else 0, topk=1024 if branches & 1 else 0)
    print(f"[case] fp8 shared rows H={heads} B={batch} br={branches} fused={fused}", flush=True)
    Run(cfg).run(fused=fused).check_all()


def test_fp8_shared_rows_every_code_and_signs():
    cfg = C.C9.small(name="f8sc", pos=20483, needles=0, heads=64, topk=512)
    g = synth.generate(cfg)
    rng = np.random.default_rng(49)
    pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for nm in ("kc", "kh", "k_raw"):
        g[nm][...] = rng.choice(pool, size=g[nm].shape)
        sc = rng.uniform(0.001, 0.01, g[nm + "_scale"].shape).astype(np.float32)
        sc[..., ::29] *= -1
        sc[..., ::41] = 0
        g[nm + "_scale"][...] = sc
    print("[case] fp8 shared rows codes", flush=True)
    Run(cfg, gen=g).run(fused=True).check_all()


def test_full_c9_decode_step():
    print("[case] full c9", flush=True)
    r = Run(C.C9).run(fused=True).check_all()
    idx = dev_to_np(r.step.idx)
    assert set(r.g["needles"][0].tolist()) <= set(idx[0, 0].tolist())
