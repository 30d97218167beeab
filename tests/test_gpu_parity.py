"""Parity of the HIP path with the fp64 oracle, stage by stage (GPU).

Small configurations span several tiles and ragged tails and finish in seconds in
the oracle; the full configurations run in the launch configuration bench.py times
and are checked on every row (decode) or on sampled rows (prefill).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import configs as C
from tests.gpu_harness import Run, assert_close, dev_to_np, sample_rows

pytestmark = pytest.mark.gpu

# reduced versions of the configurations: same head shapes, shorter contexts,
# positions that are not block aligned, several sequences
SMALL = {
    "c1_tiny_f32": C.C1,
    "c2_small": C.C2.small(name="c2_small", batch=3, pos=16389, needles=8),
    "c3_small": C.C3.small(name="c3_small", pos=65539, needles=16),
    "c4_small": C.C4.small(name="c4_small", batch=4, pos=16384 + 77, compress_tokens=1024 + 77),
    "c5_small": C.C5.small(name="c5_small", pos=8192, tq=320, needles=8),
}


def _hca_newest_ok(cfg):
    return cfg.compress != "hca_newest" or cfg.compress_t0 % cfg.m_hca == 0


@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs(name):
    cfg = SMALL[name]
    if name == "c4_small":
        cfg = cfg.small(compress_tokens=1024 + (cfg.pos % cfg.m_hca))
    assert _hca_newest_ok(cfg)
    print(f"[case] {name}", flush=True)
    Run(cfg).run().check_all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_context_k_exceeds_visible(dtype):
    # p < W, n_vis < k: padding with -1, window shorter than W, HCA nearly empty
    base = C.C1 if dtype == "f32" else C.C2
    cfg = base.small(name=f"short_{dtype}", batch=2, pos=37, needles=0, topk=64 if dtype == "f32" else 512,
                     compress="all", compress_tokens=38)
    print(f"[case] short {dtype}", flush=True)
    r = Run(cfg).run().check_all()
    idx = dev_to_np(r.step.idx)
    assert (idx[:, 0, :9] >= 0).all() and (idx[:, 0, 9:] == -1).all()


@pytest.mark.parametrize("mask", [1, 2, 3, 4, 5, 6, 7])
def test_branch_subsets_bf16(mask):
    cfg = C.C2.small(name=f"mask{mask}", batch=2, pos=4097, branches=mask, needles=4)
    print(f"[case] mask {mask}", flush=True)
    Run(cfg).run().check_all()


def test_f32_odd_heads_d128_and_bf16_h16_d64():
    a = C.C1.small(name="f32_h5_d128", heads=5, dim=128, batch=2, pos=999, needles=2, compress_tokens=1000)
    print("[case] f32 H=5 d=128", flush=True)
    Run(a).run().check_all()
    b = C.C2.small(name="bf16_h16_d64", heads=16, dim=64, idx_heads=16, idx_dim=32, batch=2, pos=3001,
                   topk=64, needles=4)
    print("[case] bf16 H=16 d=64", flush=True)
    Run(b).run().check_all()


def test_sink_and_explicit_scale():
    cfg = C.C2.small(name="sink", batch=2, pos=2050, needles=2)
    r = Run(cfg).run()
    sink = torch.linspace(-2.0, 3.0, cfg.heads, device="cuda", dtype=torch.float32)
    import compressed_attention_02_amd as V
    kw = r.step.attn_kwargs()
    kw["scale"] = 0.05
    V.decode(r.t["q"], r.t["pos"], r.step.o, sink=sink, **kw)
    torch.cuda.synchronize()
    rows = [(b, 0) for b in range(cfg.batch)]
    idx = dev_to_np(r.step.idx)
    caches = {n: r.f64(n) for n in ("kc", "vc", "kh", "vh", "k_raw", "v_raw")}
    q = O.as_f64(r.g["q"], cfg.dtype)
    for b, i in rows:
        o, l = O.decode_query(q[b, 0], cfg.pos, scale=0.05, sink=sink.cpu().numpy().astype(np.float64),
                              branches=7, m=cfg.m, m_hca=cfg.m_hca, window=cfg.window, idx=idx[b, 0],
                              raw_start=int(r.g["raw_start"][b]), **{k: v[b] for k, v in caches.items()})
        assert_close(dev_to_np(r.step.o)[b, 0], o, "bf16", "sink o")
        assert_close(dev_to_np(r.step.lse)[b, 0], l, "bf16", "sink lse")


def test_determinism_and_idx_permutation():
    cfg = SMALL["c3_small"]
    r = Run(cfg).run()
    o1, l1, i1 = (dev_to_np(x).copy() for x in (r.step.o, r.step.lse, r.step.idx))
    r.step.step(fused=False)
    torch.cuda.synchronize()
    assert np.array_equal(o1, dev_to_np(r.step.o))
    assert np.array_equal(l1, dev_to_np(r.step.lse))
    assert np.array_equal(i1, dev_to_np(r.step.idx))
    # the fused step is deterministic too (its split of the key list differs)
    r.step.step()
    torch.cuda.synchronize()
    of, lf = dev_to_np(r.step.o).copy(), dev_to_np(r.step.lse).copy()
    r.step.step()
    torch.cuda.synchronize()
    assert np.array_equal(of, dev_to_np(r.step.o)) and np.array_equal(lf, dev_to_np(r.step.lse))
    assert np.array_equal(i1, dev_to_np(r.step.idx))
    # the selected blocks in reverse order give the same output up to rounding order
    rev = torch.flip(r.step.idx, dims=[2]).contiguous()
    r.step.idx.copy_(rev)
    r.step.run_attn()
    torch.cuda.synchronize()
    o2 = dev_to_np(r.step.o)
    assert np.max(np.abs(o2 - o1)) <= 1e-6 * max(1.0, np.abs(o1).max())


def test_incremental_compress_bitwise():
    import compressed_attention_02_amd as V
    cfg = C.C5.small(name="incr", pos=4096, tq=512, needles=0)
    r = Run(cfg)
    t = r.t
    for ratio, lg, kn, vn in ((4, "logit_csa", "kc", "vc"), (128, "logit_hca", "kh", "vh")):
        V.compress(t["k_raw"], t["v_raw"], t[lg], t["raw_start"], t[kn], t[vn], t0=4096, n=512, ratio=ratio)
        torch.cuda.synchronize()
        one_k, one_v = t[kn].clone(), t[vn].clone()
        t[kn].zero_()
        t[vn].zero_()
        V.compress(t["k_raw"], t["v_raw"], t[lg], t["raw_start"], t[kn], t[vn], t0=4096, n=256, ratio=ratio)
        V.compress(t["k_raw"], t["v_raw"], t[lg], t["raw_start"], t[kn], t[vn], t0=4352, n=256 + 3, ratio=ratio)
        torch.cuda.synchronize()
        lo, hi = 4096 // ratio, (4096 + 512) // ratio
        assert torch.equal(one_k[:, lo:hi], t[kn][:, lo:hi])
        assert torch.equal(one_v[:, lo:hi], t[vn][:, lo:hi])


@pytest.mark.parametrize("name", ["c1_tiny_f32", "c2_small", "c3_small", "c4_small", "c2_b32"])
def test_fused_decode_step(name):
    # v4attn_decode_step: the HCA + window attention shares the selection's launch;
    # idx must equal the separate index_topk's bit for bit
    cfg = SMALL[name] if name != "c2_b32" else C.C2.small(name="c2_b32", batch=32, pos=4097, needles=4)
    if name == "c4_small":
        cfg = cfg.small(compress_tokens=1024 + (cfg.pos % cfg.m_hca))
    print(f"[case] fused {name}", flush=True)
    r = Run(cfg).run(fused=True).check_all()
    idx_fused = dev_to_np(r.step.idx).copy()
    o_fused = dev_to_np(r.step.o).copy()
    r.run(fused=False)
    assert np.array_equal(dev_to_np(r.step.idx), idx_fused)
    assert_close(o_fused, dev_to_np(r.step.o), cfg.dtype, "fused vs separate o")


@pytest.mark.parametrize("mask", [1, 2, 3, 4, 5, 6, 7])
def test_fused_branch_subsets(mask):
    cfg = C.C2.small(name=f"fmask{mask}", batch=2, pos=4097, branches=mask, needles=4)
    print(f"[case] fused mask {mask}", flush=True)
    Run(cfg).run(fused=True).check_all()


def test_fused_short_context_and_small_topk():
    # a row with no HCA entry yet and fewer visible blocks than k; k = 32 is a
    # single partial chunk
    cfg = C.C2.small(name="fshort", batch=2, pos=37, needles=0, topk=32, compress="all", compress_tokens=38)
    print("[case] fused short", flush=True)
    Run(cfg).run(fused=True).check_all()


@pytest.mark.parametrize("heads", [48, 80])
def test_step_odd_head_tile_counts(heads):
    # 3 and 5 tiles of 16 heads: the CSA launch's head groups must divide the tile
    # count, and the attention kernels take the KP=2 (<= 4 tiles) and KP=1 forms
    cfg = C.C2.small(name=f"h{heads}", heads=heads, batch=2, pos=4097, needles=4)
    print(f"[case] step heads={heads}", flush=True)
    Run(cfg).run(fused=True).check_all()
    Run(cfg).run(fused=False).check_all()


@pytest.mark.parametrize("tq", [8, 24, 64])
def test_prefill_index_two_sequences(tq):
    # the prefill form of the indexer score (workgroups of 8 query rows sharing each
    # key tile) over two sequences, checked row by row (the chunk starts on a block
    # boundary, as compression needs; its rows cover every position in between)
    cfg = C.C5.small(name=f"pf_ix{tq}", batch=2, pos=8192, tq=tq, needles=8)
    print(f"[case] prefill index two sequences tq={tq}", flush=True)
    r = Run(cfg)
    r.step.run_compress()
    r.step.run_index()
    torch.cuda.synchronize()
    r.check_topk()


def test_prefill_index_threshold_mode_and_repair():
    # rows of at least 256 score tiles take the threshold mode (a sampled pass sets
    # each row's threshold; tiles with at most 8 keys above it report them without
    # rounds or stores).  Sequence 0's sampled tiles (every 64th) are scaled up 8x, so
    # its threshold lands above its true k-th score: its rows are flagged and redone
    # exactly; sequence 1 takes the threshold path.  Both must match the oracle.
    cfg = C.C5.small(name="pf_theta", batch=2, pos=262144, tq=16, needles=8)
    print("[case] prefill index threshold mode and repair", flush=True)
    g = synth.generate(cfg)
    ki = synth.bf16_bits_to_f32(g["ki"]).astype(np.float64)
    n = ki.shape[1]
    sampled = (np.arange(n) // 256) % 64 == 0
    ki[0, sampled] *= 8.0
    g["ki"] = synth.f32_to_bf16_bits(ki.astype(np.float32))
    r = Run(cfg, gen=g)
    r.step.run_compress()
    r.step.run_index()
    torch.cuda.synchronize()
    r.check_topk()
    # the premise, from the oracle's scores: each of sequence 0's rows has its
    # threshold (the r-th largest sampled score, r = 3 k n_s / n_vis + 16) above its
    # k-th score, so only the repair pass can have selected it; sequence 1's rows not
    for b in range(2):
        for i in (0, cfg.tq - 1):
            s = r.oracle_scores(b, i)
            smp = np.sort(s[sampled[:s.size]])[::-1]
            rank = 3 * cfg.topk * smp.size // s.size + 16
            assert (smp[rank - 1] > np.sort(s)[::-1][cfg.topk - 1]) == (b == 0)
