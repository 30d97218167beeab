"""FP8 entries written by v4attn_compress ([wiki] the quantization and deployment
section: FP8 KV caches) against the fp64 oracle, through the C ABI.

The oracle pools the entries in fp64 (with the norm and the rotation where asked)
and quantises each row with oracle.fp8_quantize_rows: scale max|y| / 448, codes the
nearest E4M3 values of y / scale, ties to the even code.  The GPU pools in fp32, so
its y differs from the oracle's in the last fp32 bits: its scales must agree to 1e-5
relative, and its codes must be the oracle's except where the oracle's y / scale lies
within 1e-4 (relative) of the midpoint between two E4M3 values; there the code must be
one of those two.  The decoded rows must lie within half an E4M3 step of the oracle's
entries.  Then FP8 entries pooled from raw tokens serve as the HCA cache of a decode,
whose output must match the oracle's over the GPU's codes and scales.
"""
import numpy as np
import pytest
import torch

import compressed_attention_02_amd as V
import oracle as O
import synth
from synth import configs as C
from compressed_attention_02_amd.layer import to_device
from tests.gpu_harness import dev_to_np

pytestmark = pytest.mark.gpu
EPS = 1e-5
R, BASE = 64, 1e4


def _check_fp8_rows(codes, scales, ref, what):
    oc, osc = O.fp8_quantize_rows(ref)
    np.testing.assert_allclose(scales, osc, rtol=1e-5, atol=0, err_msg=f"{what}: scales")
    q = ref / np.where(osc > 0, osc, 1.0)[:, None]
    bad = codes != oc
    if bad.any():
        vg, vo = O.fp8_e4m3_decode(codes[bad]), O.fp8_e4m3_decode(oc[bad])
        mid = (vg + vo) / 2
        near = np.abs(q[bad] - mid) <= 1e-4 * np.abs(mid) + 1e-30
        assert near.all(), f"{what}: {int((~near).sum())} codes off the oracle's away from a rounding midpoint"
        # the two codes are neighbours: no E4M3 value lies strictly between them
        mags = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
        lo, hi = np.minimum(np.abs(vg), np.abs(vo)), np.maximum(np.abs(vg), np.abs(vo))
        between = ((mags[None, :] > lo[:, None]) & (mags[None, :] < hi[:, None])).any(axis=1)
        assert not between.any() and np.array_equal(np.sign(vg), np.sign(vo)), f"{what}: codes not neighbours"
    # decoded rows within half a step (in units of the scale) of the oracle's entries
    aq = np.abs(q)
    step = np.where(aq >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(aq, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(O.fp8_rows(codes, scales) - ref)
    assert np.all(err <= (step / 2 * (1 + 1e-3)) * osc[:, None] + 1e-6 * np.abs(ref).max()), f"{what}: values"
    return bad.mean()


CASES = {
    # HCA pooling of bf16 rows of 128 (K and V), no norm or rotation
    "bf16_hca": dict(base="c4", ratio="m_hca", hv=True, norm=False, rope=False),
    # CSA pooling of fp32 rows of 64, entries RMS-normalised
    "f32_csa_norm": dict(base="c1", ratio="m", hv=True, norm=True, rope=False),
    # fp32 HCA pooling
    "f32_hca": dict(base="c1", ratio="m_hca", hv=True, norm=False, rope=False),
    # the pages' shared entries: K alone, rows of 512, RMSNorm and partial RoPE
    "bf16_shared_512": dict(base="c4_512", ratio="m_hca", hv=False, norm=True, rope=True),
    "bf16_shared_512_csa": dict(base="c4_512", ratio="m", hv=False, norm=True, rope=True),
}


def _cfg(base):
    if base == "c4":
        return C.C4.small(name="f8c4", batch=2, pos=4096 + 77, compress_tokens=1024 + 77)
    if base == "c4_512":
        return C.C4.small(name="f8c6", batch=2, pos=4096 + 77, compress_tokens=1024 + 77, dim=512, shared_kv=True)
    return C.C1.small(name="f8c1", batch=2, pos=999, compress_tokens=1000)


@pytest.mark.parametrize("case", list(CASES))
def test_compress_fp8_entries(case):
    k = CASES[case]
    cfg = _cfg(k["base"])
    g = synth.generate(cfg)
    t = to_device(g)
    r = getattr(cfg, k["ratio"])
    lg = "logit_hca" if k["ratio"] == "m_hca" else ("logit_csa" if "logit_csa" in g else "logit_hca")
    t0 = cfg.compress_t0 - cfg.compress_t0 % r
    n = cfg.last_pos + 1 - t0
    rows = (cfg.last_pos + 1) // r
    ok = torch.zeros((cfg.batch, rows, cfg.dim), dtype=torch.uint8, device="cuda")
    ks = torch.full((cfg.batch, rows), -1.0, dtype=torch.float32, device="cuda")
    ov = torch.zeros_like(ok) if k["hv"] else None
    vs = torch.full_like(ks, -1.0) if k["hv"] else None
    gk = np.random.default_rng(11).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
    gv = np.random.default_rng(12).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
    kw = {}
    if k["norm"]:
        kw.update(norm_k=torch.from_numpy(gk).cuda(), norm_eps=EPS)
        if k["hv"]:
            kw["norm_v"] = torch.from_numpy(gv).cuda()
    if k["rope"]:
        kw.update(rope_dims=R, rope_base=BASE)
    print(f"[case] fp8 compress {case} r={r} d={cfg.dim}", flush=True)
    V.compress(t["k_raw"], t["v_raw"] if k["hv"] else None, t[lg], t["raw_start"], ok, ov, t0=t0, n=n, ratio=r,
               k_scale=ks, v_scale=vs, **kw)
    torch.cuda.synchronize()
    kr = O.as_f64(g["k_raw"], cfg.dtype)
    vr = O.as_f64(g["v_raw"], cfg.dtype) if k["hv"] else None
    codes_k, sc_k = dev_to_np(ok), dev_to_np(ks)
    codes_v, sc_v = (dev_to_np(ov), dev_to_np(vs)) if k["hv"] else (None, None)
    rate = []
    for b in range(cfg.batch):
        rs = int(g["raw_start"][b])
        ids, ref_k = O.compress_entries(kr[b], g[lg][b], rs, t0, n, r, gain=gk if k["norm"] else None, eps=EPS,
                                        rope_dims=R if k["rope"] else 0, rope_base=BASE)
        rate.append(_check_fp8_rows(codes_k[b, ids], sc_k[b, ids], ref_k, f"k b={b}"))
        if k["hv"]:
            _, ref_v = O.compress_entries(vr[b], g[lg][b], rs, t0, n, r, gain=gv if k["norm"] else None, eps=EPS)
            rate.append(_check_fp8_rows(codes_v[b, ids], sc_v[b, ids], ref_v, f"v b={b}"))
        # rows outside the pooled range are left alone
        keep = np.ones(rows, dtype=bool)
        keep[ids] = False
        assert not codes_k[b, keep].any() and np.all(sc_k[b, keep] == -1.0)
    assert max(rate) < 1e-3   # codes off the oracle's: only at rounding midpoints, rare


def test_zero_entries_get_zero_scale():
    # raw rows of zeros pool to zero entries: scale 0 and zero codes (no 0/0)
    cfg = C.C4.small(name="f8z", batch=1, pos=4096 + 77, compress_tokens=1024 + 77)
    g = synth.generate(cfg)
    t = to_device(g)
    t["k_raw"].zero_()
    r = cfg.m_hca
    t0 = cfg.compress_t0 - cfg.compress_t0 % r
    n = cfg.last_pos + 1 - t0
    rows = (cfg.last_pos + 1) // r
    ok = torch.full((1, rows, cfg.dim), 0x55, dtype=torch.uint8, device="cuda")
    ov = torch.zeros_like(ok)
    ks, vs = (torch.full((1, rows), -1.0, device="cuda") for _ in range(2))
    print("[case] fp8 compress of zero rows", flush=True)
    V.compress(t["k_raw"], t["v_raw"], t["logit_hca"], t["raw_start"], ok, ov, t0=t0, n=n, ratio=r, k_scale=ks,
               v_scale=vs)
    torch.cuda.synchronize()
    ids = np.arange(t0 // r, t0 // r + n // r)
    assert not dev_to_np(ok)[0, ids].any() and np.all(dev_to_np(ks)[0, ids] == 0.0)
    assert np.all(dev_to_np(vs)[0, ids] > 0.0)


def test_fp8_entries_feed_the_attention():
    # every HCA entry of the context pooled to FP8 by v4attn_compress, then attended
    # (HCA branch alone, FP8 caches): the output must match the oracle's over the
    # GPU's own codes and scales
    cfg = C.C4.small(name="f8e2e", batch=2, pos=4096 + 77, compress="all", heads=64)
    g = synth.generate(cfg)
    t = to_device(g)
    r = cfg.m_hca
    n = cfg.last_pos + 1
    rows = n // r
    B, H, d = cfg.batch, cfg.heads, cfg.dim
    kh = torch.zeros((B, rows, d), dtype=torch.uint8, device="cuda")
    vh = torch.zeros_like(kh)
    khs, vhs = (torch.zeros((B, rows), dtype=torch.float32, device="cuda") for _ in range(2))
    print("[case] fp8 entries from compress feed the attention", flush=True)
    V.compress(t["k_raw"], t["v_raw"], t["logit_hca"], t["raw_start"], kh, vh, t0=0, n=n, ratio=r,
               k_scale=khs, v_scale=vhs)
    o = torch.zeros((B, 1, H, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, 1, H), dtype=torch.float32, device="cuda")
    V.decode(t["q"], t["pos"], o, lse=lse, kh=kh, vh=vh, branch_mask=V.HCA, csa_ratio=cfg.m, hca_ratio=r,
             window=cfg.window, topk=0, pos_max=cfg.last_pos, kh_scale=khs, vh_scale=vhs)
    torch.cuda.synchronize()
    kh_g, vh_g = O.fp8_rows(dev_to_np(kh), dev_to_np(khs)), O.fp8_rows(dev_to_np(vh), dev_to_np(vhs))
    qv = O.as_f64(g["q"], cfg.dtype)
    go, gl = dev_to_np(o), dev_to_np(lse)
    for b in range(B):
        ref_o, ref_l = O.decode_query(qv[b, 0], int(g["pos"][b]), branches=V.HCA, m=cfg.m, m_hca=r,
                                      window=cfg.window, kh=kh_g[b], vh=vh_g[b])
        mx = np.abs(go[b, 0] - ref_o).max()
        mr = np.abs(go[b, 0] - ref_o).sum() / np.abs(ref_o).sum()
        assert mx <= 1e-2 and mr <= 2e-3, f"b={b}: max-abs {mx:.3e}, mean-relative {mr:.3e}"
        np.testing.assert_allclose(gl[b, 0], ref_l, rtol=0, atol=1e-2)
