"""Boundary cases of the HIP path against the fp64 oracle (GPU).

* Ragged batches: the sequences of one batch at different positions (different
  visible block counts, HCA entry counts and window starts), in the stage-by-stage
  path, the decode step, and the batch-invariant plans.
* bf16 output (out_dtype BF16): o is the fp32 result rounded to nearest even, bit
  for bit, in every path that writes o (a split's direct write, the merge kernel,
  the fp32 kernels), and within the bf16 tolerances of the oracle plus the output
  rounding.
* NaN poison: every cache row a query must not read (unselected CSA rows, rows past
  a sequence's visible blocks and HCA entries, raw rows outside its window) holds
  NaN; the outputs must stay finite and equal the oracle's.  A kernel that reads
  any such row turns its output into NaN.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import configs as C
from tests.gpu_harness import TOL, Run, dev_to_np

pytestmark = pytest.mark.gpu

RAGGED = {
    "c2_ragged": C.C2.small(name="c2_ragged", batch=3, pos=16389, needles=4, pos_back=(0, 3110, 16389 - 300)),
    "c3_ragged": C.C3.small(name="c3_ragged", batch=3, pos=65539, needles=8, pos_back=(0, 3110, 65539 - 300)),
    "c4_ragged": C.C4.small(name="c4_ragged", batch=5, pos=16461, compress="none", compress_tokens=0,
                            pos_back=(0, 77, 4096, 16461 - 130, 16461 - 60)),
}


@pytest.mark.parametrize("inv", [False, True], ids=["default", "invariant"])
@pytest.mark.parametrize("fused", [False, True], ids=["stages", "decode_step"])
@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_batch(name, fused, inv):
    cfg = RAGGED[name]
    print(f"[case] ragged {name} fused={fused} invariant={inv}", flush=True)
    r = Run(cfg, batch_invariant=inv).run(fused=fused).check_all()
    if cfg.needles:
        idx = dev_to_np(r.step.idx)
        for b in range(cfg.batch):
            assert set(r.g["needles"][b].tolist()) <= set(idx[b, 0].tolist())


# ---------------------------------------------------------------- bf16 output
OUT_CASES = {
    # one split per query (n_keys <= 128): the attention kernel writes o itself
    "direct_swa": (C.C2.small(name="o_swa", batch=2, pos=4097, branches=4, needles=0), False),
    # a prefill of 640 rows covers the chip with one split per row
    "direct_prefill": (C.C5.small(name="o_pf", pos=8192, tq=640, needles=8), False),
    # splits merged by the merge kernel, stages and decode step
    "merge_stages": (C.C2.small(name="o_c2", batch=3, pos=16389, needles=8), False),
    "merge_step": (C.C3.small(name="o_c3", pos=65539, needles=16), True),
    # fp32 attention kernel, merged and direct
    "f32_merge": (C.C1, False),
    "f32_direct": (C.C1.small(name="o_f32swa", branches=4, needles=0), False),
}


def _bf16_bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("case", list(OUT_CASES))
def test_bf16_output(case):
    cfg, fused = OUT_CASES[case]
    print(f"[case] bf16 out {case}", flush=True)
    g = synth.generate(cfg)
    r32 = Run(cfg, gen=g).run(fused=fused)
    r16 = Run(cfg, gen=g, out_bf16=True).run(fused=fused)
    o32 = dev_to_np(r32.step.o)
    o16 = dev_to_np(r16.step.o)
    assert o16.dtype == np.uint16
    # the same kernels and plan compute the same fp32 result; bf16 stores its RNE
    assert np.array_equal(o16, _bf16_bits(o32))
    assert np.array_equal(dev_to_np(r16.step.lse), dev_to_np(r32.step.lse))
    # against the oracle: the configuration's tolerance plus the output rounding
    # (round to nearest even moves a value by at most 2^-8 of its magnitude)
    rows = [(b, i) for b in range(cfg.batch) for i in range(cfg.tq)]
    if cfg.tq > 64:
        rows = [(0, i) for i in (0, 1, 2, 3, 127, 128, 255, 400, cfg.tq - 1)]
    ro, _ = r16.oracle_attn(rows)
    go = np.stack([O.bf16_to_f64(o16[b, i]) for b, i in rows])
    err = np.abs(go - ro)
    assert np.all(np.isfinite(go))
    assert np.all(err <= TOL[cfg.dtype]["max_abs"] + 2.0 ** -8 * np.abs(ro)), float(err.max())
    if cfg.dtype == "bf16":
        assert err.sum() / np.abs(ro).sum() <= TOL["bf16"]["mean_rel"] + 2.0 ** -8


# ---------------------------------------------------------------- NaN poison
POISON = {
    "c2_step": (C.C2.small(name="p_c2", batch=3, pos=16389, needles=4, pos_back=(0, 3110, 16389 - 300)), True),
    "c2_stages": (C.C2.small(name="p_c2s", batch=3, pos=16389, needles=4, pos_back=(0, 3110, 16389 - 300)), False),
    "c3_step": (C.C3.small(name="p_c3", batch=2, pos=65539, needles=8, pos_back=(0, 999)), True),
    "c1_f32": (C.C1.small(name="p_c1", compress="none", compress_tokens=0, batch=2, pos_back=(0, 1001)), False),
}


@pytest.mark.parametrize("case", list(POISON))
def test_nan_poison_rows_are_never_read(case):
    cfg, fused = POISON[case]
    print(f"[case] poison {case}", flush=True)
    g = synth.generate(cfg)
    B = cfg.batch
    # the oracle's own selection, so that every row outside it can be poisoned
    picks = []
    for b in range(B):
        p = int(g["pos"][b])
        n = O.n_visible(p, cfg.m)
        s = O.index_scores(O.as_f64(g["qi"][b, 0], cfg.dtype), g["wi"][b, 0].astype(np.float64),
                           O.as_f64(g["ki"][b, :n], cfg.dtype))
        sel = O.topk_select(s, cfg.topk)
        picks.append(sel[sel >= 0])
    # raw buffers grow by X rows before and Y after the window, all NaN
    X, Y = 100, 37
    nan16 = np.uint16(0x7FC0)
    nanv = nan16 if cfg.dtype == "bf16" else np.float32("nan")
    for nm in ("k_raw", "v_raw"):
        old = g[nm]
        new = np.full((B, old.shape[1] + X + Y, old.shape[2]), nanv, dtype=old.dtype)
        new[:, X:X + old.shape[1]] = old
        g[nm] = new
    g["raw_start"] = g["raw_start"] - X
    for b in range(B):
        p = int(g["pos"][b])
        n_vis, e_vis = O.n_visible(p, cfg.m), O.n_visible(p, cfg.m_hca)
        w_lo = max(0, p - cfg.window + 1)
        rs = int(g["raw_start"][b])
        for nm in ("k_raw", "v_raw"):   # rows before the window and after the query
            g[nm][b, :w_lo - rs] = nanv
            g[nm][b, p + 1 - rs:] = nanv
        keep = np.zeros(g["kc"].shape[1], dtype=bool)
        keep[picks[b]] = True
        for nm in ("kc", "vc"):
            g[nm][b, ~keep] = nanv
        g["ki"][b, n_vis:] = nanv
        for nm in ("kh", "vh"):
            g[nm][b, e_vis:] = nanv
    r = Run(cfg, gen=g).run(fused=fused)
    o = dev_to_np(r.step.o)
    assert np.all(np.isfinite(o)), "a poisoned row reached the output"
    assert np.all(np.isfinite(dev_to_np(r.step.lse)))
    r.check_all()
