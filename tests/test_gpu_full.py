"""Parity at the full configurations, in the launch configuration bench.py uses.

Decode configurations are checked on every sequence; the 4096-query prefill chunk
on sampled rows (first, last, rows where an HCA entry completes, random rows),
which the oracle computes one by one.
"""
import pytest

from synth import configs as C
from tests.gpu_harness import Run, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True, "one_launch"], ids=["stages", "decode_step", "one_launch"])
@pytest.mark.parametrize("name", ["c2_flash_decode_b8_128k", "c3_pro_decode_b1_1m", "c4_hca_decode_b16_1m"])
def test_full_decode_configs(name, fused):
    # fused=True is the launch configuration bench.py times (v4attn_decode_step);
    # "one_launch" is the same step with the one-launch form switched on
    import compressed_attention_02_amd as V
    cfg = C.CONFIGS[name]
    print(f"[case] full {name} fused={fused}", flush=True)
    V.set_one_launch_step(fused == "one_launch")
    try:
        r = Run(cfg).run(fused=bool(fused)).check_all()
    finally:
        V.set_one_launch_step(False)
    # planted needles are selected (structural: they carry +3 sigma of relevance)
    if cfg.needles:
        import numpy as np
        from tests.gpu_harness import dev_to_np
        idx = dev_to_np(r.step.idx)
        for b in range(cfg.batch):
            assert set(r.g["needles"][b].tolist()) <= set(idx[b, 0].tolist())


def test_full_c1():
    print("[case] full c1", flush=True)
    Run(C.C1).run().check_all()


def test_full_prefill_sampled():
    cfg = C.C5
    print("[case] full c5 prefill", flush=True)
    r = Run(cfg).run()
    r.check_compress()
    rows = sample_rows(cfg, n_random=10)
    r.check_topk(rows)
    r.check_attn(rows)
