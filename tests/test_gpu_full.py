"""Parity at the full configurations, in the launch configuration bench.py uses.

Decode configurations are checked on every sequence; the 4096-query prefill chunk
on 256 sampled rows (the first and last rows, rows where a CSA block completes near
both ends of the chunk, every row where an HCA entry completes and the row before
it, random rows), which the oracle computes one by one.
"""
from dataclasses import replace

import pytest

from synth import configs as C
from tests.gpu_harness import Run, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["stages", "decode_step"])
@pytest.mark.parametrize("name", ["c2_flash_decode_b8_128k", "c3_pro_decode_b1_1m", "c4_hca_decode_b16_1m"])
def test_full_decode_configs(name, fused):
    # fused=True is the launch configuration bench.py times (v4attn_decode_step)
    cfg = C.CONFIGS[name]
    print(f"[case] full {name} fused={fused}", flush=True)
    r = Run(cfg).run(fused=bool(fused)).check_all()
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


@pytest.mark.timeout(400)
def test_full_prefill_sampled():
    cfg = C.C5
    print("[case] full c5 prefill", flush=True)
    r = Run(cfg).run()
    r.check_compress()
    rows = sample_rows(cfg)
    assert len(rows) == 256
    r.check_topk(rows)
    r.check_attn(rows)


@pytest.mark.timeout(900)
def test_full_prefill_two_row_groups():
    # A chunk of 8192 queries at 1M context: its index scores and tile reports (about
    # 1.1 MB a row) exceed what the index call takes at a time, so its rows run in two
    # groups (the second from about row 7760), whose launches carry a row offset.
    # Sampled rows of both groups: every 128th row, the rows around the boundary and
    # the last 8.
    cfg = replace(C.C5, name="c5_prefill_8192_on_1m", tq=8192, compress_tokens=8192)
    print("[case] full prefill 8192 on 1M (two index row groups)", flush=True)
    r = Run(cfg).run()
    rows = sorted(set(range(0, cfg.tq, 128)) | set(range(7744, 7776)) | set(range(cfg.tq - 8, cfg.tq)))
    pairs = [(0, i) for i in rows]
    r.check_topk(pairs)
    r.check_attn(pairs)
