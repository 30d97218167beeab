"""The seeded input generator: shapes, determinism, rounding, planted structure."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import configs as C


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours), O.bf16_to_f64(ours).astype(np.float32))


def test_shapes_and_determinism():
    cfg = C.C2.small(pos=4099, batch=2, needles=5)
    a, b = synth.generate(cfg), synth.generate(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["q"].shape == (2, 1, 64, 128) and a["q"].dtype == np.uint16
    assert a["ki"].shape == (2, 4100 // 4, 64)
    assert a["kh"].shape == (2, 4100 // 128, 128)
    assert a["k_raw"].shape == (2, 128, 128) and int(a["raw_start"][0]) == 4099 - 127
    c = synth.generate(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(a["q"], c["q"])


def test_raw_buffers_cover_compressed_span():
    for cfg in (C.C1, C.C4.small(batch=1, pos=8192, compress_tokens=1024),
                C.C5.small(pos=2048, tq=256, needles=4)):
        assert cfg.raw_start <= cfg.compress_t0
        assert cfg.raw_start <= max(0, cfg.pos - cfg.window + 1)
        assert cfg.raw_start + cfg.raw_rows == cfg.last_pos + 1
        assert cfg.compress_t0 % cfg.m_hca == 0


def test_c1_needles_selected_by_oracle():
    cfg = C.C1
    g = synth.generate(cfg)
    p = int(g["pos"][0])
    n = O.n_visible(p, cfg.m)
    s = O.index_scores(O.as_f64(g["qi"][0, 0], "f32"), g["wi"][0, 0].astype(np.float64),
                       O.as_f64(g["ki"][0, :n], "f32"))
    sel = set(int(i) for i in O.topk_select(s, cfg.topk))
    assert set(int(i) for i in g["needles"][0]) <= sel


def test_ragged_positions():
    cfg = C.C2.small(name="rag", batch=3, pos=4097, needles=4, pos_back=(0, 1030, 3900))
    g = synth.generate(cfg)
    assert g["pos"].tolist() == [4097, 3067, 197]
    assert g["raw_start"].tolist() == [4097 - 127, 3067 - 127, 197 - 127]
    assert g["k_raw"].shape[1] == 128 and g["ki"].shape[1] == 4098 // 4
    for b in range(3):   # needles only among the blocks the sequence's query sees
        assert g["needles"][b].max() < (int(g["pos"][b]) + 1) // 4
    with pytest.raises(ValueError):
        synth.generate(C.C4.small(batch=2, pos_back=(0, 5)))   # compresses: uniform positions only


def test_sample_rows_cover_the_chunk():
    from tests.gpu_harness import sample_rows
    cfg = C.C5
    rows = [i for _, i in sample_rows(cfg)]
    assert len(rows) == 256 == len(set(rows))
    s = set(rows)
    assert set(range(8)) <= s and set(range(cfg.tq - 8, cfg.tq)) <= s
    csa = [i for i in range(cfg.tq) if (cfg.pos + i + 1) % cfg.m == 0]
    assert set(csa[:16]) <= s and set(csa[-16:]) <= s
    hca = [i for i in range(cfg.tq) if (cfg.pos + i + 1) % cfg.m_hca == 0]
    assert len(hca) == 32 and set(hca) <= s and {i - 1 for i in hca} <= s
