"""Top-k selection edge cases on the GPU: exact ties, all-equal scores (whole-row
path), clustered winners (tile rescans), the largest k, and the selected scores."""
import numpy as np
import pytest
import torch

import compressed_attention_02_amd as V
import oracle as O
import synth
from compressed_attention_02_amd.layer import to_device
from tests.gpu_harness import check_topk_row, dev_to_np

pytestmark = pytest.mark.gpu


def _run(qi, wi, ki, pos, k, m=4):
    t = to_device({"qi": qi, "wi": wi, "ki": ki, "pos": pos})
    B, Tq = qi.shape[:2]
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
    sel = torch.zeros((B, Tq, k), dtype=torch.float32, device="cuda")
    V.index_topk(t["qi"], t["wi"], t["ki"], t["pos"], idx, ratio=m, topk=k,
                 pos_max=int(pos.max()) + Tq - 1, sel_scores=sel)
    torch.cuda.synchronize()
    return dev_to_np(idx), dev_to_np(sel)


def _inputs(n_blocks, B=1, HI=64, dI=64, seed=0):
    rng = np.random.default_rng(seed)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((B, 1, HI, dI)).astype(np.float32))
    wi = rng.uniform(0, 1, (B, 1, HI)).astype(np.float32)
    ki = rng.standard_normal((B, n_blocks, dI))
    pos = np.full(B, 4 * n_blocks - 1, dtype=np.int64)
    return qi, wi, ki, pos, rng


def _scores(qi, wi, ki_bits, b=0):
    return O.index_scores(O.as_f64(qi[b, 0], "bf16"), wi[b, 0].astype(np.float64), O.as_f64(ki_bits[b], "bf16"))


@pytest.mark.parametrize("distinct", [1, 3])
def test_exact_ties_lowest_ids_win(distinct):
    n, k = 32768, 512
    qi, wi, ki, pos, rng = _inputs(n)
    rows = rng.standard_normal((distinct, ki.shape[2]))
    ki[0] = rows[rng.integers(0, distinct, n)]
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    idx, _ = _run(qi, wi, kb, pos, k)
    s = _scores(qi, wi, kb)
    # identical key rows give bit-identical scores on both sides: the sets must match exactly
    assert list(idx[0, 0]) == list(O.topk_select(s, k))


def test_clustered_winners_force_rescans():
    n, k = 262144, 1024
    qi, wi, ki, pos, rng = _inputs(n, seed=1)
    u = (wi[0, 0].astype(np.float64)[:, None] * O.as_f64(qi[0, 0], "bf16")).sum(0)
    u /= np.linalg.norm(u)
    ki[0, 5000:5900] += 4.0 * 8.0 * u        # 900 winners packed into ~4 tiles
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    idx, sel = _run(qi, wi, kb, pos, k)
    s = _scores(qi, wi, kb)
    check_topk_row(idx[0, 0], s, k, "clustered")
    assert set(range(5000, 5900)) <= set(idx[0, 0].tolist())
    np.testing.assert_allclose(sel[0, 0], s[idx[0, 0]], rtol=1e-5)


def test_max_topk_and_batch():
    n, k = 65536, 2048
    qi, wi, ki, pos, rng = _inputs(n, B=3, seed=2)
    pos[1] -= 4 * 777 + 2            # a shorter, unaligned second sequence
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    idx, sel = _run(qi, wi, kb, pos, k)
    for b in range(3):
        nv = O.n_visible(int(pos[b]), 4)
        s = O.index_scores(O.as_f64(qi[b, 0], "bf16"), wi[b, 0].astype(np.float64), O.as_f64(kb[b, :nv], "bf16"))
        check_topk_row(idx[b, 0], s, k, f"b={b}")
        np.testing.assert_allclose(sel[b, 0], s[idx[b, 0]], rtol=1e-5)


def test_small_rows_and_padding():
    # fewer visible blocks than k, exactly k, and one more than k; then rows whose
    # last wave of 64 holds 1 or 3 blocks while the reports still cover k (the
    # report of a wave with fewer than 4 elements)
    for n_vis, k in ((100, 128), (128, 128), (129, 128), (3000, 1024), (2049, 128), (2051, 128)):
        qi, wi, ki, pos, rng = _inputs(n_vis + 5, seed=n_vis)
        pos[:] = 4 * n_vis + 2
        kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
        idx, _ = _run(qi, wi, kb, pos, k)
        s = _scores(qi, wi, kb[:, :n_vis])
        check_topk_row(idx[0, 0], s, k, f"n_vis={n_vis}")
