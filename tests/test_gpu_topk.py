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
    # fewer visible blocks than k, exactly k, and one more than k; rows whose last
    # tile of 256 holds 1 or 3 blocks, with the tile reports short of k (the whole-row
    # path) and covering k (the report of a tile with fewer than 8 elements)
    for n_vis, k in ((100, 128), (128, 128), (129, 128), (3000, 1024), (2049, 128), (2051, 128), (4353, 128),
                     (4355, 136)):
        qi, wi, ki, pos, rng = _inputs(n_vis + 5, seed=n_vis)
        pos[:] = 4 * n_vis + 2
        kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
        idx, _ = _run(qi, wi, kb, pos, k)
        s = _scores(qi, wi, kb[:, :n_vis])
        check_topk_row(idx[0, 0], s, k, f"n_vis={n_vis}")


@pytest.mark.parametrize("n_vis,k,zero_rows", [(3000, 1024, 1), (65536, 512, 256)])
def test_key_range_one_bin_past_histogram(n_vis, k, zero_rows):
    """Keys spanning [key(0.0), key(~2.0156)]: the order-preserving keys of positive
    floats are their bits with the top bit set, so the span is 2^30 + ~2^16, which at
    bins of 2^17 keys needs 8193 bins, one more than the histogram holds; the bin width
    must grow to 2^18.  (3000, 1024): the tile reports fall short of k and the whole
    row is ranked; (65536, 512): the reports cover k and tile 0, all zero scores,
    reports key(0.0) into the ranking of reported keys."""
    qi, wi, ki, pos, rng = _inputs(n_vis, seed=7)
    ki[0, :zero_rows] = 0.0                          # scores exactly 0
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    s = _scores(qi, wi, kb)
    top = n_vis // 2 + 3
    ki[0] *= 1.0 / s.max()                           # scores are positively homogeneous in the key row
    ki[0, top] *= 2.0156 * s.max() / s[top]
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    s = _scores(qi, wi, kb)
    bits = np.sort(s).astype(np.float32).view(np.uint32)
    assert s.min() == 0.0 and int(np.argmax(s)) == top
    assert (1 << 30) + 4096 <= int(bits[-1]) < (1 << 30) + (1 << 17) - 4096   # the span the case is about
    idx, sel = _run(qi, wi, kb, pos, k)
    check_topk_row(idx[0, 0], s, k, f"n_vis={n_vis}")
    np.testing.assert_allclose(sel[0, 0], s[idx[0, 0]], rtol=1e-5)


@pytest.mark.parametrize("n_tied", [30, 100])
def test_cut_inside_ties_of_one_histogram_bin(n_tied):
    """500 boosted blocks with distinct scores lead the row, then n_tied copies of one
    key row (bit-identical scores) at ranks 501..500 + n_tied: k = 512 cuts inside the
    ties, so the lowest-id 12 of them are picked.  30 ties rank inside one bin of the
    first histogram level (at most 64 keys: one wave counts them); 100 take a second
    level."""
    n, k = 65536, 512
    qi, wi, ki, pos, rng = _inputs(n, seed=11)
    u = (wi[0, 0].astype(np.float64)[:, None] * O.as_f64(qi[0, 0], "bf16")).sum(0)
    u /= np.linalg.norm(u)
    rows = rng.choice(n, 500 + n_tied, replace=False)
    lead, tied = rows[:500], np.sort(rows[500:])
    ki[0, lead] += (40.0 + 0.05 * np.arange(500))[:, None] * u
    ki[0, tied] = ki[0, tied[0]] + 30.0 * u
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    s = _scores(qi, wi, kb)
    order = np.argsort(-s, kind="stable")
    assert set(order[:500].tolist()) == set(lead.tolist())           # the leaders lead,
    assert np.all(s[tied] == s[tied[0]]) and s[tied[0]] > np.delete(s, np.concatenate([lead, tied])).max()  # ties next
    idx, _ = _run(qi, wi, kb, pos, k)
    ref = O.topk_select(s, k)
    assert set(tied[:12].tolist()) <= set(ref.tolist())
    assert list(idx[0, 0]) == list(ref)


# ---------------------------------------------------------------- through the decode step
def _run_step(qi, wi, ki, pos, k, heads=128, d=128, m=4, W=128):
    """The same selection through v4attn_decode_step (its candidates per group of
    waves, the exact top-k in the picks' launch, the full-report fallback)."""
    B, n = qi.shape[0], ki.shape[1]
    rng = np.random.default_rng(7)
    e = (int(pos.max()) + 1) // 128 + 1

    def bf(shape):
        return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))

    g = {"qi": qi, "wi": wi, "ki": ki, "pos": pos, "q": bf((B, 1, heads, d)), "kc": bf((B, n, d)),
         "vc": bf((B, n, d)), "kh": bf((B, e, d)), "vh": bf((B, e, d)), "k_raw": bf((B, W, d)),
         "v_raw": bf((B, W, d)), "raw_start": (pos - W + 1).astype(np.int64)}
    t = to_device(g)
    idx = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
    o = torch.empty((B, 1, heads, d), dtype=torch.float32, device="cuda")
    V.decode_step(t["qi"], t["wi"], t["ki"], t["q"], t["pos"], o, idx, ratio=m, topk=k, pos_max=int(pos.max()),
                  kc=t["kc"], vc=t["vc"], kh=t["kh"], vh=t["vh"], k_raw=t["k_raw"], v_raw=t["v_raw"],
                  raw_start=t["raw_start"], hca_ratio=128, window=W)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(dev_to_np(o)))
    return dev_to_np(idx)


@pytest.mark.parametrize("distinct", [1, 3])
def test_step_exact_ties(distinct):
    # every group's bound equals the threshold: the picks' launch falls back to the
    # selection over the reports (and, for one distinct row, over the scores)
    n, k = 32768, 512
    qi, wi, ki, pos, rng = _inputs(n)
    rows = rng.standard_normal((distinct, ki.shape[2]))
    ki[0] = rows[rng.integers(0, distinct, n)]
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    print(f"[case] step ties distinct={distinct}", flush=True)
    idx = _run_step(qi, wi, kb, pos, k)
    assert list(idx[0, 0]) == list(O.topk_select(_scores(qi, wi, kb), k))


def test_step_clustered_winners():
    # 900 winners in about four tiles: their group keeps 64 and its bound reaches T
    n, k = 262144, 1024
    qi, wi, ki, pos, rng = _inputs(n, seed=1)
    u = (wi[0, 0].astype(np.float64)[:, None] * O.as_f64(qi[0, 0], "bf16")).sum(0)
    u /= np.linalg.norm(u)
    ki[0, 5000:5900] += 4.0 * 8.0 * u
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    print("[case] step clustered", flush=True)
    idx = _run_step(qi, wi, kb, pos, k)
    assert np.array_equal(idx, _run(qi, wi, kb, pos, k)[0])
    check_topk_row(idx[0, 0], _scores(qi, wi, kb), k, "step clustered")


@pytest.mark.parametrize("heads", [64, 128])
def test_step_max_topk_and_batch(heads):
    # k = 2048: 64 groups of candidates, a pool of 4096
    n, k = 65536, 2048
    qi, wi, ki, pos, rng = _inputs(n, B=3, seed=2)
    pos[1] -= 4 * 777 + 2
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    print(f"[case] step k=2048 heads={heads}", flush=True)
    idx = _run_step(qi, wi, kb, pos, k, heads=heads)
    assert np.array_equal(idx, _run(qi, wi, kb, pos, k)[0])
    for b in range(3):
        nv = O.n_visible(int(pos[b]), 4)
        s = O.index_scores(O.as_f64(qi[b, 0], "bf16"), wi[b, 0].astype(np.float64), O.as_f64(kb[b, :nv], "bf16"))
        check_topk_row(idx[b, 0], s, k, f"step b={b}")


def test_step_small_rows_and_padding():
    for n_vis, k in ((100, 128), (128, 128), (129, 128), (3000, 1024), (2049, 128), (2051, 128), (4353, 128),
                     (4355, 136)):
        qi, wi, ki, pos, rng = _inputs(n_vis + 5, seed=n_vis)
        pos[:] = 4 * n_vis + 2
        kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
        print(f"[case] step n_vis={n_vis} k={k}", flush=True)
        idx = _run_step(qi, wi, kb, pos, k)
        assert np.array_equal(idx, _run(qi, wi, kb, pos, k)[0])
        check_topk_row(idx[0, 0], _scores(qi, wi, kb[:, :n_vis]), k, f"step n_vis={n_vis}")


def test_rows_with_more_tiles_than_the_selection_holds():
    # 524288 visible blocks (a 2M-token context at m = 4): 2048 tiles of reports, more
    # than the selection's 512 threads keep in registers (3 tiles each), so the row
    # is selected by the whole-row path over its stored scores
    n, k = 524288, 1024
    qi, wi, ki, pos, rng = _inputs(n, seed=7)
    kb = synth.f32_to_bf16_bits(ki.astype(np.float32))
    print("[case] 2M-token row, whole-row path", flush=True)
    idx, sel = _run(qi, wi, kb, pos, k)
    s = _scores(qi, wi, kb)
    check_topk_row(idx[0, 0], s, k, "2M")
    np.testing.assert_allclose(sel[0, 0], s[idx[0, 0]], rtol=1e-5)
    # and inside the decode step (the selection hosted by the HCA/window launch)
    print("[case] step 2M-token row", flush=True)
    assert np.array_equal(_run_step(qi, wi, kb, pos, k), idx)
