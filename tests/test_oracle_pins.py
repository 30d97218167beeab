"""Pins of the fp64 oracle against things other than itself.

* hand-derived worked examples (tests/golden/worked_examples.json),
* the pages' structural constants (tests/golden/pages_constants.json),
* closed forms (identity pooling, plain means, one-hot pooling, one key, constant
  values, the sink's effect on the weight sum),
* special cases that reduce to a library routine (full causal attention via
  torch's scaled_dot_product_attention in float64, a stable argsort, np.dot),
* exhaustive brute force on tiny inputs (tests/bruteforce.py, pure Python),
* invariants (shift invariance of pooling, permutation invariance of the selected
  ids, LSE decomposition across branches, incremental compression).
A planted mistake in the oracle (dropped term, wrong sign or index, transposed
operand) fails at least one of them; test_planted_mistakes checks that claim for a
few such mistakes.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from tests import bruteforce as BF

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- worked examples
def test_worked_compress():
    g = _gold("worked_examples.json")["compress"]
    rows = np.array(g["rows"])
    ids, out = O.compress(rows, np.array(g["logits"]), 0, 0, 4, g["ratio"])
    assert list(ids) == [0]
    np.testing.assert_allclose(out[0], g["expected"], rtol=0, atol=1e-14)


def test_worked_score_topk():
    g = _gold("worked_examples.json")["score_topk"]
    s = O.index_scores(np.array(g["qi"]), np.array(g["wi"]), np.array(g["ki"]))
    np.testing.assert_allclose(s, g["expected_scores"], rtol=0, atol=1e-15)
    assert list(O.topk_select(s, g["k"])) == g["expected_idx"]


def test_worked_attend_and_sink():
    g = _gold("worked_examples.json")["attend"]
    q, K, V = (np.array(g[x]) for x in ("q", "keys", "values"))
    o, lse = O.attend(q, K, V, g["scale"])
    np.testing.assert_allclose(o, g["expected_o"], atol=1e-14)
    np.testing.assert_allclose(lse, g["expected_lse"], atol=1e-14)
    o, lse = O.attend(q, K, V, g["scale"], sink=np.array([g["sink"]]))
    np.testing.assert_allclose(o, g["expected_o_sink"], atol=1e-14)
    np.testing.assert_allclose(lse, g["expected_lse_sink"], atol=1e-14)


def test_worked_layer():
    g = _gold("worked_examples.json")["layer"]
    p, m, mh, W, k = g["p"], g["m"], g["m_hca"], g["window"], g["k"]
    kr, vr, lg = np.array(g["k_raw"]), np.array(g["v_raw"]), np.array(g["pool_logits"])
    _, kc = O.compress(kr, lg, 0, 0, p + 1, m)
    _, vc = O.compress(vr, lg, 0, 0, p + 1, m)
    _, kh = O.compress(kr, lg, 0, 0, p + 1, mh)
    _, vh = O.compress(vr, lg, 0, 0, p + 1, mh)
    s = O.index_scores(np.array(g["qi"]), np.array(g["wi"]), np.array(g["ki"])[:O.n_visible(p, m)])
    idx = O.topk_select(s, k)
    assert list(idx) == g["expected_idx"]
    o, lse = O.decode_query(np.array(g["q"]), p, scale=g["scale"], branches=7, m=m, m_hca=mh,
                            window=W, idx=idx, kc=kc, vc=vc, kh=kh, vh=vh, k_raw=kr, v_raw=vr)
    np.testing.assert_allclose(o, g["expected_o"], atol=1e-14)
    np.testing.assert_allclose(lse, g["expected_lse"], atol=1e-14)


def test_pages_constants():
    c = _gold("pages_constants.json")
    ctx = c["csa_blocks_attended_at_1m"]["context"]
    m = c["csa_ratio"]["value"]
    # a query right after a 1M-token context sees ctx/m complete CSA blocks and
    # attends top-k of them: 1024 for the Pro setting
    n_vis = O.n_visible(ctx, m)
    assert n_vis == ctx // m
    s = np.arange(n_vis, dtype=np.float64)
    sel = O.topk_select(s, c["topk_pro"]["value"])
    assert (sel >= 0).sum() == c["csa_blocks_attended_at_1m"]["value"]
    # the window holds the W most recent raw tokens
    W = c["window"]["value"]
    ks = O.decode_keyset(ctx, branches=4, m=m, m_hca=c["hca_ratio"]["value"], window=W,
                         k_raw=np.zeros((W, 1)), v_raw=np.zeros((W, 1)), raw_start=ctx - W + 1)
    assert ks["swa"][0].shape[0] == W
    assert O.n_visible(ctx, c["hca_ratio"]["value"]) == ctx // 128


# ----------------------------------------------------------------- compress
def test_compress_ratio1_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 5))
    ids, out = O.compress(x, rng.standard_normal(9), 0, 0, 9, 1)
    assert np.array_equal(out, x) and list(ids) == list(range(9))


def test_compress_equal_logits_is_mean():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((12, 3))
    _, out = O.compress(x, np.full(12, 0.7), 0, 0, 12, 4)
    np.testing.assert_allclose(out, x.reshape(3, 4, 3).mean(axis=1), rtol=0, atol=1e-15)


def test_compress_dominant_logit_returns_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 4))
    z = np.zeros(8)
    z[2] = 100.0
    z[7] = 100.0
    _, out = O.compress(x, z, 0, 0, 8, 4)
    np.testing.assert_allclose(out[0], x[2], atol=1e-40)
    np.testing.assert_allclose(out[1], x[7], atol=1e-40)


def test_compress_weights_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(4)
    z = rng.standard_normal(16)
    _, ones = O.compress(np.ones((16, 2)), z, 0, 0, 16, 8)
    np.testing.assert_allclose(ones, 1.0, atol=1e-15)
    x = rng.standard_normal((16, 3))
    _, a = O.compress(x, z, 0, 0, 16, 8)
    _, b = O.compress(x, z + np.repeat([3.5, -7.25], 8), 0, 0, 16, 8)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def test_compress_offsets_and_incremental():
    rng = np.random.default_rng(5)
    T, r, start = 40, 4, 100          # raw row 0 is position 100
    x = rng.standard_normal((T, 3))
    z = rng.standard_normal(T)
    ids, full = O.compress(x, z, start, 100, 38, r)  # 9 complete blocks, tail of 2 stays raw
    assert list(ids) == list(range(25, 34))
    ids1, a = O.compress(x, z, start, 100, 16, r)
    ids2, b = O.compress(x, z, start, 116, 22, r)
    assert list(np.concatenate([ids1, ids2])) == list(ids)
    assert np.array_equal(np.concatenate([a, b]), full)
    # block 27 pools positions 108..111 = raw rows 8..11
    w = np.exp(z[8:12] - z[8:12].max())
    np.testing.assert_allclose(full[2], (w / w.sum()) @ x[8:12], atol=1e-15)
    with pytest.raises(ValueError):
        O.compress(x, z, start, 102, 8, r)


# ----------------------------------------------------------------- indexer score
def test_score_single_head_is_relu_dot():
    rng = np.random.default_rng(6)
    qi = rng.standard_normal((1, 7))
    ki = rng.standard_normal((30, 7))
    s = O.index_scores(qi, np.ones(1), ki)
    ref = np.array([max(0.0, float(np.dot(qi[0], k))) for k in ki])
    np.testing.assert_allclose(s, ref, rtol=1e-15, atol=1e-15)
    assert (s == 0).any() and (s > 0).any()


def test_score_weight_scaling():
    rng = np.random.default_rng(7)
    qi, ki, w = rng.standard_normal((3, 5)), rng.standard_normal((20, 5)), rng.uniform(0, 1, 3)
    s = O.index_scores(qi, w, ki)
    np.testing.assert_allclose(O.index_scores(qi, 2.5 * w, ki), 2.5 * s, rtol=1e-14)
    assert np.array_equal(O.topk_select(s, 6), O.topk_select(2.5 * s, 6))


def test_score_bruteforce():
    rng = np.random.default_rng(8)
    for HI, dI, n in [(1, 1, 3), (2, 3, 5), (4, 2, 9), (3, 4, 1)]:
        qi, ki, w = rng.standard_normal((HI, dI)), rng.standard_normal((n, dI)), rng.uniform(0, 1, HI)
        s = O.index_scores(qi, w, ki)
        ref = [BF.bf_score(qi.tolist(), w.tolist(), ki[j].tolist()) for j in range(n)]
        np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- top-k
def test_topk_exhaustive_distinct():
    rng = np.random.default_rng(9)
    for n in range(1, 11):
        s = rng.standard_normal(n)
        for k in range(1, n + 2):
            got = O.topk_select(s, k)
            assert list(got) == BF.bf_topk(s.tolist(), k)
            ke = min(k, n)
            # the chosen set maximises the score sum among all sets of its size
            best = max(itertools.combinations(range(n), ke), key=lambda c: sum(s[list(c)]))
            assert sorted(best) == [int(i) for i in got[:ke]]


def test_topk_ties_go_to_lower_id():
    rng = np.random.default_rng(10)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        s = rng.integers(0, 3, n).astype(np.float64)
        k = int(rng.integers(1, n + 2))
        got = [int(i) for i in O.topk_select(s, k) if i >= 0]
        assert got == BF.bf_topk(s.tolist(), k)[:len(got)]
        rest = [j for j in range(n) if j not in got]
        for i in got:      # characterisation of the selected set under the tie rule
            for j in rest:
                assert s[i] > s[j] or (s[i] == s[j] and i < j)


def test_topk_matches_stable_argsort_and_pads():
    rng = np.random.default_rng(11)
    s = np.round(rng.standard_normal(5000), 2)       # many ties
    got = O.topk_select(s, 777)
    ref = np.sort(np.argsort(-s, kind="stable")[:777])
    assert np.array_equal(got, ref)
    pad = O.topk_select(s[:10], 16)
    assert list(pad[10:]) == [-1] * 6 and list(pad[:10]) == list(range(10))


# ----------------------------------------------------------------- attention
def test_attend_one_key():
    q = np.array([[0.3, -1.2], [2.0, 0.5]])
    k = np.array([[1.5, 0.25]])
    v = np.array([[-4.0, 9.0]])
    o, lse = O.attend(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), atol=1e-15)


def test_attend_constant_values_and_weight_sum():
    rng = np.random.default_rng(12)
    q, K = rng.standard_normal((3, 4)), rng.standard_normal((17, 4))
    o, _ = O.attend(q, K, np.full((17, 5), -2.25), 0.5)
    np.testing.assert_allclose(o, -2.25, atol=1e-14)
    # one-hot values make o the weight vector: sums to 1, equals scipy's softmax
    from scipy.special import softmax
    o, lse = O.attend(q, K, np.eye(17), 0.5)
    np.testing.assert_allclose(o.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(o, softmax(0.5 * q @ K.T, axis=1), atol=1e-15)
    # with a sink the weights sum to 1 - exp(z - lse)
    z = np.array([0.3, 2.0, -1.0])
    o, lse = O.attend(q, K, np.eye(17), 0.5, sink=z)
    np.testing.assert_allclose(o.sum(axis=1), 1.0 - np.exp(z - lse), atol=1e-14)


def test_attend_empty():
    o, lse = O.attend(np.ones((2, 3)), np.zeros((0, 3)), np.zeros((0, 3)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _sdpa_causal_last(q, K, V, scale):
    """Full causal attention of the last position via torch's library routine (fp64, CPU)."""
    qt = torch.from_numpy(q)[None, :, None, :]           # [1, H, 1, d]
    Kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("which", ["csa_m1", "hca_m1", "swa_full"])
def test_reduces_to_full_causal_attention(which):
    rng = np.random.default_rng(13)
    p, H, d, dI, HI = 37, 3, 8, 4, 2
    Kr, Vr = rng.standard_normal((p + 1, d)), rng.standard_normal((p + 1, d))
    z = rng.standard_normal(p + 1)
    q = rng.standard_normal((H, d))
    scale = 1 / math.sqrt(d)
    ref = _sdpa_causal_last(q, Kr, Vr, scale)
    kw = dict(m=1, m_hca=1, window=128, k_raw=Kr, v_raw=Vr)
    if which == "csa_m1":
        _, kc = O.compress(Kr, z, 0, 0, p + 1, 1)
        _, vc = O.compress(Vr, z, 0, 0, p + 1, 1)
        s = O.index_scores(rng.standard_normal((HI, dI)), rng.uniform(0, 1, HI), rng.standard_normal((p + 1, dI)))
        idx = O.topk_select(s, p + 5)
        o, _ = O.decode_query(q, p, branches=1, idx=idx, kc=kc, vc=vc, **kw)
    elif which == "hca_m1":
        _, kh = O.compress(Kr, z, 0, 0, p + 1, 1)
        _, vh = O.compress(Vr, z, 0, 0, p + 1, 1)
        o, _ = O.decode_query(q, p, branches=2, kh=kh, vh=vh, **kw)
    else:
        kw["window"] = p + 1
        o, _ = O.decode_query(q, p, branches=4, **kw)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def _random_layer(rng, p=29, H=2, d=6, HI=2, dI=3, m=2, mh=4, W=5, k=4, start=0):
    T = p + 1 - start
    Kr, Vr = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    n, e = O.n_visible(p, m), O.n_visible(p, mh)
    return dict(q=rng.standard_normal((H, d)), p=p, kc=rng.standard_normal((n, d)),
                vc=rng.standard_normal((n, d)), kh=rng.standard_normal((e, d)),
                vh=rng.standard_normal((e, d)), k_raw=Kr, v_raw=Vr, raw_start=start,
                idx=np.sort(rng.choice(n, k, replace=False)), m=m, m_hca=mh, window=W)


def test_idx_permutation_invariance():
    rng = np.random.default_rng(14)
    L = _random_layer(rng)
    q, p = L.pop("q"), L.pop("p")
    o1, l1 = O.decode_query(q, p, branches=7, **L)
    L["idx"] = L["idx"][::-1].copy()
    o2, l2 = O.decode_query(q, p, branches=7, **L)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_lse_decomposition_across_branches_and_splits():
    rng = np.random.default_rng(15)
    L = _random_layer(rng, p=61, W=9, k=6)
    q, p = L.pop("q"), L.pop("p")
    full = O.decode_query(q, p, branches=7, **L)
    parts = [O.decode_query(q, p, branches=b, **L) for b in (1, 2, 4)]
    o, lse = O.lse_merge(parts)
    np.testing.assert_allclose(o, full[0], atol=1e-13)
    np.testing.assert_allclose(lse, full[1], atol=1e-13)
    # an arbitrary split of one key set merges back
    ks = O.decode_keyset(p, branches=7, **L)
    K = np.concatenate([v[0] for v in ks.values()])
    V = np.concatenate([v[1] for v in ks.values()])
    cuts = [0, 3, 4, 11, K.shape[0]]
    sub = [O.attend(q, K[a:b], V[a:b], 1 / math.sqrt(q.shape[1])) for a, b in zip(cuts, cuts[1:])]
    sub.append(O.attend(q, K[:0], V[:0], 1.0))       # an empty split contributes nothing
    o, lse = O.lse_merge(sub)
    np.testing.assert_allclose(o, full[0], atol=1e-13)
    np.testing.assert_allclose(lse, full[1], atol=1e-13)


def test_window_before_context_start_and_raw_offset():
    rng = np.random.default_rng(16)
    L = _random_layer(rng, p=3, W=128, k=2, m=2, mh=4)     # p < W: window is 0..p
    q, p = L.pop("q"), L.pop("p")
    ks = O.decode_keyset(p, branches=4, **L)
    assert ks["swa"][0].shape[0] == 4
    L2 = _random_layer(rng, p=50, W=7, start=40)
    q2, p2 = L2.pop("q"), L2.pop("p")
    ks = O.decode_keyset(p2, branches=4, **L2)
    assert np.array_equal(ks["swa"][0], L2["k_raw"][44 - 40:51 - 40])


def test_prefill_rows_equal_decode():
    rng = np.random.default_rng(17)
    p0, Tq, H, d = 20, 6, 2, 4
    L = _random_layer(rng, p=p0 + Tq - 1, H=H, d=d, start=10)
    Q = rng.standard_normal((Tq, H, d))
    idx = np.stack([O.topk_select(rng.standard_normal(O.n_visible(p0 + i, 2)), 3) for i in range(Tq)])
    kw = {k: L[k] for k in ("kc", "vc", "kh", "vh", "k_raw", "v_raw", "m", "m_hca", "window")}
    o, lse = O.prefill(Q, p0, idx, branches=7, raw_start=10, **kw)
    for i in range(Tq):
        od, ld = O.decode_query(Q[i], p0 + i, branches=7, idx=idx[i], raw_start=10, **kw)
        assert np.array_equal(o[i], od) and np.array_equal(lse[i], ld)


# ----------------------------------------------------------------- brute force, exhaustive on tiny shapes
def _bf_case(rng, T, m, mh, W, k, branches, d=2, H=2, HI=2, dI=2, sink=False):
    p = T - 1
    Kr = rng.standard_normal((T, d)).round(3)
    Vr = rng.standard_normal((T, d)).round(3)
    lc, lh = rng.standard_normal(T), rng.standard_normal(T)
    q = rng.standard_normal((H, d))
    qi, wi = rng.standard_normal((HI, dI)), rng.uniform(0, 1, HI)
    n = O.n_visible(p, m)
    ki = rng.standard_normal((max(n, 1), dI))
    sk = rng.standard_normal(H) if sink else None
    scale = 1 / math.sqrt(d)
    bo, bl, bsel = BF.bf_layer(p, q.tolist(), Kr.tolist(), Vr.tolist(), lc.tolist(), lh.tolist(),
                               qi.tolist(), wi.tolist(), ki.tolist(), m=m, m_hca=mh, k=k, window=W,
                               branches=branches, scale=scale, sink=None if sk is None else sk.tolist())
    kw = dict(m=m, m_hca=mh, window=W, k_raw=Kr, v_raw=Vr)
    idx = None
    if branches & 1:
        _, kc = O.compress(Kr, lc, 0, 0, T, m)
        _, vc = O.compress(Vr, lc, 0, 0, T, m)
        idx = O.topk_select(O.index_scores(qi, wi, ki[:n]), k)
        assert [int(i) for i in idx] == bsel
        kw.update(kc=kc, vc=vc, idx=idx)
    if branches & 2:
        _, kh = O.compress(Kr, lh, 0, 0, T, mh)
        _, vh = O.compress(Vr, lh, 0, 0, T, mh)
        kw.update(kh=kh, vh=vh)
    o, lse = O.decode_query(q, p, branches=branches, sink=sk, **kw)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_bruteforce_exhaustive_tiny():
    rng = np.random.default_rng(18)
    count = 0
    for T in (1, 2, 5, 9, 16):
        for m in (1, 2, 4):
            for mh in (1, 2, 4, 8):
                n = T // m
                for W in sorted({1, 3, T}):
                    for k in sorted({1, 2, max(n, 1), n + 1}):
                        if n > 10 and k > 2:
                            k = min(k, 3)      # keep the subset enumeration small
                        for br in range(1, 8):
                            _bf_case(rng, T, m, mh, W, k, br)
                            count += 1
    assert count > 1000


def test_bruteforce_with_sink_and_empty():
    rng = np.random.default_rng(19)
    for T in (1, 3, 8):
        for br in (1, 2, 3, 7):
            _bf_case(rng, T, 4, 8, 2, 2, br, sink=True)   # T < m: CSA/HCA may be empty


# ----------------------------------------------------------------- planted mistakes
def test_planted_mistakes_are_caught():
    """A few plausible mistakes, planted in copies of oracle functions, must fail a pin."""
    rng = np.random.default_rng(20)
    qi, ki, w = rng.standard_normal((3, 4)), rng.standard_normal((9, 4)), rng.uniform(0, 1, 3)
    good = O.index_scores(qi, w, ki)
    bad_sign = np.maximum(-(ki @ qi.T), 0.0) @ w
    bad_noreluw = (ki @ qi.T) @ w
    ref = [BF.bf_score(qi.tolist(), w.tolist(), k.tolist()) for k in ki]
    assert np.allclose(good, ref) and not np.allclose(bad_sign, ref) and not np.allclose(bad_noreluw, ref)
    # window off by one (excluding the query's own token) breaks the full-causal pin
    p, d = 12, 4
    Kr, Vr, q = rng.standard_normal((p + 1, d)), rng.standard_normal((p + 1, d)), rng.standard_normal((2, d))
    ref = _sdpa_causal_last(q, Kr, Vr, 0.5)
    o_bad, _ = O.attend(q, Kr[:p], Vr[:p], 0.5)
    o_good, _ = O.attend(q, Kr, Vr, 0.5)
    assert np.allclose(o_good, ref) and not np.allclose(o_bad, ref)
    # pooling weights taken from the wrong block fail the worked example
    g = _gold("worked_examples.json")["compress"]
    rows, z = np.array(g["rows"]), np.array(g["logits"])
    e = np.exp(z[::-1] - z.max())
    assert not np.allclose((e / e.sum()) @ rows, g["expected"])


# ----------------------------------------------------------------- RMSNorm (Q/KV normalization)
def test_rms_norm_closed_forms():
    # a constant vector c*1 normalises to sign(c)*1 (eps = 0); [3, 4] has mean square
    # 12.5, so it becomes [3, 4] / sqrt(12.5) = [0.848528137..., 1.131370849...]
    for c in (2.5, -0.125, 7.0):
        assert np.array_equal(O.rms_norm(np.full(8, c), np.ones(8), 0.0), np.full(8, math.copysign(1.0, c)))
    got = O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(got, [0.8485281374238570, 1.1313708498984760], rtol=0, atol=1e-15)
    # eps enters under the root: mean square 12.5 + eps 3.5 = 16 -> [0.75, 1.0]
    assert np.allclose(O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 3.5), [0.75, 1.0], rtol=0, atol=1e-15)
    # the zero vector stays zero for eps > 0
    assert np.array_equal(O.rms_norm(np.zeros(4), np.ones(4), 1e-6), np.zeros(4))


def test_rms_norm_invariants():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 16))
    g = rng.uniform(0.5, 2.0, 16)
    y1 = O.rms_norm(x, np.ones(16), 0.0)
    # unit mean square per row, independent of a positive scale, gain elementwise
    assert np.allclose(np.mean(y1 * y1, axis=-1), 1.0, rtol=0, atol=1e-13)
    assert np.allclose(O.rms_norm(3.7 * x, np.ones(16), 0.0), y1, rtol=0, atol=1e-13)
    assert np.allclose(O.rms_norm(x, g, 0.0), y1 * g, rtol=0, atol=1e-13)
    # a plausible mistake (mean |x| instead of the root mean square) breaks the unit
    # mean square
    bad = x / np.mean(np.abs(x), axis=-1, keepdims=True)
    assert not np.allclose(np.mean(bad * bad, axis=-1), 1.0, atol=1e-3)


def test_query_norm_makes_attention_scale_free():
    # with the query normalised (eps = 0) a positive rescaling of q cannot change the
    # output; without it, it changes the softmax temperature
    rng = np.random.default_rng(32)
    d, p = 8, 40
    caches = dict(branches=6, m=4, m_hca=8, window=6, kh=rng.standard_normal((8, d)),
                  vh=rng.standard_normal((8, d)), k_raw=rng.standard_normal((p + 1, d)),
                  v_raw=rng.standard_normal((p + 1, d)), raw_start=0)
    q = rng.standard_normal((3, d))
    g = rng.uniform(0.5, 1.5, d)
    o1, l1 = O.decode_query(q, p, q_norm=g, norm_eps=0.0, **caches)
    o2, _ = O.decode_query(5.0 * q, p, q_norm=g, norm_eps=0.0, **caches)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    o3, _ = O.decode_query(5.0 * q, p, **caches)
    o4, _ = O.decode_query(q, p, **caches)
    assert not np.allclose(o3, o4, atol=1e-6)
    # and normalising is the same as feeding the normalised query
    qn = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True)) * g
    o5, l5 = O.decode_query(qn, p, **caches)
    assert np.allclose(o1, o5, rtol=0, atol=1e-12) and np.allclose(l1, l5, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- partial RoPE
def test_rope_closed_forms():
    x = np.array([0.3, -1.2, 1.0, 0.0, 1.0, 0.0])
    # dims = 0 leaves everything; only the last `dims` channels ever move
    assert np.array_equal(O.rope(x, 7, 0, 1e4), x)
    y = O.rope(x, 7, 4, 1e4)
    assert np.array_equal(y[:2], x[:2])
    # the first pair of the rotated part turns by pos radians: (1, 0) at pos 1 is
    # (cos 1, sin 1) = (0.5403023058681398, 0.8414709848078965); at pos 0 nothing moves
    y = O.rope(np.array([1.0, 0.0]), 1, 2, 1e4)
    assert np.allclose(y, [0.5403023058681398, 0.8414709848078965], rtol=0, atol=1e-15)
    assert np.array_equal(O.rope(x, 0, 4, 1e4), x)
    # the second pair of a 4-channel part turns by pos * base^(-1/2): base 1e4 and
    # pos 100 give 1 radian there (and 100 radians on the first pair:
    # cos 100 = 0.8623188722876839, sin 100 = -0.5063656411097588)
    y = O.rope(np.array([1.0, 0.0, 1.0, 0.0]), 100, 4, 1e4)
    assert np.allclose(y, [0.8623188722876839, -0.5063656411097588, 0.5403023058681398, 0.8414709848078965],
                       rtol=0, atol=1e-13)


def test_rope_group_and_relative_properties():
    rng = np.random.default_rng(41)
    q, k = rng.standard_normal((2, 16)), rng.standard_normal((2, 16))
    for m, n in ((5, 3), (1_000_003, 17), (0, 250)):
        a = O.rope(q, m, 8, 1e4)
        # norm preserved, a rotation at -m undoes one at m, angles add
        assert np.allclose(np.linalg.norm(a, axis=-1), np.linalg.norm(q, axis=-1), rtol=0, atol=1e-12)
        assert np.allclose(O.rope(a, -m, 8, 1e4), q, rtol=0, atol=1e-9)
        assert np.allclose(O.rope(O.rope(q, n, 8, 1e4), m, 8, 1e4), O.rope(q, m + n, 8, 1e4), rtol=0, atol=1e-9)
        # dot products depend on the relative position only
        lhs = np.sum(a * O.rope(k, n, 8, 1e4), axis=-1)
        rhs = np.sum(O.rope(q, m - n, 8, 1e4) * k, axis=-1)
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)
    # a plausible mistake (pairs (j, j + dims/2) instead of (2j, 2j+1)) breaks the
    # closed form of the second pair
    x = np.array([1.0, 2.0, 3.0, 4.0])
    half = x.copy()
    ang = np.array([100.0, 1.0])
    half[[0, 1]] = x[[0, 1]] * np.cos(ang) - x[[2, 3]] * np.sin(ang)
    half[[2, 3]] = x[[0, 1]] * np.sin(ang) + x[[2, 3]] * np.cos(ang)
    assert not np.allclose(half, O.rope(x, 100, 4, 1e4), atol=1e-3)


def test_rope_entries_of_identical_tokens():
    # tokens that are one unrotated vector u, each rotated at its own position: the
    # pooled entry of a block is u itself (any weights), rotated at the block's last
    # position (and normalised first when a gain is given)
    rng = np.random.default_rng(42)
    d, r, T = 16, 8, 40
    u = rng.standard_normal(d)
    raw_start = 5
    pos = raw_start + np.arange(T)
    x = O.rope(np.tile(u, (T, 1)), pos, 8, 1e4)
    z = rng.standard_normal(T)
    ids, ent = O.compress_entries(x, z, raw_start, 8, 32, r, rope_dims=8, rope_base=1e4)
    assert list(ids) == [1, 2, 3, 4]
    for bi, j in enumerate(ids):
        assert np.allclose(ent[bi], O.rope(u, (j + 1) * r - 1, 8, 1e4), rtol=0, atol=1e-12)
    g = rng.uniform(0.5, 1.5, d)
    _, ent2 = O.compress_entries(x, z, raw_start, 8, 32, r, gain=g, eps=0.0, rope_dims=8, rope_base=1e4)
    un = u / np.sqrt(np.mean(u * u)) * g
    assert np.allclose(ent2[0], O.rope(un, 2 * r - 1, 8, 1e4), rtol=0, atol=1e-12)


def test_rope_output_rotation_makes_the_layer_shift_invariant():
    # shared K = V entries rotated at their positions, the query rotated at p and the
    # output rotated at -p: shifting every position leaves the output unchanged (only
    # relative positions remain), and without the output rotation it does not.  The
    # window covers every token so that a shift adds no key (an HCA or CSA history
    # would gain empty entries); the entries' own rotation is pinned above.
    rng = np.random.default_rng(43)
    d, R = 16, 8
    p0 = 45
    u = rng.standard_normal((p0 + 1, d))       # unrotated per-token entries
    q = rng.standard_normal((2, d))
    outs = {}
    for shift in (0, 1000, 123457):
        raw = O.rope(u, shift + np.arange(p0 + 1), R, 1e4)
        for ro in (True, False):
            outs[shift, ro] = O.decode_query(q, shift + p0, branches=4, m=4, m_hca=8, window=p0 + 1,
                                             k_raw=raw, v_raw=raw, raw_start=shift, rope_dims=R, rope_base=1e4,
                                             rope_out=ro)
    for shift in (1000, 123457):
        assert np.allclose(outs[0, True][0], outs[shift, True][0], rtol=0, atol=1e-9)
        assert np.allclose(outs[0, True][1], outs[shift, True][1], rtol=0, atol=1e-9)
        assert not np.allclose(outs[0, False][0], outs[shift, False][0], atol=1e-4)


def test_shared_kv_layer_in_relative_form():
    # The pages' shared-KV layer at its own sizes (c = 512, RoPE on the last 64
    # channels, m = 4, m' = 128, a 128-token window): every entry is its own value,
    # so with the query rotated at p and the output at -p each key contributes
    # only through its position relative to p.  The same output is rebuilt here
    # from the unrotated token contents: entries pooled and normalised without any
    # rotation, each one placed at its block's last position s and turned by s - p,
    # both in the logit and as a value.
    rng = np.random.default_rng(44)
    d, R, H, p, W = 512, 64, 3, 300, 128
    u = rng.standard_normal((p + 1, d))               # unrotated token contents
    x = O.rope(u, np.arange(p + 1), R, 1e4)           # raw rows, rotated at their positions
    zc, zh = rng.standard_normal(p + 1), rng.standard_normal(p + 1)
    gk = rng.uniform(0.5, 1.5, d)
    gq = rng.uniform(0.5, 1.5, d)
    eps = 1e-6
    ids_c, ec = O.compress_entries(x, zc, 0, 0, p + 1, 4, gain=gk, eps=eps, rope_dims=R, rope_base=1e4)
    ids_h, eh = O.compress_entries(x, zh, 0, 0, p + 1, 128, gain=gk, eps=eps, rope_dims=R, rope_base=1e4)
    assert len(ids_c) == 75 and len(ids_h) == 2
    sel = np.sort(rng.choice(75, 16, replace=False))
    q = rng.standard_normal((H, d))
    o, lse = O.decode_query(q, p, q_norm=gq, norm_eps=eps, rope_dims=R, rope_base=1e4, rope_out=True,
                            branches=7, m=4, m_hca=128, window=W, idx=sel, kc=ec, kh=eh, k_raw=x, raw_start=0)
    # rebuilt: unrotated entries with their positions
    _, pc = O.compress(u, zc, 0, 0, p + 1, 4)
    _, ph = O.compress(u, zh, 0, 0, p + 1, 128)
    content = [O.rms_norm(pc[j], gk, eps) for j in sel] + [O.rms_norm(ph[j], gk, eps) for j in range(2)]
    where = [4 * (j + 1) - 1 for j in sel] + [128 * (j + 1) - 1 for j in range(2)]
    content += [u[t] for t in range(p - W + 1, p + 1)]
    where += list(range(p - W + 1, p + 1))
    rel = np.stack([O.rope(c, s - p, R, 1e4) for c, s in zip(content, where)])
    qn = O.rms_norm(q, gq, eps)
    logits = (qn @ rel.T) / math.sqrt(d)
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    ref_o = (w @ rel) / w.sum(axis=1, keepdims=True)
    ref_lse = mx[:, 0] + np.log(w.sum(axis=1))
    assert np.allclose(o, ref_o, rtol=0, atol=1e-9)
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-9)
    # leaving out the output rotation, or placing entries at their block's first
    # position, breaks it
    o2, _ = O.decode_query(q, p, q_norm=gq, norm_eps=eps, rope_dims=R, rope_base=1e4, rope_out=False,
                           branches=7, m=4, m_hca=128, window=W, idx=sel, kc=ec, kh=eh, k_raw=x, raw_start=0)
    assert not np.allclose(o2, ref_o, atol=1e-3)
    shifted = [O.rope(c, s - 3 - p, R, 1e4) if k < 18 else O.rope(c, s - p, R, 1e4)
               for k, (c, s) in enumerate(zip(content, where))]
    assert not np.allclose((w @ np.stack(shifted)) / w.sum(axis=1, keepdims=True), o, atol=1e-3)


def test_shared_entries_when_values_are_omitted():
    # a branch given without values attends with each entry as its own value
    rng = np.random.default_rng(45)
    d = 8
    kc, kh, raw = rng.standard_normal((6, d)), rng.standard_normal((2, d)), rng.standard_normal((40, d))
    q = rng.standard_normal((2, d))
    a = O.decode_query(q, 39, branches=7, m=4, m_hca=16, window=5, idx=np.array([1, 4, -1]),
                       kc=kc, kh=kh, k_raw=raw, raw_start=0)
    b = O.decode_query(q, 39, branches=7, m=4, m_hca=16, window=5, idx=np.array([1, 4, -1]),
                       kc=kc, vc=kc, kh=kh, vh=kh, k_raw=raw, v_raw=raw, raw_start=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    keys = np.concatenate([kc[[1, 4]], kh[:2], raw[35:40]])
    ref = O.attend(q, keys, keys, 1 / math.sqrt(d))
    assert np.allclose(a[0], ref[0], rtol=0, atol=1e-12)


def test_fp8_e4m3_decode_closed_forms_and_library():
    # a few codes by hand: 1.0, the smallest subnormal and normal, the largest
    # finite value, a negative one, zero and the NaN code
    d = O.fp8_e4m3_decode([0x38, 0x01, 0x08, 0x7E, 0xB8, 0x00, 0x80, 0x7F, 0xFF, 0x3C, 0x07])
    assert list(d[:7]) == [1.0, 2.0 ** -9, 2.0 ** -6, 448.0, -1.0, 0.0, -0.0]
    assert np.isnan(d[7]) and np.isnan(d[8])
    assert d[9] == 1.5 and d[10] == 7 * 2.0 ** -9
    # every code against torch's float8_e4m3fn (the OCP E4M3 format)
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])
    # positive finite codes are strictly increasing in value; sign is the top bit
    pos = mine[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(mine[0x80:0xFF], -mine[:0x7F])


def test_fp8_rows_scale_and_scores():
    # rows are scale * decode(code); the indexer score of a scaled row is the scale
    # times the score of its codes' values (the weights and the ReLU are positively
    # homogeneous)
    rng = np.random.default_rng(46)
    codes = rng.integers(0, 0x7F, size=(5, 8)).astype(np.uint8) | (rng.integers(0, 2, size=(5, 8)) << 7).astype(np.uint8)
    scales = rng.uniform(0.01, 2.0, 5)
    rows = O.fp8_rows(codes, scales)
    np.testing.assert_array_equal(rows, O.fp8_e4m3_decode(codes) * scales[:, None])
    qi, wi = rng.standard_normal((3, 8)), rng.uniform(0, 1, 3)
    s = O.index_scores(qi, wi, rows)
    s0 = O.index_scores(qi, wi, O.fp8_e4m3_decode(codes))
    np.testing.assert_allclose(s, s0 * scales, rtol=1e-14, atol=0)


def test_fp8_e4m3_encode_closed_forms_and_library():
    # closed forms: zero, the largest finite value, the smallest subnormal; ties go to
    # the even code: 2^-10 (between 0 and 2^-9) to 0, 3*2^-10 (between codes 1 and 2)
    # to 2, 1.0625 (between 1.0 = 0x38 and 1.125 = 0x39) to 0x38, 1.1875 (between 0x39
    # and 0x3A) to 0x3A; the sign is the value's own
    got = O.fp8_e4m3_encode([0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, -0.0,
                             -1.0, 440.0, 0.99])
    assert list(got) == [0x00, 0x7E, 0xFE, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x80, 0xB8, 0x7E, 0x38]
    # every finite code is its own value's code
    codes = np.arange(256, dtype=np.uint8)
    fin = (codes & 0x7F) != 0x7F
    assert np.array_equal(O.fp8_e4m3_encode(O.fp8_e4m3_decode(codes[fin])), codes[fin])
    # torch's float8_e4m3fn cast (round to nearest even) on random values and on every
    # midpoint between neighbouring magnitudes, both signs
    rng = np.random.default_rng(47)
    mags = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[1:] + mags[:-1]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000), 0.01 * rng.standard_normal(5000),
                        mids, -mids]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_e4m3_encode(x.astype(np.float64)), lib)
    with pytest.raises(ValueError):
        O.fp8_e4m3_encode([449.0])


def test_fp8_quantize_rows():
    rng = np.random.default_rng(48)
    x = rng.standard_normal((6, 64)) * rng.uniform(0.01, 10, (6, 1))
    x[2] = 0.0
    codes, scales = O.fp8_quantize_rows(x)
    # the scale puts each row's largest magnitude on 448, which decodes exactly
    assert np.array_equal(scales, np.max(np.abs(x), axis=-1) / 448.0)
    back = O.fp8_rows(codes, scales)
    top = np.argmax(np.abs(x), axis=-1)
    for r in (0, 1, 3, 4, 5):
        assert abs(back[r, top[r]]) == pytest.approx(abs(x[r, top[r]]), rel=1e-15)
    # a zero row: scale 0, codes 0, read back as zeros
    assert scales[2] == 0 and not codes[2].any() and not back[2].any()
    # nearest rounding: within half a step of the value; a step is 2^-3 of the
    # magnitude's binade above 2^-6 and 2^-9 below, in units of the scale
    q = np.abs(x) / np.where(scales > 0, scales, 1)[:, None]
    step = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(back - x) / np.where(scales > 0, scales, 1)[:, None]
    assert np.all(err <= step / 2 * (1 + 1e-12))


# ----------------------------------------------------------------- bf16 decoding
def test_bf16_to_f64_every_pattern():
    """Every one of the 65536 bf16 patterns against two references that do not use the
    oracle's "high half of a binary32 word" construction: the format's own field
    decomposition (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits;
    exponent 0 subnormal, f * 2^-133; exponent 255 infinity or NaN), evaluated with
    exact powers of two, and torch's bfloat16 -> float64 conversion.  NaN patterns
    must decode to NaN (payloads are not compared)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = O.bf16_to_f64(bits.astype(np.uint16))
    s = np.where(bits >> 15, -1.0, 1.0)
    e = ((bits >> 7) & 0xFF).astype(np.int64)
    f = (bits & 0x7F).astype(np.float64)
    with np.errstate(over="ignore"):
        mag = np.where(e == 0, f * 2.0 ** -133, (1.0 + f / 128.0) * np.exp2((e - 127).astype(np.float64)))
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    ref = s * mag
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    tb = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(tb), nan)
    assert np.array_equal(got[~nan], tb[~nan])


def test_bf16_to_f64_worked_values():
    """A few patterns decoded by hand from the format definition."""
    cases = {0x3F80: 1.0, 0xC040: -3.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x3C00: 2.0 ** -7, 0xBF00: -0.5, 0x7F80: math.inf,
             0xFF80: -math.inf}
    got = O.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    assert got.tolist() == list(cases.values())
    assert np.signbit(O.bf16_to_f64(np.array([0x8000], np.uint16)))[0]
    assert np.isnan(O.bf16_to_f64(np.array([0x7FC0, 0xFF81], np.uint16))).all()
    assert np.array_equal(O.as_f64(np.array([0x3F80], np.uint16), "bf16"), [1.0])
    assert O.as_f64(np.array([0.1], np.float32), "f32")[0] == float(np.float32(0.1))
