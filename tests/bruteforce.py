"""Pure-Python brute force of the hybrid compressed-attention layer, for tiny inputs.

Written independently of the NumPy oracle (lists, explicit loops, ``math.exp``)
so that the two can check each other.  It follows the same reading of the pages:
softmax pooling inside non-overlapping blocks; a block is visible when complete;
ReLU-weighted indexer head sum; top-k by exhaustive search over subsets; one
softmax over the CSA picks, the HCA entries and the raw window [p-W+1, p].
"""
from __future__ import annotations

import itertools
import math


def bf_pool(rows, logits):
    """rows: list of r vectors, logits: list of r floats -> pooled vector."""
    mx = max(logits)
    ws = [math.exp(z - mx) for z in logits]
    tot = sum(ws)
    d = len(rows[0])
    return [sum(ws[t] * rows[t][c] for t in range(len(rows))) / tot for c in range(d)]


def bf_compress_all(x, logits, r):
    """Compress every complete block of x (positions 0..T-1)."""
    nb = len(x) // r
    return [bf_pool(x[j * r:(j + 1) * r], logits[j * r:(j + 1) * r]) for j in range(nb)]


def bf_score(qi, wi, kij):
    s = 0.0
    for h in range(len(qi)):
        dot = 0.0
        for c in range(len(kij)):
            dot += qi[h][c] * kij[c]
        if dot > 0.0:
            s += wi[h] * dot
    return s


def bf_topk(scores, k):
    """Exhaustive: among all subsets of size min(k, n), the one whose sorted score
    list is lexicographically largest, where each element is ranked by (score,
    -id).  Returns the ascending id list padded with -1."""
    n = len(scores)
    ke = min(k, n)
    best = None
    best_key = None
    for sub in itertools.combinations(range(n), ke):
        key = sorted(((scores[j], -j) for j in sub), reverse=True)
        if best_key is None or key > best_key:
            best_key, best = key, sub
    return sorted(best) + [-1] * (k - ke)


def bf_attend(q, keys, values, scale, sink=None):
    """q: list of H vectors; keys/values: lists of vectors -> (o [H][d], lse [H])."""
    H = len(q)
    d = len(values[0]) if values else len(q[0])
    o_all, lse_all = [], []
    for h in range(H):
        logits = [scale * sum(q[h][c] * kk[c] for c in range(len(kk))) for kk in keys]
        terms = list(logits) + ([sink[h]] if sink is not None else [])
        if not terms:
            o_all.append([0.0] * d)
            lse_all.append(-math.inf)
            continue
        mx = max(terms)
        es = [math.exp(l - mx) for l in logits]
        z = sum(es) + (math.exp(sink[h] - mx) if sink is not None else 0.0)
        o_all.append([sum(es[t] * values[t][c] for t in range(len(values))) / z for c in range(d)])
        lse_all.append(mx + math.log(z))
    return o_all, lse_all


def bf_layer(p, q, k_raw, v_raw, lc, lh, qi, wi, ki, *, m, m_hca, k, window, branches, scale,
             sink=None):
    """Whole layer for one query at position p over raw positions 0..p (raw row t = position t).
    Compressed caches are built here from raw tokens; indexer keys ki are per block."""
    keys, vals = [], []
    sel = []
    if branches & 1:
        kc = bf_compress_all(k_raw[:p + 1], lc[:p + 1], m)
        vc = bf_compress_all(v_raw[:p + 1], lc[:p + 1], m)
        n_vis = len(kc)
        scores = [bf_score(qi, wi, ki[j]) for j in range(n_vis)]
        sel = bf_topk(scores, k)
        for j in sel:
            if j >= 0:
                keys.append(kc[j])
                vals.append(vc[j])
    if branches & 2:
        kh = bf_compress_all(k_raw[:p + 1], lh[:p + 1], m_hca)
        vh = bf_compress_all(v_raw[:p + 1], lh[:p + 1], m_hca)
        keys += kh
        vals += vh
    if branches & 4:
        for t in range(max(0, p - window + 1), p + 1):
            keys.append(k_raw[t])
            vals.append(v_raw[t])
    o, lse = bf_attend(q, keys, vals, scale, sink)
    return o, lse, sel
