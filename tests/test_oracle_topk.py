"""Pins of the oracle's top-k block selection.

The wave issue "[wave] NSA: selection attention forward kernel" (section
Depends on) takes block_indices from a top-k kernel whose algorithm the pages
do not give.  The reading pinned here: per row (b, m, g), the T highest
scores among the causal candidates t = 0 .. min(m // bs, NB - 1), ties to the
smaller t, NaN as -inf, -0 equal to +0, written ascending and padded with -1.
Checked against numpy's lexsort, against the defining inequalities, and
against closed forms.
"""

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import Config, block_scores


def _lexsort_reference(scores, bs, T):
    B, M, G, NB = scores.shape
    out = np.full((B, M, G, T), -1, np.int32)
    for b in range(B):
        for m in range(M):
            nc = min(m // bs, NB - 1) + 1
            for g in range(G):
                v = scores[b, m, g, :nc].astype(np.float64)
                v = np.where(np.isnan(v), -np.inf, v)
                order = np.lexsort((np.arange(nc), -v))        # by -v, then t
                sel = np.sort(order[:T])
                out[b, m, g, :len(sel)] = sel
    return out


def _special_scores(rng, shape):
    s = rng.integers(-3, 4, size=shape).astype(np.float32) / 2        # many ties
    flat = s.reshape(-1)
    pick = rng.choice(flat.size, size=flat.size // 10, replace=False)
    flat[pick[0::4]] = np.nan
    flat[pick[1::4]] = np.inf
    flat[pick[2::4]] = -np.inf
    flat[pick[3::4]] = -0.0
    return s


@pytest.mark.parametrize("shape,bs,T", [((1, 64, 1, 8), 8, 3), ((2, 100, 3, 13), 8, 5), ((1, 40, 2, 40), 1, 7),
                                        ((1, 50, 1, 4), 4, 6)])
def test_matches_lexsort(oracle_mod, shape, bs, T):
    rng = np.random.default_rng(sum(shape) + T)
    for scores in (rng.standard_normal(shape).astype(np.float32), _special_scores(rng, shape)):
        assert np.array_equal(oracle_mod.topk_blocks(scores, bs, T), _lexsort_reference(scores, bs, T))


def test_defining_inequalities(oracle_mod):
    cfg = Config("t", B=1, M=300, N=300, H=1, G=2, D=64, block_size=16, T=5, seed=3)
    scores = block_scores(cfg)
    scores[0, :, 0, :] = np.round(scores[0, :, 0, :])           # ties in one group
    out = oracle_mod.topk_blocks(scores, cfg.block_size, cfg.T)
    for m in range(cfg.M):
        nc = min(m // cfg.block_size, cfg.NB - 1) + 1
        for g in range(cfg.G):
            row = out[0, m, g]
            k = min(cfg.T, nc)
            sel = row[:k]
            assert np.all(row[k:] == -1)
            assert np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() < nc
            rest = np.setdiff1d(np.arange(nc), sel)
            if rest.size:
                v = scores[0, m, g].astype(np.float64)
                assert v[sel].min() >= v[rest].max()
                tie = v[sel].min()
                # among candidates equal to the boundary score, the smallest indices are taken
                eq = np.nonzero(v[:nc] == tie)[0]
                taken = np.intersect1d(eq, sel)
                assert np.array_equal(taken, eq[:taken.size])


def test_closed_forms(oracle_mod):
    B, M, G, NB, bs, T = 1, 200, 1, 20, 10, 4
    dec = np.broadcast_to(-np.arange(NB, dtype=np.float32), (B, M, G, NB)).copy()
    out = oracle_mod.topk_blocks(dec, bs, T)
    for m in range(M):
        nc = min(m // bs, NB - 1) + 1
        want = list(range(min(T, nc))) + [-1] * (T - min(T, nc))
        assert out[0, m, 0].tolist() == want
    inc = -dec
    out = oracle_mod.topk_blocks(inc, bs, T)
    for m in range(M):
        nc = min(m // bs, NB - 1) + 1
        k = min(T, nc)
        assert out[0, m, 0].tolist() == list(range(nc - k, nc)) + [-1] * (T - k)
    # all equal: the first T candidates
    out = oracle_mod.topk_blocks(np.zeros((B, M, G, NB), np.float32), bs, T)
    assert np.array_equal(out, oracle_mod.topk_blocks(dec, bs, T))


def test_rejects_bad_arguments(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.topk_blocks(np.zeros((1, 4, 1, 2), np.float64), 2, 1)
    with pytest.raises(ValueError):
        oracle_mod.topk_blocks(np.zeros((1, 4, 1, 2), np.float32), 2, 0)


def test_rows_entry_is_the_same_selection(oracle_mod):
    rng = np.random.default_rng(8)
    B, M, G, NB, bs, T = 1, 90, 2, 12, 8, 4
    scores = _special_scores(rng, (B, M, G, NB))
    full = oracle_mod.topk_blocks(scores, bs, T)
    ms = np.repeat(np.arange(M), G)
    rows = oracle_mod.topk_rows(scores.reshape(-1, NB), ms, bs, T)
    assert np.array_equal(rows.reshape(B, M, G, T), full)
