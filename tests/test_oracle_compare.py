"""The oracle's streaming comparison (``oracle.compare``) against the same
comparison done by hand in numpy on the oracle's own full tensors.

``compare`` evaluates the plain definition one unit at a time and keeps only
the largest errors, so that every unit of the full-size workloads can be
checked without an fp64 copy of the outputs.  These tests plant known errors,
non-finite values and empty rows in an output and check that ``compare``
reports exactly what an element-by-element numpy comparison reports.
"""

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, make_inputs


def _reference(O, L, Or, Lr):
    Od = O.astype(np.float64)
    errO = np.abs(Od - Or)
    errO[~np.isfinite(Od)] = 0.0
    fin = np.isfinite(Lr)
    errL = np.where(fin & np.isfinite(L), np.abs(L.astype(np.float64) - np.where(fin, Lr, 0.0)), 0.0)
    return errO, errL


def _unit_of_O(idx_flat, shape, gs, G):
    B, M, H, D = shape
    b, m, h, _ = np.unravel_index(idx_flat, shape)
    return (b * M + m) * G + h // gs


@pytest.mark.parametrize("cfg", [CONFIGS["tiny"].with_(M=300, N=300),
                                 Config("c", B=2, M=200, N=260, H=6, G=2, D=64, block_size=32, T=5, seed=11)])
def test_compare_matches_numpy_on_planted_errors(oracle_mod, cfg):
    q, k, v, idx = make_inputs(cfg)
    Or, Lr = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size)
    O = Or.astype(np.float16)
    L = Lr.astype(np.float32)
    rng = np.random.default_rng(5)
    # Planted errors of distinct sizes at random elements.
    flat = O.reshape(-1)
    picks = rng.choice(flat.size, 7, replace=False)
    for i, p in enumerate(picks):
        flat[p] = np.float16(float(flat[p]) + 0.01 * (i + 1))
    Lflat = L.reshape(-1)
    lp = rng.choice(Lflat.size, 3, replace=False)
    for i, p in enumerate(lp):
        Lflat[p] += np.float32(0.002 * (i + 1))
    errO, errL = _reference(O, L, Or, Lr)
    res = oracle_mod.compare(q, k, v, idx, cfg.block_size, O, L)
    assert res["max_err_O"] == errO.max()
    assert res["max_err_LSE"] == errL.max()
    assert res["bad_rows"] == 0
    assert res["units"] == cfg.B * cfg.M * cfg.G
    worst = _unit_of_O(int(np.argmax(errO)), O.shape, cfg.gs, cfg.G)
    assert res["worst_unit_O"] == worst
    b, h, m = np.unravel_index(int(np.argmax(errL)), L.shape)
    assert res["worst_unit_LSE"] == (b * cfg.M + m) * cfg.G + h // cfg.gs


def test_compare_unit_ranges_partition_the_result(oracle_mod):
    cfg = CONFIGS["tiny"].with_(M=256, N=256)
    q, k, v, idx = make_inputs(cfg)
    Or, Lr = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size)
    O = Or.astype(np.float16)
    L = Lr.astype(np.float32)
    whole = oracle_mod.compare(q, k, v, idx, cfg.block_size, O, L)
    cuts = [0, 17, 100, 101, 256]
    parts = [oracle_mod.compare(q, k, v, idx, cfg.block_size, O, L, a, b) for a, b in zip(cuts, cuts[1:])]
    assert sum(p["units"] for p in parts) == whole["units"] == 256
    assert max(p["max_err_O"] for p in parts) == whole["max_err_O"]
    assert max(p["max_err_LSE"] for p in parts) == whole["max_err_LSE"]
    # Errors outside the range are not seen.
    O2 = O.copy()
    O2[0, 200, 0, 0] += np.float16(1.0)
    assert oracle_mod.compare(q, k, v, idx, cfg.block_size, O2, L, 0, 200)["max_err_O"] == whole["max_err_O"]
    assert oracle_mod.compare(q, k, v, idx, cfg.block_size, O2, L, 200, 201)["max_err_O"] >= 0.99


def test_compare_flags_non_finite_and_empty_rows(oracle_mod):
    B, M, N, H, G, D, bs, T = 1, 130, 130, 4, 2, 64, 64, 2
    rng = np.random.default_rng(2)
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    idx = np.full((B, M, G, T), -1, np.int32)
    idx[0, ::2, :, 0] = 0                      # odd rows select nothing: O = 0, LSE = -inf
    Or, Lr = oracle_mod.oracle_full(q, k, v, idx, bs)
    O = Or.astype(np.float16)
    L = Lr.astype(np.float32)
    res = oracle_mod.compare(q, k, v, idx, bs, O, L)
    assert res["bad_rows"] == 0 and res["empty_rows"] == (M // 2) * H
    # A finite LSE on an empty row, a NaN in O, an infinite LSE on a full row.
    L2 = L.copy()
    L2[0, 0, 1] = 0.0
    O2 = O.copy()
    O2[0, 4, 3, 7] = np.nan
    L2[0, 2, 6] = np.inf
    res = oracle_mod.compare(q, k, v, idx, bs, O2, L2)
    assert res["bad_rows"] == 3
    # A nonzero O on an empty row is an O error against the reference 0.
    O3 = O.copy()
    O3[0, 1, 0, 0] = np.float16(0.25)
    assert oracle_mod.compare(q, k, v, idx, bs, O3, L)["max_err_O"] == 0.25


def test_compare_without_index_rows_is_dense_or_window(oracle_mod):
    cfg = CONFIGS["tiny"].with_(M=200, N=200)
    q, k, v, _ = make_inputs(cfg)
    Or, Lr = oracle_mod.dense_full(q, k, v)
    O = Or.astype(np.float16)
    L = Lr.astype(np.float32)
    errO, errL = _reference(O, L, Or, Lr)
    res = oracle_mod.compare(q, k, v, None, 1, O, L)
    assert res["max_err_O"] == errO.max() and res["max_err_LSE"] == errL.max()
    Wr, WLr = oracle_mod.window_full(q, k, v, 16, 3)
    W = Wr.astype(np.float16)
    WL = WLr.astype(np.float32)
    errO, errL = _reference(W, WL, Wr, WLr)
    res = oracle_mod.compare(q, k, v, None, 1, W, WL, window=(16, 3))
    assert res["max_err_O"] == errO.max() and res["max_err_LSE"] == errL.max()


def test_compare_counts_repeated_blocks(oracle_mod):
    cfg = CONFIGS["tiny"].with_(M=128, N=128)
    q, k, v, idx = make_inputs(cfg)
    idx = idx.copy()
    idx[0, 100, 0, 3] = idx[0, 100, 0, 0]       # block 0 twice in one row
    Or, Lr = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size)
    res = oracle_mod.compare(q, k, v, idx, cfg.block_size, Or.astype(np.float16), Lr.astype(np.float32))
    assert res["dup_units"] == 1


def test_compare_rejects_bad_arguments(oracle_mod):
    cfg = CONFIGS["tiny"].with_(M=64, N=64)
    q, k, v, idx = make_inputs(cfg)
    O = np.zeros_like(q)
    L = np.zeros((1, cfg.H, cfg.M), np.float32)
    with pytest.raises(ValueError):
        oracle_mod.compare(q, k, v, idx, cfg.block_size, O, L, 0, cfg.M * cfg.G + 1)
    with pytest.raises(ValueError):
        oracle_mod.compare(q, k, v, idx, cfg.block_size, O.astype(np.float32), L)
    with pytest.raises(ValueError):
        oracle_mod.compare(q, k, v, idx, cfg.block_size, O, L[:, :, :10].copy())
