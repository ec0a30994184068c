"""Pins of the oracle's sliding-window entry and of its bfloat16 decode.

Sliding window (the FlyDSL pull request "[Kernel][MI350] Add 8 wave GQA
sliding-window attention kernel", section What it does): query i attends to
keys [i - LEFT, i + RIGHT]; a negative bound is read as unbounded on that side
(so (-1, 0) is dense causal attention and (-1, -1) full attention).  bf16 I/O
is the dtype that page's kernel takes.  Each test checks the oracle against
an independent statement: torch's bfloat16 conversion, a dense masked softmax
written here with scipy, the dense entry, or a closed form.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch


def _rand(rng, B, M, N, H, G, D, scale=1.0):
    q = (rng.standard_normal((B, M, H, D)) * scale).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    return q, k, v


def _band_reference(qd, kd, vd, left, right):
    """Masked softmax attention over an explicit [M, N] band mask (fp64)."""
    B, M, H, D = qd.shape
    N, G = kd.shape[1], kd.shape[2]
    gs = H // G
    m = np.arange(M)[:, None]
    n = np.arange(N)[None, :]
    mask = np.ones((M, N), dtype=bool)
    if left >= 0:
        mask &= n >= m - left
    if right >= 0:
        mask &= n <= m + right
    rows = mask.any(axis=1)
    O = np.zeros((B, M, H, D))
    L = np.full((B, H, M), -np.inf)
    for b in range(B):
        for h in range(H):
            g = h // gs
            s = np.where(mask, qd[b, :, h] @ kd[b, :, g].T / math.sqrt(D), -np.inf)
            O[b, rows, h] = scipy.special.softmax(s[rows], axis=1) @ vd[b, :, g]
            L[b, h, rows] = scipy.special.logsumexp(s[rows], axis=1)
    return O, L


@pytest.mark.parametrize("bits_lo", [0, 1 << 15])
def test_bf16_decode_matches_torch(oracle_mod, bits_lo):
    """Exact bfloat16 decode on all 2**15 patterns of each sign."""
    bits = np.arange(bits_lo, bits_lo + (1 << 15), dtype=np.int64)
    ref = torch.tensor(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_mod.bf16_to_double(int(x)) for x in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


WINDOWS = [(0, 0), (3, 0), (5, 2), (-1, 3), (-1, -1), (7, -1), (-1, 0), (16, 0)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("shape", [(1, 40, 40, 4, 2, 16), (2, 33, 21, 3, 1, 8), (1, 20, 37, 6, 3, 32)])
def test_window_matches_band_mask(oracle_mod, shape, window):
    B, M, N, H, G, D = shape
    rng = np.random.default_rng(sum(shape) + 7 * window[0] + window[1])
    q, k, v = _rand(rng, B, M, N, H, G, D)
    O, L = oracle_mod.window_full(q, k, v, *window)
    Or, Lr = _band_reference(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), *window)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lr))
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(Lr)
    np.testing.assert_allclose(L[fin], Lr[fin], rtol=1e-12, atol=1e-12)
    assert np.all(O[np.isneginf(L).transpose(0, 2, 1)] == 0.0)


def test_causal_window_is_the_dense_entry(oracle_mod):
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 50, 50, 4, 2, 16)
    O1, L1 = oracle_mod.window_full(q, k, v, -1, 0)
    O2, L2 = oracle_mod.dense_full(q, k, v)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_zero_window_closed_form(oracle_mod):
    """(0, 0): each query sees only key m, so O = v_m and LSE = q.k_m / sqrt(D)."""
    rng = np.random.default_rng(4)
    B, M, N, H, G, D = 1, 12, 12, 4, 2, 8
    q, k, v = _rand(rng, B, M, N, H, G, D)
    O, L = oracle_mod.window_full(q, k, v, 0, 0)
    gs = H // G
    for h in range(H):
        g = h // gs
        assert np.array_equal(O[0, :, h], v[0, :, g].astype(np.float64))
        s = (q[0, :, h].astype(np.float64) * k[0, :, g].astype(np.float64)).sum(axis=1) / math.sqrt(D)
        np.testing.assert_allclose(L[0, h], s, rtol=1e-15, atol=1e-15)


def test_bf16_inputs(oracle_mod):
    """bf16 inputs (as bit patterns) give the attention of their exact values."""
    rng = np.random.default_rng(5)
    B, M, N, H, G, D = 1, 30, 30, 4, 2, 16
    qf = torch.randn(B, M, H, D, dtype=torch.float64, generator=torch.Generator().manual_seed(1))
    kf = torch.randn(B, N, G, D, dtype=torch.float64, generator=torch.Generator().manual_seed(2))
    vf = torch.randn(B, N, G, D, dtype=torch.float64, generator=torch.Generator().manual_seed(3))
    bits = [t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16) for t in (qf, kf, vf)]
    dec = [t.to(torch.bfloat16).to(torch.float64).numpy() for t in (qf, kf, vf)]
    for window in ((-1, 0), (4, 1)):
        O, L = oracle_mod.window_full(*bits, *window, dtype="bf16")
        Or, Lr = _band_reference(*dec, *window)
        np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, Lr, rtol=1e-12, atol=1e-12)
    # and through the index-row entry: every causal block selected
    bs = 8
    idx = np.broadcast_to(np.arange(4, dtype=np.int32), (B, M, G, 4)).copy()
    O, L = oracle_mod.oracle_full(*bits, idx, bs, dtype="bf16")
    Or, Lr = _band_reference(*dec, -1, 0)
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=1e-12, atol=1e-12)
    del rng


def test_window_rejects_bad_arguments(oracle_mod):
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 1, 8, 8, 2, 1, 4)
    with pytest.raises(ValueError):
        oracle_mod.window_units(q, k, v, 2, 0, np.array([[0, 8, 0]]))
    with pytest.raises(ValueError):
        oracle_mod.window_units(q.view(np.uint16), k, v, 2, 0, np.array([[0, 0, 0]]), dtype="bf16")
