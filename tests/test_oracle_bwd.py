"""Pins of the fp64 CPU oracle's backward pass against facts that do not come
from the oracle.

The gradients are those of the selection attention defined in the wave issue
"[wave] NSA: selection attention forward kernel" (sections Operation and
Algorithm; section Requirements names the backward as the reason LSE is
returned).  Each test checks the oracle against an independent statement:
torch's automatic differentiation of an explicitly masked attention written
here in fp64, the shift invariance of softmax (its gradient sums to zero over
the keys), the normalisation of the probabilities (dV summed over keys is the
summed upstream gradient), and closed forms for one visible key and for
constant values.
"""

import math

import numpy as np
import pytest
import torch

from block_sparse_attention_sel_amd.inputs import Config, block_indices, make_grad_output, make_inputs


def _rand(rng, B, M, N, H, G, D):
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    do = rng.standard_normal((B, M, H, D)).astype(np.float16)
    return q, k, v, do


def _mask(idx, M, N, bs):
    """bool [B, G, M, N]: key n visible to query m of (b, g), from block
    membership of the row's valid entries and n <= m (plain loops)."""
    B, _, G, T = idx.shape
    NB = -(-N // bs)
    mask = np.zeros((B, G, M, N), dtype=bool)
    for b in range(B):
        for g in range(G):
            for m in range(M):
                for t in idx[b, m, g]:
                    if 0 <= t < NB:
                        lo, hi = t * bs, min(N, (t + 1) * bs, m + 1)
                        mask[b, g, m, lo:hi] = True
    return mask


def _autograd(q, k, v, do, mask):
    """fp64 gradients of explicitly masked attention by torch.autograd.
    Rows with no visible key have output 0 and contribute nothing."""
    B, M, H, D = q.shape
    G = k.shape[2]
    gs = H // G
    Q = torch.tensor(q.astype(np.float64), requires_grad=True)
    K = torch.tensor(k.astype(np.float64), requires_grad=True)
    V = torch.tensor(v.astype(np.float64), requires_grad=True)
    msk = torch.tensor(mask)                                         # [B, G, M, N]
    rows = msk.any(dim=3)                                            # [B, G, M]
    Kh = K.repeat_interleave(gs, dim=2).permute(0, 2, 1, 3)          # [B, H, N, D]
    Vh = V.repeat_interleave(gs, dim=2).permute(0, 2, 1, 3)
    Qh = Q.permute(0, 2, 1, 3)                                       # [B, H, M, D]
    s = torch.matmul(Qh, Kh.transpose(2, 3).contiguous()) / math.sqrt(D)
    mh = msk.repeat_interleave(gs, dim=1)                            # [B, H, M, N]
    rh = rows.repeat_interleave(gs, dim=1)                           # [B, H, M]
    s = torch.where(mh, s, torch.tensor(-math.inf, dtype=torch.float64))
    s = torch.where(rh[..., None], s, torch.zeros((), dtype=torch.float64))
    p = torch.softmax(s, dim=3) * rh[..., None]
    o = torch.matmul(p, Vh).permute(0, 2, 1, 3)                      # [B, M, H, D]
    o.backward(torch.tensor(do.astype(np.float64)))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 24, 24, 1, 1, 4, 4, 3),
    (2, 33, 33, 4, 2, 8, 4, 4),      # ragged tail block, B and G > 1
    (1, 40, 40, 6, 2, 16, 8, 2),     # gs = 3
    (2, 17, 29, 3, 3, 5, 2, 5),      # M < N, gs = 1, odd D
    (1, 37, 21, 4, 1, 8, 4, 3),      # M > N: late queries see every key
]


def _rand_idx(rng, B, M, N, G, bs, T):
    """Random rows mixing valid, future, out-of-range, repeated and padding
    entries."""
    NB = -(-N // bs)
    return rng.integers(-2, NB + 2, size=(B, M, G, T)).astype(np.int32)


@pytest.mark.parametrize("shape", SHAPES)
def test_autograd_selected(oracle_mod, shape):
    B, M, N, H, G, D, bs, T = shape
    rng = np.random.default_rng(11 + sum(shape))
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    idx = _rand_idx(rng, B, M, N, G, bs, T)
    dq_ref, dk_ref, dv_ref = _autograd(q, k, v, do, _mask(idx, M, N, bs))
    dq, dk, dv = oracle_mod.bwd_full(q, k, v, idx, do, bs)
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("shape", [(1, 48, 48, 4, 2, 16), (2, 30, 45, 6, 3, 8), (1, 50, 20, 2, 1, 32)])
def test_autograd_dense(oracle_mod, shape):
    """idx None is dense causal attention (every key n <= m, n < N)."""
    B, M, N, H, G, D = shape
    rng = np.random.default_rng(5 + sum(shape))
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    causal = np.arange(N)[None, :] <= np.arange(M)[:, None]
    mask = np.broadcast_to(causal, (B, G, M, N))
    dq_ref, dk_ref, dv_ref = _autograd(q, k, v, do, mask)
    dq, dk, dv = oracle_mod.bwd_full(q, k, v, None, do, 4)
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_generated_rows_autograd(oracle_mod):
    """Rows from the seeded generator (both rules) at a small shape."""
    for rule in ("uniform", "geometric"):
        cfg = Config("t", B=1, M=96, N=96, H=4, G=2, D=16, block_size=8, T=4, rule=rule, seed=7)
        q, k, v, idx = make_inputs(cfg)
        do = make_grad_output(cfg)
        dq_ref, dk_ref, dv_ref = _autograd(q, k, v, do, _mask(idx, cfg.M, cfg.N, cfg.block_size))
        dq, dk, dv = oracle_mod.bwd_full(q, k, v, idx, do, cfg.block_size)
        for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
            np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_key_sums(oracle_mod):
    """Softmax is invariant to a shift of its scores, so dS sums to zero over
    the keys of each row and sum_n dK[b, n, g] = 0; probabilities sum to one,
    so sum_n dV[b, n, g] equals dO summed over the rows that see a key."""
    B, M, N, H, G, D, bs, T = 2, 64, 64, 6, 2, 16, 8, 4
    rng = np.random.default_rng(3)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    idx = _rand_idx(rng, B, M, N, G, bs, T)
    _, dk, dv = oracle_mod.bwd_full(q, k, v, idx, do, bs)
    rows = _mask(idx, M, N, bs).any(axis=3)                           # [B, G, M]
    gs = H // G
    dod = do.astype(np.float64).reshape(B, M, G, gs, D)
    want = np.einsum("bgm,bmgid->bgd", rows.astype(np.float64), dod)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=1e-12, atol=1e-11)


def test_single_visible_key(oracle_mod):
    """Query 0 sees only key 0: P = 1, so dS = 0 (dQ = 0, no dK), and key 0
    receives dV = dO of its heads."""
    B, M, N, H, G, D, bs = 1, 8, 8, 4, 2, 8, 4
    rng = np.random.default_rng(9)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    idx = np.full((B, M, G, 2), -1, np.int32)
    idx[:, :, :, 0] = 0
    units = np.array([[0, 0, 0], [0, 0, 1]], np.int64)
    dq, dk, dv = oracle_mod.bwd_units(q, k, v, idx, do, bs, units)
    assert np.all(dq == 0.0)
    assert np.all(dk == 0.0)
    gs = H // G
    for g in range(G):
        want = do[0, 0, g * gs:(g + 1) * gs].astype(np.float64).sum(axis=0)
        np.testing.assert_array_equal(dv[0, 0, g], want)
        assert np.all(dv[0, 1:, g] == 0.0)


def test_constant_values(oracle_mod):
    """Equal value rows make O independent of the scores, so dQ = dK = 0."""
    B, M, N, H, G, D, bs, T = 1, 40, 40, 4, 1, 8, 4, 3
    rng = np.random.default_rng(4)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    v[:] = v[:, :1]
    idx = _rand_idx(rng, B, M, N, G, bs, T)
    dq, dk, _ = oracle_mod.bwd_full(q, k, v, idx, do, bs)
    assert np.abs(dq).max() < 1e-12
    assert np.abs(dk).max() < 1e-12


def test_key_block_filter(oracle_mod):
    """dK/dV restricted to listed key blocks equal the matching rows of the
    full-tensor result; rows past N stay zero."""
    B, M, N, H, G, D, bs, T = 2, 45, 45, 4, 2, 8, 8, 3
    rng = np.random.default_rng(8)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    idx = _rand_idx(rng, B, M, N, G, bs, T)
    dq_full, dk_full, dv_full = oracle_mod.bwd_full(q, k, v, idx, do, bs)
    kb = np.array([[0, 0, 0], [1, 1, 2], [0, 1, 5], [1, 0, 3]], np.int64)   # block 5 is the ragged tail
    units = oracle_mod.all_units(B, M, G)
    dq, dk, dv = oracle_mod.bwd_units(q, k, v, idx, do, bs, units, kb)
    np.testing.assert_array_equal(dq.reshape(B, M, H, D), dq_full)
    for i, (b, g, t) in enumerate(kb):
        n = min(bs, N - t * bs)
        np.testing.assert_allclose(dk[i, :n], dk_full[b, t * bs:t * bs + n, g], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(dv[i, :n], dv_full[b, t * bs:t * bs + n, g], rtol=1e-13, atol=1e-14)
        assert np.all(dk[i, n:] == 0.0) and np.all(dv[i, n:] == 0.0)


def test_padding_and_repeats_change_nothing(oracle_mod):
    """Negative, future-only and out-of-range entries add nothing; a repeated
    entry selects its block once."""
    B, M, N, H, G, D, bs = 1, 32, 32, 2, 1, 8, 4
    rng = np.random.default_rng(12)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    base = np.full((B, M, G, 2), -1, np.int32)
    base[..., 0] = 0
    base[..., 1] = (np.arange(M) // bs)[None, :, None]
    noisy = np.concatenate([base, np.full((B, M, G, 1), -7, np.int32), np.full((B, M, G, 1), 99, np.int32),
                            base[..., 1:2]], axis=3)
    ref = oracle_mod.bwd_full(q, k, v, base, do, bs)
    got = oracle_mod.bwd_full(q, k, v, noisy, do, bs)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


def test_thread_count(oracle_mod):
    cfg = Config("t", B=1, M=64, N=64, H=4, G=2, D=16, block_size=8, T=3, seed=2)
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    a = oracle_mod.bwd_full(q, k, v, idx, do, 8, threads=1)
    b = oracle_mod.bwd_full(q, k, v, idx, do, 8, threads=5)
    np.testing.assert_array_equal(a[0], b[0])                 # dQ: one thread per unit
    for x, y in zip(a[1:], b[1:]):                              # dK, dV: summation order differs
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


def test_rejects_bad_arguments(oracle_mod):
    rng = np.random.default_rng(0)
    q, k, v, do = _rand(rng, 1, 8, 8, 2, 1, 4)
    idx = np.zeros((1, 8, 1, 1), np.int32)
    with pytest.raises(ValueError):
        oracle_mod.bwd_units(q, k, v, idx, do, 4, np.array([[0, 8, 0]]))
    with pytest.raises(ValueError):
        oracle_mod.bwd_units(q, k, v, idx, do[:, :4].copy(), 4, np.array([[0, 0, 0]]))


def test_term_magnitudes(oracle_mod):
    """The error-scale output: for each gradient element, the L2 norm over its
    terms of |term| with dS taken as P (|dP| + sum_d |dO_d O_d|), checked
    against dense masked matrices written here (numpy, fp64)."""
    B, M, N, H, G, D, bs, T = 1, 40, 40, 4, 2, 8, 4, 3
    rng = np.random.default_rng(31)
    q, k, v, do = _rand(rng, B, M, N, H, G, D)
    idx = _rand_idx(rng, B, M, N, G, bs, T)
    mask = _mask(idx, M, N, bs)
    gs = H // G
    sc = 1.0 / math.sqrt(D)
    wq = np.zeros((B, M, H, D))
    wk = np.zeros((B, N, G, D))
    wv = np.zeros((B, N, G, D))
    for b in range(B):
        for g in range(G):
            K = k[b, :, g].astype(np.float64)
            V = v[b, :, g].astype(np.float64)
            for i in range(gs):
                h = g * gs + i
                Q = q[b, :, h].astype(np.float64)
                dO = do[b, :, h].astype(np.float64)
                s = np.where(mask[b, g], Q @ K.T * sc, -np.inf)
                rows = mask[b, g].any(axis=1)
                P = np.zeros((M, N))
                P[rows] = np.exp(s[rows] - s[rows].max(axis=1, keepdims=True))
                P[rows] /= P[rows].sum(axis=1, keepdims=True)
                dP = dO @ V.T
                O = P @ V
                adelta = np.abs(dO * O).sum(axis=1)
                dSm = P * (np.abs(dP) + adelta[:, None])
                wq[b, :, h] = np.sqrt((dSm ** 2) @ (K ** 2)) * sc
                wk[b, :, g] += (dSm ** 2).T @ (Q ** 2) * sc * sc
                wv[b, :, g] += (P ** 2).T @ (dO ** 2)
    _, _, _, mq, mk, mv = oracle_mod.bwd_full(q, k, v, idx, do, bs, mags=True)
    np.testing.assert_allclose(mq, wq, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(mk, np.sqrt(wk), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(mv, np.sqrt(wv), rtol=1e-10, atol=1e-14)
