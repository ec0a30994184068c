"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

The operation is the one in the wave issue "[wave] NSA: selection attention
forward kernel" (sections Operation, Algorithm and Requirements).  Each test
below checks the oracle against an independent statement of what that section
fixes: a library routine (numpy's fp16 decode, scipy's softmax/logsumexp,
torch's scaled-dot-product attention), a closed form, or an invariance.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, make_inputs


def _rand_inputs(rng, B, M, N, H, G, D):
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    return q, k, v


def _dense_reference(q, k, v, idx, bs):
    """Dense masked attention: an explicit [M, N] mask per (b, g), built from
    block membership and n <= m, with scipy's softmax / logsumexp."""
    B, M, H, D = q.shape
    N, G = k.shape[1], k.shape[2]
    gs = H // G
    NB = -(-N // bs)
    qd = q.astype(np.float64)
    kd = k.astype(np.float64)
    vd = v.astype(np.float64)
    O = np.zeros((B, M, H, D))
    L = np.full((B, H, M), -np.inf)
    n_blk = np.arange(N) // bs
    causal = np.arange(N)[None, :] <= np.arange(M)[:, None]          # [M, N]
    for b in range(B):
        for g in range(G):
            sel = np.zeros((M, NB), dtype=bool)
            for t in range(idx.shape[3]):
                col = idx[b, :, g, t]
                ok = (col >= 0) & (col < NB)
                sel[np.nonzero(ok)[0], col[ok]] = True
            mask = sel[:, n_blk] & causal                               # [M, N]
            for i in range(gs):
                h = g * gs + i
                s = (qd[b, :, h, :] @ kd[b, :, g, :].T) / math.sqrt(D)   # [M, N]
                s = np.where(mask, s, -np.inf)
                rows = mask.any(axis=1)
                lse = scipy.special.logsumexp(s[rows], axis=1)
                p = scipy.special.softmax(s[rows], axis=1)
                O[b, rows, h, :] = p @ vd[b, :, g, :]
                L[b, h, rows] = lse
    return O, L


@pytest.mark.parametrize("bits_lo", [0, 1 << 15])
def test_half_decode_matches_numpy(oracle_mod, bits_lo):
    """Exact binary16 decode, checked on all 2**15 patterns of each sign."""
    bits = np.arange(bits_lo, bits_lo + (1 << 15), dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.half_to_double(int(x)) for x in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 24, 24, 1, 1, 4, 4, 3),
    (2, 33, 33, 4, 2, 8, 4, 4),      # ragged tail block, B and G > 1
    (1, 40, 40, 6, 2, 16, 8, 2),     # gs = 3
    (2, 17, 29, 3, 3, 5, 2, 5),      # M < N, gs = 1, odd D
    (1, 64, 64, 8, 1, 32, 16, 3),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_bruteforce_dense_mask(oracle_mod, shape):
    """Random index rows with padding, future and out-of-range entries and
    repeats, against dense masked attention."""
    B, M, N, H, G, D, bs, T = shape
    rng = np.random.default_rng(sum(shape))
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    NB = -(-N // bs)
    idx = rng.integers(-2, NB + 2, size=(B, M, G, T)).astype(np.int32)
    O, L = oracle_mod.oracle_full(q, k, v, idx, bs)
    Or, Lr = _dense_reference(q, k, v, idx, bs)
    fin = np.isfinite(Lr)
    assert np.array_equal(fin, np.isfinite(L))
    assert np.abs(L[fin] - Lr[fin]).max() <= 1e-12
    assert np.abs(O - Or).max() <= 1e-12


def test_bruteforce_generated_tiny_rows(oracle_mod):
    """The tiny workload's own index rows, at a reduced length."""
    cfg = CONFIGS["tiny"].with_(M=256, N=256)
    q, k, v, idx = make_inputs(cfg)
    O, L = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size)
    Or, Lr = _dense_reference(q, k, v, idx, cfg.block_size)
    assert np.abs(L - Lr).max() <= 1e-12
    assert np.abs(O - Or).max() <= 1e-12


@pytest.mark.parametrize("shape", [(1, 128, 4, 2, 16, 32), (2, 96, 6, 3, 8, 16), (1, 64, 4, 1, 64, 64)])
def test_full_selection_is_causal_attention(oracle_mod, shape):
    """When every causal block is selected the result is plain causal
    attention: torch's scaled_dot_product_attention (fp64, CPU)."""
    B, M, H, G, D, bs = shape
    rng = np.random.default_rng(7)
    q, k, v = _rand_inputs(rng, B, M, M, H, G, D)
    cfg = Config("t", B=B, M=M, N=M, H=H, G=G, D=D, block_size=bs, T=1).dense()
    from block_sparse_attention_sel_amd.inputs import block_indices
    idx = block_indices(cfg)
    O, L = oracle_mod.oracle_full(q, k, v, idx, bs)
    gs = H // G
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)           # [B, H, M, D]
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    s = (qt @ kt.transpose(-1, -2)) / math.sqrt(D)
    s = s.masked_fill(torch.ones(M, M, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                                        # [B, H, M]
    assert np.abs(O - ref.permute(0, 2, 1, 3).numpy()).max() <= 1e-12
    assert np.abs(L - lse.numpy()).max() <= 1e-12


@pytest.mark.parametrize("shape", [(1, 128, 128, 4, 2, 16), (2, 70, 90, 6, 3, 8), (1, 100, 64, 8, 1, 64)])
def test_dense_entry_is_causal_attention(oracle_mod, shape):
    """The oracle's dense entry (no index array) is causal attention with
    key n visible iff n <= m and n < N: torch's scaled_dot_product_attention
    with an explicit mask (fp64, CPU), also for M != N."""
    B, M, N, H, G, D = shape
    rng = np.random.default_rng(11)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    O, L = oracle_mod.dense_full(q, k, v)
    gs = H // G
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    mask = torch.arange(N)[None, :] <= torch.arange(M)[:, None]                  # [M, N]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    s = ((qt @ kt.transpose(-1, -2)) / math.sqrt(D)).masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    assert np.abs(O - ref.permute(0, 2, 1, 3).numpy()).max() <= 1e-12
    assert np.abs(L - lse.numpy()).max() <= 1e-12


def test_generated_rows_that_cover_the_prefix(oracle_mod):
    """Rows of the 8k workload with m < T*bs select every causal block; on
    those rows the oracle equals causal attention (torch SDPA, fp64)."""
    cfg = CONFIGS["8k"].with_(M=1024, N=1024)
    q, k, v, idx = make_inputs(cfg)
    O, L = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size)
    gs = cfg.gs
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(gs, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    rows = slice(0, cfg.T * cfg.block_size)
    assert np.abs(O[:, rows] - ref.permute(0, 2, 1, 3).numpy()[:, rows]).max() <= 1e-12


def test_permutation_invariance_bitwise(oracle_mod):
    B, M, N, H, G, D, bs, T = 2, 80, 80, 4, 2, 16, 8, 6
    rng = np.random.default_rng(3)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    NB = N // bs
    idx = rng.integers(-1, NB, size=(B, M, G, T)).astype(np.int32)
    perm = np.argsort(rng.random((B, M, G, T)), axis=-1)
    idx2 = np.ascontiguousarray(np.take_along_axis(idx, perm, axis=-1))
    O1, L1 = oracle_mod.oracle_full(q, k, v, idx, bs)
    O2, L2 = oracle_mod.oracle_full(q, k, v, idx2, bs)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_single_visible_key(oracle_mod):
    """Only key m visible: O equals that key's value row and LSE its scaled score."""
    B, M, N, H, G, D, bs, T = 1, 64, 64, 4, 2, 32, 16, 4
    rng = np.random.default_rng(11)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    idx = np.full((B, M, G, T), -1, dtype=np.int32)
    idx[..., 0] = (np.arange(M) // bs)[None, :, None]     # own block only
    units = np.array([[0, c * bs, g] for c in range(M // bs) for g in range(G)])
    O, L = oracle_mod.oracle_units(q, k, v, idx, bs, units)
    gs = H // G
    for u, (b, m, g) in enumerate(units):
        for i in range(gs):
            h = g * gs + i
            assert np.array_equal(O[u, i], v[b, m, g].astype(np.float64))
            s = math.fsum(float(a) * float(c) for a, c in zip(q[b, m, h], k[b, m, g])) / math.sqrt(D)
            assert abs(L[u, i] - s) <= 1e-13 * max(1.0, abs(s))


def test_first_query_of_a_workload(oracle_mod):
    cfg = CONFIGS["tiny"]
    q, k, v, idx = make_inputs(cfg)
    O, L = oracle_mod.oracle_units(q, k, v, idx, cfg.block_size, np.array([[0, 0, 0]]))
    for i in range(cfg.gs):
        assert np.array_equal(O[0, i], v[0, 0, 0].astype(np.float64))
        s = math.fsum(float(a) * float(c) for a, c in zip(q[0, 0, i], k[0, 0, 0])) / math.sqrt(cfg.D)
        assert abs(L[0, i] - s) <= 1e-13


def test_closed_form_zero_keys(oracle_mod):
    """K = 0: every score is 0, so LSE = ln(#visible keys) and O = mean of V
    over the visible selected keys."""
    B, M, N, H, G, D, bs, T = 1, 48, 48, 2, 1, 8, 8, 3
    rng = np.random.default_rng(5)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    k[:] = 0
    idx = rng.integers(-1, N // bs, size=(B, M, G, T)).astype(np.int32)
    O, L = oracle_mod.oracle_full(q, k, v, idx, bs)
    for m in range(M):
        blocks = {int(t) for t in idx[0, m, 0] if t >= 0}
        keys = [n for n in range(N) if n // bs in blocks and n <= m]
        for h in range(H):
            if not keys:
                assert L[0, h, m] == -np.inf and not O[0, m, h].any()
                continue
            assert abs(L[0, h, m] - math.log(len(keys))) <= 1e-14
            mean = v[0, keys, 0].astype(np.float64).mean(axis=0)
            assert np.abs(O[0, m, h] - mean).max() <= 1e-14


def test_closed_form_constant_values(oracle_mod):
    B, M, N, H, G, D, bs, T = 1, 40, 40, 4, 2, 16, 4, 5
    rng = np.random.default_rng(6)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    v[:] = np.float16(0.375)
    idx = rng.integers(0, N // bs, size=(B, M, G, T)).astype(np.int32)
    idx[..., 0] = 0                                       # key 0 always visible
    O, _ = oracle_mod.oracle_full(q, k, v, idx, bs)
    assert np.abs(O - 0.375).max() <= 1e-15


def test_padding_future_and_out_of_range_entries_change_nothing(oracle_mod):
    """Entries < 0, blocks after the query's own block, and blocks past the
    end contribute nothing: the row equals its compacted form exactly."""
    B, M, N, H, G, D, bs, T = 1, 64, 64, 4, 2, 16, 8, 8
    NB = N // bs
    rng = np.random.default_rng(8)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    clean = np.full((B, M, G, T), -1, np.int32)
    noisy = np.full((B, M, G, T), -1, np.int32)
    for m in range(M):
        c = m // bs
        for g in range(G):
            chosen = sorted(set(rng.integers(0, c + 1, size=3).tolist()) | {c})
            clean[0, m, g, : len(chosen)] = chosen
            extra = [-1, -7, NB, NB + 3] + ([c + 1] if c + 1 < NB else [])
            row = chosen + extra[: T - len(chosen)]
            rng.shuffle(row)
            noisy[0, m, g, : len(row)] = row
    O1, L1 = oracle_mod.oracle_full(q, k, v, clean, bs)
    O2, L2 = oracle_mod.oracle_full(q, k, v, noisy, bs)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_repeated_entries_use_the_union(oracle_mod):
    B, M, N, H, G, D, bs, T = 1, 32, 32, 2, 1, 8, 4, 6
    rng = np.random.default_rng(9)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    base = np.full((B, M, G, T), -1, np.int32)
    rep = np.full((B, M, G, T), -1, np.int32)
    for m in range(M):
        c = m // bs
        base[0, m, 0, :2] = [0, c] if c else [0, -1]
        rep[0, m, 0, :4] = [c, 0, c, 0]
    O1, L1 = oracle_mod.oracle_full(q, k, v, base, bs)
    O2, L2 = oracle_mod.oracle_full(q, k, v, rep, bs)
    assert oracle_mod.oracle_units.last_dup_units == M
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_empty_row(oracle_mod):
    B, M, N, H, G, D, bs, T = 1, 8, 8, 2, 1, 8, 4, 2
    rng = np.random.default_rng(10)
    q, k, v = _rand_inputs(rng, B, M, N, H, G, D)
    idx = np.full((B, M, G, T), -1, np.int32)
    idx[0, 5, 0, 0] = 1                                  # only m = 5 sees anything
    O, L = oracle_mod.oracle_full(q, k, v, idx, bs)
    others = [m for m in range(M) if m != 5]
    assert np.all(L[0][:, others] == -np.inf)
    assert not O[0, others].any()
    assert np.isfinite(L[0, :, 5]).all()


def test_thread_count_does_not_change_results(oracle_mod):
    cfg = CONFIGS["tiny"].with_(M=128, N=128)
    q, k, v, idx = make_inputs(cfg)
    O1, L1 = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size, threads=1)
    O2, L2 = oracle_mod.oracle_full(q, k, v, idx, cfg.block_size, threads=5)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_rejects_bad_arguments(oracle_mod):
    q = np.zeros((1, 4, 2, 8), np.float16)
    k = np.zeros((1, 4, 1, 8), np.float16)
    idx = np.zeros((1, 4, 1, 1), np.int32)
    with pytest.raises(ValueError):
        oracle_mod.oracle_units(q, k, k, idx, 2, np.array([[0, 4, 0]]))
    with pytest.raises(ValueError):
        oracle_mod.oracle_units(q, k, k, idx.astype(np.int64), 2, np.array([[0, 0, 0]]))
