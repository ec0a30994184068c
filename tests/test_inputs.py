"""Properties of the seeded input generator (values and index rows)."""

import numpy as np
import pytest
import scipy.stats

from block_sparse_attention_sel_amd.inputs import (CONFIGS, Config, block_indices, make_inputs,
                                                   normal_fp16, sample_units)


def _check_rows(cfg, idx):
    B, M, G, T = idx.shape
    bs = cfg.block_size
    c = (np.arange(M) // bs)[None, :, None]
    valid = idx >= 0
    # Valid entries first, then -1 padding.
    assert np.all(np.diff(valid.astype(np.int8), axis=-1) <= 0)
    # Strictly ascending valid entries (sorted, no repeats).
    v = np.where(valid, idx, np.iinfo(np.int32).max)
    d = np.diff(v, axis=-1)
    both = valid[..., 1:] & valid[..., :-1]
    assert np.all(d[both] > 0)
    # Causal: every entry at or before the own block; block 0 and block c present.
    assert np.all(np.where(valid, idx <= c[..., None], True))
    assert np.all(idx[..., 0] == 0)
    assert np.all((idx == c[..., None]).any(axis=-1))
    # Exactly min(T, c + 1) valid entries.
    assert np.array_equal(valid.sum(-1), np.broadcast_to(np.minimum(T, c + 1), valid.sum(-1).shape))


@pytest.mark.parametrize("name", ["tiny", "8k"])
def test_uniform_rows_are_well_formed(name):
    cfg = CONFIGS[name]
    _check_rows(cfg, block_indices(cfg))


def test_bs32_rows_are_well_formed():
    cfg = CONFIGS["32k-bs32"].with_(M=8192, N=8192)
    _check_rows(cfg, block_indices(cfg))


def test_geometric_rows_are_well_formed():
    cfg = CONFIGS["128k-local"].with_(M=16384, N=16384)
    _check_rows(cfg, block_indices(cfg))


def test_dense_rows_select_every_causal_block():
    cfg = CONFIGS["tiny"].dense()
    idx = block_indices(cfg)
    assert idx.shape[-1] == cfg.NB
    _check_rows(cfg, idx)


def test_uniform_inclusion_rate():
    """Each of blocks 1..c-1 is picked with probability (T-2)/(c-1)."""
    cfg = Config("u", B=1, M=64 * 41, N=64 * 41, H=1, G=64, D=8, block_size=64, T=8, seed=21)
    idx = block_indices(cfg)
    c = 40
    rows = idx[0, c * 64:(c + 1) * 64].reshape(-1, cfg.T)        # 64 * 64 rows with c = 40
    counts = np.bincount(rows[rows > 0].ravel(), minlength=c + 1)[1:c]
    expected = rows.shape[0] * (cfg.T - 2) / (c - 1)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert scipy.stats.chi2.sf(chi2, df=c - 2) > 1e-4


def test_geometric_distance_of_first_pick():
    """For large c, the closest picked block lies at distance d with the law of
    the minimum of the accepted geometric draws; the first draw alone follows
    Geom(0.1), so P(d_min = 1) is at least 0.1 and the mean distance is small."""
    cfg = CONFIGS["128k-local"].with_(M=64 * 1024, N=64 * 1024, G=8)
    idx = block_indices(cfg)
    m = np.arange(64 * 900, 64 * 1024)
    c = m // 64
    rows = idx[0, m]                                            # [m, G, T]
    others = np.where((rows > 0) & (rows < c[:, None, None]), rows, -1)
    dist = c[:, None, None] - others
    dmin = np.where(others > 0, dist, 10**9).min(axis=-1)
    frac1 = (dmin == 1).mean()
    assert frac1 > 0.5
    # All 14 picks lie within a few dozen blocks with high probability.
    far = np.where(others > 0, dist, 0).max(axis=-1)
    assert np.median(far) < 60


def test_values_are_standard_normal_fp16():
    x = normal_fp16((1 << 20,), seed=3, stream=1).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert scipy.stats.kstest(x[:20000], "norm").pvalue > 1e-4


def test_determinism_independent_of_threads():
    cfg = CONFIGS["8k"].with_(M=4096, N=4096)
    a = make_inputs(cfg, threads=1)
    b = make_inputs(cfg, threads=7)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
    x = normal_fp16((3 << 22,), seed=1, stream=2, threads=1)
    y = normal_fp16((3 << 22,), seed=1, stream=2, threads=4)
    assert x.tobytes() == y.tobytes()


def test_streams_and_seeds_differ():
    a = normal_fp16((4096,), seed=1, stream=1)
    b = normal_fp16((4096,), seed=1, stream=2)
    c = normal_fp16((4096,), seed=2, stream=1)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_sample_units_cover_edges_and_are_unique():
    cfg = CONFIGS["64k"]
    u = sample_units(cfg, 4096)
    key = (u[:, 0] * cfg.M + u[:, 1]) * cfg.G + u[:, 2]
    assert np.unique(key).size == key.size
    assert (u[:, 1] == 0).sum() == cfg.G and (u[:, 1] == cfg.M - 1).sum() == cfg.G
    assert np.all((u >= 0) & (u < np.array([cfg.B, cfg.M, cfg.G])))


def test_bf16_rounding_matches_torch():
    import torch
    from block_sparse_attention_sel_amd.inputs import normal_bf16, normal_fp16, to_bf16_bits
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(1 << 16) * np.exp(rng.uniform(-20, 20, 1 << 16))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0, -3.5]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_bf16_bits(x), want)
    # same draws as the fp16 generator: the two roundings of one float32 agree to bf16 precision
    a = normal_bf16((3, 1000), 5, 1)
    b = normal_fp16((3, 1000), 5, 1).astype(np.float32)
    af = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.all(np.abs(af - b) <= 2.0 ** -8 * np.abs(b) + 2.0 ** -14)
