"""Top-k block selection on the GPU (nsa_topk_blocks) against the oracle:
bit-exact index rows (integer output, ties broken by block index), and the
selection feeding the forward pass.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, block_scores, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu_topk(torch, scores, bs, T):
    from block_sparse_attention_sel_amd.binding import topk_blocks
    out = topk_blocks(torch.from_numpy(np.ascontiguousarray(scores)).to("cuda"), bs, T)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _special(rng, shape):
    s = (rng.integers(-3, 4, size=shape).astype(np.float32) / 2)
    flat = s.reshape(-1)
    pick = rng.choice(flat.size, size=flat.size // 8, replace=False)
    flat[pick[0::4]] = np.nan
    flat[pick[1::4]] = np.inf
    flat[pick[2::4]] = -np.inf
    flat[pick[3::4]] = -0.0
    return s


SHAPES = [
    # B, M, G, NB, bs, T
    (1, 1024, 1, 32, 32, 4),        # tiny workload's rows
    (2, 777, 3, 13, 64, 5),         # NB < 64, ragged
    (1, 3000, 2, 100, 32, 7),       # NB not a multiple of 64
    (1, 8192, 2, 128, 64, 16),      # the 8k workload's rows
    (1, 600, 1, 600, 1, 40),        # bs = 1, large T
    (1, 300, 1, 4096, 16, 3),       # the largest NB; most of the row is past the causal limit
    (1, 200, 2, 1, 64, 2),          # NB = 1
    (1, 900, 1, 900, 1, 90),        # T > 64: more keys than one register at the threshold
    (3, 499, 5, 70, 7, 9),          # B, G > 1; a wavefront's rows cross a batch boundary (m wraps to 0)
    (1, 4096, 1, 4096, 1, 16),      # bs = 1: row m has m + 1 candidates, so every register count 1..64 occurs
]


@pytest.mark.parametrize("shape", SHAPES)
def test_topk_exact(torch_cuda, oracle_mod, shape):
    B, M, G, NB, bs, T = shape
    rng = np.random.default_rng(sum(shape))
    for kind in ("normal", "special", "binary", "bits", "denormal"):
        if kind == "normal":
            scores = rng.standard_normal((B, M, G, NB)).astype(np.float32)
        elif kind == "special":
            scores = _special(rng, (B, M, G, NB))
        elif kind == "binary":  # two values: hundreds of keys tie at the T-th place
            scores = rng.integers(0, 2, size=(B, M, G, NB)).astype(np.float32)
        elif kind == "bits":  # every bit pattern: NaN payloads of both signs, infinities, denormals
            scores = rng.integers(0, 2**32, size=(B, M, G, NB), dtype=np.uint64).astype(np.uint32).view(np.float32)
        else:  # denormals and signed zeros only: the key map must keep them exact
            scores = (rng.integers(-40, 41, size=(B, M, G, NB)).astype(np.float32) * np.float32(2.0**-149))
            flat = scores.reshape(-1)
            flat[rng.random(flat.size) < 0.1] = -0.0
        got = _gpu_topk(torch_cuda, scores, bs, T)
        want = oracle_mod.topk_blocks(scores, bs, T)
        bad = np.argwhere((got != want).any(axis=3))
        _say(f"  {shape} {kind}: {len(bad)} rows differ")
        assert np.array_equal(got, want), bad[:5]


@pytest.mark.parametrize("name", ["64k", "32k-bs32", "128k-local"])
def test_topk_full_size_sampled(torch_cuda, oracle_mod, name):
    """Full-size score tensors; 4000 sampled rows (and the first and last
    query blocks) compared exactly."""
    cfg = CONFIGS[name]
    _say(f"case {cfg}")
    scores = block_scores(cfg)
    got = _gpu_topk(torch_cuda, scores, cfg.block_size, cfg.T)
    rng = np.random.default_rng(1)
    ms = np.unique(np.concatenate([np.arange(0, 2 * cfg.block_size), np.arange(cfg.M - cfg.block_size, cfg.M),
                                   rng.integers(0, cfg.M, 4000)]))
    for b in range(cfg.B):
        for g in range(cfg.G):
            want = oracle_mod.topk_rows(scores[b, ms, g], ms, cfg.block_size, cfg.T)
            assert np.array_equal(got[b, ms, g], want)
    # every row is a valid selection: ascending, causal, padded
    valid = got >= 0
    m = np.arange(cfg.M)[None, :, None, None]
    assert np.all(got[valid.nonzero()] <= np.broadcast_to(m // cfg.block_size, got.shape)[valid.nonzero()])
    assert np.all(np.diff(valid.astype(np.int8), axis=3) <= 0)           # padding only at the end
    both = valid[..., 1:] & valid[..., :-1]
    assert np.all(np.diff(got, axis=3)[both] > 0)                          # strictly ascending
    assert np.all(got[~valid] == -1)


def test_topk_feeds_the_forward(torch_cuda, oracle_mod):
    """Scores -> GPU top-k -> GPU forward equals oracle top-k -> oracle forward."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd, topk_blocks
    cfg = CONFIGS["8k"].with_(M=2048, N=2048)
    q, k, v, _ = make_inputs(cfg)
    scores = block_scores(cfg)
    idx = topk_blocks(torch.from_numpy(scores).to("cuda"), cfg.block_size, cfg.T)
    O, L = sel_attn_fwd(*(torch.from_numpy(a).to("cuda") for a in (q, k, v)), idx, cfg.block_size)
    torch.cuda.synchronize()
    ridx = oracle_mod.topk_blocks(scores, cfg.block_size, cfg.T)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    Or, Lr = oracle_mod.oracle_full(q, k, v, ridx, cfg.block_size)
    assert np.abs(O.cpu().numpy().astype(np.float64) - Or).max() <= 5e-3
    assert np.abs(L.cpu().numpy() - Lr).max() <= 1e-3


def test_topk_errors(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    s = torch.zeros((1, 64, 1, 8), dtype=torch.float32, device="cuda")
    o = torch.empty((1, 64, 1, 4), dtype=torch.int32, device="cuda")
    assert binding.nsa_topk_blocks_raw(s, o, 1, 64, 1, 8, 8, 4) == binding.NSA_SEL_OK
    assert binding.nsa_topk_blocks_raw(s, s, 1, 64, 1, 8, 8, 4) == binding.NSA_SEL_ERR_ALIAS
    assert binding.nsa_topk_blocks_raw(s, o, 1, 64, 1, 5000, 8, 4) == binding.NSA_SEL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
