"""The gather-ceiling probe (include/nsa_gather_probe.h) on the GPU: it must
stage exactly the merged blocks of every wavefront slot, which the host
recomputes from the index rows (an exact integer check of the slot layout and
the row merging that the forward kernel shares)."""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, block_indices, make_inputs, normal_fp16

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


def expected_staged(idx: np.ndarray, bs: int, N: int, qps: int) -> int:
    """Sum over slots (qps consecutive queries of one (b, g), from m = 0) of
    the number of distinct counted blocks in the slot's rows."""
    B, M, G, T = idx.shape
    NB = -(-N // bs)
    c = (np.arange(M) // bs)[None, :, None, None]
    e = np.where((idx >= 0) & (idx <= c) & (idx < NB), idx, -1).astype(np.int64)
    pad = (-M) % qps
    if pad:
        e = np.concatenate([e, np.full((B, pad, G, T), -1, np.int64)], axis=1)
    e = e.transpose(0, 2, 1, 3).reshape(B, G, -1, qps * T)
    e = np.sort(e, axis=-1)
    fresh = (e[..., 1:] != e[..., :-1]) & (e[..., 1:] >= 0)
    return int(fresh.sum() + (e[..., 0] >= 0).sum())


def _probe(torch, cfg, idx):
    from block_sparse_attention_sel_amd import binding
    k = normal_fp16((cfg.B, cfg.N, cfg.G, cfg.D), cfg.seed, 2)
    tk = torch.from_numpy(k).to("cuda")
    tv = tk.clone()
    ti = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda")
    staged = torch.zeros(1, dtype=torch.int64, device="cuda")
    qps = binding.nsa_gather_probe(tk, tv, ti, staged, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D,
                                   cfg.block_size, cfg.T, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return int(staged.item()), qps


SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 300, 300, 4, 4, 64, 32, 5),
    (2, 129, 129, 16, 2, 128, 64, 70),     # one tile, rows streamed (T > 64)
    (1, 4096, 4096, 16, 8, 64, 64, 8),
    (1, 4096, 4096, 40, 8, 128, 64, 8),
    (1, 3000, 4030, 16, 8, 64, 32, 8),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_probe_stages_the_merged_blocks(torch_cuda, shape):
    B, M, N, H, G, D, bs, T = shape
    _say(f"case probe shape={shape}")
    cfg = Config("p", B=B, M=M, N=N, H=H, G=G, D=D, block_size=bs, T=T, seed=sum(shape))
    rng = np.random.default_rng(sum(shape))
    idx = block_indices(cfg).copy()
    # Padding, future and out-of-range entries in some empty slots; rows
    # sorted so that the streamed-row path also merges to the exact union.
    c = (np.arange(M) // bs)[None, :, None, None]
    junk = np.where(rng.random(idx.shape) < 0.5, c + 1, cfg.NB + 3)
    idx = np.where((idx < 0) & (rng.random(idx.shape) < 0.5), junk, idx)
    idx = np.sort(idx, axis=-1).astype(np.int32)
    got, qps = _probe(torch_cuda, cfg, idx)
    want = expected_staged(idx, bs, N, qps)
    _say(f"  queries per slot {qps}: staged {got}, expected {want}")
    assert got == want


@pytest.mark.parametrize("name", ["64k", "32k-bs32"])
def test_probe_full_size(torch_cuda, name):
    cfg = CONFIGS[name]
    _say(f"case probe config={name}")
    idx = block_indices(cfg)
    got, qps = _probe(torch_cuda, cfg, idx)
    want = expected_staged(idx, cfg.block_size, cfg.N, qps)
    _say(f"  queries per slot {qps}: staged {got}, expected {want}")
    assert got == want
