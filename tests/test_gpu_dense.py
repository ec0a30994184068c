"""Dense causal GQA attention (include/nsa_dense.h) on the GPU against the
fp64 oracle's dense entry: every key n <= m (n < N) visible.

Tolerances as for the selection kernel: O max-abs 5e-3, LSE max-abs 1e-3.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, make_inputs, normal_fp16, sample_units

pytestmark = pytest.mark.gpu

O_TOL = 5e-3
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _qkv(B, M, N, H, G, D, seed):
    return (normal_fp16((B, M, H, D), seed, 1), normal_fp16((B, N, G, D), seed, 2),
            normal_fp16((B, N, G, D), seed, 3))


def _run(torch, q, k, v):
    from block_sparse_attention_sel_amd.binding import dense_attn_fwd
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in (q, k, v))
    O, L = dense_attn_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    return O.cpu().numpy(), L.cpu().numpy()


def _check(O, L, Or, Lr):
    O = O.astype(np.float64)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    errO = np.abs(O - Or).max()
    errL = np.abs(L - Lr).max()
    _say(f"  max|dO| = {errO:.3e}  max|dLSE| = {errL:.3e}")
    assert errO <= O_TOL
    assert errL <= LSE_TOL


SHAPES = [
    # B, M, N, H, G, D
    (1, 1024, 1024, 64, 8, 128),   # the headline's head layout (gs = 8)
    (2, 640, 640, 8, 8, 64),       # gs = 1 (four queries per tile)
    (1, 777, 900, 16, 1, 128),     # gs = 16, M < N, ragged tiles
    (1, 1000, 600, 12, 3, 64),     # gs = 4, M > N (late queries see every key)
    (1, 300, 300, 10, 2, 128),     # gs = 5: padding columns in every tile
    (1, 33, 33, 8, 8, 128),        # fewer queries than one workgroup carries
]


@pytest.mark.parametrize("shape", SHAPES)
def test_dense_parity_full_coverage(torch_cuda, shape):
    import oracle
    B, M, N, H, G, D = shape
    _say(f"case dense shape={shape}")
    q, k, v = _qkv(B, M, N, H, G, D, seed=sum(shape))
    O, L = _run(torch_cuda, q, k, v)
    Or, Lr = oracle.dense_full(q, k, v)
    _check(O, L, Or, Lr)


def test_dense_parity_headline_sampled(torch_cuda):
    """M = N = 65536, H = 64, G = 8, D = 128: the first two query blocks, the
    last one and random units, each against the oracle's dense entry."""
    import oracle
    cfg = CONFIGS["64k"]
    _say(f"case dense full-size {cfg}")
    q, k, v = _qkv(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, seed=cfg.seed)
    O, L = _run(torch_cuda, q, k, v)
    units = sample_units(cfg, 256, tail=1)
    Or, Lr = oracle.dense_units(q, k, v, units)
    gs = cfg.gs
    for i, (b, m, g) in enumerate(units):
        h = slice(g * gs, (g + 1) * gs)
        errO = np.abs(O[b, m, h].astype(np.float64) - Or[i]).max()
        errL = np.abs(L[b, h, m] - Lr[i]).max()
        assert errO <= O_TOL and errL <= LSE_TOL, (b, m, g, errO, errL)
    _say(f"  {len(units)} units within tolerance")


def test_dense_large_scores(torch_cuda):
    """Scores 16x larger keep P inside fp16 only with a correct running max."""
    import oracle
    B, M, N, H, G, D = 1, 1024, 1024, 64, 8, 128
    _say("case dense large scores")
    q, k, v = _qkv(B, M, N, H, G, D, seed=5)
    q = (q.astype(np.float32) * 16.0).astype(np.float16)
    O, L = _run(torch_cuda, q, k, v)
    Or, Lr = oracle.dense_full(q, k, v)
    _check(O, L, Or, Lr)


def test_dense_equals_selection_of_every_block_within_tolerance(torch_cuda):
    """The dense kernel and the selection kernel with every causal block
    selected compute the same function (to rounding)."""
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    from block_sparse_attention_sel_amd.inputs import block_indices
    torch = torch_cuda
    cfg = CONFIGS["64k"].with_(M=2048, N=2048).dense()
    q, k, v, idx = make_inputs(cfg)
    O1, L1 = _run(torch, q, k, v)
    tq, tk, tv, ti = (torch.from_numpy(a).to("cuda") for a in (q, k, v, idx))
    O2, L2 = sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    torch.cuda.synchronize()
    assert np.abs(O1.astype(np.float64) - O2.cpu().numpy().astype(np.float64)).max() <= 2 * O_TOL
    assert np.abs(L1 - L2.cpu().numpy()).max() <= 2 * LSE_TOL


def test_dense_repeat_runs_are_bitwise_identical(torch_cuda):
    B, M, N, H, G, D = 1, 2048, 2048, 64, 8, 128
    q, k, v = _qkv(B, M, N, H, G, D, seed=9)
    O1, L1 = _run(torch_cuda, q, k, v)
    O2, L2 = _run(torch_cuda, q, k, v)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["8k", "16k"])
def test_dense_every_unit(torch_cuda, name):
    """Every unit against the oracle, streamed in unit ranges: the 8k
    workload's shape (M = N = 8192, H = 32, G = 2, D = 128) and M = N = 16384
    with the 64k workload's heads (H = 64, G = 8, D = 128)."""
    import os
    import time

    import oracle
    cfg = CONFIGS["8k"] if name == "8k" else CONFIGS["64k"].with_(M=16384, N=16384)
    _say(f"case dense {cfg} (every unit)")
    q, k, v = _qkv(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, seed=cfg.seed)
    O, L = _run(torch_cuda, q, k, v)
    threads = max(1, min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))))
    U = cfg.B * cfg.M * cfg.G
    t0 = time.perf_counter()
    for i in range(4):
        u0, u1 = U * i // 4, U * (i + 1) // 4
        r = oracle.compare(q, k, v, None, cfg.block_size, O, L, u0, u1, threads)
        _say(f"  units {u0}..{u1 - 1}: max|dO| = {r['max_err_O']:.3e}  max|dLSE| = {r['max_err_LSE']:.3e}"
             f"  {time.perf_counter() - t0:.1f} s")
        assert r["units"] == u1 - u0 and r["bad_rows"] == 0 and r["empty_rows"] == 0
        assert r["max_err_O"] <= O_TOL and r["max_err_LSE"] <= LSE_TOL
