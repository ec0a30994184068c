"""Sliding-window attention (nsa_window_fwd, fp16 and bf16) and the bf16
selection forward (nsa_sel_fwd_bf16) on the GPU against the fp64 oracle.

Tolerances.  fp16 operands: O max-abs 5e-3 and LSE max-abs 1e-3, as for the
fp16 selection forward.  bf16 operands: the products Q K^T are exact in fp32
and summed in fp32, so LSE keeps the 1e-3 bound; O takes P rounded to bf16
(relative error at most 2^-9 each) and is itself rounded to bf16 (at most
2^-9 |O|), so |error| <= 2^-9 (sum_n P_n |v_n| + |O|) <= 2^-9 (max|V| +
max|O|); the test allows 1.25 times that for the fp32 accumulation.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import (CONFIGS, Config, make_inputs, make_inputs_bf16,
                                                   sample_units)

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


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def _host(torch, t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _bf16_values(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _o_tol(dtype, v, Or):
    if dtype == "fp16":
        return O_TOL
    return 1.25 * 2.0 ** -9 * (np.abs(_bf16_values(v)).max() + np.abs(Or).max())


def _check(O, L, Or, Lr, otol):
    assert not np.isnan(O).any() and not np.isnan(L).any()
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty)
    assert np.all(L[empty] == -np.inf)
    errO = np.abs(O - Or).max()
    errL = np.abs(L[~empty] - Lr[~empty]).max() if (~empty).any() else 0.0
    _say(f"  max|dO| = {errO:.3e} (bound {otol:.3e})  max|dLSE| = {errL:.3e}  empty rows {int(empty.sum())}")
    assert errO <= otol
    assert errL <= LSE_TOL


def _window_case(torch, cfg, left, right, dtype):
    import oracle
    from block_sparse_attention_sel_amd.binding import window_attn_fwd
    _say(f"case {cfg} window ({left}, {right}) {dtype}")
    q, k, v, _ = (make_inputs_bf16 if dtype == "bf16" else make_inputs)(cfg)
    O, L = window_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), left, right)
    torch.cuda.synchronize()
    Or, Lr = oracle.window_full(q, k, v, left, right, dtype=dtype)
    _check(_host(torch, O), L.cpu().numpy(), Or, Lr, _o_tol(dtype, v, Or))


SHAPES = {
    "gs4-d64": Config("w1", B=1, M=700, N=700, H=4, G=1, D=64, block_size=32, T=1, seed=31),
    "gs8-b2": Config("w2", B=2, M=333, N=333, H=16, G=2, D=128, block_size=64, T=1, seed=32),
    "gs16-m-gt-n": Config("w3", B=1, M=300, N=100, H=16, G=1, D=128, block_size=64, T=1, seed=33),
    "gs3-m-lt-n": Config("w4", B=1, M=200, N=450, H=6, G=2, D=64, block_size=32, T=1, seed=34),
}
WINDOWS = [(0, 0), (16, 0), (100, 0), (5, 7), (-1, 3), (-1, -1), (64, -1), (-1, 0), (300, 40)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("shape", list(SHAPES))
def test_window_fp16(torch_cuda, shape, window):
    _window_case(torch_cuda, SHAPES[shape], *window, "fp16")


@pytest.mark.parametrize("window", [(0, 0), (37, 0), (-1, 0), (10, 20), (-1, -1)])
@pytest.mark.parametrize("shape", ["gs8-b2", "gs16-m-gt-n", "gs3-m-lt-n"])
def test_window_bf16(torch_cuda, shape, window):
    _window_case(torch_cuda, SHAPES[shape], *window, "bf16")


def test_causal_window_is_the_dense_kernel(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import dense_attn_fwd, window_attn_fwd
    cfg = SHAPES["gs8-b2"]
    q, k, v, _ = make_inputs(cfg)
    tq, tk, tv = (_dev(torch, a) for a in (q, k, v))
    O1, L1 = window_attn_fwd(tq, tk, tv, -1, 0)
    O2, L2 = dense_attn_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("window", [(8192, 0), (512, 0)])
def test_window_64k_sampled(torch_cuda, window, dtype):
    """The FlyDSL page's shape (B=1, H=64, H_KV=8, D=128, seq 65536) and windows."""
    torch = torch_cuda
    import oracle
    from block_sparse_attention_sel_amd.binding import window_attn_fwd
    cfg = CONFIGS["64k"]
    _say(f"case 64k window {window} {dtype}")
    q, k, v, _ = (make_inputs_bf16 if dtype == "bf16" else make_inputs)(cfg)
    O, L = window_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), *window)
    torch.cuda.synchronize()
    units = sample_units(cfg, 300, tail=1)
    Or, Lr = oracle.window_units(q, k, v, *window, units, dtype=dtype)
    On, Ln = _host(torch, O), L.cpu().numpy()
    gs = cfg.gs
    got_O = np.stack([On[b, m, g * gs:(g + 1) * gs] for b, m, g in units])
    got_L = np.stack([Ln[b, g * gs:(g + 1) * gs, m] for b, m, g in units])
    _check(got_O, got_L, Or, Lr, _o_tol(dtype, v, Or))


BF16_SEL = {
    "tiny": CONFIGS["tiny"],
    "8k@2048": CONFIGS["8k"].with_(M=2048, N=2048),
    "32k-bs32@2048": CONFIGS["32k-bs32"].with_(M=2048, N=2048),
    "128k-local@4096": CONFIGS["128k-local"].with_(M=4096, N=4096),
}


@pytest.mark.parametrize("name", list(BF16_SEL))
def test_selection_bf16_full(torch_cuda, name):
    torch = torch_cuda
    import oracle
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = BF16_SEL[name]
    _say(f"case {cfg} bf16")
    q, k, v, idx = make_inputs_bf16(cfg)
    O, L = sel_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), _dev(torch, idx), cfg.block_size)
    torch.cuda.synchronize()
    assert O.dtype == torch.bfloat16
    Or, Lr = oracle.oracle_full(q, k, v, idx, cfg.block_size, dtype="bf16")
    _check(_host(torch, O), L.cpu().numpy(), Or, Lr, _o_tol("bf16", v, Or))


def test_selection_bf16_64k_sampled(torch_cuda):
    torch = torch_cuda
    import oracle
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = CONFIGS["64k"]
    _say("case 64k selection bf16")
    q, k, v, idx = make_inputs_bf16(cfg)
    O, L = sel_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), _dev(torch, idx), cfg.block_size)
    torch.cuda.synchronize()
    units = sample_units(cfg, 600, tail=1)
    Or, Lr = oracle.oracle_units(q, k, v, idx, cfg.block_size, units, dtype="bf16")
    On, Ln = _host(torch, O), L.cpu().numpy()
    gs = cfg.gs
    got_O = np.stack([On[b, m, g * gs:(g + 1) * gs] for b, m, g in units])
    got_L = np.stack([Ln[b, g * gs:(g + 1) * gs, m] for b, m, g in units])
    _check(got_O, got_L, Or, Lr, _o_tol("bf16", v, Or))


def test_selection_bf16_matches_fp16_path_structure(torch_cuda):
    """The bf16 entry with inputs that are exact in both types (small
    integers / 8) agrees with the fp16 entry to bf16 output rounding."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = CONFIGS["tiny"]
    _, _, _, idx = make_inputs(cfg)
    rng = np.random.default_rng(3)
    arrs = [rng.integers(-8, 9, size=s).astype(np.float32) / 8 for s in
            ((cfg.B, cfg.M, cfg.H, cfg.D), (cfg.B, cfg.N, cfg.G, cfg.D), (cfg.B, cfg.N, cfg.G, cfg.D))]
    t16 = [torch.from_numpy(a).to("cuda").half() for a in arrs]
    tbf = [torch.from_numpy(a).to("cuda").bfloat16() for a in arrs]
    ti = _dev(torch, idx)
    O16, L16 = sel_attn_fwd(*t16, ti, cfg.block_size)
    Obf, Lbf = sel_attn_fwd(*tbf, ti, cfg.block_size)
    torch.cuda.synchronize()
    assert torch.allclose(L16, Lbf, atol=1e-4, rtol=0)
    assert (O16.float() - Obf.float()).abs().max().item() <= 2.0 ** -8 * (1 + O16.float().abs().max().item())


def _oracle_threads() -> int:
    import os
    n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n))))


def _every_unit(torch, q, k, v, idx, bs, O, L, dtype, window=None, chunks=4):
    """Compares every (b, m, g) unit of a GPU result with the oracle, streamed
    in unit ranges.  The bf16 O bound takes max|O| from the GPU output: it
    differs from the reference's by at most the error being bounded."""
    import time

    import oracle
    if dtype == "bf16":
        On = O.view(torch.int16).cpu().numpy().view(np.uint16)
        otol = 1.25 * 2.0 ** -9 * (np.abs(_bf16_values(v)).max() + O.float().abs().max().item())
    else:
        On = O.cpu().numpy()
        otol = O_TOL
    Ln = L.cpu().numpy()
    B, M, _, _ = q.shape
    G = k.shape[2]
    U = B * M * G
    t0 = time.perf_counter()
    for i in range(chunks):
        u0, u1 = U * i // chunks, U * (i + 1) // chunks
        r = oracle.compare(q, k, v, idx, bs, On, Ln, u0, u1, _oracle_threads(), dtype=dtype, window=window)
        _say(f"  units {u0}..{u1 - 1}: max|dO| = {r['max_err_O']:.3e} (bound {otol:.3e}, unit {r['worst_unit_O']})"
             f"  max|dLSE| = {r['max_err_LSE']:.3e}  bad rows {r['bad_rows']}  empty rows {r['empty_rows']}"
             f"  {time.perf_counter() - t0:.1f} s")
        assert r["units"] == u1 - u0 and r["bad_rows"] == 0
        assert r["max_err_O"] <= otol and r["max_err_LSE"] <= LSE_TOL


@pytest.mark.timeout(900)
def test_selection_bf16_64k_every_unit(torch_cuda):
    """The bf16 selection forward at the 64k workload's full size, every unit."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = CONFIGS["64k"]
    _say(f"case {cfg} bf16 (every unit)")
    q, k, v, idx = make_inputs_bf16(cfg)
    O, L = sel_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), _dev(torch, idx), cfg.block_size)
    torch.cuda.synchronize()
    _every_unit(torch, q, k, v, idx, cfg.block_size, O, L, "bf16", chunks=8)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", [("64k", (512, 0), "fp16"), ("64k", (512, 0), "bf16"),
                                  ("16k", (8192, 0), "fp16")])
def test_window_every_unit(torch_cuda, case):
    """Every unit of the FlyDSL page's head layout (H=64, H_KV=8, D=128) with a
    512 window at sequence 65536, and with an 8192 window at 16384 (the window
    filling up over the first 8192 queries, then sliding)."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import window_attn_fwd
    size, window, dtype = case
    cfg = CONFIGS["64k"] if size == "64k" else CONFIGS["64k"].with_(M=16384, N=16384)
    _say(f"case {cfg} window {window} {dtype} (every unit)")
    q, k, v, _ = (make_inputs_bf16 if dtype == "bf16" else make_inputs)(cfg)
    O, L = window_attn_fwd(_dev(torch, q), _dev(torch, k), _dev(torch, v), *window)
    torch.cuda.synchronize()
    _every_unit(torch, q, k, v, None, 1, O, L, dtype, window=window, chunks=8)
