"""The workspace forward (nsa_sel_fwd_ws: one persistent dispatch whose XCDs
claim generations of wavefront slots from a schedule in the workspace) against
the fp64 CPU oracle and, bitwise, against nsa_sel_fwd (one dispatch per
generation), through the C ABI.

The persistent dispatch runs where one (b, g)'s K and V exceed one XCD's L2
(N * D * 4 bytes above 4 MiB on MI355X), so the small shapes here pair a long
key range with a short query range: every kernel instantiation (block size,
head dim, queries per tile, tiles per wavefront, cursor merge) takes the
schedule at a size the oracle finishes quickly.  The five workloads at full
size take it with many generations per XCD, where XCDs take generations over
from each other.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, make_inputs

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


def _dev(torch, *arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in arrs]


def _both(torch, tq, tk, tv, ti, cfg, fill=None):
    """(O, LSE) of nsa_sel_fwd_ws and of nsa_sel_fwd on the same inputs."""
    from block_sparse_attention_sel_amd import binding
    B, M, N, H, G, D, bs, T = cfg
    n = binding.nsa_sel_fwd_workspace_size(B, M, N, H, G, D, bs, T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    if fill is not None:
        ws.fill_(fill)
    O1 = torch.full((B, M, H, D), 7.0, dtype=torch.float16, device="cuda")
    L1 = torch.full((B, H, M), 7.0, dtype=torch.float32, device="cuda")
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    binding.nsa_sel_fwd_ws(tq, tk, tv, ti, O1, L1, B, M, N, H, G, D, bs, T, ws, n)
    binding.nsa_sel_fwd(tq, tk, tv, ti, O2, L2, B, M, N, H, G, D, bs, T)
    torch.cuda.synchronize()
    return (O1, L1), (O2, L2), ws


PERSIST_SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 700, 9000, 16, 2, 128, 64, 8),     # gs = 8: 2 queries per tile
    (2, 513, 17000, 8, 8, 64, 32, 16),     # gs = 1: 4 queries per tile, D = 64, bs = 32
    (1, 640, 8300, 32, 2, 128, 32, 70),    # gs = 16, T > 64: rows merged through cursors
    (1, 1000, 9001, 40, 8, 128, 64, 8),    # gs = 5: padding columns; ragged last block
    (1, 300, 16500, 12, 1, 64, 64, 4),     # gs = 12: 1 query per tile
    (1, 2048, 8200, 16, 8, 64, 64, 8),     # N * D * 4 below 4 MiB: nsa_sel_fwd's launches
]


def _rows(rng, B, M, G, T, bs, NB):
    """Counted entries (distinct, causal) mixed with -1 padding, a future block and
    an out-of-range one, in any order."""
    idx = np.full((B, M, G, T), -1, np.int32)
    for b in range(B):
        for m in range(M):
            c = m // bs
            for g in range(G):
                cand = rng.permutation(np.arange(0, min(c, NB - 1) + 1))
                row = list(cand[: max(1, T - 3)]) + [c + 1, NB + 3]
                row = (row + [-1] * T)[:T]
                rng.shuffle(row)
                idx[b, m, g] = row
    return idx


@pytest.mark.parametrize("shape", PERSIST_SHAPES)
def test_workspace_forward_every_instantiation(torch_cuda, shape):
    import oracle
    torch = torch_cuda
    B, M, N, H, G, D, bs, T = shape
    _say(f"case shape={shape}")
    rng = np.random.default_rng(sum(shape))
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    idx = _rows(rng, B, M, G, T, bs, -(-N // bs))
    (O1, L1), (O2, L2), _ = _both(torch, *_dev(torch, q, k, v, idx), shape)
    assert torch.equal(O1, O2) and torch.equal(L1, L2), "workspace call differs from nsa_sel_fwd"
    Or, Lr = oracle.oracle_full(q, k, v, idx, bs)
    O = O1.cpu().numpy().astype(np.float64)
    L = L1.cpu().numpy()
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty)
    errO = np.abs(O - Or).max()
    errL = np.abs(L[~empty] - Lr[~empty]).max() if (~empty).any() else 0.0
    _say(f"  max|dO| = {errO:.3e}  max|dLSE| = {errL:.3e}")
    assert errO <= O_TOL and errL <= LSE_TOL


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_forward_matches_generation_launches(torch_cuda, name):
    # Full size: many generations per XCD range, taken over across XCDs.
    # (The every-unit parity tests run this same call through sel_attn_fwd.)
    torch = torch_cuda
    cfg = CONFIGS[name]
    _say(f"case {cfg}")
    tq, tk, tv, ti = _dev(torch, *make_inputs(cfg))
    shape = (cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    (O1, L1), (O2, L2), _ = _both(torch, tq, tk, tv, ti, shape)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_workspace_contents_on_entry_do_not_matter(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    cfg = CONFIGS["32k-bs32"].with_(B=1, M=8192, N=16384)
    _say(f"case {cfg}")
    tq, tk, tv, ti = _dev(torch, *make_inputs(cfg))
    shape = (cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    (O1, L1), (O2, L2), ws = _both(torch, tq, tk, tv, ti, shape, fill=0xA5)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    # The same workspace again, as the last call left it, and once more with
    # every word at the largest value.
    for fill in (None, 0xFF):
        if fill is not None:
            ws.fill_(fill)
        O3, L3 = torch.empty_like(O1), torch.empty_like(L1)
        binding.nsa_sel_fwd_ws(tq, tk, tv, ti, O3, L3, *shape, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.equal(O3, O1) and torch.equal(L3, L1)


def test_concurrent_calls_with_their_own_workspaces(torch_cuda):
    # Two persistent dispatches on two streams share the GPU, so neither has
    # all its workgroups resident at once: their schedule waits run out and
    # the workgroups claim steps themselves.  Results must not change.
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    cfgs = [CONFIGS["64k"].with_(M=16384, N=16384), CONFIGS["128k-local"].with_(M=16384, N=16384)]
    runs = []
    for cfg in cfgs:
        tq, tk, tv, ti = _dev(torch, *make_inputs(cfg))
        shape = (cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
        (O1, L1), _, ws = _both(torch, tq, tk, tv, ti, shape)
        runs.append((tq, tk, tv, ti, shape, O1, L1, ws))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        for (tq, tk, tv, ti, shape, O1, L1, ws), st in zip(runs, streams):
            O = torch.empty_like(O1)
            L = torch.empty_like(L1)
            binding.nsa_sel_fwd_ws(tq, tk, tv, ti, O, L, *shape, ws, ws.numel(), st.cuda_stream)
            outs.append((O, L, O1, L1))
    torch.cuda.synchronize()
    for O, L, O1, L1 in outs:
        assert torch.equal(O, O1) and torch.equal(L, L1)


def test_workspace_forward_replays_in_a_hip_graph(torch_cuda):
    # The clearing kernel and the persistent dispatch, captured once and
    # replayed with eager work in between (no memset node is recorded).
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = CONFIGS["64k"].with_(M=8192, N=16384)
    tq, tk, tv, ti = _dev(torch, *make_inputs(cfg))
    ref_O, ref_L = sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    from block_sparse_attention_sel_amd import binding
    n = binding.nsa_sel_fwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    O = torch.empty_like(ref_O)
    L = torch.empty_like(ref_L)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sel_attn_fwd(tq, tk, tv, ti, cfg.block_size, out=O, lse=L, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sel_attn_fwd(tq, tk, tv, ti, cfg.block_size, out=O, lse=L, workspace=ws)
    for rep in range(3):
        O.fill_(3.0)
        L.fill_(3.0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, ref_O) and torch.equal(L, ref_L), f"replay {rep}"


def test_probe_with_a_workspace_stages_the_same_blocks(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    cfg = CONFIGS["32k-bs32"]
    tq, tk, tv, ti = _dev(torch, *make_inputs(cfg))
    n = binding.nsa_sel_fwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    counts = []
    for w in (None, ws):
        staged = torch.zeros(1, dtype=torch.int64, device="cuda")
        binding.nsa_gather_probe(tk, tv, ti, staged, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size,
                                 cfg.T, 0, w, 0 if w is None else w.numel())
        torch.cuda.synchronize()
        counts.append(int(staged.item()))
    assert counts[0] == counts[1] > 0
