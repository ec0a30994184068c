"""Selection-attention backward on the GPU (C ABI -> HIP kernels) against the
fp64 CPU oracle's backward.

The GPU pass is fed the GPU forward's O and LSE, as in training.

Tolerance, per gradient element: |GPU - oracle| <= GRAD_TOL * mag + 1e-6,
where mag is the oracle's error scale of that element, the L2 norm over its
terms of |term| with dS taken as P (|dP| + sum_d |dO_d O_d|).  The kernels
round P and dS to fp16 for the products that consume them (unit roundoff
u = 2^-11) and form Delta from the forward's fp16 O, so each term carries a
relative error of at most a few u, with a random sign: the element's error is
then about u * mag.  Emulating exactly those roundings in fp64 on the CPU gives
max error / (u * mag) of 1.0 to 2.1 over the small cases below; the GPU adds
the forward's own rounding of O and fp32 accumulation (for 2^19 terms about
0.1 u).  GRAD_TOL = 8 u leaves a factor of about 3; a dropped term, a missing
1/sqrt(D), a wrong mask or a wrong row exceeds it by orders of magnitude.  The
floor covers fp16 subnormal steps of very small P and dS.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, make_grad_output, make_inputs, sample_units

pytestmark = pytest.mark.gpu

GRAD_TOL = 8 * 2.0 ** -11


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to_dev(torch, *arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in arrs]


def _overflow_word(torch, workspace):
    """The workspace's overflow flag (32-bit word at byte offset 4): nonzero
    when a capacity bound of the key-major pass was exceeded."""
    return int(workspace[4:8].cpu().numpy().view(np.int32)[0])


def _gpu_bwd(torch, q, k, v, idx, do, bs, workspace=None):
    from block_sparse_attention_sel_amd.binding import nsa_sel_bwd_workspace_size, sel_attn_bwd, sel_attn_fwd
    tq, tk, tv, ti, tdo = _to_dev(torch, q, k, v, idx, do)
    O, L = sel_attn_fwd(tq, tk, tv, ti, bs)
    if workspace is None:
        B, M, H, D = q.shape
        _, N, G, _ = k.shape
        workspace = torch.empty(nsa_sel_bwd_workspace_size(B, M, N, H, G, D, bs, idx.shape[3]),
                                dtype=torch.uint8, device="cuda")
    dq, dk, dv = sel_attn_bwd(tq, tk, tv, ti, O, L, tdo, bs, workspace=workspace)
    torch.cuda.synchronize()
    assert _overflow_word(torch, workspace) == 0, "a capacity bound of the key-major pass was exceeded"
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _close(name, got, ref, mag):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    worst = float((err / (2.0 ** -11 * mag + 1e-30)).max()) if ref.size else 0.0
    _say(f"  {name}: max err {err.max():.3e}  max err / (u * mag) {worst:.2f}")
    assert np.all(err <= GRAD_TOL * mag + 1e-6), name


def _full(torch, q, k, v, idx, do, bs):
    import oracle
    dq, dk, dv = _gpu_bwd(torch, q, k, v, idx, do, bs)
    rq, rk, rv, mq, mk, mv = oracle.bwd_full(q, k, v, idx, do, bs, mags=True)
    _close("dQ", dq, rq, mq)
    _close("dK", dk, rk, mk)
    _close("dV", dv, rv, mv)
    return dq, dk, dv, rq, rk, rv


SMALL = {
    # gs = 4, D = 64, bs = 32
    "tiny": CONFIGS["tiny"],
    # gs = 8, ragged tail block, B = 2
    "b2-ragged": Config("b2-ragged", B=2, M=300, N=300, H=16, G=2, D=128, block_size=64, T=5, seed=21),
    # gs = 3 (tiles of 30 rows), M < N, D = 64, bs = 32
    "gs3": Config("gs3", B=1, M=200, N=333, H=6, G=2, D=64, block_size=32, T=6, seed=22),
    # gs = 16, M > N (late queries see every key block)
    "m-gt-n": Config("m-gt-n", B=1, M=500, N=180, H=16, G=1, D=128, block_size=64, T=4, seed=23),
    # gs = 1 (32 queries per tile), geometric rows
    "gs1-geom": Config("gs1-geom", B=1, M=700, N=700, H=2, G=2, D=128, block_size=32, T=6, rule="geometric",
                       seed=24),
    # every causal block selected
    "dense": Config("dense", B=1, M=512, N=512, H=8, G=1, D=64, block_size=32, T=16, seed=25).dense(),
    # key blocks selected by more than qc = 512 queries: several items, partial sums
    "multi-item": Config("multi-item", B=1, M=2500, N=2500, H=16, G=1, D=128, block_size=64, T=8, seed=26),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_full(torch_cuda, name):
    cfg = SMALL[name]
    _say(f"case {cfg}")
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    _full(torch_cuda, q, k, v, idx, do, cfg.block_size)


def test_bwd_noisy_rows_and_empty_rows(torch_cuda):
    """Rows with padding, future, out-of-range and repeated entries, and rows
    with nothing counted: dQ = 0 there, and key blocks nobody selects get
    dK = dV = 0."""
    cfg = Config("noisy", B=2, M=260, N=260, H=8, G=2, D=128, block_size=32, T=7, seed=27)
    q, k, v, _ = make_inputs(cfg)
    do = make_grad_output(cfg)
    rng = np.random.default_rng(5)
    idx = rng.integers(-3, cfg.NB + 3, size=(cfg.B, cfg.M, cfg.G, cfg.T)).astype(np.int32)
    idx[:, 40:60] = -1                       # nothing counted
    idx[:, 100:110] = 9                      # block 9 starts at key 288: future for these queries
    idx[1, :, 1, :] = np.where(idx[1, :, 1, :] == 4, 0, idx[1, :, 1, :])   # block 4 of (1, 1) unselected
    dq, dk, dv, rq, rk, rv = _full(torch_cuda, q, k, v, idx, do, cfg.block_size)
    assert np.all(dq[:, 40:60] == 0.0) and np.all(dq[:, 100:110] == 0.0)
    assert np.all(dk[1, 128:160, 1] == 0.0) and np.all(dv[1, 128:160, 1] == 0.0)


def _kblock_units(idx, bs, b, g, t):
    M = idx.shape[1]
    m = np.arange(M)
    sel = (idx[b, :, g, :] == t).any(axis=1) & (t <= m // bs)
    ms = np.nonzero(sel)[0]
    return np.stack([np.full_like(ms, b), ms, np.full_like(ms, g)], axis=1).astype(np.int64)


def _sampled(torch, cfg, n_units, kblocks):
    import oracle
    _say(f"case {cfg}")
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    dq, dk, dv = _gpu_bwd(torch, q, k, v, idx, do, cfg.block_size)
    units = sample_units(cfg, n_units, tail=1)
    rq, _, _, mq, _, _ = oracle.bwd_units(q, k, v, idx, do, cfg.block_size, units, mags=True)
    gs = cfg.gs
    got_q = np.stack([dq[b, m, g * gs:(g + 1) * gs] for b, m, g in units])
    _close(f"dQ ({len(units)} units)", got_q, rq, mq)
    bs = cfg.block_size
    for (b, g, t) in kblocks:
        u = _kblock_units(idx, bs, b, g, t)
        _, rk, rv, _, mk, mv = oracle.bwd_units(q, k, v, idx, do, bs, u, np.array([[b, g, t]]), mags=True)
        n = min(bs, cfg.N - t * bs)
        _close(f"dK block (b={b}, g={g}, t={t}; {len(u)} queries)", dk[b, t * bs:t * bs + n, g], rk[0, :n],
               mk[0, :n])
        _close(f"dV block (b={b}, g={g}, t={t}; {len(u)} queries)", dv[b, t * bs:t * bs + n, g], rv[0, :n],
               mv[0, :n])


def test_bwd_8k_sampled(torch_cuda):
    cfg = CONFIGS["8k"]
    _sampled(torch_cuda, cfg, 600, [(0, 0, cfg.NB - 1), (0, 1, 64), (0, 0, 20), (0, 1, 3)])


def test_bwd_64k_sampled(torch_cuda):
    cfg = CONFIGS["64k"]
    _sampled(torch_cuda, cfg, 300, [(0, 7, cfg.NB - 1), (0, 3, 700), (0, 0, 300)])


def test_bwd_32k_bs32_sampled(torch_cuda):
    cfg = CONFIGS["32k-bs32"]
    _sampled(torch_cuda, cfg, 200, [(1, 3, cfg.NB - 1), (0, 1, 900)])


@pytest.mark.timeout(900)
def test_bwd_8k_every_element(torch_cuda):
    """dQ, dK and dV of the 8k workload (M = N = 8192, H = 32, G = 2, D = 128),
    every element against the oracle's whole-tensor backward."""
    cfg = CONFIGS["8k"]
    _say(f"case {cfg} (every element)")
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    _full(torch_cuda, q, k, v, idx, do, cfg.block_size)


@pytest.mark.timeout(900)
def test_bwd_64k_every_element(torch_cuda):
    """dQ, dK and dV of the 64k workload (M = N = 65536, H = 64, G = 8,
    D = 128, bs = 64, T = 16) at full size, every element against the
    oracle's whole-tensor backward (about 3 minutes of oracle time on 16
    host threads)."""
    cfg = CONFIGS["64k"]
    _say(f"case {cfg} (every element)")
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    _full(torch_cuda, q, k, v, idx, do, cfg.block_size)


def test_bwd_128k_local_sampled(torch_cuda):
    cfg = CONFIGS["128k-local"]
    _sampled(torch_cuda, cfg, 200, [(0, 5, cfg.NB - 1), (0, 2, 1000)])


def test_bwd_deterministic_and_workspace_contents_do_not_matter(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import nsa_sel_bwd_workspace_size
    cfg = SMALL["multi-item"]
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    a = _gpu_bwd(torch, q, k, v, idx, do, cfg.block_size)
    n = nsa_sel_bwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    b = _gpu_bwd(torch, q, k, v, idx, do, cfg.block_size, workspace=ws)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_errors(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    cfg = CONFIGS["tiny"]
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    tq, tk, tv, ti, tdo = _to_dev(torch, q, k, v, idx, do)
    O, L = binding.sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    n = binding.nsa_sel_bwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    args = lambda wsp, wsn, dkk=dk: (tq, tk, tv, ti, O, L, tdo, dq, dkk, dv, wsp, wsn, cfg.B, cfg.M, cfg.N, cfg.H,
                                     cfg.G, cfg.D, cfg.block_size, cfg.T)
    assert binding.nsa_sel_bwd_raw(*args(ws, n - 1)) == binding.NSA_SEL_ERR_WORKSPACE
    assert binding.nsa_sel_bwd_raw(*args(ws.data_ptr() + 16, n)) == binding.NSA_SEL_ERR_WORKSPACE
    assert binding.nsa_sel_bwd_raw(*args(ws, n, dkk=dv)) == binding.NSA_SEL_ERR_ALIAS
    assert binding.nsa_sel_bwd_raw(*args(tq, n)) == binding.NSA_SEL_ERR_ALIAS   # workspace over Q
    assert binding.nsa_sel_bwd_raw(*args(ws, n)) == binding.NSA_SEL_OK
    torch.cuda.synchronize()


def test_sel_attn_autograd_matches_the_entry_points(torch_cuda):
    """sel_attn as an autograd function: its forward is sel_attn_fwd, the
    gradients it hands to q, k and v are sel_attn_bwd's cast to fp16, and lse
    carries no gradient."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn, sel_attn_bwd, sel_attn_fwd
    cfg = SMALL["b2-ragged"]
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    tq, tk, tv, ti, tdo = _to_dev(torch, q, k, v, idx, do)
    lq, lk, lv = (t.clone().requires_grad_(True) for t in (tq, tk, tv))
    out, lse = sel_attn(lq, lk, lv, ti, cfg.block_size)
    assert not lse.requires_grad and out.requires_grad
    out.backward(tdo)
    torch.cuda.synchronize()
    o_ref, l_ref = sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    dq, dk, dv = sel_attn_bwd(tq, tk, tv, ti, o_ref, l_ref, tdo, cfg.block_size)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o_ref) and torch.equal(lse, l_ref)
    assert lq.grad.dtype == torch.float16
    assert torch.equal(lq.grad, dq.half()) and torch.equal(lk.grad, dk.half()) and torch.equal(lv.grad, dv.half())


def test_sel_attn_autograd_rejects_bf16_backward(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import sel_attn
    cfg = SMALL["tiny"]
    q, k, v, idx = make_inputs(cfg)
    tq, tk, tv = (torch.from_numpy(a).to("cuda").to(torch.bfloat16).requires_grad_(True) for a in (q, k, v))
    ti = torch.from_numpy(idx).to("cuda")
    out, _ = sel_attn(tq, tk, tv, ti, cfg.block_size)
    with pytest.raises(NotImplementedError):
        out.float().sum().backward()


def test_forward_and_backward_replay_in_a_hip_graph(torch_cuda):
    """nsa_sel_fwd (64 dispatches per call) and nsa_sel_bwd captured into one
    HIP graph with preallocated outputs and workspace: every replay, with
    eager work in between, is bitwise the eager result (the library issues
    kernel launches only: no memset, allocation or synchronisation)."""
    torch = torch_cuda
    from block_sparse_attention_sel_amd import binding
    cfg = CONFIGS["8k"].with_(M=2048, N=2048)
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    tq, tk, tv, ti, tdo = _to_dev(torch, q, k, v, idx, do)
    B, M, N, H, G, D, bs, T = cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T
    ws = torch.empty(binding.nsa_sel_bwd_workspace_size(B, M, N, H, G, D, bs, T), dtype=torch.uint8, device="cuda")
    o_e, l_e = binding.sel_attn_fwd(tq, tk, tv, ti, bs)
    dq_e, dk_e, dv_e = binding.sel_attn_bwd(tq, tk, tv, ti, o_e, l_e, tdo, bs, workspace=ws)
    torch.cuda.synchronize()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    dq, dk, dv = torch.empty_like(dq_e), torch.empty_like(dk_e), torch.empty_like(dv_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call on a side stream before capture
        binding.nsa_sel_fwd(tq, tk, tv, ti, o, lse, B, M, N, H, G, D, bs, T, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = torch.cuda.current_stream().cuda_stream
        binding.nsa_sel_fwd(tq, tk, tv, ti, o, lse, B, M, N, H, G, D, bs, T, st)
        binding.nsa_sel_bwd(tq, tk, tv, ti, o, lse, tdo, dq, dk, dv, ws, ws.numel(), B, M, N, H, G, D, bs, T, st)
    for replay in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        ws.fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        _say(f"  replay {replay}")
        assert torch.equal(o, o_e) and torch.equal(lse, l_e)
        assert torch.equal(dq, dq_e) and torch.equal(dk, dk_e) and torch.equal(dv, dv_e)
        assert _overflow_word(torch, ws) == 0
