"""GPU path (C ABI -> HIP kernels) against the fp64 CPU oracle.

Tolerances: O max-abs 5e-3, LSE max-abs 1e-3; rows with nothing visible must
give O = 0 and LSE = -inf exactly; no NaN or Inf elsewhere.
"""

import math
import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, Config, block_indices, make_inputs, sample_units

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


def _to_dev(torch, *arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in arrs]


def _gpu_run(torch, q, k, v, idx, bs):
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    tq, tk, tv, ti = _to_dev(torch, q, k, v, idx)
    O, L = sel_attn_fwd(tq, tk, tv, ti, bs)
    torch.cuda.synchronize()
    return O, L


def _check_full(O, L, Or, Lr):
    O = O.astype(np.float64)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty)
    assert np.all(L[empty] == -np.inf)
    errO = np.abs(O - Or).max()
    errL = np.abs(L[~empty] - Lr[~empty]).max() if (~empty).any() else 0.0
    _say(f"  max|dO| = {errO:.3e}  max|dLSE| = {errL:.3e}")
    assert errO <= O_TOL
    assert errL <= LSE_TOL


def _parity_full(torch, cfg):
    import oracle
    _say(f"case {cfg}")
    q, k, v, idx = make_inputs(cfg)
    O, L = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    Or, Lr = oracle.oracle_full(q, k, v, idx, cfg.block_size)
    _check_full(O.cpu().numpy(), L.cpu().numpy(), Or, Lr)


REDUCED = {
    "tiny": CONFIGS["tiny"],
    "8k@2048": CONFIGS["8k"].with_(M=2048, N=2048),
    "64k@4096": CONFIGS["64k"].with_(M=4096, N=4096),
    "32k-bs32@2048": CONFIGS["32k-bs32"].with_(M=2048, N=2048),
    "128k-local@4096": CONFIGS["128k-local"].with_(M=4096, N=4096),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_parity_full_coverage(torch_cuda, name):
    _parity_full(torch_cuda, REDUCED[name])


def _parity_sampled(torch, cfg, count, tail=2):
    import oracle
    _say(f"case {cfg} (sampled {count})")
    q, k, v, idx = make_inputs(cfg)
    O, L = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    units = sample_units(cfg, count, tail=tail)
    Or, Lr = oracle.oracle_units(q, k, v, idx, cfg.block_size, units)
    ub = torch.from_numpy(units).to("cuda")
    gs = cfg.gs
    heads = ub[:, 2:3] * gs + torch.arange(gs, device="cuda")[None, :]        # [U, gs]
    Og = O[ub[:, 0:1], ub[:, 1:2], heads].float().cpu().numpy()              # [U, gs, D]
    Lg = L[ub[:, 0:1], heads, ub[:, 1:2]].cpu().numpy()                      # [U, gs]
    _check_full(Og, Lg, Or, Lr)
    # Properties that hold at any size: finite everywhere, since every row of
    # the index rules selects the query's own block.
    assert torch.isfinite(L).all().item()
    assert torch.isfinite(O).all().item()


def _oracle_threads() -> int:
    import os
    n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n))))


def parity_every_unit(torch, cfg, launch=None, chunks: int = 8):
    """Runs the forward once at the config's full size, in the launch
    configuration the bench times, and compares every (b, m, g) unit with the
    oracle, streamed in unit ranges (no fp64 copy of the outputs is kept)."""
    import time

    import oracle
    _say(f"case {cfg} (every unit)")
    q, k, v, idx = make_inputs(cfg)
    O, L = _gpu_run(torch, q, k, v, idx, cfg.block_size) if launch is None else launch(q, k, v, idx)
    On = O.cpu().numpy()
    Ln = L.cpu().numpy()
    del O, L
    U = cfg.B * cfg.M * cfg.G
    worst_o = worst_l = 0.0
    t0 = time.perf_counter()
    for i in range(chunks):
        u0, u1 = U * i // chunks, U * (i + 1) // chunks
        r = oracle.compare(q, k, v, idx, cfg.block_size, On, Ln, u0, u1, _oracle_threads())
        worst_o = max(worst_o, r["max_err_O"])
        worst_l = max(worst_l, r["max_err_LSE"])
        _say(f"  units {u0}..{u1 - 1}: max|dO| = {r['max_err_O']:.3e} (unit {r['worst_unit_O']})  "
             f"max|dLSE| = {r['max_err_LSE']:.3e} (unit {r['worst_unit_LSE']})  bad rows {r['bad_rows']}  "
             f"{time.perf_counter() - t0:.1f} s")
        assert r["units"] == u1 - u0
        assert r["bad_rows"] == 0 and r["empty_rows"] == 0 and r["dup_units"] == 0
        assert r["max_err_O"] <= O_TOL and r["max_err_LSE"] <= LSE_TOL
    return worst_o, worst_l


# Every unit of each of the five workloads at full size (wave issue, section
# Algorithm: the computation is defined for every query position m).
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(CONFIGS))
def test_parity_full_size_every_unit(torch_cuda, name):
    parity_every_unit(torch_cuda, CONFIGS[name])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["8k", "64k"])
def test_parity_dense_mode_sampled(torch_cuda, name):
    # Every causal block selected (T = NB): the first two and the last query
    # block of every group (the longest rows) plus random units.
    _parity_sampled(torch_cuda, CONFIGS[name].dense(), 512, tail=2 if name == "8k" else 1)


KERNEL_SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 300, 300, 4, 4, 64, 32, 5),      # gs = 1, ragged tail
    (2, 257, 257, 6, 2, 64, 64, 3),      # gs = 3
    (1, 200, 333, 16, 1, 128, 32, 7),    # M < N, gs = 16
    (1, 511, 511, 10, 5, 128, 64, 4),    # gs = 2
    (2, 129, 129, 16, 2, 128, 64, 70),   # T > 64: several index chunks
    (1, 96, 96, 12, 1, 64, 32, 2),       # gs = 12
]


def _random_rows(rng, B, M, G, T, bs, NB):
    """Distinct counted entries mixed with padding, future and out-of-range ones."""
    idx = np.full((B, M, G, T), -1, np.int32)
    for b in range(B):
        for m in range(M):
            c = m // bs
            for g in range(G):
                cand = rng.permutation(np.arange(0, min(c, NB - 1) + 1))
                take = list(cand[: max(1, T - 2)])
                extra = [-1, NB + 5, c + 1 if c + 1 < NB else -3, -100]
                row = (take + extra)[:T]
                row = row + [-1] * (T - len(row))
                rng.shuffle(row)                # counted entries land anywhere in the row
                idx[b, m, g] = row
    return idx


@pytest.mark.parametrize("shape", KERNEL_SHAPES)
def test_parity_every_instantiation(torch_cuda, shape):
    import oracle
    B, M, N, H, G, D, bs, T = shape
    _say(f"case shape={shape}")
    rng = np.random.default_rng(sum(shape))
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    idx = _random_rows(rng, B, M, G, T, bs, -(-N // bs))
    O, L = _gpu_run(torch_cuda, q, k, v, idx, bs)
    Or, Lr = oracle.oracle_full(q, k, v, idx, bs)
    _check_full(O.cpu().numpy(), L.cpu().numpy(), Or, Lr)


# Shapes large enough that the library picks its two-tile wavefronts (the
# grid-size rule only drops to one tile for small problems), covering each
# queries-per-tile packing (1, 2, 4), both block sizes and both head dims.
TWO_TILE_SHAPES = [
    # B, M, N, H, G, D, bs, T
    (1, 4096, 4096, 16, 8, 64, 64, 8),      # gs = 2 -> 4 queries per tile
    (2, 2048, 2048, 8, 8, 64, 32, 16),      # gs = 1 -> 4 queries per tile
    (1, 4096, 4096, 32, 2, 64, 64, 8),      # gs = 16 -> 1 query per tile
    (1, 4096, 4096, 40, 8, 128, 64, 8),     # gs = 5 -> 2 queries per tile, 6 padding columns
    (1, 4096, 4096, 48, 8, 128, 32, 12),    # gs = 6, bs = 32
    (1, 4000, 4000, 16, 8, 128, 64, 8),     # ragged last block (N % bs = 32)
    (1, 3000, 4030, 16, 8, 64, 32, 8),      # M < N, ragged last block
]


def _noisy_rows(cfg, rng):
    """The uniform rule's rows, shuffled, with padding, future and
    out-of-range entries in place of some of the -1 slots."""
    idx = block_indices(cfg).copy()
    B, M, G, T = idx.shape
    c = (np.arange(M) // cfg.block_size)[None, :, None, None]
    junk = np.stack([np.full_like(idx, -3), np.broadcast_to(c + 1, idx.shape), np.full_like(idx, cfg.NB + 2)])
    pick = rng.integers(0, 3, size=idx.shape)
    filler = np.take_along_axis(junk, pick[None], axis=0)[0]
    idx = np.where((idx < 0) & (rng.random(idx.shape) < 0.7), filler, idx)
    perm = np.argsort(rng.random(idx.shape), axis=-1)
    return np.ascontiguousarray(np.take_along_axis(idx, perm, axis=-1)).astype(np.int32)


@pytest.mark.parametrize("shape", TWO_TILE_SHAPES)
def test_parity_two_tile_wavefronts(torch_cuda, shape):
    import oracle
    B, M, N, H, G, D, bs, T = shape
    _say(f"case two-tile shape={shape}")
    cfg = Config("t", B=B, M=M, N=N, H=H, G=G, D=D, block_size=bs, T=T, seed=sum(shape))
    q, k, v, _ = make_inputs(cfg)
    idx = _noisy_rows(cfg, np.random.default_rng(sum(shape)))
    O, L = _gpu_run(torch_cuda, q, k, v, idx, bs)
    Or, Lr = oracle.oracle_full(q, k, v, idx, bs)
    _check_full(O.cpu().numpy(), L.cpu().numpy(), Or, Lr)


# At the same row length, padding and invalid entries change nothing, not even
# the rounding: the kernel's slot layout and block order depend only on T and
# the counted entries.  (64k@2048 at 2T = 32 runs two-tile wavefronts; 8k@2048
# at 2T = 32 runs paired wavefronts.)
@pytest.mark.parametrize("name", ["64k@2048", "8k@2048"])
def test_padding_and_invalid_entries_are_bitwise_invisible(torch_cuda, name):
    torch = torch_cuda
    base, size = name.split("@")
    cfg = CONFIGS[base].with_(M=int(size), N=int(size))
    _say(f"case sentinel-invariance {cfg}")
    q, k, v, idx = make_inputs(cfg)
    B, M, G, T = idx.shape
    NB = cfg.NB
    rng = np.random.default_rng(1)
    noisy = np.full((B, M, G, 2 * T), -1, np.int32)
    for m in range(M):
        c = m // cfg.block_size
        for g in range(G):
            row = [int(t) for t in idx[0, m, g] if t >= 0]
            junk = [-1, -5, NB, NB + 100] + ([c + 1 + int(rng.integers(0, NB - c - 1))] if c + 1 < NB else [])
            out = []
            for t in row:                       # keep counted order, sprinkle junk in between
                if rng.random() < 0.5:
                    out.append(junk[int(rng.integers(0, len(junk)))])
                out.append(t)
            noisy[0, m, g, : len(out)] = out[: 2 * T]
    clean = np.full((B, M, G, 2 * T), -1, np.int32)
    clean[..., :T] = idx
    O1, L1 = _gpu_run(torch, q, k, v, clean, cfg.block_size)
    O2, L2 = _gpu_run(torch, q, k, v, noisy, cfg.block_size)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


# Scores 16x larger than N(0,1) inputs give (a softmax peaked on a few keys,
# log2-domain scores spread over tens of units): P is only kept inside the
# fp16 range by a correct running max, so a wrong column reduction or lazy-max
# rule shows up here as inf/NaN or a large error, while the result itself
# does not depend on which max the kernel used.
@pytest.mark.parametrize("shape", [(1, 4096, 4096, 64, 8, 128, 64, 16), (1, 4096, 4096, 16, 8, 64, 64, 8),
                                   (1, 2048, 2048, 16, 1, 128, 32, 12)])
def test_large_scores(torch_cuda, shape):
    import oracle
    B, M, N, H, G, D, bs, T = shape
    _say(f"case large-scores shape={shape}")
    cfg = Config("s", B=B, M=M, N=N, H=H, G=G, D=D, block_size=bs, T=T, seed=sum(shape) + 7)
    q, k, v, idx = make_inputs(cfg)
    q = (q.astype(np.float32) * 16.0).astype(np.float16)
    O, L = _gpu_run(torch_cuda, q, k, v, idx, bs)
    Or, Lr = oracle.oracle_full(q, k, v, idx, bs)
    _check_full(O.cpu().numpy(), L.cpu().numpy(), Or, Lr)


def test_repeat_runs_are_bitwise_identical(torch_cuda):
    torch = torch_cuda
    cfg = CONFIGS["32k-bs32"].with_(M=2048, N=2048)
    _say(f"case determinism {cfg}")
    q, k, v, idx = make_inputs(cfg)
    O1, L1 = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    O2, L2 = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_outputs_stay_inside_their_buffers(torch_cuda):
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import nsa_sel_fwd
    cfg = CONFIGS["8k"].with_(M=1024, N=1024)
    _say(f"case guard-bands {cfg}")
    q, k, v, idx = make_inputs(cfg)
    tq, tk, tv, ti = _to_dev(torch, q, k, v, idx)
    pad = 4096
    o_buf = torch.full((q.size + 2 * pad,), 1234.0, dtype=torch.float16, device="cuda")
    l_buf = torch.full((cfg.B * cfg.H * cfg.M + 2 * pad,), -777.0, dtype=torch.float32, device="cuda")
    O = o_buf[pad:pad + q.size]
    L = l_buf[pad:pad + cfg.B * cfg.H * cfg.M]
    nsa_sel_fwd(tq, tk, tv, ti, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T,
                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(o_buf[:pad] == 1234.0) and torch.all(o_buf[-pad:] == 1234.0)
    assert torch.all(l_buf[:pad] == -777.0) and torch.all(l_buf[-pad:] == -777.0)
    assert torch.all(L != -777.0)


def test_rows_without_counted_entries(torch_cuda):
    torch = torch_cuda
    B, M, N, H, G, D, bs, T = 1, 130, 130, 8, 2, 128, 64, 3
    rng = np.random.default_rng(4)
    q = rng.standard_normal((B, M, H, D)).astype(np.float16)
    k = rng.standard_normal((B, N, G, D)).astype(np.float16)
    v = rng.standard_normal((B, N, G, D)).astype(np.float16)
    idx = np.full((B, M, G, T), -1, np.int32)
    idx[0, ::2, :, 0] = 0                               # even rows see block 0
    odd = np.arange(1, M, 2)
    idx[0, odd, :, 1] = (odd // bs + 1)[:, None]        # a future (or past-the-end) block only
    O, L = _gpu_run(torch, q, k, v, idx, bs)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    assert np.all(L[0][:, 1::2] == -np.inf)
    assert not O[0, 1::2].any()
    assert np.isfinite(L[0][:, ::2]).all()


def test_single_visible_key_rows(torch_cuda):
    """m = 0 sees only key 0: O equals V[0] exactly (p = 1, l = 1) and LSE is
    the scaled score."""
    torch = torch_cuda
    cfg = CONFIGS["64k"].with_(M=512, N=512)
    q, k, v, idx = make_inputs(cfg)
    O, L = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    for h in range(cfg.H):
        g = h // cfg.gs
        assert np.array_equal(O[0, 0, h], v[0, 0, g])
        s = math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, h], k[0, 0, g])) / math.sqrt(cfg.D)
        assert abs(L[0, h, 0] - s) <= LSE_TOL


def test_non_default_stream(torch_cuda):
    torch = torch_cuda
    import oracle
    from block_sparse_attention_sel_amd.binding import sel_attn_fwd
    cfg = CONFIGS["tiny"].with_(M=512, N=512)
    q, k, v, idx = make_inputs(cfg)
    tq, tk, tv, ti = _to_dev(torch, q, k, v, idx)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        O, L = sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    s.synchronize()
    Or, Lr = oracle.oracle_full(q, k, v, idx, cfg.block_size)
    _check_full(O.cpu().numpy(), L.cpu().numpy(), Or, Lr)


def _with_repeats(idx, rng, frac=0.5):
    """Rows whose padding slots are partly filled with copies of the row's own
    counted entries, then shuffled; returns (rows with repeats, the same rows
    with those copies as -1 in the same positions)."""
    rep = idx.copy()
    B, M, G, T = idx.shape
    clean = idx.copy()
    flat_r = rep.reshape(-1, T)
    flat_c = clean.reshape(-1, T)
    for i in range(flat_r.shape[0]):
        row = flat_r[i]
        valid = row[row >= 0]
        pads = np.nonzero(row < 0)[0]
        if valid.size == 0 or pads.size == 0:
            continue
        take = pads[rng.random(pads.size) < frac]
        row[take] = rng.choice(valid, take.size)
        perm = rng.permutation(T)
        flat_r[i] = row[perm]
        crow = flat_c[i].copy()
        crow[take] = -1
        flat_c[i] = crow[perm]
    return np.ascontiguousarray(rep), np.ascontiguousarray(clean)


# Repeated entries count once (the union), on the register merger (T <= 64
# here) and on the block map (pack * T > 128): parity with the oracle, and
# bitwise equality with the same rows without the copies at the same T.
@pytest.mark.parametrize("shape", [
    (1, 4096, 4096, 64, 8, 128, 64, 16),    # register merger, two tiles
    (1, 2048, 2048, 16, 1, 64, 32, 40),     # gs = 16, one query per tile: register merger, 80 entries
    (2, 1024, 1024, 16, 2, 128, 32, 80),    # gs = 8, pack 2: 160 entries -> block map
    (1, 1500, 1500, 8, 2, 64, 32, 48),      # gs = 4, pack 4: 192 entries -> block map
])
def test_repeated_entries_are_bitwise_the_union(torch_cuda, shape):
    import oracle
    torch = torch_cuda
    B, M, N, H, G, D, bs, T = shape
    _say(f"case repeats shape={shape}")
    cfg = Config("r", B=B, M=M, N=N, H=H, G=G, D=D, block_size=bs, T=T, seed=sum(shape) + 3)
    q, k, v, idx = make_inputs(cfg)
    rep, clean = _with_repeats(idx, np.random.default_rng(sum(shape)))
    assert (rep != clean).any()
    O1, L1 = _gpu_run(torch, q, k, v, rep, bs)
    O2, L2 = _gpu_run(torch, q, k, v, clean, bs)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    Or, Lr = oracle.oracle_full(q, k, v, rep, bs)
    assert oracle.oracle_units.last_dup_units > 0
    _check_full(O1.cpu().numpy(), L1.cpu().numpy(), Or, Lr)


# The block map covers 2048 blocks at a time: queries whose causal range
# reaches past block 2048 build a second window.  Shuffled rows put counted
# entries of both windows anywhere in the row; units of the last query blocks
# (the second window) are compared with the oracle.
def test_block_map_windows(torch_cuda):
    import oracle
    torch = torch_cuda
    cfg = Config("w", B=1, M=66560, N=66560, H=8, G=1, D=64, block_size=32, T=72, seed=31)
    _say(f"case block-map windows {cfg}")
    q, k, v, idx = make_inputs(cfg)
    rng = np.random.default_rng(31)
    tail = slice(cfg.M - 3 * cfg.block_size, cfg.M)
    rows = idx[0, tail, 0].copy()
    for i in range(rows.shape[0]):        # some entries in the second window, shuffled rows
        c = (cfg.M - 3 * cfg.block_size + i) // cfg.block_size
        free = np.nonzero(rows[i] < 0)[0]
        extra = rng.choice(np.arange(2048, c), min(free.size, 6), replace=False)
        rows[i, free[:extra.size]] = extra
        rows[i] = rows[i][rng.permutation(cfg.T)]
    idx = idx.copy()
    idx[0, tail, 0] = rows
    O, L = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    units = sample_units(cfg, 1024, tail=3)
    Or, Lr = oracle.oracle_units(q, k, v, idx, cfg.block_size, units)
    ub = torch.from_numpy(units).to("cuda")
    heads = ub[:, 2:3] * cfg.gs + torch.arange(cfg.gs, device="cuda")[None, :]
    Og = O[ub[:, 0:1], ub[:, 1:2], heads].float().cpu().numpy()
    Lg = L[ub[:, 0:1], heads, ub[:, 1:2]].cpu().numpy()
    _check_full(Og, Lg, Or, Lr)


# Race check: the unpipelined build (no copy in flight while LDS is read)
# runs the same arithmetic in the same order, so any difference from the
# pipelined kernel is a copy that overwrote LDS still being read.
@pytest.mark.parametrize("name", ["64k@4096", "32k-bs32@2048", "8k-dense@2048", "tiny"])
def test_pipelined_matches_unpipelined_bitwise(torch_cuda, name):
    torch = torch_cuda
    from block_sparse_attention_sel_amd.binding import nsa_sel_fwd_unpipelined
    base, _, size = name.partition("@")
    if base == "8k-dense":
        cfg = CONFIGS["8k"].with_(M=int(size), N=int(size)).dense()
    elif size:
        cfg = CONFIGS[base].with_(M=int(size), N=int(size))
    else:
        cfg = CONFIGS[base]
    _say(f"case unpipelined {cfg}")
    q, k, v, idx = make_inputs(cfg)
    O1, L1 = _gpu_run(torch, q, k, v, idx, cfg.block_size)
    tq, tk, tv, ti = _to_dev(torch, q, k, v, idx)
    O2 = torch.full_like(O1, float("nan"))
    L2 = torch.full_like(L1, float("nan"))
    nsa_sel_fwd_unpipelined(tq, tk, tv, ti, O2, L2, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size,
                            cfg.T, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
