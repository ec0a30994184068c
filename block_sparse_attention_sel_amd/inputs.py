"""Seeded synthetic inputs for NSA selection attention (host side, numpy only).

This module is the one piece shared by the GPU path's tests/bench and the CPU
oracle's tests.  It draws random numbers and builds block-index rows; it holds
none of the attention arithmetic.

Tensors follow the layouts of the operation's signature in the wave issue
"[wave] NSA: selection attention forward kernel" (section Operation):
Q [B, M, H, D], K [B, N, G, D], V [B, N, G, D] in fp16, block_indices
[B, M, G, T] (int32 here; the page gives no dtype).

Random values: every tensor is drawn from numpy's Philox-4x64 counter-based
generator.  A tensor is cut into fixed chunks of ``CHUNK`` elements; chunk i of
stream s under seed k uses the Philox key (k, s * 2**32 + i), so the bytes do
not depend on how many threads fill the chunks.  Values are N(0, 1) drawn in
float32 and rounded to fp16 (round-to-nearest-even).

Index rules (the selection that the top-k kernel of the NSA suite would
produce is replaced by these seeded rules):

* ``uniform``: every row holds block 0 and the query's own block
  c = floor(m / bs); the other min(T - 2, c - 1) entries are a uniform draw
  without replacement from blocks 1 .. c-1 (Floyd's sampling algorithm); the row
  is sorted ascending and padded with -1 to T entries.
* ``geometric``: as ``uniform`` but the other entries are c - d with
  d ~ Geometric(p) on {1, 2, ...}; draws that fall at or below 0 or repeat an
  earlier pick are rejected until min(T - 2, c - 1) distinct blocks are held.
* ``dense``: T = ceil(N / bs) and the row is [0, 1, ..., c, -1, ...]: every
  causal block is selected.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

# Stream ids inside one seed.
STREAM_Q, STREAM_K, STREAM_V, STREAM_IDX, STREAM_DO, STREAM_SCORES = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    M: int
    N: int
    H: int
    G: int
    D: int
    block_size: int
    T: int
    rule: str = "uniform"
    seed: int = 0
    geom_p: float = 0.1

    @property
    def gs(self) -> int:
        return self.H // self.G

    @property
    def NB(self) -> int:
        return -(-self.N // self.block_size)

    def dense(self) -> "Config":
        """Same shape with every causal block selected (T = number of KV blocks)."""
        return dataclasses.replace(self, name=self.name + "-dense", T=self.NB, rule="dense")

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads: sizes, index rules and seeds.
CONFIGS = {
    "tiny": Config("tiny", B=1, M=1024, N=1024, H=4, G=1, D=64, block_size=32, T=4, seed=0),
    "8k": Config("8k", B=1, M=8192, N=8192, H=32, G=2, D=128, block_size=64, T=16, seed=1),
    "64k": Config("64k", B=1, M=65536, N=65536, H=64, G=8, D=128, block_size=64, T=16, seed=2),
    "32k-bs32": Config("32k-bs32", B=2, M=32768, N=32768, H=64, G=4, D=128, block_size=32, T=32, seed=3),
    "128k-local": Config("128k-local", B=1, M=131072, N=131072, H=64, G=8, D=128, block_size=64, T=16,
                         rule="geometric", seed=4),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_fp16(shape, seed: int, stream: int, threads: int | None = None) -> np.ndarray:
    """fp16 array of the given shape, N(0,1), deterministic in (seed, stream)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    nchunks = -(-n // CHUNK)

    def fill(i):
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        key = np.array([seed, (stream << 32) + i], dtype=np.uint64)
        rng = np.random.Generator(np.random.Philox(key=key))
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)


def normal_bf16(shape, seed: int, stream: int, threads: int | None = None) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of the same N(0,1) float32 draws as
    normal_fp16(shape, seed, stream), rounded to bf16 instead of fp16."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = -(-n // CHUNK)

    def fill(i):
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        key = np.array([seed, (stream << 32) + i], dtype=np.uint64)
        rng = np.random.Generator(np.random.Philox(key=key))
        out[lo:hi] = to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _rng(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    key = np.array([seed, (stream << 32) + sub], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _floyd_sample(rng: np.random.Generator, n: np.ndarray, k: np.ndarray, kmax: int) -> np.ndarray:
    """For each row r, a uniform k[r]-subset of {0, ..., n[r]-1} (Floyd's algorithm).

    Returns int64 [R, kmax]; unused slots are -1.
    """
    R = n.shape[0]
    out = np.full((R, kmax), -1, dtype=np.int64)
    for i in range(kmax):
        act = i < k
        if not act.any():
            break
        rows = np.nonzero(act)[0]
        j = n[rows] - k[rows] + i            # Floyd: j runs n-k .. n-1
        r = rng.integers(0, j + 1)            # uniform in [0, j]
        taken = (out[rows, :i] == r[:, None]).any(axis=1)
        out[rows, i] = np.where(taken, j, r)
    return out


def _rows_uniform(c: np.ndarray, T: int, rng: np.random.Generator) -> np.ndarray:
    R = c.shape[0]
    kmax = max(T - 2, 0)
    n = np.maximum(c - 1, 0)                  # candidates 1 .. c-1
    k = np.minimum(kmax, n)
    picks = _floyd_sample(rng, n, k, kmax) + 1 if kmax > 0 else np.zeros((R, 0), np.int64)
    picks[picks == 0] = -1                    # unused slots (-1 + 1) back to -1
    return _assemble(c, picks, T)


def _rows_geometric(c: np.ndarray, T: int, rng: np.random.Generator, p: float) -> np.ndarray:
    R = c.shape[0]
    kmax = max(T - 2, 0)
    picks = np.full((R, kmax), -1, dtype=np.int64)
    need = np.minimum(kmax, np.maximum(c - 1, 0))
    # Rows whose whole candidate range fits take every block 1 .. c-1.
    full = (c - 1) <= kmax
    if full.any():
        cols = np.arange(kmax)
        fr = np.nonzero(full)[0]
        vals = cols[None, :] + 1
        picks[fr] = np.where(vals <= (c[fr] - 1)[:, None], vals, -1)
    count = np.where(full, need, 0)
    active = np.nonzero(count < need)[0]
    while active.size:
        d = rng.geometric(p, size=active.size)
        cand = c[active] - d
        ok = cand >= 1
        dup = (picks[active] == cand[:, None]).any(axis=1)
        ok &= ~dup
        rows = active[ok]
        picks[rows, count[rows]] = cand[ok]
        count[rows] += 1
        active = active[count[active] < need[active]]
    return _assemble(c, picks, T)


def _assemble(c: np.ndarray, picks: np.ndarray, T: int) -> np.ndarray:
    """Rows {0, c} plus picks, sorted ascending, padded with -1 at the end."""
    R = c.shape[0]
    rows = np.full((R, T), -1, dtype=np.int64)
    first = np.zeros(R, dtype=np.int64)
    cur = np.where(c > 0, c, -1)              # block 0 is the current block when c == 0
    body = np.concatenate([first[:, None], cur[:, None], picks], axis=1)[:, :T] if T >= 2 else first[:, None]
    big = np.iinfo(np.int64).max
    body = np.where(body < 0, big, body)
    body.sort(axis=1)
    body = np.where(body == big, -1, body)
    rows[:, : body.shape[1]] = body
    return rows


def block_indices(cfg: Config, threads: int | None = None) -> np.ndarray:
    """int32 [B, M, G, T] selection rows for the config's rule and seed."""
    B, M, G, T, bs = cfg.B, cfg.M, cfg.G, cfg.T, cfg.block_size
    if cfg.rule == "dense":
        c = np.arange(M, dtype=np.int64) // bs
        row = np.arange(T, dtype=np.int32)[None, :]
        one = np.where(row <= c[:, None], row, -1).astype(np.int32)          # [M, T]
        return np.ascontiguousarray(np.broadcast_to(one[None, :, None, :], (B, M, G, T)))
    out = np.empty((B, M, G, T), dtype=np.int32)
    # Work is cut into slabs of query positions; slab s draws from its own
    # Philox key, so the result does not depend on the thread count.
    slab = max(1, (1 << 16) // max(G, 1))
    jobs = [(b, lo) for b in range(B) for lo in range(0, M, slab)]

    def fill(job):
        b, lo = job
        hi = min(M, lo + slab)
        m = np.arange(lo, hi, dtype=np.int64)
        c = np.repeat(m // bs, G)
        rng = _rng(cfg.seed, STREAM_IDX, b * ((M + slab - 1) // slab) + lo // slab)
        if cfg.rule == "uniform":
            rows = _rows_uniform(c, T, rng)
        elif cfg.rule == "geometric":
            rows = _rows_geometric(c, T, rng, cfg.geom_p)
        else:
            raise ValueError(f"unknown index rule {cfg.rule!r}")
        out[b, lo:hi] = rows.reshape(hi - lo, G, T).astype(np.int32)

    if len(jobs) == 1:
        fill(jobs[0])
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, jobs))
    return out


def make_inputs(cfg: Config, threads: int | None = None):
    """(Q, K, V, block_indices) as contiguous numpy arrays for the config."""
    q = normal_fp16((cfg.B, cfg.M, cfg.H, cfg.D), cfg.seed, STREAM_Q, threads)
    k = normal_fp16((cfg.B, cfg.N, cfg.G, cfg.D), cfg.seed, STREAM_K, threads)
    v = normal_fp16((cfg.B, cfg.N, cfg.G, cfg.D), cfg.seed, STREAM_V, threads)
    idx = block_indices(cfg, threads)
    return q, k, v, idx


def make_inputs_bf16(cfg: Config, threads: int | None = None):
    """(Q, K, V, block_indices) with Q, K, V as bfloat16 bit patterns (uint16):
    the same draws and index rows as make_inputs, rounded to bf16."""
    q = normal_bf16((cfg.B, cfg.M, cfg.H, cfg.D), cfg.seed, STREAM_Q, threads)
    k = normal_bf16((cfg.B, cfg.N, cfg.G, cfg.D), cfg.seed, STREAM_K, threads)
    v = normal_bf16((cfg.B, cfg.N, cfg.G, cfg.D), cfg.seed, STREAM_V, threads)
    idx = block_indices(cfg, threads)
    return q, k, v, idx


def block_scores(cfg: Config, threads: int | None = None) -> np.ndarray:
    """Block importance scores for top-k selection, fp32 [B, M, G, NB], N(0, 1)
    (the same chunked Philox scheme as the other tensors, stream 6)."""
    shape = (cfg.B, cfg.M, cfg.G, cfg.NB)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = -(-n // CHUNK)

    def fill(i):
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        key = np.array([cfg.seed, (STREAM_SCORES << 32) + i], dtype=np.uint64)
        rng = np.random.Generator(np.random.Philox(key=key))
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def make_grad_output(cfg: Config, threads: int | None = None) -> np.ndarray:
    """Upstream gradient dO, fp16 [B, M, H, D], N(0, 1), for the backward pass."""
    return normal_fp16((cfg.B, cfg.M, cfg.H, cfg.D), cfg.seed, STREAM_DO, threads)


def sample_units(cfg: Config, count: int, seed: int = 12345, tail: int = 2) -> np.ndarray:
    """int64 [U, 3] (b, m, g) units: the first two and the last ``tail`` query
    blocks of every (b, g), plus ``count`` seeded random units, without repeats."""
    bs = cfg.block_size
    edge_m = np.unique(np.concatenate([
        np.arange(0, min(cfg.M, 2 * bs)),
        np.arange(max(0, cfg.M - tail * bs), cfg.M)]))
    b, m, g = np.meshgrid(np.arange(cfg.B), edge_m, np.arange(cfg.G), indexing="ij")
    edge = np.stack([b.ravel(), m.ravel(), g.ravel()], axis=1)
    rng = _rng(seed, 99)
    rnd = np.stack([rng.integers(0, cfg.B, count), rng.integers(0, cfg.M, count),
                    rng.integers(0, cfg.G, count)], axis=1)
    allu = np.concatenate([edge, rnd]).astype(np.int64)
    key = (allu[:, 0] * cfg.M + allu[:, 1]) * cfg.G + allu[:, 2]
    _, first = np.unique(key, return_index=True)
    return allu[np.sort(first)]
