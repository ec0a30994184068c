"""Benchmark of the NSA selection-attention forward (nsa_sel_fwd_ws) on one MI355X.

One step is one nsa_sel_fwd_ws call over the whole workload (all (b, m, g)
units of the config) with inputs and its workspace already resident in HBM;
the same forward queued as one dispatch per generation (nsa_sel_fwd, no
workspace) is timed beside it.  Prints ONE JSON
line: effective TFLOP/s as ``value``, plus ms per step, gathered-KV GB/s, the
roofline of the kernel (the larger of compulsory bytes at the HBM peak and
effective flops at the fp16 MFMA peak), cold-cache timings, the
gather-ceiling probe (the kernel's block-gather stream alone), the MFMA
utilisation, the same kernel with every causal block selected (dense mode),
the dense causal attention kernel on the same tensors (the reference point of
the speed-up goal), the backward pass (nsa_sel_bwd: dQ, dK, dV from the
forward's O and LSE) and the fp64 CPU oracle timed on a bounded sample of the
same workload.

Work counts per launch (exact, from the index rows):
  gathered bytes  = sum over units of (counted blocks) * bs * D * 2 B * 2 (K and V)
  effective flops = sum over units of 4 * D * (H/G) * (visible selected keys)
  backward flops  = sum over units of 10 * D * (H/G) * (visible selected keys)
                    (five products per (row, key): S, dP, dQ, dK, dV)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_attention_sel_amd.inputs import (CONFIGS, Config, block_indices, block_scores,  # noqa: E402
                                                   make_grad_output, make_inputs, make_inputs_bf16)

HBM_PEAK_GBPS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "nsa_sel_fwd_64k_hbm_counters.json")
# The forward kernel's sources: the counters in COUNTERS_FILE hold for this exact text.
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_sel_amd", "csrc", f)
               for f in ("nsa_sel.hip", "nsa_sel_common.h")]


def work_counts(cfg: Config, idx: np.ndarray):
    """(counted blocks, visible keys) summed over all units of one launch."""
    bs = cfg.block_size
    if cfg.rule == "dense":
        m = np.arange(cfg.M, dtype=np.int64)
        blocks = (np.minimum(m // bs, cfg.NB - 1) + 1).sum() * cfg.B * cfg.G
        keys = np.minimum(m + 1, cfg.N).sum() * cfg.B * cfg.G
        return int(blocks), int(keys)
    blocks = 0
    keys = 0
    step = max(1, (1 << 22) // (cfg.G * cfg.T))
    for b in range(cfg.B):
        for lo in range(0, cfg.M, step):
            hi = min(cfg.M, lo + step)
            t = idx[b, lo:hi].astype(np.int64)                          # [m, G, T]
            m = np.arange(lo, hi, dtype=np.int64)[:, None, None]
            c = m // bs
            ok = (t >= 0) & (t <= c) & (t < cfg.NB)
            vis = np.minimum(np.minimum((t + 1) * bs, cfg.N), m + 1) - t * bs
            blocks += int(ok.sum())
            keys += int(np.where(ok, np.maximum(vis, 0), 0).sum())
    return blocks, keys


def _kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def _counters():
    """The committed rocprofv3 counter summary of nsa_sel_fwd (HBM bytes per
    call, L2 hits), if it was taken on the current kernel source; else None."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256") != _kernel_sha():
        return None
    return rec


def compulsory_bytes(cfg: Config) -> int:
    """Bytes every launch must move at least once: Q and O [B,M,H,D] (2 B),
    K and V [B,N,G,D] (2 B), the index rows [B,M,G,T] (4 B), LSE [B,H,M] (4 B)."""
    q = cfg.B * cfg.M * cfg.H * cfg.D * 2
    kv = cfg.B * cfg.N * cfg.G * cfg.D * 2
    return 2 * q + 2 * kv + cfg.B * cfg.M * cfg.G * cfg.T * 4 + cfg.B * cfg.H * cfg.M * 4


def roofline(flops: float, compulsory: int, ms: float, traffic=None) -> dict:
    """The kernel against its binding roofline: the larger of compulsory bytes
    at the HBM peak and effective flops at the fp16 MFMA peak is the time a
    launch cannot beat; frac = that time / the measured time (= achieved /
    peak in the binding unit)."""
    t_hbm = compulsory / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (FP16_PEAK_TFLOPS * 1e12)
    s = ms * 1e-3
    if t_mfma >= t_hbm:
        return {"bound": "mfma", "achieved": round(flops / s / 1e12, 2), "peak": FP16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(t_mfma / s, 4), "traffic": traffic}
    return {"bound": "hbm", "achieved": round(compulsory / s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(t_hbm / s, 4), "traffic": traffic}


def _counter_sums(csv_path: str, counter: str):
    """Per-dispatch sums of one counter: {dispatch_id: (kernel_name, value)}."""
    import csv
    out = {}
    for row in csv.DictReader(open(csv_path)):
        if row["Counter_Name"] != counter:
            continue
        d = int(row["Dispatch_Id"])
        name, v = out.get(d, (row["Kernel_Name"], 0.0))
        out[d] = (name, v + float(row["Counter_Value"]))
    return out


def summarize_pmc(fetch_csv: str, write_csv: str, calls: int, copy_mib: int, out_path: str, l2_csv=None):
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-probe-mib N --steps S --warmup W --no-dense
    --no-cpu-baseline --no-graph` into HBM bytes per nsa_sel_fwd_ws call.  Each counter is
    scaled by what it reads for the plain N MiB device copy in the same run.
    l2_csv: an optional third run with TCC_HIT_sum and TCC_MISS_sum, giving the
    L2 hit rate of the forward's requests."""
    res = {"kernel_sha256": _kernel_sha(), "calls": calls, "copy_probe_mib": copy_mib}

    def forward(sums):
        # The dispatches of the timed forward calls: the persistent kernel and
        # its schedule clearing, or the generation kernels where the call
        # queues those.
        names = ("nsa_sel_fwd_persistent_kernel", "sched_clear_kernel")
        picked = [v for (n, v) in sums.values() if any(k in n for k in names)]
        return picked or [v for (n, v) in sums.values() if "nsa_sel_fwd_kernel" in n]

    if l2_csv:
        hit = sum(forward(_counter_sums(l2_csv, "TCC_HIT_sum")))
        miss = sum(forward(_counter_sums(l2_csv, "TCC_MISS_sum")))
        res["l2_requests_per_call"] = (hit + miss) / calls
        res["l2_hit"] = hit / (hit + miss) if hit + miss > 0 else None
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        sums = _counter_sums(path, counter)
        copy = [v for (n, v) in sums.values() if "copyBuffer" in n and v > 1000]
        kern = forward(sums)
        scale = (copy_mib * 1024.0) / copy[0]
        res[f"{tag}_kib_raw_per_call"] = sum(kern) / calls
        res[f"{tag}_copy_scale"] = scale
        res[f"{tag}_bytes_per_call"] = sum(kern) / calls * scale * 1024.0
        res["dispatches_per_call"] = len(kern) / calls
    res["hbm_bytes_per_call"] = res["fetch_bytes_per_call"] + res["write_bytes_per_call"]
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    return res


def time_launches(torch, fn, steps: int, warmup: int):
    """Runs fn() warmup times, then times `steps` calls with HIP events on the
    launch stream and with wall clock around the whole loop."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall_ms, float(np.mean(ev)), float(np.min(ev))


def time_cold(torch, fn, steps: int, flush_mib: int = 1024):
    """Times `steps` calls one by one with HIP events, writing a flush_mib
    buffer before each (outside the timed region) so that no K/V line is left
    in the L2s or the 256 MB Infinity Cache.  Returns (median, min) ms."""
    stream = torch.cuda.current_stream()
    scratch = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda")
    ev = []
    for _ in range(steps):
        scratch.zero_()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ev.append(a.elapsed_time(b))
    del scratch
    return float(np.median(ev)), float(np.min(ev))


def slot_blocks(idx: np.ndarray, bs: int, N: int, qps: int) -> int:
    """Sum over groups of qps consecutive queries of one (b, g), from m = 0, of
    the number of distinct counted blocks in their rows: the blocks a
    wavefront slot of qps queries stages (qps = the slot's queries), or the
    (tile, block) pairs its MFMAs run (qps = queries per 16-column tile)."""
    B, M, G, T = idx.shape
    NB = -(-N // bs)
    total = 0
    step = max(1, (1 << 22) // max(1, G * T))     # bounded temporaries
    step -= step % qps
    step = max(step, qps)
    for lo in range(0, M, step):
        hi = min(M, lo + step)
        c = (np.arange(lo, hi) // bs)[None, :, None, None]
        e = idx[:, lo:hi].astype(np.int64)
        e = np.where((e >= 0) & (e <= c) & (e < NB), e, -1)
        pad = (-(hi - lo)) % qps
        if pad:
            e = np.concatenate([e, np.full((B, pad, G, T), -1, np.int64)], axis=1)
        e = np.sort(e.transpose(0, 2, 1, 3).reshape(B, G, -1, qps * T), axis=-1)
        total += int(((e[..., 1:] != e[..., :-1]) & (e[..., 1:] >= 0)).sum() + (e[..., 0] >= 0).sum())
    return total


def cpu_baseline(cfg: Config, q, k, v, idx, target_s: float = 15.0):
    """The fp64 CPU oracle on random units of the same workload."""
    import oracle
    threads = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    rng = np.random.default_rng(2024)

    def pick(n):
        return np.stack([rng.integers(0, cfg.B, n), rng.integers(0, cfg.M, n),
                         rng.integers(0, cfg.G, n)], axis=1).astype(np.int64)

    def unit_flops(units):
        bs = cfg.block_size
        t = idx[units[:, 0], units[:, 1], units[:, 2]].astype(np.int64)    # [U, T]
        m = units[:, 1:2]
        ok = (t >= 0) & (t <= m // bs) & (t < cfg.NB)
        vis = np.minimum(np.minimum((t + 1) * bs, cfg.N), m + 1) - t * bs
        return 4.0 * cfg.D * cfg.gs * float(np.where(ok, np.maximum(vis, 0), 0).sum())

    # Size the sample from a first timed pass (a few units per thread start
    # slower than the steady rate, so a second, larger pass refines it).
    n = max(threads * 4, 64)
    for _ in range(2):
        probe = pick(n)
        t0 = time.perf_counter()
        oracle.oracle_units(q, k, v, idx, cfg.block_size, probe, threads)
        dt = time.perf_counter() - t0
        n = int(min(1_000_000, max(probe.shape[0], probe.shape[0] * min(target_s, 1.0) / max(dt, 1e-3))))
        if dt >= 0.5:
            break
    n = int(min(1_000_000, max(probe.shape[0], probe.shape[0] * target_s / max(dt, 1e-3))))
    units = pick(n)
    t0 = time.perf_counter()
    oracle.oracle_units(q, k, v, idx, cfg.block_size, units, threads)
    dt = time.perf_counter() - t0
    return {"value": unit_flops(units) / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{n} random (b,m,g) units of the {cfg.name} workload, fp64, {dt:.1f} s",
            "ms_per_unit": dt * 1e3 / n}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="64k", choices=sorted(CONFIGS))
    ap.add_argument("--no-dense", action="store_true", help="skip the all-causal-blocks run")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-dense-fa", action="store_true", help="skip the dense causal attention kernel")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward pass")
    ap.add_argument("--no-window", action="store_true", help="skip the sliding-window kernel runs")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 selection forward")
    ap.add_argument("--no-topk", action="store_true", help="skip the top-k block selection")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10, help="cold-cache timed calls (0 = skip)")
    ap.add_argument("--no-probe", action="store_true", help="skip the gather-ceiling probe")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (scale for HBM counters)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="write the counter summary from rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE and "
                         "optionally TCC_HIT_sum/TCC_MISS_sum) and exit")
    ap.add_argument("--pmc-calls", type=int, default=0, help="nsa_sel_fwd calls in the --pmc runs")
    args = ap.parse_args()

    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            ap.error("--summarize-pmc takes FETCH_CSV WRITE_CSV [L2_CSV]")
        res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_calls,
                            args.copy_probe_mib, COUNTERS_FILE,
                            args.summarize_pmc[2] if len(args.summarize_pmc) == 3 else None)
        print(json.dumps(res))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_sel_amd.binding import nsa_sel_fwd, nsa_sel_fwd_workspace_size, nsa_sel_fwd_ws

    cfg = CONFIGS[args.config]
    print(f"[bench] generating {cfg}", file=sys.stderr, flush=True)
    q, k, v, idx = make_inputs(cfg)
    dev = torch.device("cuda:0")
    tq, tk, tv, ti = (torch.from_numpy(a).to(dev) for a in (q, k, v, idx))
    O = torch.empty((cfg.B, cfg.M, cfg.H, cfg.D), dtype=torch.float16, device=dev)
    L = torch.empty((cfg.B, cfg.H, cfg.M), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    workspaces = {}

    def workspace(T):
        if T not in workspaces:
            n = nsa_sel_fwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, T)
            workspaces[T] = torch.empty(n, dtype=torch.uint8, device=dev)
        return workspaces[T]

    def launch(ti_=ti, T=cfg.T):
        ws = workspace(T)
        nsa_sel_fwd_ws(tq, tk, tv, ti_, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, T, ws,
                       ws.numel(), stream.cuda_stream)

    def launch_generations():
        nsa_sel_fwd(tq, tk, tv, ti, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T,
                    stream.cuda_stream)

    workspace(cfg.T)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    blocks, keys = work_counts(cfg, idx)
    gathered = blocks * cfg.block_size * cfg.D * 2 * 2
    flops = 4.0 * cfg.D * cfg.gs * keys
    compulsory = compulsory_bytes(cfg)
    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    wall_ms, ev_ms, ev_min = time_launches(torch, launch, args.steps, args.warmup)
    assert torch.isfinite(L).all().item(), "non-finite LSE"

    gbps = gathered / (ev_ms * 1e-3) / 1e9
    tflops = flops / (wall_ms * 1e-3) / 1e12
    out = {
        "metric": "NSA sel-attn fwd ms + eff. TFLOP/s & gathered GB/s, M=64k T=16 bs=64",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"nsa_sel_fwd_ws {cfg.name}", "B": cfg.B, "M": cfg.M, "N": cfg.N, "H": cfg.H,
                   "G": cfg.G, "D": cfg.D, "block_size": cfg.block_size, "T": cfg.T,
                   "index_rule": cfg.rule, "seed": cfg.seed},
        "kernel_ms": round(ev_ms, 4),
        "kernel_ms_min": round(ev_min, 4),
        "workspace_bytes": workspace(cfg.T).numel(),
        "gathered_GBps": round(gbps, 1),
        "eff_TFLOPs": round(flops / (ev_ms * 1e-3) / 1e12, 3),
        "work": {"counted_blocks": blocks, "visible_keys": keys, "gathered_bytes": gathered,
                 "effective_flops": flops, "compulsory_bytes": compulsory},
    }
    counters = _counters()
    traffic = counters.get("hbm_bytes_per_call") if counters else None
    out["roofline"] = roofline(flops, compulsory, ev_ms, traffic)
    # Beside the roofline: the time each bound alone allows, the counter
    # traffic past the L2 (measured HBM/Infinity-Cache bytes) as a rate and a
    # fraction of the HBM peak, the L2 hit rate of the kernel's requests, and
    # the logical gathered-K/V rate (cache-served re-reads included, so it may
    # exceed the HBM peak).
    detail = {"compulsory_bytes": compulsory,
              "t_hbm_ms": round(compulsory / (HBM_PEAK_GBPS * 1e9) * 1e3, 4),
              "t_mfma_ms": round(flops / (FP16_PEAK_TFLOPS * 1e12) * 1e3, 4),
              "gathered_GBps": round(gbps, 1)}
    if traffic:
        detail["traffic_GBps"] = round(traffic / (ev_ms * 1e-3) / 1e9, 1)
        detail["traffic_frac_of_hbm_peak"] = round(traffic / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        detail["traffic_over_compulsory"] = round(traffic / compulsory, 2)
    if counters and counters.get("l2_hit") is not None:
        detail["l2_hit"] = round(counters["l2_hit"], 4)

    if args.cold_steps > 0:
        print(f"[bench] cold timing, {args.cold_steps} calls", file=sys.stderr, flush=True)
        c_med, c_min = time_cold(torch, launch, args.cold_steps)
        out["cold"] = {"ms_median": round(c_med, 4), "ms_min": round(c_min, 4), "flush_MiB": 1024,
                       "eff_TFLOPs": round(flops / (c_med * 1e-3) / 1e12, 3),
                       "gathered_GBps": round(gathered / (c_med * 1e-3) / 1e9, 1)}
        detail["frac_cold_median"] = roofline(flops, compulsory, c_med)["frac"]
    out["roofline_detail"] = detail

    # The same forward as one dispatch per generation (no workspace).
    print("[bench] generation launches (nsa_sel_fwd)", file=sys.stderr, flush=True)
    _, gl_ev, gl_min = time_launches(torch, launch_generations, args.steps, args.warmup)
    out["generation_launches"] = {"kernel": "nsa_sel_fwd", "ms": round(gl_ev, 4), "ms_min": round(gl_min, 4),
                                  "over_workspace_call": round(gl_ev / ev_ms, 4)}

    if not args.no_graph:
        # One forward call captured in a HIP graph and replayed: the launch
        # cost a caller that captures the call avoids.
        print("[bench] HIP graph replay", file=sys.stderr, flush=True)
        ws = workspace(cfg.T)
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            nsa_sel_fwd_ws(tq, tk, tv, ti, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T,
                           ws, ws.numel(), side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            nsa_sel_fwd_ws(tq, tk, tv, ti, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T,
                           ws, ws.numel(), torch.cuda.current_stream(dev).cuda_stream)
        _, g_ev, g_min = time_launches(torch, graph.replay, args.steps, args.warmup)
        assert torch.isfinite(L).all().item(), "non-finite LSE after graph replay"
        out["graph"] = {"ms": round(g_ev, 4), "ms_min": round(g_min, 4),
                        "eager_over_graph": round(ev_ms / g_ev, 4)}
        del graph

    # MFMA work actually issued: every (16-column tile, staged block) pair runs
    # the QK and PV products over the whole block, 4 * 16 * bs * D flops.
    pack = 4 if 16 // cfg.gs >= 4 else 2 if 16 // cfg.gs >= 2 else 1
    tile_blocks = slot_blocks(idx, cfg.block_size, cfg.N, pack)
    mfma_flops = 4.0 * 16 * cfg.block_size * cfg.D * tile_blocks
    out["mfma"] = {"tile_blocks": tile_blocks, "executed_flops": mfma_flops,
                   "TFLOPs": round(mfma_flops / (ev_ms * 1e-3) / 1e12, 2),
                   "util": round(mfma_flops / (ev_ms * 1e-3) / (FP16_PEAK_TFLOPS * 1e12), 4)}

    if not args.no_probe:
        from block_sparse_attention_sel_amd.binding import nsa_gather_probe
        print("[bench] gather-ceiling probe", file=sys.stderr, flush=True)
        staged = torch.zeros(1, dtype=torch.int64, device=dev)
        ws = workspace(cfg.T)
        qps = nsa_gather_probe(tk, tv, ti, staged, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size,
                               cfg.T, stream.cuda_stream, ws, ws.numel())
        torch.cuda.synchronize()
        n_staged = int(staged.item())

        def probe():
            nsa_gather_probe(tk, tv, ti, staged, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size,
                             cfg.T, stream.cuda_stream, ws, ws.numel())

        _, p_ev, p_min = time_launches(torch, probe, args.steps, args.warmup)
        staged_bytes = n_staged * cfg.block_size * cfg.D * 4
        out["gather_ceiling"] = {"kernel": "nsa_gather_probe", "ms": round(p_ev, 4), "ms_min": round(p_min, 4),
                                 "kernel_over_probe": round(ev_ms / p_ev, 4), "queries_per_slot": qps,
                                 "staged_blocks": n_staged, "staged_bytes": staged_bytes,
                                 "staged_GBps": round(staged_bytes / (p_ev * 1e-3) / 1e9, 1)}

    if not args.no_dense:
        dcfg = cfg.dense()
        print(f"[bench] dense mode T={dcfg.T}", file=sys.stderr, flush=True)
        didx = block_indices(dcfg)
        tdi = torch.from_numpy(didx).to(dev)
        del didx
        d_wall, d_ev, _ = time_launches(torch, lambda: launch(tdi, dcfg.T), args.dense_steps, 1)
        dblocks, dkeys = work_counts(dcfg, None)
        out["dense_mode"] = {"T": dcfg.T, "kernel_ms": round(d_ev, 3),
                             "eff_TFLOPs": round(4.0 * cfg.D * cfg.gs * dkeys / (d_ev * 1e-3) / 1e12, 3),
                             "gathered_GBps": round(dblocks * cfg.block_size * cfg.D * 4 / (d_ev * 1e-3) / 1e9, 1),
                             "ratio_dense_over_selected": round(d_ev / ev_ms, 2)}
        del tdi

    if not args.no_dense_fa:
        # The dense causal attention the selection is measured against (same
        # Q, K, V and layouts; every key n <= m visible).
        from block_sparse_attention_sel_amd.binding import nsa_dense_fwd
        print("[bench] dense causal attention (nsa_dense_fwd)", file=sys.stderr, flush=True)

        def dense():
            nsa_dense_fwd(tq, tk, tv, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, stream.cuda_stream)

        _, f_ev, f_min = time_launches(torch, dense, args.dense_steps, 1)
        _, dkeys = work_counts(cfg.dense(), None)
        f_flops = 4.0 * cfg.D * cfg.gs * dkeys
        out["dense_fa"] = {"kernel": "nsa_dense_fwd", "ms": round(f_ev, 3), "ms_min": round(f_min, 3),
                           "eff_TFLOPs": round(f_flops / (f_ev * 1e-3) / 1e12, 2),
                           "mfma_frac": round(f_flops / (f_ev * 1e-3) / (FP16_PEAK_TFLOPS * 1e12), 4),
                           "ratio_dense_fa_over_selected": round(f_ev / ev_ms, 2)}

    if not args.no_bwd:
        # Gradients of the selection attention from this config's forward O
        # and LSE (recomputed here: the dense runs above reuse O and L).
        from block_sparse_attention_sel_amd.binding import nsa_sel_bwd, nsa_sel_bwd_workspace_size
        print("[bench] backward (nsa_sel_bwd)", file=sys.stderr, flush=True)
        launch()
        tdo = torch.from_numpy(make_grad_output(cfg)).to(dev)
        nbytes = nsa_sel_bwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dq = torch.empty((cfg.B, cfg.M, cfg.H, cfg.D), dtype=torch.float32, device=dev)
        dk = torch.empty((cfg.B, cfg.N, cfg.G, cfg.D), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)

        def bwd():
            nsa_sel_bwd(tq, tk, tv, ti, O, L, tdo, dq, dk, dv, ws, nbytes, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G,
                        cfg.D, cfg.block_size, cfg.T, stream.cuda_stream)

        _, b_ev, b_min = time_launches(torch, bwd, args.steps, args.warmup)
        assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item(), "non-finite gradients"
        b_flops = 10.0 * cfg.D * cfg.gs * keys
        out["backward"] = {"kernel": "nsa_sel_bwd", "ms": round(b_ev, 3), "ms_min": round(b_min, 3),
                           "eff_TFLOPs": round(b_flops / (b_ev * 1e-3) / 1e12, 2),
                           "effective_flops": b_flops, "ratio_bwd_over_fwd": round(b_ev / ev_ms, 2),
                           "workspace_MiB": round(nbytes / 2 ** 20, 1)}
        del tdo, ws, dq, dk, dv

    if not args.no_bf16:
        # The selection forward with bf16 Q, K, V, O (same draws, rounded to bf16).
        import torch as _t
        from block_sparse_attention_sel_amd.binding import nsa_sel_fwd_bf16_ws
        print("[bench] bf16 selection forward", file=sys.stderr, flush=True)
        qb, kb, vb, _ = make_inputs_bf16(cfg)
        bq, bk, bv = (_t.from_numpy(a.view(np.int16)).view(_t.bfloat16).to(dev) for a in (qb, kb, vb))
        del qb, kb, vb
        Ob = torch.empty((cfg.B, cfg.M, cfg.H, cfg.D), dtype=torch.bfloat16, device=dev)

        wsb = workspace(cfg.T)

        def sel_bf16():
            nsa_sel_fwd_bf16_ws(bq, bk, bv, ti, Ob, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size,
                                cfg.T, wsb, wsb.numel(), stream.cuda_stream)

        _, s_ev, s_min = time_launches(torch, sel_bf16, args.steps, args.warmup)
        out["bf16"] = {"kernel": "nsa_sel_fwd_bf16_ws", "ms": round(s_ev, 4), "ms_min": round(s_min, 4),
                       "eff_TFLOPs": round(flops / (s_ev * 1e-3) / 1e12, 3),
                       "ratio_bf16_over_fp16": round(s_ev / ev_ms, 3)}
        if args.no_window:
            del bq, bk, bv, Ob

    if not args.no_window:
        # Sliding-window attention (keys m - LEFT .. m) on the same tensors at
        # the FlyDSL page's windows.  Flops: 4 * D * (H/G) per visible
        # (query, key) pair; the page's TF column counts half of that.
        from block_sparse_attention_sel_amd.binding import nsa_window_fwd, nsa_window_fwd_bf16
        runs = []
        m = np.arange(cfg.M, dtype=np.int64)
        for left in (512, 8192):
            pairs = int(np.minimum(np.minimum(m, left) + 1, np.maximum(cfg.N - np.maximum(m - left, 0), 0)).sum())
            wflops = 4.0 * cfg.D * cfg.H * pairs * cfg.B
            for dt in ("fp16", "bf16"):
                if dt == "bf16" and args.no_bf16:
                    continue
                print(f"[bench] window ({left}, 0) {dt}", file=sys.stderr, flush=True)
                if dt == "fp16":
                    def win(left=left):
                        nsa_window_fwd(tq, tk, tv, O, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, left, 0,
                                       stream.cuda_stream)
                else:
                    def win(left=left):
                        nsa_window_fwd_bf16(bq, bk, bv, Ob, L, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, left, 0,
                                            stream.cuda_stream)
                _, w_ev, w_min = time_launches(torch, win, args.steps, args.warmup)
                runs.append({"window": [left, 0], "dtype": dt, "ms": round(w_ev, 4), "ms_min": round(w_min, 4),
                             "eff_TFLOPs": round(wflops / (w_ev * 1e-3) / 1e12, 2),
                             "page_convention_TFLOPs": round(wflops / 2 / (w_ev * 1e-3) / 1e12, 2)})
        out["window"] = {"kernel": "nsa_window_fwd / nsa_window_fwd_bf16", "runs": runs}
        if not args.no_bf16:
            del bq, bk, bv, Ob

    if not args.no_topk:
        # Top-k block selection over N(0, 1) block scores [B, M, G, NB]; bytes
        # are the causal candidates read (rows with more candidates than T)
        # plus the index rows written.
        from block_sparse_attention_sel_amd.binding import nsa_topk_blocks
        print("[bench] top-k block selection", file=sys.stderr, flush=True)
        tsc = torch.from_numpy(block_scores(cfg)).to(dev)
        tout = torch.empty((cfg.B, cfg.M, cfg.G, cfg.T), dtype=torch.int32, device=dev)

        def topk():
            nsa_topk_blocks(tsc, tout, cfg.B, cfg.M, cfg.G, cfg.NB, cfg.block_size, cfg.T, stream.cuda_stream)

        _, k_ev, k_min = time_launches(torch, topk, args.steps, args.warmup)
        nc = np.minimum(np.arange(cfg.M, dtype=np.int64) // cfg.block_size, cfg.NB - 1) + 1
        read = int(np.where(nc > cfg.T, nc, 0).sum()) * 4 * cfg.B * cfg.G
        written = cfg.B * cfg.M * cfg.G * cfg.T * 4
        out["topk"] = {"kernel": "nsa_topk_blocks", "ms": round(k_ev, 4), "ms_min": round(k_min, 4),
                       "bytes": read + written,
                       "GBps": round((read + written) / (k_ev * 1e-3) / 1e9, 1),
                       "hbm_frac": round((read + written) / (k_ev * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del tsc, tout

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, q, k, v, idx, args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
