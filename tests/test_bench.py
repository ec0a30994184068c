"""bench.py's work accounting (CPU only): the counts that every reported
throughput divides by, checked against brute force over the index rows and
against the closed forms the index rules imply, plus the counter summary that
turns two rocprofv3 --pmc runs into HBM bytes per call.
"""

import csv
import json
import os

import numpy as np
import pytest

import bench
from block_sparse_attention_sel_amd.inputs import CONFIGS, block_indices


def _brute_counts(cfg, idx):
    """Counted entries and visible keys, unit by unit and entry by entry."""
    bs, blocks, keys = cfg.block_size, 0, 0
    for b in range(cfg.B):
        for m in range(cfg.M):
            for g in range(cfg.G):
                for t in idx[b, m, g].tolist():
                    if t < 0 or t > m // bs or t >= cfg.NB:
                        continue
                    blocks += 1
                    keys += min((t + 1) * bs, cfg.N, m + 1) - t * bs
    return blocks, keys


def _noisy(cfg, seed):
    """The rule's rows with padding, future and out-of-range entries mixed in."""
    idx = block_indices(cfg).copy()
    rng = np.random.default_rng(seed)
    pick = rng.random(idx.shape) < 0.2
    m = np.arange(cfg.M)[None, :, None, None]
    junk = rng.choice(np.array([-1, -7, cfg.NB, cfg.NB + 5]), size=idx.shape)
    future = (m // cfg.block_size + 1 + rng.integers(0, 3, size=idx.shape)).astype(np.int32)
    idx[pick] = np.where(rng.random(idx.shape) < 0.5, junk, future)[pick]
    return idx


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", {"M": 300, "N": 300, "G": 2, "H": 8}),
    ("8k", {"M": 700, "N": 700}),
    ("128k-local", {"M": 900, "N": 900}),
    ("32k-bs32", {"M": 333, "N": 333}),
])
def test_work_counts_match_brute_force(name, over):
    cfg = CONFIGS[name].with_(**over)
    for idx in (block_indices(cfg), _noisy(cfg, 7)):
        assert bench.work_counts(cfg, idx) == _brute_counts(cfg, idx)


def test_work_counts_dense_rule_closed_form():
    cfg = CONFIGS["tiny"].with_(rule="dense", M=512, N=512)
    cfg = cfg.with_(T=cfg.NB)
    m = np.arange(cfg.M)
    want_blocks = int((m // cfg.block_size + 1).sum()) * cfg.B * cfg.G
    want_keys = int((m + 1).sum()) * cfg.B * cfg.G
    assert bench.work_counts(cfg, block_indices(cfg)) == (want_blocks, want_keys)


def _closed_form(cfg):
    """Every generated row holds min(T, c + 1) counted blocks, the query's own
    block c among them and every other one fully visible, so a unit sees
    m + 1 keys when all its causal blocks are selected and
    (vb - 1) * bs + (m - c * bs) + 1 otherwise."""
    m = np.arange(cfg.M, dtype=np.int64)
    c = m // cfg.block_size
    vb = np.minimum(cfg.T, c + 1)
    vis = np.where(vb == c + 1, m + 1, (vb - 1) * cfg.block_size + (m - c * cfg.block_size) + 1)
    return int(vb.sum()) * cfg.B * cfg.G, int(vis.sum()) * cfg.B * cfg.G


@pytest.mark.parametrize("name", ["tiny", "8k", "64k", "32k-bs32", "128k-local"])
def test_full_size_counts_follow_the_closed_form(name):
    cfg = CONFIGS[name]
    assert bench.work_counts(cfg, block_indices(cfg)) == _closed_form(cfg)


# Totals of counted (unit, block) pairs per workload, worked out by hand from
# the index rules alone: the sum over units of min(T, m // bs + 1).
HAND_BLOCKS = {"tiny": 3904, "8k": 246784, "64k": 8327168, "32k-bs32": 8261632, "128k-local": 16715776}


@pytest.mark.parametrize("name", sorted(HAND_BLOCKS))
def test_closed_form_totals(name):
    assert _closed_form(CONFIGS[name])[0] == HAND_BLOCKS[name]


@pytest.mark.parametrize("qps", [1, 2, 4, 8])
def test_slot_blocks_match_brute_force(qps):
    cfg = CONFIGS["tiny"].with_(M=333, N=333, G=2, H=8)
    idx = _noisy(cfg, 3)
    want = 0
    for b in range(cfg.B):
        for g in range(cfg.G):
            for m0 in range(0, cfg.M, qps):
                seen = set()
                for m in range(m0, min(cfg.M, m0 + qps)):
                    seen.update(t for t in idx[b, m, g].tolist()
                                if 0 <= t <= m // cfg.block_size and t < cfg.NB)
                want += len(seen)
    assert bench.slot_blocks(idx, cfg.block_size, cfg.N, qps) == want


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, values in rows:
            for v in values:  # one row per hardware instance, summed by the reader
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    # A 4 MiB copy that FETCH_SIZE reads as half its bytes (2048 KiB) and
    # WRITE_SIZE as all of them; two calls of two dispatches each; a small
    # copy (torch's own transfers) is ignored.
    kern = "void (anonymous namespace)::nsa_sel_fwd_kernel<64, 2, 128, 2, 2, false>(Params)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counter_csv(fetch, "FETCH_SIZE", [(1, copy, [12.0]), (2, copy, [1024.0, 1024.0]),
                                             (3, kern, [100.0, 50.0]), (4, kern, [150.0]),
                                             (5, kern, [120.0, 30.0]), (6, kern, [150.0])])
    _write_counter_csv(write, "WRITE_SIZE", [(1, copy, [24.0]), (2, copy, [4096.0]), (3, kern, [10.0]),
                                             (4, kern, [10.0]), (5, kern, [10.0]), (6, kern, [10.0])])
    out = tmp_path / "s.json"
    bench.summarize_pmc(str(fetch), str(write), calls=2, copy_mib=4, out_path=str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch_copy_scale"] == pytest.approx(2.0)
    assert rec["write_copy_scale"] == pytest.approx(1.0)
    assert rec["dispatches_per_call"] == 2
    assert rec["fetch_bytes_per_call"] == pytest.approx(300.0 * 2.0 * 1024)
    assert rec["write_bytes_per_call"] == pytest.approx(20.0 * 1024)
    assert rec["hbm_bytes_per_call"] == pytest.approx(rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"])
    assert rec["kernel_sha256"] == bench._kernel_sha()


def test_committed_counters_match_the_kernel_sources():
    # The committed HBM counters are reported only while they describe the
    # current kernel sources; this catches a kernel change without a re-run.
    rec = json.load(open(bench.COUNTERS_FILE))
    assert rec["kernel_sha256"] == bench._kernel_sha(), "re-take the FETCH_SIZE / WRITE_SIZE runs"
    assert rec["hbm_bytes_per_call"] > 0
    assert os.path.exists(bench.COUNTERS_FILE.replace(".json", ".md"))


def test_summarize_pmc_l2_hit_rate(tmp_path):
    kern = "void (anonymous namespace)::nsa_sel_fwd_kernel<64, 2, 128, 2, 2, false>(Params)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write, l2 = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "l2.csv"
    _write_counter_csv(fetch, "FETCH_SIZE", [(1, copy, [2048.0]), (2, kern, [10.0])])
    _write_counter_csv(write, "WRITE_SIZE", [(1, copy, [4096.0]), (2, kern, [1.0])])
    with open(l2, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in (("TCC_HIT_sum", 300.0), ("TCC_MISS_sum", 100.0)):
            w.writerow({"Dispatch_Id": 2, "Kernel_Name": kern, "Counter_Name": name, "Counter_Value": v})
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": name, "Counter_Value": 7.0})
    out = tmp_path / "s.json"
    rec = bench.summarize_pmc(str(fetch), str(write), calls=1, copy_mib=4, out_path=str(out), l2_csv=str(l2))
    assert rec["l2_hit"] == pytest.approx(0.75)
    assert rec["l2_requests_per_call"] == pytest.approx(400.0)


def test_compulsory_bytes_by_hand():
    cfg = CONFIGS["64k"]
    # Q and O: 65536 * 64 * 128 * 2 B each; K and V: 65536 * 8 * 128 * 2 B each;
    # index rows 65536 * 8 * 16 * 4 B; LSE 64 * 65536 * 4 B.
    want = 2 * 1073741824 + 2 * 134217728 + 33554432 + 16777216
    assert bench.compulsory_bytes(cfg) == want


def test_roofline_picks_the_binding_bound():
    # 2.5e12 flops take 1 ms at the MFMA peak; 8e9 bytes take 1 ms at the HBM peak.
    r = bench.roofline(2.5e12, 4e9, 4.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(0.25) and r["achieved"] == pytest.approx(625.0)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    r = bench.roofline(1.25e12, 16e9, 4.0, traffic=123.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.5) and r["achieved"] == pytest.approx(4000.0)
    assert r["traffic"] == 123.0
    # A physical roofline: no kernel can exceed it.
    for ms in (0.5, 1.0, 10.0):
        r = bench.roofline(2.5e12, 8e9, ms)
        assert r["frac"] == pytest.approx(1.0 / ms)
