"""nsa_sel_bwd_noalloc (include/nsa_sel_bwd.h): the backward for callers that
cannot allocate device memory, with its workspace in the library's own
scratch array, against nsa_sel_bwd with a caller-allocated workspace.

The two run the same kernels on the same inputs, so their gradients must be
bitwise equal.  Two calls in a row share the scratch: the second, with a
smaller input, must not see the first's leftovers.  Each call is checked
against the workspace entry point called right before it.
"""

import sys

import numpy as np
import pytest

from block_sparse_attention_sel_amd.inputs import CONFIGS, make_grad_output, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_pair(torch, cfg):
    from block_sparse_attention_sel_amd import binding
    _say(f"case noalloc {cfg}")
    q, k, v, idx = make_inputs(cfg)
    do = make_grad_output(cfg)
    tq, tk, tv, ti, tdo = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in (q, k, v, idx, do))
    O, L = binding.sel_attn_fwd(tq, tk, tv, ti, cfg.block_size)
    shape_q = (cfg.B, cfg.M, cfg.H, cfg.D)
    shape_kv = (cfg.B, cfg.N, cfg.G, cfg.D)
    ref = [torch.empty(shape_q, dtype=torch.float32, device="cuda"),
           torch.empty(shape_kv, dtype=torch.float32, device="cuda"),
           torch.empty(shape_kv, dtype=torch.float32, device="cuda")]
    got = [torch.full_like(t, float("nan")) for t in ref]
    n = binding.nsa_sel_bwd_workspace_size(cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    sizes = (cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D, cfg.block_size, cfg.T)
    binding.nsa_sel_bwd(tq, tk, tv, ti, O, L, tdo, *ref, ws, n, *sizes, stream)
    torch.cuda.synchronize()
    del ws
    binding.nsa_sel_bwd_noalloc(tq, tk, tv, ti, O, L, tdo, *got, *sizes, stream)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(a).all().item(), name
        assert torch.equal(a, b), name
    _say(f"  bitwise equal; workspace of nsa_sel_bwd {n / 2**20:.2f} MiB")


def test_noalloc_matches_workspace_entry_point_twice_smaller_second():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # First the 8192-query workload at full size (62.6 MiB of workspace, near
    # the 64 MiB limit), then the headline shape at 1024 queries (9.1 MiB).
    _run_pair(torch, CONFIGS["8k"])
    _run_pair(torch, CONFIGS["64k"].with_(M=1024, N=1024))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_sel_amd import binding
    cfg = CONFIGS["8k"].with_(M=16384, N=16384)
    t = torch.zeros(16, dtype=torch.float16, device="cuda")   # never touched: the sizes are refused first
    rc = binding.nsa_sel_bwd_noalloc_raw(t, t, t, t, t, t, t, t, t, t, cfg.B, cfg.M, cfg.N, cfg.H, cfg.G, cfg.D,
                                         cfg.block_size, cfg.T, 0)
    assert rc == binding.NSA_SEL_ERR_SCRATCH
