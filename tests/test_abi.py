"""The C-ABI library without a GPU: it loads, exports what the header declares,
and rejects bad arguments on the host before any HIP call."""

import os
import re
import subprocess

import pytest

from block_sparse_attention_sel_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa_sel.h")

GOOD = dict(B=1, M=256, N=256, H=8, G=1, D=128, block_size=64, T=4)
# Distinct, 16-byte aligned fake addresses far apart: validation never
# dereferences them and returns before any HIP call.
ADDR = {name: (i + 1) << 36 for i, name in enumerate(["Q", "K", "V", "I", "O", "L"])}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libnsa_sel.so not built")
    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_sel_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported
        assert getattr(lib, name) is not None


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in re.findall(r"(NSA_SEL_\w+)\s*=\s*(\d+)", text):
        assert getattr(binding, name) == int(val)


def test_status_strings(lib):
    for code in range(0, 10):
        s = binding.nsa_sel_status_string(code)
        assert isinstance(s, str) and s
    assert binding.nsa_sel_status_string(0) == "ok"
    assert "unknown" in binding.nsa_sel_status_string(99)


def _call(**over):
    args = dict(GOOD)
    ptrs = dict(ADDR)
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    return binding.nsa_sel_fwd_raw(ptrs["Q"], ptrs["K"], ptrs["V"], ptrs["I"], ptrs["O"], ptrs["L"],
                                   args["B"], args["M"], args["N"], args["H"], args["G"], args["D"],
                                   args["block_size"], args["T"], 0)


@pytest.mark.parametrize("which", ["Q", "K", "V", "I", "O", "L"])
def test_null_pointer(lib, which):
    assert _call(**{which: 0}) == binding.NSA_SEL_ERR_NULL


@pytest.mark.parametrize("over", [dict(B=0), dict(M=0), dict(N=-1), dict(H=0), dict(G=0), dict(D=0),
                                  dict(block_size=0), dict(T=0), dict(H=8, G=3)])
def test_bad_shape(lib, over):
    assert _call(**over) == binding.NSA_SEL_ERR_SHAPE


@pytest.mark.parametrize("over", [dict(D=96), dict(D=256), dict(block_size=16), dict(block_size=128),
                                  dict(H=32, G=1)])
def test_unsupported(lib, over):
    assert _call(**over) == binding.NSA_SEL_ERR_UNSUPPORTED


@pytest.mark.parametrize("which,off", [("Q", 8), ("K", 2), ("V", 4), ("O", 8), ("I", 2), ("L", 1)])
def test_misaligned(lib, which, off):
    assert _call(**{which: ADDR[which] + off}) == binding.NSA_SEL_ERR_ALIGN


def test_range(lib):
    assert _call(B=1 << 12, M=1 << 20, G=1, H=1) == binding.NSA_SEL_ERR_RANGE


def test_alias(lib):
    assert _call(O=ADDR["Q"]) == binding.NSA_SEL_ERR_ALIAS
    assert _call(L=ADDR["K"] + 64) == binding.NSA_SEL_ERR_ALIAS
    assert _call(L=ADDR["O"] + 256) == binding.NSA_SEL_ERR_ALIAS


# A fake 256-byte aligned workspace address, far from the tensors above.
WS = 1 << 44


def _call_ws(ws=WS, nbytes=1 << 30, **over):
    args = dict(GOOD)
    ptrs = dict(ADDR)
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    return binding.nsa_sel_fwd_ws_raw(ptrs["Q"], ptrs["K"], ptrs["V"], ptrs["I"], ptrs["O"], ptrs["L"],
                                      args["B"], args["M"], args["N"], args["H"], args["G"], args["D"],
                                      args["block_size"], args["T"], ws, nbytes, 0)


@pytest.mark.parametrize("over", [dict(Q=0), dict(L=0), dict(M=0), dict(H=8, G=3), dict(D=96), dict(K=ADDR["K"] + 2),
                                  dict(O=ADDR["Q"]), dict(B=1 << 12, M=1 << 20, G=1, H=1)])
def test_workspace_forward_checks_like_the_forward(lib, over):
    # The argument checks of nsa_sel_fwd come first, with the same codes.
    assert _call_ws(**dict(over)) == _call(**dict(over)) != binding.NSA_SEL_OK


def test_fwd_workspace_size(lib):
    rc, n = binding.nsa_sel_fwd_workspace_size_raw(*GOOD.values())
    assert rc == binding.NSA_SEL_OK and n > 0 and n % 4 == 0
    rc, n2 = binding.nsa_sel_fwd_workspace_size_raw(*dict(GOOD, M=65536, N=65536).values())
    assert rc == binding.NSA_SEL_OK and n2 > n
    assert binding.nsa_sel_fwd_workspace_size_raw(*dict(GOOD, M=0).values())[0] == binding.NSA_SEL_ERR_SHAPE
    assert binding.nsa_sel_fwd_workspace_size_raw(*dict(GOOD, D=96).values())[0] == binding.NSA_SEL_ERR_UNSUPPORTED
    assert lib.nsa_sel_fwd_workspace_size(*GOOD.values(), None) == binding.NSA_SEL_ERR_NULL


def test_workspace_forward_rejects_bad_workspaces(lib):
    need = binding.nsa_sel_fwd_workspace_size(*GOOD.values())
    assert _call_ws(ws=0) == binding.NSA_SEL_ERR_WORKSPACE
    assert _call_ws(ws=WS + 128) == binding.NSA_SEL_ERR_WORKSPACE
    assert _call_ws(nbytes=need - 1) == binding.NSA_SEL_ERR_WORKSPACE
    assert _call_ws(nbytes=0) == binding.NSA_SEL_ERR_WORKSPACE
    for name in ("Q", "K", "V", "I", "O", "L"):
        assert _call_ws(ws=ADDR[name]) == binding.NSA_SEL_ERR_ALIAS, name
    o_bytes = GOOD["B"] * GOOD["M"] * GOOD["H"] * GOOD["D"] * 2
    assert _call_ws(ws=ADDR["O"] + o_bytes - 256) == binding.NSA_SEL_ERR_ALIAS  # O's last 256 bytes
    with pytest.raises(binding.NsaSelError) as ei:
        binding.nsa_sel_fwd_ws(*[ADDR[n] for n in ("Q", "K", "V", "I", "O", "L")], *GOOD.values(), 0, 0)
    assert ei.value.status == binding.NSA_SEL_ERR_WORKSPACE and "workspace" in str(ei.value)


def test_binding_raises_with_message(lib):
    with pytest.raises(binding.NsaSelError) as ei:
        binding.nsa_sel_fwd(0, 1, 2, 3, 4, 5, 1, 1, 1, 1, 1, 64, 32, 1, 0)
    assert ei.value.status == binding.NSA_SEL_ERR_NULL
    assert "NULL" in str(ei.value)


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "block_sparse_attention_sel_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"(import\s+oracle|from\s+oracle|nsa_oracle)", text), f


# --- gather-ceiling probe (include/nsa_gather_probe.h) -------------------------

PROBE_HEADER = os.path.join(ROOT, "include", "nsa_gather_probe.h")
PADDR = {name: (i + 1) << 36 for i, name in enumerate(["K", "V", "I", "S"])}


@pytest.fixture(scope="module")
def probe_lib():
    if not os.path.exists(binding.PROBE_LIB_PATH):
        pytest.skip("libnsa_gather_probe.so not built")
    return binding.load_probe_library()


def test_probe_header_declares_the_binding_names():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    assert sorted(set(re.findall(r"\b(nsa_\w+)\s*\(", text))) == sorted(binding.PROBE_EXPORTED)


def test_probe_library_exports_every_declared_symbol(probe_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.PROBE_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in binding.PROBE_EXPORTED:
        assert name in exported


def _probe_call(**over):
    args = dict(GOOD)
    ptrs = dict(PADDR)
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    return binding.nsa_gather_probe_raw(ptrs["K"], ptrs["V"], ptrs["I"], ptrs["S"], args["B"], args["M"],
                                        args["N"], args["H"], args["G"], args["D"], args["block_size"],
                                        args["T"], 0)[0]


@pytest.mark.parametrize("which", ["K", "V", "I", "S"])
def test_probe_null_pointer(probe_lib, which):
    assert _probe_call(**{which: 0}) == binding.NSA_SEL_ERR_NULL


@pytest.mark.parametrize("over,code", [(dict(M=0), binding.NSA_SEL_ERR_SHAPE),
                                       (dict(H=8, G=3), binding.NSA_SEL_ERR_SHAPE),
                                       (dict(D=96), binding.NSA_SEL_ERR_UNSUPPORTED),
                                       (dict(block_size=16), binding.NSA_SEL_ERR_UNSUPPORTED),
                                       (dict(B=1 << 12, M=1 << 20, G=1, H=1), binding.NSA_SEL_ERR_RANGE)])
def test_probe_bad_sizes(probe_lib, over, code):
    assert _probe_call(**over) == code


@pytest.mark.parametrize("which,off", [("K", 8), ("V", 2), ("I", 2), ("S", 4)])
def test_probe_misaligned(probe_lib, which, off):
    assert _probe_call(**{which: PADDR[which] + off}) == binding.NSA_SEL_ERR_ALIGN


def test_probe_rejects_bad_workspaces(probe_lib, lib):
    need = binding.nsa_sel_fwd_workspace_size(*GOOD.values())
    args = [PADDR["K"], PADDR["V"], PADDR["I"], PADDR["S"], *GOOD.values(), 0]
    assert binding.nsa_gather_probe_raw(*args, WS + 64, need)[0] == binding.NSA_SEL_ERR_WORKSPACE
    assert binding.nsa_gather_probe_raw(*args, WS, need - 4)[0] == binding.NSA_SEL_ERR_WORKSPACE


# --- dense causal attention (include/nsa_dense.h) ----------------------------

DENSE_HEADER = os.path.join(ROOT, "include", "nsa_dense.h")
DGOOD = dict(B=1, M=256, N=256, H=8, G=1, D=128)


def test_dense_header_declares_the_binding_names():
    text = re.sub(r"/\*.*?\*/", "", open(DENSE_HEADER).read(), flags=re.S)
    assert sorted(set(re.findall(r"\b(nsa_\w+)\s*\(", text))) == sorted(binding.DENSE_EXPORTED)


def test_dense_symbol_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in binding.DENSE_EXPORTED:
        assert name in exported


def _dense_call(**over):
    args = dict(DGOOD)
    ptrs = {k: ADDR[k] for k in ("Q", "K", "V", "O", "L")}
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    return binding.nsa_dense_fwd_raw(ptrs["Q"], ptrs["K"], ptrs["V"], ptrs["O"], ptrs["L"], args["B"], args["M"],
                                     args["N"], args["H"], args["G"], args["D"], 0)


@pytest.mark.parametrize("which", ["Q", "K", "V", "O", "L"])
def test_dense_null_pointer(lib, which):
    assert _dense_call(**{which: 0}) == binding.NSA_SEL_ERR_NULL


@pytest.mark.parametrize("over,code", [(dict(M=0), binding.NSA_SEL_ERR_SHAPE), (dict(H=8, G=3), binding.NSA_SEL_ERR_SHAPE),
                                       (dict(D=96), binding.NSA_SEL_ERR_UNSUPPORTED),
                                       (dict(H=32, G=1), binding.NSA_SEL_ERR_UNSUPPORTED),
                                       (dict(B=1 << 12, M=1 << 20, G=1, H=1), binding.NSA_SEL_ERR_RANGE),
                                       (dict(Q=ADDR["Q"] + 8), binding.NSA_SEL_ERR_ALIGN),
                                       (dict(L=ADDR["L"] + 2), binding.NSA_SEL_ERR_ALIGN),
                                       (dict(O=ADDR["K"]), binding.NSA_SEL_ERR_ALIAS),
                                       (dict(L=ADDR["O"] + 64), binding.NSA_SEL_ERR_ALIAS)])
def test_dense_rejects_bad_arguments(lib, over, code):
    assert _dense_call(**over) == code


# --- backward (include/nsa_sel_bwd.h) ------------------------------------------

BWD_HEADER = os.path.join(ROOT, "include", "nsa_sel_bwd.h")
BNAMES = ["Q", "K", "V", "I", "O", "L", "dO", "dQ", "dK", "dV", "W"]
BADDR = {name: (i + 1) << 38 for i, name in enumerate(BNAMES)}


def test_bwd_header_declares_the_binding_names():
    text = re.sub(r"/\*.*?\*/", "", open(BWD_HEADER).read(), flags=re.S)
    assert sorted(set(re.findall(r"\b(nsa_\w+)\s*\(", text))) == sorted(binding.BWD_EXPORTED)


def test_bwd_symbols_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in binding.BWD_EXPORTED:
        assert name in exported


def test_bwd_workspace_size(lib):
    n = binding.nsa_sel_bwd_workspace_size(**GOOD)
    assert n > 0 and n % 256 == 0
    # grows with the problem
    assert binding.nsa_sel_bwd_workspace_size(**dict(GOOD, M=4096, N=4096)) > n
    assert binding.nsa_sel_bwd_workspace_size_raw(**dict(GOOD, D=96))[0] == binding.NSA_SEL_ERR_UNSUPPORTED
    assert binding.nsa_sel_bwd_workspace_size_raw(**dict(GOOD, M=0))[0] == binding.NSA_SEL_ERR_SHAPE
    # one batch of Q beyond 2^32 - 1 bytes
    rc, _ = binding.nsa_sel_bwd_workspace_size_raw(B=1, M=1 << 20, N=1024, H=16, G=1, D=128, block_size=64, T=4)
    assert rc == binding.NSA_SEL_ERR_RANGE
    assert lib.nsa_sel_bwd_workspace_size(1, 256, 256, 8, 1, 128, 64, 4, None) == binding.NSA_SEL_ERR_NULL


def _bwd_call(**over):
    args = dict(GOOD)
    ptrs = dict(BADDR)
    wsn = over.pop("wsn", None)
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    if wsn is None:
        rc, wsn = binding.nsa_sel_bwd_workspace_size_raw(**args)
    return binding.nsa_sel_bwd_raw(*(ptrs[k] for k in BNAMES), wsn, args["B"], args["M"], args["N"], args["H"],
                                   args["G"], args["D"], args["block_size"], args["T"], 0)


@pytest.mark.parametrize("which", BNAMES[:-1])
def test_bwd_null_pointer(lib, which):
    assert _bwd_call(**{which: 0}) == binding.NSA_SEL_ERR_NULL


@pytest.mark.parametrize("over,code", [
    (dict(M=0), binding.NSA_SEL_ERR_SHAPE), (dict(H=8, G=3), binding.NSA_SEL_ERR_SHAPE),
    (dict(D=96), binding.NSA_SEL_ERR_UNSUPPORTED), (dict(block_size=128), binding.NSA_SEL_ERR_UNSUPPORTED),
    (dict(Q=BADDR["Q"] + 8), binding.NSA_SEL_ERR_ALIGN), (dict(dO=BADDR["dO"] + 2), binding.NSA_SEL_ERR_ALIGN),
    (dict(dK=BADDR["dK"] + 4), binding.NSA_SEL_ERR_ALIGN), (dict(L=BADDR["L"] + 2), binding.NSA_SEL_ERR_ALIGN),
    (dict(W=0), binding.NSA_SEL_ERR_WORKSPACE), (dict(W=BADDR["W"] + 128), binding.NSA_SEL_ERR_WORKSPACE),
    (dict(wsn=256), binding.NSA_SEL_ERR_WORKSPACE),
    (dict(dQ=BADDR["O"]), binding.NSA_SEL_ERR_ALIAS), (dict(dV=BADDR["dK"] + 64), binding.NSA_SEL_ERR_ALIAS),
    (dict(W=BADDR["dO"]), binding.NSA_SEL_ERR_ALIAS), (dict(dK=BADDR["W"] + 1024), binding.NSA_SEL_ERR_ALIAS),
])
def test_bwd_rejects_bad_arguments(lib, over, code):
    assert _bwd_call(**over) == code


def _noalloc_call(**over):
    args = dict(GOOD)
    ptrs = dict(BADDR)
    for k in list(over):
        if k in ptrs:
            ptrs[k] = over.pop(k)
    args.update(over)
    return binding.nsa_sel_bwd_noalloc_raw(*(ptrs[k] for k in BNAMES[:-1]), args["B"], args["M"], args["N"],
                                           args["H"], args["G"], args["D"], args["block_size"], args["T"], 0)


@pytest.mark.parametrize("over,code", [
    (dict(Q=0), binding.NSA_SEL_ERR_NULL), (dict(dV=0), binding.NSA_SEL_ERR_NULL),
    (dict(M=0), binding.NSA_SEL_ERR_SHAPE), (dict(D=96), binding.NSA_SEL_ERR_UNSUPPORTED),
    (dict(L=BADDR["L"] + 2), binding.NSA_SEL_ERR_ALIGN),
    # sizes whose workspace exceeds the 64 MiB scratch: rejected before any HIP call
    (dict(B=1, M=65536, N=65536, H=64, G=8, D=128, block_size=64, T=16), binding.NSA_SEL_ERR_SCRATCH),
    (dict(B=2, M=4096, N=4096, H=64, G=4, D=128, block_size=32, T=32), binding.NSA_SEL_ERR_SCRATCH),
])
def test_bwd_noalloc_rejects_bad_arguments(lib, over, code):
    assert _noalloc_call(**over) == code


def test_bwd_noalloc_limit_is_the_documented_64_mib(lib):
    # The 8192-query workload named in the header fits; its workspace is
    # within 64 MiB, and one query block more than 64 MiB is refused.
    n = binding.nsa_sel_bwd_workspace_size(B=1, M=8192, N=8192, H=32, G=2, D=128, block_size=64, T=16)
    assert n <= 64 << 20
    assert binding.nsa_sel_bwd_workspace_size(B=1, M=16384, N=16384, H=32, G=2, D=128, block_size=64,
                                              T=16) > 64 << 20
    assert _noalloc_call(B=1, M=16384, N=16384, H=32, G=2, D=128, block_size=64, T=16) == \
        binding.NSA_SEL_ERR_SCRATCH


# --- top-k selection (include/nsa_topk.h) ---------------------------------------

TOPK_HEADER = os.path.join(ROOT, "include", "nsa_topk.h")


def test_topk_header_declares_the_binding_names():
    text = re.sub(r"/\*.*?\*/", "", open(TOPK_HEADER).read(), flags=re.S)
    assert sorted(set(re.findall(r"\b(nsa_\w+)\s*\(", text))) == sorted(binding.TOPK_EXPORTED)


def test_topk_symbol_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in binding.TOPK_EXPORTED:
        assert name in exported


def _topk_call(S=1 << 36, I=2 << 36, B=1, M=256, G=2, NB=4, bs=64, T=4):
    return binding.nsa_topk_blocks_raw(S, I, B, M, G, NB, bs, T, 0)


@pytest.mark.parametrize("over,code", [
    (dict(S=0), binding.NSA_SEL_ERR_NULL), (dict(I=0), binding.NSA_SEL_ERR_NULL),
    (dict(M=0), binding.NSA_SEL_ERR_SHAPE), (dict(T=0), binding.NSA_SEL_ERR_SHAPE),
    (dict(bs=0), binding.NSA_SEL_ERR_SHAPE), (dict(NB=0), binding.NSA_SEL_ERR_SHAPE),
    (dict(NB=4097), binding.NSA_SEL_ERR_UNSUPPORTED), (dict(S=(1 << 36) + 2), binding.NSA_SEL_ERR_ALIGN),
    (dict(I=(2 << 36) + 1), binding.NSA_SEL_ERR_ALIGN), (dict(B=1 << 12, M=1 << 20), binding.NSA_SEL_ERR_RANGE),
    (dict(I=(1 << 36) + 64), binding.NSA_SEL_ERR_ALIAS),
])
def test_topk_rejects_bad_arguments(lib, over, code):
    assert _topk_call(**over) == code


# --- the torch wrappers check caller-supplied buffers before any call ----------

def _cpu_inputs(B=1, M=64, N=64, H=8, G=2, D=64, T=4, dtype=None):
    import torch
    dt = dtype or torch.float16
    q = torch.zeros((B, M, H, D), dtype=dt)
    k = torch.zeros((B, N, G, D), dtype=dt)
    v = torch.zeros((B, N, G, D), dtype=dt)
    idx = torch.zeros((B, M, G, T), dtype=torch.int32)
    return q, k, v, idx


def test_wrappers_reject_bad_out_and_lse():
    import torch
    q, k, v, idx = _cpu_inputs()
    good_o = torch.empty_like(q)
    good_l = torch.empty((1, 8, 64), dtype=torch.float32)
    bad = [
        (dict(out=torch.empty((1, 64, 8, 32), dtype=torch.float16)), ValueError),   # short
        (dict(out=torch.empty_like(q, dtype=torch.float32)), TypeError),            # dtype
        (dict(out=torch.empty((1, 64, 64, 8), dtype=torch.float16).transpose(2, 3)), ValueError),  # strided
        (dict(lse=torch.empty((1, 64, 8), dtype=torch.float32)), ValueError),       # [B, M, H] instead of [B, H, M]
        (dict(lse=torch.empty((1, 8, 64), dtype=torch.float16)), TypeError),
        (dict(out=good_o.numpy()), TypeError),                                      # not a tensor
    ]
    for kw, err in bad:
        with pytest.raises(err):
            binding.sel_attn_fwd(q, k, v, idx, 32, **kw)
        with pytest.raises(err):
            binding.nsa_sel_fwd(q, k, v, idx, 32, **kw)     # the tensor form of the entry point
    # Good buffers get as far as the GPU check (these are host tensors).
    with pytest.raises(ValueError, match="GPU"):
        binding.sel_attn_fwd(q, k, v, idx, 32, out=good_o, lse=good_l)
    with pytest.raises(ValueError):
        binding.dense_attn_fwd(q, k, v, out=torch.empty((1, 64, 8, 32), dtype=torch.float16))
    with pytest.raises(ValueError):
        binding.window_attn_fwd(q, k, v, 8, 0, lse=torch.empty((1, 8, 65), dtype=torch.float32))
    with pytest.raises(ValueError):
        binding.topk_blocks(torch.zeros((1, 64, 2, 2), dtype=torch.float32), 32, 4,
                            out=torch.empty((1, 64, 2, 3), dtype=torch.int32))
    with pytest.raises(TypeError):
        binding.topk_blocks(torch.zeros((1, 64, 2, 2), dtype=torch.float32), 32, 4,
                            out=torch.empty((1, 64, 2, 4), dtype=torch.int64))


def test_bwd_wrapper_rejects_bad_workspace():
    import torch
    q, k, v, idx = _cpu_inputs()
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, 64), dtype=torch.float32)
    for ws, err in ((torch.empty(1024, dtype=torch.int8), TypeError),
                    (torch.empty((4, 256), dtype=torch.uint8), ValueError),
                    (torch.empty(2048, dtype=torch.uint8)[::2], ValueError)):
        with pytest.raises(err):
            binding.sel_attn_bwd(q, k, v, idx, o, lse, o, 32, workspace=ws)


def test_autograd_wrapper_checks_like_the_forward():
    # sel_attn runs sel_attn_fwd first, with the same checks: host tensors stop at
    # the GPU check, and no gradient machinery runs before it.
    import torch
    q, k, v, idx = _cpu_inputs()
    q.requires_grad_(True)
    with pytest.raises(ValueError, match="GPU"):
        binding.sel_attn(q, k, v, idx, 32)
    with pytest.raises(TypeError):
        binding.sel_attn(q.detach().float(), k, v, idx, 32)


def test_entry_point_forms_dispatch_on_their_arguments(lib):
    # Fifteen C arguments -> the C entry point (status from the host checks).
    with pytest.raises(binding.NsaSelError):
        binding.nsa_sel_fwd(0, 1, 2, 3, 4, 5, 1, 1, 1, 1, 1, 64, 32, 1, 0)
    # Five tensors-and-block-size arguments -> the tensor form.
    q, k, v, idx = _cpu_inputs()
    with pytest.raises(ValueError, match="GPU"):
        binding.nsa_sel_fwd(q, k, v, idx, 32)


def _bwd_capacity(idx, M, N, H, G, bs, T):
    """Brute-force item and partial-slot counts of the key-major backward pass
    for these index rows, and the bounds the library sizes its workspace with
    (include/nsa_sel_bwd.h: a key block's selecting queries are cut into items
    of qc queries; a block with two or more items writes one partial per
    item)."""
    import numpy as np
    B = idx.shape[0]
    gs = H // G
    NB = -(-N // bs)
    qc = min(2048, max(32, (8192 // gs) // 32 * 32))
    items = parts = 0
    for b in range(B):
        for g in range(G):
            sel = np.zeros((NB, M), bool)
            for m in range(M):
                row = idx[b, m, g]
                ok = (row >= 0) & (row <= m // bs) & (row < NB)
                sel[row[ok], m] = True
            n = -(-sel.sum(axis=1) // qc)
            items += int(n.sum())
            parts += int(n[n >= 2].sum())
    pairs = sum(min(bs, M - c * bs) * min(T, c + 1, NB) for c in range(-(-M // bs)))
    cap = B * G * (NB + -(-pairs // qc))
    pcap = B * G * -(-2 * pairs // qc) + 1
    return items, parts, cap, pcap


@pytest.mark.parametrize("shape", [
    # B, M, N, H, G, bs, T, rule
    (1, 2500, 2500, 16, 1, 64, 8, "uniform"),     # several items per key block
    (2, 300, 300, 16, 2, 64, 5, "uniform"),
    (1, 500, 180, 16, 1, 64, 4, "uniform"),       # M > N
    (1, 200, 333, 6, 2, 32, 6, "uniform"),        # M < N
    (1, 700, 700, 2, 2, 32, 6, "geometric"),
    (1, 640, 640, 1, 1, 32, 40, "dense-rows"),    # T > NB, every causal block (gs = 1: qc = 2048)
    (1, 1100, 1100, 16, 1, 32, 40, "dense-rows"),  # T > NB, qc = 512: blocks with three items
    (1, 1300, 1300, 32, 2, 64, 16, "noisy"),      # repeats, padding, future and out-of-range entries
])
def test_bwd_capacity_bounds_hold(shape):
    """The workspace's item list and partial slots are sized from the sizes
    alone; the counts real index rows produce must stay within them."""
    import numpy as np
    from block_sparse_attention_sel_amd.inputs import Config, block_indices
    B, M, N, H, G, bs, T, rule = shape
    NB = -(-N // bs)
    if rule == "dense-rows":
        c = np.arange(M) // bs
        row = np.arange(T)[None, :]
        idx = np.where(row <= np.minimum(c, NB - 1)[:, None], row, -1).astype(np.int32)
        idx = np.ascontiguousarray(np.broadcast_to(idx[None, :, None, :], (B, M, G, T)))
    elif rule == "noisy":
        rng = np.random.default_rng(3)
        idx = rng.integers(-3, NB + 3, size=(B, M, G, T)).astype(np.int32)
        idx[..., 1] = idx[..., 0]
    else:
        idx = block_indices(Config("c", B=B, M=M, N=N, H=H, G=G, D=64, block_size=bs, T=T, rule=rule, seed=7))
    items, parts, cap, pcap = _bwd_capacity(idx, M, N, H, G, bs, T)
    assert items <= cap and parts <= pcap
    assert items > 0
