"""Thin ctypes binding of libnsa_sel.so and libnsa_gather_probe.so.

``nsa_sel_fwd``, ``nsa_sel_fwd_bf16``, ``nsa_sel_fwd_ws``, ``nsa_sel_fwd_bf16_ws``,
``nsa_sel_fwd_workspace_size``, ``nsa_sel_bwd``, ``nsa_sel_bwd_workspace_size``, ``nsa_sel_bwd_noalloc``, ``nsa_dense_fwd``, ``nsa_window_fwd``,
``nsa_window_fwd_bf16``, ``nsa_topk_blocks`` and ``nsa_sel_status_string``
mirror the C entry points one to one (pointers may be given as ints or as torch tensors);
``sel_attn_fwd``, ``sel_attn_bwd``, ``dense_attn_fwd``, ``window_attn_fwd`` and
``topk_blocks`` are conveniences that check torch tensors, allocate the outputs and call the
entry point on the current stream (the fp16 or bf16 one by the tensors' dtype);
``sel_attn`` joins the forward and the backward as a torch.autograd.Function.
``nsa_gather_probe`` mirrors the measurement probe of include/nsa_gather_probe.h.
All arithmetic happens in the HIP kernels, except that ``sel_attn`` has torch cast
the backward's fp32 gradients to the inputs' dtype; when a library is missing every
call into it raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsa_sel.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libnsa_gather_probe.so")

# Status codes (mirror include/nsa_sel.h).
NSA_SEL_OK = 0
NSA_SEL_ERR_NULL = 1
NSA_SEL_ERR_SHAPE = 2
NSA_SEL_ERR_UNSUPPORTED = 3
NSA_SEL_ERR_ALIGN = 4
NSA_SEL_ERR_RANGE = 5
NSA_SEL_ERR_ALIAS = 6
NSA_SEL_ERR_HIP = 7
NSA_SEL_ERR_WORKSPACE = 8
NSA_SEL_ERR_SCRATCH = 9

EXPORTED = ("nsa_sel_fwd", "nsa_sel_fwd_bf16", "nsa_sel_fwd_unpipelined", "nsa_sel_fwd_workspace_size",
            "nsa_sel_fwd_ws", "nsa_sel_fwd_bf16_ws", "nsa_sel_status_string")
DENSE_EXPORTED = ("nsa_dense_fwd", "nsa_window_fwd", "nsa_window_fwd_bf16")
BWD_EXPORTED = ("nsa_sel_bwd", "nsa_sel_bwd_workspace_size", "nsa_sel_bwd_noalloc")
TOPK_EXPORTED = ("nsa_topk_blocks",)
PROBE_EXPORTED = ("nsa_gather_probe",)

_lib = None
_probe_lib = None


class NsaSelError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(nsa_sel_status_string(status))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    for name in ("nsa_sel_fwd", "nsa_sel_fwd_bf16", "nsa_sel_fwd_unpipelined"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 8 + [vp]
        getattr(lib, name).restype = ci
    for name in ("nsa_sel_fwd_ws", "nsa_sel_fwd_bf16_ws"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 8 + [vp, ctypes.c_size_t, vp]
        getattr(lib, name).restype = ci
    lib.nsa_sel_fwd_workspace_size.argtypes = [ci] * 8 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.nsa_sel_fwd_workspace_size.restype = ci
    lib.nsa_sel_status_string.argtypes = [ci]
    lib.nsa_sel_status_string.restype = ctypes.c_char_p
    lib.nsa_dense_fwd.argtypes = [vp, vp, vp, vp, vp] + [ci] * 6 + [vp]
    lib.nsa_dense_fwd.restype = ci
    for name in ("nsa_window_fwd", "nsa_window_fwd_bf16"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, vp] + [ci] * 8 + [vp]
        getattr(lib, name).restype = ci
    lib.nsa_sel_bwd_workspace_size.argtypes = [ci] * 8 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.nsa_sel_bwd_workspace_size.restype = ci
    lib.nsa_sel_bwd.argtypes = [vp] * 11 + [ctypes.c_size_t] + [ci] * 8 + [vp]
    lib.nsa_sel_bwd.restype = ci
    lib.nsa_sel_bwd_noalloc.argtypes = [vp] * 10 + [ci] * 8 + [vp]
    lib.nsa_sel_bwd_noalloc.restype = ci
    lib.nsa_topk_blocks.argtypes = [vp, vp] + [ci] * 6 + [vp]
    lib.nsa_topk_blocks.restype = ci
    if path == LIB_PATH:
        _lib = lib
    return lib


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _check(t, name: str, dtype, shape=None, device=None):
    """Argument check of a torch tensor handed to an entry point: type, dtype,
    shape, contiguity and (when given) the device of the call.  Raises
    TypeError for a wrong type or dtype and ValueError for the rest; the C ABI
    sees only pointers, so a buffer of the wrong size would be written out of
    bounds."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")


def _require_gpu(**tensors):
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def nsa_sel_status_string(status: int) -> str:
    return load_library().nsa_sel_status_string(int(status)).decode()


def nsa_sel_fwd_raw(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream=0,
                    bf16: bool = False) -> int:
    """Calls the C entry point (nsa_sel_fwd, or nsa_sel_fwd_bf16 when bf16) and
    returns its status code unchanged."""
    lib = load_library()
    fn = lib.nsa_sel_fwd_bf16 if bf16 else lib.nsa_sel_fwd
    return fn(_addr(Q), _addr(K), _addr(V), _addr(block_indices), _addr(O), _addr(LSE),
              int(B), int(M), int(N), int(H), int(G), int(D), int(block_size), int(T),
              ctypes.c_void_p(_addr(stream)))


def nsa_sel_fwd(*args, **kwargs):
    """Two forms of the one entry point.

    ``nsa_sel_fwd(q, k, v, block_indices, block_size, out=None, lse=None,
    stream=None) -> (O, LSE)``: torch tensors (see ``sel_attn_fwd``).

    ``nsa_sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D,
    block_size, T, stream=0) -> None``: the C entry point's own arguments
    (pointers as ints or tensors); raises NsaSelError on a nonzero status."""
    if len(args) + len(kwargs) <= 8 and len(args) <= 5:
        return sel_attn_fwd(*args, **kwargs)
    rc = nsa_sel_fwd_raw(*args, **kwargs)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)
    return None


def nsa_sel_fwd_unpipelined(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream=0) -> None:
    """The verification build of the forward (no copy in flight while LDS is
    read); same arguments as nsa_sel_fwd; raises NsaSelError on a nonzero status."""
    lib = load_library()
    rc = lib.nsa_sel_fwd_unpipelined(_addr(Q), _addr(K), _addr(V), _addr(block_indices), _addr(O), _addr(LSE),
                                     int(B), int(M), int(N), int(H), int(G), int(D), int(block_size), int(T),
                                     ctypes.c_void_p(_addr(stream)))
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def nsa_sel_fwd_bf16(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_sel_fwd_raw(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, bf16=True)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def nsa_sel_fwd_workspace_size_raw(B, M, N, H, G, D, block_size, T):
    """Calls the C entry point; returns (status, bytes)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    rc = lib.nsa_sel_fwd_workspace_size(int(B), int(M), int(N), int(H), int(G), int(D), int(block_size), int(T),
                                        ctypes.byref(n))
    return rc, n.value


def nsa_sel_fwd_workspace_size(B, M, N, H, G, D, block_size, T) -> int:
    """Workspace bytes of nsa_sel_fwd_ws; raises NsaSelError on a nonzero status."""
    rc, n = nsa_sel_fwd_workspace_size_raw(B, M, N, H, G, D, block_size, T)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)
    return n


def nsa_sel_fwd_ws_raw(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, workspace,
                       workspace_bytes, stream=0, bf16: bool = False) -> int:
    """Calls the C entry point (nsa_sel_fwd_ws, or nsa_sel_fwd_bf16_ws when
    bf16) and returns its status code unchanged."""
    lib = load_library()
    fn = lib.nsa_sel_fwd_bf16_ws if bf16 else lib.nsa_sel_fwd_ws
    return fn(_addr(Q), _addr(K), _addr(V), _addr(block_indices), _addr(O), _addr(LSE),
              int(B), int(M), int(N), int(H), int(G), int(D), int(block_size), int(T),
              ctypes.c_void_p(_addr(workspace)), int(workspace_bytes), ctypes.c_void_p(_addr(stream)))


def nsa_sel_fwd_ws(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, workspace, workspace_bytes,
                   stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_sel_fwd_ws_raw(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, workspace,
                            workspace_bytes, stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def nsa_sel_fwd_bf16_ws(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, workspace,
                        workspace_bytes, stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_sel_fwd_ws_raw(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, workspace,
                            workspace_bytes, stream, bf16=True)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def sel_attn_fwd(q, k, v, block_indices, block_size: int, out=None, lse=None, stream=None, workspace=None):
    """q [B,M,H,D], k/v [B,N,G,D] (all fp16 or all bf16), block_indices
    [B,M,G,T] int32, all contiguous CUDA tensors.  Returns (O [B,M,H,D] in the
    input dtype, LSE [B,H,M] fp32).  Runs nsa_sel_fwd_ws (nsa_sel_fwd_bf16_ws)
    with `workspace` (a uint8 CUDA tensor of at least
    nsa_sel_fwd_workspace_size bytes), or with one allocated per call from
    torch's caching allocator."""
    import torch

    et = q.dtype if isinstance(q, torch.Tensor) and q.dtype in (torch.float16, torch.bfloat16) else torch.float16
    for name, t, dt in (("q", q, et), ("k", k, et), ("v", v, et),
                        ("block_indices", block_indices, torch.int32)):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-d {dt} tensor")
        _check(t, name, dt, device=q.device)
    B, M, H, D = q.shape
    _, N, G, _ = k.shape
    T = block_indices.shape[3]
    if (k.shape[0], k.shape[3]) != (B, D) or v.shape != k.shape or tuple(block_indices.shape[:3]) != (B, M, G):
        raise ValueError("inconsistent shapes")
    if out is not None:
        _check(out, "out", et, (B, M, H, D), q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, M), q.device)
    _require_gpu(q=q, k=k, v=v, block_indices=block_indices)
    if out is None:
        out = torch.empty((B, M, H, D), dtype=et, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ws_bytes = nsa_sel_fwd_workspace_size(B, M, N, H, G, D, block_size, T)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or \
            workspace.device != q.device or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if et == torch.bfloat16:
        nsa_sel_fwd_bf16_ws(q, k, v, block_indices, out, lse, B, M, N, H, G, D, block_size, T, workspace,
                            workspace.numel(), stream)
    else:
        nsa_sel_fwd_ws(q, k, v, block_indices, out, lse, B, M, N, H, G, D, block_size, T, workspace,
                       workspace.numel(), stream)
    return out, lse


def nsa_sel_bwd_workspace_size_raw(B, M, N, H, G, D, block_size, T):
    """Calls the C entry point; returns (status, bytes)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    rc = lib.nsa_sel_bwd_workspace_size(int(B), int(M), int(N), int(H), int(G), int(D), int(block_size), int(T),
                                        ctypes.byref(n))
    return rc, n.value


def nsa_sel_bwd_workspace_size(B, M, N, H, G, D, block_size, T) -> int:
    """Workspace bytes of nsa_sel_bwd; raises NsaSelError on a nonzero status."""
    rc, n = nsa_sel_bwd_workspace_size_raw(B, M, N, H, G, D, block_size, T)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)
    return n


def nsa_sel_bwd_raw(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, B, M, N, H, G, D,
                    block_size, T, stream=0) -> int:
    """Calls the C entry point and returns its status code unchanged."""
    lib = load_library()
    return lib.nsa_sel_bwd(_addr(Q), _addr(K), _addr(V), _addr(block_indices), _addr(O), _addr(LSE), _addr(dO),
                           _addr(dQ), _addr(dK), _addr(dV), _addr(workspace), int(workspace_bytes), int(B), int(M),
                           int(N), int(H), int(G), int(D), int(block_size), int(T), ctypes.c_void_p(_addr(stream)))


def nsa_sel_bwd(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, B, M, N, H, G, D,
                block_size, T, stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_sel_bwd_raw(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, B, M, N, H, G,
                         D, block_size, T, stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def nsa_sel_bwd_noalloc_raw(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, B, M, N, H, G, D, block_size, T,
                            stream=0) -> int:
    """Calls the allocation-free C entry point and returns its status code unchanged."""
    lib = load_library()
    return lib.nsa_sel_bwd_noalloc(_addr(Q), _addr(K), _addr(V), _addr(block_indices), _addr(O), _addr(LSE),
                                   _addr(dO), _addr(dQ), _addr(dK), _addr(dV), int(B), int(M), int(N), int(H),
                                   int(G), int(D), int(block_size), int(T), ctypes.c_void_p(_addr(stream)))


def nsa_sel_bwd_noalloc(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, B, M, N, H, G, D, block_size, T,
                        stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_sel_bwd_noalloc_raw(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, B, M, N, H, G, D, block_size, T,
                                 stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def sel_attn_bwd(q, k, v, block_indices, out, lse, dout, block_size: int, workspace=None, stream=None):
    """Gradients of sel_attn_fwd: q/out/dout [B,M,H,D] fp16, k/v [B,N,G,D]
    fp16, block_indices [B,M,G,T] int32, lse [B,H,M] fp32, all contiguous CUDA
    tensors.  workspace: optional uint8 CUDA tensor of at least
    nsa_sel_bwd_workspace_size bytes.  Returns (dQ, dK, dV) in fp32."""
    import torch

    for name, t, dt in (("q", q, torch.float16), ("k", k, torch.float16), ("v", v, torch.float16),
                        ("block_indices", block_indices, torch.int32), ("out", out, torch.float16),
                        ("dout", dout, torch.float16)):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-d {dt} tensor")
        _check(t, name, dt, device=q.device)
    _check(lse, "lse", torch.float32, device=q.device)
    B, M, H, D = q.shape
    _, N, G, _ = k.shape
    T = block_indices.shape[3]
    if ((k.shape[0], k.shape[3]) != (B, D) or v.shape != k.shape or tuple(block_indices.shape[:3]) != (B, M, G)
            or out.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, H, M)):
        raise ValueError("inconsistent shapes")
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, device=q.device)
        if workspace.dim() != 1:
            raise ValueError("workspace must be a 1-d uint8 tensor")
    _require_gpu(q=q, k=k, v=v, block_indices=block_indices, out=out, dout=dout, lse=lse)
    nbytes = nsa_sel_bwd_workspace_size(B, M, N, H, G, D, block_size, T)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif workspace.numel() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel()} bytes; {nbytes} are needed")
    dq = torch.empty((B, M, H, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, N, G, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, N, G, D), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    nsa_sel_bwd(q, k, v, block_indices, out, lse, dout, dq, dk, dv, workspace, workspace.numel(), B, M, N, H, G, D,
                block_size, T, stream)
    return dq, dk, dv


_sel_attn_fn = None


def _sel_attn_function():
    """The torch.autograd.Function behind sel_attn (made on first use, so that
    importing this module does not import torch)."""
    global _sel_attn_fn
    if _sel_attn_fn is None:
        import torch

        class SelAttnFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, block_indices, block_size):
                out, lse = sel_attn_fwd(q, k, v, block_indices, block_size)
                ctx.block_size = block_size
                ctx.save_for_backward(q, k, v, block_indices, out, lse)
                ctx.mark_non_differentiable(lse)
                return out, lse

            @staticmethod
            def backward(ctx, dout, dlse):
                q, k, v, block_indices, out, lse = ctx.saved_tensors
                if q.dtype != torch.float16:
                    raise NotImplementedError("the selection-attention backward takes fp16 tensors")
                dq, dk, dv = sel_attn_bwd(q, k, v, block_indices, out, lse, dout.to(torch.float16).contiguous(),
                                          ctx.block_size)
                return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None

        _sel_attn_fn = SelAttnFunction
    return _sel_attn_fn


def sel_attn(q, k, v, block_indices, block_size: int):
    """sel_attn_fwd as a torch.autograd.Function: returns (out, lse); the
    gradient of out flows to q, k and v through sel_attn_bwd (fp16 tensors;
    the fp32 gradients are cast to the inputs' dtype).  lse is returned
    without a gradient: the backward takes gradients of out only."""
    return _sel_attn_function().apply(q, k, v, block_indices, block_size)


def nsa_dense_fwd_raw(Q, K, V, O, LSE, B, M, N, H, G, D, stream=0) -> int:
    """Calls the dense entry point and returns its status code unchanged."""
    lib = load_library()
    return lib.nsa_dense_fwd(_addr(Q), _addr(K), _addr(V), _addr(O), _addr(LSE), int(B), int(M), int(N), int(H),
                             int(G), int(D), ctypes.c_void_p(_addr(stream)))


def nsa_dense_fwd(Q, K, V, O, LSE, B, M, N, H, G, D, stream=0) -> None:
    """Same arguments as the C entry point; raises NsaSelError on a nonzero status."""
    rc = nsa_dense_fwd_raw(Q, K, V, O, LSE, B, M, N, H, G, D, stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def dense_attn_fwd(q, k, v, out=None, lse=None, stream=None):
    """Dense causal GQA attention: q [B,M,H,D] fp16, k/v [B,N,G,D] fp16,
    contiguous CUDA tensors.  Returns (O [B,M,H,D] fp16, LSE [B,H,M] fp32)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-d float16 tensor")
        _check(t, name, torch.float16, device=q.device)
    B, M, H, D = q.shape
    _, N, G, _ = k.shape
    if (k.shape[0], k.shape[3]) != (B, D) or v.shape != k.shape:
        raise ValueError("inconsistent shapes")
    if out is not None:
        _check(out, "out", torch.float16, (B, M, H, D), q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, M), q.device)
    _require_gpu(q=q, k=k, v=v)
    if out is None:
        out = torch.empty((B, M, H, D), dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    nsa_dense_fwd(q, k, v, out, lse, B, M, N, H, G, D, stream)
    return out, lse


def nsa_window_fwd_raw(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream=0, bf16: bool = False) -> int:
    """Calls nsa_window_fwd (or nsa_window_fwd_bf16) and returns its status code unchanged."""
    lib = load_library()
    fn = lib.nsa_window_fwd_bf16 if bf16 else lib.nsa_window_fwd
    return fn(_addr(Q), _addr(K), _addr(V), _addr(O), _addr(LSE), int(B), int(M), int(N), int(H), int(G), int(D),
              int(left), int(right), ctypes.c_void_p(_addr(stream)))


def nsa_window_fwd(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream=0) -> None:
    rc = nsa_window_fwd_raw(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def nsa_window_fwd_bf16(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream=0) -> None:
    rc = nsa_window_fwd_raw(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream, bf16=True)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def window_attn_fwd(q, k, v, left: int, right: int, out=None, lse=None, stream=None):
    """Sliding-window GQA attention (keys m-left .. m+right, negative =
    unbounded): q [B,M,H,D], k/v [B,N,G,D], all fp16 or all bf16 contiguous CUDA
    tensors.  Returns (O [B,M,H,D] in the input dtype, LSE [B,H,M] fp32)."""
    import torch

    et = q.dtype if isinstance(q, torch.Tensor) and q.dtype in (torch.float16, torch.bfloat16) else torch.float16
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != et or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-d {et} tensor")
        _check(t, name, et, device=q.device)
    B, M, H, D = q.shape
    _, N, G, _ = k.shape
    if (k.shape[0], k.shape[3]) != (B, D) or v.shape != k.shape:
        raise ValueError("inconsistent shapes")
    if out is not None:
        _check(out, "out", et, (B, M, H, D), q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, M), q.device)
    _require_gpu(q=q, k=k, v=v)
    if out is None:
        out = torch.empty((B, M, H, D), dtype=et, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if et == torch.bfloat16:
        nsa_window_fwd_bf16(q, k, v, out, lse, B, M, N, H, G, D, left, right, stream)
    else:
        nsa_window_fwd(q, k, v, out, lse, B, M, N, H, G, D, left, right, stream)
    return out, lse


def nsa_topk_blocks_raw(scores, block_indices, B, M, G, NB, block_size, T, stream=0) -> int:
    """Calls the C entry point and returns its status code unchanged."""
    lib = load_library()
    return lib.nsa_topk_blocks(_addr(scores), _addr(block_indices), int(B), int(M), int(G), int(NB),
                               int(block_size), int(T), ctypes.c_void_p(_addr(stream)))


def nsa_topk_blocks(scores, block_indices, B, M, G, NB, block_size, T, stream=0) -> None:
    rc = nsa_topk_blocks_raw(scores, block_indices, B, M, G, NB, block_size, T, stream)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)


def topk_blocks(scores, block_size: int, T: int, out=None, stream=None):
    """scores [B, M, G, NB] fp32 contiguous CUDA tensor -> block_indices
    [B, M, G, T] int32: per row the T highest-scoring causal blocks, ascending,
    padded with -1 (include/nsa_topk.h)."""
    import torch

    if not isinstance(scores, torch.Tensor) or scores.dtype != torch.float32 or scores.dim() != 4:
        raise TypeError("scores must be a 4-d float32 tensor")
    _check(scores, "scores", torch.float32)
    B, M, G, NB = scores.shape
    if out is not None:
        _check(out, "out", torch.int32, (B, M, G, T), scores.device)
    _require_gpu(scores=scores)
    if out is None:
        out = torch.empty((B, M, G, T), dtype=torch.int32, device=scores.device)
    if stream is None:
        stream = torch.cuda.current_stream(scores.device).cuda_stream
    nsa_topk_blocks(scores, out, B, M, G, NB, block_size, T, stream)
    return out


def load_probe_library(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    global _probe_lib
    if _probe_lib is not None and path == PROBE_LIB_PATH:
        return _probe_lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.nsa_gather_probe.argtypes = [vp, vp, vp, vp] + [ci] * 8 + [vp, ctypes.c_size_t, ctypes.POINTER(ci), vp]
    lib.nsa_gather_probe.restype = ci
    if path == PROBE_LIB_PATH:
        _probe_lib = lib
    return lib


def nsa_gather_probe_raw(K, V, block_indices, staged, B, M, N, H, G, D, block_size, T, stream=0, workspace=None,
                         workspace_bytes=0):
    """Calls the probe's C entry point; returns (status, queries per slot).
    workspace None: the launches of nsa_sel_fwd; a workspace: those of
    nsa_sel_fwd_ws."""
    lib = load_probe_library()
    qps = ctypes.c_int(0)
    rc = lib.nsa_gather_probe(_addr(K), _addr(V), _addr(block_indices), _addr(staged), int(B), int(M), int(N),
                              int(H), int(G), int(D), int(block_size), int(T),
                              ctypes.c_void_p(_addr(workspace) if workspace is not None else None),
                              int(workspace_bytes), ctypes.byref(qps), ctypes.c_void_p(_addr(stream)))
    return rc, qps.value


def nsa_gather_probe(K, V, block_indices, staged, B, M, N, H, G, D, block_size, T, stream=0, workspace=None,
                     workspace_bytes=0) -> int:
    """Queues the probe; raises NsaSelError on a nonzero status and returns the
    number of consecutive queries each wavefront slot carries."""
    rc, qps = nsa_gather_probe_raw(K, V, block_indices, staged, B, M, N, H, G, D, block_size, T, stream, workspace,
                                   workspace_bytes)
    if rc != NSA_SEL_OK:
        raise NsaSelError(rc)
    return qps
