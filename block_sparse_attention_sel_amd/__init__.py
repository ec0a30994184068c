"""NSA selection-attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libnsa_sel.so`` built from
``csrc/``; ``nsa_sel_fwd`` here marshals torch tensors into it.
"""

__all__ = ["nsa_sel_fwd", "nsa_sel_fwd_raw", "nsa_sel_status_string", "sel_attn_fwd", "sel_attn_bwd", "sel_attn",
           "load_library", "NsaSelError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
