"""libattn: exact scaled dot-product attention for MI355X (gfx950).

The compute path is the C-ABI library libattn.so (hand-written HIP kernels); this
package only builds it and binds its entry points with the same names.  The library is
loaded on first use of any binding name; a missing or unloadable libattn.so raises
ImportError then (there is no other implementation to fall back to).
"""

_BINDING_NAMES = ("ATTN_BF16", "ATTN_ERR_HIP", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_SCRATCH", "ATTN_ERR_UNSUPPORTED",
                  "ATTN_ERR_WORKSPACE", "ATTN_F32", "ATTN_OK", "DECODE_STATIC_SCRATCH_BYTES", "EXPORTED", "LIB",
                  "LIB_PATH", "AttnError", "attn_bwd", "attn_bwd_workspace_bytes", "attn_decode_paged",
                  "attn_decode_paged_static", "attn_decode_workspace_bytes", "attn_fwd", "attn_fwd_fp8",
                  "attn_fwd_workspace_bytes",
                  "attn_fwd_window", "attn_paged_gather", "attn_prefill_paged", "attn_status_str")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
