"""libattn: exact scaled dot-product attention for MI355X (gfx950).

The compute path is the C-ABI library libattn.so (hand-written HIP kernels); this
package only builds it and binds its entry points with the same names.
"""

from ._lib import (ATTN_BF16, ATTN_ERR_HIP, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,  # noqa: F401
                   ATTN_ERR_WORKSPACE, ATTN_F32, ATTN_OK, EXPORTED, LIB, LIB_PATH, AttnError,
                   attn_decode_paged, attn_decode_workspace_bytes, attn_fwd, attn_paged_gather,
                   attn_status_str)
