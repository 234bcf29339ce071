"""ctypes binding of libattn's C ABI (include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libattn.so.  Tensors are torch device tensors (PyTorch provides device memory and the
current stream).  There is no fallback: if libattn.so is missing or fails to load,
importing this module raises.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = ("attn_fwd", "attn_fwd_window", "attn_fwd_fp8", "attn_prefill_paged", "attn_decode_paged",
            "attn_decode_workspace_bytes", "attn_bwd", "attn_bwd_workspace_bytes", "attn_paged_gather",
            "attn_status_str")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libattn.so not built at {LIB_PATH}; run "
                          "`python -m exact_transformer_attention_amd.build` (or __graft_entry__.build())")
    # PyTorch ships its own HIP runtime under the same soname as the system one.  Loading
    # torch first makes libattn.so bind to that copy; loaded the other way round, the process
    # holds two runtimes and the streams and device pointers torch hands over are not valid
    # in the one libattn.so calls (its launches then fail).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i64, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, f32, i64, i32, vp]
    lib.attn_fwd_window.restype = i32
    lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                       i32, vp]
    lib.attn_prefill_paged.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                      vp, sz, i32, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_paged_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.attn_paged_gather.restype = i32
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i64, vp]
    lib.attn_fwd_fp8.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, f32,
                             i64, vp, sz, i32, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, f32]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_status_str.argtypes = [i32]
    lib.attn_status_str.restype = ctypes.c_char_p
    return lib


LIB = _load()


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {attn_status_str(status)} (status {status})")


def attn_status_str(status):
    return LIB.attn_status_str(int(status)).decode()


def _check(status, where):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _fwd_buffers(q, k, v, out, lse, want_lse):
    import torch
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    B, Hq, T, d = q.shape
    _require(k.shape[0] == B and v.shape == k.shape and k.shape[3] == d, "shape mismatch")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    for t in (q, k, v):
        _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    Hkv, S = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    if lse is not None:
        _require(lse.shape == (B, Hq, T) and lse.dtype == torch.float32 and lse.is_contiguous(), "bad lse")
    return out, lse, (B, Hq, Hkv, T, S, d)


def attn_fwd(q, k, v, causal=False, rope_base=0.0, pos=0, out=None, lse=None, want_lse=True,
             stream=None):
    """Exact attention.  q [B,Hq,T,d_h], k/v [B,Hkv,S,d_h] contiguous device tensors of one
    dtype (bf16 or fp32).  Returns (out, lse) with out like q and lse fp32 [B,Hq,T]
    (None if want_lse is False and no lse buffer was given)."""
    out, lse, (B, Hq, Hkv, T, S, d) = _fwd_buffers(q, k, v, out, lse, want_lse)
    st = LIB.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                      int(bool(causal)), float(rope_base), int(pos), _dtype_code(q), _stream(stream))
    _check(st, "attn_fwd")
    return out, lse


def attn_fwd_window(q, k, v, window, rope_base=0.0, pos=0, out=None, lse=None, want_lse=True, stream=None):
    """Causal sliding-window attention: query row t sees keys pos + t - window < s <= pos + t.
    Same tensors and results as attn_fwd."""
    out, lse, (B, Hq, Hkv, T, S, d) = _fwd_buffers(q, k, v, out, lse, want_lse)
    st = LIB.attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                             int(window), float(rope_base), int(pos), _dtype_code(q), _stream(stream))
    _check(st, "attn_fwd_window")
    return out, lse


def attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal=False, pos=0, out=None, lse=None, want_lse=True,
                 stream=None):
    """Exact attention on fp8 (E4M3) inputs: q8 [B,Hq,T,d_h], k8 [B,Hkv,S,d_h] and V transposed
    vt8 [B,Hkv,d_h,S], uint8 (or float8_e4m3fn) device tensors of codes, value = code * scale.
    Returns (out bf16 [B,Hq,T,d_h], lse fp32 [B,Hq,T])."""
    import torch
    for t in (q8, k8, vt8):
        _require(t.dim() == 4 and t.element_size() == 1 and t.is_cuda and t.is_contiguous(),
                 "q8, k8, vt8 must be contiguous 4-D one-byte device tensors")
    B, Hq, T, d = q8.shape
    Hkv, S = k8.shape[1], k8.shape[2]
    _require(k8.shape == (B, Hkv, S, d) and vt8.shape == (B, Hkv, d, S), "shape mismatch")
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q8.device)
    _require(out.shape == (B, Hq, T, d) and out.dtype == torch.bfloat16 and out.is_contiguous(), "bad out")
    st = LIB.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                          int(bool(causal)), float(q_scale), float(k_scale), float(v_scale), int(pos),
                          _stream(stream))
    _check(st, "attn_fwd_fp8")
    return out, lse


def attn_prefill_paged(q, k_cache, v_cache, block_table, seq_lens, block_size=16, rope_base=0.0, out=None,
                       lse=None, want_lse=True, stream=None):
    """Prefill of the last T tokens of each sequence over a paged cache.  q [N,Hq,T,d_h];
    caches [num_blocks,Hkv,block_size,d_h]; block_table [N,max_blocks] int32; seq_lens [N]
    int32 (all device tensors).  Returns (out [N,Hq,T,d_h], lse [N,Hq,T])."""
    import torch
    _require(q.dim() == 4, "q must be [N, Hq, T, d_h]")
    N, Hq, T, d = q.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    _require(k_cache.shape == v_cache.shape and k_cache.shape[2] == block_size and k_cache.shape[3] == d,
             "cache shape mismatch")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables must be int32")
    _require(block_table.dim() == 2 and block_table.shape[0] == N and seq_lens.shape == (N,), "table shape")
    for t in (q, k_cache, v_cache, block_table, seq_lens):
        _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((N, Hq, T), dtype=torch.float32, device=q.device)
    st = LIB.attn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                block_size, N, Hq, Hkv, d, T, block_table.shape[1], num_blocks, float(rope_base),
                                _ptr(out), _ptr(lse), _dtype_code(q), _stream(stream))
    _check(st, "attn_prefill_paged")
    return out, lse


def attn_decode_workspace_bytes(num_seqs, Hq, Hkv, d_h, max_blocks_per_seq, block_size=16):
    return int(LIB.attn_decode_workspace_bytes(num_seqs, Hq, Hkv, d_h, max_blocks_per_seq, block_size))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, block_size=16, rope_base=0.0,
                      out=None, lse=None, workspace=None, want_lse=True, stream=None):
    """One decode step over a paged cache.  q [N,Hq,d_h]; caches [num_blocks,Hkv,block_size,d_h];
    block_table [N,max_blocks] int32; seq_lens [N] int32 (all device tensors).
    Returns (out, lse)."""
    import torch
    N, Hq, d = q.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    _require(k_cache.shape == v_cache.shape and k_cache.shape[2] == block_size and k_cache.shape[3] == d,
             "cache shape mismatch")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables must be int32")
    _require(block_table.dim() == 2 and block_table.shape[0] == N and seq_lens.shape == (N,), "table shape")
    for t in (q, k_cache, v_cache, block_table, seq_lens):
        _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    mbps = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(N, Hq, Hkv, d, mbps, block_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = LIB.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                               block_size, N, Hq, Hkv, d, mbps, num_blocks, float(rope_base), _ptr(out),
                               _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _dtype_code(q), _stream(stream))
    _check(st, "attn_decode_paged")
    return out, lse


def attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, rope_base=0.0):
    return int(LIB.attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, float(rope_base)))


def attn_bwd(q, k, v, out, lse, dout, causal=False, window=0, rope_base=0.0, pos=0, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradients of attention with respect to q, k, v given the forward's out and lse and the
    output gradient dout.  Same shapes and options as the forward call (window > 0 means the
    causal sliding window of attn_fwd_window).  Returns (dq, dk, dv)."""
    import torch
    _, _, (B, Hq, Hkv, T, S, d) = _fwd_buffers(q, k, v, out, lse, True)
    _require(dout.shape == q.shape and dout.dtype == q.dtype and dout.is_cuda and dout.is_contiguous(), "bad dout")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        _require(t.shape == ref.shape and t.dtype == ref.dtype and t.is_contiguous(), "bad gradient buffer")
    need = attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d, rope_base)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = LIB.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, Hq, Hkv, T, S, d, int(bool(causal)), int(window), float(rope_base), int(pos),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _dtype_code(q),
                      _stream(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv


def attn_paged_gather(cache, block_table, seq_lens, block_size=16, dst=None, stream=None):
    """Contiguous copy [N,Hkv,max_blocks*block_size,d_h] of each sequence's cached rows via
    the decode kernels' block-table address code.  Rows past a sequence keep dst's contents."""
    import torch
    num_blocks, Hkv, bs, d = cache.shape
    N, mbps = block_table.shape
    if dst is None:
        dst = torch.zeros((N, Hkv, mbps * block_size, d), dtype=cache.dtype, device=cache.device)
    st = LIB.attn_paged_gather(_ptr(cache), _ptr(block_table), _ptr(seq_lens), block_size, N, Hkv, d, mbps,
                               num_blocks, cache.element_size(), _ptr(dst), _stream(stream))
    _check(st, "attn_paged_gather")
    return dst
