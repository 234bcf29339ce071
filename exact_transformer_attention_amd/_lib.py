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

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP, ATTN_ERR_SCRATCH = range(6)
# bytes of device scratch attn_decode_paged_static holds per GPU (ATTN_DECODE_STATIC_SCRATCH_BYTES)
DECODE_STATIC_SCRATCH_BYTES = 32 << 20
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = ("attn_fwd", "attn_fwd_window", "attn_fwd_workspace_bytes", "attn_fwd_fp8", "attn_prefill_paged", "attn_decode_paged",
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
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i64, vp, sz, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, f32, i64, vp, sz, i32,
                                    vp]
    lib.attn_fwd_window.restype = i32
    lib.attn_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64, f32, i64, i32]
    lib.attn_fwd_workspace_bytes.restype = sz
    lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                       i32, vp]
    lib.attn_prefill_paged.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                      vp, sz, i32, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged_static.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                             i32, vp]
    lib.attn_decode_paged_static.restype = i32
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


def _tensor(t, name, dim=None, shape=None, dtype=None):
    """Structure of one tensor argument: dimensions, shape, dtype, contiguity."""
    import torch
    _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    if dim is not None:
        _require(t.dim() == dim, f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if shape is not None:
        _require(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None:
        _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def _on_device(named):
    """Every tensor argument on one GPU (checked after the structure, before any C call)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        _require(t.is_cuda, f"{name} must be a device (GPU) tensor")
        dev = t.device if dev is None else dev
        _require(t.device == dev, f"{name} is on {t.device}, other arguments on {dev}")


def _fwd_buffers(q, k, v, out, lse, want_lse, check_device=True):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _tensor(t, n, dim=4)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    _require(k.shape[0] == B and v.shape == k.shape and k.shape[3] == d, "q, k, v shapes do not match")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _tensor(out, "out", shape=q.shape, dtype=q.dtype)
    if lse is not None:
        _tensor(lse, "lse", shape=(B, Hq, T), dtype=torch.float32)
    if check_device:
        _on_device((("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)))
    return out, lse, (B, Hq, Hkv, T, S, d)


def _paged_args(q, k_cache, v_cache, block_table, seq_lens, block_size, qdim):
    import torch
    _tensor(q, "q", dim=qdim)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _tensor(t, n, dim=4, dtype=q.dtype)
    N, d = q.shape[0], q.shape[-1]
    _require(k_cache.shape == v_cache.shape and k_cache.shape[2] == block_size and k_cache.shape[3] == d,
             "caches must be [num_blocks, Hkv, block_size, d_h] like q")
    _tensor(block_table, "block_table", dim=2, dtype=torch.int32)
    _tensor(seq_lens, "seq_lens", shape=(N,), dtype=torch.int32)
    _require(block_table.shape[0] == N, "block_table must have one row per sequence")


def attn_fwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, causal=False, window=0, rope_base=0.0, pos=0,
                             dtype_code=ATTN_BF16):
    return int(LIB.attn_fwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, int(bool(causal)), int(window),
                                            float(rope_base), int(pos), dtype_code))


def _fwd_workspace(q, workspace, dims, causal, window, rope_base, pos):
    """The workspace argument of attn_fwd / attn_fwd_window as (pointer, bytes): None asks the
    library (a buffer is allocated here when it wants one), False passes none, a 1-D device
    tensor is passed as it is."""
    import torch
    B, Hq, Hkv, T, S, d = dims
    if workspace is False:
        return None, 0
    if workspace is None:
        need = attn_fwd_workspace_bytes(B, Hq, Hkv, T, S, d, causal, window, rope_base, pos, _dtype_code(q))
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _tensor(workspace, "workspace", dim=1)
    _on_device((("q", q), ("workspace", workspace)))
    return workspace, workspace.numel() * workspace.element_size()


def attn_fwd(q, k, v, causal=False, rope_base=0.0, pos=0, out=None, lse=None, want_lse=True,
             workspace=None, stream=None):
    """Exact attention.  q [B,Hq,T,d_h], k/v [B,Hkv,S,d_h] contiguous device tensors of one
    dtype (bf16 or fp32).  Returns (out, lse) with out like q and lse fp32 [B,Hq,T]
    (None if want_lse is False and no lse buffer was given).  workspace: None (one is
    allocated here when attn_fwd_workspace_bytes asks for it: the keys are then rotated once
    ahead of the prefill), False (none: keys rotated inside the prefill), or a 1-D device
    tensor (used when it holds B*Hkv*S*d_h*2 bytes)."""
    out, lse, dims = _fwd_buffers(q, k, v, out, lse, want_lse)
    B, Hq, Hkv, T, S, d = dims
    ws, ws_bytes = _fwd_workspace(q, workspace, dims, causal, 0, rope_base, pos)
    st = LIB.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                      int(bool(causal)), float(rope_base), int(pos), _ptr(ws), ws_bytes, _dtype_code(q),
                      _stream(stream))
    _check(st, "attn_fwd")
    return out, lse


def attn_fwd_window(q, k, v, window, rope_base=0.0, pos=0, out=None, lse=None, want_lse=True, workspace=None,
                    stream=None):
    """Causal sliding-window attention: query row t sees keys pos + t - window < s <= pos + t.
    Same tensors, workspace and results as attn_fwd."""
    out, lse, dims = _fwd_buffers(q, k, v, out, lse, want_lse)
    B, Hq, Hkv, T, S, d = dims
    ws, ws_bytes = _fwd_workspace(q, workspace, dims, True, window, rope_base, pos)
    st = LIB.attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                             int(window), float(rope_base), int(pos), _ptr(ws), ws_bytes, _dtype_code(q),
                             _stream(stream))
    _check(st, "attn_fwd_window")
    return out, lse


def attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal=False, pos=0, out=None, lse=None, want_lse=True,
                 stream=None):
    """Exact attention on fp8 (E4M3) inputs: q8 [B,Hq,T,d_h], k8 [B,Hkv,S,d_h] and V transposed
    vt8 [B,Hkv,d_h,S], uint8 (or float8_e4m3fn) device tensors of codes, value = code * scale.
    Returns (out bf16 [B,Hq,T,d_h], lse fp32 [B,Hq,T])."""
    import torch
    for t, n in ((q8, "q8"), (k8, "k8"), (vt8, "vt8")):
        _tensor(t, n, dim=4)
        _require(t.element_size() == 1, f"{n} must hold one-byte codes")
    B, Hq, T, d = q8.shape
    Hkv, S = k8.shape[1], k8.shape[2]
    _require(k8.shape == (B, Hkv, S, d) and vt8.shape == (B, Hkv, d, S), "q8, k8, vt8 shapes do not match")
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q8.device)
    _tensor(out, "out", shape=(B, Hq, T, d), dtype=torch.bfloat16)
    if lse is not None:
        _tensor(lse, "lse", shape=(B, Hq, T), dtype=torch.float32)
    _on_device((("q8", q8), ("k8", k8), ("vt8", vt8), ("out", out), ("lse", lse)))
    st = LIB.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(out), _ptr(lse), B, Hq, Hkv, T, S, d,
                          int(bool(causal)), float(q_scale), float(k_scale), float(v_scale), int(pos),
                          _stream(stream))
    _check(st, "attn_fwd_fp8")
    return out, lse


def attn_prefill_paged(q, k_cache, v_cache, block_table, seq_lens, block_size=16, rope_base=0.0, out=None,
                       lse=None, want_lse=True, stream=None):
    """Prefill of the last T tokens of each sequence over a paged cache.  q [N,Hq,T,d_h];
    caches [num_blocks,Hkv,block_size,d_h] of q's dtype; block_table [N,max_blocks] int32;
    seq_lens [N] int32 (all device tensors).  Returns (out [N,Hq,T,d_h], lse [N,Hq,T])."""
    import torch
    _paged_args(q, k_cache, v_cache, block_table, seq_lens, block_size, 4)
    N, Hq, T, d = q.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((N, Hq, T), dtype=torch.float32, device=q.device)
    _tensor(out, "out", shape=q.shape, dtype=q.dtype)
    if lse is not None:
        _tensor(lse, "lse", shape=(N, Hq, T), dtype=torch.float32)
    _on_device((("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                ("seq_lens", seq_lens), ("out", out), ("lse", lse)))
    st = LIB.attn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                block_size, N, Hq, Hkv, d, T, block_table.shape[1], num_blocks, float(rope_base),
                                _ptr(out), _ptr(lse), _dtype_code(q), _stream(stream))
    _check(st, "attn_prefill_paged")
    return out, lse


def attn_decode_workspace_bytes(num_seqs, Hq, Hkv, d_h, max_blocks_per_seq, block_size=16):
    return int(LIB.attn_decode_workspace_bytes(num_seqs, Hq, Hkv, d_h, max_blocks_per_seq, block_size))


def _workspace(ws, need, name="workspace"):
    _tensor(ws, name, dim=1)
    _require(ws.numel() * ws.element_size() >= need, f"{name} holds {ws.numel() * ws.element_size()} bytes, "
                                                      f"{need} needed")


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, block_size=16, rope_base=0.0,
                      out=None, lse=None, workspace=None, want_lse=True, stream=None):
    """One decode step over a paged cache.  q [N,Hq,d_h]; caches [num_blocks,Hkv,block_size,d_h]
    of q's dtype; block_table [N,max_blocks] int32; seq_lens [N] int32; workspace a 1-D device
    buffer of at least attn_decode_workspace_bytes(...) bytes (all device tensors).
    Returns (out, lse)."""
    import torch
    _paged_args(q, k_cache, v_cache, block_table, seq_lens, block_size, 3)
    N, Hq, d = q.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    mbps = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    _tensor(out, "out", shape=q.shape, dtype=q.dtype)
    if lse is not None:
        _tensor(lse, "lse", shape=(N, Hq), dtype=torch.float32)
    need = attn_decode_workspace_bytes(N, Hq, Hkv, d, mbps, block_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, need)
    _on_device((("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                ("seq_lens", seq_lens), ("out", out), ("lse", lse), ("workspace", workspace)))
    st = LIB.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                               block_size, N, Hq, Hkv, d, mbps, num_blocks, float(rope_base), _ptr(out),
                               _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _dtype_code(q), _stream(stream))
    _check(st, "attn_decode_paged")
    return out, lse


def attn_decode_paged_static(q, k_cache, v_cache, block_table, seq_lens, block_size=16, rope_base=0.0,
                             out=None, lse=None, want_lse=True, stream=None):
    """attn_decode_paged without a workspace: the C entry point keeps the partial results in the
    library's static per-GPU scratch and allocates nothing (pass out, and lse or
    want_lse=False, for a call that allocates nothing here either).  Requests whose workspace
    would exceed DECODE_STATIC_SCRATCH_BYTES fail (RuntimeError).  Calls overlapping in time on
    one GPU share the scratch and race.  Returns (out, lse)."""
    import torch
    _paged_args(q, k_cache, v_cache, block_table, seq_lens, block_size, 3)
    N, Hq, d = q.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    mbps = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    _tensor(out, "out", shape=q.shape, dtype=q.dtype)
    if lse is not None:
        _tensor(lse, "lse", shape=(N, Hq), dtype=torch.float32)
    _on_device((("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                ("seq_lens", seq_lens), ("out", out), ("lse", lse)))
    st = LIB.attn_decode_paged_static(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                      block_size, N, Hq, Hkv, d, mbps, num_blocks, float(rope_base), _ptr(out),
                                      _ptr(lse), _dtype_code(q), _stream(stream))
    _check(st, "attn_decode_paged_static")
    return out, lse


def attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, rope_base=0.0):
    return int(LIB.attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, float(rope_base)))


def attn_bwd(q, k, v, out, lse, dout, causal=False, window=0, rope_base=0.0, pos=0, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradients of attention with respect to q, k, v given the forward's out and lse and the
    output gradient dout.  Same shapes and options as the forward call (window > 0 means the
    causal sliding window of attn_fwd_window).  Returns (dq, dk, dv)."""
    import torch
    _require(out is not None and lse is not None, "the forward's out and lse are required")
    _, _, (B, Hq, Hkv, T, S, d) = _fwd_buffers(q, k, v, out, lse, True, check_device=False)
    _tensor(dout, "dout", shape=q.shape, dtype=q.dtype)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _tensor(t, n, shape=ref.shape, dtype=ref.dtype)
    need = attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d, rope_base)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, need)
    _on_device((("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                ("dv", dv), ("workspace", workspace)))
    st = LIB.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, Hq, Hkv, T, S, d, int(bool(causal)), int(window), float(rope_base), int(pos),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _dtype_code(q),
                      _stream(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv


def attn_paged_gather(cache, block_table, seq_lens, block_size=16, dst=None, stream=None):
    """Contiguous copy [N,Hkv,max_blocks*block_size,d_h] of each sequence's cached rows through
    the decode kernel's own read path (table windows, addresses, staging).  cache
    [num_blocks,Hkv,block_size,d_h] with 256-byte rows; block_table [N,max_blocks] int32;
    seq_lens [N] int32; rows past a sequence keep dst's contents."""
    import torch
    _tensor(cache, "cache", dim=4)
    _tensor(block_table, "block_table", dim=2, dtype=torch.int32)
    num_blocks, Hkv, bs, d = cache.shape
    N, mbps = block_table.shape
    _require(bs == block_size, "cache blocks must hold block_size tokens")
    _tensor(seq_lens, "seq_lens", shape=(N,), dtype=torch.int32)
    if dst is None:
        dst = torch.zeros((N, Hkv, mbps * block_size, d), dtype=cache.dtype, device=cache.device)
    _tensor(dst, "dst", shape=(N, Hkv, mbps * block_size, d), dtype=cache.dtype)
    _on_device((("cache", cache), ("block_table", block_table), ("seq_lens", seq_lens), ("dst", dst)))
    st = LIB.attn_paged_gather(_ptr(cache), _ptr(block_table), _ptr(seq_lens), block_size, N, Hkv, d, mbps,
                               num_blocks, cache.element_size(), _ptr(dst), _stream(stream))
    _check(st, "attn_paged_gather")
    return dst
