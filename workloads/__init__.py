"""Seeded synthetic workloads for the attention path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the fp64 oracle's tests and
the HIP path's tests/bench can use it without sharing any method code.

Workloads (shapes follow the typical figures the pages quote: 8-32 heads,
head size 64-128, 4-8 KV heads for grouped-query attention, d = 4096; see
"22 interview questions on attention & transformers", the multi-head and
head-dimension answers, and "Transformer Attention Mechanism Interview Deep
Dive", the variants table and the GQA paragraph after it):

  small_f32    single-head non-causal fp32, T=S=128, d_h=64, no RoPE
  mha2k        causal MHA prefill bf16, B=4, Hq=Hkv=32, T=S=2048, d_h=128, RoPE 1e4
  gqa8k        causal GQA prefill bf16, B=2, Hq=32, Hkv=8, T=S=8192, RoPE 1e4
  gqa32k       long-context causal GQA bf16, B=1, Hq=32, Hkv=8, T=S=32768,
               sigma=0.5, RoPE 5e5 (past the T ~ 6d crossover for d=4096 that
               "Why is attention O(n^2) ..." gives in its 30-second answer)
  decode64     paged decode bf16, 64 sequences of one query token, context
               lengths uniform in [512, 8192], Hq=32, Hkv=8, d_h=128, 16-token
               blocks placed by a seeded random permutation of one pool

Generation recipe: torch.Generator('cpu').manual_seed(seed); torch.randn in
fp32 drawn in the order Q, K, V, multiplied by sigma, then rounded to the
storage dtype with round-to-nearest-even (.to(torch.bfloat16)).
"""


import numpy as np
import torch

# name -> parameters.  "seed" is fixed per workload.
CONFIGS = {
    # prefill of 1024 new tokens per sequence over a paged cache whose first 6144 tokens are
    # one shared prefix (chunked prefill with a prefix cache)
    "prefix8": dict(num_seqs=8, Hq=32, Hkv=8, d_h=128, T=1024, prefix_len=6144, extra_lens=[0] * 8,
                    rope_base=10000.0, sigma=1.0, seed=6),
    "small_f32": dict(kind="fwd", dtype="f32", B=1, Hq=1, Hkv=1, T=128, S=128, d_h=64,
                      causal=False, rope_base=0.0, pos=0, sigma=1.0, seed=1),
    "mha2k": dict(kind="fwd", dtype="bf16", B=4, Hq=32, Hkv=32, T=2048, S=2048, d_h=128,
                  causal=True, rope_base=10000.0, pos=0, sigma=1.0, seed=2),
    "gqa8k": dict(kind="fwd", dtype="bf16", B=2, Hq=32, Hkv=8, T=8192, S=8192, d_h=128,
                  causal=True, rope_base=10000.0, pos=0, sigma=1.0, seed=3),
    "gqa32k": dict(kind="fwd", dtype="bf16", B=1, Hq=32, Hkv=8, T=32768, S=32768, d_h=128,
                   causal=True, rope_base=500000.0, pos=0, sigma=0.5, seed=4),
    "decode64": dict(kind="decode", dtype="bf16", num_seqs=64, Hq=32, Hkv=8, d_h=128,
                     block_size=16, len_lo=512, len_hi=8192, rope_base=10000.0,
                     sigma=1.0, seed=5),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _TORCH_DTYPE[name]


def make_fwd_inputs(B, Hq, Hkv, T, S, d_h, dtype="bf16", sigma=1.0, seed=0, **_):
    """Q [B,Hq,T,d_h], K and V [B,Hkv,S,d_h], iid N(0, sigma^2), rounded to dtype (CPU tensors)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    td = _TORCH_DTYPE[dtype]
    q = (torch.randn((B, Hq, T, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    k = (torch.randn((B, Hkv, S, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    v = (torch.randn((B, Hkv, S, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    return q, k, v


def make_bwd_inputs(B, Hq, Hkv, T, S, d_h, dtype="bf16", sigma=1.0, seed=0, **_):
    """Q, K, V as make_fwd_inputs (same seed, same draws) followed by the output gradient
    dO [B,Hq,T,d_h] iid N(0, 1) from the same generator, rounded to dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    td = _TORCH_DTYPE[dtype]
    q = (torch.randn((B, Hq, T, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    k = (torch.randn((B, Hkv, S, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    v = (torch.randn((B, Hkv, S, d_h), generator=g, dtype=torch.float32) * sigma).to(td)
    do = torch.randn((B, Hq, T, d_h), generator=g, dtype=torch.float32).to(td)
    return q, k, v, do


def make_fp8_inputs(B, Hq, Hkv, T, S, d_h, sigma=1.0, seed=0, **_):
    """fp8 E4M3 inputs with one scale per tensor.  Q [B,Hq,T,d_h], K and V [B,Hkv,S,d_h] drawn
    as in make_fwd_inputs (fp32 N(0, sigma^2), order Q, K, V); each tensor's scale is its
    largest magnitude / 448 (the largest E4M3 value), its codes are x / scale rounded to
    E4M3 (torch.float8_e4m3fn, nearest even); V is stored transposed, [B,Hkv,d_h,S].
    Returns (q8, k8, vt8) as uint8 CPU tensors and (q_scale, k_scale, v_scale)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    xs = [torch.randn(shape, generator=g, dtype=torch.float32) * sigma
          for shape in ((B, Hq, T, d_h), (B, Hkv, S, d_h), (B, Hkv, S, d_h))]
    xs[2] = xs[2].transpose(-1, -2).contiguous()
    codes, scales = [], []
    for x in xs:
        sc = float(x.abs().max()) / 448.0
        codes.append((x / sc).to(torch.float8_e4m3fn).view(torch.uint8))
        scales.append(sc)
    return tuple(codes), tuple(scales)


def make_decode_inputs(num_seqs, Hq, Hkv, d_h, block_size=16, len_lo=512, len_hi=8192,
                       dtype="bf16", sigma=1.0, seed=0, seq_lens=None, device=None, **_):
    """Paged KV cache for one decode step.

    Draw order: seq_lens = randint(len_lo, len_hi + 1) (inclusive range) unless given;
    N = sum(ceil(L_b / block_size)) physical blocks; perm = randperm(N); sequence b
    owns perm[off_b : off_b + ceil(L_b / block_size)] in order; unused table entries
    are -1.  Then q [num_seqs,Hq,d_h], k_cache and v_cache [N,Hkv,block_size,d_h]
    iid N(0, sigma^2), rounded to dtype.  Every slot of the pool is drawn, including
    the slots past each sequence's length in its last block.  With `device` given, q and
    the caches are drawn there by a generator of that device seeded with seed + 1
    (for caches too large to draw on the host); lengths and tables stay host-drawn.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    td = _TORCH_DTYPE[dtype]
    if seq_lens is None:
        seq_lens = torch.randint(len_lo, len_hi + 1, (num_seqs,), generator=g, dtype=torch.int64)
    else:
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    nblk = [(int(L) + block_size - 1) // block_size for L in seq_lens.tolist()]
    num_blocks = sum(nblk)
    max_blocks = max(nblk) if nblk else 0
    perm = torch.randperm(num_blocks, generator=g)
    block_table = torch.full((num_seqs, max(max_blocks, 1)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(nblk):
        block_table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    kw = {}
    if device is not None:
        g = torch.Generator(device).manual_seed(int(seed) + 1)
        kw = dict(device=device)
    q = (torch.randn((num_seqs, Hq, d_h), generator=g, dtype=torch.float32, **kw) * sigma).to(td)
    k_cache = (torch.randn((num_blocks, Hkv, block_size, d_h), generator=g,
                           dtype=torch.float32, **kw) * sigma).to(td)
    v_cache = (torch.randn((num_blocks, Hkv, block_size, d_h), generator=g,
                           dtype=torch.float32, **kw) * sigma).to(td)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                seq_lens=seq_lens.to(torch.int32), block_size=block_size,
                num_blocks=num_blocks, max_blocks_per_seq=block_table.shape[1])


def make_prefill_paged_inputs(num_seqs, Hq, Hkv, d_h, T, prefix_len, extra_lens, block_size=16, dtype="bf16",
                              sigma=1.0, seed=0, shared=True, device=None, **_):
    """Paged caches for a prefill of the last T tokens of each sequence, the sequences
    starting with a common prefix of prefix_len tokens.

    Sequence b holds prefix_len + extra_lens[b] + T tokens.  With shared=True the
    prefix_len // block_size full prefix blocks are one set of physical blocks named by
    every table; the rest of the prefix (a partial block) is copied into each sequence's
    own first block.  With shared=False every sequence has private copies of the same
    values.  Draw order (generator seeded with seed, on `device` if given): prefix K and V
    [Hkv, prefix_len, d_h], then per sequence its own K and V [Hkv, extra + T, d_h], then
    q [num_seqs, Hq, T, d_h], all N(0, sigma^2) rounded to dtype; then the pool
    permutation from a host generator seeded with seed + 1.
    """
    td = _TORCH_DTYPE[dtype]
    dev = device if device is not None else "cpu"
    g = torch.Generator(dev).manual_seed(int(seed))
    bs = block_size
    lens = [prefix_len + int(e) + T for e in extra_lens]

    def draw(shape):
        return (torch.randn(shape, generator=g, dtype=torch.float32, device=dev) * sigma).to(td)

    pk, pv = draw((Hkv, prefix_len, d_h)), draw((Hkv, prefix_len, d_h))
    own = [(draw((Hkv, L - prefix_len, d_h)), draw((Hkv, L - prefix_len, d_h))) for L in lens]
    q = draw((num_seqs, Hq, T, d_h))

    nshared = prefix_len // bs if shared else 0
    nblk = [(L + bs - 1) // bs for L in lens]
    num_blocks = nshared + sum(n - nshared for n in nblk)
    perm = torch.randperm(num_blocks, generator=torch.Generator("cpu").manual_seed(int(seed) + 1))
    table = torch.full((num_seqs, max(nblk)), -1, dtype=torch.int32)
    off = nshared
    for b in range(num_seqs):
        table[b, :nshared] = perm[:nshared].to(torch.int32)
        n = nblk[b] - nshared
        table[b, nshared:nblk[b]] = perm[off:off + n].to(torch.int32)
        off += n
    k_cache = torch.zeros((num_blocks, Hkv, bs, d_h), dtype=td, device=dev)
    v_cache = torch.zeros_like(k_cache)
    tab = table.to(dev).long()
    for b in range(num_seqs):
        kk, vv = torch.cat([pk, own[b][0]], dim=1), torch.cat([pv, own[b][1]], dim=1)
        j = torch.arange(nshared * bs if b > 0 else 0, lens[b], device=dev)
        phys = tab[b][j // bs]
        k_cache[phys, :, j % bs] = kk[:, j].transpose(0, 1)
        v_cache[phys, :, j % bs] = vv[:, j].transpose(0, 1)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
                seq_lens=torch.tensor(lens, dtype=torch.int32), block_size=bs, num_blocks=num_blocks, T=T)


def prefill_paged_flops(seq_lens, Hq, T, d_h):
    """4*d_h per visible (query, key) pair: query t of sequence b sees L_b - T + t + 1 keys."""
    pairs = sum(T * (int(L) - T) + T * (T + 1) // 2 for L in seq_lens)
    return 4.0 * Hq * pairs * d_h


def fwd_flops(B, Hq, T, S, d_h, causal, **_):
    """Algorithmic FLOPs of one forward: 4*B*Hq*T*S*d_h, halved when causal."""
    f = 4.0 * B * Hq * T * S * d_h
    return f / 2.0 if causal else f


def bwd_flops(B, Hq, T, S, d_h, causal, **_):
    """Algorithmic FLOPs of one backward: the five T x S x d_h products (S recomputed, dP,
    dV, dQ, dK), 10*B*Hq*T*S*d_h, halved when causal (2.5 times the forward)."""
    f = 10.0 * B * Hq * T * S * d_h
    return f / 2.0 if causal else f


def window_flops(B, Hq, T, S, d_h, window, pos=0, **_):
    """Algorithmic FLOPs of one causal sliding-window forward: 4*d_h per visible (query, key)
    pair (QK^T and PV), counted exactly: query t sees keys max(0, pos+t-window+1) ..
    min(S-1, pos+t)."""
    t = np.arange(T, dtype=np.int64) + int(pos)
    hi = np.minimum(t, S - 1)
    lo = np.maximum(0, t - int(window) + 1)
    pairs = int(np.maximum(0, hi - lo + 1).sum())
    return 4.0 * B * Hq * pairs * d_h


def decode_kv_bytes(seq_lens, Hkv, d_h, elem_bytes=2):
    """KV bytes a decode step must read: sum_b L_b * Hkv * d_h * 2 (K and V) * elem_bytes."""
    return int(sum(int(L) for L in seq_lens)) * Hkv * d_h * 2 * elem_bytes


def fwd_io_bytes(B, Hq, Hkv, T, S, d_h, elem_bytes=2, **_):
    """Compulsory HBM bytes of one forward: read Q, K, V once, write O and the fp32 lse."""
    return elem_bytes * (2 * B * Hq * T * d_h + 2 * B * Hkv * S * d_h) + 4 * B * Hq * T


def scaled(cfg, **overrides):
    """Copy of a workload's parameters with some fields replaced (smaller test shapes)."""
    c = dict(cfg)
    c.update(overrides)
    return c


__all__ = ["CONFIGS", "make_fwd_inputs", "make_bwd_inputs", "make_fp8_inputs", "make_decode_inputs", "make_prefill_paged_inputs",
           "fwd_flops", "bwd_flops", "window_flops", "prefill_paged_flops", "decode_kv_bytes",
           "fwd_io_bytes", "scaled", "torch_dtype"]
