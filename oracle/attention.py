"""fp64 CPU oracle for exact scaled dot-product attention, RoPE and paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library.

It is the plain definition, written out in numpy float64 with library matmuls:
the full score matrix is materialised, masked with -inf on the logits, put
through a max-subtracted softmax and multiplied by V.  There is no tiling, no
online softmax and no fusion.  Sources (page title, then section):

* "22 interview questions on attention & transformers" -- "How does
  self-attention work": output of token i is the softmax(q_i.k_j / sqrt(d_k))
  weighted sum of the values; "How does Rotary Position Embedding (RoPE)
  work": rotate q and k in each 2D subspace by theta_pos = pos / base^(2i/d).
* "Transformer Attention Mechanism Interview Deep Dive" -- "Scaled dot-product
  attention" (softmax(QK^T/sqrt(d_k))V), "Causal masking" (mask on the logits
  as -inf before the softmax), the live-coding exercise (row-max subtraction,
  batch/head broadcasting), the KV-cache paragraph and the GQA discussion.
* "Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in
  Code" -- Part 3: fixed-size blocks and per-sequence block tables.

Readings taken where the pages leave a step open (each is listed in the
design notes):
* d_k is the per-head size d_h; the scale is fixed at 1/sqrt(d_h).
* RoPE pairs are adjacent dimensions (2i, 2i+1), i = 0..d_h/2-1, rotated
  counter-clockwise: (x0, x1) -> (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi)
  with phi = pos * base^(-2i/d_h).  The pairing and the sign are conventions
  the pages do not fix (parity between conventions is unpinned); the
  relative-position property holds for either.
* Query row t sits at absolute position pos + t, key s at position s; causal
  visibility is s <= pos + t.
* Grouped-query attention maps query head h to KV head h // (Hq / Hkv).
* lse is the natural log of the sum of exp(scaled logits) of the visible keys.
* A row with no visible key (only possible if pos + t < 0) yields output 0 and
  lse = -inf.
* Decode: sequence b has L_b cached tokens including the current one; token j
  is slot j % block_size of physical block block_table[b][j // block_size];
  the query is rotated at position L_b - 1; cached K is already rotated; all
  L_b keys are visible.
"""

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------- RoPE ----

def rope_inv_freq(d_h, base):
    """base^(-2i/d_h) for pair index i = 0..d_h/2-1, in fp64 (RoPE section of the
    "22 interview questions" page: theta_pos = pos / base^(2i/d))."""
    i = np.arange(d_h // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / F64(d_h))


def apply_rope(x, positions, base):
    """Rotate adjacent pairs (2i, 2i+1) of the last axis of x by phi = pos * inv_i.

    x: [..., n, d_h] float64; positions: [n] integer absolute positions.
    Returns a new array; x is not modified.  base <= 0 means no rotation.
    """
    x = np.asarray(x, dtype=F64)
    if base is None or base <= 0:
        return x.copy()
    d_h = x.shape[-1]
    pos = np.asarray(positions, dtype=np.int64).astype(F64)
    phi = pos[:, None] * rope_inv_freq(d_h, base)[None, :]          # [n, d_h/2]
    c, s = np.cos(phi), np.sin(phi)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ---------------------------------------------------- core definition ----

def sdpa(q, k, v, mask=None):
    """softmax(q k^T / sqrt(d_h) + mask) v with the row max subtracted.

    q [..., T, d], k [..., S, d], v [..., S, dv]; mask broadcastable to
    [..., T, S] with 0 for visible and -inf for hidden entries (additive mask on
    the logits, before the softmax).  Leading axes broadcast.  Returns
    (out [..., T, dv], lse [..., T], probs [..., T, S]) in float64.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    d = q.shape[-1]
    logits = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(F64(d))
    if mask is not None:
        logits = logits + mask
    m = np.max(logits, axis=-1, keepdims=True)
    dead = ~np.isfinite(m)                      # row with no visible key
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(logits - m_safe)                 # exp(-inf) = 0 for hidden keys
    denom = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        probs = np.where(dead, 0.0, e / np.where(dead, 1.0, denom))
        lse = np.where(dead[..., 0], -np.inf, (m_safe + np.log(np.where(dead, 1.0, denom)))[..., 0])
    out = np.matmul(probs, v)
    return out, lse, probs


def causal_mask(q_positions, k_positions):
    """Additive mask: 0 where key position <= query position, -inf elsewhere."""
    qp = np.asarray(q_positions, dtype=np.int64)[:, None]
    kp = np.asarray(k_positions, dtype=np.int64)[None, :]
    return np.where(kp <= qp, 0.0, -np.inf).astype(F64)


def window_mask(q_positions, k_positions, window):
    """Additive causal sliding-window mask: 0 where q - window < k <= q, -inf elsewhere.

    Each query sees the `window` most recent positions up to and including its own
    ("22 interview questions on attention & transformers", What is sparse /
    sliding-window attention: a fixed neighbourhood of size w, read here as the causal
    window of the sliding-window decoders that section names)."""
    qp = np.asarray(q_positions, dtype=np.int64)[:, None]
    kp = np.asarray(k_positions, dtype=np.int64)[None, :]
    return np.where((kp <= qp) & (kp > qp - int(window)), 0.0, -np.inf).astype(F64)


def kv_head_of(h, Hq, Hkv):
    """Contiguous grouped-query map: query head h reads KV head h // (Hq / Hkv)."""
    return h // (Hq // Hkv)


# ------------------------------------------------------------ prefill ----

def _mask(qpos, kpos, causal, window):
    if window:
        return window_mask(qpos, kpos, window)
    return causal_mask(qpos, kpos) if causal else None


def attention(q, k, v, causal=False, rope_base=0.0, pos=0, row_block=None, return_probs=False, window=0):
    """Exact attention over whole tensors.

    q [B,Hq,T,d_h], k and v [B,Hkv,S,d_h] (any float dtype; used as float64).
    RoPE (if rope_base > 0) rotates query row t at position pos + t and key s
    at position s; V is not rotated.  If causal, key s is visible to query t
    iff s <= pos + t; with window = w > 0 (causal sliding window) iff
    pos + t - w < s <= pos + t.  Returns (out [B,Hq,T,d_h], lse [B,Hq,T]) in
    float64, and also the probabilities [B,Hq,T,S] if return_probs.

    row_block bounds memory for long sequences: each (b, h) is processed in
    slices of row_block query rows, every row still getting its full
    materialised softmax over all S keys.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    B, Hq, T, d_h = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0 and k.shape == v.shape[:3] + (k.shape[3],)
    qpos = pos + np.arange(T, dtype=np.int64)
    kpos = np.arange(S, dtype=np.int64)
    kr = apply_rope(k, kpos, rope_base)
    out = np.zeros((B, Hq, T, v.shape[3]), dtype=F64)
    lse = np.zeros((B, Hq, T), dtype=F64)
    probs = np.zeros((B, Hq, T, S), dtype=F64) if return_probs else None
    rb = T if row_block is None else int(row_block)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for t0 in range(0, T, rb):
                t1 = min(T, t0 + rb)
                qr = apply_rope(q[b, h, t0:t1], qpos[t0:t1], rope_base)
                mask = _mask(qpos[t0:t1], kpos, causal, window)
                o, l, p = sdpa(qr, kr[b, g], v[b, g], mask)
                out[b, h, t0:t1] = o
                lse[b, h, t0:t1] = l
                if return_probs:
                    probs[b, h, t0:t1] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def attention_rows(q, k, v, rows, causal=False, rope_base=0.0, pos=0, window=0):
    """The same definition evaluated only at selected query rows.

    rows: int array [n, 3] of (b, h, t).  Each row is rotated at position
    pos + t and attends to all S keys of KV head h // (Hq/Hkv) (masked when
    causal).  Returns (out [n, d_h], lse [n]) in float64.  Used to check very
    large workloads on sampled outputs.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    Hq, Hkv, S = q.shape[1], k.shape[1], k.shape[2]
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    kpos = np.arange(S, dtype=np.int64)
    out = np.zeros((rows.shape[0], v.shape[3]), dtype=F64)
    lse = np.zeros(rows.shape[0], dtype=F64)
    cache = {}
    for i, (b, h, t) in enumerate(rows):
        g = kv_head_of(int(h), Hq, Hkv)
        key = (int(b), g)
        if key not in cache:
            cache = {key: apply_rope(k[b, g].astype(F64), kpos, rope_base)}
        kr = cache[key]
        p = pos + int(t)
        qr = apply_rope(q[b, h, t:t + 1].astype(F64), np.array([p]), rope_base)
        mask = _mask(np.array([p]), kpos, causal, window)
        o, l, _ = sdpa(qr, kr, v[b, g].astype(F64), mask)
        out[i] = o[0]
        lse[i] = l[0]
    return out, lse


# ----------------------------------------------------------- backward ----

def apply_rope_transpose(x, positions, base):
    """The transpose (inverse) of apply_rope: rotate each pair by -phi.  The gradient with
    respect to the unrotated vector is this map applied to the gradient with respect to the
    rotated one (the rotation is orthogonal)."""
    x = np.asarray(x, dtype=F64)
    if base is None or base <= 0:
        return x.copy()
    d_h = x.shape[-1]
    pos = np.asarray(positions, dtype=np.int64).astype(F64)
    phi = pos[:, None] * rope_inv_freq(d_h, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c + x1 * s
    out[..., 1::2] = -x0 * s + x1 * c
    return out


def attention_backward(q, k, v, dout, causal=False, rope_base=0.0, pos=0, window=0):
    """Gradients of sum(dout * attention(q, k, v)) with respect to q, k and v.

    The forward is recomputed in full (scores, mask, softmax) from the inputs; then, with
    S = q' k'^T / sqrt(d_h), P = softmax(S), O = P v (q', k' the rotated inputs):
        dv  = P^T dO
        dP  = dO v^T
        dS  = P * (dP - rowsum(dO * O))        (the softmax Jacobian applied row by row)
        dq' = dS k' / sqrt(d_h),   dk' = dS^T q' / sqrt(d_h)
        dq  = R^T dq',             dk  = R^T dk'  (RoPE is a rotation: its transpose)
    With grouped-query attention a KV head's dk and dv sum over the query heads reading it.
    The pages state only that the backward pass recomputes the scores from the saved
    statistics rather than storing P ("Why is attention O(n^2) ...", Deep dive:
    FlashAttention; "Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in
    Code", Part 2); the derivatives are the standard chain rule of the forward.
    Returns (dq [B,Hq,T,d_h], dk [B,Hkv,S,d_h], dv [B,Hkv,S,d_h]) in float64.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    dout = np.asarray(dout, dtype=F64)
    B, Hq, T, d_h = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    qpos = pos + np.arange(T, dtype=np.int64)
    kpos = np.arange(S, dtype=np.int64)
    kr = apply_rope(k, kpos, rope_base)
    mask = _mask(qpos, kpos, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    scale = 1.0 / np.sqrt(F64(d_h))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qr = apply_rope(q[b, h], qpos, rope_base)
            o, _, p = sdpa(qr, kr[b, g], v[b, g], mask)
            do = dout[b, h]
            dv[b, g] += p.T @ do
            dp = do @ v[b, g].T
            delta = np.sum(do * o, axis=-1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, h] = apply_rope_transpose(ds @ kr[b, g] * scale, qpos, rope_base)
            dk[b, g] += apply_rope_transpose(ds.T @ qr * scale, kpos, rope_base)
    return dq, dk, dv


def attention_backward_sampled(q, k, v, dout, b, g, keys, rows, causal=False, rope_base=0.0, pos=0, window=0):
    """Selected entries of attention_backward for one batch index b and one KV head g:
    dk and dv at key positions `keys` (summed over the query heads that read g), and dq at
    (h, t) pairs `rows` (h among those heads).  The same chain rule as attention_backward,
    evaluated only for the requested rows and columns of the probability matrix of each
    query head of the group; used to check full-size results entry by entry.
    Returns (dq [len(rows), d_h], dk [len(keys), d_h], dv [len(keys), d_h]) in float64."""
    q = np.asarray(q)
    Hq, T, d_h = q.shape[1], q.shape[2], q.shape[3]
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    qpos = pos + np.arange(T, dtype=np.int64)
    kpos = np.arange(S, dtype=np.int64)
    kr = apply_rope(np.asarray(k[b, g], dtype=F64), kpos, rope_base)
    vg = np.asarray(v[b, g], dtype=F64)
    mask = _mask(qpos, kpos, causal, window)
    scale = 1.0 / np.sqrt(F64(d_h))
    dq = np.zeros((len(rows), d_h))
    dk = np.zeros((len(keys), d_h))
    dv = np.zeros((len(keys), d_h))
    for h in range(g * G, (g + 1) * G):
        qr = apply_rope(np.asarray(q[b, h], dtype=F64), qpos, rope_base)
        o, _, p = sdpa(qr, kr, vg, mask)
        do = np.asarray(dout[b, h], dtype=F64)
        delta = np.sum(do * o, axis=-1, keepdims=True)
        # columns `keys` of P and dS
        ds_cols = p[:, keys] * (do @ vg[keys].T - delta)
        dv += p[:, keys].T @ do
        dk += ds_cols.T @ qr * scale
        for n, (hh, t) in enumerate(rows):
            if hh != h:
                continue
            ds_row = p[t] * (vg @ do[t] - delta[t])
            dq[n] = ds_row @ kr * scale
        del p
    dk = apply_rope_transpose(dk, keys, rope_base)
    for n, (hh, t) in enumerate(rows):
        dq[n] = apply_rope_transpose(dq[n][None], [pos + t], rope_base)[0]
    return dq, dk, dv


# ------------------------------------------------------------- decode ----

def prefill_paged(q, k_cache, v_cache, block_table, seq_lens, block_size, rope_base=0.0, heads=None):
    """Prefill of the last T tokens of each sequence against its block-tabled cache
    ("Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in Code", Part 3).

    q [N, Hq, T, d_h]; caches [num_blocks, Hkv, block_size, d_h]; block_table [N, max_blocks];
    seq_lens [N] (tokens per sequence, the new ones included).  Query row t of sequence b sits
    at position L_b - T + t and is rotated there; cached K is used as stored (already rotated);
    key s is visible iff s <= L_b - T + t.  Returns (out [N, Hq, T, d_h], lse [N, Hq, T]);
    with heads given, only those query heads, in that order (for sampling large cases).
    """
    q = np.asarray(q, dtype=F64)
    N, Hq, T, d_h = q.shape
    Hkv = k_cache.shape[1]
    heads = list(range(Hq)) if heads is None else list(heads)
    out = np.zeros((N, len(heads), T, v_cache.shape[3]), dtype=F64)
    lse = np.zeros((N, len(heads), T), dtype=F64)
    for b in range(N):
        L = int(seq_lens[b])
        kb = gather_paged(k_cache, block_table[b], L, block_size).astype(F64)   # [Hkv, L, d]
        vb = gather_paged(v_cache, block_table[b], L, block_size).astype(F64)
        qpos = (L - T) + np.arange(T, dtype=np.int64)
        mask = causal_mask(qpos, np.arange(L, dtype=np.int64))
        for i, h in enumerate(heads):
            g = kv_head_of(h, Hq, Hkv)
            qr = apply_rope(q[b, h], qpos, rope_base)
            o, l, _ = sdpa(qr, kb[g], vb[g], mask)
            out[b, i] = o
            lse[b, i] = l
    return out, lse


def gather_paged(cache, block_table, seq_len, block_size):
    """Contiguous copy of one sequence's cached rows.

    cache [num_blocks, Hkv, block_size, d_h]; token j is slot j % block_size of
    physical block block_table[j // block_size].  Returns [Hkv, seq_len, d_h]
    with the cache's own dtype (a pure copy, so exact).
    """
    j = np.arange(int(seq_len), dtype=np.int64)
    phys = np.asarray(block_table, dtype=np.int64)[j // block_size]
    slot = j % block_size
    rows = np.asarray(cache)[phys, :, slot, :]          # [L, Hkv, d_h]
    return np.ascontiguousarray(np.swapaxes(rows, 0, 1))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, block_size, rope_base=0.0):
    """One decode step over a block-tabled KV cache.

    q [N, Hq, d_h]; k_cache, v_cache [num_blocks, Hkv, block_size, d_h];
    block_table [N, max_blocks] int; seq_lens [N] (number of cached tokens,
    current one included).  The query of sequence b is rotated at position
    L_b - 1; cached K is used as stored (already rotated); all L_b keys are
    visible.  Returns (out [N, Hq, d_h], lse [N, Hq]) in float64.
    """
    q = np.asarray(q, dtype=F64)
    N, Hq, d_h = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    out = np.zeros((N, Hq, d_h), dtype=F64)
    lse = np.zeros((N, Hq), dtype=F64)
    for b in range(N):
        L = int(seq_lens[b])
        if L <= 0:
            lse[b] = -np.inf
            continue
        kb = gather_paged(k_cache, block_table[b], L, block_size).astype(F64)   # [Hkv, L, d]
        vb = gather_paged(v_cache, block_table[b], L, block_size).astype(F64)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qr = apply_rope(q[b, h][None, :], np.array([L - 1]), rope_base)
            o, l, _ = sdpa(qr, kb[g], vb[g], None)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


# ---------------------------------------------------------------- fp8 ----

def fp8_e4m3_decode(codes):
    """Values of 8-bit floating-point codes in the E4M3 format of the OCP 8-bit floating point
    specification (the fp8 operand format of gfx950's matrix cores): sign bit, 4-bit exponent
    with bias 7, 3-bit mantissa; exponent 0 encodes subnormals (m/8)*2^-6; S.1111.111 is NaN
    and there is no infinity, so the largest finite magnitude is 1.75*2^8 = 448.  The pages
    name FP8 only as a feature of newer hardware ("Why is attention O(n^2) ...", later
    FlashAttention versions); the format is this reading."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(F64)))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def attention_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal=False, pos=0):
    """Exact attention on fp8 inputs, the values being code * scale per tensor: q8 [B,Hq,T,d_h],
    k8 [B,Hkv,S,d_h] and V given transposed, vt8 [B,Hkv,d_h,S] (uint8 codes).  q and k are
    taken as already rotated (no RoPE).  Returns attention(q, k, v, causal, pos=pos) in fp64."""
    q = fp8_e4m3_decode(q8) * F64(q_scale)
    k = fp8_e4m3_decode(k8) * F64(k_scale)
    v = np.swapaxes(fp8_e4m3_decode(vt8), -1, -2) * F64(v_scale)
    return attention(q, k, v, causal=causal, pos=pos)


# ------------------------------------------------------------ metrics ----

def max_abs(got, ref):
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def rel_rms(got, ref):
    """||got - ref||_2 / ||ref||_2 over the whole tensor."""
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    return num / den if den > 0 else num
