"""fp64 emulation of the HIP kernels' rounding points, used to derive test tolerances.

A test-side model, not an oracle: it computes attention in float64 except at the few points
where the kernels round to a narrow format, and there it rounds as the kernels do (the value
taken to fp32, then to bf16 or E4M3, nearest even).  The kernels' remaining fp32 effects
(accumulation order, the hardware exp2 and log2) sit near 2^-24 relative and are left out.
Compared with the oracle on a GPU test's own inputs, the emulation predicts the error that
test should see; the bounds in tolerances.py are stated as about twice that prediction.

Rounding points of the kernels:
  forward bf16 (prefill, sliding window, paged prefill, decode):
    q' = RoPE(q) * log2(e) / sqrt(d_h) -> bf16 (the softmax scale and the base-2 change are
    folded into q before it becomes a matrix-core operand);
    k' = RoPE(k) -> bf16 (the prefill rotates at load; decode and paged prefill read keys the
    cache already holds rotated, so no rounding there);
    p = exp2(s - m) -> bf16 as the P V operand, while the normaliser sums p unrounded;
    O = (P V) / l -> bf16.
  backward bf16: q' and k' as above; p = exp2(s - lse2) recomputed from the forward's fp32
    lse; P -> bf16 for dV = P^T dO; dS = p (dP - rowsum(dO O)) -> bf16 for dq' and dk' (the
    forward's bf16 O in the row sum); dq, dk, dv -> bf16.
  forward fp8: the logits are sums of exact products of E4M3 values; p -> E4M3 for P V; O -> bf16.

The reference m: the prefill kernels hold it lazily, so which p they round depends on it.  A
wave owns 32 query rows and walks the keys in 64-key blocks; probabilities are formed against
the current reference, and only when some row of the wave has none yet or a lane's share of a
probability sum passes a cap is the reference of each row whose new maximum lies more than a
margin above it raised to that maximum (the output and sum rescaled).  bf16 prefill: each
32-key half on its own, cap 2^16, margin 8, the new reference rounded up to a 16-bit
significand.  fp8: the whole block, cap 256, margin 3, the reference exact.  A lane holds the
16 keys k of a 32-key half with (k mod 8) div 4 equal to its half of the wave.  This matters
for fp8: against the exact row maximum the largest probability is exactly 1, against a lazy
reference it is any value up to the cap and carries a full E4M3 rounding.  The decode kernel
splits each sequence over waves by a balancing rule; the model takes the exact row maximum
there (its probabilities are bf16, a small term next to q' and the output).
"""

import numpy as np
import torch

import oracle

LOG2E = 1.0 / np.log(2.0)
LN2 = np.log(2.0)


def to_bf16(x):
    """x (float64) rounded to fp32 and then to the nearest bf16, ties to even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def to_e4m3(x):
    """x (float64, |x| <= 448) rounded to fp32 and then to the nearest E4M3 value, ties to even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def visible(T, S, pos, causal, window):
    """[T, S] boolean: key s is seen by query row t (at position pos + t)."""
    qp = pos + np.arange(T)[:, None]
    kp = np.arange(S)[None, :]
    if window:
        return (kp <= qp) & (kp > qp - window)
    if causal:
        return kp <= qp
    return np.ones((T, S), dtype=bool)


def _softmax_rows(s, vis):
    """Row max m (0 for rows with nothing visible), p = exp2(s - m) with hidden keys 0, and
    the live-row flag."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    live = np.isfinite(m)
    m = np.where(live, m, 0.0)
    p = np.where(vis, np.exp2(s - m[:, None]), 0.0)
    return p, m, live


def ceil_sig16(x):
    """x rounded up (towards +inf) to a 16-bit significand."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    e = np.floor(np.log2(np.abs(x[fin])))
    ulp = np.exp2(e - 15)
    out[fin] = np.ceil(x[fin] / ulp) * ulp
    return out


def _lazy_pv(s, v, round_p, step, cap, margin, ref_grid):
    """Blocked P V with the kernels' lazily raised reference.  s [T, S] base-2 logits with
    hidden keys -inf, v [S, d]; `step` keys are handled at a time (the bf16 kernel's 32-key
    half, the fp8 kernel's 64-key block).  Returns (o [T, d] unnormalised, l [T] sum of
    unrounded p, m [T] reference, -inf where nothing was visible)."""
    T, S = s.shape
    m = np.full(T, -np.inf)
    l = np.zeros(T)
    o = np.zeros((T, v.shape[1]))
    # the lane holding key k of a block: 32-key half k div 32, lane half (k mod 8) div 4
    groups = [(np.arange(64) // 32 == hb) & ((np.arange(64) % 8) // 4 == g) for hb in range(2) for g in range(2)]
    wave = np.arange(T) // 32
    for j0 in range(0, S, step):
        sb = s[:, j0:j0 + step]
        nk = sb.shape[1]
        # before a row has a reference its probabilities are formed against 0 and may
        # overflow, as in the kernels, which then take the block maximum
        with np.errstate(over="ignore"):
            p = np.exp2(sb - np.where(np.isfinite(m), m, 0.0)[:, None])
        bad = ~np.isfinite(m)
        for sel in groups:
            if sel[:nk].any():
                bad |= ~(p[:, sel[:nk]].sum(axis=1) <= cap)
        wave_bad = np.bincount(wave, weights=bad)[wave] > 0
        if wave_bad.any():
            tmax = sb.max(axis=1)
            need = wave_bad & (tmax > m + margin)
            m_new = np.where(need, ref_grid(np.where(need, tmax, 0.0)), m)
            with np.errstate(invalid="ignore"):
                alpha = np.where(need, np.exp2(m - m_new), 1.0)
            l *= alpha
            o *= alpha[:, None]
            m = m_new
            p = np.exp2(sb - np.where(np.isfinite(m), m, 0.0)[:, None])
        p = np.where(np.isfinite(sb), p, 0.0)
        l += p.sum(axis=1)
        o += round_p(p) @ v[j0:j0 + nk]
    return o, l, m


def _finish(o, l, m, vscale=1.0):
    live = l > 0
    out = np.where(live[:, None], to_bf16(o * vscale / np.where(live, l, 1.0)[:, None]), 0.0)
    lse = np.where(live, (np.where(live, m, 0.0) + np.log2(np.where(live, l, 1.0))) * LN2, -np.inf)
    return out, lse


def forward_bf16(q, k, v, causal=False, rope_base=0.0, pos=0, window=0, rotate_k=True, lazy=True):
    """Emulated bf16 prefill: q [B,Hq,T,d], k, v [B,Hkv,S,d] (the bf16 inputs as float64).
    rotate_k=False takes k as already rotated (a cache), which the kernel does not round;
    lazy=False takes the exact row maximum as the reference instead of the prefill kernel's
    lazy one.  Returns (out [B,Hq,T,d] on the bf16 grid, lse [B,Hq,T] natural log)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    c = LOG2E / np.sqrt(d)
    vis = visible(T, S, pos, causal, window)
    kr = to_bf16(oracle.apply_rope(k, np.arange(S), rope_base)) if rotate_k else k
    out = np.zeros((B, Hq, T, v.shape[3]))
    lse = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qs = to_bf16(oracle.apply_rope(q[b, h], pos + np.arange(T), rope_base) * c)
            s = np.where(vis, qs @ kr[b, g].T, -np.inf)
            if lazy:
                o, l, m = _lazy_pv(s, v[b, g], to_bf16, 32, 65536.0, 8.0, ceil_sig16)
            else:
                p, m, live = _softmax_rows(s, vis)
                o, l = to_bf16(p) @ v[b, g], p.sum(axis=1)
            out[b, h], lse[b, h] = _finish(o, l, m)
    return out, lse


def decode_bf16(q, k_cache, v_cache, block_table, seq_lens, block_size, rope_base=0.0):
    """Emulated paged decode: q [N,Hq,d], caches [blocks,Hkv,block_size,d].  Each sequence's
    query is rotated at position L - 1 and attends to its L cached (already rotated) keys.
    Returns (out [N,Hq,d], lse [N,Hq])."""
    q = np.asarray(q, dtype=np.float64)
    N, Hq, d = q.shape
    out = np.zeros((N, Hq, d))
    lse = np.full((N, Hq), -np.inf)
    for b in range(N):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        kb = oracle.gather_paged(k_cache, block_table[b], L, block_size).astype(np.float64)[None]
        vb = oracle.gather_paged(v_cache, block_table[b], L, block_size).astype(np.float64)[None]
        o, l = forward_bf16(q[b][None, :, None, :], kb, vb, causal=True, rope_base=rope_base,
                            pos=L - 1, rotate_k=False, lazy=False)
        out[b] = o[0, :, 0]
        lse[b] = l[0, :, 0]
    return out, lse


def backward_bf16(q, k, v, dout, out, lse, causal=False, rope_base=0.0, pos=0, window=0):
    """Emulated bf16 backward, fed the forward's out (bf16 values) and lse (rounded to fp32
    here, as the kernel stores it).  Returns (dq, dk, dv) on the bf16 grid."""
    q, k, v, dout, out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout, out))
    lse = np.asarray(lse, dtype=np.float32).astype(np.float64)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    c = LOG2E / np.sqrt(d)
    vis = visible(T, S, pos, causal, window)
    qpos, kpos = pos + np.arange(T), np.arange(S)
    kr = to_bf16(oracle.apply_rope(k, kpos, rope_base))
    dq = np.zeros_like(q)
    dkr = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qs = to_bf16(oracle.apply_rope(q[b, h], qpos, rope_base) * c)
            live = np.isfinite(lse[b, h])
            lse2 = np.where(live, lse[b, h] * LOG2E, 0.0)
            p = np.where(vis & live[:, None], np.exp2(qs @ kr[b, g].T - lse2[:, None]), 0.0)
            do = dout[b, h]
            dv[b, g] += to_bf16(p).T @ do
            delta = np.sum(do * out[b, h], axis=1)
            ds = to_bf16(p * (do @ v[b, g].T - delta[:, None]))
            dkr[b, g] += ds.T @ qs * LN2            # dS^T q' / sqrt(d) with q' = qs sqrt(d) ln 2
            dq[b, h] = to_bf16(oracle.apply_rope_transpose(ds @ kr[b, g] / np.sqrt(d), qpos, rope_base))
    dk = to_bf16(oracle.apply_rope_transpose(dkr, kpos, rope_base))
    return dq, dk, to_bf16(dv)


def forward_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal=False, pos=0):
    """Emulated fp8 prefill on E4M3 codes (q8 [B,Hq,T,d], k8 [B,Hkv,S,d], vt8 [B,Hkv,d,S]).
    Returns (out [B,Hq,T,d] on the bf16 grid, lse [B,Hq,T])."""
    qc = oracle.fp8_e4m3_decode(q8)
    kc = oracle.fp8_e4m3_decode(k8)
    vc = np.swapaxes(oracle.fp8_e4m3_decode(vt8), -1, -2)
    B, Hq, T, d = qc.shape
    Hkv, S = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    f32 = np.float32
    c2 = float(f32(f32(f32(q_scale) * f32(k_scale)) * f32(LOG2E)) / f32(np.sqrt(d)))
    vis = visible(T, S, pos, causal, 0)
    out = np.zeros((B, Hq, T, d))
    lse = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s = np.where(vis, (qc[b, h] @ kc[b, h // G].T) * c2, -np.inf)
            o, l, m = _lazy_pv(s, vc[b, h // G], to_e4m3, 64, 256.0, 3.0, lambda x: x)
            out[b, h], lse[b, h] = _finish(o, l, m, float(f32(v_scale)))
    return out, lse
