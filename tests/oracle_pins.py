"""Checks that pin the fp64 oracle to facts fixed by the pages and by mathematics.

Each check takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when the fact does not hold.  The test
files run every check against the real oracle, and run the whole battery
against mutated copies to show that each plausible mistake fails at least one
check.
"""

import math

import numpy as np
import torch

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


# ------------------------------------------------------------------------
# Pure-Python scalar brute force (no numpy, no broadcasting) of the
# definition, used only for tiny shapes (T, S <= 8).
# ------------------------------------------------------------------------

def _bf_rotate(vec, p, base):
    d = len(vec)
    out = list(vec)
    if base <= 0:
        return out
    for i in range(d // 2):
        ang = p * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[2 * i], vec[2 * i + 1]
        out[2 * i] = a * c - b * s
        out[2 * i + 1] = a * s + b * c
    return out


def brute_force_attention(q, k, v, causal, base, pos, window=0):
    """q: nested lists [B][Hq][T][d]; k, v: [B][Hkv][S][d].  Returns (out, lse) as lists.
    window > 0: causal sliding window, key s visible iff pos + t - window < s <= pos + t."""
    B, Hq, T, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, S = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    out = [[[None] * T for _ in range(Hq)] for _ in range(B)]
    lse = [[[None] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for t in range(T):
                qt = _bf_rotate(q[b][h][t], pos + t, base)
                logits = []
                for s in range(S):
                    if (causal or window) and s > pos + t:
                        logits.append(None)
                        continue
                    if window and s <= pos + t - window:
                        logits.append(None)
                        continue
                    ks = _bf_rotate(k[b][g][s], s, base)
                    dot = 0.0
                    for i in range(d):
                        dot += qt[i] * ks[i]
                    logits.append(dot / math.sqrt(d))
                vis = [x for x in logits if x is not None]
                if not vis:
                    out[b][h][t] = [0.0] * d
                    lse[b][h][t] = -math.inf
                    continue
                mx = max(vis)
                e = [math.exp(x - mx) if x is not None else 0.0 for x in logits]
                z = sum(e)
                out[b][h][t] = [sum(e[s] * v[b][g][s][j] for s in range(S)) / z for j in range(d)]
                lse[b][h][t] = mx + math.log(z)
    return out, lse


def check_bruteforce_tiny(orc, n_cases=40):
    rng = _rng(1)
    for case in range(n_cases):
        T = int(rng.integers(1, 9))
        S = int(rng.integers(1, 9))
        Hq, Hkv = [(1, 1), (4, 2), (4, 1), (2, 2)][case % 4]
        d = [2, 4, 6, 8][int(rng.integers(0, 4))]
        causal = bool(case % 2)
        base = [0.0, 10000.0, 7.0][case % 3]
        pos = [0, 3][(case // 3) % 2]
        if causal and pos + T - 1 < 0:
            continue
        q = rng.standard_normal((1, Hq, T, d))
        k = rng.standard_normal((1, Hkv, S, d))
        v = rng.standard_normal((1, Hkv, S, d))
        o, l = orc.attention(q, k, v, causal=causal, rope_base=base, pos=pos)
        bo, bl = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal, base, pos)
        bo = np.array(bo, dtype=np.float64)
        bl = np.array(bl, dtype=np.float64)
        assert o.shape == bo.shape, (case, o.shape, bo.shape)
        assert np.allclose(o, bo, rtol=0, atol=1e-12), (case, np.max(np.abs(o - bo)))
        fin = np.isfinite(bl)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.allclose(l[fin], bl[fin], rtol=0, atol=1e-12), case


def check_bruteforce_window(orc, n_cases=30):
    """Causal sliding window against the scalar brute force, windows from 1 to past T."""
    rng = _rng(11)
    for case in range(n_cases):
        T = int(rng.integers(1, 9))
        S = int(rng.integers(1, 9))
        Hq, Hkv = [(1, 1), (4, 2), (2, 1)][case % 3]
        d = [2, 4, 8][int(rng.integers(0, 3))]
        base = [0.0, 10000.0][case % 2]
        pos = [0, 2, 5][case % 3]
        w = int(rng.integers(1, 11))
        q = rng.standard_normal((1, Hq, T, d))
        k = rng.standard_normal((1, Hkv, S, d))
        v = rng.standard_normal((1, Hkv, S, d))
        o, l = orc.attention(q, k, v, causal=True, rope_base=base, pos=pos, window=w)
        bo, bl = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), True, base, pos, window=w)
        bo = np.array(bo, dtype=np.float64)
        bl = np.array(bl, dtype=np.float64)
        assert np.allclose(o, bo, rtol=0, atol=1e-12), (case, np.max(np.abs(o - bo)))
        fin = np.isfinite(bl)
        assert np.array_equal(fin, np.isfinite(l)), case
        assert np.allclose(l[fin], bl[fin], rtol=0, atol=1e-12), case


def check_window_special_cases(orc):
    """A window reaching back past key 0 is plain causal attention; a window of 1 leaves
    each query its own key only (O_t = v at pos + t, lse = that logit); with Q = 0 the
    output is the mean of the values in the window."""
    rng = _rng(12)
    Hq, Hkv, T, S, d, pos = 4, 2, 9, 12, 8, 3
    q = rng.standard_normal((1, Hq, T, d))
    k = rng.standard_normal((1, Hkv, S, d))
    v = rng.standard_normal((1, Hkv, S, d))
    oc, lc = orc.attention(q, k, v, causal=True, rope_base=10000.0, pos=pos)
    for w in (pos + T, pos + T + 5, 10 ** 6):
        ow, lw = orc.attention(q, k, v, causal=True, rope_base=10000.0, pos=pos, window=w)
        assert np.array_equal(ow, oc) and np.array_equal(lw, lc), w
    o1, l1 = orc.attention(q, k, v, causal=True, rope_base=0.0, pos=pos, window=1)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for t in range(T):
            s_ = pos + t
            if s_ < S:
                assert np.allclose(o1[0, h, t], v[0, g, s_], atol=1e-14)
                assert abs(l1[0, h, t] - float(q[0, h, t] @ k[0, g, s_]) / math.sqrt(d)) < 1e-12
            else:
                assert not np.isfinite(l1[0, h, t]) and np.all(o1[0, h, t] == 0)
    for w in (2, 5):
        o0, l0 = orc.attention(np.zeros_like(q), k, v, causal=True, rope_base=10000.0, pos=pos, window=w)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for t in range(T):
                lo, hi = max(0, pos + t - w + 1), min(S, pos + t + 1)
                if hi <= lo:
                    continue
                assert np.allclose(o0[0, h, t], v[0, g, lo:hi].mean(axis=0), atol=1e-13)
                assert abs(l0[0, h, t] - math.log(hi - lo)) < 1e-13


# ------------------------------------------------------------------------
# Closed forms and special cases.
# ------------------------------------------------------------------------

def check_q_zero_gives_mean(orc):
    """Q = 0: every visible logit is 0, so O_t is the plain mean of the visible
    values and lse_t = ln(#visible)."""
    rng = _rng(2)
    for causal in (False, True):
        for (Hq, Hkv, T, S, pos, base) in [(4, 2, 7, 7, 0, 10000.0), (2, 1, 5, 9, 4, 0.0),
                                           (3, 3, 6, 6, 0, 500000.0)]:
            q = np.zeros((2, Hq, T, 8))
            k = rng.standard_normal((2, Hkv, S, 8))
            v = rng.standard_normal((2, Hkv, S, 8))
            o, l = orc.attention(q, k, v, causal=causal, rope_base=base, pos=pos)
            for b in range(2):
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    for t in range(T):
                        n = min(S, pos + t + 1) if causal else S
                        assert np.allclose(o[b, h, t], v[b, g, :n].mean(axis=0), atol=1e-13)
                        assert abs(l[b, h, t] - math.log(n)) < 1e-13


def check_single_key(orc):
    """T = S = 1: the output is v_0 and lse is the single scaled logit."""
    rng = _rng(3)
    for d in (2, 8, 64):
        q = rng.standard_normal((1, 1, 1, d))
        k = rng.standard_normal((1, 1, 1, d))
        v = rng.standard_normal((1, 1, 1, d))
        o, l = orc.attention(q, k, v, causal=True, rope_base=0.0)
        assert np.allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-14)
        assert abs(l[0, 0, 0] - float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(d)) < 1e-12


def check_causal_first_row(orc):
    """Causal, pos = 0: query 0 sees only key 0 (and RoPE at position 0 is the identity)."""
    rng = _rng(4)
    q = rng.standard_normal((1, 2, 5, 8))
    k = rng.standard_normal((1, 2, 5, 8))
    v = rng.standard_normal((1, 2, 5, 8))
    o, l = orc.attention(q, k, v, causal=True, rope_base=10000.0, pos=0)
    for h in range(2):
        assert np.allclose(o[0, h, 0], v[0, h, 0], atol=1e-14)
        assert abs(l[0, h, 0] - float(q[0, h, 0] @ k[0, h, 0]) / math.sqrt(8)) < 1e-12


def check_one_hot_logit_closed_form(orc):
    """K = rows of the identity, q = a e_j: logit j is a/sqrt(d), the rest are 0, so
    p_j = e^{a/sqrt d} / (e^{a/sqrt d} + S - 1) exactly, and lse = ln(e^{a/sqrt d} + S - 1)."""
    rng = _rng(5)
    d, S = 16, 12
    k = np.eye(S, d)[None, None]
    v = rng.standard_normal((1, 1, S, d))
    for a in (0.5, 3.0, 40.0, 400.0, 6000.0):
        for j in (0, 5, 11):
            q = np.zeros((1, 1, 1, d))
            q[0, 0, 0, j] = a
            o, l = orc.attention(q, k, v)
            z = a / math.sqrt(d)
            pj = 1.0 / (1.0 + (S - 1) * math.exp(-z))
            rest = np.delete(v[0, 0], j, axis=0).sum(axis=0)
            want = pj * v[0, 0, j] + (1.0 - pj) / (S - 1) * rest
            assert np.allclose(o[0, 0, 0], want, atol=1e-12), (a, j)
            want_lse = z + math.log1p((S - 1) * math.exp(-z))
            assert abs(l[0, 0, 0] - want_lse) < 1e-12, (a, j)


def check_rope_d2_is_plane_rotation(orc):
    """d_h = 2: one pair with frequency base^0 = 1, so RoPE is the plane rotation
    by angle pos (complex multiplication by e^{i pos}; counter-clockwise reading)."""
    rng = _rng(6)
    x = rng.standard_normal((9, 2))
    pos = np.array([0, 1, 2, 7, 100, 1000, 8191, 32767, 123456])
    for base in (10000.0, 500000.0, 3.0):
        y = orc.apply_rope(x, pos, base)
        z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * pos.astype(np.float64))
        assert np.allclose(y[:, 0], z.real, atol=1e-9) and np.allclose(y[:, 1], z.imag, atol=1e-9)


def check_rope_d4_frequencies(orc):
    """d_h = 4: pair (0,1) turns by pos, pair (2,3) by pos / sqrt(base)
    (theta = pos / base^(2i/d) with i = 1, d = 4)."""
    rng = _rng(7)
    x = rng.standard_normal((5, 4))
    pos = np.array([0, 1, 5, 77, 4095])
    for base in (10000.0, 16.0):
        y = orc.apply_rope(x, pos, base)
        for i, ang in ((0, pos.astype(np.float64)), (1, pos / math.sqrt(base))):
            z = (x[:, 2 * i] + 1j * x[:, 2 * i + 1]) * np.exp(1j * ang)
            assert np.allclose(y[:, 2 * i], z.real, atol=1e-10)
            assert np.allclose(y[:, 2 * i + 1], z.imag, atol=1e-10)


def check_rope_identity_at_zero(orc):
    rng = _rng(8)
    x = rng.standard_normal((1, 128))
    assert np.array_equal(orc.apply_rope(x, np.array([0]), 10000.0), x)
    assert np.array_equal(orc.apply_rope(x, np.array([5]), 0.0), x)


def check_rope_relative_and_norm(orc):
    """(R(m) q).(R(n) k) depends only on m - n; the rotation keeps norms."""
    rng = _rng(9)
    for base in (10000.0, 500000.0):
        for d in (64, 128):
            q = rng.standard_normal(d)
            k = rng.standard_normal(d)
            for (m, n) in ((5, 2), (100, 0), (4000, 3999)):
                ref = float(orc.apply_rope(q[None], [m], base)[0] @ orc.apply_rope(k[None], [n], base)[0])
                for c in (1, 17, 1000, 32767 - m):
                    got = float(orc.apply_rope(q[None], [m + c], base)[0]
                                @ orc.apply_rope(k[None], [n + c], base)[0])
                    assert abs(got - ref) <= 1e-10 * max(1.0, abs(ref)), (base, d, m, n, c)
            for p in (1, 33, 32767):
                y = orc.apply_rope(q[None], [p], base)[0]
                assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
                # each pair keeps its own norm
                assert np.allclose(y[0::2] ** 2 + y[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2, atol=1e-12)


# ------------------------------------------------------------------------
# Invariants.
# ------------------------------------------------------------------------

def check_rows_sum_to_one(orc):
    """Masking on the logits before the softmax keeps each probability row summing to 1,
    with zeros on hidden keys."""
    rng = _rng(10)
    q = rng.standard_normal((1, 2, 9, 8)) * 3
    k = rng.standard_normal((1, 2, 9, 8)) * 3
    v = rng.standard_normal((1, 2, 9, 8))
    for causal in (False, True):
        _, _, p = orc.attention(q, k, v, causal=causal, rope_base=10000.0, return_probs=True)
        assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-14)
        assert np.all(p >= 0)
        if causal:
            assert np.all(np.triu(p[0, 0], 1) == 0)


def check_permutation_equivariance(orc):
    """Without positions or a mask: permuting the queries permutes the outputs, and a joint
    permutation of keys and values changes nothing."""
    rng = _rng(11)
    q = rng.standard_normal((1, 1, 7, 8))
    k = rng.standard_normal((1, 1, 10, 8))
    v = rng.standard_normal((1, 1, 10, 8))
    o, l = orc.attention(q, k, v)
    pq = rng.permutation(7)
    pk = rng.permutation(10)
    o2, l2 = orc.attention(q[:, :, pq], k, v)
    assert np.allclose(o2, o[:, :, pq], atol=1e-14) and np.allclose(l2, l[:, :, pq], atol=1e-14)
    o3, l3 = orc.attention(q, k[:, :, pk], v[:, :, pk])
    assert np.allclose(o3, o, atol=1e-13) and np.allclose(l3, l, atol=1e-13)


def check_gqa_equals_repeated_mha(orc):
    """Grouped-query attention equals multi-head attention with each KV head repeated for
    its contiguous group of query heads."""
    rng = _rng(12)
    for (Hq, Hkv) in ((8, 2), (4, 1), (6, 3)):
        q = rng.standard_normal((2, Hq, 5, 8))
        k = rng.standard_normal((2, Hkv, 6, 8))
        v = rng.standard_normal((2, Hkv, 6, 8))
        o, l = orc.attention(q, k, v, causal=True, rope_base=10000.0, pos=1)
        rep = Hq // Hkv
        o2, l2 = orc.attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1),
                               causal=True, rope_base=10000.0, pos=1)
        assert np.allclose(o, o2, atol=1e-14) and np.allclose(l, l2, atol=1e-14)
        # and each query head depends only on its own KV head
        k3 = k.copy()
        k3[:, Hkv - 1] += 5.0
        o3, _ = orc.attention(q, k3, v, causal=True, rope_base=10000.0, pos=1)
        first = (Hkv - 1) * rep
        assert np.allclose(o3[:, :first], o[:, :first], atol=1e-14)
        assert not np.allclose(o3[:, first:], o[:, first:], atol=1e-6)


def blockwise_merge_attention(qr, kr, v, mask, bounds):
    """Attention computed one key block at a time and then combined, as the FlashAttention
    deep dive of "Why is attention O(n^2), how does FlashAttention help ..." argues is exact:
    every block on its own gives a softmax-normalised output o_b over its keys and the log of
    its normaliser, lse_b; since the full normaliser is the sum of the block normalisers,
    lse = log sum_b exp(lse_b) and the full output is the average of the o_b weighted by
    exp(lse_b - lse).  A block in which a row sees no key has lse_b = -inf and weight 0.
    qr [T,d], kr [S,d], v [S,dv], mask [T,S] additive (0 or -inf); bounds: key blocks."""
    T, d = qr.shape
    outs, lses = [], []
    for s0, s1 in bounds:
        logits = qr @ kr[s0:s1].T / math.sqrt(d) + mask[:, s0:s1]
        top = logits.max(axis=1)
        live = np.isfinite(top)
        shift = np.where(live, top, 0.0)
        w = np.exp(logits - shift[:, None])              # 0 for hidden keys
        z = np.where(live, w.sum(axis=1), 1.0)
        outs.append(np.where(live[:, None], (w @ v[s0:s1]) / z[:, None], 0.0))
        lses.append(np.where(live, shift + np.log(z), -np.inf))
    lse_b = np.stack(lses)                               # [blocks, T]
    top = lse_b.max(axis=0)
    weight = np.exp(lse_b - top)                         # exp(-inf) = 0
    total = weight.sum(axis=0)
    out = np.einsum("bt,btd->td", weight, np.stack(outs)) / total[:, None]
    return out, top + np.log(total)


def check_online_recurrence_equals_full(orc):
    """Blocked evaluation over arbitrary key-block partitions (including blocks that are fully
    masked for some rows), the blocks combined through their log-normalisers, gives the full
    softmax result up to rounding."""
    rng = _rng(13)
    for trial in range(12):
        T = int(rng.integers(1, 40))
        S = int(rng.integers(1, 60))
        d = 16
        pos = int(rng.integers(0, 5)) + max(0, S - T) * (trial % 2)
        q = rng.standard_normal((1, 1, T, d)) * 2
        k = rng.standard_normal((1, 1, S, d)) * 2
        v = rng.standard_normal((1, 1, S, d))
        base = 10000.0 if trial % 3 else 0.0
        o, l = orc.attention(q, k, v, causal=True, rope_base=base, pos=pos)
        cuts = sorted(set(rng.integers(1, S, size=int(rng.integers(0, 6))).tolist())) if S > 1 else []
        bounds = list(zip([0] + cuts, cuts + [S]))
        qr = orc.apply_rope(q[0, 0], pos + np.arange(T), base)
        kr = orc.apply_rope(k[0, 0], np.arange(S), base)
        mask = orc.causal_mask(pos + np.arange(T), np.arange(S))
        o2, l2 = blockwise_merge_attention(qr, kr, v[0, 0], mask, bounds)
        assert np.allclose(o2, o[0, 0], atol=1e-13), trial
        assert np.allclose(l2, l[0, 0], atol=1e-13), trial


def lse_merge(outs, lses):
    """Combine normalised partial results over disjoint key sets: weights exp(lse_j - LSE)."""
    lses = np.stack(lses)                      # [J, ...]
    M = np.max(lses, axis=0)
    w = np.exp(lses - M)
    tot = np.sum(w, axis=0)
    out = sum(w[j][..., None] * outs[j] for j in range(len(outs))) / tot[..., None]
    return out, M + np.log(tot)


def check_splitk_merge_equals_unsplit(orc):
    rng = _rng(14)
    for S in (5, 37, 100):
        q = rng.standard_normal((3, 16)) * 2
        k = rng.standard_normal((S, 16)) * 2
        v = rng.standard_normal((S, 16))
        o, l, _ = orc.sdpa(q, k, v)
        cuts = sorted(set(rng.integers(1, S, size=3).tolist()))
        parts = list(zip([0] + cuts, cuts + [S]))
        outs, lses = [], []
        for s0, s1 in parts:
            oj, lj, _ = orc.sdpa(q, k[s0:s1], v[s0:s1])
            outs.append(oj)
            lses.append(lj)
        o2, l2 = lse_merge(outs, lses)
        assert np.allclose(o2, o, atol=1e-13) and np.allclose(l2, l, atol=1e-13)


def _scatter_paged(rows, block_size, n_extra_blocks, rng, poison=np.nan):
    """Place rows [Hkv, L, d] into a randomly permuted pool; unused slots get `poison`."""
    Hkv, L, d = rows.shape
    nb = (L + block_size - 1) // block_size
    num_blocks = nb + n_extra_blocks
    perm = rng.permutation(num_blocks)[:nb]
    pool = np.full((num_blocks, Hkv, block_size, d), poison)
    for j in range(L):
        pool[perm[j // block_size], :, j % block_size, :] = rows[:, j, :]
    table = perm.astype(np.int32)
    return pool, table


def check_gather_after_scatter_is_identity(orc):
    rng = _rng(15)
    for L in (1, 15, 16, 17, 100):
        rows = rng.standard_normal((3, L, 8)).astype(np.float32)
        pool, table = _scatter_paged(rows, 16, 3, rng)
        got = orc.gather_paged(pool, table, L, 16)
        assert got.dtype == pool.dtype and np.array_equal(got, rows.astype(pool.dtype))


def check_decode_equals_last_causal_row(orc):
    """A decode step over the paged cache (K stored already rotated) equals the last row of
    causal prefill with RoPE on contiguous K."""
    rng = _rng(16)
    Hq, Hkv, d, bs = 4, 2, 8, 16
    for L in (1, 16, 33, 70):
        base = 10000.0
        q_all = rng.standard_normal((1, Hq, L, d))
        k = rng.standard_normal((1, Hkv, L, d))
        v = rng.standard_normal((1, Hkv, L, d))
        o, l = orc.attention(q_all, k, v, causal=True, rope_base=base, pos=0)
        k_rot = orc.apply_rope(k[0], np.arange(L), base)
        kpool, table = _scatter_paged(k_rot, bs, 2, np.random.default_rng(L))
        vpool, table2 = _scatter_paged(v[0], bs, 2, np.random.default_rng(L))
        assert np.array_equal(table, table2)
        od, ld = orc.decode_paged(q_all[0, :, L - 1][None], kpool, vpool, table[None],
                                  np.array([L]), bs, rope_base=base)
        assert np.allclose(od[0], o[0, :, L - 1], atol=1e-13), L
        assert np.allclose(ld[0], l[0, :, L - 1], atol=1e-13), L


def check_prefill_paged_equals_contiguous(orc):
    """Prefill through block tables (K stored already rotated) equals causal prefill with RoPE
    on contiguous K at the same positions; one new token equals the decode step; and two
    sequences whose tables share the prefix blocks give the same result as with private
    copies of those blocks."""
    rng = _rng(17)
    Hq, Hkv, d, bs, base = 4, 2, 8, 16, 10000.0
    for (L, T) in ((40, 9), (33, 33), (70, 1), (16, 5)):
        q = rng.standard_normal((1, Hq, T, d))
        k = rng.standard_normal((1, Hkv, L, d))
        v = rng.standard_normal((1, Hkv, L, d))
        o, l = orc.attention(q, k, v, causal=True, rope_base=base, pos=L - T)
        k_rot = orc.apply_rope(k[0], np.arange(L), base)
        kpool, table = _scatter_paged(k_rot, bs, 3, np.random.default_rng(L + T))
        vpool, _ = _scatter_paged(v[0], bs, 3, np.random.default_rng(L + T))
        op, lp = orc.prefill_paged(q, kpool, vpool, table[None], np.array([L]), bs, rope_base=base)
        assert np.allclose(op, o, atol=1e-12) and np.allclose(lp, l, atol=1e-12), (L, T)
        if T == 1:
            od, ld = orc.decode_paged(q[:, :, 0], kpool, vpool, table[None], np.array([L]), bs, rope_base=base)
            assert np.allclose(od, op[:, :, 0], atol=1e-13) and np.allclose(ld, lp[:, :, 0], atol=1e-13)
    # shared prefix: sequences 0 and 1 share their first 3 blocks
    P, T = 48, 7
    L0, L1 = P + 10, P + 20
    pre_k, pre_v = rng.standard_normal((2, Hkv, P, d))
    own_k = [rng.standard_normal((Hkv, L - P, d)) for L in (L0, L1)]
    own_v = [rng.standard_normal((Hkv, L - P, d)) for L in (L0, L1)]
    nb0, nb1 = -(-L0 // bs), -(-L1 // bs)
    pool_k = np.zeros((3 + (nb0 - 3) + (nb1 - 3) + 3, Hkv, bs, d))
    pool_v = np.zeros_like(pool_k)
    shared = [0, 1, 2]
    t0 = shared + [3 + i for i in range(nb0 - 3)]
    t1 = shared + [3 + (nb0 - 3) + i for i in range(nb1 - 3)]
    for (tab, L, ok, ov) in ((t0, L0, own_k[0], own_v[0]), (t1, L1, own_k[1], own_v[1])):
        kk = np.concatenate([pre_k, ok], axis=1)
        vv = np.concatenate([pre_v, ov], axis=1)
        for j in range(L):
            pool_k[tab[j // bs], :, j % bs] = kk[:, j]
            pool_v[tab[j // bs], :, j % bs] = vv[:, j]
    table = np.full((2, max(nb0, nb1)), -1, dtype=np.int32)
    table[0, :nb0], table[1, :nb1] = t0, t1
    q = rng.standard_normal((2, Hq, T, d))
    lens = np.array([L0, L1])
    os_, ls_ = orc.prefill_paged(q, pool_k, pool_v, table, lens, bs, rope_base=base)
    for b, (tab, L) in enumerate(((t0, L0), (t1, L1))):
        kk = orc.gather_paged(pool_k, tab, L, bs)
        vv = orc.gather_paged(pool_v, tab, L, bs)
        assert np.array_equal(kk[:, :P], pre_k) and np.array_equal(vv[:, :P], pre_v)
        priv_k, priv_t = _scatter_paged(kk, bs, 1, np.random.default_rng(b))
        priv_v, _ = _scatter_paged(vv, bs, 1, np.random.default_rng(b))
        ob, lb = orc.prefill_paged(q[b:b + 1], priv_k, priv_v, priv_t[None], np.array([L]), bs, rope_base=base)
        assert np.allclose(ob[0], os_[b], atol=1e-13) and np.allclose(lb[0], ls_[b], atol=1e-13)


def check_torch_sdpa_core(orc):
    """Library cross-check of scale, mask and GQA map: torch's fp64 CPU SDPA on the
    oracle's rotated q and k must agree."""
    rng = _rng(17)
    for (Hq, Hkv, T, S, causal, pos) in ((4, 2, 9, 9, True, 0), (8, 2, 5, 12, False, 0),
                                         (4, 4, 6, 10, True, 4)):
        q = rng.standard_normal((2, Hq, T, 16))
        k = rng.standard_normal((2, Hkv, S, 16))
        v = rng.standard_normal((2, Hkv, S, 16))
        base = 10000.0
        o, l = orc.attention(q, k, v, causal=causal, rope_base=base, pos=pos)
        qr = orc.apply_rope(q, pos + np.arange(T), base)
        kr = orc.apply_rope(k, np.arange(S), base)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(S)[None, :] <= (pos + np.arange(T))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr), torch.from_numpy(kr), torch.from_numpy(v), attn_mask=mask,
            enable_gqa=(Hq != Hkv)).numpy()
        assert np.allclose(o, ref, atol=1e-12), np.max(np.abs(o - ref))


def check_cross_attention_shapes(orc):
    """T != S (cross-attention style): output has the query count and the value width; a
    swap of queries and keys would change the shape."""
    rng = _rng(18)
    q = rng.standard_normal((1, 2, 3, 8))
    k = rng.standard_normal((1, 2, 11, 8))
    v = rng.standard_normal((1, 2, 11, 8))
    o, l = orc.attention(q, k, v)
    assert o.shape == (1, 2, 3, 8) and l.shape == (1, 2, 3)
    o2, l2 = orc.attention_rows(q, k, v, [(0, 1, 2), (0, 0, 0)])
    assert np.allclose(o2[0], o[0, 1, 2], atol=1e-14) and np.allclose(o2[1], o[0, 0, 0], atol=1e-14)


# ------------------------------------------------------------------------
# Backward pass: gradients of sum(dO * O) with respect to q, k and v.
# ------------------------------------------------------------------------

def _bwd_case(rng, B, Hq, Hkv, T, S, d):
    return (rng.standard_normal((B, Hq, T, d)), rng.standard_normal((B, Hkv, S, d)),
            rng.standard_normal((B, Hkv, S, d)), rng.standard_normal((B, Hq, T, d)))


def check_backward_finite_differences(orc):
    """Central differences of L = sum(dO * attention(q, k, v)) through the (separately pinned)
    forward agree with the backward's gradient, entry by entry, for causal, windowed, RoPE
    and grouped-query cases."""
    rng = _rng(30)
    eps = 1e-5
    for (Hq, Hkv, T, S, causal, base, pos, window) in ((2, 1, 5, 5, True, 10000.0, 0, 0),
                                                        (4, 2, 4, 7, False, 100.0, 0, 0),
                                                        (2, 2, 6, 9, True, 50.0, 3, 4)):
        q, k, v, do = _bwd_case(rng, 1, Hq, Hkv, T, S, 8)
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, base, pos, window)

        def loss(q_, k_, v_):
            o, _ = orc.attention(q_, k_, v_, causal=causal, rope_base=base, pos=pos, window=window)
            return float(np.sum(do * o))

        for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(6):
                idx = tuple(int(rng.integers(0, n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[which]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[which]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


def _torch_rope(x, positions, base):
    """RoPE written with torch ops (differentiable) from the pair rotation definition."""
    if base <= 0:
        return x
    d = x.shape[-1]
    i = torch.arange(d // 2, dtype=torch.float64)
    ang = torch.as_tensor(np.asarray(positions, dtype=np.float64))[:, None] * base ** (-2.0 * i / d)[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    return torch.stack((a * c - b * s, a * s + b * c), dim=-1).flatten(-2)


def check_backward_torch_autograd(orc):
    """Library cross-check: torch autograd through torch's fp64 CPU SDPA, fed by a torch RoPE,
    gives the same dq, dk and dv (grouped-query sums included)."""
    rng = _rng(31)
    for (Hq, Hkv, T, S, causal, base, pos) in ((4, 2, 9, 9, True, 10000.0, 0), (4, 1, 5, 12, False, 500.0, 0),
                                               (2, 2, 6, 10, True, 10000.0, 4)):
        q, k, v, do = _bwd_case(rng, 2, Hq, Hkv, T, S, 16)
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, base, pos)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        qr = _torch_rope(qt, pos + np.arange(T), base)
        kr = _torch_rope(kt, np.arange(S), base)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(S)[None, :] <= (pos + np.arange(T))[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(qr, kr, vt, attn_mask=mask,
                                                             enable_gqa=(Hq != Hkv))
        (o * torch.from_numpy(do)).sum().backward()
        for a, t in ((dq, qt), (dk, kt), (dv, vt)):
            assert np.allclose(a, t.grad.numpy(), atol=1e-12), np.max(np.abs(a - t.grad.numpy()))


def check_backward_invariants(orc):
    """Facts of the calculus that hold for any inputs:
    - dO = 0 gives zero gradients;
    - every probability row sums to one, so the dv rows of a KV head sum to the sum of dO
      over all query rows of the heads that read it;
    - without RoPE the output does not change when one vector is added to every key, so the
      dk rows of a head sum to zero;
    - with all keys equal every row attends uniformly whatever q is: dq = 0;
    - a single key: O = v, so dq = dk = 0 and dv = the sum of dO over rows and heads."""
    rng = _rng(32)
    q, k, v, do = _bwd_case(rng, 1, 4, 2, 6, 8, 8)
    for causal, base in ((False, 0.0), (True, 0.0), (True, 10000.0)):
        z = orc.attention_backward(q, k, v, np.zeros_like(do), causal, base)
        assert all(np.all(x == 0) for x in z)
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, base)
        for g in range(2):
            assert np.allclose(dv[0, g].sum(axis=0), do[0, 2 * g:2 * g + 2].sum(axis=(0, 1)), atol=1e-12)
        if base == 0.0:
            assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    keq = np.broadcast_to(k[:, :, :1], k.shape).copy()
    dq, _, _ = orc.attention_backward(q, keq, v, do, False, 0.0)
    assert np.allclose(dq, 0.0, atol=1e-12)
    dq, dk, dv = orc.attention_backward(q, k[:, :, :1], v[:, :, :1], do, False, 10000.0)
    assert np.allclose(dq, 0.0, atol=1e-12) and np.allclose(dk, 0.0, atol=1e-12)
    assert np.allclose(dv[0, :, 0], do[0].reshape(2, 2, 6, 8).sum(axis=(1, 2)), atol=1e-12)


def check_backward_sampled_equals_full(orc):
    """The sampled backward (used at full size) returns exactly the corresponding entries of
    the full backward: keys and rows spread over the sequence, grouped heads, RoPE, causal,
    windowed and non-causal cases."""
    rng = _rng(33)
    q, k, v, do = _bwd_case(rng, 2, 4, 2, 20, 30, 16)
    keys = [0, 3, 29, 15]
    rows = [(2, 0), (3, 19), (2, 7)]
    for causal, w, pos in ((True, 0, 10), (False, 0, 0), (True, 7, 10)):
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, 1e4, pos, w)
        a, b_, c = orc.attention_backward_sampled(q, k, v, do, 1, 1, keys, rows, causal, 1e4, pos, w)
        assert np.allclose(a, np.array([dq[1, h, t] for h, t in rows]), atol=1e-13)
        assert np.allclose(b_, dk[1, 1, keys], atol=1e-13) and np.allclose(c, dv[1, 1, keys], atol=1e-13)


# ------------------------------------------------------------------------
# FP8 inputs
# ------------------------------------------------------------------------

def check_fp8_decode(orc):
    """The E4M3 decoder against the format's closed forms (1.0, the largest finite 448, the
    smallest normal 2^-6 and subnormal 2^-9, signs, NaN), monotone over the positive codes, and
    against torch's float8_e4m3fn conversion for all 256 codes (a library cross-check)."""
    d = orc.fp8_e4m3_decode
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x00) == 0.0
    assert d(0x3C) == 1.5 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    pos = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = d(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got)) and np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)])


def check_fp8_attention_scales(orc):
    """Per-tensor scales: multiplying q's scale by a and dividing k's by a leaves the logits
    and so the output unchanged; v's scale multiplies the output and leaves lse unchanged; V is
    read transposed ([.., d_h, S]), which a per-element loop over the decoded codes checks."""
    rng = _rng(40)
    q8 = rng.integers(0, 0x70, (1, 4, 9, 16)).astype(np.uint8) | (rng.integers(0, 2, (1, 4, 9, 16)) << 7).astype(np.uint8)
    k8 = rng.integers(0, 0x70, (1, 2, 11, 16)).astype(np.uint8)
    vt8 = rng.integers(0, 0x70, (1, 2, 16, 11)).astype(np.uint8) | 0x80
    o1, l1 = orc.attention_fp8(q8, k8, vt8, 1.0, 1.0, 1.0, causal=True, pos=2)
    o2, l2 = orc.attention_fp8(q8, k8, vt8, 4.0, 0.25, 3.0, causal=True, pos=2)
    assert np.allclose(o2, 3.0 * o1, atol=1e-12) and np.allclose(l2, l1, atol=1e-12)
    d = orc.fp8_e4m3_decode
    v = np.zeros((1, 2, 11, 16))
    for h in range(2):
        for sk in range(11):
            for e in range(16):
                v[0, h, sk, e] = d(vt8[0, h, e, sk])
    ro, rl = brute_force_attention(d(q8), d(k8), v, True, 0.0, 2)
    assert np.allclose(o1, ro, atol=1e-12) and np.allclose(l1, rl, atol=1e-12)


def check_error_metrics(orc):
    """max_abs and rel_rms, the acceptance metrics of every parity test, against closed
    forms: max_abs is the largest |got - ref| over the whole tensor (sign dropped, the
    largest element, not a mean); rel_rms is ||got - ref||_2 / ||ref||_2 over the whole
    tensor (one norm of everything, not per row); a NaN in got never passes a bound."""
    ref = np.array([[1.0, -2.0, 3.0], [0.5, 0.0, -4.0]])
    err = np.zeros_like(ref)
    err[1, 2] = -0.37
    assert orc.max_abs(ref + err, ref) == 0.37 or abs(orc.max_abs(ref + err, ref) - 0.37) < 1e-15
    err[0, 1] = 0.125
    assert abs(orc.max_abs(ref + err, ref) - 0.37) < 1e-15          # the largest, sign dropped
    assert abs(orc.max_abs(ref - err, ref) - 0.37) < 1e-15
    spread = np.array([0.1, 0.2, 0.5, -0.05])
    assert abs(orc.max_abs(spread, np.zeros(4)) - 0.5) < 1e-15      # not the mean (0.2125)
    assert orc.max_abs(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    assert orc.max_abs(ref, ref) == 0.0
    rng = _rng(40)
    r = rng.standard_normal((3, 5, 7))
    for eps in (1e-3, -2.5e-2, 0.5):
        assert abs(orc.rel_rms(r * (1.0 + eps), r) - abs(eps)) < 1e-14 * (1 + abs(eps))
    # a 3-4-5 error against a 5-12-13 reference: 5 / 13
    assert abs(orc.rel_rms(np.array([8.0, 16.0, 0.0]), np.array([5.0, 12.0, 0.0])) - 5.0 / 13.0) < 1e-15
    # one norm over the whole tensor: rows of very different size
    big = np.array([[1.0, 0.0], [0.0, 10.0]])
    assert abs(orc.rel_rms(big + np.array([[1.0, 0.0], [0.0, 0.0]]), big) - 1.0 / math.sqrt(101.0)) < 1e-15
    # independent of the tensor's size (no 1/N): the same relative error on 1 and on 4096 entries
    one = np.array([2.0])
    many = np.full(4096, 2.0)
    assert abs(orc.rel_rms(one * 1.01, one) - orc.rel_rms(many * 1.01, many)) < 1e-15
    assert orc.rel_rms(np.zeros(3), np.zeros(3)) == 0.0
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert not orc.max_abs(bad, ref) <= 1.0
    assert not orc.rel_rms(bad, ref) <= 1.0


ALL_CHECKS = [
    check_error_metrics,
    check_fp8_decode, check_fp8_attention_scales,
    check_backward_finite_differences, check_backward_sampled_equals_full, check_backward_torch_autograd, check_backward_invariants,
    check_prefill_paged_equals_contiguous,
    check_bruteforce_window,
    check_window_special_cases,
    check_bruteforce_tiny, check_q_zero_gives_mean, check_single_key, check_causal_first_row,
    check_one_hot_logit_closed_form, check_rope_d2_is_plane_rotation, check_rope_d4_frequencies,
    check_rope_identity_at_zero, check_rope_relative_and_norm, check_rows_sum_to_one,
    check_permutation_equivariance, check_gqa_equals_repeated_mha,
    check_online_recurrence_equals_full, check_splitk_merge_equals_unsplit,
    check_gather_after_scatter_is_identity, check_decode_equals_last_causal_row,
    check_torch_sdpa_core, check_cross_attention_shapes,
]
