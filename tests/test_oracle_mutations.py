"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and show that the
pin battery catches each one.  The real oracle module is never modified."""

import importlib.util
import math
import os

import numpy as np
import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# --- planted mistakes --------------------------------------------------------

def m_mask_after_softmax(mod):
    orig = mod.sdpa

    def sdpa(q, k, v, mask=None):
        o, l, p = orig(q, k, v, None)
        if mask is not None:
            p = np.where(np.isfinite(mask), p, 0.0)     # zero after normalising
            o = np.matmul(p, np.asarray(v, dtype=np.float64))
        return o, l, p
    mod.sdpa = sdpa


def m_no_scale(mod):
    orig = mod.sdpa

    def sdpa(q, k, v, mask=None):
        d = np.asarray(q).shape[-1]
        return orig(np.asarray(q, dtype=np.float64) * math.sqrt(d), k, v, mask)
    mod.sdpa = sdpa


def m_scale_by_d(mod):
    orig = mod.sdpa

    def sdpa(q, k, v, mask=None):
        d = np.asarray(q).shape[-1]
        return orig(np.asarray(q, dtype=np.float64) / math.sqrt(d), k, v, mask)
    mod.sdpa = sdpa


def m_rope_freq_exponent(mod):
    mod.rope_inv_freq = lambda d_h, base: np.power(float(base), -np.arange(d_h // 2) / float(d_h))


def m_rope_clockwise(mod):
    orig = mod.apply_rope

    def apply_rope(x, positions, base):
        return orig(x, -np.asarray(positions), base)
    mod.apply_rope = apply_rope


def m_rope_rotate_half_pairs(mod):
    orig = mod.apply_rope

    def apply_rope(x, positions, base):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        perm = np.empty(d, dtype=np.int64)     # pair i with i + d/2 instead of 2i+1
        perm[0::2] = np.arange(d // 2)
        perm[1::2] = np.arange(d // 2) + d // 2
        inv = np.argsort(perm)
        return orig(x[..., perm], positions, base)[..., inv]
    mod.apply_rope = apply_rope


def m_rope_only_queries(mod):
    orig_attention = mod.attention

    def attention(q, k, v, causal=False, rope_base=0.0, pos=0, row_block=None, return_probs=False, window=0):
        real = mod.apply_rope
        calls = {"n": 0}

        def rope_skip_first(x, p, base):      # first call in attention() rotates K
            calls["n"] += 1
            return real(x, p, 0.0) if calls["n"] == 1 else real(x, p, base)
        mod.apply_rope = rope_skip_first
        try:
            return orig_attention(q, k, v, causal, rope_base, pos, row_block, return_probs, window)
        finally:
            mod.apply_rope = real
    mod.attention = attention


def m_gqa_modulo(mod):
    mod.kv_head_of = lambda h, Hq, Hkv: h % Hkv


def m_causal_off_by_one(mod):
    def causal_mask(qp, kp):
        qp = np.asarray(qp, dtype=np.int64)[:, None]
        kp = np.asarray(kp, dtype=np.int64)[None, :]
        return np.where(kp < qp, 0.0, -np.inf)
    mod.causal_mask = causal_mask


def m_lse_without_max(mod):
    orig = mod.sdpa

    def sdpa(q, k, v, mask=None):
        o, l, p = orig(q, k, v, mask)
        qq = np.asarray(q, dtype=np.float64)
        logits = np.matmul(qq, np.swapaxes(np.asarray(k, dtype=np.float64), -1, -2)) / np.sqrt(qq.shape[-1])
        if mask is not None:
            logits = logits + mask
        m = np.max(logits, axis=-1)
        return o, l - m, p
    mod.sdpa = sdpa


def m_pos_ignored(mod):
    orig = mod.attention

    def attention(q, k, v, causal=False, rope_base=0.0, pos=0, row_block=None, return_probs=False, window=0):
        return orig(q, k, v, causal, rope_base, 0, row_block, return_probs, window)
    mod.attention = attention


def m_decode_position_L(mod):
    orig = mod.decode_paged
    real = mod.apply_rope

    def decode_paged(q, k_cache, v_cache, block_table, seq_lens, block_size, rope_base=0.0):
        mod.apply_rope = lambda x, p, base: real(x, np.asarray(p) + 1, base)
        try:
            return orig(q, k_cache, v_cache, block_table, seq_lens, block_size, rope_base)
        finally:
            mod.apply_rope = real
    mod.decode_paged = decode_paged


def m_gather_swapped(mod):
    def gather_paged(cache, block_table, seq_len, block_size):
        j = np.arange(int(seq_len))
        nb = len(block_table)
        phys = np.asarray(block_table, dtype=np.int64)[j % nb]
        slot = (j // nb) % block_size
        rows = np.asarray(cache)[phys, :, slot, :]
        return np.ascontiguousarray(np.swapaxes(rows, 0, 1))
    mod.gather_paged = gather_paged


def m_probs_transposed(mod):
    def sdpa(q, k, v, mask=None):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        logits = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(q.shape[-1])
        if mask is not None:
            logits = logits + mask
        m = np.max(logits, axis=-2, keepdims=True)        # softmax over the query axis
        e = np.exp(logits - m)
        p = e / e.sum(axis=-2, keepdims=True)
        l = (m + np.log(e.sum(axis=-2, keepdims=True)))[..., 0, :]
        return np.matmul(p, v), np.broadcast_to(l[..., :1], p.shape[:-1]).copy(), p
    mod.sdpa = sdpa


def m_no_max_subtraction_overflow(mod):
    """Softmax without subtracting the row max: overflows for large logits."""
    def sdpa(q, k, v, mask=None):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        logits = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(q.shape[-1])
        if mask is not None:
            logits = logits + mask
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            e = np.exp(logits)
            z = e.sum(axis=-1, keepdims=True)
            p = e / z
            l = np.log(z)[..., 0]
        return np.matmul(p, v), l, p
    mod.sdpa = sdpa


def m_window_off_by_one(mod):
    """The window keeps one key too many (s >= q - w instead of s > q - w)."""
    def window_mask(qp, kp, window):
        qp = np.asarray(qp, dtype=np.int64)[:, None]
        kp = np.asarray(kp, dtype=np.int64)[None, :]
        return np.where((kp <= qp) & (kp >= qp - int(window)), 0.0, -np.inf)
    mod.window_mask = window_mask


def _resource(mod, old, new):
    """Re-execute the oracle's source with one substring replaced (must occur exactly once)."""
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    exec(compile(src.replace(old, new), ORACLE_SRC, "exec"), mod.__dict__)


def m_bwd_missing_delta(mod):
    """Softmax Jacobian without the rowsum(dO * O) term."""
    _resource(mod, "ds = p * (dp - delta)", "ds = p * dp")


def m_bwd_rope_forward_not_transpose(mod):
    """Gradients rotated by +phi (the forward rotation) instead of its transpose."""
    _resource(mod, "dq[b, h] = apply_rope_transpose(ds @ kr[b, g] * scale, qpos, rope_base)",
              "dq[b, h] = apply_rope(ds @ kr[b, g] * scale, qpos, rope_base)")


def m_bwd_gqa_overwrite(mod):
    """The last query head of a group overwrites dv instead of adding to it."""
    _resource(mod, "dv[b, g] += p.T @ do", "dv[b, g] = p.T @ do")


def m_bwd_dk_unscaled(mod):
    """dk without the 1/sqrt(d_h) of the scores."""
    _resource(mod, "dk[b, g] += apply_rope_transpose(ds.T @ qr * scale, kpos, rope_base)",
              "dk[b, g] += apply_rope_transpose(ds.T @ qr, kpos, rope_base)")


def m_bwd_dk_uses_unrotated_q(mod):
    """dk' formed from the unrotated queries."""
    _resource(mod, "dk[b, g] += apply_rope_transpose(ds.T @ qr * scale, kpos, rope_base)",
              "dk[b, g] += apply_rope_transpose(ds.T @ q[b, h] * scale, kpos, rope_base)")


def m_fp8_bias8(mod):
    """E4M3 exponent bias 8 instead of 7."""
    _resource(mod, "np.power(2.0, (e - 7).astype(F64))", "np.power(2.0, (e - 8).astype(F64))")


def m_fp8_no_subnormals(mod):
    """Exponent 0 decoded as a normal number."""
    _resource(mod, "mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,", "mag = np.where(e < 0, (m / 8.0) * 2.0 ** -6,")


def m_fp8_v_not_transposed(mod):
    """V codes read as [.., S, d_h] instead of transposed."""
    _resource(mod, "v = np.swapaxes(fp8_e4m3_decode(vt8), -1, -2) * F64(v_scale)",
              "v = fp8_e4m3_decode(vt8).reshape(vt8.shape[:-2] + (vt8.shape[-1], vt8.shape[-2])) * F64(v_scale)")


def m_rel_rms_no_sqrt(mod):
    """rel-RMS as a ratio of squared norms."""
    _resource(mod, "den = float(np.sqrt(np.sum(ref * ref)))\n    num = float(np.sqrt(np.sum((got - ref) ** 2)))",
              "den = float(np.sum(ref * ref))\n    num = float(np.sum((got - ref) ** 2))")


def m_rel_rms_num_no_sqrt(mod):
    """The error's norm without its square root."""
    _resource(mod, "num = float(np.sqrt(np.sum((got - ref) ** 2)))", "num = float(np.sum((got - ref) ** 2))")


def m_rel_rms_per_element(mod):
    """The ratio further divided by the element count."""
    _resource(mod, "return num / den if den > 0 else num", "return num / den / got.size if den > 0 else num")


def m_rel_rms_max_not_norm(mod):
    """The largest error over the reference norm instead of the error norm."""
    _resource(mod, "num = float(np.sqrt(np.sum((got - ref) ** 2)))", "num = float(np.max(np.abs(got - ref)))")


def m_rel_rms_row_mean(mod):
    """The mean of per-row relative errors instead of one norm over the tensor."""
    _resource(mod, "return num / den if den > 0 else num",
              "return float(np.mean(np.linalg.norm(np.atleast_2d(got - ref), axis=-1) / "
              "np.maximum(np.linalg.norm(np.atleast_2d(ref), axis=-1), 1e-300))) if den > 0 else num")


def m_max_abs_signed(mod):
    """max_abs without the absolute value."""
    _resource(mod, "np.max(np.abs(got - ref))", "np.max(got - ref)")


def m_max_abs_mean(mod):
    """The mean absolute error instead of the largest."""
    _resource(mod, "np.max(np.abs(got - ref))", "np.mean(np.abs(got - ref))")


def m_max_abs_ignores_nan(mod):
    """NaN entries skipped, so a non-finite result could pass."""
    _resource(mod, "np.max(np.abs(got - ref))", "np.nanmax(np.abs(got - ref))")


MUTATIONS = [m_rel_rms_no_sqrt, m_rel_rms_num_no_sqrt, m_rel_rms_per_element, m_rel_rms_max_not_norm,
             m_rel_rms_row_mean, m_max_abs_signed, m_max_abs_mean, m_max_abs_ignores_nan,
             m_fp8_bias8, m_fp8_no_subnormals, m_fp8_v_not_transposed, m_bwd_missing_delta, m_bwd_rope_forward_not_transpose, m_bwd_gqa_overwrite,
             m_bwd_dk_unscaled, m_bwd_dk_uses_unrotated_q,
             m_window_off_by_one, m_mask_after_softmax, m_no_scale, m_scale_by_d, m_rope_freq_exponent, m_rope_clockwise,
             m_rope_rotate_half_pairs, m_rope_only_queries, m_gqa_modulo, m_causal_off_by_one,
             m_lse_without_max, m_pos_ignored, m_decode_position_L, m_gather_swapped,
             m_probs_transposed, m_no_max_subtraction_overflow]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutate):
    mod = fresh_oracle()
    mutate(mod)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught {mutate.__name__}"


def test_unmutated_copy_passes_everything():
    mod = fresh_oracle()
    for check in oracle_pins.ALL_CHECKS:
        check(mod)
