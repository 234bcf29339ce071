"""Backward parity: attn_bwd (HIP, through the C ABI) against the fp64 oracle's chain-rule
gradients on the same seeded bf16 inputs, fed the GPU forward's out and lse.

Tolerance (per gradient tensor): relative RMS <= 1e-2 and max-abs <= 1e-2 * max|reference|.
An fp64 emulation of the kernels' rounding points (bf16 rotated q and k, bf16 P and dS,
bf16 O in rowsum(dO * O)) gives relative RMS 2.5e-3 to 4e-3 and max-abs up to 3.1e-3 * max
on these shapes, so the bound leaves about a factor of three.  Where the exact gradient is
zero the bound is 1e-4 absolute.  The gradients of the keys
near the start of a causal sequence sum over thousands of queries, so the max-abs bound is
taken relative to each tensor's scale rather than absolute."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import f64, say

pytestmark = pytest.mark.gpu

REL_RMS = 1e-2
MAX_REL = 1e-2
# A gradient that is exactly zero in exact arithmetic (window 1: each row attends only to
# itself, so dS = P * (dP - rowsum(dO * O)) cancels to 0) comes out at the rounding level of
# its O(1) terms; the scale of the max-abs bound is floored at 1e-2 (bound 1e-4) for it.
SCALE_FLOOR = 1e-2


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    scale = max(np.abs(ref).max(), SCALE_FLOOR)
    ma = np.abs(got - ref).max()
    rr = oracle.rel_rms(got, ref) if np.abs(ref).max() >= SCALE_FLOOR else 0.0
    msg = f"{what}: max_abs={ma:.3e} (scale {scale:.3e}) rel_rms={rr:.3e}"
    say(msg)
    assert ma <= MAX_REL * scale, msg
    assert rr <= REL_RMS, msg


def run_fwd_bwd(q, k, v, do, causal, window, base, pos):
    from exact_transformer_attention_amd import attn_bwd, attn_fwd, attn_fwd_window
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    if window:
        out, lse = attn_fwd_window(qd, kd, vd, window, rope_base=base, pos=pos)
    else:
        out, lse = attn_fwd(qd, kd, vd, causal=causal, rope_base=base, pos=pos)
    dq, dk, dv = attn_bwd(qd, kd, vd, out, lse, dod, causal=causal, window=window, rope_base=base, pos=pos)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # B, Hq, Hkv, T, S, causal, window, rope_base, pos, sigma: ragged tails, every GQA
    # packing of the dQ kernel (1, 2, 4 heads per KV head and more), T != S both ways,
    # a chunk at pos > 0, rows with no visible key (pos < 0), sliding windows, no RoPE,
    # the long-context scale and base
    (1, 4, 2, 200, 200, True, 0, 10000.0, 0, 1.0),
    (1, 8, 2, 130, 130, True, 0, 10000.0, 0, 1.0),
    (1, 8, 1, 100, 100, True, 0, 10000.0, 0, 1.0),
    (1, 3, 3, 77, 77, True, 0, 10000.0, 0, 1.0),
    (2, 2, 2, 150, 150, False, 0, 10000.0, 0, 1.0),
    (1, 4, 2, 96, 300, False, 0, 10000.0, 0, 1.0),
    (1, 4, 2, 300, 90, False, 0, 10000.0, 0, 1.0),
    (1, 4, 2, 64, 260, True, 0, 10000.0, 196, 1.0),
    (1, 4, 2, 70, 70, True, 0, 10000.0, -20, 1.0),
    (1, 4, 1, 300, 300, True, 50, 10000.0, 0, 1.0),
    (1, 4, 4, 200, 200, True, 1, 10000.0, 0, 1.0),
    (1, 4, 2, 257, 257, True, 0, 0.0, 0, 1.0),
    (1, 4, 1, 256, 256, True, 0, 500000.0, 0, 0.5),
    (1, 2, 1, 1, 1, True, 0, 10000.0, 0, 1.0),
    (1, 2, 1, 1, 33, False, 0, 10000.0, 0, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_shapes(case):
    B, Hq, Hkv, T, S, causal, w, base, pos, sigma = case
    say(f"bwd case {case}")
    q, k, v, do = workloads.make_bwd_inputs(B, Hq, Hkv, T, S, 128, "bf16", sigma=sigma, seed=700 + T + S)
    dq, dk, dv = run_fwd_bwd(q, k, v, do, causal, w, base, pos)
    rq, rk, rv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), causal, base, pos, w)
    check_grad(f64(dq), rq, "dq")
    check_grad(f64(dk), rk, "dk")
    check_grad(f64(dv), rv, "dv")
    if pos < 0:  # rows that see no key have zero gradient, exactly
        assert torch.all(dq[:, :, :-pos] == 0)


def test_bwd_deterministic():
    """No atomics: two calls give bit-identical gradients."""
    q, k, v, do = workloads.make_bwd_inputs(1, 8, 2, 333, 333, 128, "bf16", seed=41)
    a = run_fwd_bwd(q, k, v, do, True, 0, 10000.0, 0)
    b = run_fwd_bwd(q, k, v, do, True, 0, 10000.0, 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_window_covering_everything_equals_causal():
    q, k, v, do = workloads.make_bwd_inputs(1, 4, 2, 190, 190, 128, "bf16", seed=42)
    a = run_fwd_bwd(q, k, v, do, True, 0, 10000.0, 0)
    b = run_fwd_bwd(q, k, v, do, True, 190, 10000.0, 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_gqa8k_sampled():
    """The bench workload (causal GQA, B=2, Hq=32, Hkv=8, T=S=8192, RoPE 1e4) in the bench's
    launch configuration; one KV head's dk, dv at sampled keys and dq at sampled rows of its
    query heads, computed entry by entry by the oracle."""
    cfg = workloads.CONFIGS["gqa8k"]
    q, k, v, do = workloads.make_bwd_inputs(**cfg)
    say("bwd gqa8k: GPU forward + backward")
    dq, dk, dv = run_fwd_bwd(q, k, v, do, True, 0, cfg["rope_base"], 0)
    b, g = 1, 5
    keys = [0, 1, 63, 64, 127, 128, 4095, 4096, 8000, 8190, 8191]
    rows = [(h, t) for h in (20, 21, 22, 23) for t in (0, 1, 127, 128, 1000, 2047, 4097, 6000, 8191)]
    say("bwd gqa8k: oracle sampled")
    rq, rk, rv = oracle.attention_backward_sampled(f64(q), f64(k), f64(v), f64(do), b, g, keys, rows, True,
                                                   cfg["rope_base"], 0)
    gq = np.array([f64(dq[b, h, t]) for h, t in rows])
    check_grad(gq, rq, "dq rows")
    check_grad(f64(dk[b, g, keys]), rk, "dk keys")
    check_grad(f64(dv[b, g, keys]), rv, "dv keys")


def test_bwd_gqa8k_every_entry_written():
    """Every entry of dq, dk and dv of the bench workload is produced, whatever order the
    workgroups run in: gradients pre-filled with NaN come back finite."""
    from exact_transformer_attention_amd import attn_bwd, attn_fwd
    cfg = workloads.CONFIGS["gqa8k"]
    q, k, v, do = [x.cuda() for x in workloads.make_bwd_inputs(**cfg)]
    say("bwd gqa8k: every entry written")
    out, lse = attn_fwd(q, k, v, causal=True, rope_base=cfg["rope_base"])
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    attn_bwd(q, k, v, out, lse, do, causal=True, rope_base=cfg["rope_base"], dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(x).all()), f"{name} left unwritten"
