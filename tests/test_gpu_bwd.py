"""Backward parity: attn_bwd (HIP, through the C ABI) against the fp64 oracle's chain-rule
gradients on the same seeded bf16 inputs, fed the GPU forward's out and lse.

Tolerance (per gradient tensor, tolerances.BWD): relative RMS, and max-abs relative to the
tensor's largest reference magnitude, each about twice what the kernels' rounding model
(error_model.backward_bf16) predicts over these cases."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from cases import BWD_CASES, bwd_inputs
from gpu_common import f64, say
from tolerances import BWD

pytestmark = pytest.mark.gpu


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    # A gradient that is exactly zero in exact arithmetic (window 1: each row attends only
    # to itself, so dS = P * (dP - rowsum(dO * O)) cancels to 0) comes out at the rounding
    # level of its O(1) terms: the scale of the max-abs bound is floored for it.
    scale = max(np.abs(ref).max(), BWD["scale_floor"])
    ma = np.abs(got - ref).max()
    rr = oracle.rel_rms(got, ref) if np.abs(ref).max() >= BWD["scale_floor"] else 0.0
    msg = f"{what}: max_abs={ma:.3e} (scale {scale:.3e}) rel_rms={rr:.3e}"
    say(msg)
    assert ma <= BWD["max_rel"] * scale, msg
    assert rr <= BWD["rel_rms"], msg


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


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_shapes(case):
    B, Hq, Hkv, T, S, causal, w, base, pos, sigma = case
    say(f"bwd case {case}")
    q, k, v, do = bwd_inputs(case)
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


def test_bwd_gqa8k_every_work_item():
    """The bench workload (causal GQA, B=2, Hq=32, Hkv=8, T=S=8192, RoPE 1e4) in the bench's
    launch configuration.  For every (batch, KV head): dk and dv at one random key of every
    128-key block (each a work item of the dK/dV kernel) and dq at one random row of every
    64-row query block of a random query head of the group (each a work item of the dQ
    kernel), computed entry by entry by the oracle; the 16 KV heads in worker processes."""
    cfg = workloads.CONFIGS["gqa8k"]
    q, k, v, do = workloads.make_bwd_inputs(**cfg)
    say("bwd gqa8k: GPU forward + backward")
    dq, dk, dv = run_fwd_bwd(q, k, v, do, True, 0, cfg["rope_base"], 0)
    B, Hq, Hkv, T, S = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["S"]
    G = Hq // Hkv
    rng = np.random.default_rng(45)
    qf, kf, vf, dof = (oracle_pool.f32(x) for x in (q, k, v, do))
    tasks, picks = [], []
    for b in range(B):
        for g in range(Hkv):
            keys = [kb * 128 + int(rng.integers(128)) for kb in range(S // 128)]
            rows = [(g * G + int(rng.integers(G)), qb * 64 + int(rng.integers(64))) for qb in range(T // 64)]
            # the group's slices only (batch 0, KV head 0 of the slice, query heads 0..G-1)
            sl_q, sl_kv = (slice(b, b + 1), slice(g * G, (g + 1) * G)), (slice(b, b + 1), slice(g, g + 1))
            tasks.append(("attention_backward_sampled",
                          (qf[sl_q], kf[sl_kv], vf[sl_kv], dof[sl_q], 0, 0, keys, [(h - g * G, t) for h, t in rows]),
                          dict(causal=True, rope_base=cfg["rope_base"], pos=0)))
            picks.append((b, g, keys, rows))
    say(f"bwd gqa8k: oracle on {len(tasks)} KV heads")
    res = oracle_pool.run(tasks)
    gq, rq, gk, rk, gv, rv = [], [], [], [], [], []
    for (b, g, keys, rows), (q_ref, k_ref, v_ref) in zip(picks, res):
        gq.append(np.array([f64(dq[b, h, t]) for h, t in rows]))
        rq.append(q_ref)
        gk.append(f64(dk[b, g, keys]))
        rk.append(k_ref)
        gv.append(f64(dv[b, g, keys]))
        rv.append(v_ref)
    check_grad(np.concatenate(gq), np.concatenate(rq), "dq work items")
    check_grad(np.concatenate(gk), np.concatenate(rk), "dk work items")
    check_grad(np.concatenate(gv), np.concatenate(rv), "dv work items")


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
