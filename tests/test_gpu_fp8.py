"""FP8 prefill parity: attn_fwd_fp8 (HIP, through the C ABI) against the fp64 oracle evaluated
on the same E4M3 inputs (codes times per-tensor scales).

Tolerance (tolerances.FP8): relative RMS and max-abs relative to the output's largest
reference magnitude, each about twice what the kernel's rounding model predicts over these
cases (the probabilities are rounded to E4M3, 3 mantissa bits, for the P V product, against
the kernel's lazily held reference: error_model.forward_fp8); lse, whose logits are exact
products of E4M3 values, to 1e-3."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from cases import FP8_CASES, fp8_inputs
from gpu_common import f64, say
from tolerances import FP8

pytestmark = pytest.mark.gpu


def run_fp8(q8, k8, vt8, scales, causal, pos):
    from exact_transformer_attention_amd import attn_fwd_fp8
    out, lse = attn_fwd_fp8(q8.cuda(), k8.cuda(), vt8.cuda(), *scales, causal=causal, pos=pos)
    torch.cuda.synchronize()
    return out, lse


def check(out, lse, ro, rl, what):
    got = f64(out)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma = np.abs(got - ro).max()
    rr = oracle.rel_rms(got, ro)
    lg = f64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lg)), f"{what}: lse finiteness differs"
    le = np.abs(lg[fin] - rl[fin]).max() if fin.any() else 0.0
    msg = f"{what}: max_abs={ma:.3e} (scale {np.abs(ro).max():.3e}) rel_rms={rr:.3e} lse_max_abs={le:.3e}"
    say(msg)
    assert ma <= FP8["max_rel"] * max(np.abs(ro).max(), 1e-2), msg
    assert rr <= FP8["rel_rms"], msg
    assert le <= FP8["lse"], msg


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_shapes(case):
    B, Hq, Hkv, T, S, causal, pos = case
    say(f"fp8 case {case}")
    (q8, k8, vt8), sc = fp8_inputs(case)
    out, lse = run_fp8(q8, k8, vt8, sc, causal, pos)
    ro, rl = oracle.attention_fp8(q8.numpy(), k8.numpy(), vt8.numpy(), *sc, causal=causal, pos=pos)
    check(out, lse, ro, rl, "fp8")
    if pos < 0:
        assert torch.all(out[:, :, :-pos] == 0) and torch.all(torch.isinf(lse[:, :, :-pos]))


def test_fp8_scales_fold():
    """Scaling q up and k down by the same factor changes nothing; v's scale scales the output."""
    (q8, k8, vt8), (sq, sk, sv) = workloads.make_fp8_inputs(1, 4, 2, 256, 256, 128, seed=77)
    a = run_fp8(q8, k8, vt8, (sq, sk, sv), True, 0)
    b = run_fp8(q8, k8, vt8, (sq * 4, sk / 4, sv * 2), True, 0)
    assert torch.allclose(b[1], a[1], atol=1e-5)
    assert torch.allclose(b[0].float(), 2 * a[0].float(), rtol=1e-2, atol=1e-3)


def test_fp8_gqa8k_every_work_item():
    """The 8192-token causal GQA shape (B=2, Hq=32, Hkv=8) in the benchmark's launch
    configuration: one row of every work item (each batch, KV-head group and 64-row query
    block, a random query head of the group) plus the first 64 rows of every head, each
    evaluated by the oracle on the decoded fp8 values."""
    cfg = workloads.CONFIGS["gqa8k"]
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(**cfg)
    say("fp8 gqa8k: GPU")
    out, lse = run_fp8(q8, k8, vt8, sc, True, 0)
    rows = oracle_pool.work_item_rows(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], seed=43, first_rows=64)
    q = oracle.fp8_e4m3_decode(q8.numpy()) * sc[0]
    k = oracle.fp8_e4m3_decode(k8.numpy()) * sc[1]
    v = np.swapaxes(oracle.fp8_e4m3_decode(vt8.numpy()), -1, -2) * sc[2]
    say(f"fp8 gqa8k: oracle on {len(rows)} rows")
    ro, rl = oracle_pool.attention_rows_grouped(q, k, np.ascontiguousarray(v), rows, True, 0.0)
    idx = (rows[:, 0], rows[:, 1], rows[:, 2])
    got, gl = f64(out)[idx], f64(lse)[idx]
    ma, rr = np.abs(got - ro).max(), oracle.rel_rms(got, ro)
    say(f"fp8 gqa8k work items: max_abs={ma:.3e} rel_rms={rr:.3e} lse={np.abs(gl - rl).max():.3e}")
    assert ma <= FP8["max_rel"] * np.abs(ro).max() and rr <= FP8["rel_rms"] and np.abs(gl - rl).max() <= FP8["lse"]


def test_fp8_gqa8k_every_row_written():
    """Every row of the 8192-token shape is produced whatever order the workgroups run in:
    outputs pre-filled with NaN come back finite."""
    from exact_transformer_attention_amd import attn_fwd_fp8
    cfg = workloads.CONFIGS["gqa8k"]
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(**cfg)
    q8, k8, vt8 = q8.cuda(), k8.cuda(), vt8.cuda()
    say("fp8 gqa8k: every row written")
    out = torch.full(q8.shape, float("nan"), dtype=torch.bfloat16, device=q8.device)
    lse = torch.full(q8.shape[:3], float("nan"), dtype=torch.float32, device=q8.device)
    attn_fwd_fp8(q8, k8, vt8, *sc, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all()), "rows left unwritten"
