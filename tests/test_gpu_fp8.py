"""FP8 prefill parity: attn_fwd_fp8 (HIP, through the C ABI) against the fp64 oracle evaluated
on the same E4M3 inputs (codes times per-tensor scales).

Tolerance: relative RMS <= 5e-2 and max-abs <= 5e-2 * max|reference| of the output; lse
max-abs <= 2e-2.  The kernel rounds the probabilities to E4M3 (3 mantissa bits) for the P V
product; an fp64 emulation of exactly that rounding (with the exact row max, the worst case
for small probabilities) gives relative RMS 1.8e-2 to 2.4e-2 and max-abs up to 1.8e-2 * max
on shapes like these, independent of length, so the bounds leave a factor of 2 to 3.  The
logits are exact products of E4M3 values summed in fp32, so lse is as accurate as in bf16."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import f64, say

pytestmark = pytest.mark.gpu

REL_RMS = 5e-2
MAX_REL = 5e-2
LSE_ABS = 2e-2


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
    assert ma <= MAX_REL * max(np.abs(ro).max(), 1e-2), msg
    assert rr <= REL_RMS, msg
    assert le <= LSE_ABS, msg


CASES = [
    # B, Hq, Hkv, T, S, causal, pos: ragged tails, every GQA packing (4, 2, 1 heads per KV
    # head and more), T != S both ways, a chunk at pos > 0, rows with no visible key
    (1, 4, 2, 200, 200, True, 0),
    (1, 8, 2, 130, 132, True, 0),
    (1, 8, 1, 100, 100, True, 0),
    (1, 3, 3, 77, 80, True, 0),
    (2, 2, 2, 150, 152, False, 0),
    (1, 4, 2, 96, 300, False, 0),
    (1, 4, 2, 300, 92, False, 0),
    (1, 4, 2, 64, 260, True, 196),
    (1, 4, 2, 70, 72, True, -20),
    (1, 2, 1, 1, 4, True, 3),
    (1, 4, 1, 1024, 1024, True, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_shapes(case):
    B, Hq, Hkv, T, S, causal, pos = case
    say(f"fp8 case {case}")
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(B, Hq, Hkv, T, S, 128, seed=900 + T + S)
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


def test_fp8_gqa8k_sampled():
    """The 8192-token causal GQA shape (B=2, Hq=32, Hkv=8) in the benchmark's launch
    configuration; sampled rows computed one by one by the oracle."""
    cfg = workloads.CONFIGS["gqa8k"]
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(**cfg)
    say("fp8 gqa8k: GPU")
    out, lse = run_fp8(q8, k8, vt8, sc, True, 0)
    rows = [(b, h, t) for b in (0, 1) for h in (0, 13, 31) for t in (0, 1, 63, 64, 4095, 8191)]
    q = oracle.fp8_e4m3_decode(q8.numpy()) * sc[0]
    k = oracle.fp8_e4m3_decode(k8.numpy()) * sc[1]
    v = np.swapaxes(oracle.fp8_e4m3_decode(vt8.numpy()), -1, -2) * sc[2]
    say("fp8 gqa8k: oracle rows")
    ro, rl = oracle.attention_rows(q, k, v, rows, causal=True)
    got = np.array([f64(out[b, h, t]) for b, h, t in rows])
    gl = np.array([float(lse[b, h, t]) for b, h, t in rows])
    ma, rr = np.abs(got - ro).max(), oracle.rel_rms(got, ro)
    say(f"fp8 gqa8k rows: max_abs={ma:.3e} rel_rms={rr:.3e} lse={np.abs(gl - rl).max():.3e}")
    assert ma <= MAX_REL * np.abs(ro).max() and rr <= REL_RMS and np.abs(gl - rl).max() <= LSE_ABS


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
