"""Helpers shared by the GPU parity tests (HIP path vs the fp64 oracle)."""

import sys

import numpy as np
import torch

import oracle
import workloads
from tolerances import TOL  # against the oracle evaluated on the same (bf16- or fp32-rounded) inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(got, ref, dtype, what, lse_got=None, lse_ref=None):
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma = oracle.max_abs(got, ref)
    rr = oracle.rel_rms(got, ref)
    msg = f"{what}: max_abs={ma:.3e} rel_rms={rr:.3e}"
    if lse_got is not None:
        lg = np.asarray(lse_got, dtype=np.float64)
        lr = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lr)
        assert np.array_equal(fin, np.isfinite(lg)), f"{what}: lse finiteness differs"
        le = oracle.max_abs(lg[fin], lr[fin]) if fin.any() else 0.0
        msg += f" lse_max_abs={le:.3e}"
        assert le <= tol["lse"], msg
    say(msg)
    assert ma <= tol["max_abs"], msg
    assert rr <= tol["rel_rms"], msg
    return ma, rr


def run_fwd_gpu(q, k, v, causal, rope_base, pos, workspace=None):
    """workspace: None (the library's choice), False (keys rotated inside the prefill) or
    "ahead" (a workspace for the rotated keys, whatever the sizes)."""
    from exact_transformer_attention_amd import attn_fwd
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if isinstance(workspace, str):
        workspace = torch.empty(kd.numel() * 2, dtype=torch.uint8, device=kd.device)
    out, lse = attn_fwd(qd, kd, vd, causal=causal, rope_base=rope_base, pos=pos, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def gen(cfg):
    return workloads.make_fwd_inputs(**cfg)
