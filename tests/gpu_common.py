"""Helpers shared by the GPU parity tests (HIP path vs the fp64 oracle)."""

import sys

import numpy as np
import torch

import oracle
import workloads

# Tolerances: fp32 max-abs 1e-5; bf16 max-abs 2e-2 and relative RMS 1e-2, against the
# oracle evaluated on the same (bf16- or fp32-rounded) inputs.
TOL = {"f32": dict(max_abs=1e-5, rel_rms=1e-5, lse=1e-5),
       "bf16": dict(max_abs=2e-2, rel_rms=1e-2, lse=2e-2)}


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


def sample_rows(B, Hq, T, n, seed):
    """(b, h, t) rows to check at full size: the first and last rows of several heads plus
    random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        for h in (0, Hq - 1, Hq // 2):
            for t in (0, 1, 2, 3, 63, 64, 127, 128, T // 2, T - 2, T - 1):
                if 0 <= t < T:
                    rows.add((b, h, t))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))))
    return np.array(sorted(rows), dtype=np.int64)


def run_fwd_gpu(q, k, v, causal, rope_base, pos):
    from exact_transformer_attention_amd import attn_fwd
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = attn_fwd(qd, kd, vd, causal=causal, rope_base=rope_base, pos=pos)
    torch.cuda.synchronize()
    return out, lse


def gen(cfg):
    return workloads.make_fwd_inputs(**cfg)
