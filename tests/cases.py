"""Inputs of the GPU parity cases whose tolerances come from the kernels' rounding model.

Shared by the GPU tests (which run the kernels on them) and the CPU error-model test (which
predicts the error those tests should see): only seeded input construction, no attention
arithmetic.
"""

import numpy as np
import torch

import workloads

# Backward: B, Hq, Hkv, T, S, causal, window, rope_base, pos, sigma.  Ragged tails, every
# GQA packing of the dQ kernel (1, 2, 4 heads per KV head and more), T != S both ways, a
# chunk at pos > 0, rows with no visible key (pos < 0), sliding windows, no RoPE, the
# long-context scale and base.
BWD_CASES = [
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


def bwd_inputs(case):
    B, Hq, Hkv, T, S, causal, w, base, pos, sigma = case
    return workloads.make_bwd_inputs(B, Hq, Hkv, T, S, 128, "bf16", sigma=sigma, seed=700 + T + S)


# FP8 prefill: B, Hq, Hkv, T, S, causal, pos.  Ragged tails, every GQA packing (4, 2, 1
# heads per KV head and more), T != S both ways, a chunk at pos > 0, rows with no visible key.
FP8_CASES = [
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


def fp8_inputs(case):
    B, Hq, Hkv, T, S, causal, pos = case
    return workloads.make_fp8_inputs(B, Hq, Hkv, T, S, 128, seed=900 + T + S)


# Forward stress inputs, away from the workloads' unit scale.

LARGE_LOGIT_SIGMAS = (2.0, 3.0)


def large_logits_inputs(sigma):
    """sigma 2 or 3: logits spread over tens of units (causal, RoPE 1e4)."""
    cfg = dict(B=1, Hq=4, Hkv=2, T=300, S=300, d_h=128, dtype="bf16", sigma=sigma, seed=31 + int(sigma))
    return cfg, workloads.make_fwd_inputs(**cfg)


def rising_logits_inputs():
    """Keys whose logits grow along the sequence to ~68 nats (non-causal, no RoPE): every
    64-key block holds a new row maximum more than 2^8 above the last one, and every term of
    q.k has the same sign."""
    B, Hq, Hkv, T, S, d = 1, 4, 1, 256, 512, 128
    g = torch.Generator("cpu").manual_seed(5)
    u = torch.randn(d, generator=g)
    q = u.view(1, 1, 1, d) + 0.1 * torch.randn(B, Hq, T, d, generator=g)
    rise = torch.linspace(0.0, 68.0 * d ** 0.5, S).view(1, 1, S, 1) / float(u @ u)
    k = rise * u.view(1, 1, 1, d) + 0.05 * torch.randn(B, Hkv, S, d, generator=g)
    v = torch.randn(B, Hkv, S, d, generator=g)
    return tuple(x.to(torch.bfloat16) for x in (q, k, v))


def large_offset_inputs():
    """Every logit near 2^15 in base-2 units (all q and k rows close to one large common
    vector) with a spread of a few units between keys (no RoPE)."""
    B, Hq, Hkv, T, S, d = 1, 4, 2, 160, 200, 128
    g = torch.Generator("cpu").manual_seed(77)
    c = 44.75  # exact in bf16; c^2 * d * log2(e) / sqrt(d) ~ 2^15
    q = torch.full((B, Hq, T, d), c)
    # each k element is c or c +- 0.25 (the bf16 grain there) with probability 2 %
    step = (torch.rand(B, Hkv, S, d, generator=g) < 0.02).float() * 0.25
    sign = torch.where(torch.rand(B, Hkv, S, d, generator=g) < 0.5, -1.0, 1.0)
    k = c + step * sign
    v = torch.randn(B, Hkv, S, d, generator=g)
    return tuple(x.to(torch.bfloat16) for x in (q, k, v))


def decode_inputs(**kw):
    cfg = workloads.scaled(workloads.CONFIGS["decode64"], **kw)
    return cfg, workloads.make_decode_inputs(**cfg)


def decode_rising_inputs():
    """Cached keys whose logits rise by 8.5 (base 2) per 16-token block for 8 blocks, then stay
    level (~47 nats), over four sequences of 40 to 1500 tokens (no RoPE)."""
    cfg, d = decode_inputs(num_seqs=4, Hq=8, Hkv=2, seq_lens=[40, 300, 700, 1500])
    g = torch.Generator("cpu").manual_seed(9)
    dh = cfg["d_h"]
    u = torch.randn(dh, generator=g)
    q = (u.view(1, 1, dh) + 0.1 * torch.randn(d["q"].shape, generator=g)).to(d["q"].dtype)
    kc = d["k_cache"].float()
    for b, L in enumerate(d["seq_lens"].tolist()):
        for j in range(L):
            phys = int(d["block_table"][b, j // 16])
            kc[phys, :, j % 16] = min(j / 16.0, 8.0) * 8.5 * dh ** 0.5 / float(u @ u) * u / 1.4427 \
                + 0.05 * torch.randn(dh, generator=g)
    return dict(d, q=q, k_cache=kc.to(d["k_cache"].dtype))


# Seeded random shapes: ragged block tails, every GQA packing, T != S with query offsets,
# RoPE bases, causal / non-causal / sliding-window.

def draw_fwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        T = int(rng.integers(1, 260))
        S = T + int(rng.choice([0, 0, int(rng.integers(1, 200))]))
        mode = str(rng.choice(["causal", "full", "window"]))
        window = int(rng.integers(1, S + 40)) if mode == "window" else 0
        cases.append(dict(B=int(rng.integers(1, 3)), Hq=Hkv * G, Hkv=Hkv, T=T, S=S,
                          d_h=int(rng.choice([64, 128])), mode=mode, window=window,
                          rope_base=float(rng.choice([0.0, 10000.0, 500000.0])), pos=S - T, seed=1000 + i))
    return cases


RANDOM_FWD_CASES = draw_fwd_cases(24, seed=20260101)
RANDOM_BWD_CASES = [c for c in draw_fwd_cases(40, seed=20260202) if c["d_h"] == 128][:8]


def random_fp8_case(c):
    """The fp8 path takes S in multiples of 4 and T <= S; returns (T, S, causal, pos)."""
    S = (c["S"] + 3) // 4 * 4
    T = min(c["T"], S)
    return T, S, c["mode"] == "causal", S - T


RANDOM_FP8_CASES = [c for c in draw_fwd_cases(40, seed=20260404) if c["mode"] != "window"][:8]
