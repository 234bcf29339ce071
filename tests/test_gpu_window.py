"""Sliding-window prefill parity: attn_fwd_window (HIP, through the C ABI) against the fp64
oracle's causal sliding-window mask on the same seeded inputs."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_common import check_close, f64, gen, say

pytestmark = pytest.mark.gpu


def run_window(q, k, v, window, rope_base, pos, workspace=None):
    from exact_transformer_attention_amd import attn_fwd_window
    if workspace == "ahead":  # a workspace for keys rotated ahead, whatever the sizes
        workspace = torch.empty(k.numel() * 2, dtype=torch.uint8, device="cuda")
    out, lse = attn_fwd_window(q.cuda(), k.cuda(), v.cuda(), window, rope_base=rope_base, pos=pos,
                               workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # dtype, B, Hq, Hkv, T, S, d_h, window, rope_base, pos: windows below, at and across
    # block sizes, not multiples of them, wider than the sequence, with pos != 0, both
    # head sizes and GQA packings
    ("bf16", 1, 4, 1, 300, 300, 128, 1, 10000.0, 0),
    ("bf16", 1, 4, 1, 300, 300, 128, 17, 10000.0, 0),
    ("bf16", 1, 4, 2, 300, 300, 128, 64, 10000.0, 0),
    ("bf16", 1, 8, 2, 520, 520, 128, 100, 10000.0, 0),
    ("bf16", 2, 4, 4, 257, 257, 128, 130, 500000.0, 0),
    ("bf16", 1, 8, 2, 300, 300, 64, 77, 10000.0, 0),
    ("bf16", 1, 4, 1, 64, 400, 128, 90, 10000.0, 336),
    ("bf16", 1, 4, 1, 200, 200, 128, 10 ** 6, 10000.0, 0),
    ("bf16", 1, 2, 1, 150, 150, 128, 150, 0.0, 0),
    ("f32", 1, 2, 1, 100, 100, 64, 9, 10000.0, 0),
    ("f32", 1, 4, 2, 130, 130, 128, 70, 10000.0, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_window_shapes(case):
    dtype, B, Hq, Hkv, T, S, d, w, base, pos = case
    cfg = dict(B=B, Hq=Hq, Hkv=Hkv, T=T, S=S, d_h=d, dtype=dtype, seed=300 + T + w % 97)
    say(f"window case {case}")
    q, k, v = gen(cfg)
    out, lse = run_window(q, k, v, w, base, pos)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, rope_base=base, pos=pos, window=w)
    check_close(f64(out), ro, dtype, f"window {w}", f64(lse), rl)


@pytest.mark.parametrize("case", [c for c in CASES if c[0] == "bf16" and c[8] > 0],
                         ids=lambda c: "x".join(map(str, c)))
def test_window_keys_rotated_ahead(case):
    dtype, B, Hq, Hkv, T, S, d, w, base, pos = case
    cfg = dict(B=B, Hq=Hq, Hkv=Hkv, T=T, S=S, d_h=d, dtype=dtype, seed=300 + T + w % 97)
    say(f"window case {case}, keys rotated ahead")
    q, k, v = gen(cfg)
    out, lse = run_window(q, k, v, w, base, pos, workspace="ahead")
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, rope_base=base, pos=pos, window=w)
    check_close(f64(out), ro, dtype, f"window {w}", f64(lse), rl)


def test_window_covering_everything_equals_causal_keys_rotated_ahead():
    """With the keys rotated ahead as well: a window reaching back past key 0 gives exactly
    the causal call's result (the same rotated copy, the same kernel)."""
    from exact_transformer_attention_amd import attn_fwd, attn_fwd_window
    cfg = dict(B=1, Hq=8, Hkv=2, T=333, S=333, d_h=128, dtype="bf16", seed=32)
    q, k, v = (x.cuda() for x in gen(cfg))
    ws = torch.empty(k.numel() * 2, dtype=torch.uint8, device="cuda")
    a = attn_fwd(q, k, v, causal=True, rope_base=10000.0, workspace=ws)
    for w in (333, 5000):
        b = attn_fwd_window(q, k, v, w, rope_base=10000.0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), w


def test_window_covering_everything_equals_causal():
    """A window reaching back past key 0 must give exactly the causal kernel's result."""
    from exact_transformer_attention_amd import attn_fwd
    cfg = dict(B=1, Hq=8, Hkv=2, T=333, S=333, d_h=128, dtype="bf16", seed=31)
    q, k, v = (x.cuda() for x in gen(cfg))
    a = attn_fwd(q, k, v, causal=True, rope_base=10000.0)
    for w in (333, 5000):
        b = run_window(q, k, v, w, 10000.0, 0)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), w


def test_window_full_workload_every_work_item():
    """The 8192-token GQA workload with a 4096-key window, in the benchmark's launch
    configuration: one row of every work item (each batch, KV-head group and 64-row query
    block, a random query head of the group) plus the first 128 rows of every head, each
    evaluated by the oracle."""
    cfg = workloads.CONFIGS["gqa8k"]
    w = 4096
    q, k, v = gen(cfg)
    out, lse = run_window(q, k, v, w, cfg["rope_base"], cfg["pos"])
    assert bool(torch.isfinite(out).all())
    rows = oracle_pool.work_item_rows(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], seed=41, first_rows=128)
    say(f"window 4096: oracle on {len(rows)} rows")
    ro, rl = oracle_pool.attention_rows_grouped(oracle_pool.f32(q), oracle_pool.f32(k), oracle_pool.f32(v), rows,
                                                True, cfg["rope_base"], cfg["pos"], window=w)
    idx = (rows[:, 0], rows[:, 1], rows[:, 2])
    check_close(f64(out)[idx], ro, "bf16", "gqa8k window 4096 work items", f64(lse)[idx], rl)
