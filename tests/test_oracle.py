"""The fp64 oracle against closed forms, invariants, a scalar brute force and a library SDPA."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_attention_rows_matches_full():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 4, 20, 16))
    k = rng.standard_normal((2, 2, 20, 16))
    v = rng.standard_normal((2, 2, 20, 16))
    o, l = oracle.attention(q, k, v, causal=True, rope_base=500000.0, pos=0)
    rows = [(0, 0, 0), (1, 3, 19), (0, 2, 7), (1, 1, 13)]
    o2, l2 = oracle.attention_rows(q, k, v, rows, causal=True, rope_base=500000.0, pos=0)
    for i, (b, h, t) in enumerate(rows):
        assert np.allclose(o2[i], o[b, h, t], atol=1e-14)
        assert abs(l2[i] - l[b, h, t]) < 1e-14


def test_row_block_does_not_change_result():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 33, 8))
    k = rng.standard_normal((1, 1, 33, 8))
    v = rng.standard_normal((1, 1, 33, 8))
    a = oracle.attention(q, k, v, causal=True, rope_base=10000.0)
    b = oracle.attention(q, k, v, causal=True, rope_base=10000.0, row_block=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fully_masked_row_defined():
    """pos + t < 0 leaves a row with no visible key: output 0, lse = -inf, no NaN."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 4, 8))
    k = rng.standard_normal((1, 1, 4, 8))
    v = rng.standard_normal((1, 1, 4, 8))
    o, l = oracle.attention(q, k, v, causal=True, pos=-2)
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(l[0, 0, :2]))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l[0, 0, 2:]))


def test_logit_variance_matches_scale():
    """Unit-variance q, k give q.k variance d_k; dividing by sqrt(d_k) brings it back to 1
    ("Why is attention scaled by 1/sqrt(dk)?").  With sigma = 0.5 the scaled logits have
    variance sigma^4.  Checks the generators and the scale together."""
    for name in ("mha2k", "gqa32k"):
        cfg = workloads.CONFIGS[name]
        q, k, _ = workloads.make_fwd_inputs(**workloads.scaled(cfg, B=1, Hq=2, Hkv=2, T=512, S=512))
        qf = q.double().numpy()[0, 0]
        kf = k.double().numpy()[0, 0]
        logits = (qf @ kf.T) / math.sqrt(cfg["d_h"])
        want = cfg["sigma"] ** 4
        assert abs(logits.var() / want - 1.0) < 0.05, (name, logits.var(), want)


def test_pages_figures_golden():
    """Analytic figures the pages print, checked against the accounting the bench uses."""
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        g = json.load(f)
    # attention FLOPs per token per layer = 4*T*d with d = Hq*d_h
    fig = g["attention_flops_per_token"]
    B, Hq, T, d_h = 1, 32, 4096, 128
    per_token = workloads.fwd_flops(B, Hq, T, T, d_h, causal=False) / (B * T)
    assert per_token == fig["factor"] * T * (Hq * d_h)
    # crossover 4*T*d = 24*d^2  ->  T = 6d, about 24k tokens at d = 4096
    c = g["crossover"]
    d = c["d"]
    T_cross = c["projection_factor"] * d * d / (fig["factor"] * d)
    assert T_cross == c["ratio_to_d"] * d
    assert abs(T_cross - c["approx_tokens"]) / c["approx_tokens"] < 0.03
    # KV cache bytes = 2 * layers * heads * head_dim * seq_len * batch * bytes
    kv = g["kv_cache_bytes"]
    for ex in kv["examples"]:
        got = workloads.decode_kv_bytes([ex["seq_len"]] * ex["batch"], ex["heads"], ex["head_dim"],
                                        ex["bytes_per_element"]) * ex["layers"]
        want = kv["factor"]
        for f in ("layers", "heads", "head_dim", "seq_len", "batch", "bytes_per_element"):
            want *= ex[f]
        assert got == want, ex


def test_generators_deterministic_and_rounded():
    cfg = workloads.scaled(workloads.CONFIGS["gqa8k"], T=64, S=64)
    a = workloads.make_fwd_inputs(**cfg)
    b = workloads.make_fwd_inputs(**cfg)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    assert a[0].shape == (2, 32, 64, 128) and a[1].shape == (2, 8, 64, 128)
    d = workloads.make_decode_inputs(**workloads.scaled(workloads.CONFIGS["decode64"], num_seqs=5,
                                                        len_lo=1, len_hi=50))
    L = d["seq_lens"].tolist()
    nb = [(x + 15) // 16 for x in L]
    assert d["num_blocks"] == sum(nb)
    used = np.concatenate([d["block_table"][b, :n].numpy() for b, n in enumerate(nb)])
    assert sorted(used.tolist()) == list(range(sum(nb)))          # a permutation of the pool
    for b, n in enumerate(nb):
        assert np.all(d["block_table"][b, n:].numpy() == -1)
