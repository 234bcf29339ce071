"""Paged prefill parity: attn_prefill_paged (HIP, through the C ABI) against the fp64 oracle on
the same seeded inputs, with sequences sharing the physical blocks of a common prefix."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import check_close, f64, say

pytestmark = pytest.mark.gpu


def run(d, rope_base):
    from exact_transformer_attention_amd import attn_prefill_paged
    out, lse = attn_prefill_paged(d["q"].cuda(), d["k_cache"].cuda(), d["v_cache"].cuda(), d["block_table"].cuda(),
                                  d["seq_lens"].cuda(), block_size=d["block_size"], rope_base=rope_base)
    torch.cuda.synchronize()
    return out, lse


def oracle_of(d, rope_base, seqs=None, heads=None):
    seqs = range(d["q"].shape[0]) if seqs is None else seqs
    q = d["q"][list(seqs)]
    return oracle.prefill_paged(f64(q), f64(d["k_cache"]), f64(d["v_cache"]), d["block_table"][list(seqs)].numpy(),
                                d["seq_lens"][list(seqs)].numpy(), d["block_size"], rope_base=rope_base, heads=heads)


CASES = [
    # num_seqs, Hq, Hkv, T, prefix_len, extra_lens, rope_base
    (3, 8, 2, 100, 160, [0, 30, 77], 10000.0),
    (2, 4, 4, 1, 1000, [5, 0], 10000.0),
    (4, 16, 1, 64, 0, [0, 1, 63, 64], 10000.0),
    (2, 32, 8, 200, 37, [100, 3], 500000.0),
    (3, 4, 2, 17, 512, [200, 0, 9], 0.0),
    (1, 8, 2, 300, 64, [0], 10000.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:5]))
def test_prefill_paged_shapes(case):
    N, Hq, Hkv, T, P, extra, base = case
    say(f"paged prefill case {case}")
    d = workloads.make_prefill_paged_inputs(N, Hq, Hkv, 128, T, P, extra, seed=400 + T + P)
    out, lse = run(d, base)
    ro, rl = oracle_of(d, base)
    check_close(f64(out), ro, "bf16", "paged prefill", f64(lse), rl)


def test_shared_prefix_equals_private_copies():
    """Tables that share the prefix blocks give bit-identical results to private copies."""
    args = (4, 8, 2, 128, 96, 300, [0, 50, 120, 7])
    a = run(workloads.make_prefill_paged_inputs(*args, seed=51, shared=True), 10000.0)
    b = run(workloads.make_prefill_paged_inputs(*args, seed=51, shared=False), 10000.0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_one_new_token_matches_decode():
    """T = 1 is a decode step: same result as attn_decode_paged on the same cache."""
    from exact_transformer_attention_amd import attn_decode_paged
    d = workloads.make_prefill_paged_inputs(5, 32, 8, 128, 1, 700, [0, 33, 100, 901, 2], seed=61)
    out, lse = run(d, 10000.0)
    od, ld = attn_decode_paged(d["q"][:, :, 0].contiguous().cuda(), d["k_cache"].cuda(), d["v_cache"].cuda(),
                               d["block_table"].cuda(), d["seq_lens"].cuda(), block_size=16, rope_base=10000.0)
    torch.cuda.synchronize()
    check_close(f64(out[:, :, 0]), f64(od), "bf16", "prefill T=1 vs decode", f64(lse[:, :, 0]), f64(ld))


def test_prefill_paged_workload_sampled():
    """The benchmark's shared-prefix workload (8 sequences, 6144-token shared prefix, 1024 new
    tokens each) in the benchmark's launch configuration; two sequences and four heads
    checked against the oracle."""
    cfg = workloads.CONFIGS["prefix8"]
    d = workloads.make_prefill_paged_inputs(**cfg)
    out, lse = run(d, cfg["rope_base"])
    assert bool(torch.isfinite(out).all())
    heads = [0, 9, 22, 31]
    for b in (0, 7):
        ro, rl = oracle_of(d, cfg["rope_base"], seqs=[b], heads=heads)
        check_close(f64(out[b:b + 1, heads]), ro, "bf16", f"prefix8 seq {b}", f64(lse[b:b + 1, heads]), rl)
