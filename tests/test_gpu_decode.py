"""Paged decode parity: attn_decode_paged and attn_paged_gather (HIP, through the C ABI)
against the fp64 oracle; block-table address translation checked bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import cases
from gpu_common import check_close, f64, say
from tolerances import DECODE_RISING_LSE

pytestmark = pytest.mark.gpu


dec_inputs = cases.decode_inputs


def run_decode(d, rope_base):
    from exact_transformer_attention_amd import attn_decode_paged
    out, lse = attn_decode_paged(d["q"].cuda(), d["k_cache"].cuda(), d["v_cache"].cuda(),
                                 d["block_table"].cuda(), d["seq_lens"].cuda(), block_size=d["block_size"],
                                 rope_base=rope_base)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(d, rope_base):
    return oracle.decode_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["block_table"].numpy(),
                               d["seq_lens"].numpy(), d["block_size"], rope_base=rope_base)


@pytest.mark.parametrize("kw", [
    dict(num_seqs=6, seq_lens=[1, 15, 16, 17, 100, 513]),
    dict(num_seqs=3, Hq=8, Hkv=8, seq_lens=[33, 2, 1024]),
    dict(num_seqs=4, Hq=16, Hkv=1, seq_lens=[700, 5, 64, 1000]),
    dict(num_seqs=8, len_lo=1, len_hi=3000),
], ids=["edges", "mha", "mqa16", "random"])
def test_decode_small(kw):
    cfg, d = dec_inputs(**kw)
    say(f"decode case {kw}")
    out, lse = run_decode(d, cfg["rope_base"])
    ro, rl = oracle_decode(d, cfg["rope_base"])
    check_close(f64(out), ro, "bf16", "decode", f64(lse), rl)


def test_decode_full_workload():
    cfg, d = dec_inputs()
    say(f"decode workload {cfg} total tokens {int(d['seq_lens'].sum())} blocks {d['num_blocks']}")
    out, lse = run_decode(d, cfg["rope_base"])
    ro, rl = oracle_decode(d, cfg["rope_base"])
    check_close(f64(out), ro, "bf16", "decode64", f64(lse), rl)


def test_decode_long_runs():
    """Enough work that each wave's run spans more than 128 cache blocks (several 64-entry
    block-table windows per piece); checked on a sample of sequences (their blocks copied
    out into a compact cache for the oracle)."""
    from exact_transformer_attention_amd import attn_decode_paged
    cfg = workloads.scaled(workloads.CONFIGS["decode64"], num_seqs=32, len_lo=22000, len_hi=26000, seed=11)
    d = workloads.make_decode_inputs(**cfg, device="cuda")
    total = int(sum((int(L) + 15) // 16 for L in d["seq_lens"].tolist())) * cfg["Hkv"]
    say(f"decode long runs: {total} (sequence, KV head, block) triples")
    assert total // 2048 > 128
    bt, sl = d["block_table"], d["seq_lens"]
    out, lse = attn_decode_paged(d["q"], d["k_cache"], d["v_cache"], bt.cuda(), sl.cuda(), block_size=16,
                                 rope_base=cfg["rope_base"])
    torch.cuda.synchronize()
    for b in (0, 7, 19, 31):
        n = (int(sl[b]) + 15) // 16
        ids = bt[b, :n].long()
        kc = d["k_cache"][ids.cuda()].cpu()
        vc = d["v_cache"][ids.cuda()].cpu()
        tb = torch.arange(n, dtype=torch.int32)[None]
        ro, rl = oracle.decode_paged(f64(d["q"][b:b + 1].cpu()), f64(kc), f64(vc), tb.numpy(), sl[b:b + 1].numpy(), 16,
                                     rope_base=cfg["rope_base"])
        check_close(f64(out[b:b + 1].cpu()), ro, "bf16", f"long runs seq {b}", f64(lse[b:b + 1].cpu()), rl)


@pytest.mark.parametrize("case", ["short", "long"])
def test_gather_bit_exact(case):
    """attn_paged_gather runs the decode kernel's own read path (runs cut into pieces, table
    entries read 64 at a time and broadcast, the next piece looked up ahead, clamped slice
    addresses, LDS staging) and copies each staged block out instead of attending to it: the
    result equals the oracle's gather bit for bit.  "short": sequences of 1-900 tokens (pieces
    crossing sequence boundaries); "long": 16 sequences of 30000-33000 tokens, so each wave's
    run spans ~125 blocks and the 64-entry table windows are refilled inside a piece."""
    from exact_transformer_attention_amd import attn_paged_gather
    if case == "short":
        cfg, d = dec_inputs(num_seqs=9, len_lo=1, len_hi=900)
        cache = d["k_cache"].cuda()
    else:
        cfg = workloads.scaled(workloads.CONFIGS["decode64"], num_seqs=16, len_lo=30000, len_hi=33000, seed=13)
        d = workloads.make_decode_inputs(**cfg, device="cuda")
        cache = d["k_cache"]
        total = int(sum((int(L) + 15) // 16 for L in d["seq_lens"].tolist())) * cfg["Hkv"]
        say(f"gather long: {total} (sequence, KV head, block) triples, {total / 2048:.0f} per wave")
        assert total // 2048 > 64
    got = attn_paged_gather(cache, d["block_table"].cuda(), d["seq_lens"].cuda())
    torch.cuda.synchronize()
    pool = cache.cpu().view(torch.int16).numpy()
    for b in range(cfg["num_seqs"]):
        L = int(d["seq_lens"][b])
        ref = oracle.gather_paged(pool, d["block_table"][b].numpy(), L, 16)
        g = got[b, :, :L].cpu().view(torch.int16).numpy()
        assert np.array_equal(g, ref), b


def test_decode_one_hot_exact():
    """q = 32 k_j (rope off): the logit gap to every other key is so large that exp2 of
    the others underflows to exactly 0, P is one-hot and the output must equal V_j bit for
    bit, whichever split and block hold token j."""
    cfg, d = dec_inputs(num_seqs=4, Hq=8, Hkv=2, seq_lens=[700, 1500, 40, 2100])
    rng = np.random.default_rng(3)
    q = d["q"].clone()
    want = torch.empty_like(q)
    for b in range(4):
        L = int(d["seq_lens"][b])
        kb = oracle.gather_paged(f64(d["k_cache"]), d["block_table"][b].numpy(), L, 16)  # [Hkv, L, d]
        vb = oracle.gather_paged(d["v_cache"].view(torch.int16).numpy(), d["block_table"][b].numpy(), L, 16)
        for h in range(8):
            g = h // 4
            for _ in range(20):
                j = int(rng.integers(L))
                qj = 32.0 * kb[g, j]
                logits = kb[g] @ qj / np.sqrt(128)
                gap = logits[j] - np.max(np.delete(logits, j))
                if gap > 110:
                    break
            assert gap > 110
            q[b, h] = torch.from_numpy(qj).to(torch.bfloat16)
            want[b, h] = torch.from_numpy(vb[g, j].copy()).view(torch.bfloat16)
    d["q"] = q
    out, _ = run_decode(d, 0.0)
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))


def test_decode_poisoned_tail_slots():
    """Slots past each sequence in its last block hold NaN in V and 1e4 in K: the kernel must
    select them away (not multiply by zero), so the result equals the clean run bit for bit."""
    cfg, d = dec_inputs(num_seqs=5, seq_lens=[1, 17, 250, 511, 1000])
    clean, clean_lse = run_decode(d, cfg["rope_base"])
    kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
    for b in range(5):
        L = int(d["seq_lens"][b])
        last = int(d["block_table"][b, (L - 1) // 16])
        s0 = L % 16
        if s0:
            kc[last, :, s0:] = 1e4
            vc[last, :, s0:] = float("nan")
    d2 = dict(d, k_cache=kc, v_cache=vc)
    out, lse = run_decode(d2, cfg["rope_base"])
    assert bool(torch.isfinite(out).all())
    assert torch.equal(out, clean) and torch.equal(lse, clean_lse)


def test_decode_logits_rising_every_block():
    """Cached keys whose logits grow along each sequence (a new maximum more than 2^8 above the
    last in each of the first 8 blocks, then level near 40 nats), so the reference is raised in
    every early block and again at the start of every piece of a split sequence.  lse is held
    to about twice the kernels' rounding model's prediction (tolerances.DECODE_RISING_LSE)."""
    d = cases.decode_rising_inputs()
    say("decode rising logits")
    out, lse = run_decode(d, 0.0)
    ro, rl = oracle_decode(d, 0.0)
    check_close(f64(out), ro, "bf16", "decode rising logits")
    le = np.abs(f64(lse) - rl).max()
    say(f"decode rising logits: lse max error {le:.3e} (lse up to {rl.max():.1f})")
    assert le <= DECODE_RISING_LSE
