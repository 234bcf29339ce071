"""Parity on seeded random shapes: the forward (causal, non-causal and sliding-window, both
head sizes) and the backward of libattn against the fp64 oracle, on shapes drawn from a fixed
seed so that every run checks the same cases.  The draws mix ragged block tails, every GQA
packing, T != S with query offsets, and RoPE bases."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from cases import RANDOM_BWD_CASES, RANDOM_FP8_CASES, RANDOM_FWD_CASES, random_fp8_case
from gpu_common import check_close, f64, say
from tolerances import FP8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c", RANDOM_FWD_CASES, ids=lambda c: f"{c['mode']}-{c['B']}x{c['Hq']}/{c['Hkv']}-"
                         f"{c['T']}x{c['S']}-d{c['d_h']}-w{c['window']}")
def test_random_forward(c):
    from exact_transformer_attention_amd import attn_fwd, attn_fwd_window
    say(f"random forward {c}")
    q, k, v = workloads.make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], T=c["T"], S=c["S"], d_h=c["d_h"],
                                        dtype="bf16", seed=c["seed"])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    # every other draw with a workspace for the keys rotated ahead, whatever the sizes
    ws = torch.empty(kd.numel() * 2, dtype=torch.uint8, device="cuda") if c["seed"] % 2 else None
    if c["mode"] == "window":
        out, lse = attn_fwd_window(qd, kd, vd, c["window"], rope_base=c["rope_base"], pos=c["pos"], workspace=ws)
    else:
        out, lse = attn_fwd(qd, kd, vd, causal=c["mode"] == "causal", rope_base=c["rope_base"], pos=c["pos"],
                            workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=c["mode"] != "full", rope_base=c["rope_base"],
                              pos=c["pos"], window=c["window"])
    check_close(f64(out), ro, "bf16", "out", f64(lse), rl)


@pytest.mark.parametrize("c", RANDOM_BWD_CASES, ids=lambda c: f"{c['mode']}-{c['B']}x{c['Hq']}/{c['Hkv']}-"
                         f"{c['T']}x{c['S']}-w{c['window']}")
def test_random_backward(c):
    from exact_transformer_attention_amd import attn_bwd, attn_fwd, attn_fwd_window
    say(f"random backward {c}")
    q, k, v, do = workloads.make_bwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], T=c["T"], S=c["S"], d_h=128,
                                            seed=c["seed"])
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    causal = c["mode"] != "full"
    if c["mode"] == "window":
        out, lse = attn_fwd_window(qd, kd, vd, c["window"], rope_base=c["rope_base"], pos=c["pos"])
    else:
        out, lse = attn_fwd(qd, kd, vd, causal=causal, rope_base=c["rope_base"], pos=c["pos"])
    dq, dk, dv = attn_bwd(qd, kd, vd, out, lse, dod, causal=causal, window=c["window"], rope_base=c["rope_base"],
                          pos=c["pos"])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), causal=causal,
                                           rope_base=c["rope_base"], pos=c["pos"], window=c["window"])
    from test_gpu_bwd import check_grad
    check_grad(f64(dq), rq, "dq")
    check_grad(f64(dk), rk, "dk")
    check_grad(f64(dv), rv, "dv")


def draw_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        ns = int(rng.integers(1, 24))
        lens = [int(x) for x in rng.integers(1, 2500, ns)]
        cases.append(dict(num_seqs=ns, Hq=Hkv * G, Hkv=Hkv, seq_lens=lens,
                          rope_base=float(rng.choice([0.0, 10000.0])), seed=2000 + i))
    return cases


@pytest.mark.parametrize("c", draw_decode_cases(10, seed=20260303),
                         ids=lambda c: f"{c['num_seqs']}seq-{c['Hq']}/{c['Hkv']}")
def test_random_decode(c):
    from exact_transformer_attention_amd import attn_decode_paged
    say(f"random decode {c}")
    d = workloads.make_decode_inputs(num_seqs=c["num_seqs"], Hq=c["Hq"], Hkv=c["Hkv"], d_h=128,
                                     seq_lens=c["seq_lens"], seed=c["seed"])
    out, lse = attn_decode_paged(d["q"].cuda(), d["k_cache"].cuda(), d["v_cache"].cuda(), d["block_table"].cuda(),
                                 d["seq_lens"].cuda(), block_size=d["block_size"], rope_base=c["rope_base"])
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["block_table"].numpy(),
                                 d["seq_lens"].numpy(), d["block_size"], rope_base=c["rope_base"])
    check_close(f64(out), ro, "bf16", "decode", f64(lse), rl)


@pytest.mark.parametrize("c", RANDOM_FP8_CASES,
                         ids=lambda c: f"{c['mode']}-{c['B']}x{c['Hq']}/{c['Hkv']}-{c['T']}x{c['S']}")
def test_random_fp8(c):
    from exact_transformer_attention_amd import attn_fwd_fp8
    T, S, causal, pos = random_fp8_case(c)
    say(f"random fp8 {c} (T={T}, S={S})")
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], T=T, S=S, d_h=128,
                                                  seed=c["seed"])
    out, lse = attn_fwd_fp8(q8.cuda(), k8.cuda(), vt8.cuda(), *sc, causal=causal, pos=pos)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fp8(q8.numpy(), k8.numpy(), vt8.numpy(), *sc, causal=causal, pos=pos)
    got, gl = f64(out), f64(lse)
    ma, rr = np.abs(got - ro).max(), oracle.rel_rms(got, ro)
    fin = np.isfinite(rl)
    le = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    say(f"fp8: max_abs={ma:.3e} rel_rms={rr:.3e} lse={le:.3e}")
    assert ma <= FP8["max_rel"] * max(np.abs(ro).max(), 1e-2) and rr <= FP8["rel_rms"] and le <= FP8["lse"]


def draw_paged_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        N = int(rng.integers(1, 5))
        cases.append(dict(N=N, Hq=Hkv * int(rng.choice([1, 2, 4])), Hkv=Hkv, T=int(rng.integers(1, 200)),
                          P=int(rng.integers(0, 700)), extra=[int(x) for x in rng.integers(0, 150, N)],
                          rope_base=float(rng.choice([0.0, 10000.0])), seed=3000 + i))
    return cases


@pytest.mark.parametrize("c", draw_paged_cases(8, seed=20260505),
                         ids=lambda c: f"{c['N']}seq-{c['Hq']}/{c['Hkv']}-T{c['T']}-P{c['P']}")
def test_random_prefill_paged(c):
    from exact_transformer_attention_amd import attn_prefill_paged
    say(f"random paged prefill {c}")
    d = workloads.make_prefill_paged_inputs(c["N"], c["Hq"], c["Hkv"], 128, c["T"], c["P"], c["extra"],
                                            seed=c["seed"])
    out, lse = attn_prefill_paged(d["q"].cuda(), d["k_cache"].cuda(), d["v_cache"].cuda(), d["block_table"].cuda(),
                                  d["seq_lens"].cuda(), block_size=d["block_size"], rope_base=c["rope_base"])
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["block_table"].numpy(),
                                  d["seq_lens"].numpy(), d["block_size"], rope_base=c["rope_base"])
    check_close(f64(out), ro, "bf16", "paged prefill", f64(lse), rl)
