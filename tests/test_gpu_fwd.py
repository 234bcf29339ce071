"""Prefill parity: libattn's attn_fwd (HIP, through the C ABI) against the fp64 oracle on
the same seeded inputs."""

import os

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
import cases
from gpu_common import check_close, f64, gen, run_fwd_gpu, say
from tolerances import LARGE_LOGITS, OFFSET_LSE, RISING_LSE

pytestmark = pytest.mark.gpu


def full_case(dtype, B, Hq, Hkv, T, S, d_h, causal, rope_base, pos, seed, sigma=1.0, workspace=None):
    cfg = dict(B=B, Hq=Hq, Hkv=Hkv, T=T, S=S, d_h=d_h, dtype=dtype, sigma=sigma, seed=seed)
    say(f"case {cfg} causal={causal} rope={rope_base} pos={pos} workspace={workspace}")
    q, k, v = gen(cfg)
    out, lse = run_fwd_gpu(q, k, v, causal, rope_base, pos, workspace)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=causal, rope_base=rope_base, pos=pos)
    check_close(f64(out), ro, dtype, "out", f64(lse), rl)


# ---------------------------------------------------------------- fp32 ----

def test_small_f32_workload():
    cfg = workloads.CONFIGS["small_f32"]
    full_case("f32", cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["S"], cfg["d_h"], cfg["causal"],
              cfg["rope_base"], cfg["pos"], cfg["seed"])


F32_CASES = [
    # B, Hq, Hkv, T, S, d_h, causal, rope_base, pos
    (1, 1, 1, 1, 1, 64, False, 0.0, 0),
    (1, 2, 1, 33, 33, 64, True, 10000.0, 0),
    (2, 4, 2, 100, 100, 128, True, 10000.0, 0),
    (1, 3, 1, 70, 150, 128, False, 500000.0, 0),
    (1, 2, 2, 40, 200, 64, True, 10000.0, 160),
    (1, 8, 2, 129, 129, 128, False, 0.0, 0),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c)))
def test_f32_shapes(case):
    B, Hq, Hkv, T, S, d, causal, base, pos = case
    full_case("f32", B, Hq, Hkv, T, S, d, causal, base, pos, seed=100 + T)


# ---------------------------------------------------------------- bf16 ----

BF16_CASES = [
    # several 64-key blocks and a ragged tail, every GQA packing (1, 2, 4 heads per KV head and
    # a group of 3), both head sizes, causal and not, RoPE and not, T != S and pos != 0
    (1, 4, 4, 200, 200, 128, True, 10000.0, 0),
    (1, 4, 1, 200, 200, 128, True, 10000.0, 0),
    (1, 4, 2, 200, 200, 128, False, 10000.0, 0),
    (2, 6, 2, 130, 130, 128, True, 500000.0, 0),
    (1, 8, 2, 300, 300, 64, True, 10000.0, 0),
    (1, 2, 1, 77, 300, 128, False, 0.0, 0),
    (1, 4, 1, 64, 320, 128, True, 10000.0, 256),
    (1, 2, 2, 1, 1, 128, True, 10000.0, 0),
    (1, 4, 4, 1, 500, 128, True, 10000.0, 499),
    (1, 1, 1, 257, 257, 128, True, 10000.0, 0),
    (1, 4, 1, 520, 520, 128, True, 10000.0, 0),
    (1, 16, 2, 96, 96, 64, False, 0.0, 0),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bf16_shapes(case):
    B, Hq, Hkv, T, S, d, causal, base, pos = case
    full_case("bf16", B, Hq, Hkv, T, S, d, causal, base, pos, seed=200 + T + S)


# Keys rotated once ahead of the prefill (a workspace given whatever the sizes): the RoPE
# cases above, every head packing and both head sizes.
AHEAD_CASES = [c for c in BF16_CASES if c[7] > 0]


@pytest.mark.parametrize("case", AHEAD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bf16_keys_rotated_ahead(case):
    B, Hq, Hkv, T, S, d, causal, base, pos = case
    full_case("bf16", B, Hq, Hkv, T, S, d, causal, base, pos, seed=200 + T + S, workspace="ahead")


def test_bf16_workspace_use():
    """The rotated copy is rebuilt on every call (a poisoned workspace changes nothing); a
    workspace too small for it, or none, runs the rotation inside the prefill (the same bits
    as with no workspace); the library asks for one only when each key block has many readers."""
    from exact_transformer_attention_amd import attn_fwd, attn_fwd_workspace_bytes
    cfg = dict(B=1, Hq=8, Hkv=2, T=700, S=700, d_h=128, dtype="bf16", sigma=1.0, seed=4242)
    q, k, v = (t.cuda() for t in gen(cfg))
    need = k.numel() * 2
    ws = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    o1, l1 = attn_fwd(q, k, v, causal=True, rope_base=10000.0, workspace=ws)
    ws.fill_(0x7F)
    o2, l2 = attn_fwd(q, k, v, causal=True, rope_base=10000.0, workspace=ws)
    o3, l3 = attn_fwd(q, k, v, causal=True, rope_base=10000.0, workspace=False)
    o4, l4 = attn_fwd(q, k, v, causal=True, rope_base=10000.0, workspace=ws[:need - 16])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    assert attn_fwd_workspace_bytes(1, 8, 2, 700, 700, 128, True, 0, 10000.0, 0) == 0
    # fp32 inputs ignore a workspace (no rotated copy is made for the fp32 path)
    qf, kf, vf = q.float(), k.float(), v.float()
    f1 = attn_fwd(qf, kf, vf, causal=True, rope_base=10000.0, workspace=ws)
    f2 = attn_fwd(qf, kf, vf, causal=True, rope_base=10000.0, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(f1[0], f2[0]) and torch.equal(f1[1], f2[1])
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, rope_base=10000.0, pos=0)
    check_close(f64(o1), ro, "bf16", "out (rotated ahead)", f64(l1), rl)
    check_close(f64(o3), ro, "bf16", "out (rotated in the prefill)", f64(l3), rl)


def test_bf16_fully_masked_rows():
    """pos < 0 with causal leaves the first rows without any visible key: output 0, lse -inf."""
    cfg = dict(B=1, Hq=4, Hkv=1, T=100, S=100, d_h=128, dtype="bf16", seed=7)
    q, k, v = gen(cfg)
    for dtype in ("bf16", "f32"):
        qq, kk, vv = (x.float() for x in (q, k, v)) if dtype == "f32" else (q, k, v)
        out, lse = run_fwd_gpu(qq, kk, vv, True, 10000.0, -5)
        ro, rl = oracle.attention(f64(qq), f64(kk), f64(vv), causal=True, rope_base=10000.0, pos=-5)
        o = f64(out)
        assert np.all(o[:, :, :5] == 0) and np.all(np.isneginf(f64(lse)[:, :, :5]))
        check_close(o, ro, dtype, f"masked rows {dtype}", f64(lse), rl)


def test_bf16_deterministic():
    cfg = dict(B=1, Hq=8, Hkv=2, T=300, S=300, d_h=128, dtype="bf16", seed=8)
    q, k, v = gen(cfg)
    a = run_fwd_gpu(q, k, v, True, 10000.0, 0)
    b = run_fwd_gpu(q, k, v, True, 10000.0, 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------- full workloads ----

@pytest.mark.parametrize("name", ["mha2k", "gqa8k"])
def test_full_workload_every_element(name):
    """The causal MHA (B=4, 32 heads, T=S=2048) and GQA (B=2, 32/8 heads, T=S=8192) workloads
    in the launch configuration the benchmark times, compared with the oracle over the whole
    output and lse (every head evaluated by the oracle in a worker process)."""
    cfg = workloads.CONFIGS[name]
    say(f"workload {name}: {cfg}")
    q, k, v = gen(cfg)
    out, lse = run_fwd_gpu(q, k, v, cfg["causal"], cfg["rope_base"], cfg["pos"])
    say(f"workload {name}: oracle on {oracle_pool.pool_size()} workers")
    ro, rl = oracle_pool.attention_per_head(oracle_pool.f32(q), oracle_pool.f32(k), oracle_pool.f32(v),
                                            cfg["causal"], cfg["rope_base"], cfg["pos"])
    check_close(f64(out), ro, "bf16", f"{name} every element", f64(lse), rl)


def test_gqa32k_every_work_item():
    """The 32768-token GQA workload in the benchmark's launch configuration: one row of every
    work item of the kernel (each batch, KV-head group and 64-row query block, a random query
    head of the group) and the first 256 rows of every head, each evaluated by the oracle."""
    cfg = workloads.CONFIGS["gqa32k"]
    say(f"workload gqa32k: {cfg}")
    q, k, v = gen(cfg)
    out, lse = run_fwd_gpu(q, k, v, cfg["causal"], cfg["rope_base"], cfg["pos"])
    assert bool(torch.isfinite(out).all()), "non-finite output"
    rows = oracle_pool.work_item_rows(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], seed=cfg["seed"], first_rows=256)
    say(f"workload gqa32k: oracle on {len(rows)} rows")
    ro, rl = oracle_pool.attention_rows_grouped(oracle_pool.f32(q), oracle_pool.f32(k), oracle_pool.f32(v), rows,
                                                cfg["causal"], cfg["rope_base"], cfg["pos"])
    idx = (rows[:, 0], rows[:, 1], rows[:, 2])
    check_close(f64(out)[idx], ro, "bf16", "gqa32k work items", f64(lse)[idx], rl)


def test_gqa8k_keys_rotated_in_kernel_every_work_item():
    """The 8192-token GQA workload with no workspace (each K block rotated as it lands, the
    path a C caller without a workspace takes): one row of every work item, by the oracle."""
    cfg = workloads.CONFIGS["gqa8k"]
    say(f"workload gqa8k, keys rotated in the kernel: {cfg}")
    q, k, v = gen(cfg)
    out, lse = run_fwd_gpu(q, k, v, cfg["causal"], cfg["rope_base"], cfg["pos"], workspace=False)
    assert bool(torch.isfinite(out).all()), "non-finite output"
    rows = oracle_pool.work_item_rows(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], seed=cfg["seed"] + 1)
    say(f"workload gqa8k: oracle on {len(rows)} rows")
    ro, rl = oracle_pool.attention_rows_grouped(oracle_pool.f32(q), oracle_pool.f32(k), oracle_pool.f32(v), rows,
                                                cfg["causal"], cfg["rope_base"], cfg["pos"])
    idx = (rows[:, 0], rows[:, 1], rows[:, 2])
    check_close(f64(out)[idx], ro, "bf16", "gqa8k work items (keys rotated in the kernel)", f64(lse)[idx], rl)


@pytest.mark.parametrize("name", ["mha2k", "gqa8k", "gqa32k"])
def test_full_workload_every_row_written(name):
    """Every (batch, head, row) of a full-size workload is produced by exactly one work item,
    whatever order the workgroups run in: outputs pre-filled with NaN come back finite."""
    from exact_transformer_attention_amd import attn_fwd
    cfg = workloads.CONFIGS[name]
    say(f"workload {name}: every row written")
    q, k, v = [x.cuda() for x in gen(cfg)]
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, causal=cfg["causal"], rope_base=cfg["rope_base"], pos=cfg["pos"], out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "rows left unwritten"
    assert bool(torch.isfinite(lse).all()), "lse left unwritten"


@pytest.mark.parametrize("sigma", cases.LARGE_LOGIT_SIGMAS)
def test_bf16_large_logits(sigma):
    """Inputs with sigma 2-3 spread the logits over tens of units, so the running reference is
    raised often and by large steps (the rare rescaling path).  The bf16 rounding of the
    rotated, scaled q and the rotated k perturbs each logit by ~2^-9 of its size (~sigma^2)
    and the output by that times |v| (~sigma); the bounds are about twice what the kernels'
    rounding model predicts on these inputs (tolerances.LARGE_LOGITS)."""
    cfg, (q, k, v) = cases.large_logits_inputs(sigma)
    say(f"large logits {cfg}")
    out, lse = run_fwd_gpu(q, k, v, True, 10000.0, 0)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, rope_base=10000.0)
    o, l = f64(out), f64(lse)
    ma, rr, le = oracle.max_abs(o, ro), oracle.rel_rms(o, ro), oracle.max_abs(l, rl)
    say(f"sigma {sigma}: max_abs={ma:.3e} rel_rms={rr:.3e} lse={le:.3e}")
    tol = LARGE_LOGITS[sigma]
    assert rr <= tol["rel_rms"] and ma <= tol["max_abs"] and le <= tol["lse"]


def test_bf16_logits_rising_every_block():
    """Keys whose logits grow along the sequence: every 64-key block holds a new row maximum
    more than 2^8 above the last one, so the reference is raised in every block.  The logits
    reach ~72 and are coherent sums (every term of q.k has the same sign), so the roundings of
    the scaled q add up rather than cancel: the output keeps the workload bounds, lse is held
    to about twice the model's prediction (tolerances.RISING_LSE)."""
    q, k, v = cases.rising_logits_inputs()
    out, lse = run_fwd_gpu(q, k, v, False, 0.0, 0)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=False)
    say(f"rising logits: lse range {rl.min():.1f}..{rl.max():.1f} (nats)")
    check_close(f64(out), ro, "bf16", "rising logits")
    le = np.abs(f64(lse) - rl).max()
    say(f"rising logits: lse max error {le:.3e}")
    assert le <= RISING_LSE


@pytest.mark.gpu
def test_binding_imported_before_torch_launches():
    """A process that imports the binding before torch still runs the kernels on torch's
    tensors and stream (the binding brings torch's HIP runtime in first)."""
    import subprocess
    import sys
    code = "\n".join([
        "import exact_transformer_attention_amd._lib as L",
        "import numpy as np, torch, oracle, workloads",
        "q, k, v = workloads.make_fwd_inputs(1, 4, 2, 80, 80, 128, dtype='bf16', seed=11)",
        "dev = torch.device('cuda:0')",
        "out, lse = L.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, rope_base=10000.0)",
        "torch.cuda.synchronize()",
        "ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),",
        "                       causal=True, rope_base=10000.0)",
        "ref = ref[0] if isinstance(ref, tuple) else ref",
        "print('maxabs', float(np.abs(out.float().cpu().double().numpy() - ref).max()), flush=True)",
    ])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("binding-before-torch subprocess: attn_fwd 1x4x2 T=S=80 d_h=128 causal bf16")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240,
                       env=dict(os.environ, PYTHONPATH=root + os.pathsep + os.path.join(root, "tests")))
    assert r.returncode == 0, r.stderr[-3000:]
    err = float(r.stdout.strip().splitlines()[-1].split()[1])
    say(f"binding-before-torch: max abs error {err:.3e}")
    assert err <= 2e-2


def test_bf16_large_common_logit_offset():
    """Every logit sits near 2^15 in base-2 units (all q and k rows close to one large common
    vector), with a spread of a few units between keys.  The softmax only sees the differences;
    the running reference must be able to sit at 2^15 with a fine enough grain that the
    probabilities do not underflow (a bf16 reference has a grain of 256 there, which would
    leave every probability below 2^-128).  No RoPE, so the bf16 rounding of the scaled q is
    one common factor (relative 2.2e-3 here) on every logit: the output keeps the workload
    bounds and lse, scaled by that factor, is held to about twice the model's prediction
    (tolerances.OFFSET_LSE)."""
    q, k, v = cases.large_offset_inputs()
    for causal in (False, True):
        out, lse = run_fwd_gpu(q, k, v, causal, 0.0, 0)
        ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=causal)
        say(f"large offset causal={causal}: lse {rl.min():.1f}..{rl.max():.1f} nats "
            f"({rl.max() / np.log(2):.0f} in base 2)")
        assert np.isfinite(f64(lse)).all(), "lse not finite"
        check_close(f64(out), ro, "bf16", f"large common offset causal={causal}")
        le = np.abs(f64(lse) - rl).max()
        say(f"large offset causal={causal}: lse max error {le:.3e}")
        assert le <= OFFSET_LSE
