"""Benchmark of the attention hot path on one MI355X.

One step = one causal GQA prefill (B=2, Hq=32, Hkv=8, T=S=8192, d_h=128, bf16, RoPE 1e4;
attn_fwd) followed by one paged decode step (64 sequences, lengths uniform in
[512, 8192], Hq=32, Hkv=8, block 16; attn_decode_paged), on synthetic seeded inputs
already resident in HBM.

Prints one JSON line.  value = prefill TFLOP/s (4*B*Hq*T*S*d_h, halved for causal)
measured with HIP events on the stream the kernels run on; the decode step is reported
beside it in KV bytes read per second (sum_b L_b*Hkv*d_h*2*2 bytes).  Each comes with
its roofline fraction (bf16 dense MFMA 2516.6 TFLOP/s; HBM 8 TB/s) and the fp64 oracle
timed on the host cores on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0          # HBM3E
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 (E4M3) MFMA: twice the bf16 rate


def kernel_sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["exact_transformer_attention_amd/csrc/fwd_bf16.hip",
                   "exact_transformer_attention_amd/csrc/prefill_common.h",
                   "exact_transformer_attention_amd/csrc/attn_common.h",
                   "exact_transformer_attention_amd/csrc/fwd_params.h"]
DECODE_SOURCES = ["exact_transformer_attention_amd/csrc/decode.hip",
                  "exact_transformer_attention_amd/csrc/attn_common.h",
                  "exact_transformer_attention_amd/csrc/launchers.h"]


def measured_traffic(kind, digest):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(kind)
    if not t or t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def summarize_pmc(fetch_csv, write_csv, out_dir, extra_kind=None):
    """Per-launch HBM traffic of the timed kernels from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE; kilobytes per dispatch), scaled by the factor the same counters read
    for a plain 1 GiB device copy (run with --copy-calibration).  Writes
    profiles/traffic.json (read back by the benchmark line) and a readable summary."""
    import collections
    import csv

    def per_kernel(path, counter):
        rows = list(csv.DictReader(open(path)))
        disp = collections.defaultdict(float)
        name = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            disp[r["Dispatch_Id"]] += float(r["Counter_Value"])
            name[r["Dispatch_Id"]] = r["Kernel_Name"]
        by = collections.defaultdict(list)
        for d, v in disp.items():
            by[name[d]].append(v * 1024.0)  # KiB -> bytes
        return by

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(by, key):
        vals = [v for k, vs in by.items() if key in k for v in vs]
        return sum(vals) / len(vals) if vals else None

    copy_bytes = float(1 << 30)

    def calib(by):
        # the calibration copies are the three largest device-copy dispatches
        vals = sorted((v for k, vs in by.items() if "copyBuffer" in k for v in vs), reverse=True)[:3]
        return sorted(vals)[len(vals) // 2] if vals else None

    f_copy = calib(fetch)
    w_copy = calib(write)
    f_scale = copy_bytes / f_copy if f_copy else 1.0
    w_scale = copy_bytes / w_copy if w_copy else 1.0
    res = {"calibration": {"kernel": "1 GiB device copy", "fetch_raw_bytes": f_copy, "write_raw_bytes": w_copy,
                           "fetch_scale": f_scale, "write_scale": w_scale}}
    # kernels of one timed call; a name ending in "?" is launched only for some sizes (the
    # keys rotated ahead of the prefill) and counts zero when absent
    prefill_kernels = ["fwd_bf16_kernel", "rope_k_kernel?"]
    kinds = (((extra_kind, ["bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"], BWD_SOURCES),)
             if extra_kind == "bwd" else
             ((extra_kind, ["fwd_fp8_kernel"], FP8_SOURCES),) if extra_kind == "fp8" else
             ((extra_kind, prefill_kernels, PREFILL_SOURCES),) if extra_kind else
             (("prefill", prefill_kernels, PREFILL_SOURCES),
              ("decode", ["decode_partial_kernel", "decode_merge_kernel"], DECODE_SOURCES)))
    path = os.path.join(out_dir, "traffic.json")
    if os.path.exists(path):  # entries of the other runs are kept
        with open(path) as f:
            old = json.load(f)
        old[(extra_kind + "_calibration") if extra_kind else "calibration"] = res["calibration"]
        res = old
    for kind, keys, srcs in kinds:
        need = [k for k in keys if not k.endswith("?")]
        opt = [k[:-1] for k in keys if k.endswith("?")]
        fb = [pick(fetch, k) for k in need]
        wb = [pick(write, k) for k in need]
        if any(x is None for x in fb + wb):
            continue
        ran = [k for k in opt if pick(fetch, k) is not None and pick(write, k) is not None]
        rd = (sum(fb) + sum(pick(fetch, k) for k in ran)) * f_scale
        wr = (sum(wb) + sum(pick(write, k) for k in ran)) * w_scale
        res[kind] = {"kernels": need + ran, "fetch_bytes_per_launch": rd, "write_bytes_per_launch": wr,
                     "hbm_bytes_per_launch": rd + wr, "source_digest": kernel_sources_digest(srcs)}
    os.makedirs(out_dir, exist_ok=True)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    return res


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline_prefill(cfg, n_kv=6):
    """The fp64 oracle on a bounded sample of the prefill workload: batch 0, the query heads
    of the first n_kv KV heads, all rows (row blocks of 1024, each with its full softmax)."""
    import numpy as np
    import oracle
    import workloads
    q, k, v = workloads.make_fwd_inputs(**cfg)
    nq = n_kv * (cfg["Hq"] // cfg["Hkv"])
    qs = q[:1, :nq].double().numpy()
    ks = k[:1, :n_kv].double().numpy()
    vs = v[:1, :n_kv].double().numpy()
    t0 = time.perf_counter()
    oracle.attention(qs, ks, vs, causal=cfg["causal"], rope_base=cfg["rope_base"], pos=cfg["pos"],
                     row_block=1024)
    dt = time.perf_counter() - t0
    flops = workloads.fwd_flops(1, nq, cfg["T"], cfg["S"], cfg["d_h"], cfg["causal"])
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle",
                seconds=round(dt, 3),
                sample=f"batch 0, query heads 0-{nq - 1} (KV heads 0-{n_kv - 1}), all {cfg['T']} rows x {cfg['S']} keys, "
                       f"fp64 numpy, 1024-row blocks; {flops:.3e} algorithmic FLOP")


def cpu_baseline_decode(d, cfg, n_seqs=64):
    """The fp64 oracle on the first n_seqs sequences of the decode workload."""
    import oracle
    import workloads
    sl = d["seq_lens"][:n_seqs].numpy()
    kc, vc = d["k_cache"].float().numpy(), d["v_cache"].float().numpy()   # bf16 values, exact in fp32
    t0 = time.perf_counter()
    oracle.decode_paged(d["q"][:n_seqs].double().numpy(), kc, vc,
                        d["block_table"][:n_seqs].numpy(), sl, d["block_size"], rope_base=cfg["rope_base"])
    dt = time.perf_counter() - t0
    nbytes = workloads.decode_kv_bytes(sl, cfg["Hkv"], cfg["d_h"])
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=cpu_threads(), kind="oracle", seconds=round(dt, 3),
                sample=f"first {n_seqs} of {cfg['num_seqs']} sequences ({int(sl.sum())} tokens), fp64 numpy")


def cpu_baseline_window(cfg, window, n_kv=2):
    """The fp64 oracle on a bounded sample of the window workload: batch 0, the query heads of
    the first n_kv KV heads, all rows (the oracle materialises the full masked score matrix)."""
    import oracle
    import workloads
    q, k, v = workloads.make_fwd_inputs(**cfg)
    nq = n_kv * (cfg["Hq"] // cfg["Hkv"])
    qs, ks, vs = q[:1, :nq].double().numpy(), k[:1, :n_kv].double().numpy(), v[:1, :n_kv].double().numpy()
    t0 = time.perf_counter()
    oracle.attention(qs, ks, vs, causal=True, rope_base=cfg["rope_base"], pos=cfg["pos"], row_block=1024,
                     window=window)
    dt = time.perf_counter() - t0
    flops = workloads.window_flops(1, nq, cfg["T"], cfg["S"], cfg["d_h"], window, cfg["pos"])
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle", seconds=round(dt, 3),
                sample=f"batch 0, query heads 0-{nq - 1} (KV heads 0-{n_kv - 1}), all {cfg['T']} rows, fp64 numpy, "
                       f"1024-row blocks; {flops:.3e} algorithmic FLOP")


def fwd_workspace(q, k, causal, window, cfg):
    """The forward's workspace, allocated once before timing (False when the library asks for
    none: the keys are then rotated inside the prefill)."""
    import torch
    from exact_transformer_attention_amd import attn_fwd_workspace_bytes
    B, Hq, T, d = q.shape
    need = attn_fwd_workspace_bytes(B, Hq, k.shape[1], T, k.shape[2], d, causal, window, cfg["rope_base"],
                                    cfg["pos"])
    return torch.empty(need, dtype=torch.uint8, device=q.device) if need else False


def prefill_kernels(ws, hp):
    """The kernels of one timed prefill call (the launch duration covers all of them)."""
    return (f"rope_k_kernel + " if ws is not False else "") + f"fwd_bf16_kernel<128,{hp}>"


def window_bench(a):
    """Causal sliding-window prefill on the 8192-token GQA workload (one JSON line)."""
    import torch
    import workloads
    from exact_transformer_attention_amd import attn_fwd_window
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["gqa8k"]
    w = a.window
    q, k, v = (t.to(dev) for t in workloads.make_fwd_inputs(**cfg))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = fwd_workspace(q, k, True, w, cfg)

    def run():
        attn_fwd_window(q, k, v, w, rope_base=cfg["rope_base"], pos=cfg["pos"], out=out, lse=lse, workspace=ws)

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    assert bool(torch.isfinite(out).all())
    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    flops = workloads.window_flops(cfg["B"], cfg["Hq"], cfg["T"], cfg["S"], cfg["d_h"], w, cfg["pos"])
    tf = flops / (avg * 1e-3) / 1e12
    res = {
        "metric": "sliding-window attention fwd TFLOP/s + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded iid normal, bf16-rounded)",
        "config": {"workload": f"causal sliding-window GQA prefill B=2 Hq=32 Hkv=8 T=S=8192 d_h=128 RoPE 1e4, "
                               f"window {w}", "window": w},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("window", kernel_sources_digest(PREFILL_SOURCES)),
                     "kernel": prefill_kernels(ws, 4), "flop_per_launch": flops, "avg_launch_ms": round(avg, 4)},
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host (window sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_window(cfg, w)
    print(json.dumps(res), flush=True)


def cpu_baseline_config(name, cfg):
    """The fp64 oracle on a bounded sample of a contiguous prefill workload: the whole of the
    2048-token MHA shape; for the 32768-token shape the last 2048 rows of the query heads of
    KV head 0 of batch 0 (each row against every key it sees)."""
    import numpy as np
    import oracle
    import workloads
    q, k, v = workloads.make_fwd_inputs(**cfg)
    if name == "mha2k":
        qs, ks, vs, t0, heads = q, k, v, 0, cfg["B"] * cfg["Hq"]
        sample = f"the whole workload ({cfg['B']} x {cfg['Hq']} heads, all {cfg['T']} rows)"
    else:
        G = cfg["Hq"] // cfg["Hkv"]
        t0 = cfg["T"] - 2048
        qs, ks, vs = q[:1, :G, t0:], k[:1, :1], v[:1, :1]
        heads = G
        sample = f"batch 0, query heads 0-{G - 1} (KV head 0), rows {t0}-{cfg['T'] - 1} against every visible key"
    qs, ks, vs = (x.double().numpy() for x in (qs, ks, vs))
    t_start = time.perf_counter()
    oracle.attention(qs, ks, vs, causal=True, rope_base=cfg["rope_base"], pos=t0, row_block=1024)
    dt = time.perf_counter() - t_start
    rows = np.arange(t0, cfg["T"])
    flops = float(heads) * float(np.sum(rows + 1)) * cfg["d_h"] * 4.0  # exact visible pairs, 4 d_h each
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle", seconds=round(dt, 3),
                sample=f"{sample}, fp64 numpy, 1024-row blocks; {flops:.3e} FLOP (exact visible pairs)")


def sweep_bench(a):
    """bf16 prefill throughput across shapes (one JSON line with a row per shape): 32 query
    heads, 32/16/8/4 KV heads, T = S from 1024 to 16384 tokens (batch 16384 / T), causal with
    RoPE (base 1e4), non-causal at 4096, d_h = 128 and 64; seeded N(0, 1) inputs rounded to bf16,
    the keys rotated ahead whenever attn_fwd_workspace_bytes asks for it.  Each shape is timed
    with HIP events over --steps calls after at least 0.25 s of warm-up calls (the clocks settle
    within that)."""
    import torch
    from exact_transformer_attention_amd import attn_fwd
    rows = []
    for d in (128, 64):
        for hkv in (32, 16, 8, 4):
            for T in (1024, 2048, 4096, 8192, 16384):
                if d == 64 and T not in (2048, 8192):
                    continue
                B = max(1, 16384 // T)
                for causal in ((True, False) if T == 4096 else (True,)):
                    g = torch.Generator(device="cpu").manual_seed(T + hkv + d)
                    q = torch.randn(B, 32, T, d, generator=g).to(torch.bfloat16).cuda()
                    k = torch.randn(B, hkv, T, d, generator=g).to(torch.bfloat16).cuda()
                    v = torch.randn(B, hkv, T, d, generator=g).to(torch.bfloat16).cuda()
                    out = torch.empty_like(q)
                    lse = torch.empty(B, 32, T, device="cuda")

                    def run():
                        attn_fwd(q, k, v, causal=causal, rope_base=10000.0, out=out, lse=lse)

                    t0 = time.perf_counter()
                    n = 0
                    while n < a.warmup or time.perf_counter() - t0 < 0.25:
                        run()
                        torch.cuda.synchronize()
                        n += 1
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(a.steps):
                        run()
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1) / a.steps
                    flop = 4.0 * B * 32 * T * T * d / (2 if causal else 1)
                    tf = flop / (ms * 1e-3) / 1e12
                    rows.append({"B": B, "Hq": 32, "Hkv": hkv, "T": T, "d_h": d, "causal": causal,
                                 "ms": round(ms, 4), "tflops": round(tf, 1),
                                 "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
                    print(f"[bench] sweep {rows[-1]}", file=sys.stderr, flush=True)
                    del q, k, v, out, lse
    print(json.dumps({"metric": "bf16 prefill TFLOP/s across shapes", "unit": "TFLOP/s", "n_gpus": 1,
                      "steps": a.steps, "warmup": "at least 0.25 s", "dtype": "bf16",
                      "data": "synthetic (seeded iid normal, bf16-rounded)", "sweep": rows}))


def config_bench(a, name):
    """Causal prefill of one of the other contiguous workloads (the 2048-token MHA shape or the
    32768-token GQA shape), timed like the headline prefill (one JSON line)."""
    import torch
    import workloads
    from exact_transformer_attention_amd import attn_fwd
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS[name]
    q, k, v = (t.to(dev) for t in workloads.make_fwd_inputs(**cfg))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = fwd_workspace(q, k, True, 0, cfg)

    def run():
        attn_fwd(q, k, v, causal=True, rope_base=cfg["rope_base"], pos=cfg["pos"], out=out, lse=lse, workspace=ws)

    steps, warmup = a.steps, a.warmup
    if name == "gqa32k":  # each launch is ~8 ms: fewer launches keep the run short
        steps, warmup = max(3, a.steps // 4), max(2, a.warmup // 8)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    assert bool(torch.isfinite(out).all())
    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    flops = workloads.fwd_flops(**cfg)
    tf = flops / (avg * 1e-3) / 1e12
    G = cfg["Hq"] // cfg["Hkv"]
    hp = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    res = {
        "metric": "attention fwd TFLOP/s + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded iid normal, bf16-rounded)",
        "config": {"workload": f"causal prefill {name}: B={cfg['B']} Hq={cfg['Hq']} Hkv={cfg['Hkv']} "
                               f"T=S={cfg['T']} d_h={cfg['d_h']} RoPE {cfg['rope_base']:g} sigma {cfg['sigma']:g}",
                   **{k_: cfg[k_] for k_ in ("B", "Hq", "Hkv", "T", "S", "d_h", "causal", "rope_base")}},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(name, kernel_sources_digest(PREFILL_SOURCES)),
                     "kernel": prefill_kernels(ws, hp), "flop_per_launch": flops, "avg_launch_ms": round(avg, 4)},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_config(name, cfg)
    print(json.dumps(res), flush=True)


def prefix_bench(a):
    """Paged prefill of 1024 new tokens per sequence, 8 sequences over one shared 6144-token
    prefix (one JSON line)."""
    import torch
    import workloads
    from exact_transformer_attention_amd import attn_prefill_paged
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["prefix8"]
    d = workloads.make_prefill_paged_inputs(**cfg)
    q, kc, vc = d["q"].to(dev), d["k_cache"].to(dev), d["v_cache"].to(dev)
    bt, sl = d["block_table"].to(dev), d["seq_lens"].to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def run():
        attn_prefill_paged(q, kc, vc, bt, sl, block_size=16, rope_base=cfg["rope_base"], out=out, lse=lse)

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    assert bool(torch.isfinite(out).all())
    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    lens = d["seq_lens"].tolist()
    flops = workloads.prefill_paged_flops(lens, cfg["Hq"], cfg["T"], cfg["d_h"])
    tf = flops / (avg * 1e-3) / 1e12
    res = {
        "metric": "paged prefill (shared prefix) TFLOP/s + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded iid normal, bf16-rounded)",
        "config": {"workload": "paged prefill: 8 sequences x 1024 new tokens over one shared 6144-token prefix, "
                               "Hq=32 Hkv=8 d_h=128 block 16, RoPE 1e4 on q", "cache_blocks": d["num_blocks"]},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefix", kernel_sources_digest(PREFILL_SOURCES)),
                     "kernel": "fwd_bf16_kernel<128,4,paged>", "flop_per_launch": flops,
                     "avg_launch_ms": round(avg, 4)},
    }
    if not a.no_cpu_baseline:
        import oracle
        print("[bench] timing the oracle on the host (prefix sample)", file=sys.stderr, flush=True)
        heads = list(range(8))
        qs = d["q"][:1].double().numpy()
        t0 = time.perf_counter()
        oracle.prefill_paged(qs, d["k_cache"].double().numpy(), d["v_cache"].double().numpy(),
                             d["block_table"][:1].numpy(), d["seq_lens"][:1].numpy(), 16, rope_base=cfg["rope_base"],
                             heads=heads)
        dt = time.perf_counter() - t0
        sf = workloads.prefill_paged_flops(lens[:1], len(heads), cfg["T"], cfg["d_h"])
        res["cpu_baseline"] = dict(value=sf / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle",
                                   seconds=round(dt, 3),
                                   sample=f"sequence 0, query heads 0-7, all {cfg['T']} new rows, fp64 numpy; "
                                          f"{sf:.3e} algorithmic FLOP")
    print(json.dumps(res), flush=True)


BWD_SOURCES = ["exact_transformer_attention_amd/csrc/bwd_bf16.hip",
               "exact_transformer_attention_amd/csrc/attn_common.h",
               "exact_transformer_attention_amd/csrc/fwd_params.h"]


def bwd_bench(a):
    """Backward (attn_bwd: preprocess + dK/dV + dQ kernels) of the causal 8192-token GQA
    workload, given the forward's out and lse (one JSON line)."""
    import torch
    import workloads
    from exact_transformer_attention_amd import attn_bwd, attn_bwd_workspace_bytes, attn_fwd
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["gqa8k"]
    q, k, v, do = (t.to(dev) for t in workloads.make_bwd_inputs(**cfg))
    out, lse = attn_fwd(q, k, v, causal=True, rope_base=cfg["rope_base"], pos=cfg["pos"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(attn_bwd_workspace_bytes(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["S"], cfg["d_h"],
                                              cfg["rope_base"]), dtype=torch.uint8, device=dev)

    def run():
        attn_bwd(q, k, v, out, lse, do, causal=True, rope_base=cfg["rope_base"], pos=cfg["pos"], dq=dq, dk=dk,
                 dv=dv, workspace=ws)

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    assert all(bool(torch.isfinite(t).all()) for t in (dq, dk, dv))
    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    flops = workloads.bwd_flops(**cfg)
    tf = flops / (avg * 1e-3) / 1e12
    res = {
        "metric": "attention bwd TFLOP/s + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded iid normal, bf16-rounded)",
        "config": {"workload": "backward of causal GQA prefill B=2 Hq=32 Hkv=8 T=S=8192 d_h=128 RoPE 1e4 "
                               "(dq, dk, dv from out, lse and dO)"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("bwd", kernel_sources_digest(BWD_SOURCES)),
                     "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel<4>", "flop_per_launch": flops,
                     "avg_launch_ms": round(avg, 4)},
    }
    if not a.no_cpu_baseline:
        import oracle
        print("[bench] timing the oracle on the host (backward sample)", file=sys.stderr, flush=True)
        qh, kh, vh, doh = workloads.make_bwd_inputs(**cfg)
        nq = cfg["Hq"] // cfg["Hkv"]
        t0 = time.perf_counter()
        oracle.attention_backward(qh[:1, :nq].double().numpy(), kh[:1, :1].double().numpy(),
                                  vh[:1, :1].double().numpy(), doh[:1, :nq].double().numpy(), True,
                                  cfg["rope_base"], cfg["pos"])
        dt = time.perf_counter() - t0
        sf = workloads.bwd_flops(1, nq, cfg["T"], cfg["S"], cfg["d_h"], True)
        res["cpu_baseline"] = dict(value=sf / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle",
                                   seconds=round(dt, 3),
                                   sample=f"batch 0, KV head 0 and its {nq} query heads, all {cfg['T']} rows, "
                                          f"fp64 numpy; {sf:.3e} algorithmic FLOP")
    print(json.dumps(res), flush=True)


FP8_SOURCES = ["exact_transformer_attention_amd/csrc/fwd_fp8.hip",
               "exact_transformer_attention_amd/csrc/attn_common.h",
               "exact_transformer_attention_amd/csrc/fwd_params.h"]


def fp8_bench(a):
    """fp8 (E4M3) prefill on the causal 8192-token GQA shape (one JSON line)."""
    import torch
    import workloads
    from exact_transformer_attention_amd import attn_fwd_fp8
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["gqa8k"]
    (q8, k8, vt8), sc = workloads.make_fp8_inputs(**cfg)
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)

    def run():
        attn_fwd_fp8(q8, k8, vt8, *sc, causal=True, pos=0, out=out, lse=lse)

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    assert bool(torch.isfinite(out).all())
    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    flops = workloads.fwd_flops(**cfg)
    tf = flops / (avg * 1e-3) / 1e12
    res = {
        "metric": "fp8 attention fwd TFLOP/s + % fp8 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8", "data": "synthetic (seeded iid normal, per-tensor amax scaling to E4M3)",
        "config": {"workload": "causal GQA prefill B=2 Hq=32 Hkv=8 T=S=8192 d_h=128, E4M3 q/k/v (V transposed), "
                               "inputs taken as already rotated", "scales": [round(x, 8) for x in sc]},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic("fp8", kernel_sources_digest(FP8_SOURCES)),
                     "kernel": "fwd_fp8_kernel<4>", "flop_per_launch": flops, "avg_launch_ms": round(avg, 4)},
    }
    if not a.no_cpu_baseline:
        import oracle
        print("[bench] timing the oracle on the host (fp8 sample)", file=sys.stderr, flush=True)
        n_kv = 4
        nq = n_kv * (cfg["Hq"] // cfg["Hkv"])
        qh, kh, vh = workloads.make_fp8_inputs(**cfg)[0]
        t0 = time.perf_counter()
        oracle.attention_fp8(qh[:1, :nq].numpy(), kh[:1, :n_kv].numpy(), vh[:1, :n_kv].numpy(), *sc, causal=True)
        dt = time.perf_counter() - t0
        sf = workloads.fwd_flops(1, nq, cfg["T"], cfg["S"], cfg["d_h"], True)
        res["cpu_baseline"] = dict(value=sf / dt / 1e12, unit="TFLOP/s", cores=cpu_threads(), kind="oracle",
                                   seconds=round(dt, 3),
                                   sample=f"batch 0, query heads 0-{nq - 1} (KV heads 0-{n_kv - 1}), all {cfg['T']} rows, "
                                          f"fp64 numpy on the decoded fp8 values; {sf:.3e} algorithmic FLOP")
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for PMC byte-counter calibration)")
    ap.add_argument("--only", choices=["prefill", "decode", "window", "prefix", "bwd", "fp8", "mha2k", "gqa32k",
                                       "sweep"],
                    default=None,
                    help="time only one part (profiling runs); 'window' times the causal sliding-window "
                         "prefill (attn_fwd_window) on the same 8192-token GQA workload instead; 'prefix' "
                         "the paged prefill (attn_prefill_paged) of 8 sequences over a shared 6144-token prefix; "
                         "'bwd' the backward (attn_bwd) of the 8192-token GQA prefill; 'fp8' the fp8 prefill "
                         "(attn_fwd_fp8) on the same shape; 'sweep' the bf16 prefill over a grid of shapes")
    ap.add_argument("--window", type=int, default=4096, help="window of --only window (keys)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs into profiles/traffic.json "
                         "(with --only window or prefix: CSVs of that run, added as its own entry)")
    a = ap.parse_args()
    if a.traffic_from:
        print(json.dumps(summarize_pmc(a.traffic_from[0], a.traffic_from[1], os.path.join(ROOT, "profiles"),
                                       extra_kind=a.only if a.only in ("window", "prefix", "bwd", "fp8", "mha2k", "gqa32k")
                                       else None),
                         indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    if a.only == "window":
        window_bench(a)
        return
    if a.only == "prefix":
        prefix_bench(a)
        return
    if a.only == "bwd":
        bwd_bench(a)
        return
    if a.only == "fp8":
        fp8_bench(a)
        return
    if a.only in ("mha2k", "gqa32k"):
        config_bench(a, a.only)
        return
    if a.only == "sweep":
        sweep_bench(a)
        return

    import torch
    import workloads
    from exact_transformer_attention_amd import attn_decode_paged, attn_fwd

    dev = torch.device("cuda:0")
    pcfg = workloads.CONFIGS["gqa8k"]
    dcfg = workloads.CONFIGS["decode64"]
    do_p = a.only in (None, "prefill")
    do_d = a.only in (None, "decode")
    print(f"[bench] generating inputs", file=sys.stderr, flush=True)
    if do_p:
        q, k, v = workloads.make_fwd_inputs(**pcfg)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        out = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        pws = fwd_workspace(qd, kd, pcfg["causal"], 0, pcfg)
    if do_d:
        d = workloads.make_decode_inputs(**dcfg)
        dq = d["q"].to(dev)
        dk, dv = d["k_cache"].to(dev), d["v_cache"].to(dev)
        dbt, dsl = d["block_table"].to(dev), d["seq_lens"].to(dev)
        dout = torch.empty_like(dq)
        dlse = torch.empty(dq.shape[:2], dtype=torch.float32, device=dev)
        from exact_transformer_attention_amd import attn_decode_workspace_bytes
        ws = torch.empty(attn_decode_workspace_bytes(dcfg["num_seqs"], dcfg["Hq"], dcfg["Hkv"], dcfg["d_h"],
                                                     d["max_blocks_per_seq"], 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        attn_fwd(qd, kd, vd, causal=pcfg["causal"], rope_base=pcfg["rope_base"], pos=pcfg["pos"], out=out,
                 lse=lse, workspace=pws)

    def decode():
        attn_decode_paged(dq, dk, dv, dbt, dsl, block_size=16, rope_base=dcfg["rope_base"], out=dout,
                          lse=dlse, workspace=ws)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        if do_p:
            prefill()
        if do_d:
            decode()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(a.steps):
        ev[i][0].record(stream)
        if do_p:
            prefill()
        ev[i][1].record(stream)
        if do_d:
            decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    p_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(a.steps)]
    d_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(a.steps)]
    p_avg = sum(p_ms) / len(p_ms)
    d_avg = sum(d_ms) / len(d_ms)
    print(f"[bench] prefill ms avg {p_avg:.4f} min {min(p_ms):.4f}; decode ms avg {d_avg:.4f} "
          f"min {min(d_ms):.4f}; wall {wall:.3f}s", file=sys.stderr, flush=True)
    if do_p:
        assert bool(torch.isfinite(out).all())
    if do_d:
        assert bool(torch.isfinite(dout).all())

    if a.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()

    flops = workloads.fwd_flops(**pcfg)
    tflops = flops / (p_avg * 1e-3) / 1e12 if do_p else 0.0
    seq_lens = d["seq_lens"].tolist() if do_d else workloads.make_decode_inputs(
        **workloads.scaled(dcfg, Hq=1, Hkv=1, d_h=8))["seq_lens"].tolist()
    kv_bytes = workloads.decode_kv_bytes(seq_lens, dcfg["Hkv"], dcfg["d_h"])
    dec_gbs = kv_bytes / (d_avg * 1e-3) / 1e9 if do_d else 0.0

    res = {
        "metric": "attention fwd TFLOP/s + % bf16 MFMA peak; paged-decode KV GB/s + % HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(p_avg + d_avg, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid normal, bf16-rounded)",
        "config": {
            "workload": "causal GQA prefill B=2 Hq=32 Hkv=8 T=S=8192 d_h=128 RoPE 1e4 "
                        "+ paged decode 64 seqs L~U[512,8192] Hq=32 Hkv=8 d_h=128 block 16",
            "prefill": {k_: pcfg[k_] for k_ in ("B", "Hq", "Hkv", "T", "S", "d_h", "causal", "rope_base")},
            "decode": {"num_seqs": dcfg["num_seqs"], "Hq": dcfg["Hq"], "Hkv": dcfg["Hkv"], "d_h": dcfg["d_h"],
                       "block_size": 16, "total_tokens": int(sum(seq_lens)), "kv_bytes": kv_bytes},
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill", kernel_sources_digest(PREFILL_SOURCES)),
            "kernel": prefill_kernels(pws, 4), "flop_per_launch": flops, "avg_launch_ms": round(p_avg, 4),
        },
        "decode": {
            "value": round(dec_gbs, 1), "unit": "GB/s", "avg_step_ms": round(d_avg, 4),
            "roofline": {
                "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("decode", kernel_sources_digest(DECODE_SOURCES)),
                "kernels": "decode_partial_kernel + decode_merge_kernel", "kv_bytes_per_launch": kv_bytes,
            },
        },
    }
    if not a.no_cpu_baseline and do_p and do_d:
        print("[bench] timing the oracle on the host (prefill sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_prefill(pcfg)
        print("[bench] timing the oracle on the host (decode sample)", file=sys.stderr, flush=True)
        res["decode"]["cpu_baseline"] = cpu_baseline_decode(d, dcfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
