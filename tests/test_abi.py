"""The C ABI without a GPU: the library loads, exports every entry point the header
declares, and rejects invalid requests on the host before touching HIP."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]*?\b(attn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import exact_transformer_attention_amd as e
    return e.LIB


def test_header_declares_entry_points():
    names = header_functions()
    assert names == sorted(["attn_fwd", "attn_fwd_window", "attn_fwd_workspace_bytes", "attn_fwd_fp8", "attn_prefill_paged", "attn_decode_paged",
                            "attn_decode_paged_static", "attn_decode_workspace_bytes", "attn_bwd",
                            "attn_bwd_workspace_bytes", "attn_paged_gather", "attn_status_str"])


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    # and the exported dynamic symbol table holds exactly those attn_ entry points
    import subprocess
    import exact_transformer_attention_amd as e
    out = subprocess.run(["nm", "-D", "--defined-only", e.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (attn_\w+)", out)))
    assert exported == header_functions()


def test_status_strings(lib):
    import exact_transformer_attention_amd as e
    assert e.attn_status_str(e.ATTN_OK) == "ok"
    for s in range(1, 6):
        assert e.attn_status_str(s) not in ("ok", "unknown status")


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, T=8, S=8, d=128, causal=1,
             base=10000.0, pos=0, ws=None, wsb=0, dtype=1)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"], a["S"],
                        a["d"], a["causal"], a["base"], a["pos"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(T=0), 1), (dict(S=-1), 1), (dict(d=0), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(causal=2), 1), (dict(base=-1.0), 1), (dict(base=float("nan")), 1),
    (dict(base=float("inf")), 1), (dict(dtype=7), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(pos=1 << 41), 2),
    # one KV head's bf16 keys past a 32-bit byte range (S * d_h * 2 >= 2^32)
    (dict(S=1 << 24), 2), (dict(S=1 << 25, d=64), 2),
    # a workspace must be 16-byte aligned (the rotated keys are moved in 16-byte chunks)
    (dict(ws=ctypes.c_void_p(0x1008), wsb=1 << 20), 1),
])
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


def fwd_window(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, T=8, S=8, d=128, window=16,
             base=10000.0, pos=0, ws=None, wsb=0, dtype=1)
    a.update(kw)
    return lib.attn_fwd_window(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"],
                               a["S"], a["d"], a["window"], a["base"], a["pos"], a["ws"], a["wsb"], a["dtype"],
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(window=0), 1), (dict(window=-3), 1), (dict(q=None), 1), (dict(Hq=6, Hkv=4), 1), (dict(dtype=9), 1),
    (dict(d=96), 2), (dict(pos=1 << 41), 2), (dict(ws=ctypes.c_void_p(0x1004), wsb=1 << 20), 1),
])
def test_fwd_window_validation(lib, kw, status):
    assert fwd_window(lib, **kw) == status


def kbytes(B, Hkv, S, d):
    return B * Hkv * S * d * 2


def readers_per_key_block(Hq, Hkv, T, S, causal, window, pos):
    """Brute force: over every workgroup of the bf16 prefill (HP heads x 256/HP rows), the key
    blocks from the first its first row's window reaches to the last its last row sees;
    summed, per KV head's key block."""
    G = Hq // Hkv
    HP = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    RH = 256 // HP
    nkb = -(-S // 64)
    reads = 0
    for qb in range(-(-T // RH)):
        last = min(T - 1, qb * RH + RH - 1)
        nk = S if not causal else max(0, min(S, pos + last + 1))
        first = 0
        if window > 0:
            lo = pos + qb * RH - window + 1
            first = (0 if lo <= 0 else min(lo, nk)) // 64
        reads += len(range(first, -(-nk // 64)))
    return reads * (G // HP) / nkb


def test_fwd_workspace_bytes_follows_the_reader_count(lib):
    """Seeded shapes: the library asks for a workspace exactly when each key block is read by
    at least 16 workgroups (brute-force count above)."""
    import numpy as np
    rng = np.random.default_rng(20261204)
    asked = 0
    for _ in range(300):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
        T = int(rng.integers(1, 6000))
        S = int(rng.integers(1, 6000))
        causal = int(rng.integers(0, 2))
        window = int(rng.choice([0, 0, int(rng.integers(1, 4000))]))
        if window:
            causal = 1
        pos = int(rng.integers(-100, 3000)) if causal else 0
        d = int(rng.choice([64, 128]))
        got = lib.attn_fwd_workspace_bytes(1, Hq, Hkv, T, S, d, causal, window, 10000.0, pos, 1)
        want = 1 * Hkv * S * d * 2 if readers_per_key_block(Hq, Hkv, T, S, causal, window, pos) >= 16 else 0
        assert got == want, (Hq, Hkv, T, S, causal, window, pos, d)
        asked += got > 0
    assert 0 < asked < 300


@pytest.mark.parametrize("args,expect", [
    # 2 x 32 query heads over 8 KV heads, 8192 causal tokens, RoPE: each K block is read by
    # about 64 workgroups of 4 heads x 64 rows -> rotate once ahead
    (dict(B=2, Hq=32, Hkv=8, T=8192, S=8192, causal=1), kbytes(2, 8, 8192, 128)),
    (dict(B=1, Hq=32, Hkv=8, T=32768, S=32768, causal=1), kbytes(1, 8, 32768, 128)),
    # the same with a 4096-key window: still ~64 readers per block
    (dict(B=2, Hq=32, Hkv=8, T=8192, S=8192, causal=1, window=4096), kbytes(2, 8, 8192, 128)),
    # no grouping, 2048 tokens: workgroups of 256 rows of one head, ~4.5 readers per block
    (dict(B=4, Hq=32, Hkv=32, T=2048, S=2048, causal=1), 0),
    # 1024 grouped tokens: 16 query blocks of which ~8.5 read each K block
    (dict(B=1, Hq=32, Hkv=8, T=1024, S=1024, causal=1), 0),
    # non-causal: every query block reads every K block (16 of them at 1024 rows / 64)
    (dict(B=1, Hq=8, Hkv=2, T=1024, S=512, causal=0), kbytes(1, 2, 512, 128)),
    (dict(B=1, Hq=8, Hkv=2, T=960, S=512, causal=0), 0),
    # d_h 64 is sized the same way
    (dict(B=1, Hq=8, Hkv=2, T=1024, S=512, causal=0, d=64), kbytes(1, 2, 512, 64)),
    # no RoPE, fp32, or invalid sizes: nothing to rotate ahead
    (dict(B=2, Hq=32, Hkv=8, T=8192, S=8192, causal=1, base=0.0), 0),
    (dict(B=2, Hq=32, Hkv=8, T=8192, S=8192, causal=1, dtype=0), 0),
    (dict(B=2, Hq=30, Hkv=8, T=8192, S=8192, causal=1), 0),
    (dict(B=2, Hq=32, Hkv=8, T=8192, S=8192, causal=1, d=96), 0),
    (dict(B=0, Hq=32, Hkv=8, T=8192, S=8192, causal=1), 0),
])
def test_fwd_workspace_bytes(lib, args, expect):
    a = dict(causal=1, window=0, base=10000.0, pos=0, dtype=1, d=128)
    a.update(args)
    got = lib.attn_fwd_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["T"], a["S"], a["d"], a["causal"],
                                       a["window"], a["base"], a["pos"], a["dtype"])
    assert got == expect


def dec(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, bs=16, N=4, Hq=32, Hkv=8, d=128, mbps=10, nb=40,
             base=10000.0, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30, dtype=1)
    a.update(kw)
    return lib.attn_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["bs"], a["N"], a["Hq"], a["Hkv"],
                                 a["d"], a["mbps"], a["nb"], a["base"], a["out"], a["lse"], a["ws"], a["wsb"],
                                 a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(bt=None), 1), (dict(sl=None), 1), (dict(out=None), 1),
    (dict(N=0), 1), (dict(Hq=30), 1), (dict(mbps=0), 1), (dict(nb=0), 1), (dict(bs=0), 1),
    (dict(base=-2.0), 1), (dict(dtype=5), 1),
    (dict(dtype=0), 2), (dict(d=64), 2), (dict(bs=32), 2), (dict(Hq=64, Hkv=2), 2),
    (dict(N=1 << 20, mbps=1 << 12), 2),
    (dict(ws=None), 3), (dict(wsb=16), 3),
])
def test_decode_validation(lib, kw, status):
    assert dec(lib, **kw) == status


def dec_static(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, bs=16, N=4, Hq=32, Hkv=8, d=128, mbps=10, nb=40,
             base=10000.0, out=FAKE, lse=None, dtype=1)
    a.update(kw)
    return lib.attn_decode_paged_static(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["bs"], a["N"], a["Hq"],
                                        a["Hkv"], a["d"], a["mbps"], a["nb"], a["base"], a["out"], a["lse"],
                                        a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(bt=None), 1), (dict(sl=None), 1), (dict(out=None), 1),
    (dict(N=0), 1), (dict(Hq=30), 1), (dict(mbps=0), 1), (dict(nb=0), 1), (dict(bs=0), 1),
    (dict(base=-2.0), 1), (dict(dtype=5), 1),
    (dict(dtype=0), 2), (dict(d=64), 2), (dict(bs=32), 2), (dict(Hq=64, Hkv=2), 2),
    (dict(N=1 << 20, mbps=1 << 12), 2),
    # requests whose workspace passes the static scratch: rejected before any HIP call
    (dict(N=4000), 5), (dict(N=300, Hq=128), 5),
])
def test_decode_static_validation(lib, kw, status):
    assert dec_static(lib, **kw) == status


def test_decode_static_scratch_limit(lib):
    """The header's scratch size, the binding's copy of it, and the limits the header quotes:
    with Hq / Hkv = 4 up to num_seqs * Hkv = 14000 fits, with Hq / Hkv = 16 up to 1900."""
    import exact_transformer_attention_amd as e
    m = re.search(r"#define ATTN_DECODE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == e.DECODE_STATIC_SCRATCH_BYTES
    for G, fits in ((4, 14000), (16, 1900)):
        # num_seqs * Hkv = fits with Hkv = 8, long sequences (the most partial-result slots)
        assert 0 < lib.attn_decode_workspace_bytes(fits // 8, 8 * G, 8, 128, 4096, 16) <= limit
    assert lib.attn_decode_workspace_bytes(2000, 32, 8, 128, 4096, 16) > limit


def prefill_paged(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, bs=16, N=4, Hq=32, Hkv=8, d=128, T=64, mbps=10, nb=40,
             base=10000.0, out=FAKE, lse=None, dtype=1)
    a.update(kw)
    return lib.attn_prefill_paged(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["bs"], a["N"], a["Hq"], a["Hkv"],
                                  a["d"], a["T"], a["mbps"], a["nb"], a["base"], a["out"], a["lse"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(bt=None), 1), (dict(sl=None), 1), (dict(out=None), 1),
    (dict(N=0), 1), (dict(T=0), 1), (dict(Hq=30), 1), (dict(mbps=0), 1), (dict(nb=0), 1), (dict(base=-1.0), 1),
    (dict(dtype=4), 1),
    (dict(dtype=0), 2), (dict(d=64), 2), (dict(bs=32), 2), (dict(mbps=4097), 2),
])
def test_prefill_paged_validation(lib, kw, status):
    assert prefill_paged(lib, **kw) == status


def fwd_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, T=8, S=8, d=128, causal=1, sq=1.0, sk=1.0,
             sv=1.0, pos=0)
    a.update(kw)
    return lib.attn_fwd_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"], a["S"],
                            a["d"], a["causal"], a["sq"], a["sk"], a["sv"], a["pos"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(out=None), 1), (dict(T=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(causal=2), 1), (dict(sq=0.0), 1), (dict(sk=-1.0), 1), (dict(sv=float("nan")), 1), (dict(sq=float("inf")), 1),
    (dict(d=64), 2), (dict(S=10), 2), (dict(v=ctypes.c_void_p(0x1002)), 2), (dict(pos=1 << 41), 2),
])
def test_fwd_fp8_validation(lib, kw, status):
    assert fwd_fp8(lib, **kw) == status


def bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=4, Hkv=2, T=8,
             S=8, d=128, causal=1, window=0, base=10000.0, pos=0, ws=FAKE, wsb=1 << 30, dtype=1)
    a.update(kw)
    return lib.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                        a["Hq"], a["Hkv"], a["T"], a["S"], a["d"], a["causal"], a["window"], a["base"], a["pos"],
                        a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1), (dict(B=0), 1), (dict(T=0), 1), (dict(S=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(causal=3), 1), (dict(window=-1), 1), (dict(window=5, causal=0), 1), (dict(base=-1.0), 1),
    (dict(dtype=3), 1),
    (dict(dtype=0), 2), (dict(d=64), 2), (dict(pos=1 << 41), 2),
    (dict(ws=None), 3), (dict(wsb=100), 3),
])
def test_bwd_validation(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_workspace_bytes(lib):
    import exact_transformer_attention_amd as e
    # a 16-byte record per query row and the scaled (rotated) q in bf16, each array 256-byte
    # aligned; with RoPE also the rotated k in bf16
    rows = 2 * 32 * 8192
    assert e.attn_bwd_workspace_bytes(2, 32, 8, 8192, 8192, 128, 0.0) == rows * 16 + rows * 256
    assert e.attn_bwd_workspace_bytes(2, 32, 8, 8192, 8192, 128, 1e4) == rows * 16 + rows * 256 + 2 * 8 * 8192 * 256
    assert e.attn_bwd_workspace_bytes(1, 1, 1, 3, 5, 128, 0.0) == 256 + 768
    assert e.attn_bwd_workspace_bytes(1, 1, 1, 3, 5, 128, 1e4) == 256 + 768 + 1280
    assert e.attn_bwd_workspace_bytes(1, 6, 4, 3, 5, 128, 0.0) == 0
    assert e.attn_bwd_workspace_bytes(1, 1, 1, 3, 5, 128, -1.0) == 0


def test_workspace_bytes(lib):
    import exact_transformer_attention_amd as e
    # partial slots: one per wave of the grid (at most 2048, at most one per block) plus one per
    # (sequence, KV head); each slot holds Hq / Hkv partials of (d_h + 2) fp32; then
    # num_seqs + 1 int32 block offsets
    assert e.attn_decode_workspace_bytes(64, 32, 8, 128, 512, 16) == (2048 + 64 * 8) * 4 * 130 * 4 + 65 * 4
    assert e.attn_decode_workspace_bytes(1, 1, 1, 128, 1, 16) == 2 * 130 * 4 + 2 * 4
    assert e.attn_decode_workspace_bytes(2, 8, 2, 128, 3, 16) == (12 + 4) * 4 * 130 * 4 + 3 * 4
    assert e.attn_decode_workspace_bytes(0, 32, 8, 128, 512, 16) == 0
    assert e.attn_decode_workspace_bytes(4, 32, 6, 128, 512, 16) == 0


def test_gather_validation(lib):
    f = lib.attn_paged_gather
    assert f(None, FAKE, FAKE, 16, 1, 1, 128, 1, 1, 2, FAKE, None) == 1
    assert f(FAKE, FAKE, FAKE, 16, 1, 1, 128, 1, 1, 3, FAKE, None) == 1
    assert f(FAKE, FAKE, FAKE, 8, 1, 1, 128, 1, 1, 2, FAKE, None) == 2


def test_misaligned_pointers_rejected(lib):
    import exact_transformer_attention_amd as e
    odd = ctypes.c_void_p(0x1002)   # 2-byte aligned: a bf16 view one element in
    assert fwd(lib, q=odd) == e.ATTN_ERR_INVALID_ARG
    assert fwd(lib, out=odd) == e.ATTN_ERR_INVALID_ARG
    assert fwd(lib, lse=ctypes.c_void_p(0x1002)) == e.ATTN_ERR_INVALID_ARG
    assert fwd(lib, k=ctypes.c_void_p(0x1008)) == e.ATTN_ERR_INVALID_ARG


def test_binding_shares_torchs_hip_runtime():
    """The binding imported before torch must still leave one HIP runtime in the process:
    torch bundles its own copy under the system runtime's soname, and a second copy would
    not accept torch's streams or device pointers."""
    import subprocess
    import sys
    code = ("import exact_transformer_attention_amd._lib, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout
