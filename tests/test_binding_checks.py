"""The Python binding rejects malformed arguments with ValueError before calling the C ABI
(no GPU needed: every case fails validation first; the last check of each binding is that
all tensors sit on one GPU, which host tensors fail)."""

import pytest
import torch

bf16 = torch.bfloat16


@pytest.fixture(scope="module")
def L():
    import exact_transformer_attention_amd._lib as lib
    return lib


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def fwd_args():
    q = torch.zeros(1, 4, 8, 128, dtype=bf16)
    k = torch.zeros(1, 2, 8, 128, dtype=bf16)
    return q, k, k.clone()


def test_fwd_rejections(L):
    q, k, v = fwd_args()
    raises(lambda: L.attn_fwd(q[0], k, v), "q must be 4-D")
    raises(lambda: L.attn_fwd(q, k.float(), v), "share a dtype")
    raises(lambda: L.attn_fwd(q, k[:, :, :4].contiguous(), v), "shapes do not match")
    raises(lambda: L.attn_fwd(q.transpose(2, 3), k, v), "must be contiguous|shapes do not match")
    raises(lambda: L.attn_fwd(q, k, v, out=torch.zeros(1, 4, 8, 64, dtype=bf16)), "out must have shape")
    raises(lambda: L.attn_fwd(q, k, v, out=torch.zeros_like(q, dtype=torch.float32)), "out must be")
    raises(lambda: L.attn_fwd(q, k, v, lse=torch.zeros(1, 4, 8, dtype=bf16)), "lse must be")
    raises(lambda: L.attn_fwd(q, k, v, lse=torch.zeros(1, 4, 9)), "lse must have shape")
    raises(lambda: L.attn_fwd(q, k, v), "device")
    raises(lambda: L.attn_fwd_window(q, k, v, 4, out=torch.zeros(2, 4, 8, 128, dtype=bf16)), "out must have shape")


def test_fp8_rejections(L):
    q8 = torch.zeros(1, 4, 8, 128, dtype=torch.uint8)
    k8 = torch.zeros(1, 2, 8, 128, dtype=torch.uint8)
    vt8 = torch.zeros(1, 2, 128, 8, dtype=torch.uint8)
    raises(lambda: L.attn_fwd_fp8(q8.to(bf16), k8, vt8, 1.0, 1.0, 1.0), "one-byte codes")
    raises(lambda: L.attn_fwd_fp8(q8, k8, k8, 1.0, 1.0, 1.0), "shapes do not match")
    raises(lambda: L.attn_fwd_fp8(q8, k8, vt8, 1.0, 1.0, 1.0, out=torch.zeros(1, 4, 8, 128)), "out must be")
    raises(lambda: L.attn_fwd_fp8(q8, k8, vt8, 1.0, 1.0, 1.0, lse=torch.zeros(1, 4)), "lse must have shape")
    raises(lambda: L.attn_fwd_fp8(q8, k8, vt8, 1.0, 1.0, 1.0), "device")


def paged(N=2, Hq=4, Hkv=2, T=None, blocks=6, mbps=3):
    q = torch.zeros((N, Hq, 128) if T is None else (N, Hq, T, 128), dtype=bf16)
    kc = torch.zeros(blocks, Hkv, 16, 128, dtype=bf16)
    bt = torch.zeros(N, mbps, dtype=torch.int32)
    sl = torch.full((N,), 20, dtype=torch.int32)
    return q, kc, kc.clone(), bt, sl


def test_decode_rejections(L):
    q, kc, vc, bt, sl = paged()
    raises(lambda: L.attn_decode_paged(q[None], kc, vc, bt, sl), "q must be 3-D")
    raises(lambda: L.attn_decode_paged(q, kc.float(), vc, bt, sl), "k_cache must be")
    raises(lambda: L.attn_decode_paged(q, kc, vc[:, :, :8].contiguous(), bt, sl), "caches must be")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt.long(), sl), "block_table must be")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl[:1]), "seq_lens must have shape")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt[:1].contiguous(), sl), "one row per sequence|seq_lens must have shape")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl, out=torch.zeros(2, 4, 128)), "out must be")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl, lse=torch.zeros(2, 3)), "lse must have shape")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl, workspace=torch.zeros(8, dtype=torch.uint8)),
           "bytes, .* needed")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl, workspace=torch.zeros(4, 1 << 20, dtype=torch.uint8)),
           "workspace must be 1-D")
    raises(lambda: L.attn_decode_paged(q, kc, vc, bt, sl), "device")


def test_decode_static_rejections(L):
    q, kc, vc, bt, sl = paged()
    raises(lambda: L.attn_decode_paged_static(q[None], kc, vc, bt, sl), "q must be 3-D")
    raises(lambda: L.attn_decode_paged_static(q, kc, vc.float(), bt, sl), "v_cache must be")
    raises(lambda: L.attn_decode_paged_static(q, kc, vc, bt, sl.long()), "seq_lens must be")
    raises(lambda: L.attn_decode_paged_static(q, kc, vc, bt, sl, out=torch.zeros(2, 4, 64, dtype=bf16)),
           "out must have shape")
    raises(lambda: L.attn_decode_paged_static(q, kc, vc, bt, sl, lse=torch.zeros(2, 4, dtype=bf16)), "lse must be")
    raises(lambda: L.attn_decode_paged_static(q, kc, vc, bt, sl), "device")


def test_prefill_paged_rejections(L):
    q, kc, vc, bt, sl = paged(T=5)
    raises(lambda: L.attn_prefill_paged(q[0], kc, vc, bt, sl), "q must be 4-D")
    raises(lambda: L.attn_prefill_paged(q, kc, vc.float(), bt, sl), "v_cache must be")
    raises(lambda: L.attn_prefill_paged(q, kc, vc, bt, sl.long()), "seq_lens must be")
    raises(lambda: L.attn_prefill_paged(q, kc, vc, bt, sl, out=torch.zeros(2, 4, 5, 64, dtype=bf16)),
           "out must have shape")
    raises(lambda: L.attn_prefill_paged(q, kc, vc, bt, sl, lse=torch.zeros(2, 4, 5, dtype=bf16)), "lse must be")
    raises(lambda: L.attn_prefill_paged(q, kc, vc, bt, sl), "device")


def test_bwd_rejections(L):
    q, k, v = fwd_args()
    out, lse, do = torch.zeros_like(q), torch.zeros(1, 4, 8), torch.zeros_like(q)
    raises(lambda: L.attn_bwd(q, k, v, None, lse, do), "out and lse are required")
    raises(lambda: L.attn_bwd(q, k, v, out, lse, do.float()), "dout must be")
    raises(lambda: L.attn_bwd(q, k, v, out, lse, do, dq=torch.zeros(1, 4, 8, 128)), "dq must be")
    raises(lambda: L.attn_bwd(q, k, v, out, lse, do, dk=torch.zeros_like(q)), "dk must have shape")
    raises(lambda: L.attn_bwd(q, k, v, out, lse, do, workspace=torch.zeros(16, dtype=torch.uint8)),
           "bytes, .* needed")
    raises(lambda: L.attn_bwd(q, k, v, out, lse, do), "device")


def test_gather_rejections(L):
    _, kc, _, bt, sl = paged()
    raises(lambda: L.attn_paged_gather(kc[0], bt, sl), "cache must be 4-D")
    raises(lambda: L.attn_paged_gather(kc, bt.long(), sl), "block_table must be")
    raises(lambda: L.attn_paged_gather(kc, bt, sl[:1]), "seq_lens must have shape")
    raises(lambda: L.attn_paged_gather(kc, bt, sl, block_size=8), "block_size")
    raises(lambda: L.attn_paged_gather(kc, bt, sl, dst=torch.zeros(2, 2, 47, 128, dtype=bf16)), "dst must have shape")
    raises(lambda: L.attn_paged_gather(kc, bt, sl, dst=torch.zeros(2, 2, 48, 128)), "dst must be")
    raises(lambda: L.attn_paged_gather(kc, bt, sl), "device")
