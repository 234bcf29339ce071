"""attn_decode_paged_static, the decode entry point that allocates nothing (for callers that
cannot allocate), against attn_decode_paged, through the C ABI.

Both run the same kernels, so the outputs must be bit-identical.  Two calls in a row, the
second with a smaller request, so the second runs over what the first left in the static
scratch; a third on a stream of its own; and a request past the scratch size is refused."""

import pytest
import torch

import workloads
from gpu_common import say

pytestmark = pytest.mark.gpu


def compare(d, base, stream=None):
    from exact_transformer_attention_amd import attn_decode_paged, attn_decode_paged_static
    dev = torch.device("cuda:0")
    args = [d[k].to(dev) for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")]
    ref_out, ref_lse = attn_decode_paged(*args, block_size=d["block_size"], rope_base=base)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    if stream is None:
        attn_decode_paged_static(*args, block_size=d["block_size"], rope_base=base, out=out, lse=lse)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        attn_decode_paged_static(*args, block_size=d["block_size"], rope_base=base, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "outputs differ from attn_decode_paged"
    assert torch.equal(lse, ref_lse), "lse differs from attn_decode_paged"


def test_static_decode_equals_workspace_decode():
    cfg = workloads.CONFIGS["decode64"]
    say("no-alloc decode, call 1: 64 sequences of 512-8192 tokens, Hq 32, Hkv 8")
    compare(workloads.make_decode_inputs(**cfg), cfg["rope_base"])
    say("no-alloc decode, call 2: 6 sequences of 1-513 tokens (smaller than call 1)")
    small = workloads.scaled(cfg, num_seqs=6, seq_lens=[1, 15, 16, 17, 100, 513], seed=21)
    compare(workloads.make_decode_inputs(**small), cfg["rope_base"])
    say("no-alloc decode, call 3: 20 sequences, Hq 64, Hkv 4, on a stream of its own")
    other = workloads.scaled(cfg, num_seqs=20, Hq=64, Hkv=4, len_lo=1, len_hi=3000, seed=22)
    compare(workloads.make_decode_inputs(**other), 0.0, stream=torch.cuda.Stream())


def test_static_decode_refuses_requests_past_its_scratch():
    from exact_transformer_attention_amd import (ATTN_ERR_SCRATCH, DECODE_STATIC_SCRATCH_BYTES, AttnError,
                                                 attn_decode_paged_static, attn_decode_workspace_bytes)
    N, Hq, Hkv = 4000, 32, 8
    assert attn_decode_workspace_bytes(N, Hq, Hkv, 128, 1, 16) > DECODE_STATIC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    q = torch.zeros(N, Hq, 128, dtype=torch.bfloat16, device=dev)
    cache = torch.zeros(1, Hkv, 16, 128, dtype=torch.bfloat16, device=dev)
    table = torch.zeros(N, 1, dtype=torch.int32, device=dev)
    lens = torch.ones(N, dtype=torch.int32, device=dev)
    say("no-alloc decode: request past the scratch size")
    with pytest.raises(AttnError) as err:
        attn_decode_paged_static(q, cache, cache, table, lens)
    assert err.value.status == ATTN_ERR_SCRATCH
