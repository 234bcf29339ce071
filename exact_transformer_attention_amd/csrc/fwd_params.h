// Launch parameters shared by the prefill kernels and the host entry point.
#pragma once

#include <stdint.h>

namespace attn {

constexpr int kMaxHalfDim = 64;        // d_h <= 128
constexpr int kPageBlock = 16;         // tokens per cache block (paged prefill)
constexpr int kMaxPagedBlocks = 4096;  // block-table entries a paged prefill holds on chip

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;  // may be null
  int B, Hq, Hkv, T, S;
  int causal;
  int use_rope;
  int64_t window;  // > 0: causal sliding window, key s visible iff pos + t - window < s <= pos + t
  void* k_rot;     // bf16 with RoPE: [B, Hkv, S, d_h] buffer for k rotated ahead of the kernel, or
                   // null (k rotated as its blocks land)
  // paged prefill (k, v are block-tabled caches [blocks, Hkv, 16, d_h]; S and pos per sequence)
  int paged;
  const int32_t* block_table;  // [B, max_blocks_per_seq]
  const int32_t* seq_lens;     // [B] cached tokens, the last T of them being the queries
  int max_blocks_per_seq;
  int num_blocks;
  int n_qblocks;  // query blocks per (batch, head group)
  int n_groups;   // batch * head groups
  int xcd_remap;  // work order mode (work_order in attn_common.h)
  int64_t pos;
  float q_scale, k_scale, v_scale;  // fp8 prefill: value = code * scale
  // RoPE: rope_c[i] = rope_base^(-2i/d_h) / (2 pi), i = 0..d_h/2-1 (turns per position).
  double rope_c[kMaxHalfDim];
};

// Backward pass (bf16, d_h = 128).  The workspace holds the per-row statistics and, with
// RoPE, the rotated q and k that both gradient kernels read.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* rec;        // [B, Hq, T] 16-byte row records: -lse*log2(e) and -rowsum(dout * out),
                    // each as three bf16 pieces (hi, mid, lo) and a zero
  void* qr;         // [B, Hq, T, d_h] bf16 q, rotated (RoPE) and scaled by log2(e) / sqrt(d_h)
  void* kr;         // [B, Hkv, S, d_h] bf16 rotated k (RoPE), else null
  int B, Hq, Hkv, T, S;
  int causal;
  int use_rope;
  int64_t window;   // > 0: causal sliding window, as in FwdParams
  int64_t pos;
  int n_qblocks, n_kblocks, n_groups, xcd_remap;
  double rope_c[kMaxHalfDim];
};

}  // namespace attn
