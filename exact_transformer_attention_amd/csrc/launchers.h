// Internal launch functions, one per kernel family (defined next to their kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {

hipError_t launch_fwd_f32(const FwdParams& p, int d_h, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, int d_h, hipStream_t stream);

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;  // may be null
  float* part_o;    // [num_seqs, Hq, max_splits, d_h] fp32 normalised partial outputs
  float* part_ml;   // [num_seqs, Hq, max_splits, 2] fp32 (max in base 2, normaliser)
  int num_seqs, Hq, Hkv, max_blocks_per_seq, num_blocks;
  int max_splits;
  int blocks_per_split;
  int use_rope;
  double rope_c[64];
};

// Split size used by the decode kernels, in cache blocks of 16 tokens.
int decode_blocks_per_split(int max_blocks_per_seq);
hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream);
hipError_t launch_paged_gather(const void* cache, const int32_t* block_table,
                               const int32_t* seq_lens, int num_seqs, int Hkv, int d_h,
                               int max_blocks_per_seq, int elem_bytes, void* dst,
                               hipStream_t stream);

}  // namespace attn
