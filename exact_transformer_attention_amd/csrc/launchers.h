// Internal launch functions, one per kernel family (defined next to their kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {

hipError_t launch_fwd_f32(const FwdParams& p, int d_h, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, int d_h, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream);

// Backward: preprocess, dK/dV and dQ kernels, enqueued in that order.
hipError_t launch_bwd_bf16(BwdParams p, hipStream_t stream);

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;  // may be null
  float* part_o;      // [slots, Hq / Hkv, d_h] fp32 unnormalised outputs
  float* part_ml;     // [slots, Hq / Hkv, 2] fp32 (reference max in base 2, normaliser)
  int32_t* seq_prefix;  // [num_seqs + 1] cache blocks before each sequence (written by the kernel)
  void* copy_dst;       // copy mode (attn_paged_gather): [num_seqs, Hkv, max_blocks_per_seq * 16] rows of 256 B
  int num_seqs, Hq, Hkv, max_blocks_per_seq, num_blocks;
  int nwaves;         // grid of the partial kernel: one wave per workgroup
  int use_rope;
  double rope_c[64];
};

// Waves of the decode partial kernel: enough to fill the chip while all stay resident
// (ten 16 KiB LDS rings per compute unit).
constexpr int kDecodeWaves = 2048;
int decode_num_waves(int num_seqs, int Hkv, int max_blocks_per_seq);
// Device address of the decode's static scratch on the GPU that `stream` belongs to (the
// current GPU for the null stream); looked up once per GPU.
hipError_t decode_static_scratch(hipStream_t stream, void** ptr);
// Partial-result slots the decode kernels may write for these sizes.
long long decode_num_slots(int num_seqs, int Hkv, int max_blocks_per_seq);
hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream);
// The decode kernel's read path in copy mode: every staged cache block is written out in
// sequence order instead of being attended to (p.k_cache is the cache, p.copy_dst the
// destination; 256-byte rows).
hipError_t launch_paged_gather(const DecodeParams& p, hipStream_t stream);

}  // namespace attn
