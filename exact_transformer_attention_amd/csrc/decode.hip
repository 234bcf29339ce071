// Paged-KV decode: one new query token per sequence against a block-tabled cache.
//
// "Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in Code"
// (Part 3) describes the cache as fixed-size blocks located through a per-sequence
// block table; "Why is attention O(n^2) ..." notes that a decode step must read the
// whole KV cache and is memory-bound.  The work is therefore cut along the key axis:
// workgroup (sequence, KV head, split) reads its split's blocks once, serves all query
// heads that share the KV head, and leaves an unnormalised partial (o, m, l); a second
// kernel combines the splits with the same rescaling that the online softmax uses
// between key blocks ("Deep dive: FlashAttention" of the same page).
//
// A workgroup is one wave.  It streams its split (96 cache blocks = 1536 tokens at
// most) one 16-token block at a time through a private 2-stage LDS ring filled by
// direct 16-byte loads (global_load_lds_dwordx4) one block ahead, so the bytes in
// flight do not occupy registers and a CU can hold ten such workgroups (memory
// parallelism comes from many small, independent streams).  The wave's block-table
// entries are read once, one per lane, and broadcast per block with readlane.  Per
// block:
//   S^T[token][head] = K q^T   v_mfma_f32_16x16x32_bf16; the K operand is read from LDS
//                              (xor-swizzled rows: conflict-free), q^T sits in registers
//   probabilities              a lane owns one head (lane % 16) and 4 of the 16 tokens
//   O^T[dim][head] += V^T P^T  v_mfma_f32_16x16x16_bf16: P^T is the B operand exactly as
//                              the S^T accumulators sit in registers; V^T comes from LDS
//                              through ds_read_b64_tr_b16 (V stays row-major)
// The running max is only a reference: it is set from the first block and re-derived
// (with o and l rescaled) only when a block's probabilities sum past 2^16, so the
// common path has no cross-lane reduction.
#include <math.h>

#include "attn_common.h"
#include "launchers.h"

namespace attn {

constexpr int kDecD = 128;        // head size served by the decode kernels
constexpr int kDecBlock = 16;     // tokens per cache block
constexpr int kDecWaves = 1;
constexpr int kStages = 2;        // LDS ring depth per wave (blocks)
constexpr int kStageBytes = 2 * kDecBlock * kDecD * 2;  // K and V of one block

// Element offset of the (physical block, kv head) slice holding token block `j` of
// sequence `b`.  The only place the block table is read; used by every paged kernel.
__device__ __forceinline__ size_t paged_slice(const int32_t* __restrict__ block_table,
                                              int max_blocks_per_seq, int b, int j, int Hkv,
                                              int kvh, int d) {
  const int phys = block_table[(size_t)b * max_blocks_per_seq + j];
  return (((size_t)phys * Hkv + kvh) * kDecBlock) * (size_t)d;
}

// 16-byte chunk position of chunk c of token row t inside a staged K block: reading
// chunk c of all 16 rows (the MFMA operand pattern) then hits 16 distinct bank groups.
__device__ __forceinline__ int kpos(int t, int c) { return t * 16 + (c ^ t); }
// Same for V under the transpose-read pattern (a half wave reads 8 rows x 2 chunks).
__device__ __forceinline__ int vpos(int t, int c) { return t * 16 + (c ^ ((2 * t) & 15)); }

__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];  // kDecWaves * kStages * kStageBytes

  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int grp = lane / 16;  // 16-lane group
  const int l16 = lane % 16;
  int w = blockIdx.x;
  const int sp = w % p.max_splits;
  w /= p.max_splits;
  const int kvh = w % p.Hkv;
  const int b = w / p.Hkv;
  const int L = p.seq_lens[b];
  const int nblk = (L + kDecBlock - 1) / kDecBlock;
  const int bps = p.blocks_per_split;
  const int blk0 = sp * bps;
  if (blk0 >= nblk) return;  // uniform over the workgroup
  const int blk1 = min(nblk, blk0 + bps);
  const int G = p.Hq / p.Hkv;
  const int head = kvh * G + l16;  // valid when l16 < G

  // q^T operand: lane holds head l16, dims grp*8 + 32*kk .. +7; rotated at L-1, with
  // the base-2 softmax scale folded in.
  bf16x8 qop[4];
  {
    const float qscale = kLog2e / sqrtf((float)kDecD);
    const int64_t qposn = (int64_t)L - 1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (l16 < G) {
        const u32x4* src = (const u32x4*)((const __bf16*)p.q + ((size_t)b * p.Hq + head) * kDecD +
                                          grp * 8 + 32 * kk);
        raw = *src;
      }
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
        if (p.use_rope) {
          const int pair = (grp * 8 + 32 * kk) / 2 + e;
          const float turns = rope_turns(qposn, p.rope_c[pair]);
          float sn, cs;
          sincos_rev(turns, &sn, &cs);
          const float y0 = x0 * cs - x1 * sn;
          const float y1 = x0 * sn + x1 * cs;
          x0 = y0;
          x1 = y1;
        }
        packed[e] = pack_bf16(x0 * qscale, x1 * qscale);
      }
      qop[kk] = __builtin_bit_cast(bf16x8, packed);
    }
  }

  // This wave's contiguous share of the split.
  const int share = (bps + kDecWaves - 1) / kDecWaves;
  const int wb0 = blk0 + wid * share;
  const int wb1 = min(blk1, wb0 + share);
  const int nmine = max(0, wb1 - wb0);

  char* ring = dsm + (size_t)wid * kStages * kStageBytes;
  const __bf16* kc = (const __bf16*)p.k_cache;
  const __bf16* vc = (const __bf16*)p.v_cache;

  // This wave's block-table entries, one per lane (read once, then broadcast per block).
  const int tbl = (lane < nmine) ? p.block_table[(size_t)b * p.max_blocks_per_seq + wb0 + lane] : 0;
  const int tbl2 = (lane + 64 < nmine) ? p.block_table[(size_t)b * p.max_blocks_per_seq + wb0 + 64 + lane] : 0;

  // Direct loads of block j into stage st: load i covers token rows 4i .. 4i+3.
  auto issue = [&](int j, int st) {
    const int jj = j - wb0;
    const int phys = jj < 64 ? __builtin_amdgcn_readlane(tbl, jj) : __builtin_amdgcn_readlane(tbl2, jj - 64);
    const size_t sl = (((size_t)phys * p.Hkv + kvh) * kDecBlock) * (size_t)kDecD;
    char* kdst = ring + st * kStageBytes;
    char* vdst = kdst + kStageBytes / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + grp;
      load_lds16(kc + sl + (size_t)t * kDecD + (l16 ^ t) * 8, kdst + i * 1024);
      load_lds16(vc + sl + (size_t)t * kDecD + (l16 ^ ((2 * t) & 15)) * 8, vdst + i * 1024);
    }
  };

  float m_ref = -INFINITY;  // reference max (base 2) for head l16, same in its 4 lanes
  float l = 0.f;            // this lane's partial normaliser
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // prologue: kStages-1 blocks in flight
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < nmine) issue(wb0 + i, i);

  for (int i = 0; i < nmine; ++i) {
    const int j = wb0 + i;
    const int st = i % kStages;
    if (i + kStages - 1 < nmine) {
      issue(j + kStages - 1, (i + kStages - 1) % kStages);
      __builtin_amdgcn_s_waitcnt(0x0f70 | (8 * (kStages - 1)));  // block j has landed
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);
    }
    const char* kst = ring + st * kStageBytes;
    const char* vst = kst + kStageBytes / 2;

    // S^T = K q^T for the 16 tokens of the block.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *(const bf16x8*)(kst + kpos(l16, grp + 4 * kk) * 16);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[kk], s, 0, 0, 0);
    }
    // tokens past the sequence are selected away (their cache slots may hold anything)
    const bool tail = (j + 1) * kDecBlock > L;
    if (tail) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (j * kDecBlock + grp * 4 + r >= L) s[r] = -INFINITY;
    }
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(s[r] - mu);
    float bsum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
    if (__any(m_ref == -INFINITY || !(bsum <= 65536.f))) {
      __asm__ volatile("");  // rare: derive the reference from this block's max
      float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const bool raise = tmax > m_ref + 8.f || (m_ref == -INFINITY && tmax > -INFINITY);
      const float m_new = raise ? tmax : m_ref;
      const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;  // 0 when m_ref was -inf
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[mb][r] *= alpha;
      m_ref = m_new;
      const float mu2 = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(s[r] - mu2);
      bsum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
    }
    l += bsum;
    // masked tokens have p = 0, but their V slots may hold non-finite values: zero the
    // probabilities AND make sure the transposed V values of those rows are not used by
    // selecting the P operand only (0 * NaN would still poison the product), see below
    const u32x2 pk = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
    const s16x4 pop = __builtin_bit_cast(s16x4, pk);
    // O^T += V^T P^T, 16 dims per product.
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int t = 4 * grp + l16 / 4;
      const int dim = 16 * mb + 4 * (l16 % 4);
      const int c = dim / 8, half = (dim % 8) / 4;
      s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vst + vpos(t, c) * 16 + half * 8));
      if (tail) {
        // rows (tokens) past the sequence: this lane's 4 values come from tokens
        // 4 * grp .. 4 * grp + 3 of the block (transpose read); zero the invalid ones
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j * kDecBlock + grp * 4 + r >= L) a[r] = 0;
      }
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pop, o[mb], 0, 0, 0);
    }
  }

  // Combine the four token groups of a head: l sums, m is shared.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // Per-wave partials into LDS (reusing the ring), then merge the waves of the workgroup.
  __syncthreads();
  float* red_o = (float*)dsm;                            // [kDecWaves][16][kDecD + 1]
  float* red_ml = red_o + kDecWaves * 16 * (kDecD + 1);  // [kDecWaves][16][2]
  if (l16 < G) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[(wid * 16 + l16) * (kDecD + 1) + 16 * mb + 4 * grp + r] = o[mb][r];
    if (grp == 0) {
      red_ml[(wid * 16 + l16) * 2] = m_ref;
      red_ml[(wid * 16 + l16) * 2 + 1] = l;
    }
  }
  __syncthreads();
  const int nwav = min(kDecWaves, (blk1 - blk0 + share - 1) / share);
  for (int idx = threadIdx.x; idx < G * kDecD; idx += blockDim.x) {
    const int hh = idx / kDecD, d = idx % kDecD;
    float M = -INFINITY;
    for (int ww = 0; ww < nwav; ++ww) M = fmaxf(M, red_ml[(ww * 16 + hh) * 2]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
    for (int ww = 0; ww < nwav; ++ww) {
      const float sc = fast_exp2(red_ml[(ww * 16 + hh) * 2] - Mu);
      acc += sc * red_o[(ww * 16 + hh) * (kDecD + 1) + d];
      lsum += sc * red_ml[(ww * 16 + hh) * 2 + 1];
    }
    const size_t slot = ((size_t)b * p.Hq + kvh * G + hh) * p.max_splits + sp;
    p.part_o[slot * kDecD + d] = acc;
    if (d == 0) {
      p.part_ml[slot * 2] = M;
      p.part_ml[slot * 2 + 1] = lsum;
    }
  }
}

// Log-sum-exp merge of the split partials of one (sequence, query head).
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int d = threadIdx.x;
  const int L = p.seq_lens[b];
  const int nblk = (L + kDecBlock - 1) / kDecBlock;
  const int nsp = (nblk + p.blocks_per_split - 1) / p.blocks_per_split;
  const size_t base = (size_t)bh * p.max_splits;
  float M = -INFINITY;
  for (int i = 0; i < nsp; ++i) M = fmaxf(M, p.part_ml[(base + i) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float acc = 0.f, lsum = 0.f;
  for (int i = 0; i < nsp; ++i) {
    const float sc = fast_exp2(p.part_ml[(base + i) * 2] - Mu);
    lsum += sc * p.part_ml[(base + i) * 2 + 1];
    acc += sc * p.part_o[(base + i) * kDecD + d];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  ((__bf16*)p.out)[(size_t)bh * kDecD + d] = (__bf16)(acc * inv);
  if (p.lse && d == 0) p.lse[bh] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
}

// Exact copy of each sequence's cached rows through the block table.
__global__ __launch_bounds__(256) void paged_gather_kernel(const char* cache, const int32_t* block_table,
                                                           const int32_t* seq_lens, int Hkv, int d_h,
                                                           int max_blocks_per_seq, int elem_bytes,
                                                           char* dst) {
  int w = blockIdx.x;
  const int j = w % max_blocks_per_seq;
  w /= max_blocks_per_seq;
  const int kvh = w % Hkv;
  const int b = w / Hkv;
  const int L = seq_lens[b];
  const int nblk = (L + kDecBlock - 1) / kDecBlock;
  if (j >= nblk) return;
  const size_t src = paged_slice(block_table, max_blocks_per_seq, b, j, Hkv, kvh, d_h);
  const size_t row_bytes = (size_t)d_h * elem_bytes;
  const size_t cap = (size_t)max_blocks_per_seq * kDecBlock;
  for (int t = threadIdx.x / 16; t < kDecBlock; t += blockDim.x / 16) {
    const int tok = j * kDecBlock + t;
    if (tok >= L) break;
    const char* s = cache + (src + (size_t)t * d_h) * elem_bytes;
    char* dd = dst + (((size_t)b * Hkv + kvh) * cap + tok) * row_bytes;
    for (size_t o = (threadIdx.x % 16) * 4; o < row_bytes; o += 64)
      *(uint32_t*)(dd + o) = *(const uint32_t*)(s + o);
  }
}

int decode_blocks_per_split(int max_blocks_per_seq) {
  (void)max_blocks_per_seq;
  return 96;  // 1536 tokens per split
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  const long long grid = (long long)p.num_seqs * p.Hkv * p.max_splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  constexpr size_t lds = (size_t)kDecWaves * kStages * kStageBytes;
  static_assert(lds >= (size_t)kDecWaves * 16 * (kDecD + 1) * 4 + kDecWaves * 16 * 2 * 4,
                "the reduction buffer reuses the staging ring");
  hipLaunchKernelGGL(decode_partial_kernel, dim3((unsigned)grid), dim3(64), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(p.num_seqs * p.Hq)), dim3(kDecD), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_paged_gather(const void* cache, const int32_t* block_table, const int32_t* seq_lens,
                               int num_seqs, int Hkv, int d_h, int max_blocks_per_seq, int elem_bytes,
                               void* dst, hipStream_t stream) {
  const long long grid = (long long)num_seqs * Hkv * max_blocks_per_seq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(paged_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const char*)cache,
                     block_table, seq_lens, Hkv, d_h, max_blocks_per_seq, elem_bytes, (char*)dst);
  return hipGetLastError();
}

}  // namespace attn
