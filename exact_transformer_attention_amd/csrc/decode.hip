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
// Per wave, two 16-token blocks per step:
//   S^T[token][head] = K q^T   v_mfma_f32_16x16x32_bf16, K straight from HBM as the
//                              A operand (lane: token lane%16, 8 dims), q^T from registers
//   online softmax per lane    a lane owns one head (lane%16) and 8 of the 32 tokens
//   O^T[dim][head] += V^T P^T  P^T is the B operand as it sits in registers; V^T comes
//                              from LDS through ds_read_b64_tr_b16 (V stays row-major)
#include <math.h>

#include "attn_common.h"
#include "launchers.h"

namespace attn {

constexpr int kDecD = 128;        // head size served by the decode kernels
constexpr int kDecBlock = 16;     // tokens per cache block
constexpr int kDecWaves = 4;

// Element offset of the (physical block, kv head) slice holding token block `j` of
// sequence `b`.  The only place the block table is read; used by every paged kernel.
__device__ __forceinline__ size_t paged_slice(const int32_t* __restrict__ block_table,
                                              int max_blocks_per_seq, int b, int j, int Hkv,
                                              int kvh, int d) {
  const int phys = block_table[(size_t)b * max_blocks_per_seq + j];
  return (((size_t)phys * Hkv + kvh) * kDecBlock) * (size_t)d;
}

// LDS position (in 16-byte chunks) of chunk c of token row t inside one staged V block:
// rows of 16 chunks, chunk index xor-swizzled by 2t so the transpose reads of a
// half-wave (8 rows x 2 chunks) fall on 16 distinct bank groups.
__device__ __forceinline__ int vpos(int t, int c) { return t * 16 + (c ^ ((2 * t) & 15)); }

__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeParams p) {
  __shared__ u32x4 vlds[kDecWaves][2][kDecBlock * 16];            // 16 KiB
  __shared__ float red_o[kDecWaves][16][kDecD + 1];                // per-wave partial outputs
  __shared__ float red_ml[kDecWaves][16][2];

  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int grp = lane / 16;   // 16-lane group
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

  float m = -INFINITY;  // running max (base 2), same in all four groups for a head
  float l = 0.f;        // this lane's partial normaliser
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const __bf16* kc = (const __bf16*)p.k_cache;
  const __bf16* vc = (const __bf16*)p.v_cache;

  for (int j = wb0; j < wb1; j += 2) {
    const bool has1 = (j + 1) < wb1;
    size_t sl[2];
    sl[0] = paged_slice(p.block_table, p.max_blocks_per_seq, b, j, p.Hkv, kvh, kDecD);
    sl[1] = has1 ? paged_slice(p.block_table, p.max_blocks_per_seq, b, j + 1, p.Hkv, kvh, kDecD) : sl[0];

    // K as the A operand: token l16, dims grp*8 + 32*kk.
    bf16x8 ka[2][4];
    u32x4 vr[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ka[u][kk] = *(const bf16x8*)(kc + sl[u] + (size_t)l16 * kDecD + grp * 8 + 32 * kk);
      // V rows for LDS staging: load i covers rows 4i..4i+3, chunk chosen by the swizzle
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * i + grp;
        const int c = l16 ^ ((2 * t) & 15);
        vr[u][i] = *(const u32x4*)(vc + sl[u] + (size_t)t * kDecD + c * 8);
      }
    }

    // S^T for both blocks.
    f32x4 s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][kk], qop[kk], acc, 0, 0, 0);
      s[u] = acc;
    }
    // Mask tokens past the sequence (and the absent second block) by selection.
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = (j + u) * kDecBlock + grp * 4 + r;
        const bool vis = (u == 0 || has1) && tok < L;
        s[u][r] = vis ? s[u][r] : -INFINITY;
        tmax = fmaxf(tmax, s[u][r]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // Stage V (rows past the sequence become zeros, so a poisoned slot never reaches
    // the product).
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * i + grp;
        const int c = l16 ^ ((2 * t) & 15);
        const int tok = (j + u) * kDecBlock + t;
        const bool vis = (u == 0 || has1) && tok < L;
        u32x4 val = vr[u][i];
        if (!vis) val = (u32x4){0u, 0u, 0u, 0u};
        vlds[wid][u][vpos(t, c)] = val;
      }
    }

    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float psum = 0.f;
    u32x4 pk;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float p0 = fast_exp2(s[u][0] - m_use), p1 = fast_exp2(s[u][1] - m_use);
      const float p2 = fast_exp2(s[u][2] - m_use), p3 = fast_exp2(s[u][3] - m_use);
      psum += (p0 + p1) + (p2 + p3);
      pk[2 * u] = pack_bf16(p0, p1);
      pk[2 * u + 1] = pack_bf16(p2, p3);
    }
    l = l * alpha + psum;
    m = m_new;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);

    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_wave_barrier();

    // O^T += V^T P^T over the 32 tokens, 16 dims per product.
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int dim = 16 * mb + 4 * (l16 % 4);
      const int c = dim / 8, half = (dim % 8) / 4;
      const int t = 4 * grp + l16 / 4;
      const char* base0 = (const char*)&vlds[wid][0][0];
      const char* base1 = (const char*)&vlds[wid][1][0];
      const int off = vpos(t, c) * 16 + half * 8;
      s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(base0 + off));
      s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(base1 + off));
      const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
      const u32x4 aw = {w0[0], w0[1], w1[0], w1[1]};
      f32x4 acc = o[mb];
      acc[0] *= alpha;
      acc[1] *= alpha;
      acc[2] *= alpha;
      acc[3] *= alpha;
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw), pop, acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // reads of this stage finish before it is overwritten
  }

  // Combine the four token groups of a head: l sums, m is shared.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // Per-wave partials into LDS, then merge the waves of the workgroup.
  if (l16 < G) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[wid][l16][16 * mb + 4 * grp + r] = o[mb][r];
    if (grp == 0) {
      red_ml[wid][l16][0] = m;
      red_ml[wid][l16][1] = l;
    }
  }
  __syncthreads();
  const int nwav = min(kDecWaves, (blk1 - blk0 + share - 1) / share);
  for (int idx = threadIdx.x; idx < G * kDecD; idx += blockDim.x) {
    const int hh = idx / kDecD, d = idx % kDecD;
    float M = -INFINITY;
    for (int ww = 0; ww < nwav; ++ww) M = fmaxf(M, red_ml[ww][hh][0]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
    for (int ww = 0; ww < nwav; ++ww) {
      const float sc = fast_exp2(red_ml[ww][hh][0] - Mu);
      acc += sc * red_o[ww][hh][d];
      lsum += sc * red_ml[ww][hh][1];
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
  return 32;  // 512 tokens per split, 8 blocks per wave
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  const long long grid = (long long)p.num_seqs * p.Hkv * p.max_splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_partial_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
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
