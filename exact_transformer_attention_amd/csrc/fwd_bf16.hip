// bf16 exact attention prefill on gfx950 matrix cores (fp32 accumulation).
//
// The computation is the blocked online softmax of "Why is attention O(n^2), how does
// FlashAttention help ..." (Deep dive: FlashAttention): a block of queries stays on
// chip, key/value blocks stream through LDS, and each query row keeps a running max m,
// normaliser l and unnormalised output o that are rescaled when m grows, so the
// T x S score matrix never reaches HBM.  Causal masking sets hidden logits to -inf
// before the softmax ("Transformer Attention Mechanism Interview Deep Dive", Causal
// masking) and key blocks hidden from a whole wave are skipped.
//
// Mapping onto CDNA4 (wave64, v_mfma_f32_32x32x16_bf16):
//  * workgroup = 8 waves, two per SIMD; each wave owns 32 query rows of one head.  The
//    heads that share one KV head (grouped-query attention) are packed into the same
//    workgroup (HP heads per workgroup), so every K/V block loaded, and rotated, once
//    serves 256 query rows.  With one 32-query block per wave the per-wave state fits
//    in VGPRs, and the two waves of a SIMD overlap one's softmax/RoPE work with the
//    other's matrix products.
//  * S^T = K Q^T: K (64-key block) is the A operand read from LDS, Q^T the B operand
//    held in registers for the whole kernel.  In the accumulator layout a lane owns
//    one query column, so row sums are in-lane except for one swap with the lane 32
//    apart.
//  * The running max is subtracted inside the matrix product: one extra k-step pairs
//    a constant 1 on the K side with -m on the Q side, so the accumulators already
//    hold s - m and each probability is a single exp2.  m is kept to a 16-bit significand
//    for that purpose (the sum of two bf16 pieces, so the k-step subtracts it exactly at
//    any magnitude); it is only a reference point, so any value works as long as the same
//    one scales o, l and the final lse.
//  * The reference is not recomputed every block.  Probabilities are formed against the
//    current reference; only when a row has no reference yet, or a half block's row sum
//    exceeds 2^16 (the reference is stale by more than ~16 in log2 units), is the exact
//    block max taken, the reference raised to it, o and l rescaled and the half
//    recomputed.  p <= 2^16 stays far inside fp32 and bf16 range and o / l is unchanged.
//  * O^T = V^T P^T: P^T is the B operand exactly as the S^T accumulators sit in
//    registers (the contraction order over keys is permuted to match), V^T is read
//    from a row-major LDS tile with ds_read_b64_tr_b16.  A lane owns one query, so the
//    rescale factor is a per-lane scalar.
//  * Logits are in the base-2 domain: RoPE'd q is pre-multiplied by log2(e)/sqrt(d_h)
//    before rounding to bf16, so p = exp2(s - m).
//  * K and V move from HBM to LDS with direct 16-byte loads (global_load_lds_dwordx4),
//    so no registers are tied up by loads in flight.  V lands in its final, xor-swizzled
//    layout.  K that needs no rotation here (keys rotated once ahead by rope_k_kernel, the
//    paged cache's rotated keys, or no RoPE) lands straight in its padded operand tile;
//    otherwise raw K lands in a staging area and each thread rotates the chunks it loaded
//    (RoPE at load) into the padded K tile, with angles advanced from block to block by
//    angle addition and re-derived exactly (fp64 reduction) every 16 blocks.  A K block is
//    read by every query block of its group, so rotating it once ahead pays when those
//    are many (the host decides, given a workspace).
//  * V and direct K are loaded one block ahead; raw K two blocks ahead, the rotation of
//    block j+1 happening during block j.  Work is ordered longest-first for causal load balance and
//    mapped so all query blocks of one KV head land on one XCD; with enough query blocks
//    per group the XCD runs its groups one after the other (one group's K/V in its L2 at
//    a time), else it interleaves them longest first (work_order).
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "fwd_params.h"
#include "launchers.h"
#include "prefill_common.h"

namespace attn {

namespace {

constexpr int kNB = 1;        // 32-query n-blocks per wave
constexpr int kNW = 8;        // waves per workgroup (two per SIMD)
constexpr int kQW = 32 * kNB; // query rows per wave
constexpr int kBN = 64;       // keys per block
constexpr int kThreads = kNW * kWave;
constexpr int kResync = 16;   // blocks between exact re-derivations of the RoPE angles

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;                 // k-steps of the QK^T product
  static constexpr int DB = D / 32;                 // 32-wide dim blocks of the output
  static constexpr int KSTR = D + 8;                // rotated-K row stride in LDS (bf16)
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int NCH = kBN * CPR / kThreads;  // chunks per thread per tensor
  static constexpr int RSTEP = kWave / CPR;         // rows between a thread's chunks
};

using prefill::cmul;
using prefill::max3;
using prefill::vswz;

// Where the prefill kernel takes its keys from.
constexpr int kKeysIn = 0;       // the k tensor; with RoPE rotated as each block lands
constexpr int kKeysPaged = 1;    // a block-tabled cache, already rotated
constexpr int kKeysRotated = 2;  // a copy of k rotated ahead of the kernel (rope_k_kernel)

}  // namespace

// Keys rotated ahead of the prefill: k'[b, kvh, s] = RoPE(k[b, kvh, s]) at position s, in
// the layout of k.  One 16-byte chunk (4 pairs) per thread; the angles are reduced in fp64
// per element ("How does Rotary Position Embedding (RoPE) work?").  A K block is read by
// every query block of its group, so rotating it once here beats rotating it in each of
// them when there are enough of them (the host decides).
template <int D>
__global__ __launch_bounds__(256) void rope_k_kernel(const __bf16* __restrict__ k, __bf16* __restrict__ kr,
                                                     long long n_chunks, int S, FwdParams p) {
  constexpr int CPR = D / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int c = (int)(i % CPR);
  const int64_t ps = (i / CPR) % S;
  const u32x4 raw = *(const u32x4*)(k + i * 8);
  u32x4 outv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float sn, cs;
    sincos_rev(rope_turns(ps, p.rope_c[c * 4 + e]), &sn, &cs);
    const float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
    outv[e] = pack_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
  }
  *(u32x4*)(kr + i * 8) = outv;
}

// KSRC (where the keys come from): kKeysIn, kKeysRotated, or kKeysPaged: K and V from a
// block-tabled cache ([blocks, Hkv, 16, D], as the decode kernels read it), sequence b
// holding seq_lens[b] tokens whose last T are the queries.  Cached and pre-rotated K are
// used as they are; Q is rotated (at its positions) whenever ROPE.
template <int D, int HP, bool ROPE, int KSRC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kNW / 4, kNW / 4)))
void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D>;
  constexpr bool PAGED = KSRC == kKeysPaged;
  constexpr bool ROTK = ROPE && KSRC == kKeysIn;  // rotate K at load
  // K copied by the loads straight into its operand tile when the kernel does not rotate
  // it; otherwise K lands in Kraw and each thread rotates the chunks it loaded.
  constexpr bool KDIRECT = !ROTK;
  // K operand tiles (padded rows) of the two blocks in flight: two arrays, so that reads of
  // one are never held up by the compiler for loads into the other
  __shared__ __attribute__((aligned(16))) __bf16 Ks0[kBN * C::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Ks1[kBN * C::KSTR];
  __shared__ __attribute__((aligned(16))) u32x4 Vs[2][kBN * C::CPR];     // V, swizzled 16-byte chunks
  __shared__ __attribute__((aligned(16))) u32x4 Kraw[KDIRECT ? 1 : 2][kBN * C::CPR];  // K as loaded
  auto ks_tile = [&](auto bc) -> __bf16* {
    if constexpr (decltype(bc)::value == 0) return Ks0;
    else return Ks1;
  };
  __shared__ int32_t tbl[PAGED ? kMaxPagedBlocks : 1];                     // block table row

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar values and branches
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int g = lane / 32;

  // ---- work item: (batch, head group, query block), longest causal blocks first, all
  // blocks of one head group on one XCD (work_order).
  constexpr int RH = kNW * kQW / HP;  // rows per head per workgroup
  int qb, grp;
  {
    const int bid = blockIdx.x;
    int rank;
    work_order(bid, p.n_qblocks, p.n_groups, p.xcd_remap, rank, grp);
    qb = p.n_qblocks - 1 - rank;
  }
  const int hpg = p.Hq / HP;
  const int b = grp / hpg;
  const int hq = (grp % hpg) * HP + wid / (kNW / HP);
  const int kvh = ((grp % hpg) * HP) / (p.Hq / p.Hkv);
  const int T = p.T;
  int S = p.S;
  int64_t pos = p.pos;
  if constexpr (PAGED) {  // this sequence's keys; its queries are its last T tokens
    S = min(p.seq_lens[b], p.max_blocks_per_seq * kPageBlock);
    pos = (int64_t)S - T;
    const int nblk = (S + kPageBlock - 1) / kPageBlock;
    for (int i = tid; i < nblk; i += kThreads) tbl[i] = p.block_table[(size_t)b * p.max_blocks_per_seq + i];
    __syncthreads();
  }
  const int wrow0 = qb * RH + (wid % (kNW / HP)) * kQW;  // first query row of this wave

  const __bf16* qg = (const __bf16*)p.q + ((size_t)b * p.Hq + hq) * (size_t)T * D;
  const __bf16* kg = (const __bf16*)p.k + (PAGED ? 0 : ((size_t)b * p.Hkv + kvh) * (size_t)S * D);
  const __bf16* vg = (const __bf16*)p.v + (PAGED ? 0 : ((size_t)b * p.Hkv + kvh) * (size_t)S * D);

  // ---- keys visible to this wave / to the workgroup.
  int nk_wave = S, nk_wg = S;
  if (p.causal) {
    const int64_t lw = pos + (int64_t)min(T - 1, wrow0 + kQW - 1) + 1;
    nk_wave = (int)(lw < 0 ? 0 : (lw < S ? lw : S));
    const int64_t lg = pos + (int64_t)min(T - 1, qb * RH + RH - 1) + 1;
    nk_wg = (int)(lg < 0 ? 0 : (lg < S ? lg : S));
  }
  const int n_tiles = (nk_wg + kBN - 1) / kBN;
  // Sliding window: the first key visible to the wave's / the workgroup's first row.
  int64_t lo_wave = 0;
  int it0 = 0;
  if (p.window > 0) {
    lo_wave = pos + wrow0 - p.window + 1;
    const int64_t lo_wg = pos + (int64_t)qb * RH - p.window + 1;
    it0 = (int)(lo_wg <= 0 ? 0 : (lo_wg < nk_wg ? lo_wg : nk_wg)) / kBN;
  }

  // ---- Q^T operand in registers: lane holds query l32 of n-block nb, dims ks*16 + g*8.
  // Only the raw rows are loaded here (with the RoPE frequencies, staged in LDS); the
  // rotation and scaling run in the prologue below, while the first K/V blocks are in
  // flight.
  // The frequency is requested first, so that its wait leaves the Q rows in flight; rows
  // past T load row T - 1 instead (finite values whose outputs are never stored; no
  // per-row branch between the requests).
  __shared__ double ropec_s[ROPE ? D / 2 : 1];
  double rope_c = 0.0;
  if constexpr (ROPE) {
    if (tid < D / 2) rope_c = p.rope_c[tid];
  }
  bf16x8 qop[kNB][C::KS];
  u32x4 qraw[kNB][C::KS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int t = min(wrow0 + nb * 32 + l32, T - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qraw[nb][ks] = *(const u32x4*)(qg + (size_t)t * D + ks * 16 + g * 8);
  }
  if constexpr (ROPE) {
    if (tid < D / 2) ropec_s[tid] = rope_c;
    __syncthreads();
  }
  // Extra k-step: K side holds 1 in slots 0 and 1 of the g = 0 lanes, Q side holds -m there
  // as two bf16 pieces (m has a 16-bit significand, so the pair is exact).
  const bf16x8 ones_op = __builtin_bit_cast(bf16x8, (u32x4){g == 0 ? 0x3f803f80u : 0u, 0u, 0u, 0u});

  // ---- this thread's share of the K/V block copies: chunk `slot` of rows row0 + j*RSTEP.
  const int slot = lane % C::CPR;
  const int row0 = wid * C::NCH * C::RSTEP + lane / C::CPR;

  // RoPE angle state for the 4 pairs of this thread's chunk: (cos, sin) at key
  // tile*64 + row0, plus the per-row and per-block steps.
  float ac[4], as[4], rc[4], rs[4], tc[4], ts[4];
  double cturn[4];
  if constexpr (ROTK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cturn[e] = ropec_s[slot * 4 + e];
      sincos_rev(rope_turns((int64_t)C::RSTEP, cturn[e]), &rs[e], &rc[e]);
      sincos_rev(rope_turns((int64_t)kBN, cturn[e]), &ts[e], &tc[e]);
    }
  }

  // Direct-to-LDS loads: raw K of block `tile` into Kraw[tile & 1] (two blocks ahead of
  // its use), V of block `tile` into Vs[tile & 1] (one block ahead).  NCH loads each,
  // through a buffer resource starting at the block's first row: the per-lane offsets
  // are fixed, and rows past S read as zero (they are never visible).
  int koff[C::NCH], voff[C::NCH];
#pragma unroll
  for (int j = 0; j < C::NCH; ++j) {
    const int r = row0 + j * C::RSTEP;
    koff[j] = (r * D + slot * 8) * 2;
    voff[j] = (r * D + (slot ^ vswz<D>(r)) * 8) * 2;
  }
  auto block_rsrc = [&](const __bf16* base, int k0) {
    return make_rsrc(base + (size_t)k0 * D, (uint32_t)(S - k0) * D * 2);
  };
  // Paged: the cache element offset of key row `key` (clamped to a stored row: rows past
  // S are never visible), through the block table row held in LDS.
  auto paged_row = [&](int key) -> size_t {
    key = min(key, S - 1);
    const int phys = min(max(tbl[key / kPageBlock], 0), p.num_blocks - 1);  // never outside the pool
    return (((size_t)phys * p.Hkv + kvh) * kPageBlock + key % kPageBlock) * (size_t)D;
  };
  auto load_k = [&](int tile) {
    if constexpr (PAGED) {
#pragma unroll
      for (int j = 0; j < C::NCH; ++j)
        load_lds16(kg + paged_row(tile * kBN + row0 + j * C::RSTEP) + slot * 8,
                   &Kraw[tile & 1][(wid * C::NCH + j) * kWave]);
      return;
    }
    const i32x4 rs = block_rsrc(kg, tile * kBN);
#pragma unroll
    for (int j = 0; j < C::NCH; ++j)
      buffer_load_lds16(rs, koff[j], &Kraw[tile & 1][(wid * C::NCH + j) * kWave]);
  };
  // Direct K: the padded operand tile of a block, copied in 1 KB pieces (piece n by wave
  // n % kNW, lane i taking its bytes 16i..16i+15).  Lanes that fall on row padding read a
  // chunk of their row again (the padding is never read back).
  constexpr int kPieces = kBN * C::KSTR * 2 / 1024;
  constexpr int kPiecesPerWave = (kPieces + kNW - 1) / kNW;
  static_assert(kPieces * 1024 == kBN * C::KSTR * 2, "whole pieces");
  int kdoff[kPiecesPerWave];
#pragma unroll
  for (int j = 0; j < kPiecesPerWave; ++j) {
    const int o = (wid + kNW * j) * 1024 + lane * 16;
    const int row = o / (C::KSTR * 2), cb = o % (C::KSTR * 2);
    kdoff[j] = row * D * 2 + (cb < D * 2 ? cb : 0);
  }
  auto load_k_direct = [&](int tile, auto bc) {
    char* dst = (char*)ks_tile(bc);
    if constexpr (PAGED) {
#pragma unroll
      for (int j = 0; j < kPiecesPerWave; ++j)
        if (wid + kNW * j < kPieces)
          load_lds16(kg + paged_row(tile * kBN + kdoff[j] / (D * 2)) + kdoff[j] % (D * 2) / 2,
                     dst + (wid + kNW * j) * 1024);
      return;
    }
    const i32x4 rs = block_rsrc(kg, tile * kBN);
#pragma unroll
    for (int j = 0; j < kPiecesPerWave; ++j)
      if (wid + kNW * j < kPieces) buffer_load_lds16(rs, kdoff[j], dst + (wid + kNW * j) * 1024);
  };
  auto load_v = [&](int tile) {
    if constexpr (PAGED) {
#pragma unroll
      for (int j = 0; j < C::NCH; ++j) {
        const int r = row0 + j * C::RSTEP;
        load_lds16(vg + paged_row(tile * kBN + r) + (slot ^ vswz<D>(r)) * 8,
                   &Vs[tile & 1][(wid * C::NCH + j) * kWave]);
      }
      return;
    }
    const i32x4 rs = block_rsrc(vg, tile * kBN);
#pragma unroll
    for (int j = 0; j < C::NCH; ++j)
      buffer_load_lds16(rs, voff[j], &Vs[tile & 1][(wid * C::NCH + j) * kWave]);
  };
  // Rotate this thread's raw K chunks of block `tile` into Ks[tile & 1].  The caller has
  // waited for the loads of that block.
  auto rotate_k = [&](int tile, auto kbc, const u32x4 (&raw_in)[C::NCH]) {
    constexpr int kb = decltype(kbc)::value;  // == tile & 1
    if constexpr (ROTK) {
      float c[4], s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = ac[e];
        s[e] = as[e];
      }
#pragma unroll
      for (int j = 0; j < C::NCH; ++j) {
        const u32x4 raw = raw_in[j];
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
          out[e] = pack_bf16(x0 * c[e] - x1 * s[e], x0 * s[e] + x1 * c[e]);
          if (j + 1 < C::NCH) cmul(c[e], s[e], rc[e], rs[e]);
        }
        *(u32x4*)&ks_tile(kbc)[(row0 + j * C::RSTEP) * C::KSTR + slot * 8] = out;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) cmul(ac[e], as[e], tc[e], ts[e]);
    } else {
#pragma unroll
      for (int j = 0; j < C::NCH; ++j)
        *(u32x4*)&ks_tile(kbc)[(row0 + j * C::RSTEP) * C::KSTR + slot * 8] = raw_in[j];
    }
  };
  // Exact angles of this thread's first key of block `tile` (every kResync blocks; the
  // angle addition in rotate_k advances them in between).
  auto resync = [&](int tile, bool force = false) {
    if constexpr (ROTK) {
      if (force || tile % kResync == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sincos_rev(rope_turns((int64_t)tile * kBN + row0, cturn[e]), &as[e], &ac[e]);
      }
    }
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0f70); };  // vmcnt(0)

  // ---- running state: two query n-blocks per lane.
  float m_ref[kNB], l_run[kNB];
  // Q side of the extra k-step: -m as two bf16 pieces in slots 0 and 1 of the g = 0 lanes
  // (0 while a row has no reference yet).  Rebuilt only when the reference is raised.
  bf16x8 bop[kNB];
  auto set_bias = [&](int nb) {
    const float bias = (m_ref[nb] == -INFINITY) ? 0.f : m_ref[nb];
    const uint32_t w = prefill::split_bf16_pair(-bias);
    bop[nb] = __builtin_bit_cast(bf16x8, (u32x4){g == 0 ? w : 0u, 0u, 0u, 0u});
  };
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_ref[nb] = -INFINITY;  // reference max (base 2), a 16-bit-significand value
    l_run[nb] = 0.f;
    set_bias(nb);
  }
  f32x16 o[C::DB][kNB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][nb][r] = 0.f;

  // S'^T = K Q^T - m for both 32-key halves and both query n-blocks (the bias k-step first),
  // with the rotation of the next K block woven in: after each k-step
  // (its MFMAs issued), one unit of the rotation (one 4-pair slice of one of this
  // thread's chunks).  The scheduling barrier after each slice keeps the order, so the
  // rotation's vector instructions run while the matrix cores work on that k-step
  // (the K chunks this thread rotates per block, D / 64 of them with 4 pairs each, make
  // exactly D / 16 units, one per k-step).
  auto qk_rot = [&](const __bf16* kb, f32x16 (&s)[2][kNB], auto kbc, const u32x4 (&raw)[C::NCH]) {
    constexpr int kn = decltype(kbc)::value;  // buffer of the block being rotated
    static_assert(C::NCH * 4 == C::KS, "one rotation unit per k-step");
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones_op, bop[nb], acc, 0, 0, 0);
      }
    u32x4 out[C::NCH];
    float c[4], sn[4];
    if constexpr (ROTK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = ac[e];
        sn[e] = as[e];
      }
    }
    bf16x8 a[C::KS][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a[ks][mb] = *(const bf16x8*)(kb + (mb * 32 + l32) * C::KSTR + ks * 16 + g * 8);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (ks + 2 < C::KS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          a[ks + 2][mb] = *(const bf16x8*)(kb + (mb * 32 + l32) * C::KSTR + (ks + 2) * 16 + g * 8);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][mb], qop[nb][ks], s[mb][nb], 0, 0, 0);
      // rotation unit ks: pair slot e of chunk j
      if constexpr (!KDIRECT) {
        const int j = ks / 4, e = ks % 4;
        if constexpr (ROTK) {
          const float x0 = bf16_lo(raw[j][e]), x1 = bf16_hi(raw[j][e]);
          out[j][e] = pack_bf16(x0 * c[e] - x1 * sn[e], x0 * sn[e] + x1 * c[e]);
          if (j + 1 < C::NCH) cmul(c[e], sn[e], rc[e], rs[e]);
          else cmul(ac[e], as[e], tc[e], ts[e]);
        } else {
          out[j][e] = raw[j][e];
        }
        if (e == 3) *(u32x4*)&ks_tile(kbc)[(row0 + j * C::RSTEP) * C::KSTR + slot * 8] = out[j];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // exp2 of one 32-key half for both n-blocks -> bf16 P operands and this half's row sums.
  auto expo = [&](f32x16 (&s)[2][kNB], int mb, bf16x8 (&pop)[kNB][4], float (&lt)[kNB]) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      float lsum;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(s[mb][nb][8 * h + 2 * e]);
          const float p1 = fast_exp2(s[mb][nb][8 * h + 2 * e + 1]);
          pk[e] = pack_bf16(p0, p1);
          lsum = (h == 0 && e == 0) ? p0 + p1 : lsum + (p0 + p1);
        }
        pop[nb][mb * 2 + h] = __builtin_bit_cast(bf16x8, pk);
      }
      lt[nb] = lsum;
    }
  };
  const int a16 = lane / 16, lam = lane % 16;
  // O^T += V^T P^T for one 16-key step.  The transpose-read byte offsets of each 32-dim
  // block are the same for every key step up to a constant (the swizzle only depends on
  // row % 4), so they are computed once.
  int toff[C::DB];
  {
    const int r1 = 4 * g + lam / 4;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int col = db * 32 + 16 * (a16 % 2) + 4 * (lam % 4);  // first of 4 dims
      const int c = col / 8, half = (col % 8) / 4;
      toff[db] = (r1 * C::CPR + (c ^ vswz<D>(r1))) * 16 + half * 8;
    }
  }
  auto pv = [&](const char* vb, int kstep, const bf16x8 (&pop)[kNB][4]) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const char* p1 = vb + toff[db] + kstep * 16 * C::CPR * 16;
      const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(p1 + 8 * C::CPR * 16));
      const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
      const bf16x8 a = __builtin_bit_cast(bf16x8, (u32x4){w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[nb][kstep], o[db][nb], 0, 0, 0);
    }
  };

  // ---- epilogue: O = o / l, lse = (m + log2 l) ln 2.  Waves whose last key block comes
  // before the workgroup's last one (rows that end earlier on the causal diagonal) run it
  // right after the workgroup's last barrier, so their stores drain while the other waves
  // compute that block; no later wait holds the workgroup for them.
  auto computes = [&](int it) {  // whether this wave has keys in block it
    const int k0 = it * kBN;
    return k0 < nk_wave && (int64_t)(k0 + kBN) > lo_wave;
  };
  auto finish = [&]() {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const float lt = l_run[nb] + __shfl_xor(l_run[nb], 32);
      const int t = wrow0 + nb * 32 + l32;
      if (t < T) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        __bf16* og = (__bf16*)p.out + (((size_t)b * p.Hq + hq) * (size_t)T + t) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          u32x2 w[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            w[q4][0] = pack_bf16(o[db][nb][4 * q4 + 0] * inv, o[db][nb][4 * q4 + 1] * inv);
            w[q4][1] = pack_bf16(o[db][nb][4 * q4 + 2] * inv, o[db][nb][4 * q4 + 3] * inv);
          }
          store_block_bf16(og + db * 32, w, g);  // 16-byte pieces
        }
        if (p.lse && g == 0)
          p.lse[((size_t)b * p.Hq + hq) * (size_t)T + t] =
              lt > 0.f ? (m_ref[nb] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  };

  // ---- one block of keys.  PAR = it & 1 is a compile-time constant so that the LDS
  // buffers read (Ks[PAR], Vs[PAR]) and written (Ks[PAR ^ 1], Kraw[PAR], Vs[PAR ^ 1]) are
  // provably distinct and the scheduler may interleave the rotation of block it+1 with
  // the products of block it.
  auto step = [&](auto par, int it) {
    constexpr int PAR = decltype(par)::value;
    __syncthreads();  // block it is rotated and landed; everyone is done with block it-1
    // This thread's raw K chunks of block it+1 are read before any load is issued, and raw
    // K of block it+2 is only requested once the product of block it has read its
    // operands: the compiler cannot tell the LDS buffers apart and would otherwise wait
    // for the loads in flight to land before those reads.  Direct K of block it+1 goes
    // straight into the other operand tile.
    u32x4 raw[C::NCH];
    if constexpr (!KDIRECT) {
#pragma unroll
      for (int j = 0; j < C::NCH; ++j) raw[j] = Kraw[PAR ^ 1][(wid * C::NCH + j) * kWave + lane];
    }
    if (it + 1 < n_tiles) {
      load_v(it + 1);
      if constexpr (KDIRECT) load_k_direct(it + 1, std::integral_constant<int, PAR ^ 1>{});
    }
    const bool rot = it + 1 < n_tiles;  // rotate block it+1 during this iteration
    if (rot) resync(it + 1);
    const int k0 = it * kBN;
    const __bf16* kbuf = ks_tile(par);
    const char* vbuf = (const char*)&Vs[PAR][0];
    if (it == n_tiles - 1 && !computes(it)) finish();
    if (computes(it)) {
      f32x16 s[2][kNB];
      // The rotation of block it+1 is woven into the product; after the last block it
      // rotates stale data into a buffer nobody reads.
      qk_rot(kbuf, s, std::integral_constant<int, PAR ^ 1>{}, raw);
      if constexpr (!KDIRECT)
        if (it + 2 < n_tiles) load_k(it + 2);
      // mask (diagonal / tail blocks only)
      const bool need_mask = (k0 + kBN > S) || (p.causal && (int64_t)(k0 + kBN - 1) > pos + wrow0) ||
                             (p.window > 0 && (int64_t)k0 < lo_wave + kQW - 1);
      if (need_mask) {
        // Element (mb, r) of this lane holds key k0 + g*4 + c with the compile-time offset
        // c = mb*32 + (r/4)*8 + r%4; it is visible iff lo <= c <= hi, the bounds being this
        // query's first and last visible keys relative to k0 + g*4, clamped to 32 bits.
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int64_t lim = pos + wrow0 + nb * 32 + l32;  // last visible key of this query
          const int64_t base = (int64_t)k0 + g * 4;
          int64_t hi = (int64_t)S - 1 - base;
          if (p.causal && lim - base < hi) hi = lim - base;
          int64_t lo = 0;
          if (p.window > 0) lo = lim - p.window + 1 - base;
          int hi32 = (int)(hi < -1 ? -1 : (hi > kBN ? kBN : hi));
          int lo32 = (int)(lo < 0 ? 0 : (lo > kBN ? kBN : lo));
          // opaque to the compiler, which would otherwise compare every element against the
          // 64-bit bounds
          asm volatile("" : "+v"(hi32), "+v"(lo32));
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = mb * 32 + (r / 4) * 8 + (r % 4);
              const bool vis = (c <= hi32) & (c >= lo32);
              s[mb][nb][r] = vis ? s[mb][nb][r] : -INFINITY;
            }
        }
      }
      // Probabilities with the current reference (the product already subtracted it), one
      // 32-key half at a time; O^T += V^T P^T for that half.  The exact block max is only
      // needed when a row has no reference yet or a half's row sum exceeds 2^16 (the
      // reference is stale by more than ~16): then the reference is raised to the max
      // (rounded up to a 16-bit significand), o and l are rescaled, and the half is recomputed.
      bf16x8 pop[kNB][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float lt[kNB];
        expo(s, mb, pop, lt);
        bool bad = false;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) bad |= (m_ref[nb] == -INFINITY) || !(lt[nb] <= 65536.f);
        if (__any(bad)) {
          __asm__ volatile("");  // keep this rare path a real branch (no speculation)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            float tmax = max3(s[mb][nb][0], s[mb][nb][1], s[mb][nb][2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) tmax = max3(tmax, s[mb][nb][r], s[mb][nb][r + 1]);
            tmax = fmaxf(tmax, s[mb][nb][15]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float bias = (m_ref[nb] == -INFINITY) ? 0.f : m_ref[nb];
            const float tabs = tmax + bias;
            const bool need = tabs > m_ref[nb] + 8.f;
            const float m_new = need ? prefill::ceil_sig16(tabs) : m_ref[nb];
            const float alpha = need ? fast_exp2(m_ref[nb] - m_new) : 1.f;  // 0 when m_ref was -inf
            const float delta = need ? m_new - bias : 0.f;
            l_run[nb] *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[db][nb][r] *= alpha;
            m_ref[nb] = m_new;
            set_bias(nb);
            // this half and the next one were computed against the old reference
#pragma unroll
            for (int mm = mb; mm < 2; ++mm)
#pragma unroll
              for (int r = 0; r < 16; ++r) s[mm][nb][r] -= delta;
          }
          expo(s, mb, pop, lt);
        }
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) l_run[nb] += lt[nb];
        pv(vbuf, 2 * mb, pop);
        pv(vbuf, 2 * mb + 1, pop);
      }
    } else if constexpr (!KDIRECT) {
      if (rot) rotate_k(it + 1, std::integral_constant<int, PAR ^ 1>{}, raw);
      if (it + 2 < n_tiles) load_k(it + 2);
    }
    wait_loads();  // this thread's loads issued above have landed before the next barrier
  };

  // ---- prologue.  RoPE angles of Q: the HP = 4 heads of a workgroup share their 64
  // positions, so the (sin, cos) table of those positions is computed once, eight entries
  // per thread, into LDS (rows padded to D/2 + 2 entries), and each lane reads its 32.
  // This runs while the Q rows are in flight.
  // With fewer heads (HP = 2 or 1: 128 or 256 positions) the angle of position
  // qb*RH + 16a + b is composed from two tables of (sin, cos), one for the RH/16 positions
  // qb*RH + 16a and one for the 16 offsets b, both reduced in fp64: the entries computed
  // drop from 32 per thread to 3 or 4, for one complex product per element.
  constexpr bool kQTab = ROPE && HP == 4 && RH == 64;
  constexpr bool kQTab2 = ROPE && !kQTab;
  constexpr int kTabStride = D / 2 + 2;  // float2 entries per table row
  constexpr int kTabA = RH / 16;         // rows of the coarse table
  __shared__ __attribute__((aligned(16))) float2 qtab[kQTab ? RH * kTabStride : (kQTab2 ? (kTabA + 16) * kTabStride : 1)];
  if constexpr (kQTab || kQTab2) {
    const int64_t p0 = pos + (int64_t)qb * RH;
    constexpr int kRows = kQTab ? RH : kTabA + 16;
#pragma unroll
    for (int k = 0; k < (kRows * (D / 2) + kThreads - 1) / kThreads; ++k) {
      const int e = tid + k * kThreads, r = e / (D / 2), i = e % (D / 2);
      if (r < kRows) {
        // coarse rows: positions p0 + 16r; fine rows (after kTabA): offsets r - kTabA
        const int64_t at = kQTab ? p0 + r : (r < kTabA ? p0 + 16 * r : (int64_t)(r - kTabA));
        float sn, cs;
        sincos_rev(rope_turns(at, ropec_s[i]), &sn, &cs);
        qtab[r * kTabStride + i] = make_float2(sn, cs);
      }
    }
    // before the block copies: a barrier with direct-to-LDS loads in flight waits for them
    __syncthreads();
  }
  // Raw K of the first two blocks and V of the first in flight; the first rotated.  The
  // first block is 0, or the first one a sliding window reaches.  They are requested
  // before the Q rows are waited for, so the two latencies overlap (loads return in
  // order: the wait for Q leaves these in flight).
  if (it0 < n_tiles) {
    if constexpr (KDIRECT) {
      if (it0 & 1) load_k_direct(it0, std::integral_constant<int, 1>{});
      else load_k_direct(it0, std::integral_constant<int, 0>{});
    } else {
      load_k(it0);
    }
    load_v(it0);
    if constexpr (!KDIRECT)
      if (it0 + 1 < n_tiles) load_k(it0 + 1);
  }
  {  // Q: RoPE at its positions and the scale log2(e)/sqrt(d_h), folded into the operand
    const float qscale = kLog2e / sqrtf((float)D);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int t = wrow0 + nb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        float2 sc[4];
        if constexpr (kQTab) {
          const float4* tp = reinterpret_cast<const float4*>(qtab + (t - qb * RH) * kTabStride + ks * 8 + g * 4);
          const float4 a = tp[0], b = tp[1];
          sc[0] = make_float2(a.x, a.y);
          sc[1] = make_float2(a.z, a.w);
          sc[2] = make_float2(b.x, b.y);
          sc[3] = make_float2(b.z, b.w);
        } else if constexpr (kQTab2) {
          const int tl = t - qb * RH;
          const float4* ta = reinterpret_cast<const float4*>(qtab + (tl >> 4) * kTabStride + ks * 8 + g * 4);
          const float4* tb = reinterpret_cast<const float4*>(qtab + (kTabA + (tl & 15)) * kTabStride + ks * 8 + g * 4);
          const float4 a0 = ta[0], a1 = ta[1], b0 = tb[0], b1 = tb[1];
          const float2 ca[4] = {make_float2(a0.x, a0.y), make_float2(a0.z, a0.w), make_float2(a1.x, a1.y),
                                make_float2(a1.z, a1.w)};
          const float2 cb[4] = {make_float2(b0.x, b0.y), make_float2(b0.z, b0.w), make_float2(b1.x, b1.y),
                                make_float2(b1.z, b1.w)};
#pragma unroll
          for (int e = 0; e < 4; ++e)  // (sin, cos) of the sum of the two angles
            sc[e] = make_float2(ca[e].x * cb[e].y + ca[e].y * cb[e].x, ca[e].y * cb[e].y - ca[e].x * cb[e].x);
        }
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x0 = bf16_lo(qraw[nb][ks][e]), x1 = bf16_hi(qraw[nb][ks][e]);
          if constexpr (ROPE) {
            float sn, cs;
            sn = sc[e].x;
            cs = sc[e].y;
            const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
            x0 = y0;
            x1 = y1;
          }
          pk[e] = pack_bf16(x0 * qscale, x1 * qscale);
        }
        qop[nb][ks] = __builtin_bit_cast(bf16x8, pk);
      }
    }
  }
  // the Q operand is complete before the wait for the first blocks (its arithmetic hides
  // their latency; without a use here the compiler would sink it below the wait)
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qop[nb][ks]));
  if (it0 < n_tiles) {
    resync(it0, true);
    wait_loads();
    if constexpr (!KDIRECT) {
      u32x4 raw[C::NCH];
#pragma unroll
      for (int j = 0; j < C::NCH; ++j) raw[j] = Kraw[it0 & 1][(wid * C::NCH + j) * kWave + lane];
      if (it0 & 1) rotate_k(it0, std::integral_constant<int, 1>{}, raw);
      else rotate_k(it0, std::integral_constant<int, 0>{}, raw);
    }
  }
  int it = it0;
  if (it < n_tiles && (it & 1)) step(std::integral_constant<int, 1>{}, it++);
  for (; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // ---- epilogue (finish, above).  A wave with no key in the workgroup's last block wrote
  // its rows at the start of that block.
  if (it0 >= n_tiles || computes(n_tiles - 1)) finish();
}

namespace {
template <int D, int HP, bool ROPE, int KSRC>
hipError_t launch_one(FwdParams q, hipStream_t stream) {
  constexpr int RH = kNW * kQW / HP;
  q.n_qblocks = (q.T + RH - 1) / RH;
  q.n_groups = q.B * (q.Hq / HP);
  q.xcd_remap = work_order_mode(q.n_qblocks, q.n_groups);
  const long long grid = (long long)q.n_qblocks * q.n_groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, HP, ROPE, KSRC>), dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

template <int D, int HP>
hipError_t launch_r(const FwdParams& p, hipStream_t stream) {
  if constexpr (D == 128) {
    if (p.paged)
      return p.use_rope ? launch_one<D, HP, true, kKeysPaged>(p, stream)
                        : launch_one<D, HP, false, kKeysPaged>(p, stream);
  }
  if (p.use_rope && p.k_rot) {
    // rotate the keys once, then run the prefill on the rotated copy
    FwdParams q = p;
    const long long n_chunks = (long long)p.B * p.Hkv * p.S * (D / 8);
    if ((n_chunks + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(rope_k_kernel<D>, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, stream,
                       (const __bf16*)p.k, (__bf16*)p.k_rot, n_chunks, p.S, p);
    q.k = p.k_rot;
    return launch_one<D, HP, true, kKeysRotated>(q, stream);
  }
  return p.use_rope ? launch_one<D, HP, true, kKeysIn>(p, stream) : launch_one<D, HP, false, kKeysIn>(p, stream);
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if (G % 4 == 0) return launch_r<D, 4>(p, stream);
  if (G % 2 == 0) return launch_r<D, 2>(p, stream);
  return launch_r<D, 1>(p, stream);
}
}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d_h, hipStream_t stream) {
  if (d_h == 64) return launch_d<64>(p, stream);
  return launch_d<128>(p, stream);
}

}  // namespace attn
