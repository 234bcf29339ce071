// Paged-KV decode: one new query token per sequence against a block-tabled cache.
//
// "Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in Code"
// (Part 3) describes the cache as fixed-size blocks located through a per-sequence
// block table; "Why is attention O(n^2) ..." notes that a decode step must read the
// whole KV cache and is memory-bound.  The work is therefore cut along the key axis
// into pieces that run in parallel, each leaving an unnormalised partial (o, m, l); a
// second kernel combines the pieces of a (sequence, head) with the same rescaling the
// online softmax uses between key blocks ("Deep dive: FlashAttention" of that page).
//
// Work division.  All (sequence, KV head, cache block) triples are laid end to end
// (sequence-major, then KV head, then block) and cut into equal runs, one per wave of a
// grid sized to stay resident, so every wave streams the same number of blocks whatever
// the mix of sequence lengths.  A run that crosses the end of a (sequence, KV head)
// segment becomes several pieces; each piece writes its own partial slot.  A wave looks
// up the next piece, and loads its block-table entries and q, a few blocks before the
// current piece ends, and the first block of a piece is loaded while the last block of
// the previous one is processed, so piece boundaries do not drain the stream.
//
// A workgroup is one wave.  It streams its blocks through a private 2-stage LDS ring
// filled by direct 16-byte loads (global_load_lds_dwordx4) one block ahead, so the
// bytes in flight do not occupy registers.  Block-table entries are read 64 at a time,
// one per lane, and broadcast per block with readlane.  Per block:
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

#include <mutex>

#include "attn.h"
#include "attn_common.h"
#include "launchers.h"

namespace attn {

constexpr int kDecD = 128;        // head size served by the decode kernels
constexpr int kDecBlock = 16;     // tokens per cache block
constexpr int kStages = 2;        // LDS ring depth (blocks)
static_assert(kStages == 2, "the producer below runs exactly one block ahead");
constexpr int kStageBytes = 2 * kDecBlock * kDecD * 2;  // K and V of one block
constexpr int kDecodeLds = kStages * kStageBytes + (kDecD / 2) * 8;  // ring + RoPE table

// Element offset of the (physical block, kv head) slice of a cache [blocks, Hkv, 16, d].
__device__ __forceinline__ size_t slice_offset(int phys, int Hkv, int kvh, int d) {
  return (((size_t)phys * Hkv + kvh) * kDecBlock) * (size_t)d;
}

// 16-byte chunk position of chunk c of token row t inside a staged K block: reading
// chunk c of all 16 rows (the MFMA operand pattern) then hits 16 distinct bank groups.
__device__ __forceinline__ int kpos(int t, int c) { return t * 16 + (c ^ t); }
// Same for V under the transpose-read pattern (a half wave reads 8 rows x 2 chunks).
__device__ __forceinline__ int vpos(int t, int c) { return t * 16 + (c ^ ((2 * t) & 15)); }

// Cache blocks read for a sequence of L tokens (its table row bounds the count).
__device__ __forceinline__ int seq_blocks(int L, int max_blocks_per_seq) {
  return min((max(L, 0) + kDecBlock - 1) / kDecBlock, max_blocks_per_seq);
}

// Block counts of all sequences, scanned across the wave.  Lane l owns sequences
// l*q .. l*q+q-1 (q = ceil(num_seqs / 64)); excl is the number of blocks before them,
// nb0 / L0 the block count and length of its first sequence.
struct SeqScan {
  int excl, nb0, L0, q, total;
};
__device__ __forceinline__ SeqScan scan_seqs(const int32_t* __restrict__ seq_lens, int num_seqs,
                                             int mbps, int lane) {
  SeqScan s;
  s.q = (num_seqs + kWave - 1) / kWave;
  s.nb0 = 0;
  s.L0 = 0;
  int tot = 0;
  for (int i = 0; i < s.q; ++i) {
    const int b = lane * s.q + i;
    if (b < num_seqs) {
      const int L = seq_lens[b];
      const int nb = seq_blocks(L, mbps);
      if (i == 0) {
        s.nb0 = nb;
        s.L0 = L;
      }
      tot += nb;
    }
  }
  int inc = tot;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  s.excl = inc - tot;
  s.total = __shfl(inc, kWave - 1);
  return s;
}

// All (sequence, KV head, block) triples, laid end to end (sequence-major, then KV head,
// then block), are cut into equal runs, one per wave; both kernels derive the run
// length from the total.
__device__ __forceinline__ int run_length(int total, int nwaves) { return (total + nwaves - 1) / nwaves; }

// Lookahead, in blocks before the end of a piece, at which the next piece is looked up.
constexpr int kLookahead = 3;

// One contiguous stretch of blocks of one (sequence, KV head) segment inside one wave's
// run; its partial result goes to slot wave + segment index (distinct for distinct
// pieces, since both grow along the order).
struct Piece {
  int b, kvh, j0, n, L, slot;
};

// COPY: the same read path (work division, table windows, address, LDS ring) with the
// attention replaced by a copy of each staged K block to p.copy_dst, so that the block-table
// translation the decode performs can be compared bit for bit with a plain gather.
template <bool COPY>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char ring[];  // kDecodeLds bytes

  const int lane = threadIdx.x;
  const int grp = lane / 16;  // 16-lane group
  const int l16 = lane % 16;
  const int w = blockIdx.x;
  const int Hkv = p.Hkv;
  const int G = p.Hq / Hkv;
  const int mbps = p.max_blocks_per_seq;
  const int nwaves = (int)gridDim.x;

  // RoPE constants in LDS: each lane needs a lane-dependent subset, and indexed reads of
  // the kernel arguments would be memory loads that wait for every load in flight.
  double* rope_lds = (double*)(ring + kStages * kStageBytes);
  rope_lds[lane] = p.rope_c[lane];
  __syncthreads();

  const SeqScan sc = scan_seqs(p.seq_lens, p.num_seqs, mbps, lane);
  if (!COPY && w == 0) {  // block offsets of every sequence, for the merge kernel
    int acc = sc.excl;
    for (int i = 0; i < sc.q; ++i) {
      const int b = lane * sc.q + i;
      if (b < p.num_seqs) {
        p.seq_prefix[b] = acc;
        acc += seq_blocks(p.seq_lens[b], mbps);
      }
    }
    if (lane == 0) p.seq_prefix[p.num_seqs] = sc.total;
  }
  const int total = sc.total * Hkv;
  const int per = run_length(total, nwaves);

  // This wave's run [run_pos, run_end), taken piece by piece.
  int run_pos = w * per;
  const int run_end = min(total, run_pos + per);
  auto next_piece = [&](Piece& pc) -> bool {
    if (run_pos >= run_end) return false;
    // sequence holding run_pos: the last lane whose first block is at or before it,
    // then (more than 64 sequences) a walk over that lane's sequences
    const unsigned long long below = __ballot(sc.excl * Hkv <= run_pos && lane * sc.q < p.num_seqs);
    const int ls = 63 - __builtin_clzll(below);  // lane 0 always qualifies
    int off = __builtin_amdgcn_readlane(sc.excl, ls) * Hkv;
    int b = ls * sc.q;
    int nb = __builtin_amdgcn_readlane(sc.nb0, ls);
    int L = __builtin_amdgcn_readlane(sc.L0, ls);
    while (run_pos >= off + nb * Hkv) {  // only when q > 1 (or empty sequences)
      off += nb * Hkv;
      ++b;
      L = p.seq_lens[b];
      nb = seq_blocks(L, mbps);
    }
    const int rel = run_pos - off;
    pc.b = b;
    pc.kvh = rel / nb;
    pc.j0 = rel - pc.kvh * nb;
    pc.n = min(run_end, off + (pc.kvh + 1) * nb) - run_pos;
    pc.L = L;
    pc.slot = w + b * Hkv + pc.kvh;
    run_pos += pc.n;
    return true;
  };
  auto table_row = [&](const Piece& pc) { return p.block_table + (size_t)pc.b * mbps + pc.j0; };
  auto load_q = [&](const Piece& pc, u32x4* raw) {
    const int head = pc.kvh * G + l16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      raw[kk] = (u32x4){0u, 0u, 0u, 0u};
      if (!COPY && l16 < G)
        raw[kk] = *(const u32x4*)((const __bf16*)p.q + ((size_t)pc.b * p.Hq + head) * kDecD + grp * 8 + 32 * kk);
    }
  };
  // q^T operand: lane holds head l16, dims grp*8 + 32*kk .. +7, rotated at position
  // L-1, with the base-2 softmax scale folded in.
  const float qscale = kLog2e / sqrtf((float)kDecD);
  auto rotate_q = [&](const u32x4* raw, int L, bf16x8* qop) {
    const int64_t qposn = (int64_t)L - 1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = bf16_lo(raw[kk][e]), x1 = bf16_hi(raw[kk][e]);
        if (p.use_rope) {
          const int pair = (grp * 8 + 32 * kk) / 2 + e;
          float sn, cs;
          sincos_rev(rope_turns(qposn, rope_lds[pair]), &sn, &cs);
          const float y0 = x0 * cs - x1 * sn;
          const float y1 = x0 * sn + x1 * cs;
          x0 = y0;
          x1 = y1;
        }
        packed[e] = pack_bf16(x0 * qscale, x1 * qscale);
      }
      qop[kk] = __builtin_bit_cast(bf16x8, packed);
    }
  };

  const __bf16* kc = (const __bf16*)p.k_cache;
  const __bf16* vc = (const __bf16*)p.v_cache;
  // Direct loads of the block at physical index phys (KV head kvh) into stage st: load r
  // covers token rows 4r .. 4r+3.  Every cache byte is read once per step, so the loads
  // carry the streaming (nt) policy: measured on this part, the same paged read pattern
  // runs ~13 % faster with it than with the default policy.
  auto issue = [&](int phys, int kvh, int st) {
    phys = min(max(phys, 0), p.num_blocks - 1);  // a bad table entry never leaves the pool
    const size_t sl = slice_offset(phys, Hkv, kvh, kDecD);
    char* kdst = ring + st * kStageBytes;
    char* vdst = kdst + kStageBytes / 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * r + grp;
      load_lds16<kStreamPolicy>(kc + sl + (size_t)t * kDecD + (l16 ^ t) * 8, kdst + r * 1024);
      load_lds16<kStreamPolicy>(vc + sl + (size_t)t * kDecD + (l16 ^ ((2 * t) & 15)) * 8, vdst + r * 1024);
    }
  };

  // Three pieces are live: the consumer's (cp), the producer's (pp, one block ahead, so
  // either cp or the piece after it) and the next one (np).  np is looked up a few
  // blocks before the producer needs it, and its first table entries and q are loaded
  // then (so they do not hold registers for the whole piece).
  Piece cp, pp, np;
  if (!next_piece(cp)) return;  // uniform over the workgroup
  pp = cp;
  int tcur = (lane < pp.n) ? table_row(pp)[lane] : 0;  // producer's table window
  int tnxt = (64 + lane < pp.n) ? table_row(pp)[64 + lane] : 0;  // the following window
  u32x4 qraw[4];
  load_q(cp, qraw);
  int np_state = 0;  // 0: not looked up yet, 1: np valid, 2: no more work
  int tnp = 0;
  u32x4 qraw_np[4];
  auto fetch_np = [&]() {
    if (next_piece(np)) {
      np_state = 1;
      tnp = (lane < np.n) ? table_row(np)[lane] : 0;
      load_q(np, qraw_np);
    } else {
      np_state = 2;
    }
  };
  if (cp.n <= kLookahead) fetch_np();
  issue(__builtin_amdgcn_readlane(tcur, 0), pp.kvh, 0);
  int pi = 1;          // next block of pp to issue
  bool prod = true;    // producer still has blocks
  int gstep = 0;       // consumer block counter over all pieces (ring stage parity)

  bf16x8 qop[4];
  rotate_q(qraw, cp.L, qop);
  float m_ref = -INFINITY;  // reference max (base 2) for head l16, same in its 4 lanes
  float l = 0.f;            // this lane's partial normaliser
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int ci = 0;  // block of cp being consumed

  for (;;) {
    // producer: issue the next block (possibly the first of the next piece)
    // (at the top of a step the producer is always on the consumer's piece: it moves on
    // only while the consumer takes that piece's last block)
    if (prod && pi == pp.n) {
      if (np_state == 0) fetch_np();  // only if the piece was shorter than the lookahead
      if (np_state == 1) {
        pp = np;
        tcur = tnp;
        pi = 0;
      } else {
        prod = false;
      }
    }
    if (prod) {
      if ((pi & 63) == 0 && pi > 0) {
        // a real branch: a select would read tnxt (and wait for its load) every block
        __asm__ volatile("");
        tcur = tnxt;
      }
      issue(__builtin_amdgcn_readlane(tcur, pi & 63), pp.kvh, (gstep + 1) % kStages);
      const bool refill = (pi & 63) == 0 && pi + 64 < pp.n;
      ++pi;
      __builtin_amdgcn_s_waitcnt(0x0f78);  // vmcnt(8): the block being consumed has landed
      if (refill)  // next 64 table entries of the producer's piece
        tnxt = (pi + 63 + lane < pp.n) ? table_row(pp)[pi + 63 + lane] : 0;
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);
    }

    const int j = cp.j0 + ci;
    const int L = cp.L;
    const char* kst = ring + (gstep % kStages) * kStageBytes;
    const char* vst = kst + kStageBytes / 2;
    if constexpr (COPY) {
      // staged K: LDS chunk t * 16 + l16 holds chunk l16 ^ t of token t (issue, below kpos)
      char* dst = (char*)p.copy_dst + ((size_t)cp.b * Hkv + cp.kvh) * (size_t)mbps * kDecBlock * (kDecD * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * r + grp;
        const int tok = j * kDecBlock + t;
        const u32x4 v = *(const u32x4*)(kst + (t * 16 + l16) * 16);
        if (tok < L) *(u32x4*)(dst + (size_t)tok * (kDecD * 2) + (l16 ^ t) * 16) = v;
      }
      ++gstep;
      if (++ci < cp.n) {
        if (np_state == 0 && cp.n - ci <= kLookahead) fetch_np();
        continue;
      }
      if (np_state != 1) break;
      cp = np;
      np_state = 0;
      ci = 0;
      if (cp.n <= kLookahead) fetch_np();
      continue;
    }

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
    const u32x2 pk = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
    const s16x4 pop = __builtin_bit_cast(s16x4, pk);
    // O^T += V^T P^T, 16 dims per product.  The eight transpose reads are issued from one
    // asm block that also waits for them: the compiler cannot tell which LDS bytes a
    // ds_read_b64_tr_b16 builtin reads, so it would wait for every direct-to-LDS load in
    // flight (including the next block's) before it.
    s16x4 va[8];
    {
      const int t = 4 * grp + l16 / 4;
      const int x = (l16 % 4) / 2, half = l16 % 2;
      const uint32_t vbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)vst;
      uint32_t ad[8];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) ad[mb] = vbase + vpos(t, 2 * mb + x) * 16 + half * 8;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %9\n\t"
          "ds_read_b64_tr_b16 %2, %10\n\t"
          "ds_read_b64_tr_b16 %3, %11\n\t"
          "ds_read_b64_tr_b16 %4, %12\n\t"
          "ds_read_b64_tr_b16 %5, %13\n\t"
          "ds_read_b64_tr_b16 %6, %14\n\t"
          "ds_read_b64_tr_b16 %7, %15\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(va[0]), "=&v"(va[1]), "=&v"(va[2]), "=&v"(va[3]), "=&v"(va[4]), "=&v"(va[5]),
            "=&v"(va[6]), "=&v"(va[7])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
            "v"(ad[7]));
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      s16x4 a = va[mb];
      if (tail) {
        // masked tokens have p = 0 but their V slots may hold non-finite values
        // (0 * NaN would poison the product): this lane's 4 values come from tokens
        // 4 * grp .. 4 * grp + 3 of the block; zero the invalid ones
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j * kDecBlock + grp * 4 + r >= L) a[r] = 0;
      }
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pop, o[mb], 0, 0, 0);
    }
    ++gstep;
    if (++ci < cp.n) {
      if (np_state == 0 && cp.n - ci <= kLookahead) fetch_np();
      continue;
    }

    // End of the consumer's piece: its partial (l summed over the four token groups of
    // a head; m is shared by them).
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (l16 < G) {
      const size_t ps = (size_t)cp.slot * G + l16;
      float* po = p.part_o + ps * kDecD;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) *(f32x4*)(po + 16 * mb + 4 * grp) = o[mb];
      if (grp == 0) *(float2*)(p.part_ml + ps * 2) = make_float2(m_ref, l);
    }
    if (np_state != 1) break;
    // the producer has moved on to np (its first block is in flight): consume it next
    cp = np;
    np_state = 0;
    rotate_q(qraw_np, cp.L, qop);
    m_ref = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    ci = 0;
    if (cp.n <= kLookahead) fetch_np();
  }
}

// Log-sum-exp merge of the pieces of one (sequence, query head).
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int G = p.Hq / p.Hkv;
  const int kvh = (bh % p.Hq) / G, hh = (bh % p.Hq) % G;
  const int d = threadIdx.x;
  const int nb = seq_blocks(p.seq_lens[b], p.max_blocks_per_seq);
  const int g = b * p.Hkv + kvh;
  // waves whose runs overlap this (sequence, KV head) segment
  int w0 = 0, w1 = -1;
  if (nb > 0) {
    const int per = run_length(p.seq_prefix[p.num_seqs] * p.Hkv, p.nwaves);
    const int s0 = p.seq_prefix[b] * p.Hkv + kvh * nb;
    w0 = s0 / per;
    w1 = (s0 + nb - 1) / per;
  }
  // Eight partials per round, their loads issued together; the running max rescales
  // what was accumulated before (same recurrence as between key blocks).
  const int nparts = w1 - w0 + 1;
  float M = -INFINITY, acc = 0.f, lsum = 0.f;
  for (int i0 = 0; i0 < nparts; i0 += 8) {
    float2 ml[8];
    float ov[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ml[k] = make_float2(-INFINITY, 0.f);
      ov[k] = 0.f;
      const int i = i0 + k;
      if (i < nparts) {
        const size_t ps = (size_t)(w0 + i + g) * G + hh;
        ml[k] = *(const float2*)(p.part_ml + ps * 2);
        ov[k] = p.part_o[ps * kDecD + d];
      }
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < 8; ++k) Mb = fmaxf(Mb, ml[k].x);
    if (Mb == -INFINITY) continue;
    const float sc0 = fast_exp2(M - Mb);  // 0 while nothing was accumulated
    acc *= sc0;
    lsum *= sc0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sc = fast_exp2(ml[k].x - Mb);
      lsum += sc * ml[k].y;
      acc += sc * ov[k];
    }
    M = Mb;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  ((__bf16*)p.out)[(size_t)bh * kDecD + d] = (__bf16)(acc * inv);
  if (p.lse && d == 0) p.lse[bh] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
}

int decode_num_waves(int num_seqs, int Hkv, int max_blocks_per_seq) {
  const long long work = (long long)num_seqs * Hkv * max_blocks_per_seq;
  return (int)(work < kDecodeWaves ? work : kDecodeWaves);
}

long long decode_num_slots(int num_seqs, int Hkv, int max_blocks_per_seq) {
  return (long long)decode_num_waves(num_seqs, Hkv, max_blocks_per_seq) + (long long)num_seqs * Hkv;
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  constexpr size_t lds = kDecodeLds;
  hipLaunchKernelGGL(decode_partial_kernel<false>, dim3((unsigned)p.nwaves), dim3(64), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long grid = (long long)p.num_seqs * p.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)grid), dim3(kDecD), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_paged_gather(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_partial_kernel<true>, dim3((unsigned)p.nwaves), dim3(64), kDecodeLds, stream, p);
  return hipGetLastError();
}

// Workspace of attn_decode_paged_static, for callers that cannot allocate: the same partial
// results attn_decode_paged keeps in the caller's workspace.  Each GPU holds its own copy for
// the life of the process.  In host code `scratch` only names the symbol (the host-side
// stand-in is not a device address); the device address comes from hipGetSymbolAddress, taken
// once per GPU with that GPU current, and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = addr;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace attn
