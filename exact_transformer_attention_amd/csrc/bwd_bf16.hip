// bf16 exact attention backward on gfx950 matrix cores (fp32 accumulation).
//
// The backward pass recomputes the probabilities from the saved log-sum-exp instead of
// reading a stored T x S matrix ("Why is attention O(n^2), how does FlashAttention
// help ...", Deep dive: FlashAttention; "Self-Attention Complexity, FlashAttention,
// PagedAttention, and RoPE in Code", Part 2).  With q', k' the rotated inputs,
// S = q' k'^T / sqrt(d_h), P = softmax(S), O = P v and dO the incoming gradient:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dO * O)),
//     dq' = dS k' / sqrt(d_h),   dk' = dS^T q' / sqrt(d_h),
// and RoPE being a rotation, dq and dk are dq', dk' rotated back by the same angles.
//
// Three kernels, all on the caller's stream:
//  * preprocess: per query row, delta = rowsum(dO * O) and lse in base 2 (a row with no
//    visible key gets +inf, so its probabilities recompute to 0); with RoPE, q and k are
//    rotated once (angles reduced in fp64) into the workspace as bf16, so the two gradient
//    kernels stream plain tiles.
//  * dK/dV: a workgroup owns 128 keys of one KV head (four waves of 32).  It walks every
//    query block of every query head that reads this KV head (grouped-query sums stay in
//    registers; no atomics), streaming q' and dO tiles through LDS.  In the orientation
//    S = q' k'^T a lane owns one key column, so P and dS leave the accumulators directly
//    as the B operands of dV^T += dO^T P and dk'^T += q'^T dS (the contraction over queries
//    is permuted to match the accumulator rows), and dO^T, q'^T are read with
//    ds_read_b64_tr_b16.  The wave's own k' and V columns stay in registers.
//  * dQ: shaped like the forward kernel.  Eight waves of 32 queries (the query heads of one
//    KV head packed together) stream k' and V tiles; S^T = k' q'^T and dP^T = V dO^T put a
//    query in each lane, and dq'^T += k'^T dS^T takes dS^T straight from the accumulators.
// Probabilities and dS are rounded to bf16 for the products; everything else is fp32.
// Tiles are stored with an xor swizzle of their 16-byte chunks that keeps both the row
// reads (ds_read_b128) and the transposed reads free of bank conflicts.
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "fwd_params.h"
#include "launchers.h"

namespace attn {

namespace {

constexpr int kD = 128;
constexpr int kCPR = kD / 8;   // 16-byte chunks per row
constexpr int kKS = kD / 16;   // k-steps over the head dimension
constexpr int kDB = kD / 32;   // 32-wide blocks of the head dimension
constexpr int kRowBytes = kD * 2;
constexpr int kTileRows = 64;  // rows of a streamed tile (queries in dK/dV, keys in dQ)
constexpr int kTileChunks = kTileRows * kCPR;

constexpr int kKVW = 4;                 // dK/dV: waves per workgroup
constexpr int kKVThreads = kKVW * kWave;
constexpr int kKeysPerWG = kKVW * 32;
constexpr int kQW = 8;                  // dQ: waves per workgroup (two per SIMD)
constexpr int kQThreads = kQW * kWave;

// Chunk swizzle of tile row r (a 4-bit xor on the chunk index).  With a = r & 3 and
// b = (r >> 2) & 3: bits 2-3 are a permutation of a and so are bits 1-2, so the four rows a
// transposed read touches land in distinct 32- and 64-byte bank groups; over 16
// consecutive rows the value is a permutation of 0..15, so 8 or 16 lanes reading the same
// logical chunk of consecutive rows hit distinct banks.
__device__ __forceinline__ int bswz(int r) {
  const int a = r & 3, b = (r >> 2) & 3;
  return (b & 1) | ((((a >> 1) ^ (b >> 1)) & 1) << 1) | ((a & 1) << 2) | ((a >> 1) << 3);
}

// Byte offset of logical chunk c of row r in a swizzled tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowBytes + ((c ^ bswz(r)) << 4); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Transposed A operand: lane l gets column (l % 32) of the 32-column block for the 16 rows
// of one k-step, in the accumulator row order (rows 4g..4g+3 from the first address, rows
// 8+4g..8+4g+3 from the second).
__device__ __forceinline__ bf16x8 tr_read(const char* p0, const char* p1) {
  const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
  const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
  return __builtin_bit_cast(bf16x8, (u32x4){w0[0], w0[1], w1[0], w1[1]});
}

// Per-lane offsets of the transposed reads of 32-column block db, rows 0..15 of a tile.
__device__ __forceinline__ void tr_offsets(int lane, int (&t0)[kDB], int (&t1)[kDB]) {
  const int g = lane / 32, a16 = lane / 16, lam = lane % 16;
  const int r0 = 4 * g + lam / 4;
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    const int col = db * 32 + 16 * (a16 % 2) + 4 * (lam % 4);
    const int c = col / 8, half = (col % 8) / 4;
    t0[db] = tile_off(r0, c) + half * 8;
    t1[db] = tile_off(r0 + 8, c) + half * 8;
  }
}

// x as three bf16 pieces hi + mid + lo (each the rounding of what is left), packed as
// {hi, mid} and {lo, 0}: a matrix product against 1.0 in three k-slots adds x back with
// fp32 accuracy.  -inf gives {-inf, 0, 0}.
__device__ __forceinline__ u32x2 split3(float x) {
  u32x2 r;
  if (x == -INFINITY) {
    r[0] = pack_bf16(x, 0.f);
    r[1] = 0u;
    return r;
  }
  const float hi = bf16_lo(pack_bf16(x, 0.f));
  const float mid = bf16_lo(pack_bf16(x - hi, 0.f));
  const float lo = (x - hi) - mid;
  r[0] = pack_bf16(hi, mid);
  r[1] = pack_bf16(lo, 0.f);
  return r;
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Rotate pair (x0, x1) back by the RoPE angle of `turns` (the transpose of the rotation).
__device__ __forceinline__ void unrotate(float& x0, float& x1, float turns) {
  float sn, cs;
  sincos_rev(turns, &sn, &cs);
  const float y0 = x0 * cs + x1 * sn, y1 = x1 * cs - x0 * sn;
  x0 = y0;
  x1 = y1;
}

}  // namespace

// ---------------------------------------------------------------- preprocess ----
// Rows [0, nq) are query rows (b, h, t): the row record (-lse in base 2 and
// -rowsum(dO * O), each split into bf16 pieces) and q rotated (RoPE) and scaled by
// log2(e) / sqrt(d_h), so that q_s k'^T are base-2 logits.  Rows [nq, nq + nk) are key rows
// (b, kvh, s) to rotate (RoPE only).  16 lanes per row, 8 elements (4 pairs) per lane.
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, long long nq, long long nk) {
  const int sub = threadIdx.x % 16;
  const long long nrows = nq + nk;
  const long long stride = (long long)gridDim.x * 16;
  const float cq = kLog2e / sqrtf((float)kD);
  for (long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / 16; row < nrows; row += stride) {
    if (row < nq) {
      const size_t e0 = (size_t)row * kD + sub * 8;
      const int64_t ps = p.pos + (int64_t)(row % p.T);
      const u32x4 raw = *(const u32x4*)((const __bf16*)p.q + e0);
      u32x4 outv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
        if (p.use_rope) {
          float sn, cs;
          sincos_rev(rope_turns(ps, p.rope_c[sub * 4 + e]), &sn, &cs);
          const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
          x0 = y0;
          x1 = y1;
        }
        outv[e] = pack_bf16(x0 * cq, x1 * cq);
      }
      *(u32x4*)((__bf16*)p.qr + e0) = outv;
      const u32x4 d = *(const u32x4*)((const __bf16*)p.dout + e0);
      const u32x4 o = *(const u32x4*)((const __bf16*)p.out + e0);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += bf16_lo(d[e]) * bf16_lo(o[e]) + bf16_hi(d[e]) * bf16_hi(o[e]);
      acc += __shfl_xor(acc, 8);
      acc += __shfl_xor(acc, 4);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 1);
      if (sub == 0) {
        const float l = p.lse[row];
        const u32x2 nl = split3(l == -INFINITY ? -INFINITY : -l * kLog2e);
        const u32x2 nd = split3(-acc);
        *(u32x4*)((char*)p.rec + (size_t)row * 16) = (u32x4){nl[0], nl[1], nd[0], nd[1]};
      }
    } else {
      const long long kr = row - nq;
      const int64_t ps = kr % p.S;
      const size_t e0 = (size_t)kr * kD + sub * 8;
      const u32x4 raw = *(const u32x4*)((const __bf16*)p.k + e0);
      u32x4 outv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        sincos_rev(rope_turns(ps, p.rope_c[sub * 4 + e]), &sn, &cs);
        const float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
        outv[e] = pack_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
      }
      *(u32x4*)((__bf16*)p.kr + e0) = outv;
    }
  }
}

// ---------------------------------------------------------------------- dK/dV ----
__global__ __launch_bounds__(kKVThreads) void bwd_dkdv_kernel(BwdParams p) {
  // Double-buffered q_s and dO tiles (swizzled) and row records; one array per buffer (see
  // the dQ kernel).
  __shared__ __attribute__((aligned(16))) u32x4 Qs0[kTileChunks], Qs1[kTileChunks];
  __shared__ __attribute__((aligned(16))) u32x4 Os0[kTileChunks], Os1[kTileChunks];
  __shared__ __attribute__((aligned(16))) u32x4 Rs0[kTileRows], Rs1[kTileRows];

  const int tid = threadIdx.x;
  const int wid = tid / kWave;
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int g = lane / 32;

  // ---- work item: (batch, KV head, 128-key block).  Key blocks run in increasing order
  // (for causal attention the first blocks see the most queries); all blocks of one KV
  // head stay on one XCD so its q' / dO tiles are shared through that XCD's L2
  // (work_order).
  int kb, grp;
  {
    work_order(blockIdx.x, p.n_kblocks, p.n_groups, p.xcd_remap, kb, grp);
  }
  const int b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int T = p.T, S = p.S;
  const int64_t pos = p.pos;
  const int kb0 = kb * kKeysPerWG;
  const int kw0 = kb0 + wid * 32;  // first key of this wave
  const int key = kw0 + l32;       // this lane's key column

  const size_t kvrow0 = ((size_t)b * p.Hkv + kvh) * (size_t)S;
  const __bf16* kg = (const __bf16*)(p.use_rope ? p.kr : p.k) + kvrow0 * kD;
  const __bf16* vg = (const __bf16*)p.v + kvrow0 * kD;
  const __bf16* qbase = (const __bf16*)p.qr;
  const __bf16* obase = (const __bf16*)p.dout;

  // k'^T and V^T as B operands: lane holds key `key`, dims ks*16 + g*8 .. +7.
  bf16x8 kop[kKS], vop[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
    if (key < S) {
      kr = *(const u32x4*)(kg + (size_t)key * kD + ks * 16 + g * 8);
      vr = *(const u32x4*)(vg + (size_t)key * kD + ks * 16 + g * 8);
    }
    kop[ks] = __builtin_bit_cast(bf16x8, kr);
    vop[ks] = __builtin_bit_cast(bf16x8, vr);
  }

  // ---- queries that see at least one key of this block.
  int64_t qlo = 0, qhi = T;
  if (p.causal) qlo = (int64_t)kb0 - pos;  // key kb0 is visible from query kb0 - pos on
  if (p.window > 0) {
    const int64_t klast = (int64_t)min(kb0 + kKeysPerWG, S) - 1;
    qhi = klast + p.window - pos;  // key klast is visible to queries below this
  }
  qlo = qlo < 0 ? 0 : (qlo > T ? T : qlo);
  qhi = qhi > T ? T : qhi;
  const int qb_lo = (int)(qlo / kTileRows);
  const int nqb = qhi > qlo ? (int)((qhi + kTileRows - 1) / kTileRows) - qb_lo : 0;
  const int n_it = G * nqb;
  // Iteration it reads query tile qb_top - it / G of head it % G: every workgroup walks the
  // tiles from the top down with the heads innermost, so the workgroups of one KV head
  // that run together read the same tile at about the same time (shared in L2).
  const int qb_top = qb_lo + nqb - 1;

  // ---- tile loads: this thread's chunks of rows row0 + 4j (direct to LDS, swizzled).
  const int slot = lane % kCPR;
  const int row0 = wid * 16 + lane / kCPR;
  int goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = row0 + 4 * j;
    goff[j] = (r * kD + (slot ^ bswz(r)) * 8) * 2;
  }
  auto load_tile = [&](int it, auto bc) {
    constexpr int BUF = decltype(bc)::value;
    const int hh = it % G, qb = qb_top - it / G;
    const int q0 = qb * kTileRows;
    const size_t rowbase = ((size_t)b * p.Hq + (size_t)kvh * G + hh) * (size_t)T + q0;
    const uint32_t nrows = (uint32_t)min(T - q0, kTileRows);
    const i32x4 rq = make_rsrc(qbase + rowbase * kD, nrows * kRowBytes);
    const i32x4 ro = make_rsrc(obase + rowbase * kD, nrows * kRowBytes);
    u32x4* qd = BUF ? Qs1 : Qs0;
    u32x4* od = BUF ? Os1 : Os0;
#pragma unroll
    for (int j = 0; j < 4; ++j) buffer_load_lds16(rq, goff[j], qd + (wid * 4 + j) * kWave);
#pragma unroll
    for (int j = 0; j < 4; ++j) buffer_load_lds16(ro, goff[j], od + (wid * 4 + j) * kWave);
    if (wid == 0) buffer_load_lds16(make_rsrc((const char*)p.rec + rowbase * 16, nrows * 16), lane * 16, BUF ? Rs1 : Rs0);
  };

  int noff[kKS];  // row reads: row l32, chunk ks*2 + g
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) noff[ks] = tile_off(l32, ks * 2 + g);
  int toff0[kDB], toff1[kDB];
  tr_offsets(lane, toff0, toff1);

  f32x16 dv[kDB], dk[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dv[db] = zero16();
    dk[db] = zero16();
  }
  // 1.0 in k-slots 0-2 of the extra k-step that adds a row record's pieces (lanes g = 0)
  const bf16x8 ones3 = __builtin_bit_cast(bf16x8, (u32x4){g == 0 ? 0x3f803f80u : 0u, g == 0 ? 0x3f80u : 0u, 0u, 0u});

  // One 64-query tile against this wave's 32 keys, in four phases that keep the matrix
  // cores busy while the vector unit works (one wave per SIMD, so the overlap has to come
  // from the instruction order within the wave):
  //   A: S0 = q'0 k'^T, dP0 = dO0 V^T (sub-tile 0, queries 0-31)
  //   B: S1, dP1 for sub-tile 1, with P0 = exp2(S0 c - lse2) and dS0 woven in
  //   C: dV^T += dO0^T P0, dk'^T += q'0^T dS0, with P1, dS1 woven in
  //   D: dV^T += dO1^T P1, dk'^T += q'1^T dS1
  // Each phase's LDS operands are read one phase ahead.  A scheduling barrier after each
  // pair of products keeps the interleave.  MASK tiles straddle the causal diagonal or the
  // window edge: there hidden probabilities are set to 0 (32-bit offsets from the key).
  auto compute = [&](int it, auto bc, auto mc) {
    constexpr int BUF = decltype(bc)::value;
    constexpr bool MASK = decltype(mc)::value;
    const int q0 = (qb_top - it / G) * kTileRows;
    const char* qt = (const char*)(BUF ? Qs1 : Qs0);
    const char* ot = (const char*)(BUF ? Os1 : Os0);
    const u32x4* rt = BUF ? Rs1 : Rs0;
    // rel(r, mi) = key - (pos + query) = relb - (mi*32 + (r/4)*8 + r%4); visible iff
    // rel <= 0 and rel > -wlim
    int relb = 0, wlim = 0x7fffffff;
    if constexpr (MASK) {
      int64_t r64 = (int64_t)key - g * 4 - pos - q0;
      r64 = r64 > (1 << 30) ? (1 << 30) : (r64 < -(1 << 30) ? -(1 << 30) : r64);
      relb = (int)r64;
      if (p.window > 0) wlim = (int)(p.window < (1 << 30) ? p.window : (1 << 30));
    }
    auto rowrd = [&](const char* t, int mi, int ks) {
      return *(const bf16x8*)(t + noff[ks] + mi * 32 * kRowBytes);
    };
    auto trrd = [&](const char* t, int mi, int h, int db) {
      const int rb = (mi * 2 + h) * 16 * kRowBytes;
      return tr_read(t + rb + toff0[db], t + rb + toff1[db]);
    };
    // p and dS of element r of a sub-tile, in place (s <- p, dp <- dS); the products
    // already hold s - lse2 and dP - rowsum(dO * O)
    auto elem = [&](f32x16& s, f32x16& dp, int mi, int r) {
      float pv = fast_exp2(s[r]);
      if constexpr (MASK) {
        const int rel = relb - (mi * 32 + (r / 4) * 8 + (r % 4));
        pv = (rel <= 0 && rel > -wlim) ? pv : 0.f;
      }
      s[r] = pv;
      dp[r] = pv * dp[r];
    };
    // the row records of sub-tile mi as the A operands of the extra k-step
    auto bias = [&](int mi, bf16x8& bl, bf16x8& bd) {
      const u32x4 r = rt[mi * 32 + l32];
      const uint32_t m = g == 0 ? 0xffffffffu : 0u;
      bl = __builtin_bit_cast(bf16x8, (u32x4){r[0] & m, r[1] & m, 0u, 0u});
      bd = __builtin_bit_cast(bf16x8, (u32x4){r[2] & m, r[3] & m, 0u, 0u});
    };
    auto pack = [&](const f32x16& x, int h) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
      return __builtin_bit_cast(bf16x8, w);
    };

    bf16x8 a0[kKS], b0[kKS], a1[kKS], b1[kKS];
    bf16x8 to0[2][kDB], tq0[2][kDB], to1[2][kDB], tq1[2][kDB];
    bf16x8 bl0, bd0, bl1, bd1;
    bias(0, bl0, bd0);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      a0[ks] = rowrd(qt, 0, ks);
      b0[ks] = rowrd(ot, 0, ks);
    }
    bias(1, bl1, bd1);
    __builtin_amdgcn_sched_barrier(0);
    // ---- A (reads sub-tile 1's rows as sub-tile 0's are consumed)
    f32x16 s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl0, ones3, zero16(), 0, 0, 0);
    f32x16 d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bd0, ones3, zero16(), 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks], kop[ks], s0, 0, 0, 0);
      d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[ks], vop[ks], d0, 0, 0, 0);
      a1[ks] = rowrd(qt, 1, ks);
      b1[ks] = rowrd(ot, 1, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- B (reads sub-tile 0's transposed operands)
    f32x16 s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl1, ones3, zero16(), 0, 0, 0);
    f32x16 d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bd1, ones3, zero16(), 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[ks], kop[ks], s1, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[ks], vop[ks], d1, 0, 0, 0);
      elem(s0, d0, 0, 2 * ks);
      elem(s0, d0, 0, 2 * ks + 1);
      to0[ks / kDB][ks % kDB] = trrd(ot, 0, ks / kDB, ks % kDB);
      tq0[ks / kDB][ks % kDB] = trrd(qt, 0, ks / kDB, ks % kDB);
      __builtin_amdgcn_sched_barrier(0);
    }
    const bf16x8 pb0[2] = {pack(s0, 0), pack(s0, 1)};
    const bf16x8 ds0[2] = {pack(d0, 0), pack(d0, 1)};
    // ---- C (reads sub-tile 1's transposed operands)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to0[h][db], pb0[h], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq0[h][db], ds0[h], dk[db], 0, 0, 0);
        elem(s1, d1, 1, 2 * (h * kDB + db));
        elem(s1, d1, 1, 2 * (h * kDB + db) + 1);
        to1[h][db] = trrd(ot, 1, h, db);
        tq1[h][db] = trrd(qt, 1, h, db);
        __builtin_amdgcn_sched_barrier(0);
      }
    const bf16x8 pb1[2] = {pack(s1, 0), pack(s1, 1)};
    const bf16x8 ds1[2] = {pack(d1, 0), pack(d1, 1)};
    // ---- D
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to1[h][db], pb1[h], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq1[h][db], ds1[h], dk[db], 0, 0, 0);
      }
  };

  // Tile it lives in buffer it & 1 (a compile-time constant in each step, so the compiler
  // can tell the buffer being filled from the one being read).
  auto step = [&](auto bc, int it) {
    constexpr int BUF = decltype(bc)::value;
    __syncthreads();  // tile it has landed; everyone is done with tile it-1
    if (it + 1 < n_it) load_tile(it + 1, std::integral_constant<int, BUF ^ 1>{});
    // which of this wave's (query, key) pairs in the tile are visible
    const int64_t q0 = (int64_t)(qb_top - it / G) * kTileRows;
    bool any = kw0 < S, all = true;
    if (p.causal) {
      any = any && (int64_t)kw0 <= pos + q0 + kTileRows - 1;
      all = (int64_t)(kw0 + 31) <= pos + q0;
    }
    if (p.window > 0) {
      any = any && (int64_t)(kw0 + 31) > pos + q0 - p.window;
      all = all && (int64_t)kw0 > pos + q0 + kTileRows - 1 - p.window;
    }
    if (any) {
      if (all) compute(it, bc, std::false_type{});
      else compute(it, bc, std::true_type{});
    }
    wait_loads();
  };
  if (n_it > 0) {
    load_tile(0, std::integral_constant<int, 0>{});
    wait_loads();
  }
  for (int it = 0; it < n_it; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_it) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // ---- epilogue: dV, and dk = R^T dk' with dk' = dS^T q' / sqrt(d_h) = ln(2) dS^T q_s
  // (pairs are in-lane).
  if (key < S) {
    __bf16* dvg = (__bf16*)p.dv + (kvrow0 + key) * kD;
    __bf16* dkg = (__bf16*)p.dk + (kvrow0 + key) * kD;
    const float isd = kLn2;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      u32x2 wv[4], wk[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + q4 * 8 + g * 4;
        wv[q4][0] = pack_bf16(dv[db][4 * q4 + 0], dv[db][4 * q4 + 1]);
        wv[q4][1] = pack_bf16(dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dk[db][4 * q4 + e] * isd;
        if (p.use_rope) {
          unrotate(x[0], x[1], rope_turns((int64_t)key, p.rope_c[d0 / 2]));
          unrotate(x[2], x[3], rope_turns((int64_t)key, p.rope_c[d0 / 2 + 1]));
        }
        wk[q4][0] = pack_bf16(x[0], x[1]);
        wk[q4][1] = pack_bf16(x[2], x[3]);
      }
      store_block_bf16(dvg + db * 32, wv, g);  // 16-byte pieces
      store_block_bf16(dkg + db * 32, wk, g);
    }
  }
}

// ------------------------------------------------------------------------- dQ ----
template <int HP>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(kQW / 4, kQW / 4)))
void bwd_dq_kernel(BwdParams p) {
  // Double-buffered k' and V tiles (swizzled).  Each buffer is its own array so that the
  // compiler can tell the tile being read from the one whose direct-to-LDS loads are in
  // flight (it does not separate two halves of one array) and need not wait for them.
  __shared__ __attribute__((aligned(16))) u32x4 Ks0[kTileChunks], Ks1[kTileChunks];
  __shared__ __attribute__((aligned(16))) u32x4 Vs0[kTileChunks], Vs1[kTileChunks];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar values and branches
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int g = lane / 32;

  // ---- work item: (batch, head group, query block), longest causal blocks first, all
  // blocks of one head group on one XCD (work_order).
  constexpr int RH = kQW * 32 / HP;  // rows per head per workgroup
  int qb, grp;
  {
    const int bid = blockIdx.x;
    int rank;
    work_order(bid, p.n_qblocks, p.n_groups, p.xcd_remap, rank, grp);
    qb = p.n_qblocks - 1 - rank;
  }
  const int hpg = p.Hq / HP;
  const int b = grp / hpg;
  const int hq = (grp % hpg) * HP + wid / (kQW / HP);
  const int kvh = ((grp % hpg) * HP) / (p.Hq / p.Hkv);
  const int T = p.T, S = p.S;
  const int64_t pos = p.pos;
  const int wrow0 = qb * RH + (wid % (kQW / HP)) * 32;  // first query row of this wave
  const int t = wrow0 + l32;                            // this lane's query

  const size_t row = ((size_t)b * p.Hq + hq) * (size_t)T + t;
  const __bf16* qg = (const __bf16*)p.qr;
  const __bf16* og = (const __bf16*)p.dout;
  const size_t kvrow0 = ((size_t)b * p.Hkv + kvh) * (size_t)S;
  const __bf16* kg = (const __bf16*)(p.use_rope ? p.kr : p.k) + kvrow0 * kD;
  const __bf16* vg = (const __bf16*)p.v + kvrow0 * kD;

  // q_s^T and dO^T as B operands: lane holds query t, dims ks*16 + g*8 .. +7.
  bf16x8 qop[kKS], dop[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    u32x4 qr = {0u, 0u, 0u, 0u}, orw = {0u, 0u, 0u, 0u};
    if (t < T) {
      qr = *(const u32x4*)(qg + row * kD + ks * 16 + g * 8);
      orw = *(const u32x4*)(og + row * kD + ks * 16 + g * 8);
    }
    qop[ks] = __builtin_bit_cast(bf16x8, qr);
    dop[ks] = __builtin_bit_cast(bf16x8, orw);
  }
  // The row record as the B operands of the extra k-step (rows past T: -inf, so their
  // probabilities are 0); the K / V side holds 1.0 in the matching k-slots.
  bf16x8 bl, bd;
  {
    u32x4 r = {0xff80u, 0u, 0u, 0u};
    if (t < T) r = *(const u32x4*)((const char*)p.rec + row * 16);
    const uint32_t m = g == 0 ? 0xffffffffu : 0u;
    bl = __builtin_bit_cast(bf16x8, (u32x4){r[0] & m, r[1] & m, 0u, 0u});
    bd = __builtin_bit_cast(bf16x8, (u32x4){r[2] & m, r[3] & m, 0u, 0u});
  }
  const bf16x8 ones3 = __builtin_bit_cast(bf16x8, (u32x4){g == 0 ? 0x3f803f80u : 0u, g == 0 ? 0x3f80u : 0u, 0u, 0u});

  // ---- keys visible to this wave / to the workgroup (as in the forward kernel).
  int nk_wave = S, nk_wg = S;
  if (p.causal) {
    const int64_t lw = pos + (int64_t)min(T - 1, wrow0 + 31) + 1;
    nk_wave = (int)(lw < 0 ? 0 : (lw < S ? lw : S));
    const int64_t lg = pos + (int64_t)min(T - 1, qb * RH + RH - 1) + 1;
    nk_wg = (int)(lg < 0 ? 0 : (lg < S ? lg : S));
  }
  const int n_tiles = (nk_wg + kTileRows - 1) / kTileRows;
  int64_t lo_wave = 0;
  int it0 = 0;
  if (p.window > 0) {
    lo_wave = pos + wrow0 - p.window + 1;
    const int64_t lo_wg = pos + (int64_t)qb * RH - p.window + 1;
    it0 = (int)(lo_wg <= 0 ? 0 : (lo_wg < nk_wg ? lo_wg : nk_wg)) / kTileRows;
  }

  // ---- tile loads: 2 chunks per thread per tensor, rows row0 + 4j.
  const int slot = lane % kCPR;
  const int row0 = wid * 8 + lane / kCPR;
  int goff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = row0 + 4 * j;
    goff[j] = (r * kD + (slot ^ bswz(r)) * 8) * 2;
  }
  auto load_tile = [&](int tile, auto bc) {
    constexpr int BUF = decltype(bc)::value;
    const int k0 = tile * kTileRows;
    const uint32_t nrows = (uint32_t)min(S - k0, kTileRows);
    const i32x4 rk = make_rsrc(kg + (size_t)k0 * kD, nrows * kRowBytes);
    const i32x4 rv = make_rsrc(vg + (size_t)k0 * kD, nrows * kRowBytes);
    u32x4* kd = BUF ? Ks1 : Ks0;
    u32x4* vd = BUF ? Vs1 : Vs0;
#pragma unroll
    for (int j = 0; j < 2; ++j) buffer_load_lds16(rk, goff[j], kd + (wid * 2 + j) * kWave);
#pragma unroll
    for (int j = 0; j < 2; ++j) buffer_load_lds16(rv, goff[j], vd + (wid * 2 + j) * kWave);
  };

  int noff[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) noff[ks] = tile_off(l32, ks * 2 + g);
  int toff0[kDB], toff1[kDB];
  tr_offsets(lane, toff0, toff1);

  f32x16 dq[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dq[db] = zero16();

  auto compute = [&](int tile, auto bc) {
    constexpr int BUF = decltype(bc)::value;
    const int k0 = tile * kTileRows;
    if (!(k0 < nk_wave && (int64_t)(k0 + kTileRows) > lo_wave)) return;
    const char* kt = (const char*)(BUF ? Ks1 : Ks0);
    const char* vt = (const char*)(BUF ? Vs1 : Vs0);
    const bool need_mask = (k0 + kTileRows > S) || (p.causal && (int64_t)(k0 + kTileRows - 1) > pos + wrow0) ||
                           (p.window > 0 && (int64_t)k0 < lo_wave + 31);
    const int64_t lim = pos + t;  // last key this lane's query sees
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      bf16x8 dsb[2];
      f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones3, bl, zero16(), 0, 0, 0);
      f32x16 dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones3, bd, zero16(), 0, 0, 0);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 ak = *(const bf16x8*)(kt + noff[ks] + mb * 32 * kRowBytes);
        const bf16x8 av = *(const bf16x8*)(vt + noff[ks] + mb * 32 * kRowBytes);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qop[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dop[ks], dp, 0, 0, 0);
      }
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(s[r]);
      if (need_mask) {
        // element r holds key k0 + mb*32 + g*4 + c, c = (r/4)*8 + r%4: visible iff
        // lo <= c <= hi, this query's first and last visible keys relative to
        // k0 + mb*32 + g*4, clamped to 32 bits (opaque to the compiler, which would otherwise
        // compare every element against the 64-bit bounds)
        const int64_t base = (int64_t)k0 + mb * 32 + g * 4;
        int64_t hi = (int64_t)S - 1 - base;
        if (p.causal && lim - base < hi) hi = lim - base;
        const int64_t lo = p.window > 0 ? lim - p.window + 1 - base : 0;
        int hi32 = (int)(hi < -1 ? -1 : (hi > 32 ? 32 : hi));
        int lo32 = (int)(lo < 0 ? 0 : (lo > 32 ? 32 : lo));
        asm volatile("" : "+v"(hi32), "+v"(lo32));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = (r / 4) * 8 + (r % 4);
          pr[r] = ((c <= hi32) & (c >= lo32)) ? pr[r] : 0.f;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * h + 2 * e;
          pk[e] = pack_bf16(pr[r] * dp[r], pr[r + 1] * dp[r + 1]);
        }
        dsb[h] = __builtin_bit_cast(bf16x8, pk);
      }
      // dq'^T += k'^T dS^T over this half's two 16-key steps
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rb = (mb * 2 + h) * 16 * kRowBytes;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const bf16x8 ak = tr_read(kt + rb + toff0[db], kt + rb + toff1[db]);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, dsb[h], dq[db], 0, 0, 0);
        }
      }
    }
  };

  auto step = [&](auto bc, int tile) {
    constexpr int BUF = decltype(bc)::value;
    __syncthreads();
    if (tile + 1 < n_tiles) load_tile(tile + 1, std::integral_constant<int, BUF ^ 1>{});
    compute(tile, bc);
    wait_loads();
  };
  if (it0 < n_tiles) {
    if (it0 & 1) load_tile(it0, std::integral_constant<int, 1>{});
    else load_tile(it0, std::integral_constant<int, 0>{});
    wait_loads();
  }
  int it = it0;
  if (it < n_tiles && (it & 1)) step(std::integral_constant<int, 1>{}, it++);
  for (; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // ---- epilogue: dq = R^T dq' with dq' = dq'^T / sqrt(d_h).
  if (t < T) {
    __bf16* dqg = (__bf16*)p.dq + row * kD;
    const float isd = 1.f / sqrtf((float)kD);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      u32x2 w[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + q4 * 8 + g * 4;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dq[db][4 * q4 + e] * isd;
        if (p.use_rope) {
          unrotate(x[0], x[1], rope_turns(pos + t, p.rope_c[d0 / 2]));
          unrotate(x[2], x[3], rope_turns(pos + t, p.rope_c[d0 / 2 + 1]));
        }
        w[q4][0] = pack_bf16(x[0], x[1]);
        w[q4][1] = pack_bf16(x[2], x[3]);
      }
      store_block_bf16(dqg + db * 32, w, g);  // 16-byte pieces
    }
  }
}

namespace {
template <int HP>
hipError_t launch_dq(BwdParams p, hipStream_t stream) {
  constexpr int RH = kQW * 32 / HP;
  p.n_qblocks = (p.T + RH - 1) / RH;
  p.n_groups = p.B * (p.Hq / HP);
  p.xcd_remap = work_order_mode(p.n_qblocks, p.n_groups);
  const long long grid = (long long)p.n_qblocks * p.n_groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_dq_kernel<HP>), dim3((unsigned)grid), dim3(kQThreads), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_bwd_bf16(BwdParams p, hipStream_t stream) {
  const long long nq = (long long)p.B * p.Hq * p.T;
  const long long nk = p.use_rope ? (long long)p.B * p.Hkv * p.S : 0;
  long long grid = (nq + nk + 15) / 16;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p, nq, nk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdParams kv = p;
  kv.n_kblocks = (p.S + kKeysPerWG - 1) / kKeysPerWG;
  kv.n_groups = p.B * p.Hkv;
  kv.xcd_remap = work_order_mode(kv.n_kblocks, kv.n_groups);
  grid = (long long)kv.n_kblocks * kv.n_groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)grid), dim3(kKVThreads), 0, stream, kv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int G = p.Hq / p.Hkv;
  if (G % 4 == 0) return launch_dq<4>(p, stream);
  if (G % 2 == 0) return launch_dq<2>(p, stream);
  return launch_dq<1>(p, stream);
}

}  // namespace attn
