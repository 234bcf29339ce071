// fp8 (E4M3) exact attention prefill on gfx950 matrix cores, fp32 accumulation, bf16 output.
//
// The same blocked online softmax as the bf16 kernel ("Why is attention O(n^2), how does
// FlashAttention help ...", Deep dive: FlashAttention), with both products on the fp8
// matrix cores (v_mfma_f32_32x32x64_f8f6f4, twice the bf16 rate), which the same page names
// as what later FlashAttention versions exploit on newer hardware.
//
// Inputs are E4M3 codes with one fp32 scale per tensor (value = code * scale); q and k are
// taken as already rotated (no RoPE here), and V is given transposed, [B, Hkv, d_h, S], so
// that the P V product, which contracts over keys, reads V along its rows.
//
// Mapping onto CDNA4 (wave64, 8 waves per workgroup, two per SIMD):
//  * a wave owns 32 query rows of one head; the heads sharing a KV head are packed into one
//    workgroup (HP heads), so each 64-key K / V block in LDS serves 256 query rows;
//  * S^T = K Q^T: two 32-key halves x two 64-dim k-steps = 4 MFMAs per block; a lane owns one
//    query column, the row scale q_scale * k_scale * log2(e) / sqrt(d_h) is applied to the
//    accumulators and p = exp2(s - m) with a lazily raised reference m (as in the bf16
//    kernel, but kept low enough that every p <= 256 fits E4M3, whose largest value is 448);
//  * O^T = V^T P^T: the 64 probabilities a lane holds (16 per half, its two lane halves
//    together covering the block) are rounded to E4M3 and are exactly one B operand of a
//    64-key k-step; the V^T tile is stored with its keys in that order, so the A operand is
//    two 16-byte reads: 4 MFMAs per block;
//  * K and V^T move HBM -> LDS with direct loads (16-byte chunks for K, 4-byte groups of 4
//    keys for V^T, which performs the reordering), double-buffered one block ahead; both
//    tiles are xor-swizzled by 16-byte chunk so the operand reads hit distinct banks.
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "fwd_params.h"
#include "launchers.h"

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kDim = 128;         // head size (bytes per fp8 row)
constexpr int kBlk = 64;          // keys per block
constexpr int kW8 = 8;            // waves per workgroup
constexpr int kThr8 = kW8 * kWave;
constexpr float kPMax = 256.f;    // bound on a half-block's probability sum (so each p fits E4M3)

// K tile: 64 rows of 128 bytes (8 chunks); V^T tile: 128 rows of 64 bytes (4 chunks).
__device__ __forceinline__ int kswz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int vswz8(int d) { return (d >> 2) & 3; }

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format codes 0 / 0: both operands E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four floats -> four E4M3 bytes (round to nearest even), first argument in the low byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ f32x16 zeros16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

}  // namespace

template <int HP>
__global__ __launch_bounds__(kThr8) __attribute__((amdgpu_waves_per_eu(kW8 / 4, kW8 / 4)))
void fwd_fp8_kernel(FwdParams p) {
  // Double buffers, one array per buffer (reads of one buffer then need not wait for the
  // direct-to-LDS loads in flight into the other).
  __shared__ __attribute__((aligned(16))) u32x4 Ks0[kBlk * kDim / 16], Ks1[kBlk * kDim / 16];
  __shared__ __attribute__((aligned(16))) uint32_t Vt0[kDim * kBlk / 4], Vt1[kDim * kBlk / 4];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar values and branches
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int g = lane / 32;

  // ---- work item: (batch, head group, query block), longest causal blocks first, all
  // blocks of one head group on one XCD (work_order).
  constexpr int RH = kW8 * 32 / HP;  // rows per head per workgroup
  int qb, grp;
  {
    const int bid = blockIdx.x;
    int rank;
    work_order(bid, p.n_qblocks, p.n_groups, p.xcd_remap, rank, grp);
    qb = p.n_qblocks - 1 - rank;
  }
  const int hpg = p.Hq / HP;
  const int b = grp / hpg;
  const int hq = (grp % hpg) * HP + wid / (kW8 / HP);
  const int kvh = ((grp % hpg) * HP) / (p.Hq / p.Hkv);
  const int T = p.T, S = p.S;
  const int64_t pos = p.pos;
  const int wrow0 = qb * RH + (wid % (kW8 / HP)) * 32;  // first query row of this wave
  const int t = wrow0 + l32;                            // this lane's query

  const uint8_t* qg = (const uint8_t*)p.q + ((size_t)b * p.Hq + hq) * (size_t)T * kDim;
  const uint8_t* kg = (const uint8_t*)p.k + ((size_t)b * p.Hkv + kvh) * (size_t)S * kDim;
  const uint8_t* vg = (const uint8_t*)p.v + ((size_t)b * p.Hkv + kvh) * (size_t)kDim * S;  // V^T rows

  // ---- keys visible to this wave / to the workgroup.
  int nk_wave = S, nk_wg = S;
  if (p.causal) {
    const int64_t lw = pos + (int64_t)min(T - 1, wrow0 + 31) + 1;
    nk_wave = (int)(lw < 0 ? 0 : (lw < S ? lw : S));
    const int64_t lg = pos + (int64_t)min(T - 1, qb * RH + RH - 1) + 1;
    nk_wg = (int)(lg < 0 ? 0 : (lg < S ? lg : S));
  }
  const int n_tiles = (nk_wg + kBlk - 1) / kBlk;

  // ---- Q^T operand: lane holds query t, bytes ks*64 + g*32 .. +31 of its row.
  i32x8 qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (t < T) {
      lo = *(const u32x4*)(qg + (size_t)t * kDim + ks * 64 + g * 32);
      hi = *(const u32x4*)(qg + (size_t)t * kDim + ks * 64 + g * 32 + 16);
    }
    qop[ks] = cat8(lo, hi);
  }
  const float c2 = p.q_scale * p.k_scale * kLog2e / sqrtf((float)kDim);

  // ---- loads.  K: chunk tid of the tile (row tid / 8, stored at chunk position tid % 8,
  // holding logical chunk position ^ swizzle).  V^T: four 4-byte groups per thread; stored
  // dword w' of row d holds logical dword w (chunk (w' / 4) ^ swizzle), i.e. the keys that
  // lane half w / 8 needs at bytes 4 (w % 8) .. +3 of its operand: 4 keys starting at
  // 32 ((w % 8) / 4) + 8 (w % 4) + 4 (w / 8).
  int koff, voff[4];
  {
    const int r = tid >> 3, pp = tid & 7;
    koff = r * kDim + ((pp ^ kswz8(r)) << 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + kThr8 * j;
      const int d = e >> 4, wp = e & 15;
      const int w = (((wp >> 2) ^ vswz8(d)) << 2) | (wp & 3);
      const int u = w & 7, hh = w >> 3;
      const int key0 = (u >> 2) * 32 + (u & 3) * 8 + hh * 4;
      voff[j] = d * S + key0;
    }
  }
  auto load_tile = [&](int tile, auto bc) {
    constexpr int BUF = decltype(bc)::value;
    const int k0 = tile * kBlk;
    const i32x4 rk = make_rsrc(kg + (size_t)k0 * kDim, (uint32_t)min(S - k0, kBlk) * kDim);
    buffer_load_lds16(rk, koff, (BUF ? Ks1 : Ks0) + wid * kWave);
    // V^T: one resource over the whole head shifted by k0; keys past S in a row read the next
    // row's first keys (finite, and their probabilities are 0), the last row's read zero.
    const i32x4 rv = make_rsrc(vg + k0, (uint32_t)((size_t)kDim * S - k0));
#pragma unroll
    for (int j = 0; j < 4; ++j) buffer_load_lds4(rv, voff[j], (BUF ? Vt1 : Vt0) + wid * kWave + kThr8 * j);
  };

  // per-lane LDS byte offsets of the operand reads
  int kro[2][2];  // K rows mb*32 + l32 (mb added as an immediate), k-step ks, chunk half h
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) kro[ks][h] = l32 * kDim + (((ks * 4 + g * 2 + h) ^ kswz8(l32)) << 4);
  int vro[2];  // V^T rows db*32 + l32 (db added as an immediate), chunk half h
#pragma unroll
  for (int h = 0; h < 2; ++h) vro[h] = l32 * kBlk + (((g * 2 + h) ^ vswz8(l32)) << 4);

  float m_ref = -INFINITY, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = zeros16();

  auto compute = [&](int tile, auto bc) {
    constexpr int BUF = decltype(bc)::value;
    const int k0 = tile * kBlk;
    if (!(k0 < nk_wave)) return;
    const char* kt = (const char*)(BUF ? Ks1 : Ks0);
    const char* vt = (const char*)(BUF ? Vt1 : Vt0);
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = zeros16();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 lo = *(const u32x4*)(kt + kro[ks][0] + mb * 32 * kDim);
        const u32x4 hi = *(const u32x4*)(kt + kro[ks][1] + mb * 32 * kDim);
        s[mb] = mfma_fp8(cat8(lo, hi), qop[ks], s[mb]);
      }
    }
    // hidden keys -inf (diagonal and tail blocks only); the base-2 scale c2 is applied in
    // the exponent below
    const bool need_mask = (k0 + kBlk > S) || (p.causal && (int64_t)(k0 + kBlk - 1) > pos + wrow0);
    if (need_mask) {
      // element (mb, r) holds key k0 + g*4 + c, c = mb*32 + (r/4)*8 + r%4: visible iff
      // c <= hi, this query's last visible key relative to k0 + g*4, clamped to 32 bits
      // (opaque to the compiler, which would otherwise compare against the 64-bit bound)
      const int64_t lim = pos + t;
      const int64_t base = (int64_t)k0 + g * 4;
      int64_t hi = (int64_t)S - 1 - base;
      if (p.causal && lim - base < hi) hi = lim - base;
      int hi32 = (int)(hi < -1 ? -1 : (hi > kBlk ? kBlk : hi));
      asm volatile("" : "+v"(hi32));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = mb * 32 + (r / 4) * 8 + (r % 4);
          s[mb][r] = (c <= hi32) ? s[mb][r] : -INFINITY;
        }
    }
    // probabilities against the current reference; if a row has none yet or a half-block sum
    // exceeds kPMax, take the exact block max, raise the reference, rescale o and l, redo
    float pr[2][16], lt[2];
    auto expo = [&]() {
      const float bias = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[mb][r] = fast_exp2(fmaf(s[mb][r], c2, -bias));
        float q4[4];  // four partial sums: short dependency chains
#pragma unroll
        for (int k = 0; k < 4; ++k) q4[k] = (pr[mb][k] + pr[mb][k + 4]) + (pr[mb][k + 8] + pr[mb][k + 12]);
        lt[mb] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
      }
    };
    expo();
    const bool bad = (m_ref == -INFINITY) || !(lt[0] <= kPMax) || !(lt[1] <= kPMax);
    if (__any(bad)) {
      __asm__ volatile("");  // keep this rare path a real branch
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c2;  // c2 > 0: the max of the scaled logits
      // raised only when the max is more than 2^3 above it: every p stays <= 8, so a lane's
      // 16-key half sums to <= 128 < kPMax and the check does not fire again for it
      const bool need = tmax > m_ref + 3.f;
      const float m_new = need ? tmax : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 when m_ref was -inf
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_ref = m_new;
      expo();
    }
    l_run += lt[0] + lt[1];
    // P^T operand: byte 16 mb + r of this lane half holds key mb*32 + (r/4)*8 + g*4 + r%4
    i32x8 pop;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        pop[mb * 4 + q4] =
            (int)pack_fp8x4(pr[mb][4 * q4], pr[mb][4 * q4 + 1], pr[mb][4 * q4 + 2], pr[mb][4 * q4 + 3]);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const u32x4 lo = *(const u32x4*)(vt + vro[0] + db * 32 * kBlk);
      const u32x4 hi = *(const u32x4*)(vt + vro[1] + db * 32 * kBlk);
      o[db] = mfma_fp8(cat8(lo, hi), pop, o[db]);
    }
  };

  auto step = [&](auto bc, int tile) {
    constexpr int BUF = decltype(bc)::value;
    __syncthreads();  // tile landed; everyone is done with tile - 1
    if (tile + 1 < n_tiles) load_tile(tile + 1, std::integral_constant<int, BUF ^ 1>{});
    compute(tile, bc);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's loads have landed
  };
  if (n_tiles > 0) {
    load_tile(0, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // ---- epilogue: O = v_scale * o / l, lse = (m + log2 l) ln 2.
  const float lsum = l_run + __shfl_xor(l_run, 32);
  if (t < T) {
    const float inv = lsum > 0.f ? p.v_scale / lsum : 0.f;
    __bf16* og = (__bf16*)p.out + (((size_t)b * p.Hq + hq) * (size_t)T + t) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      u32x2 w[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        w[q4][0] = pack_bf16(o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv);
        w[q4][1] = pack_bf16(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
      }
      store_block_bf16(og + db * 32, w, g);  // 16-byte pieces
    }
    if (p.lse && g == 0)
      p.lse[((size_t)b * p.Hq + hq) * (size_t)T + t] = lsum > 0.f ? (m_ref + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

namespace {
template <int HP>
hipError_t launch_fp8_one(FwdParams q, hipStream_t stream) {
  constexpr int RH = kW8 * 32 / HP;
  q.n_qblocks = (q.T + RH - 1) / RH;
  q.n_groups = q.B * (q.Hq / HP);
  q.xcd_remap = work_order_mode(q.n_qblocks, q.n_groups);
  const long long grid = (long long)q.n_qblocks * q.n_groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_fp8_kernel<HP>), dim3((unsigned)grid), dim3(kThr8), 0, stream, q);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if (G % 4 == 0) return launch_fp8_one<4>(p, stream);
  if (G % 2 == 0) return launch_fp8_one<2>(p, stream);
  return launch_fp8_one<1>(p, stream);
}

}  // namespace attn
