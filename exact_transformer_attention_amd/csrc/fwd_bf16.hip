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
//  * workgroup = 4 waves; each wave owns 64 query rows of one head.  The heads that
//    share one KV head (grouped-query attention) are packed into the same workgroup
//    (HP heads per workgroup), so every K/V block loaded, and rotated, once serves
//    256 query rows.
//  * S^T = K Q^T: K (64-key block) is the A operand read from LDS, Q^T the B operand
//    held in registers for the whole kernel.  In the accumulator layout a lane owns
//    one query column, so the row max and row sum are in-lane except for one swap
//    with the lane 32 apart.
//  * O^T = V^T P^T: P^T is the B operand exactly as the S^T accumulators sit in
//    registers (the contraction order over keys is permuted to match), V^T is read
//    from a row-major LDS tile with ds_read_b64_tr_b16.  Again a lane owns one query,
//    so the rescale factor is a per-lane scalar.
//  * Logits are in the base-2 domain: RoPE'd q is pre-multiplied by log2(e)/sqrt(d_h)
//    before rounding to bf16, so p = exp2(s - m).
//  * The running max is raised only when a block's max exceeds it by more than 8
//    (in log2 units).  p is then at most 2^8, which fp32 accumulators and bf16 P
//    carry without loss, and the final o / l is unchanged because o and l are
//    scaled by the same reference; the rescale is skipped in most blocks.
//  * RoPE: q rotated once at load; K rotated when a block is copied from HBM to LDS,
//    using per-thread fixed angle offsets combined with a per-block base angle
//    (angle addition), all angles reduced modulo one turn in fp64.
//  * K/V blocks are double-buffered in LDS; the next block's global loads are in
//    flight while the current one is consumed.  Work is ordered longest-first for
//    causal load balance and mapped so all query blocks of one KV head land on one
//    XCD (shared L2).
#include <math.h>

#include "attn_common.h"
#include "fwd_params.h"
#include "launchers.h"

namespace attn {

namespace {

constexpr int kNW = 4;        // waves per workgroup
constexpr int kQW = 64;       // query rows per wave
constexpr int kBN = 64;       // keys per block
constexpr int kThreads = kNW * kWave;

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;             // k-steps of the QK^T product
  static constexpr int DB = D / 32;             // 32-wide dim blocks of the output
  static constexpr int KSTR = D + 8;            // K row stride in LDS (bf16)
  static constexpr int VSTR = D + 32;           // V row stride in LDS (bf16)
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int NCH = kBN * CPR / kThreads;  // chunks per thread per tensor
  static constexpr int KROW_STEP = kThreads / CPR;  // key stride between a thread's chunks
};

__device__ __forceinline__ void lds_barrier() { __syncthreads(); }

}  // namespace

template <int D, int HP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][kBN * C::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][kBN * C::VSTR];

  const int tid = threadIdx.x;
  const int wid = tid / kWave;
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int g = lane / 32;

  // ---- work item: (batch, head group, query block), longest causal blocks first.
  constexpr int RH = kNW * kQW / HP;  // rows per head per workgroup
  int qb, grp;
  {
    const int bid = blockIdx.x;
    if (p.xcd_remap) {
      const int xcd = bid % 8, slot = bid / 8, gpx = p.n_groups / 8;
      qb = p.n_qblocks - 1 - slot / gpx;
      grp = xcd + 8 * (slot % gpx);
    } else {
      qb = p.n_qblocks - 1 - bid / p.n_groups;
      grp = bid % p.n_groups;
    }
  }
  const int hpg = p.Hq / HP;
  const int b = grp / hpg;
  const int hq = (grp % hpg) * HP + wid / (kNW / HP);
  const int kvh = ((grp % hpg) * HP) / (p.Hq / p.Hkv);
  const int T = p.T, S = p.S;
  const int wrow0 = qb * RH + (wid % (kNW / HP)) * kQW;  // first query row of this wave
  const int64_t pos = p.pos;

  const __bf16* qg = (const __bf16*)p.q + ((size_t)b * p.Hq + hq) * (size_t)T * D;
  const __bf16* kg = (const __bf16*)p.k + ((size_t)b * p.Hkv + kvh) * (size_t)S * D;
  const __bf16* vg = (const __bf16*)p.v + ((size_t)b * p.Hkv + kvh) * (size_t)S * D;

  // ---- keys visible to this wave / to the workgroup.
  int nk_wave = S, nk_wg = S;
  if (p.causal) {
    const int64_t lw = pos + (int64_t)min(T - 1, wrow0 + kQW - 1) + 1;
    nk_wave = (int)(lw < 0 ? 0 : (lw < S ? lw : S));
    const int64_t lg = pos + (int64_t)min(T - 1, qb * RH + RH - 1) + 1;
    nk_wg = (int)(lg < 0 ? 0 : (lg < S ? lg : S));
  }
  const int n_tiles = (nk_wg + kBN - 1) / kBN;

  // ---- Q^T operand in registers: lane holds query l32 of n-block nb, dims ks*16 + g*8.
  bf16x8 qop[2][C::KS];
  {
    const float qscale = kLog2e / sqrtf((float)D);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int t = wrow0 + nb * 32 + l32;
      const bool ok = t < T;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (ok) raw = *(const u32x4*)(qg + (size_t)t * D + ks * 16 + g * 8);
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x0 = bf16_lo(raw[e]), x1 = bf16_hi(raw[e]);
          if (p.use_rope) {
            const float tr = rope_turns(pos + t, p.rope_c[ks * 8 + g * 4 + e]);
            float sn, cs;
            sincos_rev(tr, &sn, &cs);
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

  // ---- per-thread K/V copy assignment and fixed RoPE offsets.
  const int crow = tid / C::CPR;        // first key row of this thread's chunks
  const int cchk = tid % C::CPR;        // 16-byte chunk (8 dims = 4 pairs) within the row
  float off_c[C::NCH][4], off_s[C::NCH][4];
  double base_c[4];
  if (p.use_rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) base_c[e] = p.rope_c[cchk * 4 + e];
#pragma unroll
    for (int i = 0; i < C::NCH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float tr = rope_turns((int64_t)(crow + i * C::KROW_STEP), base_c[e]);
        sincos_rev(tr, &off_s[i][e], &off_c[i][e]);
      }
  }

  u32x4 kreg[C::NCH], vreg[C::NCH];
  auto load_tile = [&](int tile) {
    const int k0 = tile * kBN;
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int s = k0 + crow + i * C::KROW_STEP;
      if (s < S) {
        kreg[i] = *(const u32x4*)(kg + (size_t)s * D + cchk * 8);
        vreg[i] = *(const u32x4*)(vg + (size_t)s * D + cchk * 8);
      } else {
        kreg[i] = (u32x4){0u, 0u, 0u, 0u};
        vreg[i] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int tile, int buf) {
    if (p.use_rope) {
      const int64_t k0 = (int64_t)tile * kBN;
      float bc[4], bs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sincos_rev(rope_turns(k0, base_c[e]), &bs[e], &bc[e]);
#pragma unroll
      for (int i = 0; i < C::NCH; ++i) {
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = bc[e] * off_c[i][e] - bs[e] * off_s[i][e];
          const float s = bs[e] * off_c[i][e] + bc[e] * off_s[i][e];
          const float x0 = bf16_lo(kreg[i][e]), x1 = bf16_hi(kreg[i][e]);
          out[e] = pack_bf16(x0 * c - x1 * s, x0 * s + x1 * c);
        }
        *(u32x4*)&Ks[buf][(crow + i * C::KROW_STEP) * C::KSTR + cchk * 8] = out;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::NCH; ++i)
        *(u32x4*)&Ks[buf][(crow + i * C::KROW_STEP) * C::KSTR + cchk * 8] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::NCH; ++i)
      *(u32x4*)&Vs[buf][(crow + i * C::KROW_STEP) * C::VSTR + cchk * 8] = vreg[i];
  };

  // ---- running state: two query n-blocks per lane.
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x16 o[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][nb][r] = 0.f;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(it + 1);
    lds_barrier();

    const int k0 = it * kBN;
    if (k0 < nk_wave) {
      const __bf16* kb = &Ks[buf][0];
      const __bf16* vb = &Vs[buf][0];
      // S^T = K Q^T
      f32x16 s[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mb][nb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 a = *(const bf16x8*)(kb + (mb * 32 + l32) * C::KSTR + ks * 16 + g * 8);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[nb][ks], s[mb][nb], 0, 0, 0);
        }
      }
      // mask (diagonal / tail blocks only)
      const bool need_mask = (k0 + kBN > S) || (p.causal && (int64_t)(k0 + kBN - 1) > pos + wrow0);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int64_t qp = pos + wrow0 + nb * 32 + l32;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + mb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
              const bool vis = key < S && (!p.causal || (int64_t)key <= qp);
              if (!vis) s[mb][nb][r] = -INFINITY;
            }
        }
      }
      // online softmax
      bf16x8 pop[2][4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][nb][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = tmax > m_run[nb] + 8.f;
        if (__any(need)) {
          // lanes that keep their reference use alpha = 1 (their m may still be -inf)
          const float m_new = need ? tmax : m_run[nb];
          const float alpha = need ? fast_exp2(m_run[nb] - m_new) : 1.f;  // 0 when m_run was -inf
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][nb][r] *= alpha;
          m_run[nb] = m_new;
        }
        const float mu = (m_run[nb] == -INFINITY) ? 0.f : m_run[nb];
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = fast_exp2(s[mb][nb][8 * h + 2 * e] - mu);
              const float p1 = fast_exp2(s[mb][nb][8 * h + 2 * e + 1] - mu);
              psum += p0 + p1;
              pk[e] = pack_bf16(p0, p1);
            }
            pop[nb][mb * 2 + h] = __builtin_bit_cast(bf16x8, pk);
          }
        l_run[nb] += psum;
      }
      // O^T += V^T P^T
      const int a16 = lane / 16, lam = lane % 16;
      const int trow = 4 * g + lam / 4;
      const int tcol = 16 * (a16 % 2) + 4 * (lam % 4);
#pragma unroll
      for (int kstep = 0; kstep < 4; ++kstep) {
        const int kwin = kstep * 16;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const __bf16* a0p = vb + (kwin + trow) * C::VSTR + db * 32 + tcol;
          const __bf16* a1p = a0p + 8 * C::VSTR;
          const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(a0p));
          const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(a1p));
          const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
          const bf16x8 a = __builtin_bit_cast(bf16x8, (u32x4){w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[nb][kstep], o[db][nb], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(it + 1, buf ^ 1);
  }

  // ---- epilogue: O = o / l, lse = (m + log2 l) ln 2.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const int t = wrow0 + nb * 32 + l32;
    if (t < T) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      __bf16* og = (__bf16*)p.out + (((size_t)b * p.Hq + hq) * (size_t)T + t) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 w;
          w[0] = pack_bf16(o[db][nb][4 * q4 + 0] * inv, o[db][nb][4 * q4 + 1] * inv);
          w[1] = pack_bf16(o[db][nb][4 * q4 + 2] * inv, o[db][nb][4 * q4 + 3] * inv);
          *(u32x2*)(og + db * 32 + q4 * 8 + g * 4) = w;
        }
      if (p.lse && g == 0)
        p.lse[((size_t)b * p.Hq + hq) * (size_t)T + t] =
            lt > 0.f ? (m_run[nb] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

namespace {
template <int D, int HP>
hipError_t launch_one(FwdParams q, hipStream_t stream) {
  constexpr int RH = kNW * kQW / HP;
  q.n_qblocks = (q.T + RH - 1) / RH;
  q.n_groups = q.B * (q.Hq / HP);
  q.xcd_remap = (q.n_groups % 8) == 0;
  const long long grid = (long long)q.n_qblocks * q.n_groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, HP>), dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if (G % 4 == 0) return launch_one<D, 4>(p, stream);
  if (G % 2 == 0) return launch_one<D, 2>(p, stream);
  return launch_one<D, 1>(p, stream);
}
}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d_h, hipStream_t stream) {
  if (d_h == 64) return launch_d<64>(p, stream);
  return launch_d<128>(p, stream);
}

}  // namespace attn
