// fp32 exact attention (prefill), the precise reference-grade kernel of libattn.
//
// One workgroup of 256 threads owns 32 query rows of one head.  K and V blocks of
// 32 keys are streamed through LDS; every row keeps a running max m, normaliser l and
// unnormalised output o and rescales them per block, which is the online softmax of
// "Why is attention O(n^2), how does FlashAttention help ..." (Deep dive:
// FlashAttention).  Logits live in the base-2 domain (q is pre-multiplied by
// log2(e)/sqrt(d_h)) so each exponential is one exp2.  Causal masking sets hidden
// logits to -inf before the softmax ("Transformer Attention Mechanism Interview Deep
// Dive", Causal masking) and key blocks past the last visible key are never loaded.
// RoPE rotates adjacent pairs at load with the angle computed and reduced in fp64
// ("22 interview questions ...", How does RoPE work).
#include <math.h>

#include "attn_common.h"
#include "fwd_params.h"

namespace attn {

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
  constexpr int BM = 32, BN = 32, TPR = 8, NT = 256;
  constexpr int DPT = D / TPR;  // output columns per thread
  __shared__ float Qs[BM][D + 1];
  __shared__ float Ks[BN][D + 1];
  __shared__ float Vs[BN][D + 1];
  __shared__ float Ps[BM][BN + 1];

  const int tid = threadIdx.x;
  const int row = tid / TPR;
  const int col = tid % TPR;
  int w = blockIdx.x;
  const int qb = w % p.n_qblocks;
  w /= p.n_qblocks;
  const int h = w % p.Hq;
  const int b = w / p.Hq;
  const int kvh = h / (p.Hq / p.Hkv);
  const int t0 = qb * BM;
  const int T = p.T, S = p.S;

  const float* qg = (const float*)p.q + ((size_t)b * p.Hq + h) * (size_t)T * D;
  const float* kg = (const float*)p.k + ((size_t)b * p.Hkv + kvh) * (size_t)S * D;
  const float* vg = (const float*)p.v + ((size_t)b * p.Hkv + kvh) * (size_t)S * D;
  const float qscale = kLog2e / sqrtf((float)D);

  // Q tile: rotate (fp64 angle) and fold the base-2 softmax scale.
  for (int i = tid; i < BM * (D / 2); i += NT) {
    const int r = i / (D / 2), j = i % (D / 2);
    const int t = t0 + r;
    double x0 = 0.0, x1 = 0.0;
    if (t < T) {
      x0 = qg[(size_t)t * D + 2 * j];
      x1 = qg[(size_t)t * D + 2 * j + 1];
      if (p.use_rope) {
        double a = (double)(p.pos + t) * p.rope_c[j];
        a = (a - rint(a)) * 6.283185307179586;
        double s, c;
        sincos(a, &s, &c);
        const double y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
        x0 = (float)y0;
        x1 = (float)y1;
      }
    }
    Qs[r][2 * j] = (float)x0 * qscale;
    Qs[r][2 * j + 1] = (float)x1 * qscale;
  }

  // Keys that can be visible to some row of this block.
  int n_keys = S;
  if (p.causal) {
    const int64_t last = p.pos + (int64_t)min(T - 1, t0 + BM - 1) + 1;
    n_keys = (int)(last < 0 ? 0 : (last < S ? last : S));
  }
  const int64_t qpos = p.pos + t0 + row;
  // Sliding window: keys below the window of the block's first row are never visible.
  int k_first = 0;
  if (p.window > 0) {
    const int64_t lo = p.pos + t0 - p.window + 1;
    k_first = (int)(lo <= 0 ? 0 : (lo < n_keys ? lo : n_keys)) / BN * BN;
  }

  float m = -INFINITY, l = 0.f;
  float o[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) o[i] = 0.f;

  for (int kt = k_first; kt < n_keys; kt += BN) {
    __syncthreads();  // previous block's K/V/P no longer read
    for (int i = tid; i < BN * (D / 2); i += NT) {
      const int r = i / (D / 2), j = i % (D / 2);
      const int s = kt + r;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (s < S) {
        k0 = kg[(size_t)s * D + 2 * j];
        k1 = kg[(size_t)s * D + 2 * j + 1];
        v0 = vg[(size_t)s * D + 2 * j];
        v1 = vg[(size_t)s * D + 2 * j + 1];
        if (p.use_rope) {
          double a = (double)s * p.rope_c[j];
          a = (a - rint(a)) * 6.283185307179586;
          double sn, cs;
          sincos(a, &sn, &cs);
          const double y0 = (double)k0 * cs - (double)k1 * sn, y1 = (double)k0 * sn + (double)k1 * cs;
          k0 = (float)y0;
          k1 = (float)y1;
        }
      }
      Ks[r][2 * j] = k0;
      Ks[r][2 * j + 1] = k1;
      Vs[r][2 * j] = v0;
      Vs[r][2 * j + 1] = v1;
    }
    __syncthreads();

    float sc[BN / TPR];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < BN / TPR; ++i) {
      const int kk = col + TPR * i;
      const int s = kt + kk;
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc = fmaf(Qs[row][d], Ks[kk][d], acc);
      const bool vis = (s < S) && (!p.causal || (int64_t)s <= qpos) && (p.window <= 0 || (int64_t)s > qpos - p.window);
      sc[i] = vis ? acc : -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < BN / TPR; ++i) {
      const float pv = exp2f(sc[i] - m_use);
      psum += pv;
      Ps[row][col + TPR * i] = pv;
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) psum += __shfl_xor(psum, off);
    l = l * alpha + psum;
    m = m_new;
    __syncthreads();
#pragma unroll
    for (int dd = 0; dd < DPT; ++dd) {
      const int d = col + TPR * dd;
      float acc = o[dd] * alpha;
#pragma unroll 8
      for (int j = 0; j < BN; ++j) acc = fmaf(Ps[row][j], Vs[j][d], acc);
      o[dd] = acc;
    }
  }

  const int t = t0 + row;
  if (t < T) {
    float* og = (float*)p.out + (((size_t)b * p.Hq + h) * (size_t)T + t) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dd = 0; dd < DPT; ++dd) og[col + TPR * dd] = o[dd] * inv;
    if (p.lse && col == 0)
      p.lse[((size_t)b * p.Hq + h) * (size_t)T + t] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_fwd_f32(const FwdParams& p, int d_h, hipStream_t stream) {
  const int n_qb = (p.T + 31) / 32;
  FwdParams q = p;
  q.n_qblocks = n_qb;
  const long long grid = (long long)n_qb * p.Hq * p.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (d_h == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, q);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, q);
  return hipGetLastError();
}

}  // namespace attn
