// Host entry points of libattn: argument validation, parameter packing and launch.
// Every check runs before the first HIP call, so an invalid request leaves the stream
// untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "attn.h"
#include "launchers.h"

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// rope_c[i] = base^(-2i/d_h) / (2 pi): turns of rotation per position for pair i
// ("How does Rotary Position Embedding (RoPE) work?": theta = pos / base^(2i/d)).
void fill_rope(double* c, int d_h, float base) {
  for (int i = 0; i < d_h / 2; ++i)
    c[i] = std::pow((double)base, -2.0 * (double)i / (double)d_h) / kTwoPi;
  for (int i = d_h / 2; i < attn::kMaxHalfDim; ++i) c[i] = 0.0;
}

bool bad_base(float rope_base) { return !(std::isfinite(rope_base) && rope_base >= 0.f); }

// The kernels move 16-byte chunks of every head-row tensor and 4-byte words of the lse and
// block tables; misaligned pointers are rejected rather than read.
bool misaligned(const void* p, uintptr_t a) { return p && ((uintptr_t)p & (a - 1)) != 0; }

}  // namespace

extern "C" {

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_SCRATCH: return "request larger than the static decode scratch";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Rows per workgroup of one head in the bf16 prefill (the kernel's 256 query rows shared by
// the heads of a group of HP = 4, 2 or 1 query heads) and keys per block.
constexpr int kPrefillRows = 256;
constexpr int kKeyBlock = 64;

// Average number of workgroups of the bf16 prefill that read each K block: a K block
// rotated as it lands is rotated that many times.
double key_block_reads(int Hq, int Hkv, int T, int S, int causal, int64_t window, int64_t pos) {
  const int G = Hq / Hkv;
  const int HP = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const int RH = kPrefillRows / HP;
  const long long nqb = (T + RH - 1) / RH;
  double tiles = 0.0;
  for (long long qb = 0; qb < nqb; ++qb) {
    long long nk = S;
    if (causal) {
      const long long last = std::min<long long>(T - 1, qb * RH + RH - 1);
      nk = std::max<long long>(0, std::min<long long>(S, pos + last + 1));
    }
    long long it0 = 0;
    if (window > 0) {
      const long long lo = pos + qb * RH - window + 1;
      it0 = (lo <= 0 ? 0 : std::min(lo, nk)) / kKeyBlock;
    }
    tiles += (double)((nk + kKeyBlock - 1) / kKeyBlock - it0);
  }
  const long long nkb = (S + kKeyBlock - 1) / kKeyBlock;
  return tiles * (double)(G / HP) / (double)nkb;
}

// Rotating the keys ahead pays once a K block is read by about ten workgroups (one extra
// read and write of k against the rotation work saved); 16 leaves a margin.
constexpr double kRotateAheadReads = 16.0;

attn_status_t fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                       int T, int S, int d_h, int causal, int64_t window, float rope_base, int64_t pos,
                       void* workspace, size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) || misaligned(lse, 4) ||
      misaligned(workspace, 16))
    return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || d_h < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (bad_base(rope_base)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (d_h != 64 && d_h != 128) return ATTN_ERR_UNSUPPORTED;
  if (pos > ((int64_t)1 << 40) || pos < -((int64_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
  // the bf16 kernel reads one KV head's keys through a 32-bit buffer range
  if (dtype == ATTN_BF16 && (uint64_t)S * (uint64_t)d_h * 2u > 0xffffffffull) return ATTN_ERR_UNSUPPORTED;

  attn::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.T = T;
  p.S = S;
  p.causal = causal;
  p.window = window;
  p.pos = pos;
  p.use_rope = rope_base > 0.f;
  fill_rope(p.rope_c, d_h, p.use_rope ? rope_base : 1.f);
  // a workspace large enough for a rotated copy of k: the keys are rotated once, ahead
  const size_t kbytes = (size_t)B * Hkv * S * d_h * 2;
  if (dtype == ATTN_BF16 && p.use_rope && workspace && workspace_bytes >= kbytes) p.k_rot = workspace;

  hipStream_t st = (hipStream_t)stream;
  hipError_t e = (dtype == ATTN_F32) ? attn::launch_fwd_f32(p, d_h, st) : attn::launch_fwd_bf16(p, d_h, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                       int Hkv, int T, int S, int d_h, int causal, float rope_base, int64_t pos,
                       void* workspace, size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  return fwd_impl(q, k, v, out, lse, B, Hq, Hkv, T, S, d_h, causal, 0, rope_base, pos, workspace,
                  workspace_bytes, dtype, stream);
}

attn_status_t attn_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                              int Hq, int Hkv, int T, int S, int d_h, int64_t window, float rope_base,
                              int64_t pos, void* workspace, size_t workspace_bytes, attn_dtype_t dtype,
                              void* stream) {
  if (window < 1) return ATTN_ERR_INVALID_ARG;
  if (window > ((int64_t)1 << 41)) window = (int64_t)1 << 41;  // wider than any reach: plain causal
  return fwd_impl(q, k, v, out, lse, B, Hq, Hkv, T, S, d_h, 1, window, rope_base, pos, workspace,
                  workspace_bytes, dtype, stream);
}

size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int T, int S, int d_h, int causal, int64_t window,
                                float rope_base, int64_t pos, attn_dtype_t dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || Hq % Hkv != 0) return 0;
  if (d_h != 64 && d_h != 128) return 0;
  if (dtype != ATTN_BF16 || bad_base(rope_base) || !(rope_base > 0.f)) return 0;
  if (causal != 0 && causal != 1) return 0;
  if (window > 0) causal = 1;
  if (key_block_reads(Hq, Hkv, T, S, causal, window, pos) < kRotateAheadReads) return 0;
  return (size_t)B * Hkv * S * d_h * 2;
}

attn_status_t attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* out, float* lse, int B, int Hq,
                           int Hkv, int T, int S, int d_h, int causal, float q_scale, float k_scale, float v_scale,
                           int64_t pos, void* stream) {
  if (!q8 || !k8 || !vt8 || !out) return ATTN_ERR_INVALID_ARG;
  if (misaligned(q8, 16) || misaligned(k8, 16) || misaligned(out, 16) || misaligned(lse, 4))
    return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || d_h < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  for (float sc : {q_scale, k_scale, v_scale})
    if (!(std::isfinite(sc) && sc > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (d_h != 128 || S % 4 != 0 || ((uintptr_t)vt8 & 3) != 0) return ATTN_ERR_UNSUPPORTED;
  if (pos > ((int64_t)1 << 40) || pos < -((int64_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
  if ((size_t)d_h * S > 0xffffffffu) return ATTN_ERR_UNSUPPORTED;

  attn::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q8;
  p.k = k8;
  p.v = vt8;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.T = T;
  p.S = S;
  p.causal = causal;
  p.pos = pos;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  hipError_t e = attn::launch_fwd_fp8(p, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, int block_size,
                                 int num_seqs, int Hq, int Hkv, int d_h, int T, int max_blocks_per_seq,
                                 int num_blocks, float rope_base, void* out, float* lse, attn_dtype_t dtype,
                                 void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return ATTN_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(lse, 4) || misaligned(block_table, 4) || misaligned(seq_lens, 4))
    return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || d_h < 1 || T < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      block_size < 1)
    return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (bad_base(rope_base)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 || d_h != 128 || block_size != attn::kPageBlock ||
      max_blocks_per_seq > attn::kMaxPagedBlocks)
    return ATTN_ERR_UNSUPPORTED;

  attn::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.out = out;
  p.lse = lse;
  p.B = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.T = T;
  p.S = max_blocks_per_seq * block_size;
  p.causal = 1;
  p.paged = 1;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.use_rope = rope_base > 0.f;
  fill_rope(p.rope_c, d_h, p.use_rope ? rope_base : 1.f);
  hipError_t e = attn::launch_fwd_bf16(p, d_h, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"

namespace {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool bwd_sizes_ok(int B, int Hq, int Hkv, int T, int S, int d_h) {
  return B >= 1 && Hq >= 1 && Hkv >= 1 && T >= 1 && S >= 1 && d_h >= 1 && Hq % Hkv == 0;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int S, int d_h, float rope_base) {
  if (!bwd_sizes_ok(B, Hq, Hkv, T, S, d_h) || bad_base(rope_base)) return 0;
  const size_t rows = (size_t)B * Hq * T;
  size_t n = align256(rows * 16) + align256(rows * d_h * 2);
  if (rope_base > 0.f) n += align256((size_t)B * Hkv * S * d_h * 2);
  return n;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int T, int S,
                       int d_h, int causal, int64_t window, float rope_base, int64_t pos, void* workspace,
                       size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  for (const void* t : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv, (const void*)workspace})
    if (misaligned(t, 16)) return ATTN_ERR_INVALID_ARG;
  if (misaligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!bwd_sizes_ok(B, Hq, Hkv, T, S, d_h)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (window < 0 || (window > 0 && causal != 1)) return ATTN_ERR_INVALID_ARG;
  if (bad_base(rope_base)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 || d_h != 128) return ATTN_ERR_UNSUPPORTED;
  if (pos > ((int64_t)1 << 40) || pos < -((int64_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, T, S, d_h, rope_base);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (window > ((int64_t)1 << 41)) window = (int64_t)1 << 41;

  attn::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const size_t rows = (size_t)B * Hq * T;
  char* ws = (char*)workspace;
  p.rec = ws;
  ws += align256(rows * 16);
  p.qr = ws;
  ws += align256(rows * d_h * 2);
  p.use_rope = rope_base > 0.f;
  if (p.use_rope) p.kr = ws;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.T = T;
  p.S = S;
  p.causal = causal;
  p.window = window;
  p.pos = pos;
  fill_rope(p.rope_c, d_h, p.use_rope ? rope_base : 1.f);
  hipError_t e = attn::launch_bwd_bf16(p, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_decode_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_h, int max_blocks_per_seq,
                                   int block_size) {
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d_h < 1 || max_blocks_per_seq < 1 ||
      block_size < 1)
    return 0;
  const size_t slots = (size_t)attn::decode_num_slots(num_seqs, Hkv, max_blocks_per_seq);
  const size_t parts = slots * (size_t)(Hq / Hkv);
  return parts * ((size_t)d_h + 2) * sizeof(float) + ((size_t)num_seqs + 1) * sizeof(int32_t);
}

}  // extern "C"

namespace {

// Checks of a decode request (everything but the workspace); on success *need holds the
// workspace bytes the request takes.
attn_status_t decode_check(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* seq_lens, int block_size, int num_seqs, int Hq, int Hkv, int d_h,
                           int max_blocks_per_seq, int num_blocks, float rope_base, const void* out,
                           const float* lse, attn_dtype_t dtype, size_t* need) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return ATTN_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(lse, 4) || misaligned(block_table, 4) || misaligned(seq_lens, 4))
    return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || d_h < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      block_size < 1)
    return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (bad_base(rope_base)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 || d_h != 128 || block_size != 16 || Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if ((long long)num_seqs * Hkv * max_blocks_per_seq > (1LL << 30) || (long long)num_seqs * Hq > (1LL << 30))
    return ATTN_ERR_UNSUPPORTED;
  *need = attn_decode_workspace_bytes(num_seqs, Hq, Hkv, d_h, max_blocks_per_seq, block_size);
  return ATTN_OK;
}

attn_status_t decode_launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, int num_seqs, int Hq, int Hkv, int d_h, int max_blocks_per_seq,
                            int num_blocks, float rope_base, void* out, float* lse, void* workspace,
                            hipStream_t stream) {
  attn::DecodeParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.out = out;
  p.lse = lse;
  p.num_seqs = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.nwaves = attn::decode_num_waves(num_seqs, Hkv, max_blocks_per_seq);
  const size_t nparts = (size_t)attn::decode_num_slots(num_seqs, Hkv, max_blocks_per_seq) * (size_t)(Hq / Hkv);
  p.part_o = (float*)workspace;
  p.part_ml = (float*)workspace + nparts * d_h;
  p.seq_prefix = (int32_t*)(p.part_ml + nparts * 2);
  p.use_rope = rope_base > 0.f;
  fill_rope(p.rope_c, d_h, p.use_rope ? rope_base : 1.f);
  hipError_t e = attn::launch_decode_paged(p, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status_t attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens, int block_size,
                                int num_seqs, int Hq, int Hkv, int d_h, int max_blocks_per_seq,
                                int num_blocks, float rope_base, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  size_t need = 0;
  const attn_status_t st = decode_check(q, k_cache, v_cache, block_table, seq_lens, block_size, num_seqs, Hq, Hkv,
                                        d_h, max_blocks_per_seq, num_blocks, rope_base, out, lse, dtype, &need);
  if (st != ATTN_OK) return st;
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return ATTN_ERR_INVALID_ARG;
  return decode_launch(q, k_cache, v_cache, block_table, seq_lens, num_seqs, Hq, Hkv, d_h, max_blocks_per_seq,
                       num_blocks, rope_base, out, lse, workspace, (hipStream_t)stream);
}

attn_status_t attn_decode_paged_static(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, int block_size,
                                       int num_seqs, int Hq, int Hkv, int d_h, int max_blocks_per_seq,
                                       int num_blocks, float rope_base, void* out, float* lse, attn_dtype_t dtype,
                                       void* stream) {
  size_t need = 0;
  const attn_status_t st = decode_check(q, k_cache, v_cache, block_table, seq_lens, block_size, num_seqs, Hq, Hkv,
                                        d_h, max_blocks_per_seq, num_blocks, rope_base, out, lse, dtype, &need);
  if (st != ATTN_OK) return st;
  if (need > ATTN_DECODE_STATIC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (attn::decode_static_scratch((hipStream_t)stream, &scratch) != hipSuccess) return ATTN_ERR_HIP;
  return decode_launch(q, k_cache, v_cache, block_table, seq_lens, num_seqs, Hq, Hkv, d_h, max_blocks_per_seq,
                       num_blocks, rope_base, out, lse, scratch, (hipStream_t)stream);
}

attn_status_t attn_paged_gather(const void* cache, const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int num_seqs, int Hkv, int d_h, int max_blocks_per_seq,
                                int num_blocks, int elem_bytes, void* dst, void* stream) {
  if (!cache || !block_table || !seq_lens || !dst) return ATTN_ERR_INVALID_ARG;
  if (misaligned(cache, 16) || misaligned(dst, 16) || misaligned(block_table, 4) || misaligned(seq_lens, 4))
    return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 1 || Hkv < 1 || d_h < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || block_size < 1)
    return ATTN_ERR_INVALID_ARG;
  if (elem_bytes != 2 && elem_bytes != 4) return ATTN_ERR_INVALID_ARG;
  // the decode kernel's read path: 16-token blocks of 256-byte rows (bf16, d_h = 128)
  if (block_size != 16 || d_h * elem_bytes != 256) return ATTN_ERR_UNSUPPORTED;
  if ((long long)num_seqs * Hkv * max_blocks_per_seq > (1LL << 30)) return ATTN_ERR_UNSUPPORTED;

  attn::DecodeParams p;
  std::memset(&p, 0, sizeof(p));
  p.k_cache = cache;
  p.v_cache = cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.num_seqs = num_seqs;
  p.Hq = Hkv;
  p.Hkv = Hkv;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.nwaves = attn::decode_num_waves(num_seqs, Hkv, max_blocks_per_seq);
  p.copy_dst = dst;
  hipError_t e = attn::launch_paged_gather(p, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
