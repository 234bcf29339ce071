// Shared device helpers for the libattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): lane i of the
// wave writes lds_wave_base + 16 * i; lds_wave_base must be the same for the whole wave.
// The builtin only exists for the device pass; keeping it out of the host pass keeps
// clang emitting the host launch stubs of the kernels that use it.  kPolicy is the
// instruction's cache-policy field: 0 (default) or kStreamPolicy.
constexpr int kStreamPolicy = 2;  // "nt": data read once, streamed past the caches
template <int kPolicy = 0>
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, kPolicy);
#endif
}

// Buffer resource (V#) of a raw byte range: reads at offsets >= bytes return zero.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);  // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;  // raw 32-bit data, no swizzle
  return r;
}

__device__ void llvm_raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size,
                                         int voffset, int soffset, int offset,
                                         int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// 16 bytes at byte offset voffset of a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane i writes lds_wave_base + 16 * i.  The resource and LDS base are
// wave-uniform, so the per-lane address costs no vector arithmetic.
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, int voffset, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  llvm_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voffset, 0, 0, 0);
#endif
}

// 4 bytes at byte offset voffset of a buffer straight into LDS: lane i writes
// lds_wave_base + 4 * i.
__device__ __forceinline__ void buffer_load_lds4(i32x4 rsrc, int voffset, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  llvm_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 4, voffset, 0, 0, 0);
#endif
}

// sin and cos of 2*pi*rev for |rev| <= 0.5 (hardware v_sin/v_cos take revolutions).
__device__ __forceinline__ void sincos_rev(float rev, float* s, float* c) {
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

// Fractional turns of the RoPE angle p * inv, given c = inv / (2 pi) in fp64: the
// product and its reduction modulo one turn are done in fp64 (exact enough for any
// position below 2^40), and the reduced value in [-0.5, 0.5] is rounded to fp32.
__device__ __forceinline__ float rope_turns(int64_t p, double c) {
  double a = (double)p * c;
  a = a - __builtin_rint(a);
  return (float)a;
}


// Work order of a grid of n_groups x nblk workgroups, block-major rank 0 = the work item
// to start first.  Workgroup bid runs on XCD bid % 8, so with mode != 0 (n_groups a
// multiple of 8) all items of a group go to one XCD (one L2).  Mode 1: the XCD interleaves
// its groups, all items in rank order (longest first when rank 0 is the longest).  Mode 2:
// the XCD runs its groups one after the other, so its L2 holds one group's K/V at a time;
// the host picks it only when each group has enough items (nblk >= kSeqOrderMin) for the
// next group's long items to start early enough.
constexpr int kSeqOrderMin = 64;
__device__ __forceinline__ void work_order(int bid, int nblk, int n_groups, int mode, int& rank, int& grp) {
  if (mode == 2) {
    const int xcd = bid % 8, slot = bid / 8;
    rank = slot % nblk;
    grp = xcd + 8 * (slot / nblk);
  } else if (mode == 1) {
    const int xcd = bid % 8, slot = bid / 8, gpx = n_groups / 8;
    rank = slot / gpx;
    grp = xcd + 8 * (slot % gpx);
  } else {
    rank = bid / n_groups;
    grp = bid % n_groups;
  }
}
__host__ __device__ constexpr int work_order_mode(int nblk, int n_groups) {
  return (n_groups % 8) ? 0 : (nblk >= kSeqOrderMin ? 2 : 1);
}

// Writes one 32-dim block of a row held in the 32x32 accumulator layout: lane (row, g) holds
// dims 8*q4 + 4*g + 0..3 of the block as w[q4] (four bf16).  One exchange with the lane 32
// apart (the same row) gives lane g = 0 the 8 dims of q4 = 0 and 2 and lane g = 1 those of
// q4 = 1 and 3, so each lane writes two 16-byte pieces (dst 16-byte aligned).  Both lanes of
// a row must execute it.
__device__ __forceinline__ void store_block_bf16(__bf16* dst, const u32x2 (&w)[4], int g) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // q4 pair (2h, 2h + 1)
    const u32x2 send = g ? w[2 * h] : w[2 * h + 1];
    u32x2 recv;
    recv[0] = (uint32_t)__shfl_xor((int)send[0], 32);
    recv[1] = (uint32_t)__shfl_xor((int)send[1], 32);
    const u32x2 lo = g ? recv : w[2 * h], hi = g ? w[2 * h + 1] : recv;
    *(u32x4*)(dst + (2 * h + g) * 8) = (u32x4){lo[0], lo[1], hi[0], hi[1]};
  }
}

}  // namespace attn
