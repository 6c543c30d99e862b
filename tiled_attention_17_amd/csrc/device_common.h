// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// MFMA lane layouts used throughout (wave64, l = lane id, h = l / 32):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16):  lane l holds row l%32, k = 8h .. 8h+7
//                             B (16 x 32):  lane l holds col l%32, k = 8h .. 8h+7
//                             C (32 x 32):  lane l holds col l%32, rows 8(i/4) + 4h + i%4, i = 0..15
//   v_mfma_f32_32x32x2_f32    A (32 x 2):   lane l holds row l%32, k = h
//                             B (2 x 32):   lane l holds col l%32, k = h
//                             C: as above.
// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element
// j%4 of the 8-byte words addressed by lanes 4e + j/4 (e = 0..3) as its
// elements e = 0..3, i.e. a 4 x 16 block of 16-bit values is read transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware transcendental unit.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}
// max(x, value of lane l ^ 32) with one v_permlane32_swap.
__device__ __forceinline__ float max_with_other_half(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x + value of lane l ^ 32.
__device__ __forceinline__ float add_other_half(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2_ev __attribute__((ext_vector_type(2)));
typedef float f32x2_ev __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 for a pair, packed low/high (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const f32x2_ev f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_ev));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Word 3 of a gfx9 buffer resource for raw (unformatted, stride 0) loads with
// the range check against num_records enabled.
constexpr int kBufferRsrcWord3 = 0x00020000;

// One buffer_load_dwordx4 ... lds: 16 bytes per lane from byte offset voff
// of the buffer to LDS address lds + 16 * lane (the LDS side is written
// lane-linearly; completion is counted by vmcnt). A plain device function:
// the host pass of a kernel template must not see the builtin.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, bf16* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           0, 0, 0);
}

// Debug build option TATTN_ORDERED_LDS_DMA: every transfer below goes
// through the intrinsic the compiler orders, and each point that publishes a
// staged tile (publish_lds) also waits for every counter and takes a second
// barrier. A parity run of that build checks that the hand-ordered form of
// the release build computes the same results.
#ifdef TATTN_ORDERED_LDS_DMA
constexpr bool kOrderedLdsDma = true;
#else
constexpr bool kOrderedLdsDma = false;
#endif

// The same transfer issued through inline assembly, which the compiler
// does not see as a write to LDS. For the intrinsic above it conservatively
// waits for the transfer before any later LDS read of the workgroup's
// memory, which exposes the whole latency of a tile staged for the next
// step at the start of the current one; with this form the caller alone
// orders the transfer, by wait_vmem() before the barrier that publishes the
// tile (vector-memory loads complete in order, so the compiler's own counted
// waits for other loads stay correct).
// The LDS address goes in as an m0 operand, so the compiler writes m0 itself
// and knows its value afterwards (the s_nop keeps a wait state between that
// write and the transfer that reads it).
__device__ __forceinline__ void lds_dma16_async(__amdgpu_buffer_rsrc_t r, bf16* lds, int voff) {
  if (kOrderedLdsDma) {
    lds_dma16(r, lds, voff);
    return;
  }
  const unsigned m = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "{m0}"(__builtin_amdgcn_readfirstlane(m))
      : "memory");
}

// Waits until this wave's vector-memory operations are done (among them the
// buffer_load ... lds writes of a directly staged tile).
// (The builtin rather than inline assembly, so that the compiler's own wait
// insertion knows every earlier load has completed here: a wait it cannot
// see leaves loads it believes pending, and on a later path it would wait
// for them again, counting the tile staged meanwhile as well.)
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left at their maximum
}

// Publishes the tiles this wave staged (with either transfer form above) to
// the whole workgroup: its vector-memory operations are waited for, then a
// workgroup barrier. Every wave of the workgroup must call it.
__device__ __forceinline__ void publish_lds() {
  wait_vmem();
  __syncthreads();
  if (kOrderedLdsDma) {
    __builtin_amdgcn_s_waitcnt(0);  // every counter
    __syncthreads();
  }
}

// 8 bf16 from two transposed 4-element LDS reads (see the header comment).
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const bf16* p0, const bf16* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  u32x4 r;
  r[0] = __builtin_bit_cast(u32x2, a)[0];
  r[1] = __builtin_bit_cast(u32x2, a)[1];
  r[2] = __builtin_bit_cast(u32x2, b)[0];
  r[3] = __builtin_bit_cast(u32x2, b)[1];
  return as_bf16x8(r);
}

// Swap bits 2 and 3 of a row index (an involution). Placing key r of a
// 32-key block at LDS row swap23(r) makes the fp32 accumulator of the
// transposed score tile hold, in lane half h, the 8 consecutive keys
// 16t + 8h .. 16t + 8h + 7 at accumulator slots 8t .. 8t + 7, which is exactly
// the B-operand order the next MFMA (over keys) needs.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Workgroup id -> logical tile id so that consecutive logical tiles (the
// query tiles of one head, which share K and V) land on the same XCD: the
// dispatcher places workgroup w on XCD w % 8.
__device__ __forceinline__ int xcd_tile(int w, int total, int remap) {
  return remap ? (w & 7) * (total >> 3) + (w >> 3) : w;
}

}  // namespace tattn
