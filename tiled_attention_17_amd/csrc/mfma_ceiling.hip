// Measurement probe (not part of the attention path): the sustained bf16
// matrix-core rate of the whole chip, and its shader clock, for operand data
// and companion work like the attention kernels'. It is the compute-bound
// end of the roofline (Lecture 17 page §6.2-§6.4) measured instead of taken
// from the datasheet: the published dense peak assumes the nominal 2.4 GHz,
// and the clock the power management holds depends on what the matrix
// cores multiply.
//
// One 512-thread workgroup per CU (96 KB of LDS keeps a second one out), two
// waves per SIMD, as in the attention kernels. Each wave runs `iters`
// iterations of 8 units of 32768 FLOPs: one v_mfma_f32_32x32x16_bf16 per
// unit, or two v_mfma_f32_16x16x32_bf16 (MODE bit 8). Other MODE bits:
//   1  operands from random bf16 data (8 register pairs loaded once per
//      lane), else constants;
//   2  the A operand of every unit read from LDS (ds_read_b128, random
//      contents, conflict-free), as the attention kernels read K and V^T;
//   4  one softmax-like element per unit (fma, exp2, add, half a bf16 pack),
//      the forward's vector work per MFMA;
//   16 no matrix work (the other work alone);
//   32 each group of four consecutive MFMAs shares one B operand;
//   64 each group of four consecutive MFMAs shares one A operand
//      (32 and 64: how much of the power follows operand changes from one
//      MFMA to the next; with 2, one LDS read per four MFMAs);
//   128 each pair of consecutive MFMAs shares one A operand (with 2, one
//      LDS read per two MFMAs, as a wave of 64 queries would read K and V^T).
// Lane 0 of each wave writes the s_memtime (shader clock) and
// s_memrealtime (100 MHz) ticks around its loop; their ratio is the clock.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_ev __attribute__((ext_vector_type(2)));
typedef float f32x2_ev __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kLdsVecs = 6 * 1024;  // 96 KB of u32x4
constexpr int kRndPerThread = 16;   // u32x4 operand words per thread

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_ceiling_kernel(unsigned long long* out, float* sink, int iters, const u32x4* rnd, int rnd_vecs) {
  __shared__ __attribute__((aligned(16))) u32x4 lds[kLdsVecs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = blockIdx.x * kThreads * kRndPerThread;
  for (int i = tid; i < kLdsVecs; i += kThreads) lds[i] = rnd[(base + i) % rnd_vecs];
  bf16x8 ra[8], rb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (MODE & 1) {
      ra[i] = __builtin_bit_cast(bf16x8, rnd[(base + tid * kRndPerThread + i) % rnd_vecs]);
      rb[i] = __builtin_bit_cast(bf16x8, rnd[(base + tid * kRndPerThread + 8 + i) % rnd_vecs]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ra[i][e] = (__bf16)(0.25f * (e + 1));
        rb[i][e] = (__bf16)(0.5f * (i + 1));
      }
    }
  }
  __syncthreads();
  f32x16 c[4] = {};
  f32x4 e[8] = {};
  float v[8], acc = 0.f;
  unsigned pk = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.25f * i + 1e-3f * (float)(tid & 7);
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (MODE & 2) {
          const int idx = ((((it * 2 + u) & 11) * 4 + i) * 64 + lane) % kLdsVecs;
          a[i] = __builtin_bit_cast(bf16x8, lds[idx]);
        } else {
          a[i] = ra[4 * u + i];
        }
      }
      if (!(MODE & 16)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 ai = (MODE & 64) ? a[0] : (MODE & 128) ? a[i & 2] : a[i];
          const bf16x8 bi = (MODE & 32) ? rb[4 * u] : rb[4 * u + i];
          if (MODE & 8) {
            e[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai, bi, e[2 * i], 0, 0, 0);
            e[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bi, ai, e[2 * i + 1], 0, 0, 0);
          } else {
            c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ai, bi, c[i], 0, 0, 0);
          }
        }
      } else if (MODE & 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pk ^= __builtin_bit_cast(u32x4, a[i])[i];
      }
      if (MODE & 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(v[4 * u + i], 0.127f, -3.0f));
          acc += p;
          v[4 * u + i] = p;
        }
        const f32x2_ev f = {v[4 * u], v[4 * u + 1]}, g = {v[4 * u + 2], v[4 * u + 3]};
        pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_ev)) ^
              __builtin_bit_cast(unsigned, __builtin_convertvector(g, bf16x2_ev));
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = acc + (float)pk;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += e[j][i];
  sink[blockIdx.x * kThreads + tid] = s;  // keeps every result live
  if (lane == 0) {
    unsigned long long* o = out + ((size_t)blockIdx.x * (kThreads / 64) + wave) * 2;
    o[0] = t1 - t0;
    o[1] = r1 - r0;
  }
}

template <int MODE>
hipError_t launch(void* out, void* sink, const void* rnd, int rnd_vecs, int grid, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_ceiling_kernel<MODE>, dim3(grid), dim3(kThreads), 0, st, (unsigned long long*)out,
                     (float*)sink, iters, (const u32x4*)rnd, rnd_vecs);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Buffer sizes for a launch of `grid` workgroups: `out` holds grid * 8 * 2
// uint64 (per wave: shader-clock ticks, 100 MHz ticks), `sink` grid * 512
// floats; `rnd` is any buffer of rnd_vecs >= 1 16-byte words of bf16 data
// (read modulo its size). Returns 0, 1 for an unknown mode or a bad
// argument, or 2 when the launch failed.
int tattn_probe_mfma_ceiling(int mode, void* out, void* sink, const void* rnd, int rnd_vecs, int grid, int iters,
                             void* stream) {
  if (out == nullptr || sink == nullptr || rnd == nullptr || rnd_vecs < 1 || grid < 1 || iters < 1) return 1;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (mode) {
    case 0: e = launch<0>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 1: e = launch<1>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 3: e = launch<3>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 5: e = launch<5>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 7: e = launch<7>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 9: e = launch<9>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 15: e = launch<15>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 19: e = launch<19>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 21: e = launch<21>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 33: e = launch<33>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 65: e = launch<65>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 97: e = launch<97>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 71: e = launch<71>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 129: e = launch<129>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    case 135: e = launch<135>(out, sink, rnd, rnd_vecs, grid, iters, st); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
