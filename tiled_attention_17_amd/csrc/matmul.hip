// Matrix product C = A B^T for gfx950: bf16 operands, fp32 accumulation,
// bf16 result (round to nearest even).
//
// The Lecture 17 page §2.1 defines C_ij = sum_k A_ik B_kj and §5.2-§5.3
// describe the tiled GEMM: a workgroup loads one tile of each operand into
// on-chip memory, accumulates the partial products of a C tile in registers
// while it walks the reduction dimension, and writes the C tile once. Here B
// is given as [N, K] (both operands contiguous along k, as Q and K are in
// S = Q K^T). The kernel exists to measure how throughput depends on the
// matrix size on 256 compute units: a C tile is the unit of work, and tiles
// beyond a whole number of rounds over the units leave most of the chip idle
// (wave quantization, CS336 Lecture 5 notes §6.2).
//
// MI355X mapping:
//   * one workgroup = 4 waves = one 128 x 128 C tile; wave (wm, wn) owns the
//     64 x 64 quarter (wm, wn) as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16;
//   * the MFMA's A operand is a 32-row block of B and its B operand a 32-row
//     block of A, so the fp32 accumulator holds, per lane, one row m of C and
//     4 consecutive columns n per slot group: C is written 8 bytes at a time;
//   * per 64-wide step of k, both 128 x 64 operand tiles go straight from
//     HBM/L2 to LDS with buffer_load ... lds (1 KB per instruction, no VGPR
//     staging), double-buffered (64 KiB of LDS per workgroup, two workgroups
//     per compute unit); each tile has a buffer resource of its own, so rows
//     past M or N read as zeros through the range check, and chunks past K
//     are given an out-of-range offset;
//   * tile rows are 128 bytes; chunk c of row r sits at chunk position
//     c ^ gswz(r), which keeps the operand reads (16 consecutive rows at one
//     chunk per quarter wave) free of bank conflicts without padding.
#include "device_common.h"
#include "launch.h"

namespace tattn {

struct GemmCfg {
  static constexpr int BM = 128;          // rows of C (of A) per workgroup
  static constexpr int BN = 128;          // columns of C (rows of B) per workgroup
  static constexpr int BK = 64;           // reduction step
  static constexpr int THREADS = 256;     // 4 waves, 2 x 2 over the tile
  static constexpr int TILE = 128 * BK;   // bf16 elements of one operand tile
  static constexpr int STAGE = 2 * TILE;  // A tile then B tile
  static constexpr int NI = 128 * BK * 2 / 1024 / 4;  // 1 KB DMA instructions per wave per operand
};

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void matmul_nt_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B,
                           bf16* __restrict__ C, int M, int N, int K, int tiles_n, int total_tiles,
                           int remap) {
  using G = GemmCfg;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * G::STAGE];

  const int t = xcd_tile(blockIdx.x, total_tiles, remap);
  const int tm = __builtin_amdgcn_readfirstlane(t / tiles_n);
  const int tn = __builtin_amdgcn_readfirstlane(t - (t / tiles_n) * tiles_n);
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // DMA lanes: instruction i of this wave fills tile rows 8 (4 wave + i) .. +7;
  // lane L writes row + L / 8 at chunk position L % 8 (logical chunk p ^ gswz).
  int voff[G::NI], chunk[G::NI];
#pragma unroll
  for (int i = 0; i < G::NI; ++i) {
    const int r = 8 * (G::NI * wave + i) + lane / 8;
    chunk[i] = (lane % 8) ^ gswz(r);
    voff[i] = (r * K + 8 * chunk[i]) * 2;
  }
  // Rows of an operand matrix with `rows` rows from tile row r0, columns from k0.
  auto stage = [&](const bf16* X, int rows, int r0, int k0, bf16* tile) {
    const int rem = (rows - r0) * K - k0;  // elements from the tile's first element to the end
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + (size_t)r0 * K + k0), 0, rem * 2, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int off = k0 + 8 * chunk[i] < K ? voff[i] : 0x7fffffff;  // past K: zeros
      lds_dma16(rs, tile + 8 * (G::NI * wave + i) * G::BK, off);
    }
  };
  auto a_tile = [&](int b) { return smem + b * G::STAGE; };
  auto b_tile = [&](int b) { return smem + b * G::STAGE + G::TILE; };

  // operand read offsets: row lq of a 32-row block, logical chunk 2 s + h
  int ro[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ro[s] = lq * G::BK + 8 * ((2 * s + h) ^ gswz(lq));

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int n_k = (K + G::BK - 1) / G::BK;
  stage(A, M, m0, 0, a_tile(0));
  stage(B, N, n0, 0, b_tile(0));
  wait_vmem();
  __syncthreads();

  for (int kt = 0; kt < n_k; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_k) {
      stage(A, M, m0, (kt + 1) * G::BK, a_tile(cur ^ 1));
      stage(B, N, n0, (kt + 1) * G::BK, b_tile(cur ^ 1));
    }
    const bf16* at = a_tile(cur) + (64 * wm) * G::BK;
    const bf16* bt = b_tile(cur) + (64 * wn) * G::BK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 x[2], y[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        x[j] = as_bf16x8(*(const u32x4*)(bt + 32 * j * G::BK + ro[s]));
        y[j] = as_bf16x8(*(const u32x4*)(at + 32 * j * G::BK + ro[s]));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32x32x16(x[nb], y[mb], acc[nb][mb]);
    }
    wait_vmem();  // next tiles written to LDS
    __syncthreads();
  }

  // lane: row m of C; slot group r: columns n .. n + 3
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 64 * wm + 32 * mb + lq;
    if (m >= M) continue;
    bf16* crow = C + (size_t)m * N;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 64 * wn + 32 * nb + 8 * r + 4 * h;
        const f32x16& c = acc[nb][mb];
        if (vec && n + 3 < N) {
          u32x2 w;
          w[0] = pack_bf16x2(c[4 * r], c[4 * r + 1]);
          w[1] = pack_bf16x2(c[4 * r + 2], c[4 * r + 3]);
          *(u32x2*)(crow + n) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) crow[n + e] = (bf16)c[4 * r + e];
        }
      }
  }
}

hipError_t launch_matmul_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                            void* stream) {
  const int64_t tiles_m = (M + GemmCfg::BM - 1) / GemmCfg::BM;
  const int64_t tiles_n = (N + GemmCfg::BN - 1) / GemmCfg::BN;
  const int64_t total = tiles_m * tiles_n;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(matmul_nt_bf16_kernel, dim3((unsigned)total), dim3(GemmCfg::THREADS), 0,
                     (hipStream_t)stream, (const bf16*)a, (const bf16*)b, (bf16*)c, (int)M, (int)N,
                     (int)K, (int)tiles_n, (int)total, (int)(total % 8 == 0));
  return hipGetLastError();
}

}  // namespace tattn
