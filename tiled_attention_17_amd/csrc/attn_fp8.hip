// MXFP8 attention forward and the MXFP8 quantizer for gfx950.
//
// Format (CS336 Lecture 5 transcript, low-precision formats): E4M3 elements
// (4 exponent bits, 3 mantissa bits, largest finite 448) with one
// power-of-two scale, stored as a biased 8-bit exponent (E8M0), for every 32
// consecutive elements. A block's scale is the smallest power of two 2^e with
// amax <= 448 * 2^e (amax the block's largest magnitude), so nothing
// saturates. The blocks run along the reduction dimension of each product:
// along d for Q and K (S = Q K^T), along the keys for V (O = P V), which is
// why V is quantized into a transposed copy V^T [d, N] (the transcript's
// catch: an operand used transposed needs its own quantization).
//
// The forward maps straight onto v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x
// E4M3, two 32-element scale blocks per operand row). Its lane layout
// (measured on MI355X): lane l, half h = l / 32, byte j holds k =
// 32 (j / 16) + 16 h + (j % 16) of row l % 32; the scale of k-block b of a
// row comes from lane row + 32 b. Accordingly:
//   * a wave owns 32 queries and computes S^T = K Q^T (K from LDS, Q^T in
//     VGPRs) with the query in the lane, as the bf16 kernels do;
//   * K rows sit in LDS in the order kperm (bits 2 and 4:3 of the row
//     index rotated), which leaves key 32 c + 16 h + i in accumulator slot i
//     of block c: exactly byte 16 c + i of the next product's P^T operand,
//     so P never crosses lanes;
//   * P is itself quantized to MXFP8 in its two 32-key blocks: the block's
//     exponent comes from the block's largest score (a by-product of the row
//     maximum), is folded into the exponential's argument, and its scale
//     rides along in the product's B-scale operand; the row sum l adds the
//     unrounded fp32 values;
//   * K and V^T tiles (64 keys) go straight to LDS with buffer_load ... lds,
//     XOR-swizzled by 16-byte chunk so operand reads are conflict-free; the
//     scale bytes of a tile are staged into LDS beside them.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace tattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Marks x as used here (an empty asm reading its registers): work producing
// x stays above this point, which keeps the compiler from sinking it below
// a later wait. A plain device function: the host pass of a kernel template
// must not see the register constraint.
__device__ __forceinline__ void consume(const f32x16& x) { asm volatile("" ::"v"(x)); }

// ---------------------------------------------------------------------------
// quantizer
// ---------------------------------------------------------------------------

// E8M0 scale byte of a block with largest magnitude amax (bits of a
// non-negative float): the smallest e with amax <= 448 * 2^e, plus 127,
// clamped to 0..254. With amax = m 2^x (m in [1, 2)), e = x - 8 + (m > 1.75);
// zero and subnormal blocks get 0.
__device__ __forceinline__ unsigned mx_scale_code(unsigned amax_bits) {
  const int ex = (int)(amax_bits >> 23);
  if (ex == 0) return 0u;
  const int code = ex - 8 + ((amax_bits & 0x7fffff) > 0x600000 ? 1 : 0);
  return (unsigned)min(max(code, 0), 254);
}

// 2^(127 - code) as a float (the reciprocal of the block scale), code <= 253.
__device__ __forceinline__ float mx_inv_scale(unsigned code) {
  return __uint_as_float((254u - code) << 23);
}

// Four E4M3 bytes (round to nearest even) of four floats within +-448.
__device__ __forceinline__ unsigned pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Row-blocked: x [rows, cols] bf16 (cols % 32 == 0) -> q [rows, cols] E4M3
// and sc [rows, cols / 32]. One thread per 32-element block.
__global__ __launch_bounds__(256) void mx_quantize_rows_kernel(const bf16* __restrict__ x,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ sc,
                                                               int64_t blocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= blocks) return;
  float v[32];
  const u32x4* src = (const u32x4*)(x + b * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 t = as_bf16x8(src[c]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * c + e] = (float)t[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const unsigned code = mx_scale_code(__float_as_uint(amax));
  const float inv = mx_inv_scale(code);
  u32x4 o[2];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    o[w / 4][w % 4] = pack_e4m3x4(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv, v[4 * w + 3] * inv);
  u32x4* dst = (u32x4*)(q + b * 32);
  dst[0] = o[0];
  dst[1] = o[1];
  sc[b] = (uint8_t)code;
}

// Column-blocked and transposed: x [batch, rows, cols] bf16 (rows % 32 == 0)
// -> q [batch, cols, rows] E4M3 (q[c][r] = x[r][c] scaled) and
// sc [batch, cols, rows / 32]: each 32-row block of a column shares a scale.
// A workgroup takes a tile of TR = 128 rows x TC = 64 columns through LDS
// (16-byte loads, 8 threads per 128-byte row segment, when cols % 8 == 0;
// element loads otherwise). Thread t then owns
// column t / 4 and its 32-row block t % 4, so four adjacent threads write
// one 128-byte run of a q row.
constexpr int kQtTR = 128, kQtTC = 64;
__global__ __launch_bounds__(256) void mx_quantize_cols_t_kernel(const bf16* __restrict__ x,
                                                                 uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ sc, int rows,
                                                                 int cols, int row_tiles, int col_tiles) {
  constexpr int TR = kQtTR, TC = kQtTC, PITCH = TC + 8;  // 144-byte LDS rows, 16-byte aligned
  __shared__ __attribute__((aligned(16))) bf16 tile[TR * PITCH];
  // Column c of row r sits at c ^ swz(r): the four threads reading one column
  // (rows 32 apart, the same bank at this pitch) then hit four different
  // 16-byte slots; a 16-byte group of 8 columns stays contiguous.
  auto swz = [](int r) { return 8 * ((r >> 5) & 3); };
  const int per_batch = row_tiles * col_tiles;
  const int batch = blockIdx.x / per_batch;
  const int rem = blockIdx.x - batch * per_batch;
  const int rt = rem / col_tiles, ct = rem - rt * col_tiles;
  const int r0 = rt * TR, c0 = ct * TC;
  const bf16* xb = x + (size_t)batch * rows * cols;
  const int t = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < TR * TC / (8 * 256); ++pass) {
    const int r = pass * 32 + t / 8, cc = 8 * (t % 8);
    const bf16* src = xb + (size_t)(r0 + r) * cols + c0 + cc;
    bf16* dst = tile + r * PITCH + (cc ^ swz(r));
    if (cols % 8 == 0) {  // 16-byte aligned row segments
      u32x4 w = {0, 0, 0, 0};
      if (r0 + r < rows && c0 + cc < cols) w = *(const u32x4*)src;
      *(u32x4*)dst = w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = (r0 + r < rows && c0 + cc + e < cols) ? src[e] : (bf16)0.f;
    }
  }
  __syncthreads();
  const int c = t / 4, blk = t % 4;
  if (c0 + c >= cols || r0 + 32 * blk >= rows) return;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = (float)tile[(32 * blk + r) * PITCH + (c ^ swz(32 * blk))];
    amax = fmaxf(amax, fabsf(v[r]));
  }
  const unsigned code = mx_scale_code(__float_as_uint(amax));
  const float inv = mx_inv_scale(code);
  u32x4 o[2];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    o[w / 4][w % 4] = pack_e4m3x4(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv, v[4 * w + 3] * inv);
  uint8_t* qrow = q + ((size_t)batch * cols + c0 + c) * rows + r0 + 32 * blk;
  ((u32x4*)qrow)[0] = o[0];
  ((u32x4*)qrow)[1] = o[1];
  sc[((size_t)batch * cols + c0 + c) * (rows / 32) + r0 / 32 + blk] = (uint8_t)code;
}

hipError_t launch_mx_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols, bool transpose,
                              void* q, void* sc, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  if (!transpose) {
    const int64_t blocks = batch * rows * cols / 32;
    const int64_t wgs = (blocks + 255) / 256;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_quantize_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, st, (const bf16*)x,
                       (uint8_t*)q, (uint8_t*)sc, blocks);
  } else {
    const int64_t col_tiles = (cols + kQtTC - 1) / kQtTC;
    const int64_t row_tiles = (rows + kQtTR - 1) / kQtTR;
    const int64_t wgs = batch * row_tiles * col_tiles;
    if (wgs > INT32_MAX || rows > INT32_MAX || cols > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_quantize_cols_t_kernel, dim3((unsigned)wgs), dim3(256), 0, st, (const bf16*)x,
                       (uint8_t*)q, (uint8_t*)sc, (int)rows, (int)cols, (int)row_tiles, (int)col_tiles);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP8 attention forward
// ---------------------------------------------------------------------------
template <int D>
struct Fp8Tile {
  static constexpr int NW = 4;             // waves per workgroup (32 queries each)
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;            // keys per tile (one 64-deep value product)
  static constexpr int KT = BN * D;        // K tile bytes (rows of D bytes)
  static constexpr int VT = D * BN;        // V^T tile bytes (rows of 64 bytes)
  static constexpr int KSC = BN * 4;       // K scale bytes (4 per key row, D / 32 used)
  static constexpr int VSC = 2 * 32 * 4;   // V^T scale bytes, laid out [key block][d % 32][d / 32]
  static constexpr int STAGE = KT + VT + KSC + VSC;
  static constexpr int KS = D / 64;        // 64-deep steps of the score product
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int KCH = D / 16;       // 16-byte chunks per K row
};

// LDS row r of a 32-row K block holds key kperm(r): row bits [a1 a0 h e1 e0]
// carry key bits [h a1 a0 e1 e0], so accumulator slot 4a + e of lane half h
// (C row 8a + 4h + e) holds key 16h + 4a + e.
__device__ __forceinline__ int kperm(int r) {
  return (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}
// 16-byte chunk swizzles: a quarter wave reads 16 consecutive rows at one
// logical chunk; (row bits below the 256-byte period, chunk ^ swizzle) is
// distinct over them.
template <int D>
__device__ __forceinline__ int k8swz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
__device__ __forceinline__ int v8swz(int r) { return (r >> 2) & 3; }

// At least three waves per SIMD (168 VGPRs at D = 128): the step's serial
// chain (score MFMAs, softmax, P packing, value MFMAs, barrier) leaves the
// matrix core idle unless other waves fill in, and a third wave pays for the
// partial last round of workgroups it brings (headline shape: 188.6 us
// against 195.1 us with two waves).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void attn_fwd_mxfp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ QS,
                           const uint8_t* __restrict__ K8, const uint8_t* __restrict__ KS,
                           const uint8_t* __restrict__ VT8, const uint8_t* __restrict__ VTS,
                           bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles,
                           int total_tiles, float c, int remap) {
  using T = Fp8Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];
  auto kt_ = [&](int b) { return smem + b * T::STAGE; };
  auto vt_ = [&](int b) { return smem + b * T::STAGE + T::KT; };
  auto ks_ = [&](int b) { return smem + b * T::STAGE + T::KT + T::VT; };
  auto vs_ = [&](int b) { return smem + b * T::STAGE + T::KT + T::VT + T::KSC; };

  const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
  const int bh = __builtin_amdgcn_readfirstlane(tile / n_qtiles);
  const int qt = __builtin_amdgcn_readfirstlane(tile - (tile / n_qtiles) * n_qtiles);
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_row = qt * T::BM + wave * 32 + lq;
  const bool q_ok = q_row < N;
  const uint8_t* Kh = K8 + (size_t)bh * N * D;
  const uint8_t* VTh = VT8 + (size_t)bh * D * N;
  const uint8_t* KSh = KS + (size_t)bh * N * (D / 32);
  const uint8_t* VTSh = VTS + (size_t)bh * D * (N / 32);

  // Q^T operand and its scales: step s covers d 64 s .. 64 s + 63; this lane
  // holds d 64 s + 16 h + 0..15 (bytes 0..15) and 64 s + 32 + 16 h + 0..15
  // (bytes 16..31) and supplies the scale of d-block 2 s + h. (Every scale
  // operand below is a byte in bits 7:0 of its register: op_sel 0.)
  i32x8 qf[T::KS];
  int qsc[T::KS];
  {
    const uint8_t* qrow = Q8 + ((size_t)bh * N + q_row) * D;
    const uint8_t* qs = QS + ((size_t)bh * N + q_row) * (D / 32);
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
      u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      unsigned e = 127;
      if (q_ok) {
        a = *(const u32x4*)(qrow + 64 * s + 16 * h);
        b = *(const u32x4*)(qrow + 64 * s + 32 + 16 * h);
        e = qs[2 * s + h];
      }
      qf[s] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      qsc[s] = (int)e;
    }
  }

  // DMA lanes of the K tile: 1 KB instructions of 1024 / D rows; lane L
  // fills row r0 + L / KCH at chunk position L % KCH (logical chunk p ^ swz).
  constexpr int KRPI = 1024 / D, KNI = T::BN / KRPI / T::NW;
  constexpr int VRPI = 16, VNI = D / VRPI / T::NW;
  int kvoff[KNI], vvoff[VNI], vchunk[VNI];
#pragma unroll
  for (int i = 0; i < KNI; ++i) {
    const int r = (wave * KNI + i) * KRPI + lane / T::KCH;
    const int ch = (lane % T::KCH) ^ k8swz<D>(r);
    kvoff[i] = (32 * (r / 32) + kperm(r % 32)) * D + 16 * ch;
  }
#pragma unroll
  for (int i = 0; i < VNI; ++i) {
    const int r = (wave * VNI + i) * VRPI + lane / 4;
    vchunk[i] = (lane % 4) ^ v8swz(r);
    vvoff[i] = r * N + 16 * vchunk[i];
  }
  // Staging of tile j into buffer buf in two parts, so that no wait for
  // memory sits at the start of a step: stage_issue loads the scale bytes
  // into registers first and then sends K and V^T straight to LDS (the
  // compiler's wait for the scale loads then leaves the later LDS DMAs in
  // flight); stage_commit, after the step's work, writes the scale bytes.
  unsigned ksw = 0, vse = 127;  // this thread's K scale word and V^T scale byte
  auto stage_issue = [&](int j, int buf) {
    const int k0 = j * T::BN;
    if (tid < T::BN) {  // scale bytes: K [row][D/32] by LDS row
      const int key = k0 + 32 * (tid / 32) + kperm(tid % 32);
      ksw = 0;
      if (key < N) {
        if (D == 128) ksw = *(const unsigned*)(KSh + (size_t)key * 4);
        else ksw = *(const unsigned short*)(KSh + (size_t)key * 2);
      }
    }
    if (tid < 2 * D) {  // V^T [key block][d % 32][d / 32]
      const int d = tid >> 1, kb = j * 2 + (tid & 1);
      vse = kb * 32 < N ? VTSh[(size_t)d * (N / 32) + kb] : 127u;
    }
    const int krem = N > k0 ? (N - k0) * D : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + (size_t)k0 * D), 0, krem, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < KNI; ++i)
      lds_dma16(kr, (bf16*)(kt_(buf) + (wave * KNI + i) * 1024), kvoff[i]);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(VTh + k0), 0, D * N - k0, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < VNI; ++i) {
      const int off = k0 + 16 * vchunk[i] < N ? vvoff[i] : 0x7fffffff;  // keys past N: zeros
      lds_dma16(vr, (bf16*)(vt_(buf) + (wave * VNI + i) * 1024), off);
    }
  };
  auto stage_commit = [&](int buf) {
    if (tid < T::BN) *(unsigned*)(ks_(buf) + 4 * tid) = ksw;
    if (tid < 2 * D) {
      const int d = tid >> 1, blk = tid & 1;
      vs_(buf)[blk * 128 + (d % 32) * 4 + d / 32] = (uint8_t)vse;
    }
  };
  static_assert(2 * D <= 256, "one V^T scale byte per thread");

  // operand read offsets (bytes) within a tile
  int kro[2 * T::KS], vro[2];
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    kro[2 * s] = lq * D + 16 * ((4 * s + h) ^ k8swz<D>(lq));
    kro[2 * s + 1] = lq * D + 16 * ((4 * s + 2 + h) ^ k8swz<D>(lq));
  }
  vro[0] = lq * 64 + 16 * (h ^ v8swz(lq));
  vro[1] = lq * 64 + 16 * ((2 + h) ^ v8swz(lq));

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = (N + T::BN - 1) / T::BN;
  stage_issue(0, 0);
  stage_commit(0);
  wait_vmem();
  __syncthreads();

  // Only the last tile of a ragged N holds keys past N; the others run a
  // body without the per-element selects (the compiler would otherwise
  // if-convert them into every tile).
  auto body = [&](auto masked_t, int j) {
    constexpr bool masked = decltype(masked_t)::value;
    const int cur = j & 1;
    if (j + 1 < n_kt) stage_issue(j + 1, cur ^ 1);
    const uint8_t* kt = kt_(cur);
    const uint8_t* vt = vt_(cur);

    // S^T for the two 32-key blocks of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[cb][i] = 0.f;
      const uint8_t* krow = kt + 32 * cb * D;
      // the row's scale word; this lane supplies d-block 2 s + h of step s
      const unsigned kw = *(const unsigned*)(ks_(cur) + 4 * (32 * cb + lq));
#pragma unroll
      for (int s = 0; s < T::KS; ++s) {
        const u32x4 a = *(const u32x4*)(krow + kro[2 * s]);
        const u32x4 b = *(const u32x4*)(krow + kro[2 * s + 1]);
        const i32x8 kf = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        const int ksc = (int)((kw >> (8 * (2 * s + h))) & 0xffu);
        sacc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[s], sacc[cb], 0, 0, 0, ksc, 0,
                                                                   qsc[s]);
      }
    }

    // online softmax (Lecture 17 page §8.3), lazy running max, keys past N masked
    const int key0 = j * T::BN;
    if (masked) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + 32 * cb + 16 * h + i >= N) sacc[cb][i] = -INFINITY;
    }
    float bmax[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float mx = sacc[cb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[cb][i]);
      bmax[cb] = max_with_other_half(mx);  // both halves of a 32-key block
    }
    const float mx = fmaxf(bmax[0], bmax[1]);
    const float mt = mx == -INFINITY ? -INFINITY : mx * c;
    const float m_new = mt > m_run + 8.0f ? mt : m_run;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    // P in MXFP8: block cb's exponent e puts its largest p at [128, 256)
    int pe[2];
    i32x8 pw;
    float lsum = 0.f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float x = bmax[cb] == -INFINITY ? 0.f : bmax[cb] * c - m_ref;
      pe[cb] = min(max((int)floorf(x) - 7, -127), 127);
      const float off = m_ref + (float)pe[cb];
      float pv[16], ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = fast_exp2(fmaf(sacc[cb][i], c, -off));
        if (masked) pv[i] = sacc[cb][i] == -INFINITY ? 0.f : pv[i];
        ls += pv[i];
      }
      lsum += __builtin_amdgcn_ldexpf(ls, pe[cb]);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        pw[4 * cb + w] = (int)pack_e4m3x4(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
    }
    l_run = fmaf(alpha, l_run, lsum);
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    const int psc = (h ? pe[1] : pe[0]) + 127;  // this lane supplies key block h's scale

    // O^T += V^T P^T: one 64-deep product per 32-row block of d
    const unsigned vw = *(const unsigned*)(vs_(cur) + h * 128 + lq * 4);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const uint8_t* vrow = vt + 32 * db * 64;
      const u32x4 a = *(const u32x4*)(vrow + vro[0]);
      const u32x4 b = *(const u32x4*)(vrow + vro[1]);
      const i32x8 vf = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      const int vsc = (int)((vw >> (8 * db)) & 0xffu);
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pw, oacc[db], 0, 0, 0, vsc, 0, psc);
    }
    // The step's results are consumed here (an empty asm reading the
    // accumulators), so that the compiler keeps the step's work above the
    // waits for the staged tile instead of sinking it below them.
#pragma unroll
    for (int db = 0; db < T::DB; ++db) consume(oacc[db]);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < n_kt) stage_commit(cur ^ 1);
    wait_vmem();  // next tiles written to LDS
    __syncthreads();
  };
  const int n_full = N / T::BN;
  int j = 0;
  for (; j < n_full; ++j) body(std::false_type{}, j);
  if (j < n_kt) body(std::true_type{}, j);

  // O = o / l (bf16), LSE = ln 2 (m + log2 l)
  const float l_tot = add_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    bf16* orow = O + ((size_t)bh * N + q_row) * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
        *(u32x2*)(orow + 32 * db + 8 * r + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + q_row] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

hipError_t launch_attn_fwd_mxfp8(const Fp8Args& a) {
  constexpr int BM = 128;
  const int n_qtiles = (int)((a.N + BM - 1) / BM);
  const int64_t total = a.BH * n_qtiles;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  const int remap = total % 8 == 0 ? 1 : 0;
  const hipStream_t st = (hipStream_t)a.stream;
  const float c = a.scale * kLog2e;
  if (a.d == 64)
    hipLaunchKernelGGL(attn_fwd_mxfp8_kernel<64>, dim3((unsigned)total), dim3(256), 0, st,
                       (const uint8_t*)a.q8, (const uint8_t*)a.qs, (const uint8_t*)a.k8,
                       (const uint8_t*)a.ks, (const uint8_t*)a.vt8, (const uint8_t*)a.vts, (bf16*)a.o,
                       a.lse, (int)a.N, n_qtiles, (int)total, c, remap);
  else
    hipLaunchKernelGGL(attn_fwd_mxfp8_kernel<128>, dim3((unsigned)total), dim3(256), 0, st,
                       (const uint8_t*)a.q8, (const uint8_t*)a.qs, (const uint8_t*)a.k8,
                       (const uint8_t*)a.ks, (const uint8_t*)a.vt8, (const uint8_t*)a.vts, (bf16*)a.o,
                       a.lse, (int)a.N, n_qtiles, (int)total, c, remap);
  return hipGetLastError();
}

}  // namespace tattn
