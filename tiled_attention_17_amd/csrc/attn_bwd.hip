// Fused attention backward for gfx950 (bf16 storage, fp32 accumulation).
//
// Method: the backward pass keeps no N x N matrix and recomputes the score
// and probability tiles from Q, K and the saved LSE (CS336 Lecture 5 notes
// "GPU 架构与大模型高效计算" §7.2 item 3, Recomputation; CS336 2026 Lecture 05
// note, "FlashAttention 解析" ②). The gradients are the exact derivative of
// O = softmax(scale Q K^T) V for the loss sum(O * dO):
//   P = exp(scale S - LSE), dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
//   dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches on the caller's stream, no atomics (deterministic):
//   1. row_dot:  D_i = sum_k dO_ik O_ik (memory-bound, one pass over O, dO);
//   2. dkdv:     one workgroup per 32*NW keys; each wave keeps its 32 keys of
//                K and V in VGPRs and sweeps all query tiles (64 queries per
//                step, Q/dO/LSE/D staged in LDS, double-buffered), computing
//                S = Q K^T and dP = dO V^T with the key in the lane (MFMA C
//                layout) so that P and dS feed dV^T += dO^T P and
//                dK^T += Q^T dS directly as B operands; dO^T and Q^T come from
//                ds_read_b64_tr_b16 transposed LDS reads;
//   3. dq:       one workgroup per 32*NW queries; each wave keeps Q and dO of
//                its 32 queries in VGPRs and sweeps all key tiles, computing
//                S^T = K Q^T and dP^T = V dO^T with the query in the lane, then
//                dQ^T += K^T dS^T (K^T via transposed LDS reads).
// The recomputation of S, P and dP in both sweeps trades extra MFMA work for
// never storing dS or taking atomics on dQ.
#include "device_common.h"
#include "launch.h"

namespace tattn {

constexpr int kBwdBlk = 64;  // rows per streamed tile (queries in dkdv, keys in dq)

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_rowdot_kernel(const bf16* __restrict__ O,
                                                              const bf16* __restrict__ dO,
                                                              float* __restrict__ Dv,
                                                              int64_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements (16 bytes) each
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    u32x4 a = *(const u32x4*)(O + row * D + part * 8);
    u32x4 b = *(const u32x4*)(dO + row * D + part * 8);
    bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV
// ---------------------------------------------------------------------------
template <int D, int NW>
struct DkdvCfg {
  static constexpr int BKV = 32 * NW;          // keys per workgroup
  static constexpr int BQ = kBwdBlk;           // queries per step
  static constexpr int PITCH = D + 8;
  static constexpr int TILE = BQ * PITCH;
  static constexpr int THREADS = NW * 64;
  static constexpr int CHUNKS = BQ * D / 8;
  static constexpr int CPT = CHUNKS / THREADS;
  static constexpr int DK = D / 16;
  static constexpr int DB = D / 32;
  static_assert(CHUNKS % THREADS == 0, "tile must split evenly");
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int n_ktiles, int total_tiles, float c,
    float scale, int remap) {
  using C = DkdvCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * C::TILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][C::BQ];  // [buf][lse2 | D][query]
  // stage b: Q tile at smem + 2 b TILE, dO tile right after it
  auto qs = [&](int b) { return smem + 2 * b * C::TILE; };
  auto ds = [&](int b) { return smem + (2 * b + 1) * C::TILE; };

  const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
  const int bh = tile / n_ktiles;
  const int kt = tile - bh * n_ktiles;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lk = lane & 31, h = lane >> 5;
  const int key = kt * C::BKV + wave * 32 + lk;  // the key this lane owns
  const bool k_ok = key < N;

  // K^T and V^T as B operands: lane (key lk, half h) holds d = 16 s + 8 h .. +7.
  bf16x8 kf[C::DK], vf[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (k_ok) {
      x = *(const u32x4*)(K + base + (size_t)key * D + 16 * s + 8 * h);
      y = *(const u32x4*)(V + base + (size_t)key * D + 16 * s + 8 * h);
    }
    kf[s] = as_bf16x8(x);
    vf[s] = as_bf16x8(y);
  }

  u32x4 qreg[C::CPT], dreg[C::CPT];
  float sreg = 0.f;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8, q = j * C::BQ + row;
      u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (q < N) {
        a = *(const u32x4*)(Q + base + (size_t)q * D + col);
        b = *(const u32x4*)(dO + base + (size_t)q * D + col);
      }
      qreg[i] = a;
      dreg[i] = b;
    }
    if (tid < 2 * C::BQ) {
      const int q = j * C::BQ + (tid % C::BQ);
      if (tid < C::BQ)
        sreg = q < N ? LSE[(size_t)bh * N + q] * kLog2e : INFINITY;  // P = 0 past N
      else
        sreg = q < N ? Dv[(size_t)bh * N + q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(u32x4*)(qs(buf) + swap23(row) * C::PITCH + col) = qreg[i];
      *(u32x4*)(ds(buf) + swap23(row) * C::PITCH + col) = dreg[i];
    }
    if (tid < 2 * C::BQ) stat[buf][tid / C::BQ][tid % C::BQ] = sreg;
  };

  f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[db][i] = dvacc[db][i] = 0.f;

  const int g = lane >> 4, j16 = lane & 15;
  const int tr_col = 16 * (g & 1) + 4 * (j16 & 3);
  const int tr_row = 4 * h + (j16 >> 2);  // LDS row of query 16t + 8h + e is 16t + 4h + e (e < 4)

  const int n_qt = (N + C::BQ - 1) / C::BQ;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_qt; ++j) {
    const int cur = j & 1;
    if (j + 1 < n_qt) load_tile(j + 1);

    unsigned pk[2][8], dsk[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
      const bf16* qp = qs(cur) + (32 * qb + lk) * C::PITCH + 8 * h;
      const bf16* dp = ds(cur) + (32 * qb + lk) * C::PITCH + 8 * h;
#pragma unroll
      for (int s = 0; s < C::DK; ++s) {
        sacc = mfma32x32x16(as_bf16x8(*(const u32x4*)(qp + 16 * s)), kf[s], sacc);
        dpacc = mfma32x32x16(as_bf16x8(*(const u32x4*)(dp + 16 * s)), vf[s], dpacc);
      }
      // slot i holds query 32 qb + 16 (i/8) + 8 h + i%8 (of this tile) for key lk.
      const float* lse2 = stat[cur][0] + 32 * qb + 8 * h;
      const float* drow = stat[cur][1] + 32 * qb + 8 * h;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int qi = 16 * (i >> 3) + (i & 7);
        const float p0 = fast_exp2(fmaf(sacc[i], c, -lse2[qi]));
        const float p1 = fast_exp2(fmaf(sacc[i + 1], c, -lse2[qi + 1]));
        const float s0 = p0 * (dpacc[i] - drow[qi]);
        const float s1 = p1 * (dpacc[i + 1] - drow[qi + 1]);
        pk[qb][i >> 1] = pack_bf16x2(p0, p1);
        dsk[qb][i >> 1] = pack_bf16x2(s0, s1);
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS over 4 steps of 16 queries.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 pw = {pk[t >> 1][4 * (t & 1)], pk[t >> 1][4 * (t & 1) + 1],
                        pk[t >> 1][4 * (t & 1) + 2], pk[t >> 1][4 * (t & 1) + 3]};
      const u32x4 sw = {dsk[t >> 1][4 * (t & 1)], dsk[t >> 1][4 * (t & 1) + 1],
                        dsk[t >> 1][4 * (t & 1) + 2], dsk[t >> 1][4 * (t & 1) + 3]};
      const bf16* dtp = ds(cur) + (16 * t + tr_row) * C::PITCH + tr_col;
      const bf16* qtp = qs(cur) + (16 * t + tr_row) * C::PITCH + tr_col;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 a = lds_read_tr_pair(dtp + 32 * db, dtp + 8 * C::PITCH + 32 * db);
        dvacc[db] = mfma32x32x16(a, as_bf16x8(pw), dvacc[db]);
        const bf16x8 b = lds_read_tr_pair(qtp + 32 * db, qtp + 8 * C::PITCH + 32 * db);
        dkacc[db] = mfma32x32x16(b, as_bf16x8(sw), dkacc[db]);
      }
    }

    if (j + 1 < n_qt) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (k_ok) {
    bf16* dkrow = dK + base + (size_t)key * D;
    bf16* dvrow = dV + base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dkacc[db][4 * r] * scale, dkacc[db][4 * r + 1] * scale);
        wk[1] = pack_bf16x2(dkacc[db][4 * r + 2] * scale, dkacc[db][4 * r + 3] * scale);
        wv[0] = pack_bf16x2(dvacc[db][4 * r], dvacc[db][4 * r + 1]);
        wv[1] = pack_bf16x2(dvacc[db][4 * r + 2], dvacc[db][4 * r + 3]);
        *(u32x2*)(dkrow + 32 * db + 8 * r + 4 * h) = wk;
        *(u32x2*)(dvrow + 32 * db + 8 * r + 4 * h) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
template <int D, int NW>
struct DqCfg {
  static constexpr int BM = 32 * NW;
  static constexpr int BN = kBwdBlk;
  static constexpr int PITCH = D + 8;
  static constexpr int TILE = BN * PITCH;
  static constexpr int THREADS = NW * 64;
  static constexpr int CHUNKS = BN * D / 8;
  static constexpr int CPT = CHUNKS / THREADS;
  static constexpr int DK = D / 16;
  static constexpr int DB = D / 32;
  static_assert(CHUNKS % THREADS == 0, "tile must split evenly");
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dQ, int N, int n_qtiles, int total_tiles, float c, float scale,
    int remap) {
  using C = DqCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * C::TILE];
  // stage b: K tile at smem + 2 b TILE, V tile right after it
  auto ks = [&](int b) { return smem + 2 * b * C::TILE; };
  auto vs = [&](int b) { return smem + (2 * b + 1) * C::TILE; };

  const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int q_row = qt * C::BM + wave * 32 + lq;
  const bool q_ok = q_row < N;

  bf16x8 qf[C::DK], dof[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (q_ok) {
      x = *(const u32x4*)(Q + base + (size_t)q_row * D + 16 * s + 8 * h);
      y = *(const u32x4*)(dO + base + (size_t)q_row * D + 16 * s + 8 * h);
    }
    qf[s] = as_bf16x8(x);
    dof[s] = as_bf16x8(y);
  }
  const float lse2 = q_ok ? LSE[(size_t)bh * N + q_row] * kLog2e : INFINITY;
  const float drow = q_ok ? Dv[(size_t)bh * N + q_row] : 0.f;

  u32x4 kreg[C::CPT], vreg[C::CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8, kk = j * C::BN + row;
      u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (kk < N) {
        a = *(const u32x4*)(K + base + (size_t)kk * D + col);
        b = *(const u32x4*)(V + base + (size_t)kk * D + col);
      }
      kreg[i] = a;
      vreg[i] = b;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(u32x4*)(ks(buf) + swap23(row) * C::PITCH + col) = kreg[i];
      *(u32x4*)(vs(buf) + swap23(row) * C::PITCH + col) = vreg[i];
    }
  };

  f32x16 dqacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  const int g = lane >> 4, j16 = lane & 15;
  const int tr_col = 16 * (g & 1) + 4 * (j16 & 3);
  const int tr_row = 4 * h + (j16 >> 2);

  const int n_kt = (N + C::BN - 1) / C::BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    const int cur = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    const bool ragged = (j + 1) * C::BN > N;

    unsigned dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
      const bf16* kp = ks(cur) + (32 * kb + lq) * C::PITCH + 8 * h;
      const bf16* vp = vs(cur) + (32 * kb + lq) * C::PITCH + 8 * h;
#pragma unroll
      for (int s = 0; s < C::DK; ++s) {
        sacc = mfma32x32x16(as_bf16x8(*(const u32x4*)(kp + 16 * s)), qf[s], sacc);
        dpacc = mfma32x32x16(as_bf16x8(*(const u32x4*)(vp + 16 * s)), dof[s], dpacc);
      }
      // slot i holds key j*64 + 32 kb + 16 (i/8) + 8 h + i%8 for query lq.
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = fast_exp2(fmaf(sacc[i], c, -lse2));
        float p1 = fast_exp2(fmaf(sacc[i + 1], c, -lse2));
        if (ragged) {
          const int k0 = j * C::BN + 32 * kb + 16 * (i >> 3) + 8 * h + (i & 7);
          if (k0 >= N) p0 = 0.f;
          if (k0 + 1 >= N) p1 = 0.f;
        }
        dsk[kb][i >> 1] = pack_bf16x2(p0 * (dpacc[i] - drow), p1 * (dpacc[i + 1] - drow));
      }
    }

    // dQ^T += K^T dS^T over 4 steps of 16 keys.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 sw = {dsk[t >> 1][4 * (t & 1)], dsk[t >> 1][4 * (t & 1) + 1],
                        dsk[t >> 1][4 * (t & 1) + 2], dsk[t >> 1][4 * (t & 1) + 3]};
      const bf16* ktp = ks(cur) + (16 * t + tr_row) * C::PITCH + tr_col;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 a = lds_read_tr_pair(ktp + 32 * db, ktp + 8 * C::PITCH + 32 * db);
        dqacc[db] = mfma32x32x16(a, as_bf16x8(sw), dqacc[db]);
      }
    }

    if (j + 1 < n_kt) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (q_ok) {
    bf16* row = dQ + base + (size_t)q_row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(dqacc[db][4 * r] * scale, dqacc[db][4 * r + 1] * scale);
        w[1] = pack_bf16x2(dqacc[db][4 * r + 2] * scale, dqacc[db][4 * r + 3] * scale);
        *(u32x2*)(row + 32 * db + 8 * r + 4 * h) = w;
      }
  }
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  const hipStream_t st = (hipStream_t)a.stream;
  const float c = a.scale * kLog2e;
  const int64_t rows = a.BH * a.N;
  {
    constexpr int rows_per_block = 256 / (D / 8);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_rowdot_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const bf16*)a.o, (const bf16*)a.dout, a.row_dot, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = 4;
    const int n_kt = (int)((a.N + 32 * NW - 1) / (32 * NW));
    const int64_t total = a.BH * n_kt;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NW>), dim3((unsigned)total), dim3(NW * 64), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.row_dot, (bf16*)a.dk, (bf16*)a.dv, (int)a.N, n_kt, (int)total, c,
                       a.scale, (int)(total % 8 == 0));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = 4;
    const int n_qt = (int)((a.N + 32 * NW - 1) / (32 * NW));
    const int64_t total = a.BH * n_qt;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NW>), dim3((unsigned)total), dim3(NW * 64), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.row_dot, (bf16*)a.dq, (int)a.N, n_qt, (int)total, c, a.scale,
                       (int)(total % 8 == 0));
    return hipGetLastError();
  }
}

hipError_t launch_attn_bwd(const BwdArgs& a) {
  return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a);
}

}  // namespace tattn
