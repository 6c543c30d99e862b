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
//   2. dkdv:     one workgroup per 128 keys; each wave keeps K^T and V^T of
//                its 32 keys in VGPRs and sweeps the query tiles (64 queries
//                per step, Q/dO/LSE/D staged in LDS, double-buffered),
//                computing S = Q K^T and dP = dO V^T with the key in the lane
//                so that P and dS feed dV^T += dO^T P and dK^T += Q^T dS as B
//                operands; dO^T and Q^T come from ds_read_b64_tr_b16
//                transposed LDS reads;
//   3. dq:       one workgroup per 256 queries; each wave keeps Q^T and dO^T
//                of its 32 queries in VGPRs and sweeps the key tiles,
//                computing S^T = K Q^T and dP^T = V dO^T with the query in
//                the lane, then dQ^T += K^T dS^T.
// The dQ sweep uses the forward's tile shapes (tile_common.h): K and V go
// straight to LDS with buffer_load ... lds, K^T is transposed in registers
// while staging, so every MFMA operand read is one ds_read_b128. (The same
// treatment of the dK/dV sweep, with Q^T and dO^T transposed while staging,
// measured 2 % slower there: that kernel runs one wave per SIMD and is bound
// by its serial vector work, not by the transposed reads.) The
// recomputation of S, P and dP in both sweeps trades extra MFMA work for
// never storing dS or taking atomics on dQ.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace tattn {

constexpr int kBwdBlk = 64;  // queries per streamed tile of the dK/dV sweep


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

// Query tiles a dK/dV workgroup needs under the causal mask (query i sees
// key j iff j <= i + Nk - Nq): from the first query that sees the tile's
// first key; tiles before j_full hold a (query, key) pair the mask hides.
// A key tile's mask edge spans at most BKV - 1 + BQ - 1 query positions, so
// at most kMaxMaskedSteps query tiles are masked (3 for 128 keys, 64 queries).
constexpr int kMaxMaskedSteps = 3;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int Nq, int Nk, int BH, int n_ktiles,
    int total_tiles, float c, float scale, int causal, int remap) {
  using C = DkdvCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * C::TILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][C::BQ];  // [buf][lse2 | D][query]
  // stage b: Q tile at smem + 2 b TILE, dO tile right after it
  auto qs = [&](int b) { return smem + 2 * b * C::TILE; };
  auto ds = [&](int b) { return smem + (2 * b + 1) * C::TILE; };

  // Causal launches take the key tiles that see the most queries (the
  // first ones) first; others keep one head's tiles on one XCD.
  int bh, kt;
  if (causal) {
    kt = (int)blockIdx.x / BH;
    bh = (int)blockIdx.x - kt * BH;
  } else {
    const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
    bh = tile / n_ktiles;
    kt = tile - bh * n_ktiles;
  }
  bh = __builtin_amdgcn_readfirstlane(bh);
  kt = __builtin_amdgcn_readfirstlane(kt);
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const int tid = threadIdx.x, lane = tid & 63, lk = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int key = kt * C::BKV + wave * 32 + lk;  // the key this lane owns
  const bool k_ok = key < Nk;
  const int off = Nk - Nq;
  const int k_lo = kt * C::BKV, k_hi = min(k_lo + C::BKV, Nk) - 1;
  const int j0 = causal ? max(0, k_lo - off) / C::BQ : 0;
  const int j_full = causal ? max(0, (k_hi - off + C::BQ - 1) / C::BQ) : 0;

  // K^T and V^T as B operands: lane (key lk, half h) holds d = 16 s + 8 h .. +7.
  bf16x8 kf[C::DK], vf[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (k_ok) {
      x = *(const u32x4*)(K + kbase + (size_t)key * D + 16 * s + 8 * h);
      y = *(const u32x4*)(V + kbase + (size_t)key * D + 16 * s + 8 * h);
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
      if (q < Nq) {
        a = *(const u32x4*)(Q + qbase + (size_t)q * D + col);
        b = *(const u32x4*)(dO + qbase + (size_t)q * D + col);
      }
      qreg[i] = a;
      dreg[i] = b;
    }
    if (tid < 2 * C::BQ) {
      const int q = j * C::BQ + (tid % C::BQ);
      if (tid < C::BQ)
        sreg = q < Nq ? LSE[(size_t)bh * Nq + q] * kLog2e : INFINITY;  // P = 0 past Nq
      else
        sreg = q < Nq ? Dv[(size_t)bh * Nq + q] : 0.f;
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

  const int n_qt = (Nq + C::BQ - 1) / C::BQ;
  auto step = [&](auto masked, int j) {
    constexpr bool MASKED = decltype(masked)::value;
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
        float p0 = fast_exp2(fmaf(sacc[i], c, -lse2[qi]));
        float p1 = fast_exp2(fmaf(sacc[i + 1], c, -lse2[qi + 1]));
        if (MASKED) {  // hidden pairs (key > query + Nk - Nq) get P = 0
          const int q0 = j * C::BQ + 32 * qb + 8 * h + qi;
          p0 = key > q0 + off ? 0.f : p0;
          p1 = key > q0 + 1 + off ? 0.f : p1;
        }
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
  };

  if (j0 < n_qt) {
    load_tile(j0);
    store_tile(j0 & 1);
    __syncthreads();
  }
  int j = j0;
#pragma unroll
  for (int m = 0; m < kMaxMaskedSteps; ++m)
    if (j < min(j_full, n_qt)) step(std::true_type{}, j++);
  for (; j < n_qt; ++j) step(std::false_type{}, j);

  if (k_ok) {
    bf16* dkrow = dK + kbase + (size_t)key * D;
    bf16* dvrow = dV + kbase + (size_t)key * D;
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
// One workgroup per 256 queries: 8 waves of 32 queries, two per SIMD. Each
// wave keeps Q^T and dO^T of its queries in VGPRs (B operands) and sweeps the
// key tiles of 64 keys, with the query in the lane throughout:
//   S^T = K Q^T and dP^T = V dO^T   (K, V row-major in LDS, as the forward's
//                                     K tile: rows at swap23(key), chunks
//                                     swizzled; staged with buffer_load ... lds)
//   P^T = 2^(c S^T - LSE2), dS^T = P^T (dP^T - D)   (LSE2 and D per lane)
//   dQ^T += K^T dS^T                 (K^T staged transposed in LDS, as the
//                                     forward's V^T tile, by a register
//                                     transpose; read with ds_read_b128)
// so every MFMA operand read is one ds_read_b128 and no transposed LDS read
// is needed. dQ = scale dQ^T^T at the end.
template <int D>
struct DqTile {
  static constexpr int NW = 8;
  static constexpr int BM = 32 * NW;
  using T = FwdTile<D, 64>;
  static constexpr int STAGE = 3 * T::KTILE;  // K rows, V rows, K^T
};

template <bool MASKED, int D>
__device__ __forceinline__ void dq_scores_to_ds(const f32x16* sacc, const f32x16* dpacc, float c,
                                                float lse2, float drow, int key0, int kmax, int h,
                                                u32x4* pw) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      // slot i of block kb: key key0 + 32 kb + 16 (i/8) + 8 h + i%8
      float p0 = fast_exp2(fmaf(sacc[kb][i], c, -lse2));
      float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -lse2));
      if (MASKED) {
        const int k = key0 + 32 * kb + 16 * (i >> 3) + 8 * h + (i & 7);
        p0 = k > kmax ? 0.f : p0;
        p1 = k + 1 > kmax ? 0.f : p1;
      }
      pw[2 * kb + (i >> 3)][(i & 7) >> 1] =
          pack_bf16x2(p0 * (dpacc[kb][i] - drow), p1 * (dpacc[kb][i + 1] - drow));
    }
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                        const bf16* __restrict__ V, const bf16* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ Dv,
                        bf16* __restrict__ dQ, int Nq, int Nk, int BH, int n_qtiles, int total_tiles,
                        float c, float scale, int causal, int remap) {
  using C = DqTile<D>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];
  auto ks = [&](int b) { return smem + b * C::STAGE; };
  auto vs = [&](int b) { return smem + b * C::STAGE + T::KTILE; };
  auto kts = [&](int b) { return smem + b * C::STAGE + 2 * T::KTILE; };

  // Causal launches take the query tiles that see the most keys (the last
  // ones) first; others keep one head's tiles on one XCD.
  int bh, qt;
  if (causal) {
    const int r = (int)blockIdx.x / BH;
    bh = (int)blockIdx.x - r * BH;
    qt = n_qtiles - 1 - r;
  } else {
    const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
    bh = tile / n_qtiles;
    qt = tile - bh * n_qtiles;
  }
  bh = __builtin_amdgcn_readfirstlane(bh);
  qt = __builtin_amdgcn_readfirstlane(qt);
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const bf16* Kh = K + kbase;
  const bf16* Vh = V + kbase;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc<D>(Kh, Nk);
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_row = qt * C::BM + wave * 32 + lq;
  const bool q_ok = q_row < Nq;
  // Keys this tile's queries see: up to the last query's causal window;
  // tiles from n_full on hold a key some query of the tile may not see.
  const int off = Nk - Nq;
  const int q_lo = qt * C::BM, q_hi = min(q_lo + C::BM, Nq) - 1;
  const int lim = causal ? min(Nk, q_hi + off + 1) : Nk;
  const int n_kt = lim > 0 ? (lim + 63) / 64 : 0;
  const int all_see = causal ? min(Nk, q_lo + off + 1) : Nk;
  const int n_full = all_see > 0 ? all_see / 64 : 0;
  const int kmax = causal ? min(Nk - 1, q_row + off) : Nk - 1;

  bf16x8 qf[T::DK], dof[T::DK];
  load_q<D>(Q + qbase + (size_t)q_row * D, q_ok, h, qf);
  load_q<D>(dO + qbase + (size_t)q_row * D, q_ok, h, dof);
  // A query that sees no key has LSE = -inf; all its keys are masked.
  const float lse2 = q_ok ? LSE[(size_t)bh * Nq + q_row] * kLog2e : INFINITY;
  const float drow = q_ok ? Dv[(size_t)bh * Nq + q_row] : 0.f;

  const VtOffsets vo(lq, h);
  const KOffsets<D, true> ko(lq, h);
  const KDirect<D, 64, C::NW> kd(0, wave, lane);
  Stager<D, 64, 512, 64, false> st;  // K^T through registers
  auto stage_direct = [&](int j, int buf) {
    kd.load(Kh, Nk, j, 64, ks(buf));
    kd.load(Vh, Nk, j, 64, vs(buf));
  };

  f32x16 dqacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  if (n_kt > 0) {
    stage_direct(0, 0);
    st.load(krs, krs, 0, 0, 0, tid);
    st.store(ks(0), kts(0), 0, tid);
    wait_vmem();
    __syncthreads();
  }
  auto step = [&](auto masked, int j) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = j & 1;
    const bool more = j + 1 < n_kt;
    if (more) {
      stage_direct(j + 1, cur ^ 1);
      st.load(krs, krs, j + 1, j + 1, 0, tid);
    }
    f32x16 sacc[2], dpacc[2];
    score_tile<D>(ks(cur), qf, ko, sacc);
    score_tile<D>(vs(cur), dof, ko, dpacc);
    u32x4 pw[4];
    dq_scores_to_ds<MASKED, D>(sacc, dpacc, c, lse2, drow, j * 64, kmax, h, pw);
    if (more) st.store(ks(cur ^ 1), kts(cur ^ 1), 0, tid);
    pv_tile<D>(kts(cur), pw, vo, dqacc);  // dQ^T += K^T dS^T
    wait_vmem();
    __syncthreads();
  };
  // Key tiles from n_full on are masked (a 256-query tile's mask edge spans
  // up to five 64-key tiles; they run in a loop of their own).
  const int n_plain = min(n_full, n_kt);
  int j = 0;
  for (; j < n_plain; ++j) step(std::false_type{}, j);
  for (; j < n_kt; ++j) step(std::true_type{}, j);

  if (q_ok) {
    bf16* row = dQ + qbase + (size_t)q_row * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
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
  // With no query, the dK/dV kernel alone runs (it writes zeros); with no
  // key, the dQ kernel alone runs (likewise).
  const int64_t rows = a.BH * a.Nq;
  if (rows > 0) {
    constexpr int rows_per_block = 256 / (D / 8);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_rowdot_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const bf16*)a.o, (const bf16*)a.dout, a.row_dot, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.Nk > 0) {
    constexpr int NW = 4;
    const int n_kt = (int)((a.Nk + 32 * NW - 1) / (32 * NW));
    const int64_t total = a.BH * n_kt;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NW>), dim3((unsigned)total), dim3(NW * 64), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.row_dot, (bf16*)a.dk, (bf16*)a.dv, (int)a.Nq, (int)a.Nk, (int)a.BH,
                       n_kt, (int)total, c, a.scale, a.causal ? 1 : 0,
                       (int)(!a.causal && total % 8 == 0));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    constexpr int BM = DqTile<D>::BM;
    const int n_qt = (int)((a.Nq + BM - 1) / BM);
    const int64_t total = a.BH * n_qt;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), dim3((unsigned)total), dim3(512), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.row_dot, (bf16*)a.dq, (int)a.Nq, (int)a.Nk, (int)a.BH, n_qt,
                       (int)total, c, a.scale, a.causal ? 1 : 0, (int)(!a.causal && total % 8 == 0));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_bwd(const BwdArgs& a) {
  return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a);
}

}  // namespace tattn
