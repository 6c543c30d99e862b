// Fused attention forward for gfx950: O = softmax(scale Q K^T) V and LSE.
//
// Method: the Lecture 17 page "Tensor Core, HBM, SRAM and FlashAttention",
// §8.2 (take a Q tile, stream K/V tiles, form each score tile on chip, never
// write S or P to HBM) and §8.3 (online softmax: m' = max(m, max s),
// alpha = e^(m - m'), p = e^(s - m'), l' = alpha l + sum p, o' = alpha o + p V,
// O = o / l at the end). Exponentials are taken in base 2 with
// c = scale * log2(e) folded into one FMA: e^(scale s - m) = 2^(c s - m2).
//
// MI355X mapping (bf16 kernel):
//   * one workgroup = NW waves, each wave owns 32 query rows (BM = 32 NW);
//   * the wave computes the TRANSPOSED score tile S^T = K Q^T on
//     v_mfma_f32_32x32x16_bf16, so each lane owns one query column: the row
//     statistics m and l, the rescale factor alpha and 1/l are per-lane
//     scalars and need one cross-half exchange (v_permlane32_swap) per tile;
//   * Q^T (the B operand) stays in VGPRs for the whole key sweep;
//   * K and V tiles (64 keys) are staged through LDS, double-buffered, with
//     16-byte coalesced global loads issued one tile ahead; K rows are placed
//     at swap23(key) so the score accumulator is already in the operand order
//     of the next product, and V is read transposed with ds_read_b64_tr_b16
//     for O^T = V^T P^T (so V needs no transposing copy);
//   * rows are padded by 16 bytes in LDS to spread banks;
//   * the last key tile of a ragged N masks keys >= N (p = 0).
#include "device_common.h"
#include "launch.h"

namespace tattn {

// ---------------------------------------------------------------------------
// bf16 forward
// ---------------------------------------------------------------------------
template <int D, int NW>
struct FwdBf16Cfg {
  static constexpr int R = 32;                 // query rows per wave
  static constexpr int BM = R * NW;            // query rows per workgroup
  static constexpr int BN = 64;                // keys per step
  static constexpr int PITCH = D + 8;          // LDS row pitch (bf16 elements)
  static constexpr int TILE = BN * PITCH;      // elements per staged K or V tile
  static constexpr int THREADS = NW * 64;
  static constexpr int CHUNKS = BN * D / 8;    // 16-byte chunks per K or V tile
  static constexpr int CPT = CHUNKS / THREADS; // chunks per thread per tile
  static constexpr int DK = D / 16;            // k-steps of the score product
  static constexpr int DB = D / 32;            // 32-wide blocks of d
  static_assert(CHUNKS % THREADS == 0, "tile must split evenly over the workgroup");
  static constexpr size_t LDS_BYTES = 2 * 2 * TILE * sizeof(bf16);
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 4 ? 2 : 1, 2))) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_tiles,
    float c, int remap) {
  using C = FwdBf16Cfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * C::TILE];
  // stage b: K tile at smem + 2 b TILE, V tile right after it
  auto ks = [&](int b) { return smem + 2 * b * C::TILE; };
  auto vs = [&](int b) { return smem + (2 * b + 1) * C::TILE; };

  const int tile = xcd_tile(blockIdx.x, total_tiles, remap);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * N * D;
  const bf16* Qb = Q + base;
  const bf16* Kb = K + base;
  const bf16* Vb = V + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int h = lane >> 5;
  const int q_row = qt * C::BM + wave * C::R + lq;   // the query this lane owns
  const bool q_ok = q_row < N;

  // Q^T as the B operand: lane (query lq, half h) holds d = 16 s + 8 h .. +7.
  bf16x8 qf[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 x = {0, 0, 0, 0};
    if (q_ok) x = *(const u32x4*)(Qb + (size_t)q_row * D + 16 * s + 8 * h);
    qf[s] = as_bf16x8(x);
  }

  const int n_kt = (N + C::BN - 1) / C::BN;
  u32x4 kreg[C::CPT], vreg[C::CPT];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8);
      const int col = (ch % (D / 8)) * 8;
      const int key = j * C::BN + row;
      u32x4 zk = {0, 0, 0, 0}, zv = {0, 0, 0, 0};
      if (key < N) {
        zk = *(const u32x4*)(Kb + (size_t)key * D + col);
        zv = *(const u32x4*)(Vb + (size_t)key * D + col);
      }
      kreg[i] = zk;
      vreg[i] = zv;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::THREADS;
      const int row = ch / (D / 8);
      const int col = (ch % (D / 8)) * 8;
      *(u32x4*)(ks(buf) + swap23(row) * C::PITCH + col) = kreg[i];
      *(u32x4*)(vs(buf) + row * C::PITCH + col) = vreg[i];
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;  // running max of c * s (base-2 domain)
  float l_run = 0.f;        // running sum over this lane's half of the keys

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // Lane-constant parts of the transposed V read (see device_common.h).
  const int g = lane >> 4;
  const int j16 = lane & 15;
  const int v_col = 16 * (g & 1) + 4 * (j16 & 3);
  const int v_row = 8 * h + (j16 >> 2);

  for (int j = 0; j < n_kt; ++j) {
    const int cur = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);

    // S^T = K Q^T for the 64 keys of this step: two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      const bf16* kp = ks(cur) + (32 * kb + lq) * C::PITCH + 8 * h;
#pragma unroll
      for (int s = 0; s < C::DK; ++s) {
        bf16x8 kf = as_bf16x8(*(const u32x4*)(kp + 16 * s));
        sacc[kb] = mfma32x32x16(kf, qf[s], sacc[kb]);
      }
    }

    // Keys of this lane: key(kb, i) = j*64 + 32 kb + 16 (i/8) + 8 h + i%8.
    const bool ragged = (j + 1) * C::BN > N;
    if (ragged) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j * C::BN + 32 * kb + 16 * (i >> 3) + 8 * h + (i & 7);
          if (key >= N) sacc[kb][i] = -INFINITY;
        }
    }

    // Online softmax update for the query this lane owns.
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    float lsum = 0.f;
    unsigned pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = fast_exp2(fmaf(sacc[kb][i], c, -m_new));
        float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -m_new));
        if (ragged) {
          if (sacc[kb][i] == -INFINITY) p0 = 0.f;
          if (sacc[kb][i + 1] == -INFINITY) p1 = 0.f;
        }
        lsum += p0 + p1;
        pk[kb][i >> 1] = pack_bf16x2(p0, p1);
      }
    l_run = fmaf(alpha, l_run, lsum);
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // O^T += V^T P^T over the 4 steps of 16 keys.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pw = {pk[t >> 1][4 * (t & 1) + 0], pk[t >> 1][4 * (t & 1) + 1],
                  pk[t >> 1][4 * (t & 1) + 2], pk[t >> 1][4 * (t & 1) + 3]};
      const bf16x8 pf = as_bf16x8(pw);
      const bf16* vp = vs(cur) + (16 * t + v_row) * C::PITCH + v_col;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        bf16x8 vf = lds_read_tr_pair(vp + 32 * db, vp + 4 * C::PITCH + 32 * db);
        oacc[db] = mfma32x32x16(vf, pf, oacc[db]);
      }
    }

    if (j + 1 < n_kt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: O = o / l, LSE = ln(2) (m + log2 l).
  const float l_tot = add_other_half(l_run);
  const float inv = 1.f / l_tot;
  if (q_ok) {
    bf16* orow = O + base + (size_t)q_row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r + 0] * inv, oacc[db][4 * r + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
        *(u32x2*)(orow + 32 * db + 8 * r + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + q_row] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward (fp32 storage and arithmetic; v_mfma_f32_32x32x2_f32)
// ---------------------------------------------------------------------------
template <int D>
struct FwdF32Cfg {
  static constexpr int NW = 4;
  static constexpr int R = 32;
  static constexpr int BM = R * NW;
  static constexpr int BN = 32;
  static constexpr int KPITCH = D + 1;   // odd pitch: rows of the A operand hit distinct banks
  static constexpr int VPITCH = D + 4;
  static constexpr int THREADS = NW * 64;
  static constexpr int DB = D / 32;
  static constexpr int DK = D / 2;
};

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, float c) {
  using C = FwdF32Cfg<D>;
  __shared__ float kt[C::BN * C::KPITCH];
  __shared__ float vt[C::BN * C::VPITCH];

  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x - bh * n_qtiles;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int q_row = qt * C::BM + wave * C::R + lq;
  const bool q_ok = q_row < N;

  float qf[C::DK];  // lane (query lq, half h) holds Q[q][2 s + h]
#pragma unroll
  for (int s = 0; s < C::DK; ++s) qf[s] = q_ok ? Q[base + (size_t)q_row * D + 2 * s + h] : 0.f;

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = (N + C::BN - 1) / C::BN;
  for (int j = 0; j < n_kt; ++j) {
    for (int e = tid; e < C::BN * D; e += C::THREADS) {
      const int row = e / D, col = e % D, key = j * C::BN + row;
      const bool ok = key < N;
      kt[row * C::KPITCH + col] = ok ? K[base + (size_t)key * D + col] : 0.f;
      vt[row * C::VPITCH + col] = ok ? V[base + (size_t)key * D + col] : 0.f;
    }
    __syncthreads();

    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < C::DK; ++s) sacc = mfma32x32x2f32(kt[lq * C::KPITCH + 2 * s + h], qf[s], sacc);

    // key of slot i: j*32 + 8 (i/4) + 4 h + i%4
    const bool ragged = (j + 1) * C::BN > N;
    if (ragged) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (j * C::BN + 8 * (i >> 2) + 4 * h + (i & 3) >= N) sacc[i] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    float p[16], lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(fmaf(sacc[i], c, -m_new));
      if (ragged && sacc[i] == -INFINITY) p[i] = 0.f;
      lsum += p[i];
    }
    l_run = fmaf(alpha, l_run, lsum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    // O^T += V^T P^T: k-step s pairs key(s, 0) and key(s, 1).
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int key = 8 * (s >> 2) + 4 * h + (s & 3);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        oacc[db] = mfma32x32x2f32(vt[key * C::VPITCH + 32 * db + lq], p[s], oacc[db]);
    }
    __syncthreads();
  }

  const float l_tot = add_other_half(l_run);
  const float inv = 1.f / l_tot;
  if (q_ok) {
    float* orow = O + base + (size_t)q_row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(f32x4*)(orow + 32 * db + 8 * r + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + q_row] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, int NW>
static hipError_t launch_bf16(const FwdArgs& a) {
  using C = FwdBf16Cfg<D, NW>;
  const int n_qtiles = (int)((a.N + C::BM - 1) / C::BM);
  const int64_t total = (int64_t)a.BH * n_qtiles;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  const int remap = (total % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>), dim3((unsigned)total), dim3(C::THREADS), 0,
                     (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     (bf16*)a.o, a.lse, (int)a.N, n_qtiles, (int)total, a.scale * kLog2e, remap);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const FwdArgs& a) {
  using C = FwdF32Cfg<D>;
  const int n_qtiles = (int)((a.N + C::BM - 1) / C::BM);
  const int64_t total = (int64_t)a.BH * n_qtiles;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)total), dim3(C::THREADS), 0,
                     (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                     (float*)a.o, a.lse, (int)a.N, n_qtiles, a.scale * kLog2e);
  return hipGetLastError();
}

// Workgroup size choice: the largest query tile whose grid still covers
// every compute unit at least once (wave quantization, CS336 Lecture 5
// notes §6.2), else the smallest.
int fwd_bf16_waves(int64_t BH, int64_t N, int num_cus) {
  for (int nw : {8, 4}) {
    const int64_t tiles = BH * ((N + 32 * nw - 1) / (32 * nw));
    if (tiles >= num_cus) return nw;
  }
  return 2;
}

hipError_t launch_attn_fwd(const FwdArgs& a) {
  if (a.dtype_fp32) {
    return a.d == 64 ? launch_f32<64>(a) : launch_f32<128>(a);
  }
  const int nw = a.waves ? a.waves : fwd_bf16_waves(a.BH, a.N, a.num_cus);
  if (a.d == 64) {
    return nw == 8 ? launch_bf16<64, 8>(a) : nw == 4 ? launch_bf16<64, 4>(a) : launch_bf16<64, 2>(a);
  }
  return nw == 8 ? launch_bf16<128, 8>(a) : nw == 4 ? launch_bf16<128, 4>(a) : launch_bf16<128, 2>(a);
}

}  // namespace tattn
