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
// Two launches on the caller's stream, no atomics (deterministic):
//   1. dq:       one workgroup per 256 queries (or, at d = 64 on grids that
//                would not fill whole rounds of the chip, per 128 queries,
//                two workgroups per compute unit); each wave keeps Q^T and dO^T
//                of its 32 queries in VGPRs, first forms the row terms
//                D_i = sum_k dO_ik O_ik of its queries (and writes them for
//                the second launch), then sweeps the key tiles, computing
//                S^T = K Q^T and dP^T = V dO^T with the query in the lane,
//                then dQ^T += K^T dS^T; at d = 128 in the forward's ping-pong
//                schedule (one wave's dS work under the other's products on
//                each SIMD);
//   2. dkdv:     one workgroup per 256 keys (or per 128 keys, two per
//                compute unit, at d = 64 and on grids that would not fill
//                whole rounds); each wave keeps K^T of its 32
//                keys in VGPRs, the workgroup keeps the V rows of its keys
//                in LDS, and the query tiles stream through LDS (64 or 32
//                queries per stage, sub-steps of 32), computing S = Q K^T and
//                dP = dO V^T with the key in the lane so that P and dS feed
//                dV^T += dO^T P and dK^T += Q^T dS as B operands; dO^T and
//                Q^T come from ds_read_b64_tr_b16 transposed reads of the
//                row-major tiles.
// Both sweeps run two waves per SIMD and stage tiles with buffer_load ...
// lds (tile_common.h). The dQ sweep uses the forward's tile shapes: K^T is
// transposed in registers while staging, so every MFMA operand read is one
// ds_read_b128. The dK/dV sweep reads its transposed operands with
// transposed LDS reads instead, under a chunk swizzle that keeps both read
// kinds free of bank conflicts. The recomputation of S, P and dP in both
// sweeps trades extra MFMA work for never storing dS or taking atomics on
// dQ.
#include <type_traits>

#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace tattn {



// ---------------------------------------------------------------------------
// 2. dK, dV
// ---------------------------------------------------------------------------
// One workgroup per 32 NW keys: NW waves of 32 keys. With NW = 8 one
// workgroup fills a compute unit (two waves per SIMD); with NW = 4 two
// workgroups share one (one wave of each per SIMD), which halves the
// workgroup size for grids that would leave compute units idle or run a
// partial last round. Each wave keeps K^T of its keys in VGPRs (a B
// operand); the V rows of the workgroup's keys sit in LDS for the whole
// sweep. The query tiles stream through LDS in stages of BQ queries (Q and
// dO rows by buffer_load ... lds, double-buffered; BQ = 64, or 32 for
// NW = 4 at d = 128, where two workgroups' stages of 64 would not fit in
// LDS), each processed as sub-steps of 32 queries with the key in the
// lane:
//   S = Q K^T and dP = dO V^T         (Q, dO rows as A operands; K^T from
//                                      VGPRs, V rows from LDS as B operands)
//   P = 2^(c S - LSE2), dS = P (dP - D)  (LSE2 and D per accumulator slot)
//   dV^T += dO^T P and dK^T += Q^T dS  (dO^T and Q^T by transposed reads,
//                                      ds_read_b64_tr_b16, of the same tiles)
// The tiles use the transposable chunk swizzle kswz<D, 1>, under which both
// the row reads and the transposed reads are free of bank conflicts. Key r
// of a wave's 32 sits at LDS row swap23(r), so lane lq owns key
// 32 wave + swap23(lq) and K^T is loaded in that order.
// ceil(x / m) for m > 0, and 0 for x <= 0.
__device__ __forceinline__ int ceil_div_nonneg(int x, int m) { return x > 0 ? (x + m - 1) / m : 0; }

template <int D, int NW_>
struct DkdvTile {
  static constexpr int NW = NW_;
  static constexpr int BKV = 32 * NW;   // keys per workgroup
  static constexpr int BQ = NW == 8 || D == 64 ? 64 : 32;  // queries per stage
  static constexpr int QTILE = BQ * D;  // one Q or dO stage, bf16 elements
  static constexpr int DK = D / 16;
  static constexpr int DB = D / 32;
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                          const bf16* __restrict__ V, const bf16* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dv,
                          bf16* __restrict__ dK, bf16* __restrict__ dV, int Nq, int Nk, int BH,
                          int n_ktiles, int total_tiles, float c, float scale, int causal, int remap) {
  using C = DkdvTile<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::BKV * D + 4 * C::QTILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][C::BQ];  // [buf][lse2 | D][query]
  bf16* const vs = smem;
  auto qs = [&](int b) { return smem + C::BKV * D + 2 * b * C::QTILE; };
  auto dos = [&](int b) { return smem + C::BKV * D + (2 * b + 1) * C::QTILE; };

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
  const bf16* Qh = Q + qbase;
  const bf16* dOh = dO + qbase;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw_lo = kt * C::BKV + 32 * wave;  // this wave's first key
  const int key = kw_lo + swap23(lq);         // the key this lane owns
  const bool k_ok = key < Nk;
  const int off = Nk - Nq;
  const int n_st = (Nq + C::BQ - 1) / C::BQ;
  // Under the causal mask the first stage is the one holding the first
  // query that sees the workgroup's first key.
  const int j0 = causal ? max(0, kt * C::BKV - off) / C::BQ : 0;

  // V rows of the workgroup's keys (rows >= Nk read as zeros), once.
  const KDirect<D, C::BKV, C::NW, 1> vd(0, wave, lane);
  vd.load(V + kbase, Nk, kt, C::BKV, vs);
  const KDirect<D, C::BQ, C::NW, 1> qd(0, wave, lane);
  bf16x8 kf[C::DK];
  load_q<D>(K + kbase + (size_t)key * D, k_ok, h, kf);

  // The statistics are loaded before the stage's LDS DMA and used only when
  // written to LDS after the stage's work: a use right after the load would
  // make the compiler wait for the DMA issued behind it as well.
  float sreg = 0.f;
  auto stage = [&](int j, int buf) {
    if (tid < 2 * C::BQ) {
      const int q = j * C::BQ + (tid & (C::BQ - 1));
      if (tid < C::BQ)
        sreg = q < Nq ? LSE[(size_t)bh * Nq + q] : INFINITY;  // P = 0 past Nq
      else
        sreg = q < Nq ? Dv[(size_t)bh * Nq + q] : 0.f;
    }
    qd.load(Qh, Nq, j, C::BQ, qs(buf));
    qd.load(dOh, Nq, j, C::BQ, dos(buf));
  };
  auto store_stats = [&](int buf) {
    if (tid < 2 * C::BQ)
      stat[buf][tid / C::BQ][tid & (C::BQ - 1)] = tid < C::BQ ? sreg * kLog2e : sreg;
  };

  // Transposed reads: in each group of 16 lanes, lane 4e + g addresses the
  // 4 values d = 32 db + 16 ((lane >> 4) & 1) + 4 g .. + 3 of query
  // 16 t + 8 h + 4 e2 + e; lane j of the group then holds d = 32 db + lq
  // for 4 consecutive queries. With the swizzle's chunk bits below the row
  // bits, the offset for block db is the one for db = 0 XOR 32 db.
  int troff[2][C::DB];
  {
    const int g = lane & 3, e = (lane >> 2) & 3, clo = 2 * ((lane >> 4) & 1) + (g >> 1);
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int r = swap23(8 * h + 4 * e2 + e);
      const int base = r * D + 8 * (clo ^ kswz<D, 1>(r)) + 4 * (g & 1);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) troff[e2][db] = base ^ (32 * db);
    }
  }
  const KOffsets<D, true, 1> ko(lq, h);

  f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[db][i] = dvacc[db][i] = 0.f;

  // Queries 32 u .. 32 u + 31 of stage j held in buffer cur.
  auto substep = [&](auto masked, int cur, int j, int u) {
    constexpr bool MASKED = decltype(masked)::value;
    const bf16* qt = qs(cur) + 32 * u * D;
    const bf16* dt = dos(cur) + 32 * u * D;
    f32x16 sacc, dpacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < C::DK; ++s) {
      sacc = mfma32x32x16(k_read(qt, ko, s, 0), kf[s], sacc);
      dpacc = mfma32x32x16(k_read(dt, ko, s, 0), k_read(vs, ko, s, wave), dpacc);
    }
    // Issue order: the three reads of step s + 1 between the two MFMAs of
    // step s (left alone, the scheduler hoists every read and spills).
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int s = 0; s < C::DK - 1; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    // Slot 8 t + e holds query 32 u + 16 t + 8 h + e of the stage.
    const float* ls = stat[cur][0] + 32 * u + 8 * h;
    const float* dd = stat[cur][1] + 32 * u + 8 * h;
    u32x4 pw[2], sw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 l4[2] = {*(const f32x4*)(ls + 16 * t), *(const f32x4*)(ls + 16 * t + 4)};
      const f32x4 d4[2] = {*(const f32x4*)(dd + 16 * t), *(const f32x4*)(dd + 16 * t + 4)};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = 8 * t + e;
        float p0 = fast_exp2(fmaf(sacc[i], c, -l4[e >> 2][e & 3]));
        float p1 = fast_exp2(fmaf(sacc[i + 1], c, -l4[e >> 2][(e & 3) + 1]));
        if (MASKED) {  // hidden pairs (key > query + Nk - Nq) get P = 0
          const int q0 = j * C::BQ + 32 * u + 16 * t + 8 * h + e;
          p0 = key > q0 + off ? 0.f : p0;
          p1 = key > q0 + 1 + off ? 0.f : p1;
        }
        pw[t][e >> 1] = pack_bf16x2(p0, p1);
        sw[t][e >> 1] = pack_bf16x2(p0 * (dpacc[i] - d4[e >> 2][e & 3]),
                                    p1 * (dpacc[i + 1] - d4[e >> 2][(e & 3) + 1]));
      }
      __builtin_amdgcn_sched_barrier(0);  // one half's statistics live at a time
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16* dtt = dt + 16 * t * D;
      const bf16* qtt = qt + 16 * t * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 a = lds_read_tr_pair(dtt + troff[0][db], dtt + troff[1][db]);
        dvacc[db] = mfma32x32x16(a, as_bf16x8(pw[t]), dvacc[db]);
        const bf16x8 b = lds_read_tr_pair(qtt + troff[0][db], qtt + troff[1][db]);
        dkacc[db] = mfma32x32x16(b, as_bf16x8(sw[t]), dkacc[db]);
      }
    }
    // Two operands (four transposed reads) ahead of the MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * C::DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  if (j0 < n_st) {
    stage(j0, 0);
    wait_vmem();
    store_stats(0);
  }
  wait_vmem();  // the V rows
  __syncthreads();
  // One stage: prefetch the next, the two sub-steps (MODE 0: none of the
  // wave's pairs visible, 1: the mask edge runs through the stage, 2: all
  // visible), publish the prefetched stage.
  auto run_stage = [&](auto mode, int j) {
    constexpr int MODE = decltype(mode)::value;
    const int cur = (j - j0) & 1;
    const bool more = j + 1 < n_st;
    if (more) stage(j + 1, cur ^ 1);
    if (MODE != 0) {
#pragma unroll 1
      for (int u = 0; u < C::BQ / 32; ++u) substep(std::integral_constant<bool, MODE == 1>{}, cur, j, u);
    }
    if (more) store_stats(cur ^ 1);
    wait_vmem();
    __syncthreads();
  };
  // This wave's stages run in three phases, each a loop of one kind (no
  // branch inside a loop body, which would make the accumulators' live
  // ranges fork): stages before j_vis hold no visible pair, stages from
  // j_all on hold only visible pairs, and the mask edge of 32 keys crosses
  // at most two stages (of 32 or 64 queries) in between. Every wave runs
  // every stage's barrier.
  int j_vis = j0, j_all = j0;
  if (kw_lo >= Nk) {
    j_vis = j_all = max(j0, n_st);
  } else if (causal) {
    // first stage with a visible pair: BQ j + BQ - 1 + off >= kw_lo;
    // first stage with all pairs visible: BQ j + off >= kw_lo + 31
    j_vis = min(max(j0, ceil_div_nonneg(kw_lo - off - (C::BQ - 1), C::BQ)), max(j0, n_st));
    j_all = min(max(j_vis, ceil_div_nonneg(kw_lo + 31 - off, C::BQ)), max(j0, n_st));
  }
  j_vis = __builtin_amdgcn_readfirstlane(j_vis);
  j_all = __builtin_amdgcn_readfirstlane(j_all);
  int j = j0;
  for (; j < j_vis; ++j) run_stage(std::integral_constant<int, 0>{}, j);
  for (; j < j_all; ++j) run_stage(std::integral_constant<int, 1>{}, j);
  for (; j < n_st; ++j) run_stage(std::integral_constant<int, 2>{}, j);

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
// One workgroup per 32 NW queries: NW waves of 32 queries, two per SIMD
// (NW = 8: one workgroup per compute unit; NW = 4: two). Each
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
// The row term D_i = dO_i . O_i of dS for the query this lane owns: the lane
// holds the dO values of its half of the row (the layout of load_q), takes
// the matching O values and adds the other half's partial sum. Lanes of the
// first half write it to drow_out for the dK/dV sweep, which runs after this
// one; every query row gets its term, also one that sees no key (the dK/dV
// sweep multiplies its masked pairs' zero P by it).
template <int D>
__device__ __forceinline__ float row_term(const bf16* orow, const bf16x8* dof, bool q_ok, int h,
                                          float* drow_out) {
  bf16x8 of[D / 16];
  load_q<D>(orow, q_ok, h, of);
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)of[s][e], (float)dof[s][e], acc);
  const float d = add_other_half(acc);
  if (q_ok && h == 0) *drow_out = d;
  return d;
}

template <int D, int NW_ = 8>
struct DqTile {
  static constexpr int NW = NW_;
  static constexpr int BM = 32 * NW;
  using T = FwdTile<D, 64>;
  static constexpr int STAGE = 3 * T::KTILE;  // K rows, V rows, K^T
};

// K^T of rows [r0, r0 + ROWS) of a 64-key tile through registers, staged
// by WAVES waves as the forward stages V^T (Stager's V part: each lane loads
// the same 8 d-values of two adjacent keys and transpose_v_pair turns them
// into 8 consecutive keys of two d rows), with one buffer resource per tile
// (from the tile's first row to the end of the head, so rows past N read as
// zeros) and per-lane offsets fixed for the whole sweep. The address
// registers then stay live across the loop: a per-tile offset register,
// reused by the compiler for a later LDS read while the load was in flight,
// had the next step's first MFMA wait for the whole staged tile. Waves past
// the last pass (at d = 64) load and store nothing.
template <int D, int WAVES = 8, int ROWS = 64>
struct KtStager {
  using T = FwdTile<D, 64>;
  static constexpr int VPASS = ROWS / T::VKEYS;
  static constexpr int VPW = (VPASS + WAVES - 1) / WAVES;
  static_assert(ROWS % T::VKEYS == 0, "rows must split into whole passes");
  u32x4 va[VPW], vb[VPW];
  int wave_, r0_;
  int off[VPW];  // byte offset of key kv (and kv + 1 at + 2 D) within a tile
  // Pass (wave + i * WAVES) of VPASS (at d = 64 not every wave stages).
  __device__ __forceinline__ bool has_pass(int i) const {
    return VPASS % WAVES == 0 || wave_ + i * WAVES < VPASS;
  }
  // t: thread index within the staging waves.
  __device__ __forceinline__ KtStager(int t, int r0 = 0) {
    const int wave = t >> 6, lane = t & 63, p = lane >> 4, r = lane & 15;
    wave_ = __builtin_amdgcn_readfirstlane(wave);
    r0_ = r0;
    const int col = 8 * (r % T::CPR), g = r / T::CPR;
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int kv = r0 + (wave + i * WAVES) * T::VKEYS + 8 * g + 2 * p;
      off[i] = (kv * D + col) * 2;
    }
  }
  __device__ __forceinline__ void load(const bf16* kh, int n_rows, int tile) {
    const int row0 = tile * 64;
    const int rem = n_rows > row0 ? n_rows - row0 : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kh + (size_t)row0 * D), 0, rem * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < VPW; ++i)
      if (has_pass(i)) {
        va[i] = buffer_load16(r, off[i]);
        vb[i] = buffer_load16(r, off[i] + 2 * D);
      }
  }
  __device__ __forceinline__ void store(bf16* kt, int t) const {
    const int lane = t & 63, p = lane >> 4, r = lane & 15;
    const int d0 = 8 * (r % T::CPR) + 2 * p, g = r / T::CPR;
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      if (!has_pass(i)) continue;
      u32x4 lo, hi;
      transpose_v_pair(va[i], vb[i], lo, hi);
      const int slot = (r0_ + (wave_ + i * WAVES) * T::VKEYS) / 8 + g;
      *(u32x4*)(kt + d0 * 64 + 8 * (slot ^ vt_swz(d0))) = lo;
      *(u32x4*)(kt + (d0 + 1) * 64 + 8 * (slot ^ vt_swz(d0 + 1))) = hi;
    }
  }
  // Global loads one load() issues (for the scheduling hints).
  static constexpr int kLoads = 2 * VPW;
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

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D == 128 && NW == 4 ? 1 : 2, 2)))
void attn_bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                        const bf16* __restrict__ V, const bf16* __restrict__ O,
                        const bf16* __restrict__ dO, const float* __restrict__ LSE,
                        float* __restrict__ Dv,
                        bf16* __restrict__ dQ, int Nq, int Nk, int BH, int n_qtiles, int total_tiles,
                        float c, float scale, int causal, int remap) {
  using C = DqTile<D, NW>;
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
  const float drow = row_term<D>(O + qbase + (size_t)q_row * D, dof, q_ok, h, Dv + (size_t)bh * Nq + q_row);

  const VtOffsets vo(lq, h);
  const KOffsets<D, true> ko(lq, h);
  const KDirect<D, 64, C::NW> kd(0, wave, lane);
  KtStager<D, NW> st(tid);  // K^T through registers
  auto stage_direct = [&](int j, int buf) {
    kd.template load<true>(Kh, Nk, j, 64, ks(buf));
    kd.template load<true>(Vh, Nk, j, 64, vs(buf));
  };

  f32x16 dqacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  if (n_kt > 0) {
    stage_direct(0, 0);
    st.load(Kh, Nk, 0);
    st.store(kts(0), tid);
    wait_vmem();
    __syncthreads();
  }
  wait_vmem();  // Q^T, dO^T and the row statistics, on every path into the sweep
  auto step = [&](auto masked, int j) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = j & 1;
    const bool more = j + 1 < n_kt;
    if (more) {
      stage_direct(j + 1, cur ^ 1);
      st.load(Kh, Nk, j + 1);
    }
    f32x16 sacc[2], dpacc[2];
    score_tile<D>(ks(cur), qf, ko, sacc);
    score_tile<D>(vs(cur), dof, ko, dpacc);
    u32x4 pw[4];
    dq_scores_to_ds<MASKED, D>(sacc, dpacc, c, lse2, drow, j * 64, kmax, h, pw);
    if (more) st.store(kts(cur ^ 1), tid);
    pv_tile<D>(kts(cur), pw, vo, dqacc);  // dQ^T += K^T dS^T
    publish_lds();  // next K, V tiles (transfers) and K^T (stores)
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
// 3b. dQ, ping-pong: the sweep above with the forward's ping-pong schedule.
// The 8 waves form two groups of 4 (one wave of each per SIMD); a wave's
// work on key tile j is split into an MFMA phase (dQ^T += K^T dS^T of tile j
// around S^T = K Q^T and dP^T = V dO^T of tile j + 1) and a VALU phase
// (dS^T of tile j + 1). Group B runs one phase behind group A and every
// phase ends at a workgroup barrier, so on each SIMD one wave's dS work
// runs under the other wave's products. K, V rows and K^T are
// double-buffered; each group stages half of every tile in its VALU phase:
// group A the K and V rows of tile j + 2 (buffer_load ... lds) and K^T of
// tile j + 1 (loaded into registers at the start of the MFMA phase, stored
// transposed in the VALU phase), group B one tile further (j + 3, j + 2),
// which keeps each buffer free until both groups have read it.
// ---------------------------------------------------------------------------
template <int D, int NVMEM = 0, bool DO_S = true, bool DO_PV = true>
__device__ __forceinline__ void dq_mfma_phase(const bf16* ks, const bf16* vs, const bf16* kt,
                                              const bf16x8* qf, const bf16x8* dof, const u32x4* pw,
                                              const VtOffsets& vo, const KOffsets<D, true>& ko,
                                              const bf16x8* pre, f32x16* sacc, f32x16* dpacc,
                                              f32x16* dqacc) {
  using T = FwdTile<D, 64>;
  constexpr int NPV = DO_PV ? T::NT * T::DB : 0;
#pragma unroll
  for (int k = 0; k < NPV / 2; ++k) {
    const int t = pv_step_t<T::NT>(k, T::DB), db = k % T::DB;
    const bf16x8 kf = k < kPrefetch ? pre[k] : vt_read<D>(kt, vo, t, db);
    dqacc[db] = mfma32x32x16(kf, as_bf16x8(pw[t]), dqacc[db]);
  }
  if (DO_S) {
    // four independent chains: S^T and dP^T of both 32-key blocks
    f32x16 a[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) a[x][i] = 0.f;
#pragma unroll
    for (int s = 0; s < T::DK; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        a[kb] = mfma32x32x16(k_read<D>(ks, ko, s, kb), qf[s], a[kb]);
        a[2 + kb] = mfma32x32x16(k_read<D>(vs, ko, s, kb), dof[s], a[2 + kb]);
      }
    sacc[0] = a[0];
    sacc[1] = a[1];
    dpacc[0] = a[2];
    dpacc[1] = a[3];
  }
#pragma unroll
  for (int k = NPV / 2; k < NPV; ++k) {
    const int t = pv_step_t<T::NT>(k, T::DB), db = k % T::DB;
    dqacc[db] = mfma32x32x16(vt_read<D>(kt, vo, t, db), as_bf16x8(pw[t]), dqacc[db]);
  }
  // Issue order: global loads, then one LDS read after each MFMA, which
  // keeps kPrefetch operands in flight.
  constexpr int NMFMA = NPV + (DO_S ? 4 * T::DK : 0);
  if (NVMEM > 0) __builtin_amdgcn_sched_group_barrier(0x020, NVMEM, 0);
  if (!DO_PV) __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + kPrefetch < NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_pingpong_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                 const bf16* __restrict__ V, const bf16* __restrict__ O,
                                 const bf16* __restrict__ dO, const float* __restrict__ LSE,
                                 float* __restrict__ Dv,
                                 bf16* __restrict__ dQ, int Nq, int Nk, int BH, int n_qtiles,
                                 int total_tiles, float c, float scale, int causal, int remap) {
  using C = DqTile<D>;
  using T = typename C::T;
  using Kt = KtStager<D, 4, 32>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];
  auto ks = [&](int b) { return smem + (b & 1) * C::STAGE; };
  auto vs = [&](int b) { return smem + (b & 1) * C::STAGE + T::KTILE; };
  auto kts = [&](int b) { return smem + (b & 1) * C::STAGE + 2 * T::KTILE; };

  // Tile order as in the lock-step sweep.
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
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // 0: group A, 1: group B
  const int gtid = tid & 255;  // thread index within the group
  const int r0 = 32 * grp;     // rows of each tile this group stages
  const int q_row = qt * C::BM + wave * 32 + lq;
  const bool q_ok = q_row < Nq;
  const int off = Nk - Nq;
  const int q_lo = qt * C::BM, q_hi = min(q_lo + C::BM, Nq) - 1;
  const int lim = causal ? min(Nk, q_hi + off + 1) : Nk;
  const int n_kt = lim > 0 ? (lim + 63) / 64 : 0;
  const int all_see = causal ? min(Nk, q_lo + off + 1) : Nk;
  const int n_full = all_see > 0 ? all_see / 64 : 0;
  const int kmax = causal ? min(Nk - 1, q_row + off) : Nk - 1;

  f32x16 dqacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  bf16x8 dof[T::DK];
  load_q<D>(dO + qbase + (size_t)q_row * D, q_ok, h, dof);
  const float drow = row_term<D>(O + qbase + (size_t)q_row * D, dof, q_ok, h, Dv + (size_t)bh * Nq + q_row);
  if (n_kt > 0) {  // workgroup-uniform
    bf16x8 qf[T::DK];
    load_q<D>(Q + qbase + (size_t)q_row * D, q_ok, h, qf);
    // A query that sees no key has LSE = -inf; all its keys are masked.
    const float lse2 = q_ok ? LSE[(size_t)bh * Nq + q_row] * kLog2e : INFINITY;
    const VtOffsets vo(lq, h);
    const KOffsets<D, true> ko(lq, h);
    const KDirect<D, 32, 4> kd(r0, wave & 3, lane);
    Kt st(gtid, r0);
    auto stage_rows = [&](int t) {  // this group's K and V rows of tile t
      kd.template load<true>(Kh, Nk, t, 64, ks(t));
      kd.template load<true>(Vh, Nk, t, 64, vs(t));
    };

    {  // prologue: everyone stages K, V rows of tiles 0 and 1 and K^T of tile 0
      const KDirect<D, 64, C::NW> kd0(0, wave, lane);
      kd0.template load<true>(Kh, Nk, 0, 64, ks(0));
      kd0.template load<true>(Vh, Nk, 0, 64, vs(0));
      kd0.template load<true>(Kh, Nk, 1, 64, ks(1));
      kd0.template load<true>(Vh, Nk, 1, 64, vs(1));
      KtStager<D> st0(tid);
      st0.load(Kh, Nk, 0);
      st0.store(kts(0), tid);
    }
    publish_lds();  // also Q^T, dO^T and the row statistics
    if (grp == 1) phase_barrier();

    f32x16 sacc[2], dpacc[2];
    u32x4 pw[4];
    bf16x8 pre[kPrefetch];  // first K^T operands of the next MFMA phase

    // MFMA phase of tile 0: S^T and dP^T only
    dq_mfma_phase<D, 0, true, false>(ks(0), vs(0), kts(0), qf, dof, pw, vo, ko, pre, sacc, dpacc,
                                     dqacc);
    phase_barrier();
    if (grp == 1) {  // VALU phase "j = -1": group B stages K^T of tile 1, rows of tile 2
      st.load(Kh, Nk, 1);
      st.store(kts(1), gtid);
      stage_rows(2);
    }
    if (n_full == 0)
      dq_scores_to_ds<true, D>(sacc, dpacc, c, lse2, drow, 0, kmax, h, pw);
    else
      dq_scores_to_ds<false, D>(sacc, dpacc, c, lse2, drow, 0, kmax, h, pw);
    prefetch_pv<D, 64>(kts(0), vo, pre);
    wait_vmem();
    phase_barrier();

    auto body = [&](auto masked, int j) {
      constexpr bool MASKED = decltype(masked)::value;
      const int tr = j + 2 + grp, tt = j + 1 + grp;  // rows / K^T staged here
      // MFMA phase: dQ^T += K^T dS^T of tile j, S^T and dP^T of tile j + 1.
      st.load(Kh, Nk, tt);
      dq_mfma_phase<D, Kt::kLoads>(ks(j + 1), vs(j + 1), kts(j), qf, dof, pw, vo, ko, pre, sacc,
                                   dpacc, dqacc);
      phase_barrier();
      // VALU phase: K^T stores (their loads had the MFMA phase to arrive),
      // then the row transfers (issued after the stores, so that the
      // compiler's wait for the K^T loads does not also wait for them),
      // dS^T of tile j + 1 and the first operands of the next MFMA phase.
      st.store(kts(tt), gtid);
      stage_rows(tr);
      dq_scores_to_ds<MASKED, D>(sacc, dpacc, c, lse2, drow, (j + 1) * 64, kmax, h, pw);
      prefetch_pv<D, 64>(kts(j + 1), vo, pre);
      wait_vmem();
      phase_barrier();
    };
    // bodies j = 0 .. n_kt - 2 (body j takes dS of tile j + 1); tiles from
    // n_full on hold a key some query of the tile may not see.
    const int n_body = n_kt - 1;
    const int n_plain = min(max(n_full - 1, 0), n_body);
    int j = 0;
    for (; j < n_plain; ++j) body(std::false_type{}, j);
    for (; j < n_body; ++j) body(std::true_type{}, j);
    // last tile: dQ product only
    dq_mfma_phase<D, 0, false>(ks(j + 1), vs(j + 1), kts(j), qf, dof, pw, vo, ko, pre, sacc, dpacc,
                               dqacc);
    phase_barrier();
    phase_barrier();
    if (grp == 0) phase_barrier();
  }

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

// One launch of the dQ sweep: the lock-step kernel with NW waves per
// workgroup (32 NW queries), or the 8-wave ping-pong kernel.
template <int D, int NW, bool PINGPONG>
static hipError_t launch_dq(const BwdArgs& a, float c) {
  constexpr int BM = DqTile<D, NW>::BM;
  const int n_qt = (int)((a.Nq + BM - 1) / BM);
  const int64_t total = a.BH * n_qt;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  constexpr auto kernel = [] {
    if constexpr (PINGPONG) return &attn_bwd_dq_pingpong_kernel<D>;
    else return &attn_bwd_dq_kernel<D, NW>;
  }();
  hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(NW * 64), 0, (hipStream_t)a.stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.o,
                     (const bf16*)a.dout, a.lse, a.row_dot, (bf16*)a.dq, (int)a.Nq, (int)a.Nk, (int)a.BH,
                     n_qt, (int)total, c, a.scale, a.causal ? 1 : 0, (int)(!a.causal && total % 8 == 0));
  return hipGetLastError();
}

// Waves per dQ workgroup (4: 128 queries, lock-step; 8: 256 queries, the
// ping-pong sweep at d = 128 and the lock-step one at d = 64). At d = 128
// a tile's MFMA phase (48 products) is longer than its dS phase and the
// ping-pong sweep overlaps the two (its 96 KiB of LDS leave room for one
// workgroup per compute unit, so it keeps 8 waves); at d = 64 (24 products)
// the dS work dominates and the lock-step sweep, with half the barriers,
// is faster, and its 4-wave workgroups (two per compute unit) win where
// the 8-wave grid would leave compute units idle or end in a partial
// round, as in the dK/dV sweep.
int dq_waves(const BwdArgs& a) {
  if (a.dq_waves == 4 || a.dq_waves == 8) return a.dq_waves;
  if (a.d != 64) return 8;
  const int64_t g8 = a.BH * ((a.Nq + 255) / 256);
  return (g8 % a.num_cus == 0 || g8 >= 4 * (int64_t)a.num_cus) ? 8 : 4;
}

// ---------------------------------------------------------------------------
template <int D, int NW>
static hipError_t launch_dkdv(const BwdArgs& a, float c) {
  constexpr int BKV = DkdvTile<D, NW>::BKV;
  const int n_kt = (int)((a.Nk + BKV - 1) / BKV);
  const int64_t total = a.BH * n_kt;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NW>), dim3((unsigned)total), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     (const bf16*)a.dout, a.lse, a.row_dot, (bf16*)a.dk, (bf16*)a.dv, (int)a.Nq, (int)a.Nk,
                     (int)a.BH, n_kt, (int)total, c, a.scale, a.causal ? 1 : 0,
                     (int)(!a.causal && total % 8 == 0));
  return hipGetLastError();
}

// Waves per dK/dV workgroup. At d = 64 the 4-wave workgroups (two per
// compute unit) measured as fast or faster on every shape tried. At
// d = 128 they hold stages of 32 queries (twice the barriers and stage
// transfers), which costs ≈1.5 % on grids of whole rounds of 8-wave
// workgroups, but their finer grain wins where the 8-wave grid would
// leave compute units idle or end in a partial round (wave quantization,
// CS336 Lecture 5 notes §6.2).
int dkdv_waves(const BwdArgs& a) {
  if (a.dkdv_waves == 4 || a.dkdv_waves == 8) return a.dkdv_waves;
  if (a.d == 64) return 4;
  const int64_t g8 = a.BH * ((a.Nk + 255) / 256);
  return (g8 % a.num_cus == 0 || g8 >= 4 * (int64_t)a.num_cus) ? 8 : 4;
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  const float c = a.scale * kLog2e;
  // The dQ sweep runs first: it also writes the row terms D_i that the
  // dK/dV sweep reads. With no query, the dK/dV kernel alone runs (it writes
  // zeros and reads no row term); with no key, the dQ kernel alone runs
  // (likewise).
  const int64_t rows = a.BH * a.Nq;
  if (rows > 0) {
    const hipError_t e = dq_waves(a) == 4 ? launch_dq<D, 4, false>(a, c) : launch_dq<D, 8, D == 128>(a, c);
    if (e != hipSuccess) return e;
  }
  if (a.Nk > 0) {
    const hipError_t e = dkdv_waves(a) == 8 ? launch_dkdv<D, 8>(a, c) : launch_dkdv<D, 4>(a, c);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_bwd(const BwdArgs& a) {
  return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a);
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the row terms D_i (the only scratch the backward
// uses) go to this fixed device array. Each device holds its own copy, at
// its own address; in host code the name is only a stand-in for the symbol,
// so kernels get the device address hipGetSymbolAddress reports, looked up
// once per device (with that device current) and kept. The dQ sweep writes
// every D_i a call reads before the dK/dV sweep reads it, so nothing needs
// clearing between calls; calls that overlap on one device share the array
// and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kNoAllocRows];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_addr[kMaxScratchDevices];

hipError_t scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = (float*)p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_attn_bwd_noalloc(const BwdArgs& a) {
  if (a.BH * a.Nq > kNoAllocRows) return hipErrorInvalidValue;
  BwdArgs b = a;
  const hipError_t e = scratch_address(&b.row_dot);
  if (e != hipSuccess) return e;
  return launch_attn_bwd(b);
}

}  // namespace tattn
