// Fused attention forward for gfx950: O = softmax(scale Q K^T) V and LSE.
//
// Method: the Lecture 17 page "Tensor Core, HBM, SRAM and FlashAttention",
// §8.2 (take a Q tile, stream K/V tiles, form each score tile on chip, never
// write S or P to HBM) and §8.3 (online softmax: m' = max(m, max s),
// alpha = e^(m - m'), p = e^(s - m'), l' = alpha l + sum p, o' = alpha o + p V,
// O = o / l at the end). Exponentials are taken in base 2 with
// c = scale * log2(e) folded into one FMA: e^(scale s - m) = 2^(c s - m2).
//
// MI355X mapping (bf16 kernels):
//   * one workgroup = NW waves, each wave owns 32 query rows (BM = 32 NW);
//   * the wave computes the TRANSPOSED score tile S^T = K Q^T on
//     v_mfma_f32_32x32x16_bf16, so each lane owns one query column: the row
//     statistics m and l, the rescale factor alpha and 1/l are per-lane
//     scalars and need one cross-half exchange (v_permlane32_swap) per tile;
//   * Q^T (the B operand) stays in VGPRs for the whole key sweep;
//   * K and V tiles (128 keys in the 256-query ping-pong kernel, 64 in the
//     smaller kernels) are staged through LDS, double-buffered: K goes
//     straight from memory to LDS (buffer_load ... lds, 16 bytes per lane),
//     V through registers (16-byte loads); K rows are placed at swap23(key)
//     so the score accumulator is already in the operand order of the next
//     product;
//   * V is stored TRANSPOSED in LDS (V^T, one row of 64 keys per d), so the
//     A operand of O^T += V^T P^T is one ds_read_b128 per MFMA. The
//     transpose is done once per workgroup while staging: each lane loads the
//     same 8 d-values of two adjacent keys, v_perm_b32 pairs the keys, and
//     v_permlane32_swap / v_permlane16_swap exchange the pairs of 4 lanes
//     (a 4 x 4 dword transpose), leaving each lane 8 consecutive keys of two
//     d rows. (A ds_read_b64_tr_b16 of row-major V moves half the bytes per
//     LDS instruction at a third of the b128 rate: the LDS, not the matrix
//     core, then bounds the kernel.)
//   * the 16-byte slots of a V^T row are XOR-swizzled by vt_swz(d) so that
//     the MFMA operand reads are free of bank conflicts and the transposed
//     writes at most two-way conflicted;
//   * the last key tile of a ragged N masks keys >= N (p = 0) and stages
//     zeros for them.
#include <type_traits>

#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace tattn {

// ---------------------------------------------------------------------------
// bf16 forward: shared pieces
// ---------------------------------------------------------------------------
// The running max is only moved when a tile's max exceeds it by more than
// this (base-2 units): p = 2^(c s - m) then stays <= 2^8, exact in the fp32
// sum and in the bf16 operand's exponent range, and the rescale of the
// output accumulator (a multiply per accumulator element) is skipped for
// almost every tile. The shift cancels in o / l, so the result is the same
// softmax as with the running max itself.
constexpr float kLazyRescale = 8.0f;

// Most key tiles of one query tile that need a mask: with BN-key tiles and
// BM queries, the keys seen by some but not all queries of the tile span at
// most BM - 1 positions, which touch at most ceil((BN - 1 + BM - 1) / BN)
// tiles: 3 for (BM, BN) = (256, 128), (128, 64) and fewer for (64, 64).
constexpr int kMaxMaskedTiles = 3;

// Online softmax update (Lecture 17 page, §8.3) for the query this lane owns,
// over one key tile whose first key is key0. Produces P (bf16, packed in
// the B-operand order of the value product), updates the running (m, l) and
// rescales the output accumulator by alpha when the running max moves.
// MASKED tiles drop keys past kmax, the last key this lane's query may see
// (the end of the key range, or of its causal window): p = 0 for them. A row
// that has not seen a visible key yet keeps m = -inf, l = 0, o = 0 (its
// exponentials are taken against 0 instead of -inf).
template <bool MASKED, int DB, int NKB = 2>
__device__ __forceinline__ void softmax_tile(f32x16* sacc, float c, int key0, int kmax, int h,
                                             float& m_run, float& l_run, f32x16* oacc,
                                             u32x4* pw) {
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + 32 * kb + 16 * (i >> 3) + 8 * h + (i & 7) > kmax) sacc[kb][i] = -INFINITY;
  }
  float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = (kb < 2 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
  mx = max_with_other_half(mx);
  const float mt = (MASKED && mx == -INFINITY) ? -INFINITY : mx * c;
  const float m_new = mt > m_run + kLazyRescale ? mt : m_run;
  const float m_ref = (MASKED && m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m_run - m_ref);
  // The row sum adds the fp32 p (the sum of the bf16-rounded operands would
  // put up to 2^-9 relative error into LSE when a few keys dominate a row).
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      float p0 = fast_exp2(fmaf(sacc[kb][i], c, -m_ref));
      float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -m_ref));
      if (MASKED) {
        p0 = sacc[kb][i] == -INFINITY ? 0.f : p0;
        p1 = sacc[kb][i + 1] == -INFINITY ? 0.f : p1;
      }
      ls0 += p0;
      ls1 += p1;
      pw[2 * kb + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(p0, p1);
    }
  l_run = fmaf(alpha, l_run, ls0 + ls1);
  m_run = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
  }
}

// Unmasked key tile of the ping-pong kernel, after the first tile of the
// range (so the running max m_run is finite): the exponentials are taken
// against m_run as it stands, without a row max. The running max only has
// to keep p = 2^(c s - m_run) from overflowing (the shift cancels in o / l),
// so a block's max is needed only when one of its scores has moved far past
// m_run, and that shows in the block's sum. Per 32-key block: if any lane's
// sum of its 16 p exceeds kFastSumLimit (or is inf or NaN), the wave takes
// the block's max, moves m_run to it, scales o, l and the tile's earlier
// blocks (sum and bf16 P) by alpha = 2^(m_old - m_new), and redoes the block
// (scores more than ~20 above the running max in base-2 units: almost never
// after a row's first tile).
constexpr float kFastSumLimit = 16777216.0f;  // 2^24

// x * a for the two bf16 halves of a packed word, repacked (round to nearest even).
__device__ __forceinline__ unsigned scale_bf16x2(unsigned w, float a) {
  return pack_bf16x2(__uint_as_float(w << 16) * a, __uint_as_float(w & 0xFFFF0000u) * a);
}

template <int DB, int NKB>
__device__ __forceinline__ void softmax_tile_running_max(f32x16* sacc, float c, float& m_run,
                                                         float& l_run, f32x16* oacc, u32x4* pw) {
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    float b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = fast_exp2(fmaf(sacc[kb][i], c, -m_run));
      const float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -m_run));
      b0 += p0;
      b1 += p1;
      pw[2 * kb + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(p0, p1);
    }
    float bs = b0 + b1;
    if (__any(!(bs <= kFastSumLimit))) {
      float mx = sacc[kb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      const float m_new = fmaxf(m_run, max_with_other_half(mx) * c);
      const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      l_run *= alpha;
      ls *= alpha;
#pragma unroll
      for (int t = 0; t < 2 * kb; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) pw[t][e] = scale_bf16x2(pw[t][e], alpha);
      m_run = m_new;
      b0 = b1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(fmaf(sacc[kb][i], c, -m_run));
        const float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -m_run));
        b0 += p0;
        b1 += p1;
        pw[2 * kb + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(p0, p1);
      }
      bs = b0 + b1;
    }
    ls += bs;
  }
  l_run += ls;
}

// One MFMA phase of the ping-pong schedule: O^T += V^T P^T for the current
// tile (second half of the keys, then first half) around S^T = K Q^T for
// the next tile (NKB independent chains that alternate, so that none waits
// on its own previous result). The score tile is complete well before the
// phase ends, so the next VALU phase can start on it at once. With DO_S
// false only the value product is issued (last tile).
template <int D, int BN, int NVMEM = 0, bool DO_S = true, bool DO_PV = true>
__device__ __forceinline__ void mfma_phase(const bf16* kt, const bf16* vt, const bf16x8* qf,
                                           const u32x4* pw, const VtOffsets& vo,
                                           const KOffsets<D>& ko, const bf16x8* pre, f32x16* sacc,
                                           f32x16* oacc) {
  using T = FwdTile<D, BN>;
  constexpr int NPV = DO_PV ? T::NT * T::DB : 0;
#pragma unroll
  for (int k = 0; k < NPV / 2; ++k) {
    const int t = pv_step_t<T::NT>(k, T::DB), db = k % T::DB;
    const bf16x8 vf = k < kPrefetch ? pre[k] : vt_read<D>(vt, vo, t, db);
    oacc[db] = mfma32x32x16(vf, as_bf16x8(pw[t]), oacc[db]);
  }
  if (DO_S) {
    f32x16 a[T::NKB];
#pragma unroll
    for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) a[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < T::DK; ++s)
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
        a[kb] = mfma32x32x16(k_read<D>(kt, ko, s, kb), qf[s], a[kb]);
#pragma unroll
    for (int kb = 0; kb < T::NKB; ++kb) sacc[kb] = a[kb];
  }
#pragma unroll
  for (int k = NPV / 2; k < NPV; ++k) {
    const int t = pv_step_t<T::NT>(k, T::DB), db = k % T::DB;
    oacc[db] = mfma32x32x16(vt_read<D>(vt, vo, t, db), as_bf16x8(pw[t]), oacc[db]);
  }
  // Issue order: global loads, then one LDS read after each MFMA, which
  // keeps kPrefetch operands in flight (without the prefetched value
  // operands, the first kPrefetch reads go ahead of the first MFMA).
  constexpr int NMFMA = NPV + (DO_S ? T::NKB * T::DK : 0);
  if (NVMEM > 0) __builtin_amdgcn_sched_group_barrier(0x020, NVMEM, 0);
  if (!DO_PV) __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + kPrefetch < NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Epilogue: O = o / l, LSE = ln 2 (m + log2 l), as bf16 (final result) or
// fp32 (PARTIAL: the result over one key range, merged later). A row that
// saw no visible key has l = 0 and m = -inf: O = 0, LSE = -inf.
template <int D, bool PARTIAL>
__device__ __forceinline__ void store_output(const f32x16* oacc, float m_run, float l_run,
                                             void* orow, float* lse, bool q_ok, int h) {
  const float l_tot = add_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!q_ok) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (PARTIAL) {
        const f32x4 w = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                         oacc[db][4 * r + 3] * inv};
        *(f32x4*)((float*)orow + 32 * db + 8 * r + 4 * h) = w;
      } else {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r + 0] * inv, oacc[db][4 * r + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
        *(u32x2*)((bf16*)orow + 32 * db + 8 * r + 4 * h) = w;
      }
    }
  if (h == 0) *lse = (m_run + fast_log2(l_tot)) * kLn2;
}

// Workgroup -> (head, query tile, key split). Causal launches put the query
// tiles that see the most keys first (consecutive workgroups take one query
// tile of every head and split, and the dispatcher starts them in order), so
// the short tiles fill in behind the long ones; other launches keep the query
// tiles of one head (which share K and V) on one XCD.
struct TileId {
  int bh, qt, split;
};
__device__ __forceinline__ TileId decode_tile(const FwdParams& p) {
  TileId t;
  int rest;
  if (p.causal) {
    const int hs = p.BH * p.n_splits;
    const int r = (int)blockIdx.x / hs;
    rest = (int)blockIdx.x - r * hs;
    t.qt = p.n_qtiles - 1 - r;
  } else {
    const int w = xcd_tile(blockIdx.x, p.total_tiles, p.remap);
    rest = w / p.n_qtiles;
    t.qt = w - rest * p.n_qtiles;
  }
  t.bh = rest / p.n_splits;
  t.split = rest - t.bh * p.n_splits;
  // The divisions above run on the vector unit; marking the results
  // wave-uniform keeps every address derived from them in scalar registers
  // (else each buffer_load ... lds would sit in a readfirstlane loop).
  t.bh = __builtin_amdgcn_readfirstlane(t.bh);
  t.qt = __builtin_amdgcn_readfirstlane(t.qt);
  t.split = __builtin_amdgcn_readfirstlane(t.split);
  return t;
}

// Keys one workgroup visits: the split's range [k_begin, k_end), cut short
// by the causal window of its last query (query i sees keys
// j <= i + Nk - Nq). n_tiles key tiles of BN keys hold a key some query of
// the tile sees; the first n_full of them are seen in full by every query of
// the tile and need no mask.
struct KeyRange {
  int k_begin, k_end, n_tiles, n_full;
};
template <int BN>
__device__ __forceinline__ KeyRange key_range(const FwdParams& p, int split, int q_lo, int bm) {
  KeyRange r;
  r.k_begin = split * p.split_keys;
  r.k_end = min(p.Nk, r.k_begin + p.split_keys);
  const int off = p.Nk - p.Nq;
  const int q_hi = min(q_lo + bm, p.Nq) - 1;
  const int lim = p.causal ? min(r.k_end, q_hi + off + 1) : r.k_end;
  r.n_tiles = lim > r.k_begin ? (lim - r.k_begin + BN - 1) / BN : 0;
  const int seen_by_all = (p.causal ? min(r.k_end, q_lo + off + 1) : r.k_end) - r.k_begin;
  r.n_full = seen_by_all > 0 ? seen_by_all / BN : 0;
  return r;
}
// Last key of the range that query q_row sees.
__device__ __forceinline__ int row_kmax(const FwdParams& p, const KeyRange& r, int q_row) {
  return p.causal ? min(r.k_end - 1, q_row + p.Nk - p.Nq) : r.k_end - 1;
}

// Writes one wave's rows: O and LSE, or the fp32 partial of the key split.
template <int D>
__device__ __forceinline__ void write_result(const FwdParams& p, const TileId& t, int q_row,
                                             bool q_ok, int h, const f32x16* oacc, float m_run,
                                             float l_run) {
  if (p.n_splits > 1) {
    const size_t row = ((size_t)t.split * p.BH + t.bh) * p.Nq + q_row;
    store_output<D, true>(oacc, m_run, l_run, p.o_part + row * D, p.lse_part + row, q_ok, h);
  } else {
    const size_t row = (size_t)t.bh * p.Nq + q_row;
    store_output<D, false>(oacc, m_run, l_run, (bf16*)p.o + row * D, p.lse + row, q_ok, h);
  }
}

// Result of a query tile none of whose queries sees a key of the range.
template <int D>
__device__ __forceinline__ void write_empty(const FwdParams& p, const TileId& t, int q_row,
                                            bool q_ok, int h) {
  f32x16 z[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) z[db][i] = 0.f;
  write_result<D>(p, t, q_row, q_ok, h, z, -INFINITY, 0.f);
}

// ---------------------------------------------------------------------------
// bf16 forward, generic: NW waves in lock step, one barrier per key tile.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 4 ? 2 : 1, 2)))
void attn_fwd_bf16_kernel(const FwdParams p) {
  using T = FwdTile<D>;
  constexpr int BM = 32 * NW;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::STAGE];
  auto ks = [&](int b) { return smem + b * T::STAGE; };
  auto vs = [&](int b) { return smem + b * T::STAGE + T::KTILE; };

  const TileId ti = decode_tile(p);
  const bf16* Kh = (const bf16*)p.k + (size_t)ti.bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc<D>(Kh, p.Nk);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc<D>((const bf16*)p.v + (size_t)ti.bh * p.Nk * D, p.Nk);
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addresses
  const int q_row = ti.qt * BM + wave * 32 + lq;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<T::BN>(p, ti.split, ti.qt * BM, BM);
  if (kr.n_tiles == 0) {
    write_empty<D>(p, ti, q_row, q_ok, h);
    return;
  }
  const int t0 = kr.k_begin / T::BN;  // first key tile of the range
  const int kmax = row_kmax(p, kr, q_row);
  const VtOffsets vo(lq, h);
  const KOffsets<D, true> ko(lq, h);

  bf16x8 qf[T::DK];
  load_q<D>((const bf16*)p.q + ((size_t)ti.bh * p.Nq + q_row) * D, q_ok, h, qf);

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = kr.n_tiles;
  // The next tile's K goes straight to LDS and its whole V into registers
  // at the start of a step; V is transposed into LDS after the step's value
  // product, so its loads have the whole step to arrive.
  const KDirect<D, 64, NW> kd(0, wave, lane);
  Stager<D, 64, NW * 64, 64, false> st;
  kd.load(Kh, p.Nk, t0, 64, ks(0));
  st.load(krs, vrs, t0, t0, 0, tid);
  st.store(ks(0), vs(0), 0, tid);
  wait_vmem();
  __syncthreads();

  auto step = [&](auto masked, int j) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = j & 1;
    const bool more = j + 1 < n_kt;
    if (more) {
      kd.template load<true>(Kh, p.Nk, t0 + j + 1, 64, ks(cur ^ 1));
      st.load(krs, vrs, t0 + j + 1, t0 + j + 1, 0, tid);
    }
    f32x16 sacc[2];
    u32x4 pw[4];
    score_tile<D>(ks(cur), qf, ko, sacc);
    softmax_tile<MASKED, T::DB>(sacc, p.c, kr.k_begin + j * T::BN, kmax, h, m_run, l_run, oacc, pw);
    pv_tile<D>(vs(cur), pw, vo, oacc);
    if (more) st.store(ks(cur ^ 1), vs(cur ^ 1), 0, tid);
    publish_lds();  // K tile written to LDS by its transfer, V^T by the stores
  };
  // Tiles from n_full on are masked; there are at most kMaxMaskedTiles.
  const int n_plain = min(kr.n_full, n_kt);
  int j = 0;
  for (; j < n_plain; ++j) step(std::false_type{}, j);
#pragma unroll
  for (int m = 0; m < kMaxMaskedTiles; ++m)
    if (j < n_kt) step(std::true_type{}, j++);
  write_result<D>(p, ti, q_row, q_ok, h, oacc, m_run, l_run);
}

// ---------------------------------------------------------------------------
// bf16 forward, keys split inside the workgroup: two groups of NW waves take
// the same BM = 32 NW queries, group 0 the first half of the key tiles and
// group 1 the second, each with LDS buffers of its own, in lock step (one
// barrier per key tile). At the end group 1 hands its running (m, l, o) to
// group 0 through LDS, and group 0 merges the two partial results exactly as
// the online update of the Lecture 17 page (§8.3) merges two key blocks:
// m = max(m0, m1), l = 2^(m0 - m) l0 + 2^(m1 - m) l1, o likewise. For grids
// of at most one wave per SIMD (few heads, short sequences) this puts a
// second wave on every SIMD, whose work hides the first one's latencies,
// without a second launch. Unmasked launches only: the ragged end of the
// key range is the only masked tile, and it is group 1's last.
// ---------------------------------------------------------------------------
// Key tiles of BN = 64 keys, or 128 at d = 64 (half the barriers per key,
// each step's products twice as many; the four tile stages then take
// 128 KiB of LDS, as at D = 128 with 64-key tiles), so one workgroup fits
// on a compute unit: with NW = 2 that is one wave per SIMD.
template <int D, int NW, int BN>
__global__ __launch_bounds__(2 * NW * 64) __attribute__((amdgpu_waves_per_eu(D == 128 && NW == 2 ? 1 : 2, 2)))
void attn_fwd_bf16_ksplit_kernel(const FwdParams p) {
  static_assert(BN == 64 || (BN == 128 && D == 64), "128-key tiles only at d = 64");
  using T = FwdTile<D, BN>;
  constexpr int BM = 32 * NW;
  constexpr int NE = 16 * T::DB + 2;  // floats one lane hands over: o, m, l
  static_assert(NW * NE * 64 * 4 <= 4 * T::STAGE * 2, "hand-over must fit the tile buffers");
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / NW, wave = wave_all - grp * NW;
  const int gtid = tid - grp * NW * 64;  // thread index within the group
  auto ks = [&](int b) { return smem + (2 * grp + b) * T::STAGE; };
  auto vs = [&](int b) { return smem + (2 * grp + b) * T::STAGE + T::KTILE; };

  const TileId ti = decode_tile(p);
  const bf16* Kh = (const bf16*)p.k + (size_t)ti.bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc<D>(Kh, p.Nk);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc<D>((const bf16*)p.v + (size_t)ti.bh * p.Nk * D, p.Nk);
  const int q_row = ti.qt * BM + wave * 32 + lq;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<T::BN>(p, 0, ti.qt * BM, BM);
  if (kr.n_tiles == 0) {
    if (grp == 0) write_empty<D>(p, ti, q_row, q_ok, h);
    return;
  }
  // Group 0 takes tiles [0, n_half), group 1 [n_half, n_kt); both run n_half
  // steps (group 1's last one idle when n_kt is odd).
  const int n_kt = kr.n_tiles, n_half = (n_kt + 1) / 2;
  const int my_first = grp ? n_half : 0, my_n = grp ? n_kt - n_half : n_half;
  const int t0 = kr.k_begin / T::BN + my_first;  // this group's first key tile
  const int kmax = row_kmax(p, kr, q_row);
  const VtOffsets vo(lq, h);
  const KOffsets<D, true> ko(lq, h);

  bf16x8 qf[T::DK];
  load_q<D>((const bf16*)p.q + ((size_t)ti.bh * p.Nq + q_row) * D, q_ok, h, qf);

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // The next tile's K goes straight to LDS and its whole V into registers
  // at the start of a step; V is transposed into LDS after the step's value
  // product, so its loads have the whole step to arrive.
  const KDirect<D, BN, NW> kd(0, wave, lane);
  Stager<D, BN, NW * 64, BN, false> st;
  if (my_n > 0) {
    kd.load(Kh, p.Nk, t0, BN, ks(0));
    st.load(krs, vrs, t0, t0, 0, gtid);
    st.store(ks(0), vs(0), 0, gtid);
  }
  wait_vmem();
  __syncthreads();

  // Step i of this group: its key tile my_first + i (local LDS buffer i & 1).
  auto step = [&](auto masked, int i) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = i & 1;
    const bool more = i + 1 < my_n;
    if (more) {
      kd.template load<true>(Kh, p.Nk, t0 + i + 1, BN, ks(cur ^ 1));
      st.load(krs, vrs, t0 + i + 1, t0 + i + 1, 0, gtid);
    }
    f32x16 sacc[T::NKB];
    u32x4 pw[T::NT];
    // A 128-key tile is two 64-key halves: K rows 64.. and the second V^T sub-tile.
#pragma unroll
    for (int hf = 0; hf < BN / 64; ++hf) score_tile<D>(ks(cur) + hf * 64 * D, qf, ko, sacc + 2 * hf);
    softmax_tile<MASKED, T::DB, T::NKB>(sacc, p.c, kr.k_begin + (my_first + i) * T::BN, kmax, h, m_run,
                                        l_run, oacc, pw);
#pragma unroll
    for (int hf = 0; hf < BN / 64; ++hf) pv_tile<D>(vs(cur) + hf * 64 * D, pw + 4 * hf, vo, oacc);
    if (more) st.store(ks(cur ^ 1), vs(cur ^ 1), 0, gtid);
    publish_lds();  // K tile written to LDS by its transfer, V^T by the stores
  };
  // Only the range's last tile (index n_full of a ragged end, group 1's
  // last) holds keys past the end. Each group runs n_half barriers.
  const int n_plain = min(max(kr.n_full - my_first, 0), my_n);
  int i = 0;
  for (; i < n_plain; ++i) step(std::false_type{}, i);
  if (i < my_n) step(std::true_type{}, i++);
  for (; i < n_half; ++i) publish_lds();  // the same barriers as a working step

  // Hand-over: group 1's lane values to LDS ([wave][element][lane]), group 0 merges.
  float* xb = (float*)smem + (size_t)wave * NE * 64 + lane;
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) xb[(16 * db + e) * 64] = oacc[db][e];
    xb[(NE - 2) * 64] = m_run;
    xb[(NE - 1) * 64] = l_run;
  }
  __syncthreads();
  if (grp == 1) return;
  const float m1 = xb[(NE - 2) * 64], l1 = xb[(NE - 1) * 64];
  const float m = fmaxf(m_run, m1);
  const float m_ref = m == -INFINITY ? 0.f : m;  // neither group saw a visible key
  const float a0 = fast_exp2(m_run - m_ref), a1 = fast_exp2(m1 - m_ref);
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = a0 * oacc[db][e] + a1 * xb[(16 * db + e) * 64];
  write_result<D>(p, ti, q_row, q_ok, h, oacc, m, a0 * l_run + a1 * l1);
}

// ---------------------------------------------------------------------------
// bf16 forward, ping-pong: 8 waves in two groups of 4 (one wave of each group
// per SIMD). Within a wave the work of one key tile is split into an MFMA
// phase (S^T of tile j+1 and O^T += V^T P^T of tile j) and a VALU phase
// (online softmax of tile j+1). Group B runs one phase behind group A, and
// every phase ends at a workgroup barrier, so on each SIMD one wave feeds
// the matrix core while the other wave computes exponentials: a wave's own
// VALU work does not overlap its own MFMAs, but another wave's does.
// K and V tiles are double-buffered; each group stages half of every V tile
// during its VALU phase (group A: V_{j+1}; group B, one phase later in time
// but one tile ahead: V_{j+2}), which keeps each buffer free until both
// groups have read it. 128-key K tiles go straight to LDS, sent whole by
// group A at the start of its MFMA phase j (K_{j+2}); 64-key K tiles go
// through registers, half by each group (K_{j+2}, K_{j+3}).
// ---------------------------------------------------------------------------
template <int D, int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_pingpong_kernel(const FwdParams p) {
  using T = FwdTile<D, BN>;
  constexpr int BM = 256;
  // With 64-key tiles each group issues the global loads of its staging
  // share at the start of its MFMA phase (a phase before writing them to
  // LDS); with 128-key tiles the staging registers would not fit beside the
  // larger score tile there, so the loads go out at the start of the VALU
  // phase and are written after the softmax.
  constexpr bool kEarlyLoads = BN == 64;
  // K is staged straight into LDS at 128-key width, through registers at 64
  constexpr bool kDirectK = BN == 128;
  using StG = Stager<D, BN / 2, 256, BN, !kDirectK>;
  constexpr int NVMEM = StG::KCPT + (StG::VPASS % StG::WAVES == 0 ? 2 * StG::VPW : 0);
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::STAGE];
  auto ks = [&](int b) { return smem + (b & 1) * T::STAGE; };
  auto vs = [&](int b) { return smem + (b & 1) * T::STAGE + T::KTILE; };

  const TileId ti = decode_tile(p);
  const bf16* Kh = (const bf16*)p.k + (size_t)ti.bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc<D>(Kh, p.Nk);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc<D>((const bf16*)p.v + (size_t)ti.bh * p.Nk * D, p.Nk);
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addresses
  const int grp = wave >> 2;          // 0: group A, 1: group B
  const int gtid = tid & 255;         // thread index within the group
  const int r0 = (BN / 2) * grp;      // rows of each tile this group stages
  const int q_row = ti.qt * BM + wave * 32 + lq;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<BN>(p, ti.split, ti.qt * BM, BM);
  if (kr.n_tiles == 0) {
    write_empty<D>(p, ti, q_row, q_ok, h);
    return;
  }
  // Key tiles are numbered from the range's first (t0 + local index); the
  // LDS buffers alternate with the local index.
  const int t0 = kr.k_begin / BN;
  const int kmax = row_kmax(p, kr, q_row);
  const VtOffsets vo(lq, h);
  const KOffsets<D> ko(lq, h);
  // With K staged straight into LDS (128-key tiles), group A sends the whole
  // of K_{j+2} at the start of its MFMA phase j: that buffer's last reader,
  // group B's MFMA phase j-1, is done, the phase itself reads only K_{j+1}
  // and V, and the transfer is waited for at the end of A's VALU phase j, a
  // phase before group A reads the tile. The transfers' issue time then
  // falls in the shorter MFMA phase instead of both groups' VALU phases.
  const KDirect<D, BN, 4> kda(0, wave & 3, lane);
  auto stage_k = [&](int t) {  // local K tile t, by group A (direct mode)
    if (kDirectK && grp == 0) kda.template load<true>(Kh, p.Nk, t0 + t, BN, ks(t));
  };

  bf16x8 qf[T::DK];
  load_q<D>((const bf16*)p.q + ((size_t)ti.bh * p.Nq + q_row) * D, q_ok, h, qf);

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int n_kt = kr.n_tiles;

  {  // prologue: everyone stages K_0, V_0 and K_1
    Stager<D, BN, 512, BN> st0;
    st0.load(krs, vrs, t0, t0, 0, tid);
    st0.store(ks(0), vs(0), 0, tid);
    st0.load(krs, vrs, t0 + 1, t0 + 1, 0, tid);
    st0.store(ks(1), vs(1), 0, tid);  // V_1 rows are restaged below; K_1 is final
  }
  __syncthreads();
  if (grp == 1) phase_barrier();

  f32x16 sacc[T::NKB];
  u32x4 pw[T::NT];
  bf16x8 pre[kPrefetch];  // first V^T operands of the next MFMA phase
  // Group A stages V_{j+1} in VALU phase j, group B V_{j+2} (and K through
  // registers, 64-key tiles: K_{j+2} and K_{j+3}).
  // Tiles past the end of the head are zero-filled without memory traffic;
  // tiles past the end of the range go into buffers no wave reads any more.
  StG st;

  // MFMA phase of tile 0: scores only
  mfma_phase<D, BN, 0, true, false>(ks(0), vs(0), qf, pw, vo, ko, pre, sacc, oacc);
  phase_barrier();
  if (grp == 1) st.load(krs, vrs, t0 + 2, t0 + 1, r0, gtid);  // VALU phase "j = -1"
  if (kr.n_full == 0)
    softmax_tile<true, T::DB, T::NKB>(sacc, p.c, kr.k_begin, kmax, h, m_run, l_run, oacc, pw);
  else
    softmax_tile<false, T::DB, T::NKB>(sacc, p.c, kr.k_begin, kmax, h, m_run, l_run, oacc, pw);
  if (grp == 1) st.store(ks(2), vs(1), r0, gtid);
  prefetch_pv<D, BN>(vs(0), vo, pre);
  if (kDirectK) wait_vmem();
  phase_barrier();

  auto body = [&](auto masked, int j) {
    constexpr bool MASKED = decltype(masked)::value;
    // MFMA phase: O^T += V^T P^T of tile j, S^T of tile j+1.
    const int tk = j + 2 + grp, tv = j + 1 + grp;
    if (kEarlyLoads) st.load(krs, vrs, t0 + tk, t0 + tv, r0, gtid);
    stage_k(j + 2);
    mfma_phase<D, BN, kEarlyLoads ? NVMEM : 0>(ks(j + 1), vs(j), qf, pw, vo, ko, pre, sacc, oacc);
    phase_barrier();
    // VALU phase: staging of later tiles (with early loads first, so that
    // the LDS writes drain under the softmax), online softmax of tile j+1,
    // and the first operand reads of the next MFMA phase.
    if (kEarlyLoads) {
      st.store(ks(tk), vs(tv), r0, gtid);
    } else {
      st.load(krs, vrs, t0 + tk, t0 + tv, r0, gtid);
    }
    if (MASKED)
      softmax_tile<true, T::DB, T::NKB>(sacc, p.c, kr.k_begin + (j + 1) * BN, kmax, h, m_run, l_run,
                                        oacc, pw);
    else
      softmax_tile_running_max<T::DB, T::NKB>(sacc, p.c, m_run, l_run, oacc, pw);
    if (!kEarlyLoads) st.store(ks(tk), vs(tv), r0, gtid);
    prefetch_pv<D, BN>(vs(j + 1), vo, pre);
    if (kDirectK) wait_vmem();  // K tile written to LDS
    phase_barrier();
  };
  // bodies j = 0 .. n_kt - 2 (body j takes the softmax of tile j + 1); the
  // tiles from n_full on hold keys some query may not see and are masked.
  // There are at most kMaxMaskedTiles of them (a 256-query tile's causal
  // window edge spans at most 255 keys, i.e. three 128-key tiles; a ragged
  // end adds no tile), so the masked bodies are unrolled: a loop of them
  // beside the loop of plain bodies would not fit the register file.
  const int n_body = n_kt - 1;
  const int n_plain = min(max(kr.n_full - 1, 0), n_body);
  int j = 0;
  for (; j < n_plain; ++j) body(std::false_type{}, j);
#pragma unroll
  for (int m = 0; m < kMaxMaskedTiles; ++m)
    if (j < n_body) body(std::true_type{}, j++);
  // last tile: value product only
  mfma_phase<D, BN, 0, false>(ks(j), vs(j), qf, pw, vo, ko, pre, sacc, oacc);
  phase_barrier();
  phase_barrier();
  if (grp == 0) phase_barrier();
  write_result<D>(p, ti, q_row, q_ok, h, oacc, m_run, l_run);
}

// ---------------------------------------------------------------------------
// bf16 forward for one query per head (decoding): a stream over K and V with
// no matrix product worth the matrix cores (an MFMA tile would leave 31 of
// its 32 query rows empty). Each key row is held by LPK = D / 8 lanes, 16
// bytes each: the score is a v_dot2 over the lane's 8 d-values reduced over
// its LPK lanes with DPP, and the lane's 8 output values take p * v. A wave
// takes 64-key blocks wave, wave + WAVES, ... of the workgroup's key range
// with all 2 * 64 * D * 2 bytes of a block's K and V loads in flight at
// once, keeps the running (m, l, o) of the online update (Lecture 17 page
// §8.3) per lane, and the waves merge theirs through LDS at the end.
// ---------------------------------------------------------------------------
template <int D>
struct DecodeCfg {
  static constexpr int WAVES = 4;
  static constexpr int LPK = D / 8;     // lanes per key row
  static constexpr int KPI = 64 / LPK;  // keys per load instruction: 4 (d = 128) or 8 (d = 64)
  static constexpr int KPB = 64;        // keys per wave and block
  static constexpr int U = KPB / KPI;   // load instructions per tensor and block
};

// Sum over the LPK = 8 or 16 lanes of a row group (DPP within rows of 16).
// Two packed bf16 from a 32-bit word. (A by-value argument on purpose:
// __builtin_bit_cast applied directly to an element of a vector value, as in
// bit_cast(T, v[j]), was compiled as a cast of element 0 for every j.)
__device__ __forceinline__ bf16x2_ev as_bf16x2(unsigned u) { return __builtin_bit_cast(bf16x2_ev, u); }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int LPK>
__device__ __forceinline__ float sum_lane_group(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);  // row_half_mirror: the other quad of each 8 lanes
  if (LPK == 16) x += dpp_f32<0x140>(x);  // row_mirror: the other half of each 16 lanes
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16_decode_kernel(const FwdParams p) {
  using C = DecodeCfg<D>;
  __shared__ float xch[C::WAVES][D + 2];  // per wave: o, m, l

  const TileId ti = decode_tile(p);  // one query tile (N_q = 1)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch = lane % C::LPK, kg = lane / C::LPK;  // d-chunk of the lane, key within a load
  const KeyRange kr = key_range<C::KPB>(p, ti.split, 0, 1);
  const int k_lim = row_kmax(p, kr, 0) + 1;  // first key past what the query sees
  const bf16* Kh = (const bf16*)p.k + (size_t)ti.bh * p.Nk * D;
  const bf16* Vh = (const bf16*)p.v + (size_t)ti.bh * p.Nk * D;
  const u32x4 qv = *(const u32x4*)((const bf16*)p.q + (size_t)ti.bh * D + 8 * ch);

  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's key group only

  for (int b = wave; b < kr.n_tiles; b += C::WAVES) {
    const int key0 = kr.k_begin + b * C::KPB;
    // Rows past N_k read as zero (range-checked resources over this block).
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(C::KPB, p.Nk - key0)));
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + (size_t)key0 * D), 0, rows * D * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vh + (size_t)key0 * D), 0, rows * D * 2, kBufferRsrcWord3);
    u32x4 kk[C::U], vv[C::U];
#pragma unroll
    for (int i = 0; i < C::U; ++i) kk[i] = buffer_load16_stream(krs, ((i * C::KPI + kg) * D + 8 * ch) * 2);
#pragma unroll
    for (int i = 0; i < C::U; ++i) vv[i] = buffer_load16_stream(vrs, ((i * C::KPI + kg) * D + 8 * ch) * 2);

    // Scores in the exp2 domain (c = scale log2 e); keys the query does not
    // see (past the split's range or the causal window) get -inf.
    float sc[C::U], bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kk[i][j]), as_bf16x2(qv[j]), a, false);
      a = sum_lane_group<C::LPK>(a) * p.c;
      sc[i] = key0 + i * C::KPI + kg < k_lim ? a : -INFINITY;
      bmax = fmaxf(bmax, sc[i]);
    }
    // Block maximum over the wave's key groups (lanes ^ LPK .. ^ 32).
#pragma unroll
    for (int x = C::LPK; x < 32; x *= 2) bmax = fmaxf(bmax, __shfl_xor(bmax, x, 64));
    bmax = max_with_other_half(bmax);
    const float m_new = fmaxf(m_run, bmax);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      const float pr = fast_exp2(sc[i] - m_ref);  // 0 for a key the query does not see
      l_run += pr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = fmaf(pr, __uint_as_float(vv[i][j] << 16), o[2 * j]);
        o[2 * j + 1] = fmaf(pr, __uint_as_float(vv[i][j] & 0xFFFF0000u), o[2 * j + 1]);
      }
    }
  }

  // Sum l and o over the wave's key groups; every lane then holds the
  // wave's totals for its d-chunk.
#pragma unroll
  for (int x = C::LPK; x < 32; x *= 2) {
    l_run += __shfl_xor(l_run, x, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], x, 64);
  }
  l_run = add_other_half(l_run);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = add_other_half(o[e]);
  if (kg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) xch[wave][8 * ch + e] = o[e];
    if (ch == 0) {
      xch[wave][D] = m_run;
      xch[wave][D + 1] = l_run;
    }
  }
  __syncthreads();
  if (wave != 0 || kg != 0) return;

  // Merge of the waves: m = max m_w, l = sum 2^(m_w - m) l_w, o likewise.
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::WAVES; ++w) m = fmaxf(m, xch[w][D]);
  const float m_ref = m == -INFINITY ? 0.f : m;  // no wave saw a visible key
  float l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < C::WAVES; ++w) {
    const float a = fast_exp2(xch[w][D] - m_ref);
    l = fmaf(a, xch[w][D + 1], l);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(a, xch[w][8 * ch + e], acc[e]);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = (m + fast_log2(l)) * kLn2;  // -inf for a row without keys
  if (p.n_splits > 1) {
    const size_t row = (size_t)ti.split * p.BH + ti.bh;
    f32x4 w0 = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    f32x4 w1 = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    *(f32x4*)(p.o_part + row * D + 8 * ch) = w0;
    *(f32x4*)(p.o_part + row * D + 8 * ch + 4) = w1;
    if (ch == 0) p.lse_part[row] = lse;
  } else {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
    *(u32x4*)((bf16*)p.o + (size_t)ti.bh * D + 8 * ch) = w;
    if (ch == 0) p.lse[ti.bh] = lse;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward (fp32 storage and arithmetic; v_mfma_f32_32x32x2_f32)
// ---------------------------------------------------------------------------
// Buffer resource over rows [row0, min(row0 + rows, n)) of a row-major
// fp32 [n, D] matrix: loads at or past the last of those rows return zeros
// without touching memory (no branch, and so no wait where paths would
// join). With row0 >= n the range is empty.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rows_rsrc(const float* base, int row0, int rows,
                                                                int n) {
  const int cnt = max(0, min(rows, n - row0));
  // The arguments are wave-uniform, but the compiler cannot always tell;
  // without these it puts every load in a loop over the distinct values.
  const uintptr_t a = (uintptr_t)(base + (size_t)row0 * D);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uintptr_t)hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(cnt * D * 4), kBufferRsrcWord3);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ f32x4 buffer_load_f32x4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

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
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const FwdParams p) {
  using C = FwdF32Cfg<D>;
  __shared__ float kt[C::BN * C::KPITCH];
  __shared__ float vt[C::BN * C::VPITCH];

  const TileId ti = decode_tile(p);
  const size_t kbase = (size_t)ti.bh * p.Nk * D;
  const float* K = (const float*)p.k;
  const float* V = (const float*)p.v;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addresses
  const int q_row = ti.qt * C::BM + wave * C::R + lq;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<C::BN>(p, ti.split, ti.qt * C::BM, C::BM);
  const int kmax = row_kmax(p, kr, q_row);

  float qf[C::DK];  // lane (query lq, half h) holds Q[q][2 s + h]
  const __amdgpu_buffer_rsrc_t qr = f32_rows_rsrc<D>((const float*)p.q + (size_t)ti.bh * p.Nq * D,
                                                     ti.qt * C::BM + wave * C::R, C::R, p.Nq);
#pragma unroll
  for (int s = 0; s < C::DK; ++s) qf[s] = buffer_load_f32(qr, 4 * (lq * D + 2 * s + h));

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // The next tile's K and V are loaded into registers while the current one
  // is worked on, and written to LDS after the workgroup is done with it.
  constexpr int EPT = C::BN * D / C::THREADS;  // elements of each tile per thread
  float kn[EPT], vn[EPT];
  auto load_tile = [&](int j) {
    const int key0 = kr.k_begin + j * C::BN;
    const __amdgpu_buffer_rsrc_t kr_ = f32_rows_rsrc<D>(K + kbase, key0, C::BN, p.Nk);
    const __amdgpu_buffer_rsrc_t vr_ = f32_rows_rsrc<D>(V + kbase, key0, C::BN, p.Nk);
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int e = tid + r * C::THREADS;  // element e of the tile: row e / D, column e % D
      kn[r] = buffer_load_f32(kr_, 4 * e);
      vn[r] = buffer_load_f32(vr_, 4 * e);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int e = tid + r * C::THREADS, row = e / D, col = e % D;
      kt[row * C::KPITCH + col] = kn[r];
      vt[row * C::VPITCH + col] = vn[r];
    }
  };
  if (kr.n_tiles > 0) load_tile(0);

  for (int j = 0; j < kr.n_tiles; ++j) {
    const int key0 = kr.k_begin + j * C::BN;
    store_tile();
    __syncthreads();
    if (j + 1 < kr.n_tiles) load_tile(j + 1);

    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < C::DK; ++s) sacc = mfma32x32x2f32(kt[lq * C::KPITCH + 2 * s + h], qf[s], sacc);

    // key of slot i: key0 + 8 (i/4) + 4 h + i%4; keys past kmax are dropped
    const bool masked = j >= kr.n_full;
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + 8 * (i >> 2) + 4 * h + (i & 3) > kmax) sacc[i] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = max_with_other_half(mx);
    // A row with no visible key so far keeps m = -inf, l = 0, o = 0.
    const float mt = mx == -INFINITY ? -INFINITY : mx * p.c;
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float pr[16], lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr[i] = fast_exp2(fmaf(sacc[i], p.c, -m_ref));
      if (masked && sacc[i] == -INFINITY) pr[i] = 0.f;
      lsum += pr[i];
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
        oacc[db] = mfma32x32x2f32(vt[key * C::VPITCH + 32 * db + lq], pr[s], oacc[db]);
    }
    __syncthreads();
  }

  const float l_tot = add_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    const bool part = p.n_splits > 1;
    const size_t row = part ? ((size_t)ti.split * p.BH + ti.bh) * p.Nq + q_row
                            : (size_t)ti.bh * p.Nq + q_row;
    float* orow = (part ? p.o_part : (float*)p.o) + row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(f32x4*)(orow + 32 * db + 8 * r + 4 * h) = w;
      }
    if (h == 0) (part ? p.lse_part : p.lse)[row] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward, keys split inside the workgroup: NG waves take the same 32
// queries, wave g every NG-th key tile (g, g + NG, ...), and at the end
// waves 1 .. NG-1 hand their running (m, l, o) to wave 0 through LDS, which
// merges them by the online update's rule (Lecture 17 page §8.3). Both
// operands that vary with the keys come straight from memory into registers
// (the next tile's while the current one is worked on), so the loop has no
// LDS traffic and no workgroup barrier. For small grids (few heads, short
// sequences): there 128-query workgroups keep only a few SIMDs busy, each
// with a long serial chain of fp32 MFMAs.
// ---------------------------------------------------------------------------
template <int D>
struct FwdF32SplitCfg {
  // Waves (key groups) per workgroup: one per SIMD, so that each has the
  // registers for its current and next tile's operands. A compute unit's
  // fp32 matrix rate is what it is, so more waves would not make one
  // workgroup finish sooner.
  static constexpr int NG = 4;
  static constexpr int BM = 32;
  static constexpr int BN = 32;
  static constexpr int DH = D / 2;        // d-values per lane half of the score operands
  static constexpr int DB = D / 32;
  static constexpr int NV = 16 * DB;      // V^T operand values per lane and tile
  static constexpr int NE = 16 * DB + 2;  // floats one lane hands over: o, m, l
};

template <int D>
__global__ __launch_bounds__(FwdF32SplitCfg<D>::NG * 64) void attn_fwd_f32_ksplit_kernel(
    const FwdParams p) {
  using C = FwdF32SplitCfg<D>;
  __shared__ float xch[(C::NG - 1) * C::NE * 64];

  const TileId ti = decode_tile(p);
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_row = ti.qt * C::BM + lq;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<C::BN>(p, ti.split, ti.qt * C::BM, C::BM);
  const int kmax = row_kmax(p, kr, q_row);
  const float* Kh = (const float*)p.k + (size_t)ti.bh * p.Nk * D;
  const float* Vh = (const float*)p.v + (size_t)ti.bh * p.Nk * D;

  // Score operands: step s of lane half h contracts d = h D/2 + s. Any
  // assignment of d to the steps gives the same dot product; this one makes
  // each lane's share of a Q or K row contiguous (16-byte loads).
  float qf[C::DH];
  {
    const __amdgpu_buffer_rsrc_t qr = f32_rows_rsrc<D>((const float*)p.q + (size_t)ti.bh * p.Nq * D,
                                                       ti.qt * C::BM, C::BM, p.Nq);
#pragma unroll
    for (int c = 0; c < C::DH / 4; ++c) {
      const f32x4 x = buffer_load_f32x4(qr, 4 * (lq * D + h * C::DH + 4 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e];
    }
  }

  // Tile j: K rows as the A operand of S^T = K Q^T (lane: key lq, its d-half
  // h), V^T as the A operand of O^T += V^T P^T (lane: d = 32 db + lq; step s
  // takes key 8 (s/4) + 4 h + s%4, the key of accumulator slot s of S^T).
  // Rows past N_k read as zero.
  auto load_tile = [&](int j, float* kd, float* vd) {
    const int key0 = kr.k_begin + j * C::BN;
    const __amdgpu_buffer_rsrc_t kr_ = f32_rows_rsrc<D>(Kh, key0, C::BN, p.Nk);
    const __amdgpu_buffer_rsrc_t vr_ = f32_rows_rsrc<D>(Vh, key0, C::BN, p.Nk);
#pragma unroll
    for (int c = 0; c < C::DH / 4; ++c) {
      const f32x4 x = buffer_load_f32x4(kr_, 4 * (lq * D + h * C::DH + 4 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) kd[4 * c + e] = x[e];
    }
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        vd[s * C::DB + db] = buffer_load_f32(vr_, 4 * ((8 * (s >> 2) + 4 * h + (s & 3)) * D + 32 * db + lq));
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_mine = kr.n_tiles > g ? (kr.n_tiles - g + C::NG - 1) / C::NG : 0;
  float kn[C::DH], vn[C::NV];
  if (n_mine > 0) load_tile(g, kn, vn);
  for (int i = 0; i < n_mine; ++i) {
    const int j = g + C::NG * i;
    const int key0 = kr.k_begin + j * C::BN;
    float kc[C::DH], vc[C::NV];
#pragma unroll
    for (int e = 0; e < C::DH; ++e) kc[e] = kn[e];
#pragma unroll
    for (int e = 0; e < C::NV; ++e) vc[e] = vn[e];
    // Unconditional (the last step reloads its own tile): a load under a
    // branch would make the compiler wait for it where the paths join.
    load_tile(i + 1 < n_mine ? j + C::NG : j, kn, vn);

    // Two independent accumulation chains over d, added at the end.
    f32x16 sa, sb;
#pragma unroll
    for (int e = 0; e < 16; ++e) sa[e] = sb[e] = 0.f;
#pragma unroll
    for (int s = 0; s < C::DH; s += 2) {
      sa = mfma32x32x2f32(kc[s], qf[s], sa);
      sb = mfma32x32x2f32(kc[s + 1], qf[s + 1], sb);
    }
    float sv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = sa[e] + sb[e];

    // key of slot e: key0 + 8 (e/4) + 4 h + e%4; keys past kmax are dropped
    const bool masked = j >= kr.n_full;
    if (masked) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 8 * (e >> 2) + 4 * h + (e & 3) > kmax) sv[e] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sv[e]);
    mx = max_with_other_half(mx);
    // A row with no visible key so far keeps m = -inf, l = 0, o = 0.
    const float mt = mx == -INFINITY ? -INFINITY : mx * p.c;
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float pr[16], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pr[e] = fast_exp2(fmaf(sv[e], p.c, -m_ref));
      if (masked && sv[e] == -INFINITY) pr[e] = 0.f;
      lsum += pr[e];
    }
    l_run = fmaf(alpha, l_run, lsum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = mfma32x32x2f32(vc[s * C::DB + db], pr[s], oacc[db]);
  }

  // Hand-over ([wave - 1][element][lane]) and merge in wave 0:
  // m = max_g m_g, l = sum_g 2^(m_g - m) l_g, o likewise.
  float* xb = xch + lane;
  if (g > 0) {
    float* w = xb + (size_t)(g - 1) * C::NE * 64;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) w[(16 * db + e) * 64] = oacc[db][e];
    w[(C::NE - 2) * 64] = m_run;
    w[(C::NE - 1) * 64] = l_run;
  }
  __syncthreads();
  if (g > 0) return;
  float m = m_run;
  for (int k = 0; k < C::NG - 1; ++k) m = fmaxf(m, xb[(k * C::NE + C::NE - 2) * 64]);
  const float m_ref = m == -INFINITY ? 0.f : m;  // no group saw a visible key
  const float a0 = fast_exp2(m_run - m_ref);
  float l = a0 * l_run;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] *= a0;
  for (int k = 0; k < C::NG - 1; ++k) {
    const float* r = xb + (size_t)k * C::NE * 64;
    const float a = fast_exp2(r[(C::NE - 2) * 64] - m_ref);
    l = fmaf(a, r[(C::NE - 1) * 64], l);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] = fmaf(a, r[(16 * db + e) * 64], oacc[db][e]);
  }

  const float l_tot = add_other_half(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    const bool part = p.n_splits > 1;
    const size_t row = part ? ((size_t)ti.split * p.BH + ti.bh) * p.Nq + q_row
                            : (size_t)ti.bh * p.Nq + q_row;
    float* orow = (part ? p.o_part : (float*)p.o) + row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(f32x4*)(orow + 32 * db + 8 * r + 4 * h) = w;
      }
    if (h == 0) (part ? p.lse_part : p.lse)[row] = (m + fast_log2(l_tot)) * kLn2;
  }
}

// fp32 key split for the smallest grids (d = 64): 16 queries per workgroup
// on v_mfma_f32_16x16x4_f32, so that a grid of few 32-query tiles (one head
// of 256 queries: 8 workgroups) spreads over twice the compute units; the
// fp32 matrix rate per SIMD is the same for both shapes. Four waves (key
// groups) per workgroup, one per SIMD, K and V straight from memory into
// registers, as in the 32-query kernel above. Lane l = 16 g + c holds query
// c of the tile; its accumulator slot 4 kb + i holds key 16 kb + 4 g + i of a
// 32-key tile, and the four lanes of a query (g = 0..3) hold its keys in
// turn, so the row maximum and sum take two cross-lane steps.
template <int D>
struct FwdF32Split16Cfg {
  static constexpr int NG = 4;         // waves (key groups) per workgroup
  static constexpr int BM = 16;        // queries per workgroup
  static constexpr int BN = 32;        // keys per tile: two 16-key blocks
  static constexpr int DQ = D / 4;     // d-values per lane group of the score operands
  static constexpr int DB = D / 16;    // 16-row blocks of O^T
  static constexpr int NV = 8 * DB;    // V operand values per lane and tile
  static constexpr int NE = 4 * DB + 2;  // floats one lane hands over: o, m, l
};

__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(FwdF32Split16Cfg<D>::NG * 64) void attn_fwd_f32_ksplit16_kernel(
    const FwdParams p) {
  using C = FwdF32Split16Cfg<D>;
  __shared__ float xch[(C::NG - 1) * C::NE * 64];

  const TileId ti = decode_tile(p);
  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_row = ti.qt * C::BM + lc;
  const bool q_ok = q_row < p.Nq;
  const KeyRange kr = key_range<C::BN>(p, ti.split, ti.qt * C::BM, C::BM);
  const int kmax = row_kmax(p, kr, q_row);
  const float* Kh = (const float*)p.k + (size_t)ti.bh * p.Nk * D;
  const float* Vh = (const float*)p.v + (size_t)ti.bh * p.Nk * D;

  // Score operands: step s of lane group lg contracts d = lg D/4 + s (any
  // assignment of d to the steps gives the same dot product; this one keeps
  // a lane's share of a Q or K row contiguous).
  float qf[C::DQ];
  {
    const __amdgpu_buffer_rsrc_t qr = f32_rows_rsrc<D>((const float*)p.q + (size_t)ti.bh * p.Nq * D,
                                                       ti.qt * C::BM, C::BM, p.Nq);
#pragma unroll
    for (int c = 0; c < C::DQ / 4; ++c) {
      const f32x4 x = buffer_load_f32x4(qr, 4 * (lc * D + lg * C::DQ + 4 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e];
    }
  }

  // Tile j: K rows as the A operand of S^T = K Q^T (block kb: lane holds key
  // 16 kb + lc, its d-quarter lg); V as the A operand of O^T += V^T P^T
  // (lane: d = 16 db + lc; step 4 kb + i takes key 16 kb + 4 lg + i, the key
  // of accumulator slot 4 kb + i). Rows past N_k read as zero.
  auto load_tile = [&](int j, float* kd, float* vd) {
    const int key0 = kr.k_begin + j * C::BN;
    const __amdgpu_buffer_rsrc_t kr_ = f32_rows_rsrc<D>(Kh, key0, C::BN, p.Nk);
    const __amdgpu_buffer_rsrc_t vr_ = f32_rows_rsrc<D>(Vh, key0, C::BN, p.Nk);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < C::DQ / 4; ++c) {
        const f32x4 x = buffer_load_f32x4(kr_, 4 * ((16 * kb + lc) * D + lg * C::DQ + 4 * c));
#pragma unroll
        for (int e = 0; e < 4; ++e) kd[kb * C::DQ + 4 * c + e] = x[e];
      }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        vd[t * C::DB + db] =
            buffer_load_f32(vr_, 4 * ((16 * (t >> 2) + 4 * lg + (t & 3)) * D + 16 * db + lc));
  };

  f32x4 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_mine = kr.n_tiles > g ? (kr.n_tiles - g + C::NG - 1) / C::NG : 0;
  float kn[2 * C::DQ], vn[C::NV];
  if (n_mine > 0) load_tile(g, kn, vn);
  for (int i = 0; i < n_mine; ++i) {
    const int j = g + C::NG * i;
    const int key0 = kr.k_begin + j * C::BN;
    float kc[2 * C::DQ], vc[C::NV];
#pragma unroll
    for (int e = 0; e < 2 * C::DQ; ++e) kc[e] = kn[e];
#pragma unroll
    for (int e = 0; e < C::NV; ++e) vc[e] = vn[e];
    // Unconditional (the last step reloads its own tile): a load under a
    // branch would make the compiler wait for it where the paths join.
    load_tile(i + 1 < n_mine ? j + C::NG : j, kn, vn);

    // S^T of the two 16-key blocks: two independent chains over d.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::DQ; ++s) {
      s0 = mfma16x16x4f32(kc[s], qf[s], s0);
      s1 = mfma16x16x4f32(kc[C::DQ + s], qf[s], s1);
    }
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = s0[e];
      sv[4 + e] = s1[e];
    }

    // key of slot e: key0 + 16 (e/4) + 4 lg + e%4; keys past kmax are dropped
    const bool masked = j >= kr.n_full;
    if (masked) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key0 + 16 * (e >> 2) + 4 * lg + (e & 3) > kmax) sv[e] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = max_with_other_half(mx);
    // A row with no visible key so far keeps m = -inf, l = 0, o = 0.
    const float mt = mx == -INFINITY ? -INFINITY : mx * p.c;
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float pr[8], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(fmaf(sv[e], p.c, -m_ref));
      if (masked && sv[e] == -INFINITY) pr[e] = 0.f;
      lsum += pr[e];
    }
    l_run = fmaf(alpha, l_run, lsum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[db][e] *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = mfma16x16x4f32(vc[t * C::DB + db], pr[t], oacc[db]);
  }

  // Hand-over ([wave - 1][element][lane]) and merge in wave 0:
  // m = max_g m_g, l = sum_g 2^(m_g - m) l_g, o likewise.
  float* xb = xch + lane;
  if (g > 0) {
    float* w = xb + (size_t)(g - 1) * C::NE * 64;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[(4 * db + e) * 64] = oacc[db][e];
    w[(C::NE - 2) * 64] = m_run;
    w[(C::NE - 1) * 64] = l_run;
  }
  __syncthreads();
  if (g > 0) return;
  float m = m_run;
  for (int k = 0; k < C::NG - 1; ++k) m = fmaxf(m, xb[(k * C::NE + C::NE - 2) * 64]);
  const float m_ref = m == -INFINITY ? 0.f : m;  // no group saw a visible key
  const float a0 = fast_exp2(m_run - m_ref);
  float l = a0 * l_run;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[db][e] *= a0;
  for (int k = 0; k < C::NG - 1; ++k) {
    const float* r = xb + (size_t)k * C::NE * 64;
    const float a = fast_exp2(r[(C::NE - 2) * 64] - m_ref);
    l = fmaf(a, r[(C::NE - 1) * 64], l);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[db][e] = fmaf(a, r[(4 * db + e) * 64], oacc[db][e]);
  }

  // each lane summed its own keys: add the query's four lanes
  float l_tot = l + __shfl_xor(l, 16, 64);
  l_tot = add_other_half(l_tot);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    const bool part = p.n_splits > 1;
    const size_t row = part ? ((size_t)ti.split * p.BH + ti.bh) * p.Nq + q_row
                            : (size_t)ti.bh * p.Nq + q_row;
    float* orow = (part ? p.o_part : (float*)p.o) + row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const f32x4 w = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
      *(f32x4*)(orow + 16 * db + 4 * lg) = w;
    }
    if (lg == 0) (part ? p.lse_part : p.lse)[row] = (m + fast_log2(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// merge of key-split partial results
// ---------------------------------------------------------------------------
// For each row: LSE = ln sum_r e^(LSE_r), O = sum_r e^(LSE_r - LSE) O_r, with
// the largest LSE_r subtracted first; parts with LSE_r = -inf weigh 0 and a
// row whose parts are all empty gets O = 0, LSE = -inf. This is the
// rescaling of the online update (Lecture 17 page §8.3) applied to partial
// results written back to memory (CS336 Lecture 5 transcript, FlashAttention
// passage). One row per D / 4 threads, 16-byte accesses; memory-bound.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         int n_parts, int64_t rows,
                                                         void* __restrict__ o,
                                                         float* __restrict__ lse) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int r = 0; r < n_parts; ++r) mx = fmaxf(mx, lse_part[r * rows + row]);
  const float shift = mx == -INFINITY ? 0.f : mx;
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < n_parts; ++r) {
    const float w = expf(lse_part[r * rows + row] - shift);  // 0 for an empty part
    const f32x4 x = *(const f32x4*)(o_part + ((size_t)r * rows + row) * D + 4 * part);
    wsum += w;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, x[e], acc[e]);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (OUT_F32) {
    const f32x4 y = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *(f32x4*)((float*)o + row * D + 4 * part) = y;
  } else {
    u32x2 y;
    y[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    y[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(u32x2*)((bf16*)o + row * D + 4 * part) = y;
  }
  if (part == 0) lse[row] = wsum > 0.f ? shift + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Keys per ping-pong phase: 128 halves the number of phases (and so the
// per-phase cost of barriers and of refilling the operand pipeline).
constexpr int kPingPongBN = 128;
constexpr int kSplitAlign = 128;  // split boundaries fall on whole key tiles of every kernel

int64_t split_keys_for(int64_t Nk, int n_splits) {
  const int64_t tiles = (Nk + kSplitAlign - 1) / kSplitAlign;
  const int64_t per = (tiles + n_splits - 1) / n_splits;
  return (per > 0 ? per : 1) * kSplitAlign;
}

static FwdParams make_params(const FwdArgs& a, int bm, int64_t* total_out) {
  FwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.Nq = (int)a.Nq;
  p.Nk = (int)a.Nk;
  p.BH = (int)a.BH;
  p.n_qtiles = (int)((a.Nq + bm - 1) / bm);
  const int64_t sk = a.n_splits > 1 ? split_keys_for(a.Nk, a.n_splits) : 0;
  p.n_splits = a.n_splits > 1 ? (int)((a.Nk + sk - 1) / sk) : 1;
  p.split_keys = a.n_splits > 1 ? (int)sk : (int)(((a.Nk + kSplitAlign - 1) / kSplitAlign) * kSplitAlign);
  if (p.split_keys == 0) p.split_keys = kSplitAlign;
  if (p.n_splits > 1) {
    p.o_part = a.partial;
    p.lse_part = a.partial + (size_t)p.n_splits * a.BH * a.Nq * a.d;
  }
  const int64_t total = (int64_t)a.BH * p.n_qtiles * p.n_splits;
  p.total_tiles = (int)total;
  p.c = a.scale * kLog2e;
  p.causal = a.causal ? 1 : 0;
  p.remap = (!a.causal && total % 8 == 0) ? 1 : 0;
  *total_out = total;
  return p;
}

// The one launch of an attention kernel in a forward call. The caller's
// events, when given, are bound to the start and the end of this dispatch
// (hipExtLaunchKernel), so that their elapsed time is the kernel's own,
// without marker commands between back-to-back launches.
static hipError_t launch_fwd_kernel(void (*kernel)(FwdParams), int64_t total, int threads, const FwdArgs& a,
                                    const FwdParams& p) {
  FwdParams arg = p;
  void* args[] = {&arg};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)total),
                                          dim3(threads), args, 0, (hipStream_t)a.stream, (hipEvent_t)a.ev_start,
                                          (hipEvent_t)a.ev_stop, 0);
  const hipError_t last = hipGetLastError();
  return e != hipSuccess ? e : last;
}

template <int D, int NW>
static hipError_t launch_bf16(const FwdArgs& a, const FwdParams& p, int64_t total) {
  if constexpr (NW == 8)
    return launch_fwd_kernel(attn_fwd_bf16_pingpong_kernel<D, kPingPongBN>, total, 512, a, p);
  else
    return launch_fwd_kernel(attn_fwd_bf16_kernel<D, NW>, total, NW * 64, a, p);
}

template <int D>
static hipError_t launch_bf16_decode(const FwdArgs& a, const FwdParams& p, int64_t total) {
  return launch_fwd_kernel(attn_fwd_bf16_decode_kernel<D>, total, DecodeCfg<D>::WAVES * 64, a, p);
}

template <int D, int NW, int BN = 64>
static hipError_t launch_bf16_ksplit(const FwdArgs& a, const FwdParams& p, int64_t total) {
  return launch_fwd_kernel(attn_fwd_bf16_ksplit_kernel<D, NW, BN>, total, 2 * NW * 64, a, p);
}

// Key tile of the key-split kernel at d = 64: 128 keys when the grid holds
// more than half as many workgroups as compute units and each wave group
// gets at least four such tiles (N_k >= 1024); fewer or shorter sweeps
// measured faster with 64-key tiles (the 128-key pipeline's first tile and
// hand-over weigh more there).
static int ksplit_bn(const FwdArgs& a, int64_t total) {
  if (a.d != 64) return 64;
  if (a.ksplit_bn == 64 || a.ksplit_bn == 128) return a.ksplit_bn;
  return (2 * total > (int64_t)a.num_cus && a.Nk >= 1024) ? 128 : 64;
}

// Whether to split a workgroup's keys between two wave groups: for unmasked
// launches without key splits on the smaller tiles, when the grid holds at
// most one wave per SIMD and each group gets at least two 64-key tiles.
static bool use_ksplit(const FwdArgs& a, int64_t splits, int nw) {
  if (a.causal || splits != 1 || nw >= 8 || a.ksplit == 1) return false;
  if (a.ksplit == 2) return true;
  const int64_t waves_total = a.BH * ((a.Nq + 31) / 32);
  return waves_total <= 4 * (int64_t)a.num_cus && (a.Nk + 63) / 64 >= 4;
}

template <int D>
static hipError_t launch_f32(const FwdArgs& a, const FwdParams& p, int64_t total, bool ksplit, bool small) {
  if constexpr (D == 64) {
    if (small)
      return launch_fwd_kernel(attn_fwd_f32_ksplit16_kernel<D>, total, FwdF32Split16Cfg<D>::NG * 64, a, p);
  }
  if (ksplit) return launch_fwd_kernel(attn_fwd_f32_ksplit_kernel<D>, total, FwdF32SplitCfg<D>::NG * 64, a, p);
  return launch_fwd_kernel(attn_fwd_f32_kernel<D>, total, FwdF32Cfg<D>::THREADS, a, p);
}

// fp32: split each workgroup's keys between its waves (32 queries per
// workgroup) when 128-query workgroups would not cover every compute unit.
static bool use_f32_ksplit(const FwdArgs& a) {
  if (a.ksplit == 1) return false;
  if (a.ksplit == 2) return true;
  const int64_t tiles = a.BH * ((a.Nq + FwdF32Cfg<64>::BM - 1) / FwdF32Cfg<64>::BM) *
                        (a.n_splits > 1 ? a.n_splits : 1);
  return tiles < (int64_t)a.num_cus;
}

// fp32 at d = 64: 16-query tiles (the 16x16x4 kernel) when even the key
// split's 32-query tiles would leave more than half of the compute units idle.
static bool use_f32_small(const FwdArgs& a, bool ksplit) {
  if (a.d != 64 || !ksplit || a.f32_bm == 32) return false;
  if (a.f32_bm == 16) return true;
  const int64_t tiles = a.BH * ((a.Nq + FwdF32SplitCfg<64>::BM - 1) / FwdF32SplitCfg<64>::BM) *
                        (a.n_splits > 1 ? a.n_splits : 1);
  return 2 * tiles <= (int64_t)a.num_cus;
}

// Workgroup size choice: the largest query tile whose grid (with the key
// splits) still covers every compute unit at least once (wave quantization,
// CS336 Lecture 5 notes §6.2), else the smallest; tiles of more than twice
// the query count (mostly empty rows, as in decoding) are passed over.
int fwd_bf16_waves(int64_t BH, int64_t Nq, int64_t splits, int num_cus) {
  for (int nw : {8, 4}) {
    if (32 * nw > 2 * Nq) continue;
    const int64_t tiles = BH * ((Nq + 32 * nw - 1) / (32 * nw)) * splits;
    if (tiles >= num_cus) return nw;
  }
  return 2;
}

// Key splits when the query tiles alone leave compute units idle (few
// query tiles per head, as for one device's query shard or in decoding,
// Lecture 17 page §9.2). With at least 128 queries the 256-query ping-pong
// tiles are split until they fill the chip once (each split keeping at least
// four 128-key tiles); with fewer, the smaller tiles are split for about two
// workgroups per compute unit (each split at least two 128-key tiles).
// min_pp_tiles: the fewest 128-key tiles a split of the 256-query ping-pong
// tiles may hold.
static int auto_splits(int64_t BH, int64_t Nq, int64_t Nk, bool fp32, int num_cus, int64_t min_pp_tiles) {
  const int64_t key_tiles = (Nk + kSplitAlign - 1) / kSplitAlign;
  auto clamp_splits = [&](int64_t s, int64_t min_tiles) -> int {
    s = s < key_tiles / min_tiles ? s : key_tiles / min_tiles;
    if (s < 2) return 1;
    return (int)(s < kMaxSplits ? s : kMaxSplits);
  };
  if (!fp32 && Nq == 1) {
    // One query per head (the one-query kernel): about one workgroup per
    // compute unit, each split at least four 128-key tiles. More and
    // shorter streams measured slower on the decode workload (2 splits:
    // 5.8 TB/s, 4: 5.1 TB/s), and the merge is a launch of its own.
    return clamp_splits((num_cus + BH - 1) / BH, 4);
  }
  if (!fp32 && Nq >= 128) {
    const int64_t t8 = BH * ((Nq + 255) / 256);
    if (t8 >= num_cus) return 1;
    const int s = clamp_splits((num_cus + t8 - 1) / t8, min_pp_tiles);
    // Split the 256-query tiles only where that fills at least half a round.
    if (s > 1 && 2 * t8 * s >= num_cus) return s;
  }
  const int bm = fp32 ? FwdF32Cfg<64>::BM : 32 * fwd_bf16_waves(BH, Nq, 1, num_cus);
  const int64_t tiles = BH * ((Nq + bm - 1) / bm);
  if (tiles <= 0 || tiles >= num_cus) return 1;
  return clamp_splits((2 * (int64_t)num_cus + tiles - 1) / tiles, fp32 ? 2 : 4);
}

// Split counts of a whole launch: splits of the ping-pong tiles keep at
// least 16 key tiles (2048 keys) and fill at least half a round. With
// shorter ranges the smaller unsplit tiles measured faster than a split and
// its merge (B=1 H=16 N=2048: 41.6 µs unsplit in 4-wave tiles against 48.9
// µs with 2 splits; B=2 H=10 N=2048 66.2 against 74.6), with 2048 keys a
// split measured equal or better (B=1 H=12 N=4096: 121.2 against 127.4 µs),
// and the query shard's long range (16384 keys) gains most (308 -> 244 µs).
// Grids too small for that split the smaller tiles instead, each split at
// least 4 key tiles in bf16 (B=1 H=2 N=4096: 4 splits 36.7 µs against 59.1
// µs for 2 splits of the ping-pong tiles; B=1 H=4 N=2048: 27.6 against 33.1
// µs unsplit).
int fwd_auto_splits(int64_t BH, int64_t Nq, int64_t Nk, bool fp32, int num_cus) {
  return auto_splits(BH, Nq, Nk, fp32, num_cus, 16);
}

// Wave quantization of the last round (CS336 Lecture 5 notes §6.2): a bf16
// grid of 256-query tiles whose workgroup count exceeds the CU count by a
// remainder of at most half the CUs runs that remainder as a round of its own
// with most of the chip idle. Splitting the keys of only the heads in that
// last round fills the chip for it; measured with the two launches made
// separately: 18 heads of N = 4096 (a last round 1/8 full) 200.7 -> 155.8 µs,
// 20 heads (1/4) 201.1 -> 167.5 µs, 24 heads (1/2) 208.7 -> 195.0 µs, 40
// heads (2.5 rounds) 319.4 -> 311.8 µs.
bool fwd_tail_plan(int64_t BH, int64_t Nq, int64_t Nk, bool fp32, bool causal, int num_cus, FwdTailPlan* plan) {
  if (fp32 || causal || Nq < 128 || num_cus <= 0 || BH < 2) return false;
  if (fwd_bf16_waves(BH, Nq, 1, num_cus) != 8) return false;
  const int64_t tpw = (Nq + 255) / 256;  // 256-query tiles per head
  const int64_t total = BH * tpw;
  const int64_t rem = total % num_cus;
  if (total <= num_cus || rem == 0 || 2 * rem > num_cus) return false;
  const int64_t head_split = (total - rem) / tpw;  // heads of the whole rounds
  const int64_t tail = BH - head_split;
  if (head_split < 1 || tail < 1 || head_split * tpw < num_cus) return false;
  // The tail heads alone leave most of the chip idle: their splits may be
  // as short as 4 key tiles (2 heads of N = 4096: 8 splits).
  const int s = auto_splits(tail, Nq, Nk, false, num_cus, 4);
  if (s < 2) return false;
  plan->head_split = head_split;
  plan->tail_splits = s;
  return true;
}

static hipError_t launch_attn_fwd_one(const FwdArgs& a);

hipError_t launch_attn_fwd(const FwdArgs& a) {
  if (a.tail_heads <= 0) return launch_attn_fwd_one(a);
  // The heads of the whole rounds, unsplit, then the tail heads with their
  // key splits, on the same stream. The caller's start event goes with the
  // first attention launch, the stop event with the second.
  const int64_t h1 = a.BH - a.tail_heads;
  FwdArgs b = a;
  b.BH = h1;
  b.n_splits = 1;
  b.tail_heads = 0;
  b.ev_stop = nullptr;
  hipError_t e = launch_attn_fwd_one(b);
  if (e != hipSuccess) return e;
  FwdArgs t = a;
  const size_t qo = (size_t)h1 * a.Nq * a.d * 2, kv = (size_t)h1 * a.Nk * a.d * 2;
  t.q = (const char*)a.q + qo;
  t.k = (const char*)a.k + kv;
  t.v = (const char*)a.v + kv;
  t.o = (char*)a.o + qo;
  t.lse = a.lse + (size_t)h1 * a.Nq;
  t.BH = a.tail_heads;
  t.n_splits = a.tail_splits;
  t.tail_heads = 0;
  t.ev_start = nullptr;
  return launch_attn_fwd_one(t);
}

static hipError_t launch_attn_fwd_one(const FwdArgs& a) {
  int64_t total = 0;
  if (a.dtype_fp32) {
    const bool ks = use_f32_ksplit(a), small = use_f32_small(a, ks);
    const FwdParams p = make_params(a, small ? FwdF32Split16Cfg<64>::BM : ks ? FwdF32SplitCfg<64>::BM
                                                                          : FwdF32Cfg<64>::BM, &total);
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipError_t e = a.d == 64 ? launch_f32<64>(a, p, total, ks, small) : launch_f32<128>(a, p, total, ks, false);
    if (e != hipSuccess || p.n_splits == 1) return e;
    return launch_attn_merge(p.o_part, p.lse_part, p.n_splits, a.BH * a.Nq, a.d, a.o, a.lse, true,
                             a.stream);
  }
  const int64_t splits = a.n_splits > 1 ? (a.Nk + split_keys_for(a.Nk, a.n_splits) - 1) /
                                               split_keys_for(a.Nk, a.n_splits)
                                         : 1;
  if (a.Nq == 1 && a.decode != 1) {
    const FwdParams p = make_params(a, 1, &total);
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipError_t e = a.d == 64 ? launch_bf16_decode<64>(a, p, total) : launch_bf16_decode<128>(a, p, total);
    if (e != hipSuccess || p.n_splits == 1) return e;
    return launch_attn_merge(p.o_part, p.lse_part, p.n_splits, a.BH * a.Nq, a.d, a.o, a.lse, false,
                             a.stream);
  }
  const int nw = a.waves ? a.waves : fwd_bf16_waves(a.BH, a.Nq, splits, a.num_cus);
  const FwdParams p = make_params(a, 32 * nw, &total);
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipError_t e;
  if (use_ksplit(a, splits, nw)) {
    if (a.d == 64 && ksplit_bn(a, total) == 128)
      e = nw == 4 ? launch_bf16_ksplit<64, 4, 128>(a, p, total) : launch_bf16_ksplit<64, 2, 128>(a, p, total);
    else if (a.d == 64)
      e = nw == 4 ? launch_bf16_ksplit<64, 4>(a, p, total) : launch_bf16_ksplit<64, 2>(a, p, total);
    else
      e = nw == 4 ? launch_bf16_ksplit<128, 4>(a, p, total) : launch_bf16_ksplit<128, 2>(a, p, total);
  } else if (a.d == 64) {
    e = nw == 8 ? launch_bf16<64, 8>(a, p, total) : nw == 4 ? launch_bf16<64, 4>(a, p, total)
                                                           : launch_bf16<64, 2>(a, p, total);
  } else {
    e = nw == 8 ? launch_bf16<128, 8>(a, p, total) : nw == 4 ? launch_bf16<128, 4>(a, p, total)
                                                             : launch_bf16<128, 2>(a, p, total);
  }
  if (e != hipSuccess || p.n_splits == 1) return e;
  return launch_attn_merge(p.o_part, p.lse_part, p.n_splits, a.BH * a.Nq, a.d, a.o, a.lse, false,
                           a.stream);
}

hipError_t launch_attn_merge(const float* o_part, const float* lse_part, int n_parts, int64_t rows,
                             int64_t d, void* o, float* lse, bool out_fp32, void* stream) {
  const int64_t threads = rows * (d / 4);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const hipStream_t st = (hipStream_t)stream;
  if (d == 64) {
    if (out_fp32)
      hipLaunchKernelGGL((attn_merge_kernel<64, true>), dim3((unsigned)blocks), dim3(256), 0, st, o_part,
                         lse_part, n_parts, rows, o, lse);
    else
      hipLaunchKernelGGL((attn_merge_kernel<64, false>), dim3((unsigned)blocks), dim3(256), 0, st, o_part,
                         lse_part, n_parts, rows, o, lse);
  } else {
    if (out_fp32)
      hipLaunchKernelGGL((attn_merge_kernel<128, true>), dim3((unsigned)blocks), dim3(256), 0, st, o_part,
                         lse_part, n_parts, rows, o, lse);
    else
      hipLaunchKernelGGL((attn_merge_kernel<128, false>), dim3((unsigned)blocks), dim3(256), 0, st, o_part,
                         lse_part, n_parts, rows, o, lse);
  }
  return hipGetLastError();
}

}  // namespace tattn
