// Tile building blocks of the bf16 attention kernels (gfx950): LDS layouts of
// row-major K-like tiles and transposed V^T-like tiles, their staging from
// HBM (buffer loads with range checks, buffer_load ... lds, and a register
// transpose), and the two MFMA products they feed. The forward uses them for
// S^T = K Q^T and O^T += V^T P^T; the backward's dQ sweep uses the same
// shapes for S^T = K Q^T, dP^T = V dO^T and dQ^T += K^T dS^T.
#pragma once

#include "device_common.h"

namespace tattn {

template <int D, int BN_ = 64>
struct FwdTile {
  static constexpr int BN = BN_;             // keys per step (64 or 128)
  static constexpr int NKB = BN / 32;        // 32-key blocks of a score tile
  static constexpr int NT = BN / 16;         // 16-key steps of the value product
  static constexpr int KTILE = BN * D;       // K tile, bf16 elements (rows of D, chunk-swizzled)
  static constexpr int VTILE = D * BN;       // V^T tile: D rows of BN keys, no padding
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int DK = D / 16;          // k-steps of the score product
  static constexpr int DB = D / 32;          // 32-wide blocks of d
  static constexpr int CPR = D / 8;          // 16-byte chunks per K or V row
  static constexpr int VKEYS = 128 / CPR;    // keys one wave transposes per pass
};

// K tiles hold key swap23(r) at LDS row r (rows of D bf16, no padding); the
// 16-byte chunk c of row r sits at chunk position c ^ kswz(r). An operand
// read touches 16 consecutive rows at one logical chunk: for D = 128
// (256-byte rows) kswz(r) = r & 15 spreads them over the 16 chunk positions
// of a bank period, for D = 64 (128-byte rows, two per period)
// (r & 1, kswz(r)) = (r & 1, (r >> 1) & 7) does. kswz(32 b + r) = kswz(r).
// The layout is written lane-linearly by buffer_load ... lds (1 KB per
// instruction), so no padding is possible and the swizzle is what keeps the
// reads free of bank conflicts.
//
// SW = 1 is a second swizzle for tiles that are also read transposed
// (ds_read_b64_tr_b16, the backward's dK/dV sweep): such a read touches, per
// half wave, rows of 4 consecutive keys (bits 0-1 of r vary) at 4 consecutive
// logical chunks. SW = 1 permutes the bits of the same row bits so that
// those 16 (row, chunk) pairs land on 16 distinct chunk positions (D = 128:
// bits 0-1 of r go to bits 2-3 of the swizzle; D = 64: bit 1 goes to bit 2,
// and bit 0 already selects the bank half), while 16 consecutive rows still
// map one-to-one, so both read kinds are free of bank conflicts.
template <int D, int SW = 0>
__device__ __forceinline__ int kswz(int r) {
  if (SW == 0) return D == 128 ? (r & 15) : ((r >> 1) & 7);
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane element offsets of the K operand reads: step s of key block kb
// (row 32 kb + lq, logical chunk 2 s + h) is at o(s) + 32 kb D, where
// o(s) = lq D + 8 ((2 s + h) ^ kswz(lq)) = (lq D + 8 (h ^ kswz(lq))) ^ 16 s
// (the chunk bits sit below the row bits). COMPACT keeps one register and
// does the XOR per read; otherwise all D / 16 offsets are kept.
template <int D, bool COMPACT = false, int SW = 0>
struct KOffsets {
  int o[COMPACT ? 1 : D / 16];
  __device__ __forceinline__ KOffsets(int lq, int h) {
    if (COMPACT) {
      o[0] = lq * D + 8 * (h ^ kswz<D, SW>(lq));
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) o[s] = lq * D + 8 * ((2 * s + h) ^ kswz<D, SW>(lq));
    }
  }
  __device__ __forceinline__ int at(int s) const { return COMPACT ? (o[0] ^ (16 * s)) : o[s]; }
};

template <int D, bool COMPACT, int SW>
__device__ __forceinline__ bf16x8 k_read(const bf16* kt, const KOffsets<D, COMPACT, SW>& ko, int s,
                                         int kb) {
  return as_bf16x8(*(const u32x4*)(kt + ko.at(s) + 32 * kb * D));
}

// A V^T tile of BN keys is BN / 64 sub-tiles of D rows x 64 keys (128-byte
// rows). vt_swz is the XOR swizzle of the 8 sixteen-byte slots of row d:
// reads of one MFMA operand touch 16 consecutive rows at one logical slot,
// and (d & 1, vt_swz(d)) is distinct across them (no read conflict); the
// transposed writes touch rows d = 8r + e (r = 0..15) at one slot, where
// vt_swz takes each value twice (two-way write conflict). Also
// vt_swz(32 b + x) = vt_swz(x) ^ 2 b for x < 32, b < 4.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

// Buffer resource over one head's [N, D] K or V slice. A load whose byte
// offset is at or past N * D * 2 returns zeros without touching memory,
// which is how rows >= N of a ragged last tile are staged (no branches).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16* base, int N) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, N * D * 2, kBufferRsrcWord3);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// The same load for data read once, as a stream: cache policy NT
// (nontemporal; bit 1 of the policy operand on gfx950). On the one-query
// kernel's K and V stream it raised the achieved HBM read rate from 5.8 to
// 6.7 TB/s (a plain read probe: 6.4 against 7.1 TB/s).
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// Per-lane element offsets of the V^T operand reads: the A operand of step t,
// d block db (rows d = 32 db + lq, keys 16 t + 8 h .. + 7) sits in sub-tile
// t / 4 at o[(t % 4) ^ db] + db * 32 * 64. With d = 32 db + lq,
// vt_swz(d) = f0 ^ 2 db for f0 = vt_swz(lq), so the swizzled slot
// (2 (t % 4) + h) ^ vt_swz(d) equals (2 ((t % 4) ^ db) + h) ^ f0: four
// per-lane offsets serve every read.
struct VtOffsets {
  int o[4];
  __device__ __forceinline__ VtOffsets(int lq, int h) {
    const int f0 = vt_swz(lq);
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = lq * 64 + 8 * ((2 * u + h) ^ f0);
  }
};

template <int D>
__device__ __forceinline__ bf16x8 vt_read(const bf16* vt, const VtOffsets& vo, int t, int db) {
  return as_bf16x8(*(const u32x4*)(vt + (t >> 2) * D * 64 + vo.o[(t & 3) ^ db] + db * 32 * 64));
}

// Issue order of a run of NMFMA MFMAs that each consume one LDS read: the
// reads run LOOKAHEAD operands ahead of the MFMAs, one read per MFMA in
// between (left alone, the scheduler hoists every read and runs out of
// registers). NVMEM global loads of the same region go first (left alone,
// the scheduler sinks them to the end of the region, which wastes the
// latency they were issued early to hide).
template <int NMFMA, int LOOKAHEAD = 3, int NVMEM = 0>
__device__ __forceinline__ void interleave_lds_mfma() {
  if (NVMEM > 0) __builtin_amdgcn_sched_group_barrier(0x020, NVMEM, 0);  // global loads first
  __builtin_amdgcn_sched_group_barrier(0x100, LOOKAHEAD, 0);
#pragma unroll
  for (int i = 0; i < NMFMA - LOOKAHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LOOKAHEAD, 0);
}

// S^T = K Q^T for one 64-key tile whose rows sit at swap23(key) in `kt`.
// sacc[kb][i] then holds key 32 kb + 16 (i/8) + 8 h + i%8 for this lane's query.
template <int D>
__device__ __forceinline__ void score_tile(const bf16* kt, const bf16x8* qf,
                                           const KOffsets<D, true>& ko, f32x16* sacc) {
  using T = FwdTile<D>;
  f32x16 a0, a1;
#pragma unroll
  for (int i = 0; i < 16; ++i) a0[i] = a1[i] = 0.f;
#pragma unroll
  for (int s = 0; s < T::DK; ++s) {
    a0 = mfma32x32x16(k_read<D>(kt, ko, s, 0), qf[s], a0);
    a1 = mfma32x32x16(k_read<D>(kt, ko, s, 1), qf[s], a1);
  }
  interleave_lds_mfma<2 * T::DK>();
  sacc[0] = a0;
  sacc[1] = a1;
}

// O^T += V^T P^T for one 64-key tile: step t covers keys 16 t + 8 h + 0..7.
template <int D>
__device__ __forceinline__ void pv_tile(const bf16* vt, const u32x4* pw, const VtOffsets& vo,
                                        f32x16* oacc) {
  using T = FwdTile<D>;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bf16x8 pf = as_bf16x8(pw[t]);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) oacc[db] = mfma32x32x16(vt_read<D>(vt, vo, t, db), pf, oacc[db]);
  }
  interleave_lds_mfma<4 * T::DB>();
}

// Value-product steps of a ping-pong MFMA phase (the forward's O^T += V^T P^T,
// the dQ sweep's dQ^T += K^T dS^T) in issue order: the keys of the tile's
// second half (steps t = NT/2 .. NT-1) first -- their V^T columns were
// staged by the other group a full phase before the phase starts, so the
// first operands can be read before the phase's barrier -- then the first
// half (t = 0 .. NT/2-1).
template <int NT>
__device__ __forceinline__ constexpr int pv_step_t(int k, int db_count) {
  return (k / db_count + NT / 2) % NT;
}
constexpr int kPrefetch = 3;  // V^T operand reads issued before the barrier

// First kPrefetch V^T operands of the next MFMA phase (see pv_step_t).
template <int D, int BN>
__device__ __forceinline__ void prefetch_pv(const bf16* vt, const VtOffsets& vo, bf16x8* pre) {
  using T = FwdTile<D, BN>;
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) pre[k] = vt_read<D>(vt, vo, pv_step_t<T::NT>(k, T::DB), k % T::DB);
}

// Q^T as the B operand: lane (query lq, half h) holds d = 16 s + 8 h .. +7.
template <int D>
__device__ __forceinline__ void load_q(const bf16* qrow, bool q_ok, int h, bf16x8* qf) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 x = {0, 0, 0, 0};
    if (q_ok) x = *(const u32x4*)(qrow + 16 * s + 8 * h);
    qf[s] = as_bf16x8(x);
  }
}

// Transposes the two 16-byte V chunks this lane loaded (keys 2p, 2p+1 of a
// pass, p = lane / 16, the same 8 d-values d0 .. d0+7) into two 16-byte V^T
// pieces: 8 consecutive keys of rows d0 + 2p and d0 + 2p + 1.
__device__ __forceinline__ void transpose_v_pair(u32x4 a, u32x4 b, u32x4& lo, u32x4& hi) {
  unsigned c[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[2 * j] = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);      // (a.lo, b.lo): d = 2j
    c[2 * j + 1] = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);  // (a.hi, b.hi): d = 2j + 1
  }
  // c[i] = key pair p of row d0 + i. Exchange over lane bit 5, then bit 4.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto r = __builtin_amdgcn_permlane32_swap(c[i], c[i + 4], false, false);
    c[i] = r[0];
    c[i + 4] = r[1];
  }
#pragma unroll
  for (int i : {0, 1, 4, 5}) {
    auto r = __builtin_amdgcn_permlane16_swap(c[i], c[i + 2], false, false);
    c[i] = r[0];
    c[i + 2] = r[1];
  }
  // Now c[2u] / c[2u+1] = key pair u of rows d0 + 2p / d0 + 2p + 1.
  lo = (u32x4){c[0], c[2], c[4], c[6]};
  hi = (u32x4){c[1], c[3], c[5], c[7]};
}

// Rows [r0, r0 + ROWS) of a K tile and of a V^T tile, staged by THREADS
// threads: global -> registers (buffer loads: rows >= N read as zeros),
// then registers -> LDS. K chunks are spread over all threads; V is staged
// in passes of VKEYS keys per wave (each lane: two 16-byte loads).
template <int D, int ROWS, int THREADS, int BN = 64, bool WITH_K = true>
struct Stager {
  using T = FwdTile<D, BN>;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int KCPT = WITH_K ? ROWS * T::CPR / THREADS : 0;  // K chunks per thread
  static constexpr int VPASS = ROWS / T::VKEYS;          // V passes in total
  static constexpr int VPW = (VPASS + WAVES - 1) / WAVES;
  static_assert(!WITH_K || ROWS * T::CPR % THREADS == 0, "K rows must split evenly over the threads");
  static_assert(ROWS % T::VKEYS == 0, "V rows must split into whole passes");
  u32x4 k[KCPT > 0 ? KCPT : 1], va[VPW], vb[VPW];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                       int kt_k, int kt_v, int r0, int t) {
#pragma unroll
    for (int i = 0; i < KCPT; ++i) {
      const int ch = t + i * THREADS;
      const int row = r0 + ch / T::CPR, col = (ch % T::CPR) * 8;
      k[i] = buffer_load16(kr, ((kt_k * T::BN + row) * D + col) * 2);
    }
    const int wave = t >> 6, lane = t & 63, p = lane >> 4, r = lane & 15;
    const int col = 8 * (r % T::CPR), g = r / T::CPR;
    // Waves past the last pass load a valid pass again and store nothing: a
    // load under a wave-uniform condition made the compiler merge the
    // loaded registers with their old values right after the loads, and
    // that merge waited for the loads (and everything issued before them).
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int pass = VPASS % WAVES == 0 ? wave + i * WAVES : min(wave + i * WAVES, VPASS - 1);
      const int kv = kt_v * T::BN + r0 + pass * T::VKEYS + 8 * g + 2 * p;
      va[i] = buffer_load16(vr, (kv * D + col) * 2);
      vb[i] = buffer_load16(vr, ((kv + 1) * D + col) * 2);
    }
  }
  __device__ __forceinline__ void store(bf16* kt, bf16* vt, int r0, int t) {
#pragma unroll
    for (int i = 0; i < KCPT; ++i) {
      const int ch = t + i * THREADS;
      const int row = r0 + ch / T::CPR, col = (ch % T::CPR) * 8;
      const int lr = swap23(row);
      *(u32x4*)(kt + lr * D + 8 * ((col / 8) ^ kswz<D>(lr))) = k[i];
    }
    const int wave = t >> 6, lane = t & 63, p = lane >> 4, r = lane & 15;
    const int d0 = 8 * (r % T::CPR) + 2 * p, g = r / T::CPR;
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int pass = wave + i * WAVES;
      if (VPASS % WAVES == 0 || pass < VPASS) {
        u32x4 lo, hi;
        transpose_v_pair(va[i], vb[i], lo, hi);
        const int slot = (r0 + pass * T::VKEYS) / 8 + g;
        bf16* sub = vt + (slot >> 3) * D * 64;  // 64-key sub-tile
        *(u32x4*)(sub + d0 * 64 + 8 * ((slot & 7) ^ vt_swz(d0))) = lo;
        *(u32x4*)(sub + (d0 + 1) * 64 + 8 * ((slot & 7) ^ vt_swz(d0 + 1))) = hi;
      }
    }
  }
};

// Rows [r0, r0 + ROWS) of a K tile staged straight into LDS by WAVES waves
// with buffer_load ... lds: each instruction writes 1 KB of LDS
// lane-linearly (lane L -> 16 bytes at L * 16), and each lane loads the
// global chunk that belongs there in the swizzled layout (LDS row r holds
// key swap23(r), chunk position p holds logical chunk p ^ kswz(r)). The
// per-lane byte offsets within a tile are fixed; each tile gets a buffer
// resource of its own that starts at the tile's first row and ends at the
// head's last row, so rows >= N read as zeros through the range check of
// the per-lane offset (the scalar offset stays 0), and staging a tile costs
// no VALU work. Completion is waited for with vmcnt before the barrier that
// publishes the tile.

template <int D, int ROWS, int WAVES = 4, int SW = 0>
struct KDirect {
  static constexpr int RPI = 1024 / (2 * D);              // rows per instruction
  static constexpr int NI = ROWS / (WAVES * RPI);         // instructions per wave
  static_assert(ROWS % (WAVES * RPI) == 0, "rows must split evenly over the waves");
  int voff[NI];
  int lds_row0;  // first LDS row of this wave's first instruction
  __device__ __forceinline__ KDirect(int r0, int wave_in_group, int lane) {
    lds_row0 = r0 + wave_in_group * NI * RPI;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int lr = lds_row0 + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ kswz<D, SW>(lr);
      voff[i] = (swap23(lr) * D + 8 * c) * 2;
    }
  }
  // Tile `tile` (rows tile * bn ..) of a head whose K rows start at kbase
  // and number n_rows. ASYNC issues the transfers with lds_dma16_async.
  template <bool ASYNC = false>
  __device__ __forceinline__ void load(const bf16* kbase, int n_rows, int tile, int bn, bf16* kt) const {
    const int row0 = tile * bn;
    const int rem = n_rows > row0 ? n_rows - row0 : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (size_t)row0 * D), 0, rem * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (ASYNC) lds_dma16_async(r, kt + (lds_row0 + i * RPI) * D, voff[i]);
      else lds_dma16(r, kt + (lds_row0 + i * RPI) * D, voff[i]);
    }
  }
};


__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace tattn
