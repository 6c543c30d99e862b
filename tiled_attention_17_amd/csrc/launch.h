// Host-side launch descriptors shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH;       // batch * heads
  int64_t Nq;       // queries per head
  int64_t Nk;       // keys (and values) per head
  int64_t d;        // head dimension
  float scale;
  bool dtype_fp32;  // false: bf16
  bool causal;      // query i sees key j iff j <= i + Nk - Nq
  int n_splits;     // key-range splits (1: one pass; > 1: partials in `partial`, then a merge)
  float* partial;   // workspace for n_splits > 1: O parts [S, BH, Nq, d] then LSE parts [S, BH, Nq]
  void* stream;
  int num_cus;      // compute units of the device (grid sizing)
  int waves;        // 0 = choose; else waves per workgroup of the bf16 kernel (2, 4 or 8)
  int ksplit;       // 0 = choose; 1 = never; 2 = split a workgroup's keys between its waves
                    // where the launch allows it (bf16: two wave groups, no mask, no key splits,
                    // waves < 8; fp32: always)
  int decode;       // 0 = choose; 1 = never use the one-query kernel for N_q = 1 (bf16)
  int f32_bm;       // 0 = choose; 16 or 32 = query tile of the fp32 key-split kernel (d = 64)
  int ksplit_bn = 0;  // 0 = choose; 64 or 128 = key tile of the bf16 key-split kernel (d = 64)
  int64_t tail_heads = 0;  // > 0: heads [BH - tail_heads, BH) run with tail_splits splits (fwd_tail_plan)
  int tail_splits = 0;
  void* ev_start = nullptr;  // hipEvent_t bound to the start of the attention kernel (or null)
  void* ev_stop = nullptr;   // hipEvent_t bound to its end (or null)
};

// Parameters of one forward kernel launch (kernel argument, by value).
// Workgroup w covers query tile qt of head bh and keys
// [split * split_keys, min(Nk, (split + 1) * split_keys)); with n_splits == 1
// it writes O (input dtype) and LSE, otherwise the fp32 partial result of its
// key range to o_part / lse_part.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* o_part;    // [n_splits, BH, Nq, d]
  float* lse_part;  // [n_splits, BH, Nq]
  int Nq;
  int Nk;
  int BH;
  int n_qtiles;
  int n_splits;
  int split_keys;   // multiple of 128
  int total_tiles;  // BH * n_qtiles * n_splits
  float c;          // scale * log2(e)
  int causal;
  int remap;        // XCD-contiguous tile order (non-causal launches)
};

constexpr int kMaxSplits = 128;  // largest number of key splits of one forward launch

// Keys per split chosen for (Nk, n_splits): a multiple of 128.
int64_t split_keys_for(int64_t Nk, int n_splits);
// Number of key splits the library picks when the caller leaves it open.
int fwd_auto_splits(int64_t BH, int64_t Nq, int64_t Nk, bool fp32, int num_cus);

// The library's plan for a grid whose last round of workgroups would be at
// most half full: the heads [0, head_split) run unsplit in whole rounds, the
// remaining heads with tail_splits key splits (and a merge) over the whole
// chip. Returns false (no such plan) where it does not apply.
struct FwdTailPlan {
  int64_t head_split;
  int tail_splits;
};
bool fwd_tail_plan(int64_t BH, int64_t Nq, int64_t Nk, bool fp32, bool causal, int num_cus, FwdTailPlan* plan);
hipError_t launch_attn_merge(const float* o_part, const float* lse_part, int n_parts, int64_t rows,
                             int64_t d, void* o, float* lse, bool out_fp32, void* stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* row_dot;   // workspace: D_i = dO_i . O_i, [BH, Nq] floats
  int64_t BH;
  int64_t Nq;       // queries per head (q, o, dout, lse, dq)
  int64_t Nk;       // keys per head (k, v, dk, dv)
  int64_t d;
  float scale;
  bool causal;      // query i sees key j iff j <= i + Nk - Nq
  void* stream;
  int num_cus;
  int dkdv_waves = 0;  // 0 = choose; 4 or 8 = waves per dK/dV workgroup (128 or 256 keys)
  int dq_waves = 0;    // 0 = choose; 4 or 8 = waves per dQ workgroup (128 or 256 queries)
};

// Waves per workgroup of the dK/dV and dQ sweeps for these arguments (4 or 8).
int dkdv_waves(const BwdArgs& a);
int dq_waves(const BwdArgs& a);

hipError_t launch_attn_fwd(const FwdArgs& a);

// MXFP8 forward: E4M3 Q, K [BH, N, d] with scales [BH, N, d/32], V^T [BH, d, N]
// with scales [BH, d, N/32]; O bf16 [BH, N, d], LSE [BH, N].
struct Fp8Args {
  const void* q8;
  const void* qs;
  const void* k8;
  const void* ks;
  const void* vt8;
  const void* vts;
  void* o;
  float* lse;
  int64_t BH;
  int64_t N;
  int64_t d;
  float scale;
  void* stream;
};
hipError_t launch_attn_fwd_mxfp8(const Fp8Args& a);
// MXFP8 quantizer: x [batch, rows, cols] bf16 -> q, sc; transpose = false:
// q [batch, rows, cols], sc [batch, rows, cols/32]; transpose = true:
// q [batch, cols, rows], sc [batch, cols, rows/32].
hipError_t launch_mx_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols, bool transpose,
                              void* q, void* sc, void* stream);
// C = A B^T, bf16: A [M, K], B [N, K], C [M, N].
hipError_t launch_matmul_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                            void* stream);
hipError_t launch_attn_bwd(const BwdArgs& a);

// Query rows (B * H * N_q) the allocation-free backward accepts: its row
// terms D_i live in a fixed device array of this many floats (16 MiB), one
// copy per device for the life of the process.
constexpr int64_t kNoAllocRows = int64_t(1) << 22;
// The backward of launch_attn_bwd with a.row_dot ignored: the row terms go
// to that fixed array instead (a.BH * a.Nq <= kNoAllocRows, checked by the
// caller). Allocates nothing.
hipError_t launch_attn_bwd_noalloc(const BwdArgs& a);
int fwd_bf16_waves(int64_t BH, int64_t Nq, int64_t splits, int num_cus);

}  // namespace tattn
