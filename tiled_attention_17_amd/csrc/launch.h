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
  int64_t N;        // sequence length (queries = keys)
  int64_t d;        // head dimension
  float scale;
  bool dtype_fp32;  // false: bf16
  void* stream;
  int num_cus;      // compute units of the device (grid sizing)
  int waves;        // 0 = choose; else waves per workgroup of the bf16 kernel (2, 4 or 8)
};

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
  float* row_dot;   // workspace: D_i = dO_i . O_i, [BH, N] floats
  int64_t BH;
  int64_t N;
  int64_t d;
  float scale;
  void* stream;
  int num_cus;
};

hipError_t launch_attn_fwd(const FwdArgs& a);
hipError_t launch_attn_bwd(const BwdArgs& a);
int fwd_bf16_waves(int64_t BH, int64_t N, int num_cus);

}  // namespace tattn
