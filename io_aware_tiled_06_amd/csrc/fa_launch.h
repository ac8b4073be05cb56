// fa_launch.h -- host-side launchers behind the C interface. Arguments reach
// these only after validation (see api.hip); they launch and return the HIP
// status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum ElemType { kF32 = 0, kF16 = 1, kBF16 = 2 };

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, H, N, d;
  float scale;
  int dtype;
  hipStream_t stream;
};

inline int elem_bytes(int dtype) { return dtype == kF32 ? 4 : 2; }

// Query rows per workgroup of the fused kernel for (dtype, d).
int flash_rows_per_block(int dtype, int d);

// Fused tiled forward pass over all B*H heads (one launch).
hipError_t launch_flash(const AttnArgs& a);
// The same with causal masking: query i sees keys j <= i.
hipError_t launch_flash_causal(const AttnArgs& a);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;  // caller's float32 scratch: D [B,H,N], then LSE*log2(e) [B,H,N]
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  int dtype;
  hipStream_t stream;
};

// Rows (queries or keys) per workgroup of the backward kernels.
int bwd_rows_per_block();

// Backward pass: D = rowsum(dO * O), then dQ, then dK and dV (three launches).
hipError_t launch_bwd(const BwdArgs& a, bool causal);

// Largest number of heads one launch of the three-pass path may cover
// (grid-size limit); 0 means N is too large for that path.
int64_t naive_max_heads_per_launch(int N, int d, int dtype);

// Three-pass materialising forward pass; heads are processed in chunks that
// fit `ws_bytes` (at least one head).
hipError_t launch_naive(const AttnArgs& a, void* ws, size_t ws_bytes);

}  // namespace fa
