// naive.hip -- standard, materialising attention in three passes: the traffic
// comparator of the fused kernel ("FlashAttention, simplified", "The problem";
// "What FlashAttention actually buys", "The actual problem"). The scores S and
// probabilities P of a chunk of heads go through device memory:
//   pass 1  S = scale * Q K^T        (float32, written)
//   pass 2  P = softmax_rows(S), LSE (S read once, P written in the input type)
//   pass 3  O = P V                  (P read once)
// The contractions still run on the matrix cores, so the comparison isolates
// the cost of the N x N round trips rather than a slow GEMM.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

// ---------------------------------------------------------------------------
// Pass 1, half precision: S^T tiles on the matrix cores. A workgroup covers
// 128 queries (4 waves x 32) against 64 keys; operands are read straight from
// global memory (the head is small enough to live in L2).
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void naive_scores_half(const char* q, const char* k, float* s, int n,
                                                          int tiles_k, int tiles_q, float scale) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int b = blockIdx.x;
  const int tk = b % tiles_k;
  b /= tiles_k;
  const int tq = b % tiles_q;
  const int hl = b / tiles_q;  // head within the chunk
  const int64_t head = (int64_t)hl * n * D * 2;
  const int q_row = tq * 128 + wave * 32 + l32;
  const int q_ld = q_row < n ? q_row : n - 1;
  const int key0 = tk * 64;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const u32x4 b_op = ld_global16(q + head + ((int64_t)q_ld * D + kk * 16 + g * 8) * 2);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int key = key0 + kb * 32 + l32;
      key = key < n ? key : n - 1;
      const u32x4 a_op = ld_global16(k + head + ((int64_t)key * D + kk * 16 + g * 8) * 2);
      acc[kb] = Mfma<E>::run(a_op, b_op, acc[kb]);
    }
  }
  if (q_row >= n) return;
  float* srow = s + (int64_t)hl * n * n + (int64_t)q_row * n;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + kb * 32 + i * 8 + g * 4;  // 4 consecutive keys
      if ((n & 3) == 0 && key + 3 < n) {
        f32x4 w = {acc[kb][i * 4] * scale, acc[kb][i * 4 + 1] * scale, acc[kb][i * 4 + 2] * scale,
                   acc[kb][i * 4 + 3] * scale};
        *reinterpret_cast<f32x4*>(srow + key) = w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key + e < n) srow[key + e] = acc[kb][i * 4 + e] * scale;
      }
    }
}

// Pass 1, float32: one thread per score (only used for small float32 cases).
template <int D>
__global__ __launch_bounds__(256) void naive_scores_f32(const float* q, const float* k, float* s, int n,
                                                         int64_t total, float scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t nn = (int64_t)n * n;
  const int64_t hl = i / nn, rem = i % nn;
  const int qr = (int)(rem / n), kr = (int)(rem % n);
  const float* qp = q + (hl * n + qr) * D;
  const float* kp = k + (hl * n + kr) * D;
  float acc = 0.f;
#pragma unroll 8
  for (int t = 0; t < D; ++t) acc = fmaf(qp[t], kp[t], acc);
  s[i] = acc * scale;
}

// ---------------------------------------------------------------------------
// Pass 2: one workgroup per score row. Rows of up to 256*EPT keys stay in
// registers, so S is read exactly once; EPT == 0 streams longer rows twice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <int DT> struct Store;
template <> struct Store<kF32> {
  static __device__ __forceinline__ void put(char* p, int64_t i, float x) { reinterpret_cast<float*>(p)[i] = x; }
};
template <> struct Store<kBF16> {
  static __device__ __forceinline__ void put(char* p, int64_t i, float x) {
    reinterpret_cast<__bf16*>(p)[i] = (__bf16)x;
  }
};
template <> struct Store<kF16> {
  static __device__ __forceinline__ void put(char* p, int64_t i, float x) {
    reinterpret_cast<_Float16*>(p)[i] = (_Float16)x;
  }
};

template <int DT, int EPT>
__global__ __launch_bounds__(256) void naive_softmax(const float* s, char* pbuf, float* lse, int n,
                                                      int64_t lse_off) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;  // row within the chunk: head * n + query
  const float* srow = s + row * n;
  const int64_t pbase = row * n;
  const int tid = threadIdx.x;
  float m = -INFINITY;
  if constexpr (EPT > 0) {
    float x[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * 256;
      x[e] = i < n ? srow[i] : -INFINITY;
      m = fmaxf(m, x[e]);
    }
    m = block_reduce(m, true, red);
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      x[e] = exp2_fast((x[e] - m) * kLog2e);
      l += x[e];
    }
    l = block_reduce(l, false, red);
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * 256;
      if (i < n) Store<DT>::put(pbuf, pbase + i, x[e] * inv);
    }
    if (tid == 0 && lse) lse[lse_off + row] = m + logf(l);
  } else {
    for (int i = tid; i < n; i += 256) m = fmaxf(m, srow[i]);
    m = block_reduce(m, true, red);
    float l = 0.f;
    for (int i = tid; i < n; i += 256) l += exp2_fast((srow[i] - m) * kLog2e);
    l = block_reduce(l, false, red);
    const float inv = 1.f / l;
    for (int i = tid; i < n; i += 256) Store<DT>::put(pbuf, pbase + i, exp2_fast((srow[i] - m) * kLog2e) * inv);
    if (tid == 0 && lse) lse[lse_off + row] = m + logf(l);
  }
}

// ---------------------------------------------------------------------------
// Pass 3, half precision: O^T = V^T P^T on the matrix cores. A workgroup
// covers 128 queries; V tiles of 64 keys are transposed into LDS (same layout
// as the fused kernel), P is read from global memory in the key order that
// layout expects.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ld_half_pair(const uint16_t* row, int key, int n) {
  const uint32_t lo = key < n ? row[key] : 0u;
  const uint32_t hi = key + 1 < n ? row[key + 1] : 0u;
  return lo | (hi << 16);
}

// 4 consecutive probabilities (keys key..key+3) of one row as two words.
__device__ __forceinline__ u32x2 ld_p4(const uint16_t* row, int key, int n) {
  if ((n & 3) == 0 && key + 3 < n) return *reinterpret_cast<const u32x2*>(row + key);
  u32x2 r;
  r[0] = ld_half_pair(row, key, n);
  r[1] = ld_half_pair(row, key + 2, n);
  return r;
}

template <class E, int D>
__global__ __launch_bounds__(256) void naive_pv_half(const char* pbuf, const char* v, char* o, int n, int tiles_q) {
  constexpr int BC = 64, NT = 256;
  using VS = VStage<D, BC, NT>;
  __shared__ __attribute__((aligned(16))) char smem[VS::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int tq = blockIdx.x % tiles_q, hl = blockIdx.x / tiles_q;
  const int q_row = tq * 128 + wave * 32 + l32;
  const int q_ld = q_row < n ? q_row : n - 1;
  const uint16_t* prow = reinterpret_cast<const uint16_t*>(pbuf) + (int64_t)hl * n * n + (int64_t)q_ld * n;
  const uint16_t* vh = reinterpret_cast<const uint16_t*>(v) + (int64_t)hl * n * D;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  VS vs;
  const int n_tiles = (n + BC - 1) / BC;
  for (int j = 0; j < n_tiles; ++j) {
    const int key0 = j * BC;
    vs.load(vh, key0, n, tid);
    __syncthreads();  // previous tile fully consumed
    vs.store(smem, tid);
    __syncthreads();
    // B operand for (kb, h): keys kb*32 + h*16 + {g*4 + 0..3, 8 + g*4 + 0..3}.
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kbase = key0 + kb * 32 + h * 16 + g * 4;
        const u32x2 x = ld_p4(prow, kbase, n), y = ld_p4(prow, kbase + 8, n);
        pf[kb][h] = u32x4{x[0], x[1], y[0], y[1]};
      }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[db] = Mfma<E>::run(VS::read(smem, db * 32 + l32, kb * 32 + h * 16 + g * 8), pf[kb][h], acc[db]);
  }
  if (q_row >= n) return;
  char* orow = o + ((int64_t)hl * n + q_row) * D * 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = Mfma<E>::pack2(acc[db][i * 4 + 0], acc[db][i * 4 + 1]);
      w[1] = Mfma<E>::pack2(acc[db][i * 4 + 2], acc[db][i * 4 + 3]);
      *reinterpret_cast<u32x2*>(orow + (db * 32 + i * 8 + g * 4) * 2) = w;
    }
}

// Pass 3, float32: one thread per output element (small float32 cases only).
template <int D>
__global__ __launch_bounds__(256) void naive_pv_f32(const float* pbuf, const float* v, float* o, int n,
                                                     int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int dcol = (int)(i % D);
  const int64_t hq = i / D;  // head * n + query
  const int64_t hl = hq / n;
  const float* prow = pbuf + hq * n;
  const float* vh = v + hl * n * D;
  float acc = 0.f;
  for (int j = 0; j < n; ++j) acc = fmaf(prow[j], vh[(int64_t)j * D + dcol], acc);
  o[i] = acc;
}

template <int DT>
void launch_softmax(const float* s, char* pbuf, float* lse, int n, int64_t rows, int64_t lse_off,
                    hipStream_t st) {
  const dim3 grid((unsigned)rows), block(256);
  if (n <= 256) hipLaunchKernelGGL((naive_softmax<DT, 1>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
  else if (n <= 1024) hipLaunchKernelGGL((naive_softmax<DT, 4>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
  else if (n <= 4096) hipLaunchKernelGGL((naive_softmax<DT, 16>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
  else if (n <= 16384) hipLaunchKernelGGL((naive_softmax<DT, 64>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
  else if (n <= 32768) hipLaunchKernelGGL((naive_softmax<DT, 128>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
  else hipLaunchKernelGGL((naive_softmax<DT, 0>), grid, block, 0, st, s, pbuf, lse, n, lse_off);
}

template <class E, int DT, int D>
hipError_t chunk_half(const AttnArgs& a, int64_t h0, int hc, float* s, char* pbuf) {
  const int n = a.N;
  const int64_t off = h0 * (int64_t)n * D * 2;
  const char* q = static_cast<const char*>(a.q) + off;
  const char* k = static_cast<const char*>(a.k) + off;
  const char* v = static_cast<const char*>(a.v) + off;
  char* o = static_cast<char*>(a.o) + off;
  const int tiles_k = (n + 63) / 64, tiles_q = (n + 127) / 128;
  hipLaunchKernelGGL((naive_scores_half<E, D>), dim3((unsigned)((int64_t)tiles_k * tiles_q * hc)), dim3(256), 0,
                     a.stream, q, k, s, n, tiles_k, tiles_q, a.scale);
  launch_softmax<DT>(s, pbuf, a.lse, n, (int64_t)hc * n, h0 * n, a.stream);
  hipLaunchKernelGGL((naive_pv_half<E, D>), dim3((unsigned)((int64_t)tiles_q * hc)), dim3(256), 0, a.stream,
                     pbuf, v, o, n, tiles_q);
  return hipGetLastError();
}

template <int D>
hipError_t chunk_f32(const AttnArgs& a, int64_t h0, int hc, float* s, char* pbuf) {
  const int n = a.N;
  const int64_t off = h0 * (int64_t)n * D;
  const float* q = static_cast<const float*>(a.q) + off;
  const float* k = static_cast<const float*>(a.k) + off;
  const float* v = static_cast<const float*>(a.v) + off;
  float* o = static_cast<float*>(a.o) + off;
  const int64_t total_s = (int64_t)hc * n * n;
  hipLaunchKernelGGL((naive_scores_f32<D>), dim3((unsigned)((total_s + 255) / 256)), dim3(256), 0, a.stream, q, k,
                     s, n, total_s, a.scale);
  launch_softmax<kF32>(s, pbuf, a.lse, n, (int64_t)hc * n, h0 * n, a.stream);
  const int64_t total_o = (int64_t)hc * n * D;
  hipLaunchKernelGGL((naive_pv_f32<D>), dim3((unsigned)((total_o + 255) / 256)), dim3(256), 0, a.stream,
                     reinterpret_cast<const float*>(pbuf), v, o, n, total_o);
  return hipGetLastError();
}

}  // namespace

int64_t naive_max_heads_per_launch(int N, int d, int dtype) {
  // Every launch must stay below 2^32 work-items in its one grid dimension.
  const int64_t lim = ((int64_t)1 << 32) - 256;
  const int64_t n = N;
  int64_t per_head;  // work-items one head adds to the largest of the three launches
  if (dtype == kF32) {
    per_head = n * n > n * d ? n * n : n * d;
  } else {
    const int64_t tk = (n + 63) / 64, tq = (n + 127) / 128;
    per_head = tk * tq * 256;
  }
  if (n * 256 > per_head) per_head = n * 256;  // softmax: one workgroup per row
  return per_head > 0 ? lim / per_head : 0;
}

hipError_t launch_naive(const AttnArgs& a, void* ws, size_t ws_bytes) {
  const int64_t bh = (int64_t)a.B * a.H;
  const int64_t nn = (int64_t)a.N * a.N;
  const int64_t per_head = nn * (4 + elem_bytes(a.dtype));
  int64_t hc = (int64_t)(ws_bytes / (size_t)per_head);
  if (hc > bh) hc = bh;
  const int64_t cap = naive_max_heads_per_launch(a.N, a.d, a.dtype);
  if (hc > cap) hc = cap;
  if (hc < 1) return hipErrorInvalidValue;  // rejected by validation before this point
  float* s = static_cast<float*>(ws);
  char* pbuf = static_cast<char*>(ws) + hc * nn * 4;
  for (int64_t h0 = 0; h0 < bh; h0 += hc) {
    const int c = (int)((bh - h0) < hc ? (bh - h0) : hc);
    hipError_t e;
    switch (a.dtype) {
      case kBF16:
        e = a.d == 128 ? chunk_half<BF16, kBF16, 128>(a, h0, c, s, pbuf) : chunk_half<BF16, kBF16, 64>(a, h0, c, s, pbuf);
        break;
      case kF16:
        e = a.d == 128 ? chunk_half<F16, kF16, 128>(a, h0, c, s, pbuf) : chunk_half<F16, kF16, 64>(a, h0, c, s, pbuf);
        break;
      default:
        e = a.d == 128 ? chunk_f32<128>(a, h0, c, s, pbuf) : chunk_f32<64>(a, h0, c, s, pbuf);
        break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fa
