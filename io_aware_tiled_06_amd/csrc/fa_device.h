// fa_device.h -- device-side building blocks shared by the gfx950 attention
// kernels: vector types, matrix-core wrappers, element conversion, the
// workgroup-to-XCD mapping and the K/V staging into LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage tags for the two half-precision element types.
struct BF16 {};
struct F16 {};

// log2(e) and ln(2) in float32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 matrix-core product, C += A * B, half-precision operands, float32
// accumulation. Operand layout (64 lanes): lane l supplies row (l % 32) of A
// and column (l % 32) of B, each with 8 consecutive elements of the
// contraction index, group (l / 32). The accumulator holds, in register r of
// lane l, element [row (r/4)*8 + (l/32)*4 + r%4][column l % 32].
template <class E> struct Mfma;
template <> struct Mfma<BF16> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even), low element first
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <> struct Mfma<F16> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by the lane 32 positions away
// (v_permlane32_swap). After the swap each lane holds both its own value and
// its partner's in the two results, whichever way round; max and sum are
// symmetric, so both lanes of a pair get bitwise the same answer.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_min(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are handed to the 8 XCDs of an MI355X round robin (XCD = id % 8).
// Map the hardware id to a logical id so that each XCD receives one contiguous
// range of logical workgroups; consecutive logical ids share a head, so the
// K/V of a head are fetched into one XCD's L2 instead of all eight.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  constexpr int kXcd = 8;
  const int per = nblk / kXcd, rem = nblk % kXcd;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Row staging: ROWS rows of ROW_BYTES bytes copied from global memory into
// LDS at a padded pitch of PITCH bytes. Thread item i covers 16-byte chunk
// (row i / (ROW_BYTES/16), chunk i % (ROW_BYTES/16)), so consecutive lanes
// read consecutive bytes of a row.
// K tiles (any element type) and float32 V tiles use this.
template <int ROWS, int ROW_BYTES, int PITCH, int NT>
struct RowStage {
  static constexpr int kRowChunks = ROW_BYTES / 16;
  static constexpr int kChunks = ROWS * kRowChunks;
  static constexpr int kPer = kChunks / NT;
  static_assert(ROW_BYTES % 16 == 0 && PITCH % 16 == 0, "16-byte rows");
  static_assert(kChunks % NT == 0, "tile must split evenly over the threads");
  static constexpr int kPitch = PITCH;
  static constexpr int kBytes = ROWS * PITCH;
  u32x4 r[kPer];

  // base: first byte of row 0 of the head; rows are ROW_BYTES apart. Rows at
  // or past n_valid re-read row n_valid - 1: always in bounds, never branched
  // on; the scores of those keys are masked and their probabilities are 0.
  __device__ __forceinline__ void load(const char* base, int row0, int n_valid, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * NT;
      const int row = item / kRowChunks, ch = item % kRowChunks;
      const int key = min(row0 + row, n_valid - 1);
      r[i] = ld_global16(base + (int64_t)key * ROW_BYTES + ch * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * NT;
      const int row = item / kRowChunks, ch = item % kRowChunks;
      *reinterpret_cast<u32x4*>(lds + row * PITCH + ch * 16) = r[i];
    }
  }
  // 16 bytes of row `row` starting at byte `byte_off`.
  static __device__ __forceinline__ u32x4 read16(const char* lds, int row, int byte_off) {
    return *reinterpret_cast<const u32x4*>(lds + row * PITCH + byte_off);
  }
  static __device__ __forceinline__ float read4(const char* lds, int row, int byte_off) {
    return *reinterpret_cast<const float*>(lds + row * PITCH + byte_off);
  }
};

// V tile staging, transposed: LDS holds V^T, [D rows][BC keys], so that one
// 16-byte read gives a lane 8 keys of one feature column -- the operand layout
// of the P V product on the matrix cores. Within each group of 16 keys the
// key order is 0-3, 8-11, 4-7, 12-15: lane group 0 then reads keys
// {0-3, 8-11} and lane group 1 keys {4-7, 12-15}, which is exactly how the
// score accumulator distributes keys over the two lane groups.
// Thread item i covers 4 consecutive keys (kg = i % (BC/4)) of 8 consecutive
// features (dg = i / (BC/4)); it loads 4 rows of 16 bytes, transposes them in
// registers and writes 8 runs of 4 keys.
template <int D, int BC, int NT>
struct VStage {
  static constexpr int kItems = (BC / 4) * (D / 8);
  static constexpr int kPer = (kItems + NT - 1) / NT;
  static constexpr int kPitch = BC * 2 + 16;  // bytes per V^T row
  static constexpr int kBytes = D * kPitch;
  u32x4 r[kPer][4];

  // Keys at or past n_valid re-read key n_valid - 1 (in bounds, no branch);
  // their probabilities are 0.
  __device__ __forceinline__ void load(const uint16_t* base, int row0, int n_valid, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * NT;
      if (kItems % NT != 0 && item >= kItems) continue;
      const int kg = item % (BC / 4), dg = item / (BC / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(row0 + kg * 4 + j, n_valid - 1);
        r[i][j] = ld_global16(base + (int64_t)key * D + dg * 8);
      }
    }
  }
  // LDS element position of key `k` (0 <= k < BC) within a V^T row.
  static __device__ __forceinline__ int slot(int k) {
    const int a = (k >> 2) & 3;                       // which run of 4 in the 16-group
    const int a_swapped = ((a & 1) << 1) | (a >> 1);  // 0,1,2,3 -> 0,2,1,3
    return (k & ~15) | (a_swapped << 2) | (k & 3);
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * NT;
      if (kItems % NT != 0 && item >= kItems) continue;
      const int kg = item % (BC / 4), dg = item / (BC / 4);
      const int col = slot(kg * 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // features dg*8 + 2w (low halves) and dg*8 + 2w + 1 (high halves)
        const uint32_t a0 = r[i][0][w], a1 = r[i][1][w], a2 = r[i][2][w], a3 = r[i][3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int d0 = dg * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(lds + d0 * kPitch + col * 2) = lo;
        *reinterpret_cast<u32x2*>(lds + (d0 + 1) * kPitch + col * 2) = hi;
      }
    }
  }
  // 16-byte operand: feature row `d`, key slots [s0, s0 + 8).
  static __device__ __forceinline__ u32x4 read(const char* lds, int d, int s0) {
    return *reinterpret_cast<const u32x4*>(lds + d * kPitch + s0 * 2);
  }
};

}  // namespace fa
