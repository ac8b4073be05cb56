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
typedef short s16x4 __attribute__((ext_vector_type(4)));

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
  // the two bf16 of a packed pair as floats (exact)
  static __device__ __forceinline__ float lo(uint32_t pair) { return __uint_as_float(pair << 16); }
  static __device__ __forceinline__ float hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
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
  static __device__ __forceinline__ float lo(uint32_t pair) { return (float)__builtin_bit_cast(f16x2, pair)[0]; }
  static __device__ __forceinline__ float hi(uint32_t pair) { return (float)__builtin_bit_cast(f16x2, pair)[1]; }
};

// Register r of a 32x32 product in lane group g (= lane / 32) holds row
// kb*32 + (r/4)*8 + g*4 + r%4 of the block kb it covers (the accumulator
// layout above); for transposed scores S^T that row index is a key.
__device__ __forceinline__ int score_key(int kb, int r, int g) {
  return kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
}

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

// Wait until every vector-memory load issued so far has returned
// (s_waitcnt vmcnt(0); the expcnt and lgkmcnt fields are left at their
// maxima, i.e. not waited on). Issued once the loads that a loop reads but
// never reissues (the query tile) are in flight: the compiler then knows they
// are complete inside the loop and does not make its first products wait on
// the loads of the next K/V tile, which come later in the same in-order count.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }


__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies and transposing LDS reads (gfx950).
// ---------------------------------------------------------------------------

// Raw buffer resource over `bytes` bytes from `base` (stride 0, untyped 32-bit
// data format, the gfx9 descriptor word 3 = 0x00020000); the hardware returns
// zero for offsets at or past `bytes`. Four scalar registers.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const i32x4 r = {(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), bytes, 0x00020000};
  return r;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p);
}

// One 16-byte load per lane from `rsrc` at byte `voff`, written straight into
// LDS (buffer_load_dwordx4 ... lds): lane i fills LDS bytes
// [lds + 16 i, lds + 16 i + 16); `lds` is wave-uniform and goes through M0,
// which is restored afterwards. Completion is counted by vmcnt.
// An SALU write of M0 needs one wait state before an LDS-direct load reads
// it (the "manually inserted wait states" rule of the gfx9 family ISA); the
// s_nop provides it, since the compiler's hazard checks do not see inside
// inline assembly. Without it the load may use the previous M0 and write its
// 16 bytes to the wrong LDS slot.
// Issued as inline assembly on purpose: the compiler then does not know that
// this load writes LDS, and does not put a full vmcnt wait in front of every
// later transposing LDS read (it cannot tell them apart from the copy's
// destination). Every LDS read of copied data is ordered by hand instead: an
// explicit vmcnt wait (vm_wait) and a workgroup barrier, never by the compiler.
// Race-guard build (FA_DEBUG_POISON): before a copy is issued, this lane's
// destination bytes are filled with all-ones (a NaN in fp32, fp16 and bf16)
// and the write is waited for. A slot then holds NaN from the moment it is
// refilled -- after the barrier that follows its last read -- until the new
// tile lands, so a read that is not ordered after the copy's wait and
// barrier, or a copy issued into a slot still being read, shows up as NaN in
// the outputs instead of as stale or early data.
#ifdef FA_DEBUG_POISON
// One temporary register, written and consumed inside the block; the stores
// have completed (lgkmcnt(0)) before the block ends.
__device__ __forceinline__ void poison_lds(uint32_t lds, int bytes_per_lane) {
  const uint32_t a = lds + (uint32_t)(threadIdx.x & 63) * (uint32_t)bytes_per_lane;
  uint32_t tmp;
  if (bytes_per_lane == 16)
    asm volatile(
        "v_mov_b32 %0, -1\n\t"
        "ds_write_b32 %1, %0\n\t"
        "ds_write_b32 %1, %0 offset:4\n\t"
        "ds_write_b32 %1, %0 offset:8\n\t"
        "ds_write_b32 %1, %0 offset:12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(tmp)
        : "v"(a)
        : "memory");
  else
    asm volatile(
        "v_mov_b32 %0, -1\n\t"
        "ds_write_b32 %1, %0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(tmp)
        : "v"(a)
        : "memory");
}
#endif

__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds, uint32_t voff) {
#ifdef FA_DEBUG_POISON
  poison_lds(lds, 16);
#endif
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

// The same with 4 bytes per lane (buffer_load_dword ... lds): lane i fills
// LDS bytes [lds + 4 i, lds + 4 i + 4).
__device__ __forceinline__ void load_lds4(i32x4 rsrc, uint32_t lds, uint32_t voff) {
#ifdef FA_DEBUG_POISON
  poison_lds(lds, 4);
#endif
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order). Inline assembly, so that it stays exactly
// where it is written; the "memory" clobber keeps memory accesses on their side.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Transposing 8-byte LDS read of 16-bit data (ds_read_b64_tr_b16). Within
// each group of 16 lanes, source lane s reads four consecutive elements
// E[s][0..3] at its own address; lane i of the group receives
// E[4k + i/4][i % 4] for k = 0..3. With source lane s pointing at row
// (row0 + s/4), columns (col0 + 4 (s%4)) .. +3 of a row-major matrix, lane i
// therefore receives column col0 + i of rows row0 .. row0 + 3.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* lds) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)const_cast<char*>(lds));
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte chunk placement of the K and V tiles in LDS. A tile row r of RB =
// 2 D bytes is kept at r * RB; its chunk c sits in slot c ^ k(r) (K) or
// c ^ v(r) (V). The XOR keeps every read of the attention loop free of bank
// conflicts on 32 or 64 four-byte banks:
//  * K (16-byte reads): 16 consecutive rows, one chunk -> 16 distinct slots
//    (d = 128), or 16 distinct (row parity, slot) pairs (d = 64);
//  * V (transposing 8-byte reads): 4 consecutive rows x 4 consecutive chunks
//    -> 16 distinct slots (d = 128) / (row parity, slot) pairs (d = 64), and
//    any 16 lanes of it -> 8 distinct slots modulo 8.
//  * dual: a tile read both ways (the backward pass reads Q, dO and K both
//    as 16-byte rows and transposed): an XOR-linear map of the row's low four
//    bits, found by exhaustive search over such maps on a CPU model of both
//    access patterns; conflict free for both, on 32 or 64 banks.
template <int D> struct TileSwizzle;
template <> struct TileSwizzle<128> {
  static __device__ __forceinline__ int k(int r) { return r & 15; }
  static __device__ __forceinline__ int v(int r) {
    const int t = r & 3;
    return 4 * t + 2 * (t >> 1);
  }
  // bits (r0, r1, r0^r2, r1^r3)
  static __device__ __forceinline__ int dual(int r) { return (r & 3) | (((r ^ (r >> 2)) & 3) << 2); }
};
template <> struct TileSwizzle<64> {
  static __device__ __forceinline__ int k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
  static __device__ __forceinline__ int v(int r) { return 2 * (r & 3); }
  // bits (r1, r0^r2, r0^r1^r3)
  static __device__ __forceinline__ int dual(int r) {
    const int b0 = (r >> 1) & 1, b1 = (r ^ (r >> 2)) & 1, b2 = (r ^ (r >> 1) ^ (r >> 3)) & 1;
    return b0 | (b1 << 1) | (b2 << 2);
  }
};

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
