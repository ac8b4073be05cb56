// flash_bwd.hip -- attention backward pass for gfx950 (bf16 / fp16 inputs).
//
// Method: the gradient of the forward pass with the score tiles recomputed
// from the forward's row statistic LSE instead of stored ("What FlashAttention
// actually buys", "Why the distinction matters downstream": the backward pass
// recomputes rather than reading a stored N x N matrix). With S = scale Q K^T,
// P = exp(S - LSE) (row softmax, the forward's normaliser), O = P V:
//   D_i  = dO_i . O_i                       (kernel bwd_delta)
//   dP   = dO V^T,  dS = P * (dP - D)
//   dQ   = scale dS K                        (kernel bwd_dq: per query tile)
//   dV   = P^T dO,  dK = scale dS^T Q         (kernel bwd_dkdv: per key tile)
// Neither kernel writes anything N x N; every product runs on the matrix cores
// with float32 accumulation, P and dS rounded to the input type first.
//
// Layout of the products (32x32x16 matrix-core tiles, see fa_device.h):
//  * bwd_dq mirrors the forward kernel: a wave owns 32 query rows and keeps
//    Q^T and dO^T in registers; per 32-key tile it forms S^T = K Q^T and
//    dP^T = V dO^T (lane = query, registers = keys), P^T and dS^T in place,
//    and dQ^T += K^T dS^T with K^T read transposed from the K tile in LDS.
//  * bwd_dkdv is the same with the roles of queries and keys swapped: a wave
//    owns 32 keys and keeps K^T and V^T in registers; per 32-query tile it
//    forms S = Q K^T and dP = dO V^T (lane = key, registers = queries),
//    dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read transposed.
// Streamed tiles travel global -> LDS directly (buffer_load ... lds) through
// rings of LDS slots; tiles read both as rows and transposed use the `dual`
// chunk swizzle. Both kernels are software pipelined. In bwd_dkdv's step t
// the matrix cores form S and dP of tile t+1 and add the gradient products
// of tile t-1, while the vector ALUs turn tile t's S and dP into P and dS;
// no work of a step waits on a product issued in the same step. bwd_dq forms
// tile t's S and dP first and covers their latency with tile t-1's dQ
// product (fewer live registers: two waves per SIMD also for causal).
#include <atomic>
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;  // forward's natural-log row normaliser [B,H,N]
  float* delta;      // D [B,H,N], written by bwd_delta, read by the others
  float* lse2;       // LSE * log2(e) [B,H,N], written by bwd_delta
  char* dq;
  char* dk;
  char* dv;
  int n;         // tokens per head
  int n_tiles;   // 128-row tiles per head (query tiles for dq, key tiles for dkdv)
  int n_blocks;  // workgroups in the grid
  float c;       // scale * log2(e)
  float scale;
};

constexpr int kBwdWaves = 4;
constexpr int kDkdvWideWaves = 8;  // bwd_dkdv8
constexpr int kDqWideWaves = 8;    // bwd_dq on 256-row query tiles
#ifndef FA_BWD_DQ_WIDE
#define FA_BWD_DQ_WIDE 1
#endif
#ifndef FA_BWD_WIDE
#define FA_BWD_WIDE 1
#endif
constexpr int kBwdRows = kBwdWaves * 32;  // rows (queries or keys) per workgroup

// ---------------------------------------------------------------------------
// D_i = sum_d dO[i][d] * O[i][d], float32. D/8 lanes per row, 16 bytes each.
// Also LSE_i * log2(e), the row statistic in the base-2 units of P = 2^(c s -
// LSE log2 e), so that the other kernels read it ready to use.
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void bwd_delta(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 8;     // lanes per row
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t off = (row * D + (lane % LPR) * 8) * 2;
    const u32x4 a = ld_global16(p.o + off);
    const u32x4 b = ld_global16(p.dout + off);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += Mfma<E>::lo(a[w]) * Mfma<E>::lo(b[w]) + Mfma<E>::hi(a[w]) * Mfma<E>::hi(b[w]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && lane % LPR == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// Direct-copy bookkeeping shared by both kernels: copy t of a wave fills 1 KB
// ((wave*per + t) KB) of a 32-row tile; the lane's 16 bytes are row `row[t]`,
// chunk `col[t]` / 16 of the global tile.
template <int D, int PER>
struct TileCopy {
  static constexpr int RB = D * 2;
  static constexpr int kTile = 32 * RB;
  int row[PER];
  uint32_t col[PER];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int pos = (wave * PER + t) * 1024 + lane * 16;
      const int r = pos / RB, slot = (pos % RB) / 16;
      row[t] = r;
      col[t] = (slot ^ TileSwizzle<D>::dual(r)) * 16;
    }
  }
  // Rows at or past n re-read row n-1 (in bounds, masked by the caller).
  __device__ __forceinline__ void copy(const char* head, int tile, int n, char* dst, int wave) const {
    const int row0 = tile * 32;
    const i32x4 rs = buffer_rsrc(head + (int64_t)row0 * RB, kTile);
    const uint32_t l0 = lds_addr(dst) + wave * PER * 1024;
    const int last = n - 1 - row0;
#pragma unroll
    for (int t = 0; t < PER; ++t) load_lds16(rs, l0 + t * 1024, min(row[t], last) * RB + col[t]);
  }
};

// LDS read offsets within a dual-swizzled 32-row tile.
//  rows(kk): 16-byte operand, row l32, chunk 2 kk + g (A operand, rows of the
//            tile on the lanes);
//  tr(db, r8): transposing read, rows 4g + s/4 + 8 r8 (+ 16 h added by the
//            caller, which leaves the swizzle unchanged), features
//            db*32 + 16 ((lane/16) % 2) + 4 (s % 4), s = lane % 16.
template <int D>
struct DualOffsets {
  static constexpr int RB = D * 2;
  uint32_t rows[D / 16];
  uint32_t tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) rows[kk] = l32 * RB + ((2 * kk + g) ^ TileSwizzle<D>::dual(l32)) * 16;
    const int s = lane & 15, gp = (lane >> 4) & 1;
#pragma unroll
    for (int r8 = 0; r8 < 2; ++r8) {
      const int row = g * 4 + (s >> 2) + 8 * r8;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int ch = db * 4 + 2 * gp + ((s >> 1) & 1);
        tr[db][r8] = row * RB + (ch ^ TileSwizzle<D>::dual(row)) * 16 + (s & 1) * 8;
      }
    }
  }
  // 8-element transposed operand of feature block db, contraction half h.
  __device__ __forceinline__ u32x4 read_t(const char* tile, int db, int h) const {
    const u32x2 lo = lds_read_tr16(tile + tr[db][0] + h * 16 * RB);
    const u32x2 hi = lds_read_tr16(tile + tr[db][1] + h * 16 * RB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  __device__ __forceinline__ u32x4 read_row(const char* tile, int kk) const {
    return *reinterpret_cast<const u32x4*>(tile + rows[kk]);
  }
};

// 8 consecutive features (kk*16 + g*8 ..) of row `row` of a head, the B
// operand layout of a 32x32x16 product.
template <int D>
__device__ __forceinline__ void load_operand(const char* head, int row, int g, u32x4 (&f)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = ld_global16(head + ((int64_t)row * D + kk * 16 + g * 8) * 2);
}

// Packs 16 float32 values of a score register block into the B operand of a
// product over its 32 rows (two halves of 8 contraction slots).
template <class E>
__device__ __forceinline__ void pack_operand(const float (&x)[16], u32x4 (&f)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int w = 0; w < 4; ++w) f[h][w] = Mfma<E>::pack2(x[h * 8 + 2 * w], x[h * 8 + 2 * w + 1]);
}

template <class E, int D>
__device__ __forceinline__ void store_rows_t(char* head, int row, int n, int g, const f32x16 (&acc)[D / 32],
                                             float mul) {
  if (row >= n) return;
  char* dst = head + (int64_t)row * D * 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = Mfma<E>::pack2(acc[db][i * 4 + 0] * mul, acc[db][i * 4 + 1] * mul);
      w[1] = Mfma<E>::pack2(acc[db][i * 4 + 2] * mul, acc[db][i * 4 + 3] * mul);
      *reinterpret_cast<u32x2*>(dst + (db * 32 + i * 8 + g * 4) * 2) = w;
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 query rows; K and V tiles streamed.
//
// Step t forms S^T and dP^T of tile t, then adds the dQ product of tile t-1
// (independent of them, it covers their latency), then turns tile t's scores
// into dS. K tile t is read as rows in step t and transposed in step t+1; V
// tile t as rows in step t. Step t copies K_{t+2} into K_{t-2}'s slot (last
// read in step t-1) and V_{t+3} into V_{t-1}'s (last read in step t-1); at
// its end K_{t+1} and V_{t+1} must have landed: this step's copies may still
// be in flight.
// ---------------------------------------------------------------------------
template <class E, int D, bool CAUSAL, int NW = kBwdWaves>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq(BwdParams p) {
  constexpr int NBUF = 4, KK = D / 16, DB = D / 32;
  constexpr int BR = NW * 32;  // query rows per workgroup
  constexpr int kTile = 32 * D * 2;
  constexpr int PER = kTile / 1024 / NW;
  __shared__ __attribute__((aligned(1024))) char smem[2 * NBUF * kTile];  // K ring, V ring
  auto kbuf = [&](int b) { return smem + b * kTile; };
  auto vbuf = [&](int b) { return smem + (NBUF + b) * kTile; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_tiles;
  const int qt = CAUSAL ? p.n_tiles - 1 - blk % p.n_tiles : blk % p.n_tiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 2;

  TileCopy<D, PER> cp;
  cp.init(wave, lane);
  DualOffsets<D> off;
  off.init(lane);

  const int q_row = qt * BR + wave * 32 + l32;
  const int q_ld = min(q_row, N - 1);
  u32x4 qf[KK], dof[KK];
  load_operand<D>(p.q + head, q_ld, g, qf);
  load_operand<D>(p.dout + head, q_ld, g, dof);
  const float lse2 = p.lse2[(int64_t)bh * N + q_ld];
  const float di = p.delta[(int64_t)bh * N + q_ld];
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + 31) / 32;
  const int n_full = N / 32;
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (BR / 32)) : n_tiles;
  const int diag = CAUSAL ? (qt * BR + wave * 32) / 32 : n_tiles;
  const int my_last = min(diag, n_tiles - 1);
  const int key_lim = CAUSAL ? min(q_row, N - 1) : N - 1;
  // Ring start, virtual steps -3..-1 (K first in each): V0; K0, V1; K1, V2.
  for (int t = -3; t < 0; ++t) {
    if (t + 2 >= 0 && t + 2 < kt_end) cp.copy(p.k + head, t + 2, N, kbuf(t + 2), wave);
    if (t + 3 < kt_end) cp.copy(p.v + head, t + 3, N, vbuf(t + 3), wave);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // S^T = K Q^T and dP^T = V dO^T of one tile.
  auto scores = [&](const char* kt, const char* vt, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = Mfma<E>::run(off.read_row(kt, kk), qf[kk], s);
      dp = Mfma<E>::run(off.read_row(vt, kk), dof[kk], dp);
    }
  };
  // dS^T of one tile, rounded to the element type (hidden keys: exact zeros).
  auto grad_scores = [&](const f32x16& s, const f32x16& dp, u32x4(&dsf)[2], int key0, bool mask) {
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = exp2_fast(fmaf(s[r], p.c, -lse2));
      ds[r] = pr * (dp[r] - di);
      if (mask && key0 + score_key(0, r, g) > key_lim) ds[r] = 0.f;
    }
    pack_operand<E>(ds, dsf);
  };
  // dQ^T += K^T dS^T of one tile.
  auto accumulate = [&](const char* kt, const u32x4(&dsf)[2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[db] = Mfma<E>::run(off.read_t(kt, db, h), dsf[h], acc[db]);
  };
  auto needs_mask = [&](int t) { return t == n_full || (CAUSAL && t == diag); };

  // Before step 0: the query-side operands and statistics and every prologue
  // copy have landed. A wait the compiler sees: it then puts none of its own
  // in front of the loop's uses of qf, dof, lse2 and di, which would also
  // count (one in-order counter) the K/V copies a step has just issued.
  wait_vmem_all();
  __syncthreads();
  u32x4 db_[2][2];

  auto step = [&](int t, const u32x4(&ds_prev)[2], u32x4(&ds_cur)[2], auto slot_tag, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int b = STEADY ? decltype(slot_tag)::value : t % NBUF;
    if (STEADY || t + 2 < kt_end) cp.copy(p.k + head, t + 2, N, kbuf((b + 2) % NBUF), wave);
    if (STEADY || t + 3 < kt_end) cp.copy(p.v + head, t + 3, N, vbuf((b + 3) % NBUF), wave);
    f32x16 s, dp;
    if (STEADY || t <= my_last) scores(kbuf(b), vbuf(b), s, dp);
    if (STEADY || (t >= 1 && t - 1 <= my_last)) accumulate(kbuf((b + 3) % NBUF), ds_prev);
    if (STEADY || t <= my_last) grad_scores(s, dp, ds_cur, t * 32, !STEADY && needs_mask(t));
    if (STEADY)
      vm_wait<2 * PER>();
    else
      vm_wait<0>();
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;
  int t = 0;
  // steady groups of four from t = 0 (mod 4): every copy exists and is whole,
  // every tile lies below every wave's diagonal and needs no mask
  const int steady_end = CAUSAL ? min(n_full, qt * (BR / 32)) : n_full;
#define FA_BWD_STEP(I) step(t + (I), db_[((I) + 1) % 2], db_[(I) % 2], std::integral_constant<int, (I) % NBUF>{}, T{})
  // step 0 has no previous tile: run it at run time
  step(0, db_[1], db_[0], std::integral_constant<int, 0>{}, F{});
  db_[1][0] = db_[0][0];
  db_[1][1] = db_[0][1];
  t = 1;
  for (; t < kt_end && (t % 4) != 0; ++t) {
    step(t, db_[1], db_[0], std::integral_constant<int, 0>{}, F{});
    db_[1][0] = db_[0][0];
    db_[1][1] = db_[0][1];
  }
  for (; t + 6 < kt_end && t + 6 < n_full && t + 3 < steady_end; t += 4) {
    FA_BWD_STEP(0);
    FA_BWD_STEP(1);
    FA_BWD_STEP(2);
    FA_BWD_STEP(3);
  }
#undef FA_BWD_STEP
  for (; t < kt_end; ++t) {
    step(t, db_[1], db_[0], std::integral_constant<int, 0>{}, F{});
    db_[1][0] = db_[0][0];
    db_[1][1] = db_[0][1];
  }
  if (my_last == kt_end - 1) accumulate(kbuf((kt_end - 1) % NBUF), db_[1]);
  store_rows_t<E, D>(p.dq + head, q_row, N, g, acc, p.scale);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 key rows; Q, dO, LSE and D tiles streamed.
//
// Query tile u (counted from the workgroup's first, qt_begin) is read as rows
// for S(u), dP(u) in step u-1, transposed for dV, dK in step u+1, and its
// statistics in step u. A ring of six slots: step u copies tile u+4 into tile
// u-2's slot (last read in step u-1); at its end tile u+2 (read in step u+1)
// must have landed: the copies of steps u-1 and u may still be in flight.
// One workgroup per CU (the four 32-key waves hold K, V and both
// accumulators: about 400 registers each), so LDS is plentiful.
// ---------------------------------------------------------------------------
template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv(BwdParams p) {
  constexpr int NW = kBwdWaves, NBUF = 6, KK = D / 16, DB = D / 32;
  constexpr int kTile = 32 * D * 2;
  constexpr int PER = kTile / 1024 / NW;
  constexpr int kStats = 256;  // 32 LSE*log2(e) floats then 32 D floats
  constexpr int kSlot = 2 * kTile + kStats;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kSlot];
  auto qbuf = [&](int b) { return smem + b * kSlot; };
  auto dobuf = [&](int b) { return smem + b * kSlot + kTile; };
  auto stbuf = [&](int b) { return smem + b * kSlot + 2 * kTile; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_tiles, kt = blk % p.n_tiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 2;
  const float* lse_h = p.lse2 + (int64_t)bh * N;
  const float* del_h = p.delta + (int64_t)bh * N;

  TileCopy<D, PER> cp;
  cp.init(wave, lane);
  DualOffsets<D> off;
  off.init(lane);
  // Statistics of one 32-query tile: wave 0 copies the 32 LSE*log2(e) values,
  // wave 1 the 32 D values, 4 bytes per lane from lanes 0..31 (rows past N
  // re-read row N-1: in bounds; those query rows are masked below).
  auto copy_stats = [&](int tile, char* dst) {
    if (wave < 2 && lane < 32) {
      const float* src = wave == 0 ? lse_h : del_h;
      const int row0 = tile * 32;
      const i32x4 rs = buffer_rsrc(src + row0, 128);
      load_lds4(rs, lds_addr(dst) + wave * 128, min(lane, N - 1 - row0) * 4);
    }
  };

  const int key_row = kt * kBwdRows + wave * 32 + l32;
  const int k_ld = min(key_row, N - 1);
  u32x4 kf[KK], vf[KK];
  load_operand<D>(p.k + head, k_ld, g, kf);
  load_operand<D>(p.v + head, k_ld, g, vf);
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + 31) / 32;
  const int n_full = N / 32;
  // causal: queries before this workgroup's first key see none of its keys,
  // and this wave's keys are first seen by its diagonal query tile
  const int qt_begin = CAUSAL ? min(n_tiles, kt * (kBwdRows / 32)) : 0;
  const int diag = CAUSAL ? (kt * kBwdRows + wave * 32) / 32 : 0;
  const int cnt = n_tiles - qt_begin;
  const int first = diag - qt_begin;  // first local tile this wave works on
  auto issue = [&](int u) {
    const int b = u % NBUF;
    cp.copy(p.q + head, qt_begin + u, N, qbuf(b), wave);
    cp.copy(p.dout + head, qt_begin + u, N, dobuf(b), wave);
    copy_stats(qt_begin + u, stbuf(b));
  };
  for (int u = 0; u < 4; ++u)
    if (u < cnt) issue(u);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};

  // S = Q K^T and dP = dO V^T of one tile (lane = key, registers = queries).
  auto scores = [&](int b, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = Mfma<E>::run(off.read_row(qbuf(b), kk), kf[kk], s);
      dp = Mfma<E>::run(off.read_row(dobuf(b), kk), vf[kk], dp);
    }
  };
  // P and dS of one tile, rounded to the element type; hidden pairs (query
  // past N, or causal query before the key) get exact zeros by selection, so
  // that padding rows' values never enter a product.
  auto grad_scores = [&](int b, int u, const f32x16& s, const f32x16& dp, u32x4(&pf)[2], u32x4(&dsf)[2],
                         bool mask) {
    const float* st = reinterpret_cast<const float*>(stbuf(b));
    float pr[16], ds[16];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      // queries (r/4)*8 + g*4 + r%4 of the tile, r = 4 rr + e
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + rr * 8 + g * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 32 + rr * 8 + g * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rr * 4 + e;
        const float x = exp2_fast(fmaf(s[r], p.c, -l4[e]));
        pr[r] = x;
        ds[r] = x * (dp[r] - d4[e]);
        if (mask) {
          const int qi = (qt_begin + u) * 32 + score_key(0, r, g);
          if (qi >= N || (CAUSAL && qi < key_row)) pr[r] = ds[r] = 0.f;
        }
      }
    }
    pack_operand<E>(pr, pf);
    pack_operand<E>(ds, dsf);
  };
  // dV^T += dO^T P and dK^T += Q^T dS of one tile.
  auto accumulate = [&](int b, const u32x4(&pf)[2], const u32x4(&dsf)[2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dv[db] = Mfma<E>::run(off.read_t(dobuf(b), db, h), pf[h], dv[db]);
        dk[db] = Mfma<E>::run(off.read_t(qbuf(b), db, h), dsf[h], dk[db]);
      }
  };
  auto needs_mask = [&](int u) {
    const int t = qt_begin + u;
    return t == n_full || (CAUSAL && t == diag);
  };

  // Before step 0: kf, vf and every prologue copy have landed. A wait the
  // compiler sees, so that it puts none of its own in front of the loop's
  // uses of kf and vf (such a wait would also count the copies a step has
  // just issued).
  wait_vmem_all();
  __syncthreads();
  f32x16 sb[2], dpb[2];
  u32x4 pb[2][2], db_[2][2];
  if (0 >= first) scores(0, sb[0], dpb[0]);

  auto step = [&](int u, f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, const u32x4(&p_prev)[2],
                  const u32x4(&ds_prev)[2], u32x4(&p_cur)[2], u32x4(&ds_cur)[2], auto slot_tag, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int b = STEADY ? decltype(slot_tag)::value : u % NBUF;
    if (STEADY || u + 4 < cnt) issue(u + 4);
    if (STEADY || (u + 1 < cnt && u + 1 >= first)) scores((b + 1) % NBUF, s_nxt, dp_nxt);
    if (STEADY || (u >= 1 && u - 1 >= first)) accumulate((b + NBUF - 1) % NBUF, p_prev, ds_prev);
    if (STEADY || u >= first) grad_scores(b, u, s_cur, dp_cur, p_cur, ds_cur, !STEADY && needs_mask(u));
    if (STEADY) {
      if (wave < 2)
        vm_wait<2 * (2 * PER + 1)>();
      else
        vm_wait<2 * 2 * PER>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;
  auto rotate = [&]() {
    sb[0] = sb[1];
    dpb[0] = dpb[1];
    pb[1][0] = pb[0][0];
    pb[1][1] = pb[0][1];
    db_[1][0] = db_[0][0];
    db_[1][1] = db_[0][1];
  };
  int u = 0;
  // run-time steps until a steady group can start: u = 1 (mod 6) and (causal)
  // past every wave's diagonal tile (local tile 3)
  const int steady_from = CAUSAL ? 7 : 1;
  for (; u < cnt && u < steady_from; ++u) {
    step(u, sb[0], dpb[0], sb[1], dpb[1], pb[1], db_[1], pb[0], db_[0], std::integral_constant<int, 0>{}, F{});
    rotate();
  }
  // steady groups of six: every copy exists and is whole, no mask
#define FA_BWD_STEP(I)                                                                                          \
  step(u + (I), sb[(I) % 2], dpb[(I) % 2], sb[((I) + 1) % 2], dpb[((I) + 1) % 2], pb[((I) + 1) % 2],            \
       db_[((I) + 1) % 2], pb[(I) % 2], db_[(I) % 2], std::integral_constant<int, ((I) + 1) % NBUF>{}, T{})
  if (u == steady_from) {
    for (; u + 9 < cnt && qt_begin + u + 9 < n_full; u += 6) {
      FA_BWD_STEP(0);
      FA_BWD_STEP(1);
      FA_BWD_STEP(2);
      FA_BWD_STEP(3);
      FA_BWD_STEP(4);
      FA_BWD_STEP(5);
    }
  }
#undef FA_BWD_STEP
  for (; u < cnt; ++u) {
    step(u, sb[0], dpb[0], sb[1], dpb[1], pb[1], db_[1], pb[0], db_[0], std::integral_constant<int, 0>{}, F{});
    rotate();
  }
  if (cnt >= 1 && cnt - 1 >= first) accumulate((cnt - 1) % NBUF, pb[1], db_[1]);
  store_rows_t<E, D>(p.dk + head, key_row, N, g, dk, p.scale);
  store_rows_t<E, D>(p.dv + head, key_row, N, g, dv, 1.f);
}

// ---------------------------------------------------------------------------
// dK, dV at d = 128 on large grids, non-causal: 8 waves, 256 keys per
// workgroup, two waves per SIMD. (The causal mask's extra state does not
// fit in the 256 registers two waves per SIMD allow; causal attention keeps
// bwd_dkdv.) Keeping V in registers as well as K and both accumulators
// would need about 400 registers (one wave per SIMD, bwd_dkdv); here each
// wave's 32 V rows are staged once into LDS and read from there as the B
// operand of dP. They are kept unswizzled at a padded pitch (rows 4 banks
// apart: 16-byte row reads are conflict free), so a read's chunk offset is
// a constant in the instruction and one register addresses them all.
//
// Half-pipelined like bwd_dq: step u forms S and dP of query tile u, then
// adds tile u-1's dV and dK products (independent of them), then forms P and
// dS of tile u. Tile u is read as rows in step u and transposed in step u+1;
// step u copies tile u+2 into tile u-2's slot of a 4-slot ring (last read in
// step u-1); at its end tile u+1 must have landed (only step u's copies may
// still be in flight).
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(kDkdvWideWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv8(BwdParams p) {
  static_assert(D == 128, "8-wave copies need 1 KB per wave per tile");
  constexpr int NW = kDkdvWideWaves, NBUF = 4, KK = D / 16, DB = D / 32;
  constexpr int KR = NW * 32;  // keys per workgroup
  constexpr int kTile = 32 * D * 2;
  constexpr int PER = kTile / 1024 / NW;
  constexpr int kStats = 256;  // 32 LSE*log2(e) floats then 32 D floats
  constexpr int kSlot = 2 * kTile + kStats;
  constexpr int RB = D * 2, kVPitch = RB + 16;  // V row bytes, padded pitch
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kSlot + NW * 32 * kVPitch];
  auto qbuf = [&](int b) { return smem + b * kSlot; };
  auto dobuf = [&](int b) { return smem + b * kSlot + kTile; };
  auto stbuf = [&](int b) { return smem + b * kSlot + 2 * kTile; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  char* const vrows = smem + NBUF * kSlot + wave * 32 * kVPitch;  // this wave's 32 V rows
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_tiles, kt = blk % p.n_tiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 2;
  const float* lse_h = p.lse2 + (int64_t)bh * N;
  const float* del_h = p.delta + (int64_t)bh * N;

  TileCopy<D, PER> cp;
  cp.init(wave, lane);
  DualOffsets<D> off;
  off.init(lane);
  auto copy_stats = [&](int tile, char* dst) {
    if (wave < 2 && lane < 32) {
      const float* src = wave == 0 ? lse_h : del_h;
      const int row0 = tile * 32;
      const i32x4 rs = buffer_rsrc(src + row0, 128);
      load_lds4(rs, lds_addr(dst) + wave * 128, min(lane, N - 1 - row0) * 4);
    }
  };

  const int key_row = kt * KR + wave * 32 + l32;
  const int k_ld = min(key_row, N - 1);
  u32x4 kf[KK];
  load_operand<D>(p.k + head, k_ld, g, kf);
  {
    // this wave's 32 V rows, 16 bytes per lane and load (rows past N re-read
    // row N-1; a wave whose keys all lie past N stages the last real tile,
    // and its results are never stored)
    const int vt = min(kt * (KR / 32) + wave, (N - 1) / 32);
#pragma unroll
    for (int i = 0; i < 32 * RB / 16 / 64; ++i) {
      const int item = i * 64 + lane, r = item / (RB / 16), c = item % (RB / 16);
      const int key = min(vt * 32 + r, N - 1);
      *reinterpret_cast<u32x4*>(vrows + r * kVPitch + c * 16) = ld_global16(p.v + head + (int64_t)key * RB + c * 16);
    }
  }
  const uint32_t v_lane = l32 * kVPitch + g * 16;  // row l32, chunk 2 kk + g at + 32 kk
  __builtin_amdgcn_sched_barrier(0);

  const int cnt = (N + 31) / 32;  // query tiles
  const int n_full = N / 32;
  auto issue = [&](int u, int b) {
    cp.copy(p.q + head, u, N, qbuf(b), wave);
    cp.copy(p.dout + head, u, N, dobuf(b), wave);
    copy_stats(u, stbuf(b));
  };
  for (int u = 0; u < 2; ++u)
    if (u < cnt) issue(u, u);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};

  // S = Q K^T and dP = dO V^T of one tile (lane = key, registers = queries).
  auto scores = [&](int b, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = Mfma<E>::run(off.read_row(qbuf(b), kk), kf[kk], s);
      dp = Mfma<E>::run(off.read_row(dobuf(b), kk), *reinterpret_cast<const u32x4*>(vrows + v_lane + kk * 32), dp);
    }
  };
  // P and dS of one tile (as bwd_dkdv).
  auto grad_scores = [&](int b, int u, const f32x16& s, const f32x16& dp, u32x4(&pf)[2], u32x4(&dsf)[2],
                         bool mask) {
    const float* st = reinterpret_cast<const float*>(stbuf(b));
    float pr[16], ds[16];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + rr * 8 + g * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 32 + rr * 8 + g * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rr * 4 + e;
        const float x = exp2_fast(fmaf(s[r], p.c, -l4[e]));
        pr[r] = x;
        ds[r] = x * (dp[r] - d4[e]);
        if (mask && u * 32 + score_key(0, r, g) >= N) pr[r] = ds[r] = 0.f;
      }
    }
    pack_operand<E>(pr, pf);
    pack_operand<E>(ds, dsf);
  };
  // dV^T += dO^T P and dK^T += Q^T dS of one tile.
  auto accumulate = [&](int b, const u32x4(&pf)[2], const u32x4(&dsf)[2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dv[db] = Mfma<E>::run(off.read_t(dobuf(b), db, h), pf[h], dv[db]);
        dk[db] = Mfma<E>::run(off.read_t(qbuf(b), db, h), dsf[h], dk[db]);
      }
  };

  // K, the V rows and the first two tiles have landed (a wait the compiler
  // sees: it then puts none of its own in the loop).
  wait_vmem_all();
  __syncthreads();
  u32x4 pb[2][2], db_[2][2];  // P and dS of the current and the previous tile

  // STEADY: the slot is known at compile time, the copy exists and is whole
  // and no tile needs a mask; otherwise decided at run time (workgroup-wide
  // decisions and this wave's own kept apart, so every wave passes the same
  // barriers).
  auto step = [&](int u, const u32x4(&p_prev)[2], const u32x4(&ds_prev)[2], u32x4(&p_cur)[2],
                  u32x4(&ds_cur)[2], auto slot_tag, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int b = STEADY ? decltype(slot_tag)::value : u % NBUF;
    const bool copy = STEADY || u + 2 < cnt;
    if (copy) issue(u + 2, (b + 2) % NBUF);
    f32x16 s, dp;
    scores(b, s, dp);
    if (STEADY || u >= 1) accumulate((b + NBUF - 1) % NBUF, p_prev, ds_prev);
    // tile u's P and dS wait for its score products anyway; keeping them
    // after tile u-1's products lets both pairs share registers
    __builtin_amdgcn_sched_barrier(0);
    grad_scores(b, u, s, dp, p_cur, ds_cur, !STEADY && u == n_full);
    if (copy) {
      if (wave < 2)
        vm_wait<2 * PER + 1>();
      else
        vm_wait<2 * PER>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;
  auto rotate = [&]() {
    pb[1][0] = pb[0][0];
    pb[1][1] = pb[0][1];
    db_[1][0] = db_[0][0];
    db_[1][1] = db_[0][1];
  };
  // step 0 has no previous tile: run it at run time
  step(0, pb[1], db_[1], pb[0], db_[0], std::integral_constant<int, 0>{}, F{});
  rotate();
  int u = 1;
  // steady groups of four from u = 1: copies up to tile u + 5 exist and are
  // whole, and no tile of the group is the ragged last one
#define FA_BWD8_STEP(I)                                                                          \
  step(u + (I), pb[((I) + 1) % 2], db_[((I) + 1) % 2], pb[(I) % 2], db_[(I) % 2],                \
       std::integral_constant<int, ((I) + 1) % NBUF>{}, T{})
  for (; u + 5 < cnt && u + 5 < n_full; u += 4) {
    FA_BWD8_STEP(0);
    FA_BWD8_STEP(1);
    FA_BWD8_STEP(2);
    FA_BWD8_STEP(3);
  }
#undef FA_BWD8_STEP
  for (; u < cnt; ++u) {
    step(u, pb[1], db_[1], pb[0], db_[0], std::integral_constant<int, 0>{}, F{});
    rotate();
  }
  accumulate((cnt - 1) % NBUF, pb[1], db_[1]);
  // an opaque copy of the row index: the compiler would otherwise form the
  // 64-bit store addresses before the loop and keep them live through it
  int kr = key_row;
  asm volatile("" : "+v"(kr));
  store_rows_t<E, D>(p.dk + head, kr, N, g, dk, p.scale);
  store_rows_t<E, D>(p.dv + head, kr, N, g, dv, 1.f);
}

// ---------------------------------------------------------------------------
// float32 inputs: the same three steps with every value in float32, products
// on the float32 matrix cores (32x32x2: lane l supplies A[l%32][l/32] and
// B[l/32][l%32], one element each). Tiles are staged through registers into
// two LDS buffers, as in the float32 forward pass; one wave per SIMD.
//
// Feature pairing of the score products: product 4i + e contracts features
// 8i + e (lane group 0) and 8i + 4 + e (lane group 1) of both operands.
// Products over a 32-row tile pair rows score_key(0, r, g) of lane group g
// for register r, so a score register is directly the B operand.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_f32(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 4;     // lanes per row, 4 floats each
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t off = (row * D + (lane % LPR) * 4) * 4;
    const f32x4 a = __builtin_bit_cast(f32x4, ld_global16(p.o + off));
    const f32x4 b = __builtin_bit_cast(f32x4, ld_global16(p.dout + off));
    acc = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && lane % LPR == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// Features 8i + 4g + e (e = 0..3) of row `row`: the operand of products 4i + e.
template <int D>
__device__ __forceinline__ void load_operand_f32(const char* head, int row, int g, f32x4 (&f)[D / 8]) {
#pragma unroll
  for (int i = 0; i < D / 8; ++i)
    f[i] = __builtin_bit_cast(f32x4, ld_global16(head + ((int64_t)row * D + i * 8 + g * 4) * 4));
}

template <int D>
__device__ __forceinline__ void store_rows_f32(char* head, int row, int n, int g, const f32x16 (&acc)[D / 32],
                                               float mul) {
  if (row >= n) return;
  char* dst = head + (int64_t)row * D * 4;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 w = {acc[db][i * 4 + 0] * mul, acc[db][i * 4 + 1] * mul, acc[db][i * 4 + 2] * mul,
                       acc[db][i * 4 + 3] * mul};
      *reinterpret_cast<f32x4*>(dst + (db * 32 + i * 8 + g * 4) * 4) = w;
    }
}

// dQ (float32): one workgroup per 128 query rows, K and V tiles streamed.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dq_f32(BwdParams p) {
  constexpr int NT = kBwdWaves * 64, BC = 32;
  using KS = RowStage<BC, D * 4, D * 4 + 16, NT>;
  using VS = RowStage<BC, D * 4, D * 4 + 32, NT>;
  constexpr int kStage = KS::kBytes + VS::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_tiles;
  const int qt = CAUSAL ? p.n_tiles - 1 - blk % p.n_tiles : blk % p.n_tiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 4;
  const char* K = p.k + head;
  const char* V = p.v + head;

  const int q_row = qt * kBwdRows + wave * 32 + l32;
  const int q_ld = min(q_row, N - 1);
  f32x4 qf[D / 8], dof[D / 8];
  load_operand_f32<D>(p.q + head, q_ld, g, qf);
  load_operand_f32<D>(p.dout + head, q_ld, g, dof);
  const float lse2 = p.lse2[(int64_t)bh * N + q_ld];
  const float di = p.delta[(int64_t)bh * N + q_ld];

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  const int n_tiles = (N + BC - 1) / BC;
  const int n_full = N / BC;
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (kBwdRows / BC)) : n_tiles;
  const int diag = CAUSAL ? (qt * kBwdRows + wave * 32) / BC : n_tiles;
  const int my_last = min(diag, n_tiles - 1);
  const int key_lim = CAUSAL ? min(q_row, N - 1) : N - 1;

  KS ks;
  VS vs;
  ks.load(K, 0, N, tid);
  vs.load(V, 0, N, tid);
  ks.store(smem, tid);
  vs.store(smem + KS::kBytes, tid);
  wait_vmem_all();
  __syncthreads();
  for (int j = 0; j < kt_end; ++j) {
    const char* kb = smem + (j & 1) * kStage;
    const char* vb = kb + KS::kBytes;
    const bool more = j + 1 < kt_end;
    if (more) {
      ks.load(K, (j + 1) * BC, N, tid);
      vs.load(V, (j + 1) * BC, N, tid);
    }
    if (j <= my_last) {
      // S^T = K Q^T and dP^T = V dO^T (lane = query, registers = keys)
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const f32x4 a = __builtin_bit_cast(f32x4, KS::read16(kb, l32, (i * 8 + g * 4) * 4));
        const f32x4 b = __builtin_bit_cast(f32x4, VS::read16(vb, l32, (i * 8 + g * 4) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[i][e], st, 0, 0, 0);
          dpt = __builtin_amdgcn_mfma_f32_32x32x2f32(b[e], dof[i][e], dpt, 0, 0, 0);
        }
      }
      // dS = P (dP - D); hidden keys (past N, or causal after the query) get
      // an exact zero by selection
      const int key0 = j * BC;
      const bool mask = j == n_full || (CAUSAL && j == diag);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(fmaf(st[r], p.c, -lse2));
        ds[r] = pr * (dpt[r] - di);
        if (mask && key0 + score_key(0, r, g) > key_lim) ds[r] = 0.f;
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(KS::read4(kb, score_key(0, r, g), (db * 32 + l32) * 4),
                                                         ds[r], acc[db], 0, 0, 0);
    }
    if (more) {
      char* nb = smem + ((j + 1) & 1) * kStage;
      ks.store(nb, tid);
      vs.store(nb + KS::kBytes, tid);
    }
    __syncthreads();
  }
  store_rows_f32<D>(p.dq + head, q_row, N, g, acc, p.scale);
}

// dK, dV (float32): one workgroup per 128 key rows; Q, dO and the two
// per-query statistics (LSE*log2(e), D) streamed 32 queries at a time.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_f32(BwdParams p) {
  constexpr int NT = kBwdWaves * 64, BC = 32;
  using QS = RowStage<BC, D * 4, D * 4 + 16, NT>;
  using OS = RowStage<BC, D * 4, D * 4 + 32, NT>;
  constexpr int kStats = 2 * BC * 4;  // LSE*log2(e) then D, 32 floats each
  constexpr int kStage = QS::kBytes + OS::kBytes + kStats;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_tiles, kt = blk % p.n_tiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 4;
  const char* Q = p.q + head;
  const char* dO = p.dout + head;
  const float* lse_h = p.lse2 + (int64_t)bh * N;
  const float* del_h = p.delta + (int64_t)bh * N;

  const int key_row = kt * kBwdRows + wave * 32 + l32;
  const int k_ld = min(key_row, N - 1);
  f32x4 kf[D / 8], vf[D / 8];
  load_operand_f32<D>(p.k + head, k_ld, g, kf);
  load_operand_f32<D>(p.v + head, k_ld, g, vf);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16{};
  const int n_tiles = (N + BC - 1) / BC;
  const int n_full = N / BC;
  // causal: queries before this workgroup's first key see none of its keys,
  // and this wave's keys are first seen by its diagonal query tile
  const int qt_begin = CAUSAL ? min(n_tiles, kt * (kBwdRows / BC)) : 0;
  const int diag = CAUSAL ? (kt * kBwdRows + wave * 32) / BC : 0;

  // statistics of one query tile: threads 0..31 stage LSE*log2(e), 32..63 D
  // (queries past N re-read query N-1: in bounds, masked below)
  float stat = 0.f;
  auto load_stats = [&](int tile) {
    if (tid < 2 * BC) stat = (tid < BC ? lse_h : del_h)[min(tile * BC + tid % BC, N - 1)];
  };
  auto store_stats = [&](char* st) {
    if (tid < 2 * BC) reinterpret_cast<float*>(st)[tid] = stat;
  };
  QS qs;
  OS os;
  if (qt_begin < n_tiles) {
    qs.load(Q, qt_begin * BC, N, tid);
    os.load(dO, qt_begin * BC, N, tid);
    load_stats(qt_begin);
    qs.store(smem, tid);
    os.store(smem + QS::kBytes, tid);
    store_stats(smem + QS::kBytes + OS::kBytes);
  }
  wait_vmem_all();
  __syncthreads();
  for (int u = qt_begin; u < n_tiles; ++u) {
    const char* qb = smem + ((u - qt_begin) & 1) * kStage;
    const char* ob = qb + QS::kBytes;
    const float* stb = reinterpret_cast<const float*>(ob + OS::kBytes);
    const bool more = u + 1 < n_tiles;
    if (more) {
      qs.load(Q, (u + 1) * BC, N, tid);
      os.load(dO, (u + 1) * BC, N, tid);
      load_stats(u + 1);
    }
    if (!CAUSAL || u >= diag) {
      // S = Q K^T and dP = dO V^T (lane = key, registers = queries)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const f32x4 a = __builtin_bit_cast(f32x4, QS::read16(qb, l32, (i * 8 + g * 4) * 4));
        const f32x4 b = __builtin_bit_cast(f32x4, OS::read16(ob, l32, (i * 8 + g * 4) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], kf[i][e], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x2f32(b[e], vf[i][e], dp, 0, 0, 0);
        }
      }
      // P and dS; hidden pairs (query past N, or causal query before the key)
      // get exact zeros by selection
      const bool mask = u == n_full || (CAUSAL && u == diag);
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = score_key(0, r, g);
        const float x = exp2_fast(fmaf(s[r], p.c, -stb[ql]));
        pr[r] = x;
        ds[r] = x * (dp[r] - stb[BC + ql]);
        if (mask) {
          const int qi = u * BC + ql;
          if (qi >= N || (CAUSAL && qi < key_row)) pr[r] = ds[r] = 0.f;
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = score_key(0, r, g);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(OS::read4(ob, ql, (db * 32 + l32) * 4), pr[r], dv[db], 0,
                                                        0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(QS::read4(qb, ql, (db * 32 + l32) * 4), ds[r], dk[db], 0,
                                                        0, 0);
        }
    }
    if (more) {
      char* nb = smem + ((u + 1 - qt_begin) & 1) * kStage;
      qs.store(nb, tid);
      os.store(nb + QS::kBytes, tid);
      store_stats(nb + QS::kBytes + OS::kBytes);
    }
    __syncthreads();
  }
  store_rows_f32<D>(p.dk + head, key_row, N, g, dk, p.scale);
  store_rows_f32<D>(p.dv + head, key_row, N, g, dv, 1.f);
}

// Kernel parameters of one backward pass; *rows = B * H * N.
BwdParams bwd_params(const BwdArgs& a, int64_t* rows) {
  BwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<const char*>(a.o);
  p.dout = static_cast<const char*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = static_cast<char*>(a.dq);
  p.dk = static_cast<char*>(a.dk);
  p.dv = static_cast<char*>(a.dv);
  p.n = a.N;
  p.n_tiles = (a.N + kBwdRows - 1) / kBwdRows;
  p.n_blocks = a.B * a.H * p.n_tiles;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  *rows = (int64_t)a.B * a.H * a.N;
  p.lse2 = a.delta + *rows;
  return p;
}

// Compute units of the current device (cached per device; concurrent first
// calls store the same value).
int bwd_device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class E, int D, bool CAUSAL>
hipError_t run_bwd(const BwdArgs& a) {
  int64_t rows;
  const BwdParams p = bwd_params(a, &rows);
  constexpr int kRowsPerBlock = 4 * (64 / (D / 8));
  hipLaunchKernelGGL((bwd_delta<E, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     a.stream, p, rows);
  bool dq_done = false;
  if constexpr (D == 128) {
    // 256-row query tiles (8 waves) when the grid still has at least two of
    // them per CU: each K/V tile reaches LDS once for twice the rows
    constexpr int kRows = kDqWideWaves * 32;
    BwdParams w = p;
    w.n_tiles = (a.N + kRows - 1) / kRows;
    w.n_blocks = a.B * a.H * w.n_tiles;
    if (FA_BWD_DQ_WIDE && w.n_blocks >= 2 * bwd_device_cus()) {
      hipLaunchKernelGGL((bwd_dq<E, D, CAUSAL, kDqWideWaves>), dim3(w.n_blocks), dim3(kDqWideWaves * 64), 0,
                         a.stream, w);
      dq_done = true;
    }
  }
  if (!dq_done) hipLaunchKernelGGL((bwd_dq<E, D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  if constexpr (D == 128 && !CAUSAL) {
    // 256-key workgroups, two waves per SIMD, when the grid still has at
    // least two of them per CU
    constexpr int kKeys = kDkdvWideWaves * 32;
    BwdParams w = p;
    w.n_tiles = (a.N + kKeys - 1) / kKeys;
    w.n_blocks = a.B * a.H * w.n_tiles;
    if (FA_BWD_WIDE && w.n_blocks >= 2 * bwd_device_cus()) {
      hipLaunchKernelGGL((bwd_dkdv8<E, D>), dim3(w.n_blocks), dim3(kDkdvWideWaves * 64), 0, a.stream, w);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dkdv<E, D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t run_bwd_f32(const BwdArgs& a) {
  int64_t rows;
  const BwdParams p = bwd_params(a, &rows);
  constexpr int kRowsPerBlock = 4 * (64 / (D / 4));
  hipLaunchKernelGGL((bwd_delta_f32<D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     a.stream, p, rows);
  hipLaunchKernelGGL((bwd_dq_f32<D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  hipLaunchKernelGGL((bwd_dkdv_f32<D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a) {
  switch (a.dtype) {
    case kBF16:
      return a.d == 128 ? run_bwd<BF16, 128, CAUSAL>(a) : run_bwd<BF16, 64, CAUSAL>(a);
    case kF16:
      return a.d == 128 ? run_bwd<F16, 128, CAUSAL>(a) : run_bwd<F16, 64, CAUSAL>(a);
    default:
      return a.d == 128 ? run_bwd_f32<128, CAUSAL>(a) : run_bwd_f32<64, CAUSAL>(a);
  }
}

}  // namespace

int bwd_rows_per_block() { return kBwdRows; }

hipError_t launch_bwd(const BwdArgs& a, bool causal) { return causal ? launch_bwd_t<true>(a) : launch_bwd_t<false>(a); }

}  // namespace fa
