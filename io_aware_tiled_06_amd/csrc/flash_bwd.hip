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
// Streamed tiles travel global -> LDS directly (buffer_load ... lds) through a
// 4-slot ring, three tiles ahead; tiles read both as rows and transposed use
// the `dual` chunk swizzle.
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
constexpr int kBwdRows = kBwdWaves * 32;  // rows (queries or keys) per workgroup

// ---------------------------------------------------------------------------
// D_i = sum_d dO[i][d] * O[i][d], float32. D/8 lanes per row, 16 bytes each.
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
  if (row < rows && lane % LPR == 0) p.delta[row] = acc;
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
// ---------------------------------------------------------------------------
template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq(BwdParams p) {
  constexpr int NW = kBwdWaves, NBUF = 4, KK = D / 16, DB = D / 32;
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

  const int q_row = qt * kBwdRows + wave * 32 + l32;
  const int q_ld = min(q_row, N - 1);
  u32x4 qf[KK], dof[KK];
  load_operand<D>(p.q + head, q_ld, g, qf);
  load_operand<D>(p.dout + head, q_ld, g, dof);
  const float lse2 = p.lse[(int64_t)bh * N + q_ld] * kLog2e;
  const float di = p.delta[(int64_t)bh * N + q_ld];
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + 31) / 32;
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (kBwdRows / 32)) : n_tiles;
  const int diag = CAUSAL ? (qt * kBwdRows + wave * 32) / 32 : n_tiles;
  const int my_last = min(diag, n_tiles - 1);
  const int key_lim = CAUSAL ? min(q_row, N - 1) : N - 1;
  for (int t = 0; t < 3; ++t)
    if (t < kt_end) {
      cp.copy(p.k + head, t, N, kbuf(t), wave);
      cp.copy(p.v + head, t, N, vbuf(t), wave);
    }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  for (int j = 0; j < kt_end; ++j) {
    const int b = j % NBUF;
    const bool copies = j + 3 < kt_end;
    if (copies) {
      cp.copy(p.k + head, j + 3, N, kbuf((b + 3) % NBUF), wave);
      cp.copy(p.v + head, j + 3, N, vbuf((b + 3) % NBUF), wave);
      vm_wait<6 * PER>();  // tiles j+1.. may be in flight; tile j has landed
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    if (j <= my_last) {
      const char* kt = kbuf(b);
      const char* vt = vbuf(b);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s = Mfma<E>::run(off.read_row(kt, kk), qf[kk], s);     // S^T = K Q^T
        dp = Mfma<E>::run(off.read_row(vt, kk), dof[kk], dp);  // dP^T = V dO^T
      }
      const int key0 = j * 32;
      const bool mask = j == n_tiles - 1 || (CAUSAL && j == diag);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(fmaf(s[r], p.c, -lse2));
        const bool hidden = mask && key0 + score_key(0, r, g) > key_lim;
        ds[r] = hidden ? 0.f : pr * (dp[r] - di);
      }
      u32x4 dsf[2];
      pack_operand<E>(ds, dsf);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[db] = Mfma<E>::run(off.read_t(kt, db, h), dsf[h], acc[db]);  // dQ^T += K^T dS^T
    }
    __syncthreads();  // tile j's slot is rewritten by the copies issued in step j+1
  }
  store_rows_t<E, D>(p.dq + head, q_row, N, g, acc, p.scale);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 key rows; Q, dO, LSE and D tiles streamed.
// ---------------------------------------------------------------------------
template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv(BwdParams p) {
  constexpr int NW = kBwdWaves, NBUF = 4, KK = D / 16, DB = D / 32;
  constexpr int kTile = 32 * D * 2;
  constexpr int PER = kTile / 1024 / NW;
  constexpr int kStats = 256;  // 32 LSE floats then 32 D floats
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
  const float* lse_h = p.lse + (int64_t)bh * N;
  const float* del_h = p.delta + (int64_t)bh * N;

  TileCopy<D, PER> cp;
  cp.init(wave, lane);
  DualOffsets<D> off;
  off.init(lane);
  // LSE and D of one 32-query tile: wave 0 copies the 32 LSE values, wave 1
  // the 32 D values, 4 bytes per lane from lanes 0..31 (rows past N re-read
  // row N-1: in bounds; those query rows are masked below).
  auto copy_stats = [&](int tile, char* dst) {
    if (wave < 2 && lane < 32) {
      const float* src = wave == 0 ? lse_h : del_h;
      const int row0 = tile * 32;
      const i32x4 rs = buffer_rsrc(src + row0, 128);
      load_lds4(rs, lds_addr(dst) + wave * 128, min(lane, N - 1 - row0) * 4);
    }
  };
  const int copies_per_tile = 2 * PER + (wave < 2 ? 1 : 0);

  const int key_row = kt * kBwdRows + wave * 32 + l32;
  const int k_ld = min(key_row, N - 1);
  u32x4 kf[KK], vf[KK];
  load_operand<D>(p.k + head, k_ld, g, kf);
  load_operand<D>(p.v + head, k_ld, g, vf);
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + 31) / 32;
  // causal: queries before this workgroup's first key see none of its keys
  const int qt_begin = CAUSAL ? min(n_tiles, kt * (kBwdRows / 32)) : 0;
  const int diag = CAUSAL ? (kt * kBwdRows + wave * 32) / 32 : -1;  // this wave's diagonal query tile
  auto issue = [&](int t) {
    const int b = t % NBUF;
    cp.copy(p.q + head, t, N, qbuf(b), wave);
    cp.copy(p.dout + head, t, N, dobuf(b), wave);
    copy_stats(t, stbuf(b));
  };
  for (int t = qt_begin; t < qt_begin + 3; ++t)
    if (t < n_tiles) issue(t);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};

  for (int i = qt_begin; i < n_tiles; ++i) {
    const int b = i % NBUF;
    const bool copies = i + 3 < n_tiles;
    if (copies) {
      issue(i + 3);
      if (copies_per_tile == 2 * PER + 1)
        vm_wait<3 * (2 * PER + 1)>();
      else
        vm_wait<3 * 2 * PER>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    if (!CAUSAL || i >= diag) {
      const char* qtile = qbuf(b);
      const char* dot = dobuf(b);
      const float* st = reinterpret_cast<const float*>(stbuf(b));
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s = Mfma<E>::run(off.read_row(qtile, kk), kf[kk], s);   // S = Q K^T
        dp = Mfma<E>::run(off.read_row(dot, kk), vf[kk], dp);   // dP = dO V^T
      }
      // LSE and D of this lane's 16 query rows (r/4)*8 + g*4 + r%4
      float lse2[16], dlt[16];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(st + rr * 8 + g * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 32 + rr * 8 + g * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lse2[rr * 4 + e] = a[e] * kLog2e;
          dlt[rr * 4 + e] = d4[e];
        }
      }
      const int q0 = i * 32;
      const bool mask = i == n_tiles - 1 || (CAUSAL && i == diag);
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + score_key(0, r, g);
        const float x = exp2_fast(fmaf(s[r], p.c, -lse2[r]));
        // hidden pairs get exact zeros (selected, so that padding rows' values
        // never enter a product)
        const bool hidden = mask && (qi >= N || (CAUSAL && qi < key_row));
        pr[r] = hidden ? 0.f : x;
        ds[r] = hidden ? 0.f : x * (dp[r] - dlt[r]);
      }
      u32x4 pf[2], dsf[2];
      pack_operand<E>(pr, pf);
      pack_operand<E>(ds, dsf);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dv[db] = Mfma<E>::run(off.read_t(dot, db, h), pf[h], dv[db]);     // dV^T += dO^T P
          dk[db] = Mfma<E>::run(off.read_t(qtile, db, h), dsf[h], dk[db]);  // dK^T += Q^T dS
        }
    }
    __syncthreads();  // tile i's slot is rewritten by the copies issued in step i+1
  }
  store_rows_t<E, D>(p.dk + head, key_row, N, g, dk, p.scale);
  store_rows_t<E, D>(p.dv + head, key_row, N, g, dv, 1.f);
}

template <class E, int D, bool CAUSAL>
hipError_t run_bwd(const BwdArgs& a) {
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
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  constexpr int kRowsPerBlock = 4 * (64 / (D / 8));
  hipLaunchKernelGGL((bwd_delta<E, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     a.stream, p, rows);
  hipLaunchKernelGGL((bwd_dq<E, D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  hipLaunchKernelGGL((bwd_dkdv<E, D, CAUSAL>), dim3(p.n_blocks), dim3(kBwdWaves * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a) {
  switch (a.dtype) {
    case kBF16:
      return a.d == 128 ? run_bwd<BF16, 128, CAUSAL>(a) : run_bwd<BF16, 64, CAUSAL>(a);
    default:
      return a.d == 128 ? run_bwd<F16, 128, CAUSAL>(a) : run_bwd<F16, 64, CAUSAL>(a);
  }
}

}  // namespace

int bwd_rows_per_block() { return kBwdRows; }

hipError_t launch_bwd(const BwdArgs& a, bool causal) { return causal ? launch_bwd_t<true>(a) : launch_bwd_t<false>(a); }

}  // namespace fa
