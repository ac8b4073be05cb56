// flash_fwd.hip -- fused tiled attention forward pass for gfx950.
//
// Method ("FlashAttention, simplified", section "The trick"; "FlashAttention"
// (interactiveprimer), "The bottleneck is memory, not multiplication"): a
// workgroup owns one tile of query rows of one (batch, head). It keeps the
// query tile in registers and streams the K/V tiles of that head through LDS.
// Per tile it forms the scores on the matrix cores, updates each row's running
// maximum m and running sum l, rescales its output accumulator by
// exp(m_old - m_new) when the maximum grows, and adds the tile's
// probabilities times V. After the last tile each row is divided once by l.
// The N x N scores exist only as register tiles.
//
// MI355X mapping:
//  * One wave = 32 query rows. Scores are formed transposed, S^T = K Q^T, so
//    that each lane holds one query row (lane % 32) and 16 keys per 32-key
//    block: row statistics are in-lane, plus one exchange with the lane 32
//    away (permlane32 swap). The same register layout is the B operand of
//    O^T = V^T P^T, so probabilities never leave registers.
//  * K tiles are copied to LDS row major; V tiles are transposed on the way
//    into LDS so the P V product reads 16-byte operands.
//  * K/V tiles are double buffered: the next tile is fetched into registers
//    while the current one is consumed, and written to the other LDS buffer
//    before the one barrier per tile.
//  * Softmax runs in base 2: p = 2^(c*s - m) with c = scale*log2(e), one FMA and
//    one v_exp_f32 per score. The accumulator is rescaled only when some row's
//    maximum grows by more than 2^8 (the running maximum may lag the true one
//    by less than that; probabilities then stay below 2^8, well inside the
//    range of every element type). The result is the same in exact
//    arithmetic because numerator and denominator share the same m.
//  * Workgroup ids are remapped so that each XCD works on contiguous heads.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units

struct FwdParams {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;         // tokens per head
  int n_qtiles;  // query tiles per head
  int n_blocks;  // workgroups in the grid
  float c;       // scale * log2(e)
};

// Score of register r of 32-key block kb in lane group g is key
// kb*32 + (r/4)*8 + g*4 + r%4 of the tile.
__device__ __forceinline__ int score_key(int kb, int r, int g) {
  return kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
}

// Hide keys at or past n (only in the last, ragged tile): they must lose the
// row extremum. `hide` is -inf when c >= 0 (maximum) and +inf otherwise.
template <int NS>
__device__ __forceinline__ void hide_tail(f32x16 (&s)[NS], int key0, int n, int g, float hide) {
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + score_key(kb, r, g) >= n) s[kb][r] = hide;
}

// max over the row's keys of c*s, for the two lanes of a pair (same query row).
// For c < 0 the maximum of c*s is c times the minimum of s.
template <int NS>
__device__ __forceinline__ float row_max_scaled(const f32x16 (&s)[NS], float c) {
  float e = s[0][0];
  if (c >= 0.f) {
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) e = fmaxf(e, s[kb][r]);
    e = pair_max(e);
  } else {
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) e = fminf(e, s[kb][r]);
    e = pair_min(e);
  }
  return e * c;
}

// Running-maximum update for one tile; returns true (wave-uniform) when the
// accumulator must be multiplied by `alpha`.
__device__ __forceinline__ bool update_max(float m_tile, float& m_run, float& l_run, float& alpha) {
  if (!__any(m_tile > m_run + kLazyRescale)) return false;
  const float m_new = fmaxf(m_run, m_tile);
  // m_new == -inf only if every score so far is -inf; keep the state as is.
  alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
  m_run = m_new;
  l_run *= alpha;
  return true;
}

// ---------------------------------------------------------------------------
// Half-precision inputs (bf16 / fp16): matrix cores, float32 accumulation.
// ---------------------------------------------------------------------------
template <class E, int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void flash_fwd_half(FwdParams p) {
  constexpr int NT = NW * 64, BR = NW * 32;
  constexpr int NS = BC / 32;  // 32-key blocks per tile
  using KS = RowStage<BC, D * 2, D * 2 + 16, NT>;
  using VS = VStage<D, BC, NT>;
  constexpr int kStage = KS::kBytes + VS::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 2;  // bytes
  const char* Q = p.q + head;
  const char* K = p.k + head;
  const char* V = p.v + head;
  const float c = p.c;

  // This lane's query row; rows past the end load row N-1 and are not stored.
  const int q_row = qt * BR + wave * 32 + l32;
  const int q_ld = q_row < N ? q_row : N - 1;
  u32x4 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = ld_global16(Q + ((int64_t)q_ld * D + kk * 16 + g * 8) * 2);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int n_tiles = (N + BC - 1) / BC;

  KS ks;
  VS vs;
  ks.load(K, 0, N, tid);
  vs.load(reinterpret_cast<const uint16_t*>(V), 0, N, tid);
  ks.store(smem, tid);
  vs.store(smem + KS::kBytes, tid);
  __syncthreads();

  // One K/V tile: scores, online-softmax update, P V. Only the last tile can
  // hold keys past N; MASK is true for that one alone.
  auto step = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* kbuf = smem + (j & 1) * kStage;
    const char* vbuf = kbuf + KS::kBytes;
    const bool more = j + 1 < n_tiles;
    if (more) {
      ks.load(K, (j + 1) * BC, N, tid);
      vs.load(reinterpret_cast<const uint16_t*>(V), (j + 1) * BC, N, tid);
    }

    // S^T = K Q^T for this tile: NS blocks of 32 keys x 32 queries.
    f32x16 s[NS];
#pragma unroll
    for (int kb = 0; kb < NS; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < NS; ++kb)
        s[kb] = Mfma<E>::run(KS::read16(kbuf, kb * 32 + l32, (kk * 16 + g * 8) * 2), qf[kk], s[kb]);

    const int key0 = j * BC;
    if constexpr (MASK) hide_tail(s, key0, N, g, c >= 0.f ? -INFINITY : INFINITY);

    float alpha;
    if (update_max(row_max_scaled(s, c), m_run, l_run, alpha)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }

    // Probabilities, rounded to the element type: B operand of O^T += V^T P^T.
    // Register r of block kb is key slot (r % 8) of half (r / 8) of that block.
    u32x4 pf[NS][2];
    float lsum = 0.f;
    const float neg_m = -m_run;
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = h * 8 + 2 * w;
          float p0 = exp2_fast(fmaf(s[kb][r], c, neg_m));
          float p1 = exp2_fast(fmaf(s[kb][r + 1], c, neg_m));
          if constexpr (MASK) {
            // explicit zero: with c == 0 a hidden score would give 0 * inf
            if (key0 + score_key(kb, r, g) >= N) p0 = 0.f;
            if (key0 + score_key(kb, r + 1, g) >= N) p1 = 0.f;
          }
          lsum += p0 + p1;
          pf[kb][h][w] = Mfma<E>::pack2(p0, p1);
        }
    l_run += lsum;

#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < NS; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[db] = Mfma<E>::run(VS::read(vbuf, db * 32 + l32, kb * 32 + h * 16 + g * 8), pf[kb][h],
                                 acc[db]);

    if (more) {
      char* nbuf = smem + ((j + 1) & 1) * kStage;
      ks.store(nbuf, tid);
      vs.store(nbuf + KS::kBytes, tid);
    }
    __syncthreads();
  };
  const int n_full = N / BC;
  for (int j = 0; j < n_full; ++j) step(j, std::false_type{});
  if (n_full < n_tiles) step(n_full, std::true_type{});

  // Epilogue: one division per row ("rescale once at the end"), O rounded to
  // nearest even; LSE = ln(2^m * l) = (m + log2 l) * ln 2.
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  if (q_row < N) {
    char* orow = p.o + head + (int64_t)q_row * D * 2;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = Mfma<E>::pack2(acc[db][i * 4 + 0] * inv, acc[db][i * 4 + 1] * inv);
        w[1] = Mfma<E>::pack2(acc[db][i * 4 + 2] * inv, acc[db][i * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + (db * 32 + i * 8 + g * 4) * 2) = w;
      }
    if (g == 0 && p.lse) p.lse[(int64_t)bh * N + q_row] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: every step in float32, products on the float32 matrix cores
// (32x32x2: lane l supplies A[l%32][l/32] and B[l/32][l%32], one element each;
// the accumulator layout is that of the half-precision product).
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void flash_fwd_f32(FwdParams p) {
  constexpr int NT = NW * 64, BR = NW * 32;
  constexpr int BC = 32;
  using KS = RowStage<BC, D * 4, D * 4 + 16, NT>;
  using VS = RowStage<BC, D * 4, D * 4 + 32, NT>;
  constexpr int kStage = KS::kBytes + VS::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * D * 4;
  const char* Q = p.q + head;
  const char* K = p.k + head;
  const char* V = p.v + head;
  const float c = p.c;

  const int q_row = qt * BR + wave * 32 + l32;
  const int q_ld = q_row < N ? q_row : N - 1;
  // Query features 8i + 4g + e (e = 0..3) feed product 4i + e, lane group g.
  f32x4 qf[D / 8];
#pragma unroll
  for (int i = 0; i < D / 8; ++i)
    qf[i] = __builtin_bit_cast(f32x4, ld_global16(Q + ((int64_t)q_ld * D + i * 8 + g * 4) * 4));

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int n_tiles = (N + BC - 1) / BC;

  KS ks;
  VS vs;
  ks.load(K, 0, N, tid);
  vs.load(V, 0, N, tid);
  ks.store(smem, tid);
  vs.store(smem + KS::kBytes, tid);
  __syncthreads();

  auto step = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* kbuf = smem + (j & 1) * kStage;
    const char* vbuf = kbuf + KS::kBytes;
    const bool more = j + 1 < n_tiles;
    if (more) {
      ks.load(K, (j + 1) * BC, N, tid);
      vs.load(V, (j + 1) * BC, N, tid);
    }

    f32x16 s[1] = {f32x16{}};
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const f32x4 a = __builtin_bit_cast(f32x4, KS::read16(kbuf, l32, (i * 8 + g * 4) * 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[i][e], s[0], 0, 0, 0);
    }

    const int key0 = j * BC;
    if constexpr (MASK) hide_tail(s, key0, N, g, c >= 0.f ? -INFINITY : INFINITY);

    float alpha;
    if (update_max(row_max_scaled(s, c), m_run, l_run, alpha)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }

    float pr[16];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pv = exp2_fast(fmaf(s[0][r], c, -m_run));
      if constexpr (MASK) {
        if (key0 + score_key(0, r, g) >= N) pv = 0.f;
      }
      pr[r] = pv;
      lsum += pv;
    }
    l_run += lsum;

    // O^T += V^T P^T, one product per score register: lane group g supplies
    // key score_key(0, r, g) for both operands.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(
            VS::read4(vbuf, score_key(0, r, g), (db * 32 + l32) * 4), pr[r], acc[db], 0, 0, 0);

    if (more) {
      char* nbuf = smem + ((j + 1) & 1) * kStage;
      ks.store(nbuf, tid);
      vs.store(nbuf + KS::kBytes, tid);
    }
    __syncthreads();
  };
  const int n_full = N / BC;
  for (int j = 0; j < n_full; ++j) step(j, std::false_type{});
  if (n_full < n_tiles) step(n_full, std::true_type{});

  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  if (q_row < N) {
    char* orow = p.o + head + (int64_t)q_row * D * 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 w = {acc[db][i * 4 + 0] * inv, acc[db][i * 4 + 1] * inv, acc[db][i * 4 + 2] * inv,
                   acc[db][i * 4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + (db * 32 + i * 8 + g * 4) * 4) = w;
      }
    if (g == 0 && p.lse) p.lse[(int64_t)bh * N + q_row] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// Tile configuration per (element type, head size).
constexpr int kWavesHalf = 4;
constexpr int kWavesF32 = 4;

template <class E, int D, int BC>
hipError_t run_half(const AttnArgs& a) {
  constexpr int BR = kWavesHalf * 32;
  FwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.n = a.N;
  p.n_qtiles = (a.N + BR - 1) / BR;
  p.n_blocks = a.B * a.H * p.n_qtiles;
  p.c = a.scale * kLog2e;
  hipLaunchKernelGGL((flash_fwd_half<E, D, BC, kWavesHalf>), dim3(p.n_blocks), dim3(kWavesHalf * 64), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t run_f32(const AttnArgs& a) {
  constexpr int BR = kWavesF32 * 32;
  FwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.n = a.N;
  p.n_qtiles = (a.N + BR - 1) / BR;
  p.n_blocks = a.B * a.H * p.n_qtiles;
  p.c = a.scale * kLog2e;
  hipLaunchKernelGGL((flash_fwd_f32<D, kWavesF32>), dim3(p.n_blocks), dim3(kWavesF32 * 64), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

int flash_rows_per_block(int dtype, int /*d*/) { return (dtype == kF32 ? kWavesF32 : kWavesHalf) * 32; }

hipError_t launch_flash(const AttnArgs& a) {
  switch (a.dtype) {
    case kBF16:
      return a.d == 128 ? run_half<BF16, 128, 64>(a) : run_half<BF16, 64, 128>(a);
    case kF16:
      return a.d == 128 ? run_half<F16, 128, 64>(a) : run_half<F16, 64, 128>(a);
    default:
      return a.d == 128 ? run_f32<128>(a) : run_f32<64>(a);
  }
}

}  // namespace fa
