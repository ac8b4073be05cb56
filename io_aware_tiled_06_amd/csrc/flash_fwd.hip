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

// Hide keys past `lim` (this lane's last visible key) in a tile starting at
// key0: they must lose the row extremum.
template <int NS>
__device__ __forceinline__ void hide_after(f32x16 (&s)[NS], int key0, int lim, int g, float hide) {
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + score_key(kb, r, g) > lim) s[kb][r] = hide;
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

// The same with the sign of c known at compile time (NEG: c < 0), so that no
// branch splits the code around it.
template <bool NEG, int NS>
__device__ __forceinline__ float row_max_scaled_fixed(const f32x16 (&s)[NS], float c) {
  float e = s[0][0];
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) e = NEG ? fminf(e, s[kb][r]) : fmaxf(e, s[kb][r]);
  e = NEG ? pair_min(e) : pair_max(e);
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
//
// A wave owns QB blocks of 32 query rows. QB = 1 is used: two waves share
// each SIMD and cover each other's LDS and barrier waits. (QB = 2 halves the
// LDS reads per flop, since every K or V operand then feeds two products, but
// needs 448 registers per lane, hence one wave per SIMD; measured slower on
// MI355X.) Key tiles of BC = 32. K and
// V tiles are copied from global memory straight into LDS (16 bytes per lane,
// no register staging) with the chunk placement of TileSwizzle<D>, into a
// ring of NBUF = 4 buffers each, three tiles ahead of use. The loop is
// software pipelined: while the matrix cores form the scores of tile j+1, the
// vector ALUs turn the scores of tile j into probabilities; while the cores
// add P_j V_j into the accumulator, the vector ALUs find the row maxima of
// tile j+1. One barrier per tile publishes the tiles two steps ahead and
// frees the buffers the next copies overwrite.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, int QB, bool NEG, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QB == 1 ? 2 : 1)))
void flash_fwd_half(FwdParams p) {
  static_assert(!CAUSAL || QB == 1, "causal masking assumes one 32-row block per wave");
  constexpr int BR = NW * 32 * QB;
  constexpr int BC = 32;
  constexpr int NBUF = 4;
  constexpr int RB = D * 2;   // bytes per K / V row
  constexpr int KK = D / 16;  // contraction steps of the score product
  constexpr int DB = D / 32;  // 32-feature blocks of the output
  constexpr int kTile = BC * RB;
  constexpr int kPer = kTile / 1024 / NW;  // 1 KB direct copies per wave per tile
  static_assert(kTile % (1024 * NW) == 0, "a tile must split into 1 KB copies evenly over the waves");
  using Swz = TileSwizzle<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * NBUF * kTile];  // K ring, V ring
  auto kbuf = [&](int b) { return smem + b * kTile; };
  auto vbuf = [&](int b) { return smem + (NBUF + b) * kTile; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles;
  // causal: the last query tiles of a head have the most keys; start them first
  const int qt = CAUSAL ? p.n_qtiles - 1 - blk % p.n_qtiles : blk % p.n_qtiles;
  const int N = p.n;
  const int64_t head = (int64_t)bh * N * RB;  // bytes
  const char* Q = p.q + head;
  const char* K = p.k + head;
  const char* V = p.v + head;
  const float c = p.c;

  // Direct-copy sources. Copy t of this wave fills LDS bytes
  // [(wave*kPer + t) KB, +1 KB) of a tile; this lane's 16 bytes are row cp_row[t],
  // slot (pos % RB)/16, which holds chunk slot ^ swizzle(row) of that row.
  int cp_row[kPer];
  uint32_t cp_k[kPer], cp_v[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int pos = (wave * kPer + t) * 1024 + lane * 16;
    const int r = pos / RB, slot = (pos % RB) / 16;
    cp_row[t] = r;
    cp_k[t] = (slot ^ Swz::k(r)) * 16;
    cp_v[t] = (slot ^ Swz::v(r)) * 16;
  }
  // Copy tile `tile` of a head's K or V into `dst`. Rows at or past N (the
  // ragged last tile only) re-read row N-1: in bounds, never used.
  auto copy_tile = [&](const char* src, int tile, char* dst, const uint32_t(&col)[kPer]) {
    const int row0 = tile * BC;
    const i32x4 rs = buffer_rsrc(src + (int64_t)row0 * RB, kTile);
    const uint32_t l0 = lds_addr(dst) + wave * kPer * 1024;
    const int last = N - 1 - row0;
    if (last >= BC - 1) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) load_lds16(rs, l0 + t * 1024, cp_row[t] * RB + col[t]);
    } else {
#pragma unroll
      for (int t = 0; t < kPer; ++t) load_lds16(rs, l0 + t * 1024, min(cp_row[t], last) * RB + col[t]);
    }
  };

  // LDS read addresses (loop invariant). K operand of contraction step kk:
  // row l32 of the tile, chunk 2 kk + g. V^T operand of feature block db:
  // transposing reads of rows 4g + s/4 (+ 16 h, + 8), columns
  // db*32 + 16*((lane/16)%2) + 4*(s%4), s = lane % 16.
  uint32_t k_off[KK], v_off[DB];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) k_off[kk] = l32 * RB + ((2 * kk + g) ^ Swz::k(l32)) * 16;
  {
    const int s = lane & 15, gp = (lane >> 4) & 1;
    const int row = g * 4 + (s >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = db * 4 + 2 * gp + ((s >> 1) & 1);
      v_off[db] = row * RB + (ch ^ Swz::v(row)) * 16 + (s & 1) * 8;
    }
  }

  // This lane's query rows (one per block); rows past the end load row N-1
  // and are not stored. The query loads are issued before any copy (the
  // scheduling barrier keeps them there), so the copy counts below are the
  // last operations in the vector-memory queue.
  int q_row[QB];
  u32x4 qf[QB][KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    q_row[qb] = qt * BR + (wave * QB + qb) * 32 + l32;
    const int q_ld = q_row[qb] < N ? q_row[qb] : N - 1;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[qb][kk] = ld_global16(Q + ((int64_t)q_ld * D + kk * 16 + g * 8) * 2);
  }
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + BC - 1) / BC;
  const int n_full = N / BC;
  // Key tiles this workgroup visits: all of them, or (causal) up to the one
  // holding its last query row. This wave stops at its own last tile: for
  // causal attention the diagonal tile `diag` (its 32 rows start at key
  // 32 diag), where keys after each row's own position are hidden; and
  // `key_lim` is this lane's last visible key.
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (BR / BC)) : n_tiles;
  const int diag = CAUSAL ? (qt * BR + wave * 32) / BC : n_tiles;
  const int my_last = min(diag, n_tiles - 1);
  const int key_lim = CAUSAL ? min(q_row[0], N - 1) : N - 1;
  // Ring start: tiles 0..2 of K and V.
  for (int t = 0; t < 3; ++t)
    if (t < kt_end) {
      copy_tile(K, t, kbuf(t), cp_k);
      copy_tile(V, t, vbuf(t), cp_v);
    }

  f32x16 acc[QB][DB];
  float l_run[QB], m_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
    l_run[qb] = 0.f;
  }
  // keys past N must lose the row extremum: -inf for c >= 0, +inf for c < 0
  constexpr float hide = NEG ? INFINITY : -INFINITY;
  typedef f32x16 Scores[QB];

  // S^T = K Q^T for one tile (32 keys x 32 queries per block).
  auto scores = [&](const char* kb_lds, Scores& s) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kb_lds + k_off[kk]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = Mfma<E>::run(a, qf[qb][kk], s[qb]);
    }
  };
  // Probabilities of one tile, rounded to the element type: the B operand of
  // O^T += V^T P^T (register r is key slot r % 8 of half r / 8). Their float32
  // sum (before rounding: the row normaliser and LSE are float32) goes to l.
  auto probs = [&](const Scores& s, u32x4(&pf)[QB][2], int key0, bool mask) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ls[2];
      const float neg_m = -m_run[qb];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = h * 8 + 2 * w;
          float p0 = exp2_fast(fmaf(s[qb][r], c, neg_m));
          float p1 = exp2_fast(fmaf(s[qb][r + 1], c, neg_m));
          if (mask) {
            // explicit zero: with c == 0 a hidden score would give 0 * inf
            if (key0 + score_key(0, r, g) > key_lim) p0 = 0.f;
            if (key0 + score_key(0, r + 1, g) > key_lim) p1 = 0.f;
          }
          pf[qb][h][w] = Mfma<E>::pack2(p0, p1);
          ls[h] = w == 0 ? p0 + p1 : ls[h] + (p0 + p1);
        }
      l_run[qb] += ls[0] + ls[1];
    }
  };
  // O^T += V^T P^T for one tile.
  auto accumulate = [&](const char* vb_lds, const u32x4(&pf)[QB][2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* a = vb_lds + v_off[db] + h * 16 * RB;
        const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 8 * RB);
        const u32x4 vt = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = Mfma<E>::run(vt, pf[qb][h], acc[qb][db]);
      }
  };
  // Running maxima with the scores s of the next tile: moved lazily; the
  // accumulator and the sum follow them.
  auto advance_max = [&](const Scores& s) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const f32x16 one[1] = {s[qb]};
      float alpha;
      if (update_max(row_max_scaled_fixed<NEG>(one, c), m_run[qb], l_run[qb], alpha)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
      }
    }
  };
  auto mask_tail = [&](Scores& s, int key0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 one[1] = {s[qb]};
      hide_after(one, key0, key_lim, g, hide);
      s[qb] = one[0];
    }
  };
  // Tiles that need masking: the ragged last one, and (causal) the diagonal.
  auto needs_mask = [&](int t) { return t == n_full || (CAUSAL && t == diag); };

  // Step 0 reads K_1 and V_0; tiles 0 and 1 have landed once at most the
  // copies of tile 2 are in flight (vector-memory operations complete in
  // issue order).
  if (kt_end > 2)
    vm_wait<2 * kPer>();
  else
    vm_wait<0>();
  __syncthreads();
  Scores sa, sb;
  scores(kbuf(0), sa);
  if (needs_mask(0)) mask_tail(sa, 0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const f32x16 one[1] = {sa[qb]};
    m_run[qb] = row_max_scaled_fixed<NEG>(one, c);
  }

  // One step: tile j's probabilities and P V, tile j+1's scores and maximum.
  // Copies of K_{j+3} and V_{j+3} go out first, into the buffers of tile
  // j-1, which the previous barrier freed; at the end the copies of tiles
  // j+2, issued one step earlier, must have landed before the barrier.
  // STEADY: buffers known at compile time (B = j % NBUF), tile j+1 needs no
  // mask for any wave, copies of this step exist. Otherwise everything is
  // decided at run time; the workgroup-wide decisions (copies, barrier) and
  // this wave's own (does it still work on tile j, j+1) are kept apart, so
  // every wave passes the same barriers.
  auto step = [&](int j, Scores& s_cur, Scores& s_nxt, auto b_tag, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int b = STEADY ? decltype(b_tag)::value : j % NBUF;
    const bool copies = STEADY || j + 3 < kt_end;
    if (copies) {
      copy_tile(K, j + 3, kbuf((b + 3) % NBUF), cp_k);
      copy_tile(V, j + 3, vbuf((b + 3) % NBUF), cp_v);
    }
    const bool wg_next = STEADY || j + 1 < kt_end;
    const bool next = STEADY || j + 1 <= my_last;
    const bool cur = STEADY || j <= my_last;
    if (next) scores(kbuf((b + 1) % NBUF), s_nxt);
    if (cur) {
      u32x4 pf[QB][2];
      probs(s_cur, pf, j * BC, !STEADY && needs_mask(j));
      accumulate(vbuf(b), pf);
    }
    if (next) {
      if (!STEADY && needs_mask(j + 1)) mask_tail(s_nxt, (j + 1) * BC);
      advance_max(s_nxt);
    }
    if (wg_next) {
      if (copies)
        vm_wait<2 * kPer>();
      else
        vm_wait<0>();
      __syncthreads();
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  int j = 0;
  // steady groups: every step's copies exist (j + 3 + 3 < kt_end), the tile
  // after the group's last one is full (j + 4 < n_full) and (causal) lies
  // below every wave's diagonal (j + 4 < qt * BR / BC, wave 0's diagonal)
  const int steady_end = CAUSAL ? min(n_full, qt * (BR / BC)) : n_full;
  for (; j + 6 < kt_end && j + 4 < steady_end; j += 4) {
    step(j, sa, sb, std::integral_constant<int, 0>{}, T{});
    step(j + 1, sb, sa, std::integral_constant<int, 1>{}, T{});
    step(j + 2, sa, sb, std::integral_constant<int, 2>{}, T{});
    step(j + 3, sb, sa, std::integral_constant<int, 3>{}, T{});
  }
  for (; j < kt_end; ++j) {
    step(j, sa, sb, std::integral_constant<int, 0>{}, F{});
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sa[qb] = sb[qb];
  }

  // Epilogue: one division per row ("rescale once at the end"), O rounded to
  // nearest even; LSE = ln(2^m * l) = (m + log2 l) * ln 2.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (q_row[qb] < N) {
      char* orow = p.o + head + (int64_t)q_row[qb] * RB;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w[0] = Mfma<E>::pack2(acc[qb][db][i * 4 + 0] * inv, acc[qb][db][i * 4 + 1] * inv);
          w[1] = Mfma<E>::pack2(acc[qb][db][i * 4 + 2] * inv, acc[qb][db][i * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + (db * 32 + i * 8 + g * 4) * 2) = w;
        }
      if (g == 0 && p.lse) p.lse[(int64_t)bh * N + q_row[qb]] = (m_run[qb] + log2f(l_tot)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: every step in float32, products on the float32 matrix cores
// (32x32x2: lane l supplies A[l%32][l/32] and B[l/32][l%32], one element each;
// the accumulator layout is that of the half-precision product).
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
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
  const int bh = blk / p.n_qtiles;
  const int qt = CAUSAL ? p.n_qtiles - 1 - blk % p.n_qtiles : blk % p.n_qtiles;
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
  const int n_full = N / BC;
  // key tiles of this workgroup and of this wave (see flash_fwd_half)
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (BR / BC)) : n_tiles;
  const int diag = CAUSAL ? (qt * BR + wave * 32) / BC : n_tiles;
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

  auto step = [&](int j, auto mask_tag) {
    constexpr bool MASK_ANY = decltype(mask_tag)::value;
    const bool MASK = MASK_ANY && (j == n_full || (CAUSAL && j == diag));
    const char* kbuf = smem + (j & 1) * kStage;
    const char* vbuf = kbuf + KS::kBytes;
    const bool more = j + 1 < kt_end;
    if (more) {
      ks.load(K, (j + 1) * BC, N, tid);
      vs.load(V, (j + 1) * BC, N, tid);
    }

    if (!CAUSAL || j <= my_last) {
      f32x16 s[1] = {f32x16{}};
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const f32x4 a = __builtin_bit_cast(f32x4, KS::read16(kbuf, l32, (i * 8 + g * 4) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[i][e], s[0], 0, 0, 0);
      }

      const int key0 = j * BC;
      if (MASK) hide_after(s, key0, key_lim, g, c >= 0.f ? -INFINITY : INFINITY);

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
        if (MASK) {
          if (key0 + score_key(0, r, g) > key_lim) pv = 0.f;
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
    }

    if (more) {
      char* nbuf = smem + ((j + 1) & 1) * kStage;
      ks.store(nbuf, tid);
      vs.store(nbuf + KS::kBytes, tid);
    }
    __syncthreads();
  };
  if (CAUSAL) {
    for (int j = 0; j < kt_end; ++j) step(j, std::true_type{});
  } else {
    for (int j = 0; j < n_full; ++j) step(j, std::false_type{});
    if (n_full < n_tiles) step(n_full, std::true_type{});
  }

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
constexpr int kQueryBlocksHalf = 1;
constexpr int kWavesF32 = 4;

template <class E, int D, int QB, bool CAUSAL>
hipError_t run_half(const AttnArgs& a) {
  constexpr int BR = kWavesHalf * 32 * QB;
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
  if (a.scale < 0.f)
    hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, QB, true, CAUSAL>), dim3(p.n_blocks),
                       dim3(kWavesHalf * 64), 0, a.stream, p);
  else
    hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, QB, false, CAUSAL>), dim3(p.n_blocks),
                       dim3(kWavesHalf * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
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
  hipLaunchKernelGGL((flash_fwd_f32<D, kWavesF32, CAUSAL>), dim3(p.n_blocks), dim3(kWavesF32 * 64), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

int flash_rows_per_block(int dtype, int /*d*/) { return dtype == kF32 ? kWavesF32 * 32 : kWavesHalf * 32 * kQueryBlocksHalf; }

template <bool CAUSAL>
hipError_t launch(const AttnArgs& a) {
  constexpr int QB = kQueryBlocksHalf;
  switch (a.dtype) {
    case kBF16:
      return a.d == 128 ? run_half<BF16, 128, QB, CAUSAL>(a) : run_half<BF16, 64, QB, CAUSAL>(a);
    case kF16:
      return a.d == 128 ? run_half<F16, 128, QB, CAUSAL>(a) : run_half<F16, 64, QB, CAUSAL>(a);
    default:
      return a.d == 128 ? run_f32<128, CAUSAL>(a) : run_f32<64, CAUSAL>(a);
  }
}

hipError_t launch_flash(const AttnArgs& a) { return launch<false>(a); }
hipError_t launch_flash_causal(const AttnArgs& a) { return launch<true>(a); }

}  // namespace fa
