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
//    tile: row statistics are in-lane, plus one exchange with the lane 32
//    away (permlane32 swap). The same register layout is the B operand of
//    O^T = V^T P^T, so probabilities never leave registers.
//  * K and V tiles are copied from global memory straight into LDS (16 bytes
//    per lane, XOR-swizzled chunks) through rings of four slots; V^T operands
//    come from transposing LDS reads. One barrier per tile.
//  * Softmax runs in base 2: p = 2^(c*s - m) with c = scale*log2(e), one FMA and
//    one v_exp_f32 per score. The running maximum m is moved only when a
//    tile's probabilities would grow too large (see flash_fwd_half); the
//    result is the same in exact arithmetic because numerator and denominator
//    share the same m.
//  * Workgroup ids are remapped so that each XCD works on contiguous heads.
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

#ifdef FA_DEBUG_CLOCK
// Phase-clock build (libflashattn_clock.so, for measurement only; the
// library proper has none of this). Wave 0 of every workgroup of
// flash_fwd_half appends one record of eight 64-bit words, taking its slot
// from a counter: s_memrealtime (100 MHz) at its start and at its end; the
// s_memtime cycles from its start to the end of its prologue (the first
// copies landed), to the end of its loop and to the end of its stores; the
// HW_ID and XCC_ID registers (the CU it ran on); and a tag 1 | NW << 8 |
// SPLIT << 16 | D << 24 | block << 32. fa_clock_clear and fa_clock_read
// (below) reset and read them.
constexpr int kClockMaxRecords = 65536;
__device__ unsigned long long fa_clock_records[8 * kClockMaxRecords];
__device__ unsigned int fa_clock_count;
#endif

namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units
// Operands of the next step's products read one step early: the first
// FA_FWD_KP K operands of the score product (FA_FWD_KP_D64 at d = 64) and the
// first FA_FWD_VP V^T operands of the P V product (tunable at build time).
// With the maximum-ILP schedule the build uses, two V^T operands measured
// fastest everywhere (one and three slower by 0.5-3 %). One K operand is
// fastest at d = 128 (two: 1.4 % slower at 10,000 tokens, the same at 4096
// and 32K); at d = 64 two are 1.3-2.3 % faster (the 512-token batch, N = 1000,
// causal).
#ifndef FA_FWD_VP
#define FA_FWD_VP 2
#endif
#ifndef FA_FWD_KP
#define FA_FWD_KP 1
#endif
#ifndef FA_FWD_KP_D64
#define FA_FWD_KP_D64 2
#endif

struct FwdParams {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;         // tokens per head
  int n_qtiles;  // query tiles per head
  int n_blocks;  // workgroups in this launch
  int blk0;      // first (query tile, head) index of this launch
  float c;       // scale * log2(e)
};


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
// A workgroup of NW waves owns NW * 32 query rows; key tiles of BC = 32.
// Every SIMD runs two waves: of two 4-wave workgroups per CU, or of one
// 8-wave workgroup (used on large grids: each K/V tile is then copied into
// LDS once for 256 query rows instead of 128). At d = 64 the one-group
// kernels fit three 4-wave workgroups per CU (three waves per SIMD). (Two 32-row blocks per wave
// would halve the LDS reads per product but needs about 460 registers per
// lane, hence one wave per SIMD; measured slower on MI355X.)
//
// Software pipeline, step t: the matrix cores form the scores of tile t+1 and
// add P_{t-1} V_{t-1} into the accumulator; the vector ALUs turn tile t's
// scores into probabilities. No work of a step waits on a product issued in
// the same step, so each wave's matrix and vector work can overlap freely and
// the two waves of a SIMD fill each other's gaps. K tiles are copied four
// tiles ahead and V tiles two (rings of four slots each; a slot is rewritten
// only after the barrier that follows its last read). The first K operands
// of the next step's score product and the first V^T operands of its P V
// product are read from LDS during the current step, so the matrix cores
// start each step without waiting on LDS.
//
// Running maximum: tile t's probabilities are first computed with m as it
// stands. If every lane's sum of its 16 probabilities is at most a limit L,
// every probability is at most L (they are non-negative) and the tile is
// done: no row maximum is taken. Otherwise (the tiles where a row's scores
// jump far above m) the tile's exact maximum is found, m, the running sums
// and the accumulator are rescaled by 2^(m_old - m_new), and the tile's
// probabilities are recomputed, now at most 1. m therefore never exceeds the
// running maximum and trails it by less than log2(L). A trailing m
// multiplies every probability of a row by one common factor, shared by
// numerator and denominator; floating point rounds relative to magnitude,
// so each probability keeps its relative rounding error, and L only has to
// keep the numbers in range. fp16: P must stay below 65504, so L = 2^15 (the
// largest power of two below it). bf16: P has the exponent range of fp32,
// and L = 2^40 leaves the float32 accumulator sum_j p_j v_j room for
// N * max|v| up to 2^87. (Limits of 2^8, 2^12 and 2^15
// measured 1-2 % faster at 32K and causal each step up; 2^40 for bf16 another
// 1.7 %, 2.7 % causal: on the 32K workload's peaky scores the maximum rarely
// jumps that far.)
//
// Normaliser of O (bf16 inputs): the probabilities enter the P V product
// rounded to bf16 (8 significant bits), so O is divided by the sum of those
// rounded values, l_r, while LSE keeps the sum of the unrounded ones, l. With
// l the weights of a row would miss summing to 1 by the rounding of its
// largest probabilities: on a row dominated by one key, O would be off by up
// to |v| * 2^-9 on top of the rounding of O itself (half an ulp, 2^-6, at
// |O| >= 4), which exceeded 2e-2 on the 32K workload's peaky rows. With l_r the weights
// sum to 1 and a dominant key's value comes through unchanged; LSE needs the
// unrounded sum (l_r would move it by up to 2^-9). For fp16 (11 bits) the
// rounding is 8 times smaller and O is divided by l.
//
// Small grids (SPLIT = 2): when there are fewer query tiles than two per CU,
// one wave per SIMD would be all the chip runs. The workgroup then has two
// groups of NW waves over the same query rows; group 0 takes the first half
// of the key tiles and group 1 the second, each through its own pair of
// rings. At the end group 1 hands its (m, l, accumulator) to group 0 through
// LDS, which merges the two partial softmaxes exactly (the same rescaling
// the running maximum uses) and writes the result.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, int SPLIT, bool NEG, bool CAUSAL>
__global__ __launch_bounds__(NW * 64 * SPLIT) __attribute__((amdgpu_waves_per_eu(D == 64 && SPLIT == 1 ? 3 : 2)))
void flash_fwd_half(FwdParams p) {
  static_assert(SPLIT == 1 || SPLIT == 2, "one or two key groups");
  constexpr int BR = NW * 32;
  constexpr int BC = 32;
  constexpr int NBUF = 4;
  constexpr int RB = D * 2;   // bytes per K / V row
  constexpr int KK = D / 16;  // contraction steps of the score product
  constexpr int DB = D / 32;  // 32-feature blocks of the output
  constexpr int kTile = BC * RB;
  constexpr int kPer = kTile / 1024 / NW;  // 1 KB direct copies per wave per tile
  constexpr float kSumLimit = std::is_same<E, BF16>::value ? 0x1p40f : 32768.f;  // L, per lane and tile
  static_assert(kTile % (1024 * NW) == 0, "a tile must split into 1 KB copies evenly over the waves");
  using Swz = TileSwizzle<D>;
  __shared__ __attribute__((aligned(1024))) char smem[SPLIT * 2 * NBUF * kTile];  // per group: K ring, V ring

#ifdef FA_DEBUG_CLOCK
  const unsigned long long clk_t0 = __builtin_amdgcn_s_memtime(), clk_r0 = __builtin_amdgcn_s_memrealtime();
#endif
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = SPLIT == 1 ? 0 : wave_id / NW;         // key group
  const int wave = SPLIT == 1 ? wave_id : wave_id % NW;  // position of the wave's 32 rows
  const int l32 = lane & 31, g = lane >> 5;
  char* const gsmem = smem + grp * 2 * NBUF * kTile;
  auto kbuf = [&](int b) { return gsmem + b * kTile; };
  auto vbuf = [&](int b) { return gsmem + (NBUF + b) * kTile; };
  const int blk = p.blk0 + xcd_remap(blockIdx.x, p.n_blocks);
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
  // ragged last tile only) re-read row N-1: in bounds, never used. FULL (a
  // compile-time tag): the caller knows the tile is whole.
  auto copy_tile = [&](const char* src, int tile, char* dst, const uint32_t(&col)[kPer], auto full_tag) {
    const int row0 = tile * BC;
    const i32x4 rs = buffer_rsrc(src + (int64_t)row0 * RB, kTile);
    const uint32_t l0 = lds_addr(dst) + wave * kPer * 1024;
    const int last = N - 1 - row0;
    if (decltype(full_tag)::value || last >= BC - 1) {
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

  // This lane's query row; rows past the end load row N-1 and are not stored.
  // The query loads are issued before any copy (the scheduling barrier keeps
  // them there), so the copy counts below are the last operations in the
  // vector-memory queue. With two key groups, both groups' waves at one
  // position need the same 32 query rows: the rows go through LDS instead
  // (see copy_q below), loaded once per workgroup and with whole-row copies.
  const int q_row = qt * BR + wave * 32 + l32;
  u32x4 qf[KK];
  if constexpr (SPLIT == 1) {
    const int q_ld = q_row < N ? q_row : N - 1;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = ld_global16(Q + ((int64_t)q_ld * D + kk * 16 + g * 8) * 2);
  }
  __builtin_amdgcn_sched_barrier(0);

  const int n_tiles = (N + BC - 1) / BC;
  const int n_full = N / BC;
  // Key tiles this workgroup visits: all of them, or (causal) up to the one
  // holding its last query row. This wave stops at its own last tile: for
  // causal attention the diagonal tile `diag` (its 32 rows start at key
  // 32 diag), where keys after each row's own position are hidden; and
  // `key_lim` is this lane's last visible key.
  //
  // Below, t counts this group's key tiles: local tile t is tile kt0 + t of
  // the head, for t < cnt. The workgroup runs `steps` steps (the larger
  // group's count); `last` is the last local tile this wave works on (-1: none).
  const int kt_end = CAUSAL ? min(n_tiles, (qt + 1) * (BR / BC)) : n_tiles;
  const int diag = CAUSAL ? (qt * BR + wave * 32) / BC : n_tiles;
  const int key_lim = CAUSAL ? min(q_row, N - 1) : N - 1;
  const int half = (kt_end + 1) / 2;
  const int kt0 = SPLIT == 2 && grp == 1 ? half : 0;
  const int cnt = SPLIT == 1 ? kt_end : (grp == 1 ? kt_end - half : half);
  const int steps = SPLIT == 1 ? kt_end : half;
  // (causal: the wave's diagonal tile, if it falls in this group's range)
  const int last = CAUSAL ? min(diag, kt0 + cnt - 1) - kt0 : cnt - 1;
  // whole tiles of every group, counted from its start
  const int full_all = SPLIT == 1 ? min(kt_end, n_full) : min(kt_end - half, n_full - half);
  using F = std::false_type;
  using T = std::true_type;
  // Two key groups: the workgroup's NW blocks of 32 query rows are copied
  // like K tiles (same chunk swizzle, so the K operand offsets read them in
  // the layout of a direct query load) into the V slots 2 and 3 of the two
  // groups, which the ring start below leaves empty: block b goes to group
  // b % 2, slot 2 + b / 2, copied by that group's waves. They are read once
  // every copy has landed, and step 0 (which refills V slot 2) comes after
  // one more barrier. Rows past N re-read row N-1, as the direct load does.
  auto qslot = [&](int b) { return smem + (b % 2) * 2 * NBUF * kTile + (NBUF + 2 + b / 2) * kTile; };
  if constexpr (SPLIT == 2) {
    static_assert(NW <= 4, "the query blocks must fit in the free V slots");
#pragma unroll
    for (int b = grp; b < NW; b += 2) {
      const int row0 = min(qt * BR + b * 32, N - 1);
      const i32x4 rs = buffer_rsrc(Q + (int64_t)row0 * RB, kTile);
      const uint32_t l0 = lds_addr(qslot(b)) + wave * kPer * 1024;
      const int last = N - 1 - row0;
#pragma unroll
      for (int t = 0; t < kPer; ++t) load_lds16(rs, l0 + t * 1024, min(cp_row[t], last) * RB + cp_k[t]);
    }
  }
  // Ring start: the copies of virtual steps -4..-1 (step t copies K_{t+4} and
  // V_{t+2}, in that order): K0; K1; K2, V0; K3, V1.
  for (int t = -4; t < 0; ++t) {
    if (t + 4 < cnt) copy_tile(K, kt0 + t + 4, kbuf(t + 4), cp_k, F{});
    if (t + 2 >= 0 && t + 2 < cnt) copy_tile(V, kt0 + t + 2, vbuf(t + 2), cp_v, F{});
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // l_run: this lane's share of the sum of the unrounded probabilities (for
  // LSE). bf16 only: lr_acc, the sums of the rounded probabilities (the
  // normaliser of O, see above), formed on the matrix cores. Per step and key
  // half, v_mfma_f32_16x16x32_bf16 takes the probabilities as its B operand
  // (lane l: query l % 32, 8 keys of lane group l / 16, the same registers as
  // the P V product) and a constant 0/1 A operand whose row 0 selects the
  // lane groups of queries 0-15 (0 and 2) and row 1 those of queries 16-31
  // (1 and 3): output row 0, column n, is query n's sum over the half, row 1
  // query n + 16's. Rows 0 and 1 sit in registers 0 and 1 of lanes 0-15.
  // (The same sums on the vector ALU, one v_dot2 per pair, measured twice as
  // costly: the kernel runs at a power-limited clock, 1.7 GHz, where every
  // extra instruction shows.)
  constexpr bool kRoundedSum = std::is_same<E, BF16>::value;
  float l_run = 0.f, lr_run = 0.f, m_run;
  f32x4 lr_acc = {};
  bf16x8 sel_ones;
  {
    const int row = lane & 15, blk = lane >> 4;
    const bool one = (row == 0 && (blk & 1) == 0) || (row == 1 && (blk & 1) == 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) sel_ones[i] = one ? (__bf16)1.0f : (__bf16)0.0f;
  }
  // hidden keys must lose the row extremum: -inf for c >= 0, +inf for c < 0
  constexpr float hide = NEG ? INFINITY : -INFINITY;

  // S^T = K Q^T for one tile (32 keys x 32 queries); its first KP operands
  // were read one step earlier (prefetch_k).
  constexpr int KP = D == 64 ? FA_FWD_KP_D64 : FA_FWD_KP;
  u32x4 pre_k[KP];
  auto prefetch_k = [&](const char* kb_lds) {
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) pre_k[kk] = *reinterpret_cast<const u32x4*>(kb_lds + k_off[kk]);
  };
  auto scores = [&](const char* kb_lds, f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 a = kk < KP ? pre_k[kk < KP ? kk : 0] : *reinterpret_cast<const u32x4*>(kb_lds + k_off[kk]);
      s = Mfma<E>::run(a, qf[kk], s);
    }
  };
  // Probabilities of one tile with the current m, rounded to the element type:
  // the B operand of O^T += V^T P^T (register r is key slot r % 8 of half
  // r / 8). Returns their float32 sum (before rounding: the row normaliser and
  // LSE are float32). Hidden keys get an explicit zero (with c == 0 a hidden
  // score would give 0 * inf). MASK_RT: the mask is decided at run time by
  // `mask`; otherwise no key of the tile is hidden.
  auto probs = [&](const f32x16& s, u32x4(&pf)[2], int key0, bool mask, auto mask_rt) {
    constexpr bool MASK_RT = decltype(mask_rt)::value;
    float ls[2];
    const float neg_m = -m_run;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = h * 8 + 2 * w;
        float p0 = exp2_fast(fmaf(s[r], c, neg_m));
        float p1 = exp2_fast(fmaf(s[r + 1], c, neg_m));
        if (MASK_RT && mask) {
          if (key0 + score_key(0, r, g) > key_lim) p0 = 0.f;
          if (key0 + score_key(0, r + 1, g) > key_lim) p1 = 0.f;
        }
        pf[h][w] = Mfma<E>::pack2(p0, p1);
        ls[h] = w == 0 ? p0 + p1 : ls[h] + (p0 + p1);
      }
    return ls[0] + ls[1];
  };
  // V^T operand (feature block db, key half h) of a tile, two transposing reads.
  auto read_vt = [&](const char* vb_lds, int db, int h) {
    const char* a = vb_lds + v_off[db] + h * 16 * RB;
    const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 8 * RB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // The first VP operands of the next step's P V product, read during the
  // current step: that step's first products then need no LDS round trip
  // right after the barrier, when both waves of a SIMD would wait on it.
  constexpr int VP = FA_FWD_VP;
  u32x4 pre_v[VP > 0 ? VP : 1];
  auto prefetch_v = [&](const char* vb_lds) {
#pragma unroll
    for (int i = 0; i < VP; ++i) pre_v[i] = read_vt(vb_lds, i / 2, i % 2);
  };
  // O^T += V^T P^T for one tile (its first VP operands were read ahead by
  // prefetch_v).
  auto accumulate = [&](const char* vb_lds, const u32x4(&pf)[2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = db * 2 + h;
        const u32x4 vt = i < VP ? pre_v[i < VP ? i : 0] : read_vt(vb_lds, db, h);
        acc[db] = Mfma<E>::run(vt, pf[h], acc[db]);
      }
  };
  // Exact maximum of c*s over a tile for this lane's row (both lanes of the
  // pair get the same value); hidden keys are set to `hide` first.
  auto tile_max = [&](f32x16& s, int key0, bool mask, auto mask_rt) {
    f32x16 one[1] = {s};
    if (decltype(mask_rt)::value && mask) {
      hide_after(one, key0, key_lim, g, hide);
      s = one[0];
    }
    return row_max_scaled_fixed<NEG>(one, c);
  };
  // Tile t's probabilities into pf and its share of the running sum.
  auto softmax_tile = [&](f32x16& s, u32x4(&pf)[2], int key0, bool mask, auto mask_rt) {
    float lt = probs(s, pf, key0, mask, mask_rt);
    if (__any(!(lt <= kSumLimit))) {
      const float m_new = fmaxf(m_run, tile_max(s, key0, mask, mask_rt));
      if constexpr (kRoundedSum) {
        // every lane takes part: lanes 0-15 rescale the sums of queries
        // lane and lane + 16, whose factors lanes lane and lane + 16 hold
        const float a_all = m_new != m_run ? exp2_fast(m_run - m_new) : 1.f;
        const float a_hi = __shfl(a_all, (lane & 15) + 16);
        lr_acc[0] *= a_all;
        lr_acc[1] *= a_hi;
      }
      if (m_new != m_run) {
        const float alpha = exp2_fast(m_run - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      lt = probs(s, pf, key0, mask, mask_rt);
    }
    l_run += lt;
    if constexpr (kRoundedSum) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lr_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel_ones, __builtin_bit_cast(bf16x8, pf[h]), lr_acc, 0, 0, 0);
    }
  };
  // Tiles that need masking: the ragged last one, and (causal) the diagonal.
  auto needs_mask = [&](int t) { return kt0 + t == n_full || (CAUSAL && kt0 + t == diag); };

  // Wait for the query loads (two key groups: the query copies) and every
  // prologue copy. The wait is one the compiler sees (it does not see the
  // copies): it then knows the query fragments are in registers on every path
  // into the loop, and puts no wait of its own in front of the loop's score
  // products. Such a wait would
  // count this step's K/V copies too (one in-order counter) and make every
  // step wait for the copies it has just issued.
  wait_vmem_all();
  __syncthreads();
#ifdef FA_DEBUG_CLOCK
  const unsigned long long clk_t1 = __builtin_amdgcn_s_memtime();
#endif
  if constexpr (SPLIT == 2) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const u32x4*>(qslot(wave) + k_off[kk]);
  }
  f32x16 sb[2];
  u32x4 pb[2][2];
  m_run = -INFINITY;
  if (last >= 0) {
    prefetch_k(kbuf(0));
    scores(kbuf(0), sb[0]);
    m_run = tile_max(sb[0], kt0 * BC, needs_mask(0), T{});  // the first tile sets m exactly
  }
  prefetch_k(kbuf(1));
  __syncthreads();  // step 0 copies K_4 into K_0's slot and V_2 into V slot 2, read by every wave by now

  // One step. Copies of K_{t+4} and V_{t+2} go out first, into the slots of
  // K_t (last read in step t-1) and V_{t-2} (last read in step t-1). During the
  // step the first operands of K_{t+2} are read ahead. At the end K_{t+3} and
  // V_{t+1} (read by step t+1) must have landed: at most this step's copies
  // may be in flight.
  // STEADY: slots known at compile time (b = t % NBUF), every copy is of a
  // whole tile, no tile of the step needs a mask and every wave works on all
  // of them. Otherwise everything is decided at run time; the workgroup-wide
  // decisions (copies, barrier) and this wave's own (does it still work on
  // tile t, t+1) are kept apart, so every wave passes the same barriers.
  // MASK_RT: tile t may need the mask (decided at run time); without it the
  // step has no masking code at all.
  auto step = [&](int t, f32x16& s_cur, f32x16& s_nxt, const u32x4(&p_prev)[2], u32x4(&p_cur)[2], auto slot_tag,
                  auto steady_tag, auto mask_rt) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int b = STEADY ? decltype(slot_tag)::value : t % NBUF;
    using Full = std::integral_constant<bool, STEADY>;
    if (STEADY || t + 4 < cnt) copy_tile(K, kt0 + t + 4, kbuf(b), cp_k, Full{});
    if (STEADY || t + 2 < cnt) copy_tile(V, kt0 + t + 2, vbuf((b + 2) % NBUF), cp_v, Full{});
    if (STEADY || t + 1 <= last) scores(kbuf((b + 1) % NBUF), s_nxt);
    if (STEADY || (t >= 1 && t - 1 <= last)) accumulate(vbuf((b + 3) % NBUF), p_prev);
    prefetch_k(kbuf((b + 2) % NBUF));  // stale (unused) past the last tile
    prefetch_v(vbuf(b));               // V_t, landed before this step began
    if (STEADY || t <= last) softmax_tile(s_cur, p_cur, (kt0 + t) * BC, !STEADY && needs_mask(t), mask_rt);
    if (STEADY)
      vm_wait<2 * kPer>();
    else
      vm_wait<0>();
    __syncthreads();
  };
  // run-time steps keep tile t's scores in sb[0] and P_{t-1} in pb[1]
  auto rotate = [&]() {
    sb[0] = sb[1];
    pb[1][0] = pb[0][0];
    pb[1][1] = pb[0][1];
  };
  step(0, sb[0], sb[1], pb[1], pb[0], std::integral_constant<int, 0>{}, F{}, T{});
  rotate();
  int t = 1;
  // Steady groups of four steps from t = 1 (mod 4): in every group, copies up
  // to local tile t + 7 exist and are whole, and (causal) the tiles up to
  // t + 4 lie below every wave's diagonal (wave 0's is qt * BR / BC; the
  // second group's tiles start at `half`).
  const int steady_end =
      (CAUSAL ? min(n_full, qt * (BR / BC)) : n_full) - (SPLIT == 2 ? half : 0);
#define FA_STEADY_STEP(I)                                                                      \
  step(t + (I), sb[(I) % 2], sb[((I) + 1) % 2], pb[((I) + 1) % 2], pb[(I) % 2],               \
       std::integral_constant<int, ((I) + 1) % NBUF>{}, T{}, F{})
  // Two 4-wave workgroups share a CU (d = 128, one key group). Measured with
  // the phase clock, one of them runs ahead, and in the last round of a
  // launch the other then finishes alone at one wave per SIMD for about a
  // fifth of the launch. Over the last 30 % of its steps a workgroup lowers
  // its waves' issue priority in three bands, so that the one behind
  // catches up and both end together (+0.6 to +3.6 % on such launches; the
  // CU shares less efficiently between equal priorities, so the gain is
  // smaller than the time spent alone).
  constexpr bool kPrioBands = !CAUSAL && D == 128 && NW == 4 && SPLIT == 1;
  if constexpr (kPrioBands) __builtin_amdgcn_s_setprio(3);
  for (; t + 7 < full_all && t + 4 < steady_end; t += 4) {
    if constexpr (kPrioBands) {
      const int rem = steps - t;
      if (rem * 10 < steps)
        __builtin_amdgcn_s_setprio(0);
      else if (rem * 5 < steps)
        __builtin_amdgcn_s_setprio(1);
      else if (rem * 10 < 3 * steps)
        __builtin_amdgcn_s_setprio(2);
    }
    FA_STEADY_STEP(0);
    FA_STEADY_STEP(1);
    FA_STEADY_STEP(2);
    FA_STEADY_STEP(3);
  }
#undef FA_STEADY_STEP
  if constexpr (kPrioBands) __builtin_amdgcn_s_setprio(0);
  // Remaining steps in pairs with the buffers' roles swapped (no register
  // moves), then at most one more. Only the ragged last tile and (causal) a
  // wave's diagonal tile need the mask, so the pairs before the first such
  // tile of this wave run without masking code (a run-time mask flag costs a
  // comparison per score). Each wave still runs `steps` steps in all.
  const int t_mask = min(n_full, CAUSAL ? diag : n_full) - kt0;
  for (; t + 1 < steps && t + 1 < t_mask; t += 2) {
    step(t, sb[0], sb[1], pb[1], pb[0], std::integral_constant<int, 0>{}, F{}, F{});
    step(t + 1, sb[1], sb[0], pb[0], pb[1], std::integral_constant<int, 0>{}, F{}, F{});
  }
  for (; t + 1 < steps; t += 2) {
    step(t, sb[0], sb[1], pb[1], pb[0], std::integral_constant<int, 0>{}, F{}, T{});
    step(t + 1, sb[1], sb[0], pb[0], pb[1], std::integral_constant<int, 0>{}, F{}, T{});
  }
  if (t < steps) {
    step(t, sb[0], sb[1], pb[1], pb[0], std::integral_constant<int, 0>{}, F{}, T{});
    rotate();
  }
  // P V of this wave's last tile if no step followed it (its V landed before
  // the last barrier).
  if (last >= 0 && last == steps - 1) accumulate(vbuf(last % NBUF), pb[1]);

#ifdef FA_DEBUG_CLOCK
  const unsigned long long clk_t2 = __builtin_amdgcn_s_memtime();
#endif
  if constexpr (kRoundedSum) {
    // the whole row's rounded sum, for this lane's query
    const float s0 = __shfl(lr_acc[0], lane & 15), s1 = __shfl(lr_acc[1], lane & 15);
    lr_run = (lane & 16) ? s1 : s0;
  }
  if constexpr (SPLIT == 2) {
    // Group 1 hands (m, l, accumulator) to group 0 through LDS (the rings are
    // free once every wave has passed the barrier); lane-major per wave.
    constexpr int kX = 3 + 16 * DB;
    static_assert(NW * kX * 64 * 4 <= SPLIT * 2 * NBUF * kTile, "exchange must fit in the rings");
    float* const xch = reinterpret_cast<float*>(smem) + wave * kX * 64 + lane;
    __syncthreads();
    if (grp == 1) {
      xch[0] = m_run;
      xch[64] = l_run;
      xch[128] = lr_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(3 + db * 16 + r) * 64] = acc[db][r];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xch[0], l1 = xch[64], lr1 = xch[128];
    const float m_new = fmaxf(m_run, m1);
    const float a0 = m_run == m_new ? 1.f : exp2_fast(m_run - m_new);
    const float a1 = m1 == m_new ? 1.f : exp2_fast(m1 - m_new);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = a0 * acc[db][r] + a1 * xch[(3 + db * 16 + r) * 64];
    l_run = a0 * l_run + a1 * l1;
    if constexpr (kRoundedSum) lr_run = a0 * lr_run + a1 * lr1;
    m_run = m_new;
  }

  // Epilogue: each row is divided by its sum l once, after the last tile
  // ("FlashAttention, simplified", "The trick"); O rounded to nearest even;
  // LSE = ln(2^m * l) = (m + log2 l) * ln 2.
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / (kRoundedSum ? lr_run : l_tot);
  // O leaves through LDS where the rings have room: a lane holds 4-feature
  // pieces of its row spread over the whole row, so stores straight from the
  // accumulator write 16 bytes into each of 32 rows per instruction (32 cache
  // lines). Each wave writes its 32 rows to LDS row-major (rows padded by 16
  // bytes, which spreads a column over the banks) and reads them back as whole
  // 16-byte chunks: every store instruction then writes 1 KB of consecutive
  // rows. The region is the wave's own, so only the rings' last readers must
  // be done (SPLIT == 1: a barrier; SPLIT == 2: the region lies past the
  // exchange area, and group 0 alone is left). The 8-wave, 256-row
  // workgroups have no room for it and store directly.
  constexpr int kRowPad = RB + 16;
  constexpr int kStage = SPLIT == 2 ? (NW * (3 + 16 * DB) * 64 * 4 + 1023) / 1024 * 1024 : 0;
  constexpr bool kStaged = kStage + NW * 32 * kRowPad <= SPLIT * 2 * NBUF * kTile;
  if constexpr (kStaged) {
    // (the lane's position recomputed here, so that nothing derived from it
    // stays live through the loop for the epilogue's sake)
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int l32_e = lane_e & 31, g_e = lane_e >> 5;
    const int q_row_e = qt * BR + wave * 32 + l32_e;
    constexpr int CPR = RB / 16;  // 16-byte chunks per row
    char* const ostage = smem + kStage + wave * 32 * kRowPad;
    if constexpr (SPLIT == 1) __syncthreads();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = Mfma<E>::pack2(acc[db][i * 4 + 0] * inv, acc[db][i * 4 + 1] * inv);
        w[1] = Mfma<E>::pack2(acc[db][i * 4 + 2] * inv, acc[db][i * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(ostage + l32_e * kRowPad + (db * 32 + i * 8 + g_e * 4) * 2) = w;
      }
    const int row0 = qt * BR + wave * 32;
    char* const o0 = p.o + head + (int64_t)row0 * RB;
#pragma unroll
    for (int k = 0; k < 32 * RB / 1024; ++k) {
      const int r = k * (1024 / RB) + lane_e / CPR, ch = lane_e % CPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(ostage + r * kRowPad + ch * 16);
      if (row0 + r < N) *reinterpret_cast<u32x4*>(o0 + r * RB + ch * 16) = w;
    }
    if (q_row_e < N && g_e == 0 && p.lse) p.lse[(int64_t)bh * N + q_row_e] = (m_run + log2f(l_tot)) * kLn2;
  } else if (q_row < N) {
    char* orow = p.o + head + (int64_t)q_row * RB;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = Mfma<E>::pack2(acc[db][i * 4 + 0] * inv, acc[db][i * 4 + 1] * inv);
        w[1] = Mfma<E>::pack2(acc[db][i * 4 + 2] * inv, acc[db][i * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + (db * 32 + i * 8 + g * 4) * 2) = w;
      }
    if (g == 0 && p.lse) p.lse[(int64_t)bh * N + q_row] = (m_run + log2f(l_tot)) * kLn2;
  }
#ifdef FA_DEBUG_CLOCK
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores complete
  const unsigned long long clk_t3 = __builtin_amdgcn_s_memtime();
  if (wave_id == 0 && lane == 0) {
    const unsigned slot = atomicAdd(&fa_clock_count, 1u);
    if (slot < kClockMaxRecords) {
      unsigned long long* r = fa_clock_records + 8 * (size_t)slot;
      r[0] = clk_r0;
      r[1] = __builtin_amdgcn_s_memrealtime();
      r[2] = clk_t1 - clk_t0;
      r[3] = clk_t2 - clk_t0;
      r[4] = clk_t3 - clk_t0;
      r[5] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
      r[6] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      r[7] = 1ull | (unsigned long long)NW << 8 | (unsigned long long)SPLIT << 16 | (unsigned long long)D << 24 |
             (unsigned long long)(unsigned)blk << 32;
    }
  }
#endif
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
constexpr int kWavesF32 = 4;

// Compute units of the current device (cached per device).
int device_cus() {
  // Per-device cache; concurrent first calls from several host threads store
  // the same value, so relaxed atomics suffice.
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
  p.blk0 = 0;
  p.c = a.scale * kLog2e;
  const int cus = device_cus();
  // Query tiles [blk0, blk0 + n) with each tile's keys split over two wave
  // groups (8-wave workgroups, one per CU).
  auto launch_split = [&](int blk0, int n) {
    FwdParams q = p;
    q.blk0 = blk0;
    q.n_blocks = n;
    if (a.scale < 0.f)
      hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, 2, true, CAUSAL>), dim3(n), dim3(kWavesHalf * 64 * 2), 0,
                         a.stream, q);
    else
      hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, 2, false, CAUSAL>), dim3(n), dim3(kWavesHalf * 64 * 2),
                         0, a.stream, q);
  };
  // fewer query tiles than two per CU: split each tile's keys over two wave groups
  if (p.n_blocks < 2 * cus) {
    launch_split(0, p.n_blocks);
    return hipGetLastError();
  }
  // Long sequences on large grids at d = 128: workgroups of 8 waves (256
  // query rows, one per CU) copy each K/V tile once for twice the rows,
  // halving the copy traffic into LDS and the K/V re-reads from L2. Only for
  // N >= 8192 (shorter heads pad a 256-row tile or run too few steps to gain:
  // measured slower from N = 16 to 1024) and with at least four full rounds of
  // workgroups, so that a partial last round stays a small share.
  if constexpr (D == 128) {
    constexpr int kWide = 2 * kWavesHalf;
    const int nq = (a.N + kWide * 32 - 1) / (kWide * 32);
    const int nb = a.B * a.H * nq;
    if (a.N >= 8192 && nb >= 4 * device_cus()) {
      p.n_qtiles = nq;
      p.n_blocks = nb;
      if (a.scale < 0.f)
        hipLaunchKernelGGL((flash_fwd_half<E, D, kWide, 1, true, CAUSAL>), dim3(nb), dim3(kWide * 64), 0,
                           a.stream, p);
      else
        hipLaunchKernelGGL((flash_fwd_half<E, D, kWide, 1, false, CAUSAL>), dim3(nb), dim3(kWide * 64), 0,
                           a.stream, p);
      return hipGetLastError();
    }
  }
  // A partial last round of at most one tile per CU (the 10,000-token
  // workload: 632 tiles on 512 slots) would run at one wave per SIMD: launch
  // the full rounds as they are, then the rest with the key split (measured
  // +1-4 % at 10K). Not for causal attention, whose light last tiles fill in
  // beside the heavy first ones within one launch (a second launch measured
  // 40 % slower there).
  const int full = p.n_blocks / (2 * cus) * (2 * cus);
  const int rest = p.n_blocks - full;
  const int n_main = !CAUSAL && rest > 0 && rest <= cus ? full : p.n_blocks;
  p.n_blocks = n_main;
  if (a.scale < 0.f)
    hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, 1, true, CAUSAL>), dim3(n_main), dim3(kWavesHalf * 64), 0,
                       a.stream, p);
  else
    hipLaunchKernelGGL((flash_fwd_half<E, D, kWavesHalf, 1, false, CAUSAL>), dim3(n_main), dim3(kWavesHalf * 64), 0,
                       a.stream, p);
  if (n_main < full + rest) {
    // The remaining 128-row tiles as twice as many 64-row tiles, each with its
    // keys split over two groups of two waves: one workgroup per CU (its LDS),
    // spread over up to twice the CUs. Blocks run head-major in both tilings,
    // so the remainder starts at the same (head, first row) in 64-row units.
    constexpr int kNarrow = 2;
    const int nq64 = (a.N + kNarrow * 32 - 1) / (kNarrow * 32);
    const int bh0 = full / p.n_qtiles, qt0 = full % p.n_qtiles;
    const int blk0 = bh0 * nq64 + qt0 * (BR / (kNarrow * 32));
    const int n64 = a.B * a.H * nq64 - blk0;
    if (n64 <= cus) {
      FwdParams q = p;
      q.n_qtiles = nq64;
      q.blk0 = blk0;
      q.n_blocks = n64;
      if (a.scale < 0.f)
        hipLaunchKernelGGL((flash_fwd_half<E, D, kNarrow, 2, true, CAUSAL>), dim3(n64), dim3(kNarrow * 64 * 2), 0,
                           a.stream, q);
      else
        hipLaunchKernelGGL((flash_fwd_half<E, D, kNarrow, 2, false, CAUSAL>), dim3(n64), dim3(kNarrow * 64 * 2), 0,
                           a.stream, q);
      return hipGetLastError();
    }
    launch_split(full, rest);
  }
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
  p.blk0 = 0;
  p.c = a.scale * kLog2e;
  hipLaunchKernelGGL((flash_fwd_f32<D, kWavesF32, CAUSAL>), dim3(p.n_blocks), dim3(kWavesF32 * 64), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

int flash_rows_per_block(int dtype, int /*d*/) { return dtype == kF32 ? kWavesF32 * 32 : kWavesHalf * 32; }

template <bool CAUSAL>
hipError_t launch(const AttnArgs& a) {
  switch (a.dtype) {
    case kBF16:
      return a.d == 128 ? run_half<BF16, 128, CAUSAL>(a) : run_half<BF16, 64, CAUSAL>(a);
    case kF16:
      return a.d == 128 ? run_half<F16, 128, CAUSAL>(a) : run_half<F16, 64, CAUSAL>(a);
    default:
      return a.d == 128 ? run_f32<128, CAUSAL>(a) : run_f32<64, CAUSAL>(a);
  }
}

hipError_t launch_flash(const AttnArgs& a) { return launch<false>(a); }
hipError_t launch_flash_causal(const AttnArgs& a) { return launch<true>(a); }

}  // namespace fa

#ifdef FA_DEBUG_CLOCK
// Phase-clock build only: reset the record counter; copy up to `max_records`
// records (8 words each) to `host`. Returns the number of records the kernels
// wrote since the last reset (records past the buffer's 65536 are dropped, so
// a return value above that means some were lost), or a negative HIP error
// code. Both calls are synchronous with respect to the device.
extern "C" int fa_clock_clear() {
  const unsigned int zero = 0;
  const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(fa::fa_clock_count), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  return e == hipSuccess ? 0 : -(int)e;
}

extern "C" int fa_clock_read(unsigned long long* host, int max_records) {
  unsigned int n = 0;
  hipError_t e = hipMemcpyFromSymbol(&n, HIP_SYMBOL(fa::fa_clock_count), sizeof n, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return -(int)e;
  unsigned int m = n < (unsigned)fa::kClockMaxRecords ? n : (unsigned)fa::kClockMaxRecords;
  if (max_records < 0) max_records = 0;
  if (m > (unsigned)max_records) m = (unsigned)max_records;
  if (m > 0 && host) {
    e = hipMemcpyFromSymbol(host, HIP_SYMBOL(fa::fa_clock_records), (size_t)m * 8 * sizeof(unsigned long long), 0,
                            hipMemcpyDeviceToHost);
    if (e != hipSuccess) return -(int)e;
  }
  return (int)n;
}
#endif

