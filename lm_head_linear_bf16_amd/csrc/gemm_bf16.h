// bf16 MFMA GEMM core for gfx950 and the three contractions of the fused
// LM-head cross-entropy built on it.
//
// Every GEMM here computes C[m, n] = sum_k A(m, k) B(n, k), bf16 in, fp32
// accumulate, with each operand read in its natural row-major layout: either
// K contiguous (h and W for the logits, the stored exponentials E for dH) or
// K as the row index (W for dH, E for dW), the latter transposed on its way
// out of LDS by the gfx950 transpose read.
//
// Tiling (CDNA4: 64-wide waves, 160 KB LDS, v_mfma_f32_16x16x32_bf16):
//   * block tile 256 x 256, K step 64, 512 threads = 8 waves in a 2 (M) x 4
//     (N) grid, each wave owning a 128 x 64 accumulator (8 x 4 MFMA tiles of
//     16 x 16, 128 fp32 per lane), two waves per SIMD so one wave's waits are
//     covered by the other's MFMAs;
//   * two LDS stages of (256 + 256) x 64 bf16 = 64 KB each, filled by
//     buffer loads straight into LDS, 16 bytes per lane (no VGPR staging).
//     The 16-byte chunk
//     c of row r sits at chunk position c ^ ((r >> 1) & 7): the LDS serves a
//     16-byte read to 16 lanes per cycle, and the 16 rows those lanes read
//     then fall on 16 distinct bank groups (measured: no bank-conflict
//     cycles);
//   * each 32-wide K step reads the next step's fragments while it issues
//     its MFMAs, one LDS read between two MFMAs (explicit scheduling groups);
//     the stage barrier sits in the middle of the last step's MFMAs and the
//     loop body has no branch, so the next tile's first reads and the global
//     loads of the tile after overlap MFMA work; the global loads are spread
//     between MFMAs, one operand's after the barrier, the other's early in
//     the next step;
//   * blocks are renumbered so that consecutive logical tiles run on one XCD
//     (the dispatcher deals block ids round-robin over the 8 XCDs) and tiles
//     are walked in groups of `group_m` rows of tiles, so operand slabs are
//     shared in that XCD's L2.
//
// Rows past M (or N) are read as zeros (the buffer range ends at the last
// valid row; gathered rows are clamped to the last valid one) and masked in
// the epilogues.  K must be a multiple of 64.
#pragma once

#include "fldce_common.h"

namespace fldce {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWavesM = 2, kWavesN = 4, kWaves = kWavesM * kWavesN;
constexpr int kGemmThreads = kWaves * 64;
constexpr int kTM = kBM / kWavesM / 16, kTN = kBN / kWavesN / 16;  // 16x16 tiles per wave: 8 x 4
constexpr int kABytes = kBM * kBK * 2;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;
constexpr int kGemmLds = 2 * kStageBytes;  // 128 KB
constexpr int kRoundsA = kBM / (kWaves * 8), kRoundsB = kBN / (kWaves * 8);

struct TileCoord {
  int tm, tn, split;
  bool active;
};

// Block id -> (tile row, tile column, split), XCD-aware and grouped.  The
// dispatcher deals block ids round-robin over the 8 XCDs, so XCD x runs the
// blocks bid = x, x + 8, ...; the work items (tiles_m x tiles_n x splits,
// tiles_m possibly fewer than the grid was sized for, known only on the
// device) are cut into 8 contiguous ranges, one per XCD, so every XCD gets
// the same share and neighbouring tiles share its L2.  Within the order,
// tiles go in groups of `group_m` tile rows.  Blocks without an item are
// inactive.
__host__ __device__ inline TileCoord tile_coord_of(int bid, int tiles_m, int tiles_n, int splits,
                                                   int group_m) {
  const int x = bid % 8, idx = bid / 8;
  const int tiles = tiles_m * tiles_n;
  const int A = tiles * splits;
  const int per = A / 8, rem = A % 8;
  TileCoord c{0, 0, 0, idx < per + (x < rem ? 1 : 0)};
  if (!c.active) return c;
  int b = x * per + min(x, rem) + idx;
  c.split = b / tiles;
  b -= c.split * tiles;
  const int width = group_m * tiles_n;
  const int g = b / width;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int w = b - g * width;
  c.tm = first_m + w % gm;
  c.tn = w / gm;
  return c;
}
__device__ __forceinline__ TileCoord tile_coord(int tiles_m, int tiles_n, int splits, int group_m) {
  return tile_coord_of(blockIdx.x, tiles_m, tiles_n, splits, group_m);
}

// 16-byte chunk position of logical chunk c (0..7) in LDS row r.
__device__ __forceinline__ int lds_chunk(int c, int r) { return c ^ ((r >> 1) & 7); }

// Scheduling groups with loads: NL times (one MFMA, one global->LDS load,
// DR LDS reads), then ND (MFMA, LDS read) pairs, then the rest of NM MFMAs.
template <int NL, int DR, int ND, int NM>
__device__ __forceinline__ void spread_groups() {
  static_assert(NL + ND <= NM, "more groups than MFMAs");
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one load
    __builtin_amdgcn_sched_group_barrier(0x100, DR, 0);  // DR LDS reads
  }
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (NM > NL + ND) __builtin_amdgcn_sched_group_barrier(0x008, NM - NL - ND, 0);
}

typedef floatx4 Acc[kTM][kTN];
typedef short v4i16 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Operand tiles.  Tile<false>: the operand is row-major with K contiguous
// (rows = the M or N index); its LDS tile is 256 rows x 64 K (128 B rows,
// 16-byte chunk c of row r at position lds_chunk(c, r)); a fragment is one
// 16-byte LDS read.
//
// Tile<true>: the operand is row-major with K as the ROW index (e.g. W [V, H]
// as the K = V operand of dH, or E [C, V] as the K = C operand
// of dW); its LDS tile is 64 K-rows x 256 columns (512 B rows, 32-byte
// segment s of row r at position s ^ tr_swz(r)) and a fragment is gathered
// with two ds_read_b64_tr_b16.  Within each 16-lane group that instruction
// returns, to lane i, element (i mod 4) of the 8-byte reads of lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4; when those lanes read rows k..k+3 at
// columns 4*(lane mod 4), lane i receives column i of rows k..k+3, i.e. four
// consecutive K of its own row, which is the MFMA operand layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tr_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// Buffer resources for the operand loads.  A raw buffer load takes its base
// and byte range from a descriptor in scalar registers, a per-lane byte
// offset from a vector register and a wave-uniform byte offset from a scalar
// register; lanes whose vector offset is at or past the range read zero
// without touching memory (the scalar offset is not range-checked).  So the
// per-lane offsets are computed once per tile and each K step changes only
// scalars.  Third descriptor word: raw 32-bit data of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n,
                                           kRsrcWord3);
}
__device__ __forceinline__ void buffer_to_lds(Rsrc r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, FLDCE_LPTR(lds), 16, voff, soff, 0, 0);
}

template <bool kTr, bool kGather = false>
struct Tile;

// K contiguous, rows read through a buffer whose range ends at the last
// valid row: rows past it load as zeros.  Per lane the row offset r * ldx
// (r < 256) is in the vector offset, K (k_begin + 64 t) in the scalar one.
// Needs 256 * ldx * 2 < 2^32 (ldx < 2^23), which the entry points ensure.
template <>
struct Tile<false, false> {
  static constexpr int kReads = 1;  // LDS reads per fragment
  Rsrc rs;
  uint32_t voff[4];
  uint32_t kb;  // K offset in bytes
  // rows = number of valid rows (M or N); r0 = first row of the tile.
  __device__ __forceinline__ void init(const bf16* X, int64_t ldx, int rows, int cols, int r0,
                                       int64_t k_begin, int lane, int wave,
                                       const int* = nullptr, int64_t = 0) {
    (void)cols;
    rs = make_rsrc(X + (int64_t)r0 * ldx, (int64_t)(rows - r0) * ldx * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * kWaves * 8 + wave * 8 + (lane >> 3);
      voff[i] = (uint32_t)((int64_t)r * ldx * 2 + lds_chunk(lane & 7, r) * 16);
    }
    kb = (uint32_t)(k_begin * 2);
  }
  // load i (of 4) of K tile t into the LDS tile
  __device__ __forceinline__ void issue1(char* tile, int t, int wave, int i) const {
    buffer_to_lds(rs, tile + wave * 8 * 128 + i * kWaves * 8 * 128, voff[i],
                  kb + (uint32_t)t * (kBK * 2));
  }
  // fragments for 16-row sub-tiles at rows off + 16 t
  template <int T>
  __device__ __forceinline__ void frags(const char* tile, int ks, int off, int lane, bf16x8 (&f)[T]) const {
    const char* b = tile + (off + (lane & 15)) * 128 + (lds_chunk(ks * 4 + (lane >> 4), lane & 15) << 4);
#pragma unroll
    for (int t = 0; t < T; ++t) f[t] = *(const bf16x8*)(b + t * 16 * 128);
  }
};

// K contiguous, rows gathered: tile row q is source row gidx[goff + q]
// (clamped to the valid rows), read with per-lane global addresses.
template <>
struct Tile<false, true> {
  static constexpr int kReads = 1;
  const bf16* p[4];
  __device__ __forceinline__ void init(const bf16* X, int64_t ldx, int rows, int cols, int r0,
                                       int64_t k_begin, int lane, int wave,
                                       const int* gidx = nullptr, int64_t goff = 0) {
    (void)cols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * kWaves * 8 + wave * 8 + (lane >> 3);
      const int64_t q = min(r0 + r, rows - 1);
      p[i] = X + (int64_t)gidx[goff + q] * ldx + lds_chunk(lane & 7, r) * 8 + k_begin;
    }
  }
  __device__ __forceinline__ void issue1(char* tile, int t, int wave, int i) const {
    __builtin_amdgcn_global_load_lds(FLDCE_GPTR(p[i] + (int64_t)t * kBK),
                                     FLDCE_LPTR(tile + wave * 8 * 128 + i * kWaves * 8 * 128), 16, 0, 0);
  }
  template <int T>
  __device__ __forceinline__ void frags(const char* tile, int ks, int off, int lane, bf16x8 (&f)[T]) const {
    Tile<false, false>().frags<T>(tile, ks, off, lane, f);
  }
};

// K as the row index: each K step reads 64 source rows through a buffer
// based at its first row (and the tile's first column), whose range ends at
// the last valid row, so rows past it load as zeros; per lane the offset of
// its row (< 64) and column is fixed.  Only scalars change per step.
template <>
struct Tile<true, false> {
  static constexpr int kReads = 2;
  const bf16* X;  // column c0 of row 0
  int64_t ldx, kb, tail;  // tail: bytes from column c0 of a row to the end of that row
  int krows;
  uint32_t voff[4];
  // rows = number of valid K rows of the source; cols = valid columns;
  // c0 = first column of the tile; kb = first K row
  __device__ __forceinline__ void init(const bf16* X_, int64_t ld, int rows, int cols, int c0,
                                       int64_t kb_, int lane, int wave, const int* = nullptr,
                                       int64_t = 0) {
    X = X_ + c0;
    ldx = ld;
    krows = rows;
    kb = kb_;
    tail = (ld - c0) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 16 + wave * 2 + (lane >> 5);  // LDS row this lane fills
      const int pos = lane & 31;                       // 16-byte unit in the 512 B row
      const int u = (((pos >> 1) ^ tr_swz(r)) << 1) | (pos & 1);
      voff[i] = (uint32_t)((int64_t)r * ld * 2 + (int64_t)(min(c0 + u * 8, cols - 8) - c0) * 2);
    }
  }
  __device__ __forceinline__ void issue1(char* tile, int t, int wave, int i) const {
    const int64_t row0 = kb + (int64_t)t * kBK;
    // valid bytes from the base: the rest of row row0 and the rows after it
    const Rsrc rs = make_rsrc(X + row0 * ldx, (krows - row0 - 1) * ldx * 2 + tail);
    buffer_to_lds(rs, tile + wave * 2 * 512 + i * 16 * 512, voff[i], 0);
  }
  template <int T>
  __device__ __forceinline__ void frags(const char* tile, int ks, int off, int lane, bf16x8 (&f)[T]) const {
    const int grp = lane >> 4, s4 = lane & 15;
    const int fsw = tr_swz(grp * 8 + (s4 >> 2));
    const char* b = tile + (ks * 32 + grp * 8 + (s4 >> 2)) * 512 + (s4 & 3) * 8;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const char* q = b + (((off >> 4) + t) ^ fsw) * 32;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3)))*)(q));
      const v4i16 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3)))*)(q + 4 * 512));
      f[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

// Main loop: acc[i][j] (wave sub-tile i along M, j along N) accumulates
// sum_k A(m, k) B(n, k) for m in [m0, m0+256), n in [n0, n0+256) over K tiles
// [kt0, kt0 + nk), starting from zero (kZeroAcc) or from the values the
// caller put in acc.  For a normal operand X_rows/X_cols are (valid rows,
// unused); for a transposed one (valid K rows, valid columns).
// Load orders of the main loop: every load of a K step issued at once after
// the stage barrier (kLoadBurst), or each operand's loads spread over the
// window between two barriers: the first operand's after barrier t (K tile
// t+2), one next to each of four MFMAs, and the other's at the start of step
// t+1 (same tile), interleaved with that step's fragment reads, which leaves
// them about a quarter step less to land.  Measured at the headline shapes
// (one box, same inputs): the logits and dH GEMMs fastest with A first (W,
// E), dW with B first (E, streamed from HBM; the small h^T mostly hits the
// L2): 1.4-2.8% per GEMM over the burst.
enum { kLoadBurst = 0, kLoadAFirst = 1, kLoadBFirst = 2 };

template <bool kATr, bool kBTr, bool kZeroAcc = true, bool kBGather = false,
          int kOrder = kLoadAFirst>
__device__ __forceinline__ void gemm_mainloop(const bf16* __restrict__ A, int64_t lda, int a_rows,
                                              int a_cols, int m0, const bf16* __restrict__ B,
                                              int64_t ldb, int b_rows, int b_cols, int n0, int64_t kt0,
                                              int nk, char* smem, Acc& acc,
                                              const int* b_gidx = nullptr, int64_t b_goff = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  if constexpr (kZeroAcc) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = floatx4{};
  }
  if (nk <= 0) return;

  Tile<kATr> ta;
  Tile<kBTr, kBGather> tb;
  ta.init(A, lda, a_rows, a_cols, m0, kt0 * kBK, lane, wave);
  tb.init(B, ldb, b_rows, b_cols, n0, kt0 * kBK, lane, wave, b_gidx, b_goff);
  auto stage_a = [&](int stage) { return smem + stage * kStageBytes; };
  auto stage_b = [&](int stage) { return smem + stage * kStageBytes + kABytes; };
  auto frag_a = [&](int stage, int ks, int i, bf16x8& f) {
    bf16x8 x[1];
    ta.template frags<1>(stage_a(stage), ks, wm * kTM * 16 + 16 * i, lane, x);
    f = x[0];
  };
  auto frags_b = [&](int stage, int ks, bf16x8(&b)[kTN]) {
    tb.template frags<kTN>(stage_b(stage), ks, wn * kTN * 16, lane, b);
  };
  auto mma = [&](const bf16x8(&a)[kTM], const bf16x8(&b)[kTN], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        if (i * kTN + j >= i0 && i * kTN + j < i1)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  constexpr int NM = kTM * kTN, NH = NM / 2;
  constexpr int RA = Tile<kATr>::kReads, RB = Tile<kBTr, kBGather>::kReads;
  static_assert(kTM == 8 && kRoundsA == 4 && kRoundsB == 4, "4 loads per operand, 2 A fragments each");
  bf16x8 fa0[kTM], fb0[kTN], fa1[kTM], fb1[kTN];
  // loads q of the operand issued after the barrier (early) or at the start
  // of the next step (late)
  auto early1 = [&](int stage, int t, int q) {
    if constexpr (kOrder == kLoadBFirst) tb.issue1(stage_b(stage), t, wave, q);
    else ta.issue1(stage_a(stage), t, wave, q);
  };
  auto late1 = [&](int stage, int t, int q) {
    if constexpr (kOrder == kLoadBFirst) ta.issue1(stage_a(stage), t, wave, q);
    else tb.issue1(stage_b(stage), t, wave, q);
  };
  constexpr int NL = kOrder == kLoadBurst ? 0 : 4;  // loads placed in the scheduling groups
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    early1(0, 0, q);
    late1(0, 0, q);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // K tile 0 landed in every wave
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    early1(1, min(1, nk - 1), q);
    if constexpr (kOrder == kLoadBurst) late1(1, min(1, nk - 1), q);
  }
#pragma unroll
  for (int i = 0; i < kTM; ++i) frag_a(0, 0, i, fa0[i]);
  frags_b(0, 0, fb0);
  // The stage barrier of step t sits after 48 of its 64 MFMAs per wave; the
  // next step's first fragments are read during the 16 after it.  The last
  // steps re-load the last K tile (unused), so the body has no branch.
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (kOrder != kLoadBurst) late1(st ^ 1, min(t + 1, nk - 1), q);
      frag_a(st, 1, 2 * q, fa1[2 * q]);
      frag_a(st, 1, 2 * q + 1, fa1[2 * q + 1]);
    }
    frags_b(st, 1, fb1);
    mma(fa0, fb0, 0, NM);
    spread_groups<NL, NL ? 2 * RA : 0, (NL ? 0 : kTM * RA) + kTN * RB, NM>();
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1, 0, NH);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K tile t+1 landed in every wave; stage st fully read
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      early1(st, min(t + 2, nk - 1), q);
      if constexpr (kOrder == kLoadBurst) late1(st, min(t + 2, nk - 1), q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      frag_a(st ^ 1, 0, 2 * q, fa0[2 * q]);
      frag_a(st ^ 1, 0, 2 * q + 1, fa0[2 * q + 1]);
    }
    frags_b(st ^ 1, 0, fb0);
    mma(fa1, fb1, NH, NM);
    spread_groups<NL, NL ? 2 * RA : 0, (NL ? 0 : kTM * RA) + kTN * RB, NM - NH>();
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Accumulator layout of v_mfma_f32_16x16x32_bf16: lane holds column
// (lane & 15) and rows 4 * (lane >> 4) + r, r = 0..3, of each 16 x 16 tile.
__device__ __forceinline__ int acc_row(int wm, int i, int lane, int r) {
  return wm * kTM * 16 + i * 16 + (lane >> 4) * 4 + r;
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * kTN * 16 + j * 16 + (lane & 15); }

// ---------------------------------------------------------------------------
// Logits GEMM and its epilogues, computed transposed: A = W (rows =
// vocabulary, M = V), B = the chunk's gathered rows of h (rows = tokens),
// so each lane holds 32 vocabulary values of each of its 4 tokens and the
// per-token reductions over the vocabulary are in-lane plus two exchanges
// among the 4 lanes that share a token.  With z = s * (a + b_j) (a the
// accumulator, b the bias or 0), per token and 128-wide vocabulary slab (one
// wave's M range), part[slab * ldp + j] for chunk row j receives:
//
//   kEpiMax  (max_v z, sum_v exp(z - max))            page 1's per-block
//            logsumexp partials (shard partials; flagged rows below)
//   kEpiRef  (S, S), S = sum_v e_v,  e_v = exp(z - r),  r = ref[i] the
//            row's target logit: the partials of the same logsumexp relative
//            to a reference known before the GEMM, so e_v / sum_v e_v is the
//            softmax and the e_v themselves can be stored (kStoreExp) as the
//            operand of both backward products.  A row where some slab's S
//            exceeds kRefSumMax (some logit about 30 nats or more above the
//            target logit) is flagged by the row combine and redone with
//            kEpiMax / kEpiLse.
//   kEpiLse  no partials; e_v = exp(z - lse_i) with ref = lse (given or
//            combined), minus tsub at the target column tcol[j] (page 1,
//            cross_entropy_kernel steps 5 and 6 without the row factor): a
//            vocabulary shard's backward, and flagged rows.
//   kEpiNone no partials (kStoreRaw only).
//
// and rpart[slab * ldp + j] = sum_v z when rpart != nullptr (label
// smoothing).  kStoreExp stores e_v, kStoreRaw the logits a + b_j (bf16)
// into E, row-major [chunk rows, ldE] (ldE = padded vocabulary, a multiple
// of 64); columns V .. ldE - 1 are written as 0.
//
// Tokens: the GEMM's token q is chunk row j = q, or j = gidx[q] when
// kIndirect (rows listed on the device; q < *gcount); chunk row j is batch
// row rows[c0 + j] (ref is indexed by batch row).  Without kIndirect the
// chunk holds min(*count - c0, cmax) tokens (cmax when count is null) and the
// grid covers cmax: tiles past the count exit at once.  With kIndirect a
// small grid strides over the tiles (usually there are none).
// ---------------------------------------------------------------------------
enum { kEpiMax = 0, kEpiRef = 1, kEpiLse = 2, kEpiNone = 3 };
enum { kStoreNone = 0, kStoreExp = 1, kStoreRaw = 2 };

struct LogitsArgs {
  const bf16* W;        // [V, H]
  const bf16* bias;     // [V] or nullptr
  const bf16* h;        // gathered chunk rows [>= tokens, H]
  int V, cmax, H;
  float s;              // logit scale
  const int* count;     // compacted row count (nullptr: cmax rows)
  int64_t c0;           // first compacted row of the chunk
  const int* rows;      // chunk row j -> batch row rows[c0 + j] (nullptr: c0 + j)
  const int* gidx;      // kIndirect: GEMM token q -> chunk row gidx[q]
  const int* gcount;    // kIndirect: number of listed rows
  floatx2* part;        // [slabs, ldp]
  float* rpart;         // [slabs, ldp] or nullptr
  int64_t ldp;
  bf16* E;              // [rows, ldE] or nullptr
  int64_t ldE;
  const float* ref;     // kEpiRef / kEpiLse: per batch row
  const int* tcol;      // kEpiLse: target column per chunk row (-1: none)
  float tsub;           // kEpiLse: subtracted at the target column
  int group_m;
};

// active: the wave's 128 vocabulary rows start below V (else it only takes
// part in the block-wide E store, with zeros).
//
// With a store, the tile goes through LDS as [token][vocabulary] (free after
// the main loop) and E is written as whole 512-byte row pieces.  A lane
// holds 4 consecutive vocabulary entries of one token per sub-tile: one
// 8-byte LDS write as soon as they are computed; 16-byte chunk ch of staged
// row t sits at ch ^ (t & 15), so the 16 tokens one write instruction touches
// fall on distinct bank groups and the 16-byte row reads are conflict-free.
// Entries past V are zero.
template <int kEpi, int kStore, bool kFull>
__device__ __forceinline__ void logits_epilogue(Acc& acc, const LogitsArgs& a, int C, int m0,
                                                int n0, int wm, int wn, int lane, bool active,
                                                const int (&jrow)[kTN], const float (&rl2)[kTN],
                                                const int (&tc)[kTN], char* smem) {
  const int V = a.V;
  const float s = a.s, sl = s * kLog2e;
  const int vbase = m0 + wm * kTM * 16;
  auto in_v = [&](int i, int r) { return kFull || m0 + acc_row(wm, i, lane, r) < V; };
  bf16* stg = reinterpret_cast<bf16*>(smem);  // [256][256]
  if constexpr (kStore != kStoreNone) {
    __syncthreads();  // every wave is done with the operand stages
    __builtin_amdgcn_sched_barrier(0);
  }
  auto put = [&](int i, int j, const floatx4& v) {
    const int tl = acc_col(wn, j, lane), vl = acc_row(wm, i, lane, 0);
    bf16x4 b;
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = (kFull || m0 + vl + r < V) ? (bf16)v[r] : (bf16)0.f;
    *(bf16x4*)&stg[tl * kBM + ((((vl >> 3) ^ (tl & 15)) << 3) | (vl & 7))] = b;
  };
  if constexpr (kEpi == kEpiMax || kEpi == kEpiRef) {
    float mx[kTN], sum[kTN], rs[kTN];
    if constexpr (kEpi == kEpiMax) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        mx[j] = -INFINITY;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (in_v(i, r)) mx[j] = fmaxf(mx[j], acc[i][j][r]);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 16, 64));
        mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 32, 64));
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const float off = mx[j] * sl;
        sum[j] = 0.f;
        rs[j] = 0.f;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (in_v(i, r)) {
              sum[j] += fast_exp2(__builtin_fmaf(acc[i][j][r], sl, -off));
              if (a.rpart != nullptr) rs[j] += acc[i][j][r];
            }
      }
    } else {  // kEpiRef: e = 2^((z - r) log2 e)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {  // row sums of z first, so each e frees its accumulator
        rs[j] = 0.f;
        if (a.rpart != nullptr) {
#pragma unroll
          for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (in_v(i, r)) rs[j] += acc[i][j][r];
        }
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        sum[j] = 0.f;
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          floatx4 e;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = fast_exp2(__builtin_fmaf(acc[i][j][r], sl, -rl2[j]));
            if (in_v(i, r)) sum[j] += e[r];
          }
          if constexpr (kStore == kStoreExp) put(i, j, e);
          if constexpr (kStore == kStoreRaw) put(i, j, acc[i][j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      sum[j] += __shfl_xor(sum[j], 16, 64);
      sum[j] += __shfl_xor(sum[j], 32, 64);
      if (a.rpart != nullptr) {
        rs[j] += __shfl_xor(rs[j], 16, 64);
        rs[j] += __shfl_xor(rs[j], 32, 64);
      }
    }
    if (active && lane < 16) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int tok = n0 + acc_col(wn, j, lane);
        if (tok < C) {
          const int64_t o = (int64_t)(vbase / 128) * a.ldp + jrow[j];
          a.part[o] = kEpi == kEpiMax ? floatx2{mx[j] * s, sum[j]} : floatx2{sum[j], sum[j]};
          if (a.rpart != nullptr) a.rpart[o] = rs[j] * s;  // sum of z over the slab
        }
      }
    }
  } else if constexpr (kEpi == kEpiLse) {  // e = exp(z - lse), the target column minus tsub
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        floatx4 e;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(__builtin_fmaf(acc[i][j][r], sl, -rl2[j]));
          if (m0 + acc_row(wm, i, lane, r) == tc[j]) e[r] -= a.tsub;
        }
        put(i, j, e);
      }
  } else {  // kEpiNone: the logits themselves
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) put(i, j, acc[i][j]);
  }
  if constexpr (kStore != kStoreNone) {
    __syncthreads();
#pragma unroll 4
    for (int p = 0; p < kBM * kBN / 8 / kGemmThreads; ++p) {
      const int u = threadIdx.x + kGemmThreads * p;
      const int tl = u / (kBM / 8), ch = u % (kBM / 8);
      const int tok = n0 + tl;
      const int64_t col = m0 + ch * 8;
      if (tok < C && col < a.ldE) {  // ldE % 64 == 0: a chunk is wholly in or out
        const int jr = a.gidx != nullptr ? a.gidx[tok] : tok;
        __builtin_nontemporal_store(*(const bf16x8*)&stg[tl * kBM + ((ch ^ (tl & 15)) << 3)],
                                    (bf16x8*)(a.E + (int64_t)jr * a.ldE + col));
      }
    }
  }
}

// One 256 x 256 logits tile (vocabulary tile tm, token tile tn) with its epilogue.
template <int kEpi, int kStore, bool kIndirect>
__device__ __forceinline__ void logits_tile(const LogitsArgs& a, int C, int tm, int tn,
                                            char* smem) {
  const int m0 = tm * kBM, n0 = tn * kBN;
  Acc acc;
  // (the gathered-row variant keeps the burst: spread, it needs 16 bytes of spill)
  gemm_mainloop<false, false, true, kIndirect, kIndirect ? kLoadBurst : kLoadAFirst>(
      a.W, a.H, a.V, 0, m0, a.h, a.H, C, 0, n0, 0, a.H / kBK, smem, acc, a.gidx, 0);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int vbase = m0 + wm * kTM * 16;
  const bool active = vbase < a.V;  // uniform over the wave
  // waves past V return, unless the E store's barriers need every wave
  if (kStore == kStoreNone && !active) return;
  const bool full = vbase + kTM * 16 <= a.V;
  if (a.bias != nullptr) {  // F.linear's bias, before the logit scale
    bf16x4 bv[kTM];  // rows row0 .. row0 + 3 of sub-tile i (row0 % 4 == 0): one 8-byte load
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int row0 = m0 + acc_row(wm, i, lane, 0);
      if (row0 + 3 < a.V) {
        bv[i] = *(const bf16x4*)(a.bias + row0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[i][r] = row0 + r < a.V ? a.bias[row0 + r] : (bf16)0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float b = (float)bv[i][r];
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j][r] += b;
      }
  }
  // the lane's 4 tokens: chunk rows, reference (log2 units) and target column
  int jrow[kTN], tc[kTN];
  float rl2[kTN];
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int q = min(n0 + acc_col(wn, j, lane), C - 1);
    jrow[j] = kIndirect ? a.gidx[q] : q;
    rl2[j] = 0.f;
    tc[j] = -1;
    if constexpr (kEpi == kEpiRef || kEpi == kEpiLse) {
      const int64_t i = a.rows != nullptr ? (int64_t)a.rows[a.c0 + jrow[j]] : a.c0 + jrow[j];
      rl2[j] = a.ref[i] * kLog2e;
    }
    if constexpr (kEpi == kEpiLse) tc[j] = a.tcol[jrow[j]];
  }
  if (full)
    logits_epilogue<kEpi, kStore, true>(acc, a, C, m0, n0, wm, wn, lane, active, jrow, rl2, tc,
                                        smem);
  else
    logits_epilogue<kEpi, kStore, false>(acc, a, C, m0, n0, wm, wn, lane, active, jrow, rl2, tc,
                                         smem);
}

template <int kEpi, int kStore, bool kIndirect>
__global__ __launch_bounds__(kGemmThreads, 1) void k_logits_bf16(const LogitsArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int C;
  if constexpr (kIndirect) {
    C = min(*a.gcount, a.cmax);
  } else {
    C = a.cmax;
    if (a.count != nullptr) {
      const int64_t n = (int64_t)*a.count - a.c0;
      C = n < 0 ? 0 : (n < a.cmax ? (int)n : a.cmax);
    }
  }
  const int tiles_v = (int)cdiv(a.V, kBM), tiles_t = (int)cdiv(C, kBN);
  if constexpr (!kIndirect) {
    const TileCoord tc = tile_coord(tiles_v, tiles_t, 1, a.group_m);
    if (!tc.active) return;
    logits_tile<kEpi, kStore, false>(a, C, tc.tm, tc.tn, smem);
  } else {
    for (int item = blockIdx.x; item < tiles_v * tiles_t; item += gridDim.x) {
      logits_tile<kEpi, kStore, true>(a, C, item % tiles_v, item / tiles_v, smem);
      __syncthreads();  // every wave is done with the LDS stages before the next tile's loads
    }
  }
}

// ---------------------------------------------------------------------------
// dH, split over K = vocabulary: out[split][m][n] (fp32, m < the rows that
// exist) = sum_v E[m, v] W[v, n] over this split's K tiles.  A = E [M = chunk
// rows, ldE] (K contiguous): the stored exp(z - r) with the target entry
// patched, so that alpha_m E[m, :] is the row's gradient g without its
// smoothing term; B = W read as K rows (vocabulary rows of W [V, H],
// transposed in LDS).  Rows of W past V read as zeros (the buffer range
// ends at row V - 1), and E is zero in those columns.
//
// M = chunk rows: the grid covers M + extra (upper bound) x max_splits; the
// rows that exist are min(*count - c0, M) (+ extra: the all-ones row after
// them, whose product is sum_v W_v for the smoothing term), and the split
// count is chosen for them (choose_splits; k_splitk_scatter recomputes it).
// With a single split and no extra row there is nothing to reduce: the
// epilogue writes alpha_m times row m, minus coef_m epsV wsum when wsum is
// given, straight to row rows[c0 + m] of dst (fp32 when dst_f32, else bf16)
// and the reduction kernel returns at once.
// ---------------------------------------------------------------------------
struct DhArgs {
  const bf16* E;  // [>= rows, ldE]
  int64_t ldE;
  int M, extra;       // chunk rows (upper bound), extra all-ones row (0 or 1)
  const int* count;   // compacted row count (nullptr: M rows)
  int64_t c0;
  const bf16* W;      // [V, H]
  int V, H, k_tiles, max_splits;
  float* out;         // split partials [split][rows + extra][H]
  int group_m;
  void* dst;          // dH [N, H], fp32 when dst_f32
  int dst_f32;
  const int* rows;    // chunk row -> batch row rows[c0 + row]
  const float *alpha, *coef, *wsum;
  float epsV;
};

// One dH work item: block bid of a grid of at least (row tiles x H tiles x
// max_splits) blocks.
__device__ __forceinline__ void dh_item(const DhArgs& a, int bid, char* smem) {
  const int H = a.H, k_tiles = a.k_tiles, extra = a.extra;
  const int64_t c0 = a.c0;
  const float* __restrict__ wsum = a.wsum;
  int Me = a.M;
  if (a.count != nullptr) {
    const int64_t n = (int64_t)*a.count - c0;
    Me = n < 0 ? 0 : (n < a.M ? (int)n : a.M);
  }
  const int Mr = Me;  // real rows
  Me += extra;
  const int splits = choose_splits(cdiv(Me, kBM) * cdiv(H, kBN), k_tiles, a.max_splits);
  const TileCoord tc = tile_coord_of(bid, (int)cdiv(Me, kBM), (int)cdiv(H, kBN), splits, a.group_m);
  if (!tc.active) return;
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  const int kt0 = (int)((int64_t)k_tiles * tc.split / splits);
  const int kt1 = (int)((int64_t)k_tiles * (tc.split + 1) / splits);
  Acc acc;
  gemm_mainloop<false, true, true, false, kLoadAFirst>(a.E, a.ldE, Me, 0, m0, a.W, H, a.V, H, n0,
                                                       kt0, kt1 - kt0, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  if (splits == 1 && extra == 0) {  // nothing to reduce: rows go straight to their place in dH
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + acc_row(wm, i, lane, r);
        if (row >= Mr) continue;
        const int64_t drow = (int64_t)a.rows[c0 + row] * H;
        const float al = a.alpha[row], ce = wsum != nullptr ? a.coef[row] * a.epsV : 0.f;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int col = n0 + acc_col(wn, j, lane);
          if (col >= H) continue;
          const float v = al * acc[i][j][r] - (wsum != nullptr ? ce * wsum[col] : 0.f);
          if (a.dst_f32) static_cast<float*>(a.dst)[drow + col] = v;
          else static_cast<bf16*>(a.dst)[drow + col] = (bf16)v;
        }
      }
    return;
  }
  float* o = a.out + (int64_t)tc.split * Me * H;  // partials [split][Me][H]
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int col = n0 + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + acc_row(wm, i, lane, r);
        if (row < Me && col < H) o[(int64_t)row * H + col] = acc[i][j][r];  // re-read from the MALL
      }
    }
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dh_bf16(const DhArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  dh_item(a, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// dW = g^T h over K = the chunk's tokens, computed as its transpose
// dW^T = (alpha h)^T E: A = (alpha h)^T [H, ldh] with the chunk's tokens
// contiguous (each token's row of h times its alpha, a 2 * H * Kp byte copy
// made per chunk), B = E [Kp token rows, ldE] read as K rows (vocabulary
// columns, transposed in LDS): alpha_t E[t, v] is g[t, v] without its
// smoothing term, which is the same for every vocabulary row,
// -(eps / V) sum_t c_t h_t = -epsV * usum, and is subtracted from the
// final value (written by the final chunk) when usum != nullptr.  In this order the
// transposed operand is the one with 4 fragments per wave rather than 8 (16
// LDS reads per 32-wide K step instead of 20: main loop 2.62 against
// 2.72 ms at the 4B-scale shape).  Tiles are still numbered over (vocabulary
// tile, H tile), so the order, and what the L2 shares, are unchanged; the
// accumulators hold the tile transposed (rows = H, columns = vocabulary),
// and the epilogue transposes it back through LDS.  h^T columns C..Kp-1 are
// zero (E rows there are finite).
// kMode 0: out (bf16) = acc                      (single chunk)
// kMode 1: acc32 = acc, or out (bf16) = acc      (first of several chunks)
// kMode 3: acc32 += acc, or out (bf16) = acc32 + acc   (a later chunk)
// A chunk is the final one when no rows follow it: last_chunk, or, with
// count != nullptr, *count - c0 <= cmax (chunks hold the compacted rows in
// order, so the chunks after the one holding the last row are empty).  The
// final chunk writes the bf16 result; an empty later chunk returns at once,
// since an earlier one was final.  acc32 keeps each tile in the
// accumulators' own register layout (tile, then sub-tile (i, j), then
// thread, 4 floats each), so a thread reads and writes its 128 values as 32
// coalesced 16-byte pieces.  Mode 3 adds them after its main loop, where the
// operand registers are free (loaded into the accumulators before it, they
// leave too few registers for the bf16 epilogue).
// ---------------------------------------------------------------------------
// The chunk's tokens: Kp = the padded count (multiple of 64), or, when
// count != nullptr, min(*count - c0, cmax) rounded up to 64.
struct DwArgs {
  const bf16* E;      // [>= Kp rows, ldE]
  int64_t ldE;
  int cmax;           // chunk rows (upper bound)
  const int* count;   // compacted row count (nullptr: cmax rows)
  int64_t c0;
  int V;
  const bf16* hT;     // (alpha h)^T [H, ldh]
  int64_t ldh;
  int H;
  bf16* out;          // dW [V, H]
  float* acc32;       // fp32 accumulator across chunks (tile layout)
  int group_m;
  const float* usum;  // sum_t coef_t h_t, or nullptr
  float epsV;
  int last_chunk;
};

// One dW tile: block bid of a grid of (vocabulary tiles x H tiles) blocks.
template <int kMode>
__device__ __forceinline__ void dw_tile(const DwArgs& a, int bid, char* smem) {
  static_assert(kMode == 0 || kMode == 1 || kMode == 3, "dW modes: 0, 1, 3");
  const int cmax = a.cmax, V = a.V, H = a.H;
  const float* __restrict__ usum = a.usum;
  const float epsV = a.epsV;
  const TileCoord tc = tile_coord_of(bid, (int)cdiv(V, kBM), (int)cdiv(H, kBN), 1, a.group_m);
  if (!tc.active) return;
  const int v0 = tc.tm * kBM, h0 = tc.tn * kBN;  // vocabulary rows and H columns of dW
  int Ce = cmax;
  bool final_chunk = kMode == 0 || a.last_chunk != 0;
  if (a.count != nullptr) {
    const int64_t n = (int64_t)*a.count - a.c0;
    Ce = n < 0 ? 0 : (n < cmax ? (int)n : cmax);
    if (n <= cmax) final_chunk = true;
    if (kMode == 3 && n <= 0) return;  // an earlier chunk held the last row and wrote dW
  }
  const int Kp = (int)round_up(Ce, kBK);
  Acc acc;  // acc[i][j][r] = dW[v0 + acc_col(wn, j)][h0 + acc_row(wm, i, r)]
  floatx4* t32 = reinterpret_cast<floatx4*>(a.acc32) +
                 ((int64_t)tc.tm * cdiv(H, kBN) + tc.tn) * (kTM * kTN * kGemmThreads) + threadIdx.x;
  gemm_mainloop<false, true, true, false, kLoadBFirst>(a.hT, a.ldh, H, 0, h0, a.E, a.ldE, max(Kp, 1),
                                                       (int)a.ldE, v0, 0, Kp / kBK, smem, acc);
  if constexpr (kMode == 3) {  // (after the main loop, where the operand registers are free)
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] += __builtin_nontemporal_load(t32 + (i * kTN + j) * kGemmThreads);
  }
  if (!final_chunk) {  // carried to the next chunk in fp32
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) __builtin_nontemporal_store(acc[i][j], t32 + (i * kTN + j) * kGemmThreads);
    return;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  {
    // Stage the bf16 tile in LDS as [vocabulary][H] (free after the main
    // loop) and write it out as 512-byte rows.  A lane holds 4 consecutive H
    // of one vocabulary row per sub-tile: one 8-byte write.  16-byte chunk
    // ch of staged row r sits at ch ^ (r & 15), so the 16 rows one write
    // instruction touches fall on distinct banks and the 16-byte row reads
    // stay conflict-free.
    bf16* stg = reinterpret_cast<bf16*>(smem);  // [256][256]
    __syncthreads();  // every wave is done reading the operand stages
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int vl = acc_col(wn, j, lane), hl = acc_row(wm, i, lane, 0);
        floatx4 corr = floatx4{};  // the smoothing term, the same for every vocabulary row
        if (usum != nullptr) corr = epsV * *(const floatx4*)(usum + h0 + hl);
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (bf16)(acc[i][j][r] - corr[r]);
        *(bf16x4*)&stg[vl * kBN + ((((hl >> 3) ^ (vl & 15)) << 3) | (hl & 7))] = w;
      }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kBM * kBN / 8 / kGemmThreads; ++p) {
      const int u = threadIdx.x + kGemmThreads * p;
      const int rl = u / (kBN / 8), ch = u % (kBN / 8);
      const int row = v0 + rl, col = h0 + ch * 8;
      if (row < V && col < H)  // H % 64 == 0: a chunk is wholly in or out
        __builtin_nontemporal_store(*(const bf16x8*)&stg[rl * kBN + ((ch ^ (rl & 15)) << 3)],
                                    (bf16x8*)(a.out + (int64_t)row * H + col));
    }
    return;
  }
}

template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dw_bf16(const DwArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  dw_tile<kMode>(a, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// dH and dW in one launch (used with several chunks, kMode 1 or 3): blocks
// [0, dh_blocks) are dH work items, the rest dW tiles.  Blocks are
// dispatched in order, so the long dH items start first and the dW tiles,
// whose fp32 accumulator read-modify-write is bound by HBM, run beside them
// and fill the CUs that dH's partly filled last wave leaves idle.
// dh_blocks is a multiple of 8, so a dW tile's block id keeps its XCD
// (block b runs on XCD b mod 8) and the dW tile order is unchanged.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dhdw_bf16(const DhArgs d, const DwArgs w,
                                                                    int dh_blocks) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  if ((int)blockIdx.x < dh_blocks) dh_item(d, blockIdx.x, smem);
  else dw_tile<kMode>(w, blockIdx.x - dh_blocks, smem);
}

}  // namespace fldce
