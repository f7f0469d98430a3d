// bf16 MFMA GEMM core for gfx950 and the three contractions of the fused
// LM-head cross-entropy built on it.
//
// Every GEMM here computes C[m, n] = sum_k A(m, k) B(n, k), bf16 in, fp32
// accumulate, with each operand read in its natural row-major layout: either
// K contiguous (h and W for the logits, g for dH) or K as the row index (W
// for dH, g and h for dW), the latter transposed on its way out of LDS by
// the gfx950 transpose read.  No operand is transposed in memory.
//
// Tiling (CDNA4: 64-wide waves, 160 KB LDS, v_mfma_f32_16x16x32_bf16):
//   * block tile 256 x 256, K step 64, 512 threads = 8 waves in a 2 (M) x 4
//     (N) grid, each wave owning a 128 x 64 accumulator (8 x 4 MFMA tiles of
//     16 x 16, 128 fp32 per lane), two waves per SIMD so one wave's waits are
//     covered by the other's MFMAs;
//   * two LDS stages of (256 + 256) x 64 bf16 = 64 KB each, filled with
//     direct global->LDS 16-byte loads (no VGPR staging).  The 16-byte chunk
//     c of row r sits at chunk position c ^ ((r >> 1) & 7): the LDS serves a
//     16-byte read to 16 lanes per cycle, and the 16 rows those lanes read
//     then fall on 16 distinct bank groups (measured: no bank-conflict
//     cycles);
//   * each 32-wide K step reads the next step's fragments while it issues
//     its MFMAs, one LDS read between two MFMAs (explicit scheduling groups);
//     the stage barrier sits in the middle of the last step's MFMAs and the
//     loop body has no branch, so the next tile's first reads and the global
//     loads of the tile after overlap MFMA work;
//   * blocks are renumbered so that consecutive logical tiles run on one XCD
//     (the dispatcher deals block ids round-robin over the 8 XCDs) and tiles
//     are walked in groups of `group_m` rows of tiles, so operand slabs are
//     shared in that XCD's L2.
//
// Rows past M (or N) are loaded from the last valid row (loads stay in
// bounds) and masked in the epilogues.  K must be a multiple of 64.
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

// Scheduling groups: ND (MFMA, LDS read) pairs, then the remaining MFMAs.
template <int I, int NM, int ND>
__device__ __forceinline__ void interleave_groups() {
  if constexpr (I < ND) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    interleave_groups<I + 1, NM, ND>();
  } else if constexpr (NM > ND) {
    __builtin_amdgcn_sched_group_barrier(0x008, NM - ND, 0);
  }
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
// as the K = V operand of dH, or g [C, V] and h [C, H] as the K = C operands
// of dW); its LDS tile is 64 K-rows x 256 columns (512 B rows, 32-byte
// segment s of row r at position s ^ tr_swz(r)) and a fragment is gathered
// with two ds_read_b64_tr_b16.  Within each 16-lane group that instruction
// returns, to lane i, element (i mod 4) of the 8-byte reads of lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4; when those lanes read rows k..k+3 at
// columns 4*(lane mod 4), lane i receives column i of rows k..k+3, i.e. four
// consecutive K of its own row, which is the MFMA operand layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tr_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

template <bool kTr>
struct Tile;

template <>
struct Tile<false> {
  static constexpr int kReads = 1;  // LDS reads per fragment
  const bf16* p[4];
  // rows = number of valid rows (M or N); r0 = first row of the tile.  With
  // gidx, tile row q is source row gidx[goff + q] (a gather), else goff + q.
  __device__ __forceinline__ void init(const bf16* X, int64_t ldx, int rows, int cols, int r0,
                                       int64_t k_begin, int lane, int wave,
                                       const int* gidx = nullptr, int64_t goff = 0) {
    (void)cols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * kWaves * 8 + wave * 8 + (lane >> 3);
      const int64_t q = min(r0 + r, rows - 1);
      const int64_t src = gidx != nullptr ? (int64_t)gidx[goff + q] : goff + q;
      p[i] = X + src * ldx + lds_chunk(lane & 7, r) * 8 + k_begin;
    }
  }
  __device__ __forceinline__ void issue(char* tile, int t, int wave) const {
    char* s = tile + wave * 8 * 128;
    const int64_t ko = (int64_t)t * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(FLDCE_GPTR(p[i] + ko), FLDCE_LPTR(s + i * kWaves * 8 * 128), 16, 0, 0);
  }
  // fragments for 16-row sub-tiles at rows off + 16 t
  template <int T>
  __device__ __forceinline__ void frags(const char* tile, int ks, int off, int lane, bf16x8 (&f)[T]) const {
    const char* b = tile + (off + (lane & 15)) * 128 + (lds_chunk(ks * 4 + (lane >> 4), lane & 15) << 4);
#pragma unroll
    for (int t = 0; t < T; ++t) f[t] = *(const bf16x8*)(b + t * 16 * 128);
  }
};

template <>
struct Tile<true> {
  static constexpr int kReads = 2;
  const bf16* p[4];  // column pointers (row 0 of the source)
  int64_t ldx;
  int krows, k_begin;
  // rows = number of valid K rows of the source; cols = valid columns;
  // r0 = first column of the tile; k_begin = first K row
  __device__ __forceinline__ void init(const bf16* X, int64_t ld, int rows, int cols, int c0,
                                       int64_t kb, int lane, int wave, const int* = nullptr,
                                       int64_t = 0) {
    ldx = ld;
    krows = rows;
    k_begin = (int)kb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 16 + wave * 2 + (lane >> 5);  // LDS row this lane fills
      const int pos = lane & 31;                       // 16-byte unit in the 512 B row
      const int u = (((pos >> 1) ^ tr_swz(r)) << 1) | (pos & 1);
      p[i] = X + min(c0 + u * 8, cols - 8);
    }
  }
  __device__ __forceinline__ void issue(char* tile, int t, int wave) const {
    char* s = tile + wave * 2 * 512;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(k_begin + t * kBK + i * 16 + wave * 2 + (lane >> 5), krows - 1);
      __builtin_amdgcn_global_load_lds(FLDCE_GPTR(p[i] + (int64_t)row * ldx), FLDCE_LPTR(s + i * 16 * 512), 16,
                                       0, 0);
    }
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
// [kt0, kt0 + nk).  For a normal operand X_rows/X_cols are (valid rows,
// unused); for a transposed one (valid K rows, valid columns).
template <bool kATr, bool kBTr>
__device__ __forceinline__ void gemm_mainloop(const bf16* __restrict__ A, int64_t lda, int a_rows,
                                              int a_cols, int m0, const bf16* __restrict__ B,
                                              int64_t ldb, int b_rows, int b_cols, int n0, int64_t kt0,
                                              int nk, char* smem, Acc& acc,
                                              const int* b_gidx = nullptr, int64_t b_goff = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = floatx4{};
  if (nk <= 0) return;

  Tile<kATr> ta;
  Tile<kBTr> tb;
  ta.init(A, lda, a_rows, a_cols, m0, kt0 * kBK, lane, wave);
  tb.init(B, ldb, b_rows, b_cols, n0, kt0 * kBK, lane, wave, b_gidx, b_goff);
  auto issue = [&](int stage, int t) {
    ta.issue(smem + stage * kStageBytes, t, wave);
    tb.issue(smem + stage * kStageBytes + kABytes, t, wave);
  };
  auto frags = [&](int stage, int ks, bf16x8(&a)[kTM], bf16x8(&b)[kTN]) {
    ta.template frags<kTM>(smem + stage * kStageBytes, ks, wm * kTM * 16, lane, a);
    tb.template frags<kTN>(smem + stage * kStageBytes + kABytes, ks, wn * kTN * 16, lane, b);
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
  constexpr int ND = kTM * Tile<kATr>::kReads + kTN * Tile<kBTr>::kReads;
  constexpr int ND1 = ND < NM ? ND : NM, ND2 = ND < NM - NH ? ND : NM - NH;
  bf16x8 fa0[kTM], fb0[kTN], fa1[kTM], fb1[kTN];
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // stage 0 landed in every wave
  issue(1, min(1, nk - 1));
  frags(0, 0, fa0, fb0);
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    frags(st, 1, fa1, fb1);
    mma(fa0, fb0, 0, NM);
    interleave_groups<0, NM, ND1>();
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1, 0, NH);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t+1 landed in every wave; stage st fully read
    __builtin_amdgcn_sched_barrier(0);
    // After the last tile these re-load the last tile into the idle stage and
    // read a landed stage; both results go unused (keeps the body branch-free).
    issue(st, min(t + 2, nk - 1));
    frags(st ^ 1, 0, fa0, fb0);
    mma(fa1, fb1, NH, NM);
    interleave_groups<0, NM - NH, ND2>();
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
// Logits GEMM with the softmax-partials epilogue, computed transposed:
// A = W (rows = vocabulary, M = V), B = h chunk (rows = tokens, N = C), so
// each lane holds 32 vocabulary values of each of its 4 tokens and the
// per-token reductions over the vocabulary are in-lane plus two exchanges
// among the 4 lanes that share a token.
//
// For each token and each 128-wide vocabulary slab (one wave's M range) it
// writes part[slab * ldp + token] = (max_j z, sum_j exp(z - max)) with
// z = s * (a + b_j) (b = bias, or 0 when bias == nullptr), and rpart[slab * ldp + token] = sum_j z when rpart != nullptr
// (kPart); with kStoreZ it stores the unscaled logits a + b_j (bf16; the
// dlogits pass applies s) into zbuf in the blocked layout below (ldz =
// padded vocabulary, a multiple of 64).
// ---------------------------------------------------------------------------
//
// Token rows: chunk token j (< the chunk's row count, read from `count` when
// it is not null) is row rows[c0 + j] of h when rows != nullptr (gathered
// here), else row j of h (h = the chunk's rows, already gathered).  The grid covers cmax tokens; tiles past the
// count exit at once.
// Epilogue of the logits GEMM for one wave's 128 (vocabulary) x 64 (token)
// accumulators; kFull: all 128 vocabulary rows exist (every tile but the last
// vocabulary tile), so no per-element bound checks.  In phases over the 4
// token groups j, so the 4 independent reductions overlap: maxima, the
// cross-lane exchanges, the sums of exp (and of z), the partial stores, then
// the z stores.
template <bool kStoreZ, bool kPart, bool kFull>
__device__ __forceinline__ void logits_epilogue(const Acc& acc, int V, int C, int m0, int n0,
                                                int wm, int wn, int lane, float s,
                                                floatx2* __restrict__ part,
                                                float* __restrict__ rpart, int64_t ldp,
                                                bf16* __restrict__ zbuf, int64_t ldz) {
  const int vbase = m0 + wm * kTM * 16;
  auto in_v = [&](int i, int r) { return kFull || m0 + acc_row(wm, i, lane, r) < V; };
  if (kPart) {
    const float sl = s * kLog2e;
    float mx[kTN], sum[kTN], rs[kTN];
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
            if (rpart != nullptr) rs[j] += acc[i][j][r];
          }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      sum[j] += __shfl_xor(sum[j], 16, 64);
      sum[j] += __shfl_xor(sum[j], 32, 64);
      if (rpart != nullptr) {
        rs[j] += __shfl_xor(rs[j], 16, 64);
        rs[j] += __shfl_xor(rs[j], 32, 64);
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int tok = n0 + acc_col(wn, j, lane);
        if (tok < C) {
          part[(int64_t)(vbase / 128) * ldp + tok] = floatx2{mx[j] * s, sum[j]};
          if (rpart != nullptr) rpart[(int64_t)(vbase / 128) * ldp + tok] = rs[j] * s;  // sum z
        }
      }
    }
  }
  if (kStoreZ) {
    // blocked layout: zblk(tok, v) = ((tok / 16) * (ldz / 4) + v / 4) * 64 + (tok % 16) * 4 + v % 4,
    // so one store instruction (16 tokens x 16 vocabulary) writes 512 contiguous bytes
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int tok = n0 + acc_col(wn, j, lane);
      if (tok >= C) continue;
      bf16* zt = zbuf + ((int64_t)(tok >> 4) * (ldz >> 2)) * 64 + (tok & 15) * 4;
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int row0 = m0 + acc_row(wm, i, lane, 0);
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)acc[i][j][r];
        bf16* dst = zt + (int64_t)(row0 >> 2) * 64;
        if (kFull || row0 + 3 < V) {
          __builtin_nontemporal_store(v, (bf16x4*)dst);  // read once, by dlogits
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row0 + r < V) dst[r] = v[r];
        }
      }
    }
  }
}

template <bool kStoreZ, bool kPart>
__global__ __launch_bounds__(kGemmThreads, 1) void k_logits_bf16(
    const bf16* __restrict__ W, const bf16* __restrict__ bias, const bf16* __restrict__ h, int V,
    int cmax, int H, float s, const int* __restrict__ rows, const int* __restrict__ count,
    int64_t c0, floatx2* __restrict__ part, float* __restrict__ rpart, int64_t ldp,
    bf16* __restrict__ zbuf, int64_t ldz, int group_m) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int C = cmax;
  if (count != nullptr) {
    const int64_t n = (int64_t)*count - c0;
    C = n < 0 ? 0 : (n < cmax ? (int)n : cmax);
  }
  const TileCoord tc = tile_coord((int)cdiv(V, kBM), (int)cdiv(C, kBN), 1, group_m);
  if (!tc.active) return;
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  Acc acc;
  gemm_mainloop<false, false>(W, H, V, 0, m0, h, H, C, 0, n0, 0, H / kBK, smem, acc, rows,
                              rows != nullptr ? c0 : 0);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int vbase = m0 + wm * kTM * 16;
  if (vbase >= V) return;
  const bool full = vbase + kTM * 16 <= V;
  if (bias != nullptr) {  // F.linear's bias, before the logit scale
    bf16x4 bv[kTM];  // rows row0 .. row0 + 3 of sub-tile i (row0 % 4 == 0): one 8-byte load
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int row0 = m0 + acc_row(wm, i, lane, 0);
      if (row0 + 3 < V) {
        bv[i] = *(const bf16x4*)(bias + row0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[i][r] = row0 + r < V ? bias[row0 + r] : (bf16)0.f;
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
  if (full)
    logits_epilogue<kStoreZ, kPart, true>(acc, V, C, m0, n0, wm, wn, lane, s, part, rpart, ldp, zbuf,
                                          ldz);
  else
    logits_epilogue<kStoreZ, kPart, false>(acc, V, C, m0, n0, wm, wn, lane, s, part, rpart, ldp,
                                           zbuf, ldz);
}

// ---------------------------------------------------------------------------
// dH = g W, split over K = vocabulary: out[split][m][n] (fp32, m < the rows
// that exist) for this split's K tiles.  A = g [M = C tokens, ldg] (K contiguous); B = W read as
// K rows (vocabulary rows of W [V, H], transposed in LDS).  Rows of W past
// V are clamped: g is zero in those columns.
// ---------------------------------------------------------------------------
// M = chunk tokens: the grid covers M (upper bound) x max_splits; the tokens
// that exist are min(*count - c0, M) when count != nullptr, and the split
// count is chosen for them (choose_splits; k_splitk_scatter recomputes it).
// With a single split there is nothing to reduce: the epilogue writes row m
// straight to row rows[c0 + m] of dst (fp32 when dst_f32, else bf16) and the
// reduction kernel returns at once.
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dh_bf16(
    const bf16* __restrict__ g, int64_t ldg, int M, const int* __restrict__ count, int64_t c0,
    const bf16* __restrict__ W, int V, int H, int k_tiles, int max_splits, float* __restrict__ out,
    int group_m, void* __restrict__ dst, int dst_f32, const int* __restrict__ rows) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int Me = M;
  if (count != nullptr) {
    const int64_t n = (int64_t)*count - c0;
    Me = n < 0 ? 0 : (n < M ? (int)n : M);
  }
  const int splits = choose_splits(cdiv(Me, kBM) * cdiv(H, kBN), k_tiles, max_splits);
  const TileCoord tc = tile_coord((int)cdiv(Me, kBM), (int)cdiv(H, kBN), splits, group_m);
  if (!tc.active) return;
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  const int kt0 = (int)((int64_t)k_tiles * tc.split / splits);
  const int kt1 = (int)((int64_t)k_tiles * (tc.split + 1) / splits);
  Acc acc;
  gemm_mainloop<false, true>(g, ldg, Me, 0, m0, W, H, V, H, n0, kt0, kt1 - kt0, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  if (splits == 1) {  // nothing to reduce: rows go straight to their place in dH
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + acc_row(wm, i, lane, r);
        if (row >= Me) continue;
        const int64_t drow = (int64_t)rows[c0 + row] * H;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int col = n0 + acc_col(wn, j, lane);
          if (col >= H) continue;
          if (dst_f32) static_cast<float*>(dst)[drow + col] = acc[i][j][r];
          else static_cast<bf16*>(dst)[drow + col] = (bf16)acc[i][j][r];
        }
      }
    return;
  }
  float* o = out + (int64_t)tc.split * Me * H;  // partials [split][Me][H]
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

// ---------------------------------------------------------------------------
// dW = g^T h over K = the chunk's tokens, computed as its transpose
// dW^T = h^T g: A = h^T [H, ldh] with the chunk's tokens contiguous (a
// 2 * H * Kp byte copy made per chunk), B = g [Kp token rows, ldg] read as
// K rows (vocabulary columns, transposed in LDS).  In this order the
// transposed operand is the one with 4 fragments per wave rather than 8 (16
// LDS reads per 32-wide K step instead of 20: main loop 2.62 against
// 2.72 ms at the 4B-scale shape).  Tiles are still numbered over (vocabulary
// tile, H tile), so the order, and what the L2 shares, are unchanged; the
// accumulators hold the tile transposed (rows = H, columns = vocabulary),
// and the epilogue transposes it back through LDS.  g rows and h^T columns
// C..Kp-1 are zero.
// kMode 0: out (bf16) = acc                      (single chunk)
// kMode 1: acc32 = acc                           (first of several chunks)
// kMode 2: acc32 += acc                          (middle chunk)
// kMode 3: out (bf16) = acc32 + acc              (last chunk)
// ---------------------------------------------------------------------------
// The chunk's tokens: Kp = the padded count (multiple of 64), or, when
// count != nullptr, min(*count - c0, cmax) rounded up to 64.
template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dw_bf16(
    const bf16* __restrict__ g, int64_t ldg, int cmax, const int* __restrict__ count, int64_t c0,
    int V, const bf16* __restrict__ hT, int64_t ldh, int H, bf16* __restrict__ out,
    float* __restrict__ acc32, int group_m) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const TileCoord tc = tile_coord((int)cdiv(V, kBM), (int)cdiv(H, kBN), 1, group_m);
  if (!tc.active) return;
  const int v0 = tc.tm * kBM, h0 = tc.tn * kBN;  // vocabulary rows and H columns of dW
  int Ce = cmax;
  if (count != nullptr) {
    const int64_t n = (int64_t)*count - c0;
    Ce = n < 0 ? 0 : (n < cmax ? (int)n : cmax);
  }
  const int Kp = (int)round_up(Ce, kBK);
  Acc acc;  // acc[i][j][r] = dW[v0 + acc_col(wn, j)][h0 + acc_row(wm, i, r)]
  gemm_mainloop<false, true>(hT, ldh, H, 0, h0, g, ldg, max(Kp, 1), (int)ldg, v0, 0, Kp / kBK, smem,
                             acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  if constexpr (kMode == 0) {
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
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (bf16)acc[i][j][r];
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
                                    (bf16x8*)(out + (int64_t)row * H + col));
    }
    return;
  }
  // Modes 1-3: the fp32 tile goes through LDS in two halves of 128
  // vocabulary rows (128 KB each; the waves with wn = 2 * half, 2 * half + 1
  // hold them), so the accesses to acc32 (and out) are 16-byte pieces of
  // whole 1-KB rows.  A lane writes 4 consecutive H (16 bytes) of one row;
  // 16-byte chunk ch of staged row r sits at ch ^ (r & 15).
  float* stg = reinterpret_cast<float*>(smem);  // [128][256]
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // the operand stages, or the previous half, are no longer read
    if ((wn >> 1) == half) {
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int vl = acc_col(wn, j, lane) - half * (kBM / 2), hl = acc_row(wm, i, lane, 0);
          *(floatx4*)&stg[vl * kBN + (((hl >> 2) ^ (vl & 15)) << 2)] = acc[i][j];
        }
    }
    __syncthreads();
#pragma unroll 4
    for (int p = 0; p < kBM / 2 * kBN / 4 / kGemmThreads; ++p) {
      const int u = threadIdx.x + kGemmThreads * p;
      const int rl = u / (kBN / 4), ch = u % (kBN / 4);
      const int row = v0 + half * (kBM / 2) + rl, col = h0 + ch * 4;
      if (row < V && col < H) {  // H % 64 == 0: a piece is wholly in or out
        const floatx4 v = *(const floatx4*)&stg[rl * kBN + ((ch ^ (rl & 15)) << 2)];
        floatx4* a32 = (floatx4*)(acc32 + (int64_t)row * H + col);
        if constexpr (kMode == 1) {
          *a32 = v;
        } else if constexpr (kMode == 2) {
          *a32 = *a32 + v;
        } else {
          const floatx4 t = *a32 + v;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)t[e];
          *(bf16x4*)(out + (int64_t)row * H + col) = o;
        }
      }
    }
  }
}

}  // namespace fldce
