// bf16 MFMA GEMM core for gfx950 and the three contractions of the fused
// LM-head cross-entropy built on it.
//
// Every GEMM here is "NT": C[m, n] = sum_k A[m, k] * B[n, k] with both A and
// B row-major and K contiguous, bf16 in, fp32 accumulate.  Operands whose K
// is not contiguous in the caller's layout are transposed once into the
// workspace beforehand (W^T, h^T, g^T), so one main loop serves all three.
//
// Tiling (CDNA4: 64-wide waves, 160 KB LDS, v_mfma_f32_32x32x16_bf16):
//   * block tile 256 x 256, K step 64, 256 threads = 4 waves in a 2 x 2 grid,
//     each wave owns a 128 x 128 accumulator (16 MFMA tiles of 32 x 32 =
//     256 fp32 per lane, held in AGPRs);
//   * two LDS stages of (256 + 256) x 64 bf16 = 64 KB each, filled with
//     direct global->LDS 16-byte loads (no VGPR staging); the 16-byte chunk
//     at column c of row r is stored at chunk position c ^ (r & 7) so the
//     MFMA fragment reads (8 rows x 16 B per 8 lanes) are bank-conflict free;
//   * fragments are double-buffered in registers across the four 16-wide K
//     sub-steps; the barrier for the next stage sits before the last
//     sub-step's MFMAs so the next tile's first fragment reads overlap them;
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
constexpr int kGemmThreads = 256;
constexpr int kABytes = kBM * kBK * 2;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;
constexpr int kGemmLds = 2 * kStageBytes;  // 128 KB

struct TileCoord {
  int tm, tn, split;
};

// Block id -> (tile row, tile column, split), XCD-aware and grouped.
__device__ __forceinline__ TileCoord tile_coord(int tiles_m, int tiles_n, int splits, int group_m) {
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int per = nblk / 8, rem = nblk % 8;
  const int x = bid % 8, idx = bid / 8;
  int b = (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
  const int tiles = tiles_m * tiles_n;
  TileCoord c;
  c.split = b / tiles;
  b -= c.split * tiles;
  (void)splits;
  const int width = group_m * tiles_n;
  const int g = b / width;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int w = b - g * width;
  c.tm = first_m + w % gm;
  c.tn = w / gm;
  return c;
}

// Main loop: acc[i][j] (wave sub-tile i along M, j along N) accumulates
// A[m0 .. m0+255, k] * B[n0 .. n0+255, k] over K tiles [kt0, kt0 + nk).
__device__ __forceinline__ void gemm_mainloop(const bf16* __restrict__ A, int64_t lda, int M, int m0,
                                              const bf16* __restrict__ B, int64_t ldb, int N, int n0,
                                              int64_t kt0, int nk, char* smem, floatx16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
  if (nk <= 0) return;

  // Per-thread source rows: wave w, round i fills LDS rows i*32 + w*8 .. +7,
  // lane -> row (lane >> 3), chunk position (lane & 7) holding chunk c.
  const int rr = lane >> 3;
  const int c = (lane & 7) ^ rr;
  const bf16* pA[8];
  const bf16* pB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = i * 32 + wave * 8 + rr;
    pA[i] = A + (int64_t)min(m0 + r, M - 1) * lda + c * 8 + kt0 * kBK;
    pB[i] = B + (int64_t)min(n0 + r, N - 1) * ldb + c * 8 + kt0 * kBK;
  }
  auto issue = [&](int stage, int t) {
    char* sA = smem + stage * kStageBytes + wave * 8 * 128;
    char* sB = sA + kABytes;
    const int64_t ko = (int64_t)t * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(FLDCE_GPTR(pA[i] + ko), FLDCE_LPTR(sA + i * 32 * 128), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(FLDCE_GPTR(pB[i] + ko), FLDCE_LPTR(sB + i * 32 * 128), 16, 0, 0);
  };
  auto frags = [&](int stage, int ks, bf16x8(&a)[4], bf16x8(&b)[4]) {
    const int pos = ((ks * 2 + (lane >> 5)) ^ (lane & 7)) << 4;
    const char* sA = smem + stage * kStageBytes + (wm * 128 + (lane & 31)) * 128 + pos;
    const char* sB = smem + stage * kStageBytes + kABytes + (wn * 128 + (lane & 31)) * 128 + pos;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(sA + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)(sB + j * 32 * 128);
  };
  auto mma = [&](const bf16x8(&a)[4], const bf16x8(&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };

  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // stage 0 landed in every wave
  if (nk > 1) issue(1, 1);
  frags(0, 0, fa0, fb0);
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    frags(st, 1, fa1, fb1);
    mma(fa0, fb0);
    frags(st, 2, fa0, fb0);
    mma(fa1, fb1);
    frags(st, 3, fa1, fb1);
    mma(fa0, fb0);
    if (t + 1 < nk) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // stage st^1 landed in every wave; stage st fully read
      __builtin_amdgcn_sched_barrier(0);
      if (t + 2 < nk) issue(st, t + 2);
      frags(st ^ 1, 0, fa0, fb0);
    }
    mma(fa1, fb1);
  }
}

// ---------------------------------------------------------------------------
// Logits GEMM with the softmax-partials epilogue, computed transposed:
// A = W (rows = vocabulary, M = V), B = h chunk (rows = tokens, N = C), so
// each lane holds 64 vocabulary values of 4 tokens and the per-token
// reductions over the vocabulary are in-lane plus one exchange between the
// two half-waves.
//
// For each token and each 128-wide vocabulary slab (one wave's M range) it
// writes part[slab * ldp + token] = (max_j z, sum_j exp(z - max)) with
// z = s * a (kPart); with kStoreZ it stores z (bf16) into zbuf[token, vocab].
// ---------------------------------------------------------------------------
template <bool kStoreZ, bool kPart>
__global__ __launch_bounds__(kGemmThreads, 1) void k_logits_bf16(
    const bf16* __restrict__ W, const bf16* __restrict__ h, int V, int C, int H, float s,
    floatx2* __restrict__ part, int64_t ldp, bf16* __restrict__ zbuf, int64_t ldz, int group_m) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tiles_m = (int)cdiv(V, kBM), tiles_n = (int)cdiv(C, kBN);
  const TileCoord tc = tile_coord(tiles_m, tiles_n, 1, group_m);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  floatx16 acc[4][4];
  gemm_mainloop(W, H, V, m0, h, H, C, n0, 0, H / kBK, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int vbase = m0 + wm * 128;
  if (vbase >= V) return;
  const int tbase = n0 + wn * 128;
  const bool full = vbase + 128 <= V;
  const float sl = s * kLog2e;
  const int half = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = tbase + j * 32 + (lane & 31);
    if (kPart) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = vbase + i * 32 + (r >> 2) * 8 + half + (r & 3);
        if (full || row < V) mx = fmaxf(mx, acc[i][j][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float off = mx * sl;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = vbase + i * 32 + (r >> 2) * 8 + half + (r & 3);
        if (full || row < V) sum += fast_exp2(__builtin_fmaf(acc[i][j][r], sl, -off));
      }
    sum += __shfl_xor(sum, 32, 64);
    if (lane < 32 && tok < C) part[(int64_t)(vbase / 128) * ldp + tok] = floatx2{mx * s, sum};
    }
    if (kStoreZ && tok < C) {
      bf16* zrow = zbuf + (int64_t)tok * ldz;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = vbase + i * 32 + g * 8 + half;
          bf16x4 v;
          v[0] = (bf16)(acc[i][j][g * 4 + 0] * s);
          v[1] = (bf16)(acc[i][j][g * 4 + 1] * s);
          v[2] = (bf16)(acc[i][j][g * 4 + 2] * s);
          v[3] = (bf16)(acc[i][j][g * 4 + 3] * s);
          if (full || row0 + 3 < V) {
            *(bf16x4*)(zrow + row0) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (row0 + e < V) zrow[row0 + e] = v[e];
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K GEMM with fp32 output: out[split][m][n] = sum over this split's K
// tiles.  Used for dH = g W (A = g [C, Vp], B = W^T [H, Vp]).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_splitk_bf16(
    const bf16* __restrict__ A, int64_t lda, int M, const bf16* __restrict__ B, int64_t ldb, int N,
    int k_tiles, int splits, float* __restrict__ out, int group_m) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
  const TileCoord tc = tile_coord(tiles_m, tiles_n, splits, group_m);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  const int kt0 = (int)((int64_t)k_tiles * tc.split / splits);
  const int kt1 = (int)((int64_t)k_tiles * (tc.split + 1) / splits);
  floatx16 acc[4][4];
  gemm_mainloop(A, lda, M, m0, B, ldb, N, n0, kt0, kt1 - kt0, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float* o = out + (int64_t)tc.split * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M && col < N) o[(int64_t)row * N + col] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// dW GEMM: A = g^T [V, Cp], B = h^T [H, Cp]; out rows = vocabulary.
// mode 0: out (bf16) = acc                      (single chunk)
// mode 1: acc32 = acc                           (first of several chunks)
// mode 2: acc32 += acc                          (middle chunk)
// mode 3: out (bf16) = acc32 + acc              (last chunk)
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dw_bf16(
    const bf16* __restrict__ A, int64_t lda, int M, const bf16* __restrict__ B, int64_t ldb, int N,
    int k_tiles, bf16* __restrict__ out, float* __restrict__ acc32, int group_m) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
  const TileCoord tc = tile_coord(tiles_m, tiles_n, 1, group_m);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  floatx16 acc[4][4];
  gemm_mainloop(A, lda, M, m0, B, ldb, N, n0, 0, k_tiles, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M && col < N) {
          const int64_t e = (int64_t)row * N + col;
          const float v = acc[i][j][r];
          if (kMode == 0) out[e] = (bf16)v;
          else if (kMode == 1) acc32[e] = v;
          else if (kMode == 2) acc32[e] += v;
          else out[e] = (bf16)(acc32[e] + v);
        }
      }
    }
}

}  // namespace fldce
