// Memory-bound and per-row kernels of the fused LM-head cross-entropy, plus
// the fp32 GEMM used when the inputs are float32.  All reductions run in a
// fixed order (no floating-point atomics), so results repeat bit for bit.
#pragma once

#include "fldce_common.h"

namespace fldce {

// ---------------------------------------------------------------------------
// Divisor of the "mean" reduction (model page, fused_linear_cross_entropy_-
// forward: total = number of targets != ignore_index), computed on the device
// so no host synchronisation is needed.  D = 1 for "sum"; the caller's total
// when > 0; else max(count, 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_divisor(const int64_t* __restrict__ target, int64_t N,
                                                  int64_t ignore, int reduction, int64_t total,
                                                  float* __restrict__ D) {
  __shared__ long long cnt[1024];
  long long c = 0;
  if (reduction == 1 && total <= 0)
    for (int64_t i = threadIdx.x; i < N; i += 1024) c += (target[i] != ignore);
  cnt[threadIdx.x] = c;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) cnt[threadIdx.x] += cnt[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float d = 1.f;
    if (reduction == 1) d = total > 0 ? (float)total : (float)(cnt[0] > 0 ? cnt[0] : 1);
    *D = d;
  }
}

// ---------------------------------------------------------------------------
// Row compaction.  Rows whose target is ignore_index contribute nothing (page
// 1, cross_entropy_kernel step 2 zeroes them), so the bf16 path multiplies
// only the others: rows[k] = index of the k-th row with target != ignore
// (ascending), *count = their number.  One block; each thread takes four
// consecutive rows per pass and a block-wide prefix sum gives their
// positions, so the order (and everything after it) is deterministic.
// In the same pass, when the pointers are not null: the divisor D as
// k_divisor computes it (the count is the number of non-ignored rows),
// a[i] = va, b[i] = vb, c[i] = vc on ignored rows (outputs no later kernel
// writes for them), and zeros[0 .. nzeros) = 0 (the per-chunk counters of
// flagged rows).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_prep_rows(const int64_t* __restrict__ target, int64_t N,
                                                    int64_t ignore, int* __restrict__ rows,
                                                    int* __restrict__ count, int reduction,
                                                    int64_t total, float* __restrict__ D, float* a,
                                                    float va, float* b, float vb, float* c,
                                                    float vc, int* zeros = nullptr,
                                                    int nzeros = 0) {
  __shared__ int wtot[16];
  for (int k = threadIdx.x; k < nzeros; k += 1024) zeros[k] = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = 0;
  for (int64_t s0 = 0; s0 < N; s0 += 4096) {
    const int64_t i0 = s0 + (int64_t)threadIdx.x * 4;
    bool v[4];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t i = i0 + k;
      const bool in = i < N;
      const bool ign = in && target[i] == ignore;
      v[k] = in && !ign;
      cnt += v[k] ? 1 : 0;
      if (ign) {
        if (a) a[i] = va;
        if (b) b[i] = vb;
        if (c) c[i] = vc;
      }
    }
    int x = cnt;  // inclusive prefix sum over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    int pos = base + x - cnt;
    for (int w = 0; w < wave; ++w) pos += wtot[w];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (v[k]) rows[pos++] = (int)(i0 + k);
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += wtot[w];
    base += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *count = base;
    if (D != nullptr) {
      float d = 1.f;
      if (reduction == 1) d = total > 0 ? (float)total : (float)(base > 0 ? base : 1);
      *D = d;
    }
  }
}

// Outputs of ignored rows that no later kernel writes: a[i] = va, b[i] = vb,
// c[i] = vc where target[i] == ignore (pointers may be null).
__global__ __launch_bounds__(256) void k_ignored_rows_init(const int64_t* __restrict__ target,
                                                           int64_t N, int64_t ignore, float* a,
                                                           float va, float* b, float vb, float* c,
                                                           float vc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N || target[i] != ignore) return;
  if (a) a[i] = va;
  if (b) b[i] = vb;
  if (c) c[i] = vc;
}

// Rows of dH that belong to ignored targets are exactly +0 (one block per
// row, grid-stride over the rows).
template <typename T>
__global__ __launch_bounds__(256) void k_zero_ignored_rows(const int64_t* __restrict__ target,
                                                           int64_t N, int64_t ignore,
                                                           T* __restrict__ out, int64_t H) {
  for (int64_t i = blockIdx.x; i < N; i += gridDim.x) {
    if (target[i] != ignore) continue;
    for (int64_t e = threadIdx.x; e < H; e += 256) out[i * H + e] = from_f32<T>(0.f);
  }
}

// Number of rows of a chunk: the compacted rows [c0, c0 + cmax) that exist.
__device__ __forceinline__ int64_t chunk_rows(const int* count, int64_t c0, int64_t cmax) {
  if (count == nullptr) return cmax;
  const int64_t n = (int64_t)*count - c0;
  return n < 0 ? 0 : (n < cmax ? n : cmax);
}

// ---------------------------------------------------------------------------
// dst[c, r] = src[r, c] for r < R, c < Cn; dst[c, r] = 0 for R <= r < Rp.
// 64 x 64 tiles through LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int64_t R, int64_t Cn,
                                                   int64_t lds, T* __restrict__ dst, int64_t ldd,
                                                   int64_t Rp) {
  __shared__ float tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t r = r0 + ty + 4 * k, c = c0 + tx;
    tile[ty + 4 * k][tx] = (r < R && c < Cn) ? to_f32(src[r * lds + c]) : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t c = c0 + ty + 4 * k, r = r0 + tx;
    if (c < Cn && r < Rp) dst[c * ldd + r] = from_f32<T>(tile[tx][ty + 4 * k]);
  }
}

// Column sums of each kColSlab-row slab of src [R, Cn]: colpart[slab, c]
// (fixed order).  Used for sum_j W[j, :], which gives the row sums of the
// logits.  Threads run along columns, so each row read is coalesced.
constexpr int kColSlab = 1024;
template <typename T>
__global__ __launch_bounds__(256) void k_colsum_slabs(const T* __restrict__ src, int64_t R,
                                                      int64_t Cn, float* __restrict__ colpart) {
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  if (c >= Cn) return;
  const int64_t r0 = (int64_t)blockIdx.x * kColSlab, r1 = min(R, r0 + kColSlab);
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) s += to_f32(src[r * Cn + c]);
  colpart[(int64_t)blockIdx.x * Cn + c] = s;
}

// Gathered chunk rows of h (row r of the chunk = source row rows[c0 + r],
// r < the chunk's count R; rows R .. round_up(R, 64) - 1 are zero, later
// rows up to Rp are not written: no GEMM reads them): hT [Cn, Rp] (ldd, when
// dst != nullptr, the B operand of dW) and the row-major copy hc [Rp, Cn]
// (when hc != nullptr, the B operand of the logits GEMM, so the GEMM reads
// contiguous rows instead of chasing indices in every tile's prologue).
// 64 x 64 tiles through LDS, 16-byte accesses (Cn % 8 == 0).
__global__ __launch_bounds__(256) void k_transpose_gather_bf16(const bf16* __restrict__ src,
                                                               const int* __restrict__ rows,
                                                               const int* __restrict__ count,
                                                               int64_t c0, int64_t cmax, int64_t Cn,
                                                               bf16* __restrict__ dst, int64_t ldd,
                                                               int64_t Rp, bf16* __restrict__ hc) {
  __shared__ bf16 tile[64][64 + 8];
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  const int64_t R = chunk_rows(count, c0, cmax);
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0c = (int64_t)blockIdx.y * 64;
  if (r0 >= round_up(R, 64)) return;  // rows past the padded count are never read
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lr = ty + 32 * p;
    const int64_t r = r0 + lr, c = c0c + tx * 8;
    bf16x8 v = bf16x8{};
    if (r < R && c + 8 <= Cn) v = *(const bf16x8*)(src + (int64_t)rows[c0 + r] * Cn + c);
    *(bf16x8*)&tile[lr][tx * 8] = v;
    if (hc != nullptr && r < Rp && c + 8 <= Cn) *(bf16x8*)(hc + r * Cn + c) = v;
  }
  if (dst == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lc = ty + 32 * p;
    const int64_t c = c0c + lc, r = r0 + tx * 8;
    if (c >= Cn || r + 8 > Rp) continue;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[tx * 8 + e][lc];
    *(bf16x8*)(dst + c * ldd + r) = v;
  }
}

// Column sums of each 256-row slab of a bf16 matrix src [R, Cn] (Cn % 8 ==
// 0): colpart[slab, c] in float32, rows in order.  Eight columns per thread
// (16-byte loads), 256 threads = 2048 columns per block.  Used for
// sum_v W_v, the label-smoothing term of dH, when it is not taken from an
// all-ones row of the dH GEMM.
__global__ __launch_bounds__(256) void k_colsum_slabs_bf16(const bf16* __restrict__ src, int64_t R,
                                                           int64_t Cn,
                                                           float* __restrict__ colpart) {
  const int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= Cn) return;
  const int64_t r0 = (int64_t)blockIdx.x * 256, r1 = min(R, r0 + 256);
  float acc[8] = {};
  for (int64_t r = r0; r < r1; ++r) {
    const bf16x8 v = *(const bf16x8*)(src + r * Cn + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) colpart[(int64_t)blockIdx.x * Cn + c + e] = acc[e];
}

// out[c] = sum_b part[b * ld + c] for c < Cn, b ascending, cast to T.
template <typename T>
__global__ __launch_bounds__(256) void k_colsum_finish(const float* __restrict__ part, int64_t nb,
                                                       int64_t ld, int64_t Cn, T* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= Cn) return;
  float s = 0.f;
  int64_t b = 0;
  for (; b + 8 <= nb; b += 8) {  // eight loads in flight, added in order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(b + u) * ld + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; b < nb; ++b) s += part[b * ld + c];
  out[c] = from_f32<T>(s);
}

// ---------------------------------------------------------------------------
// Per-row dot products (one wave per row):
//   zt[i] = s * (<h_i, W[y_i - v0]> + b[y_i - v0])
//                                   if y_i != ignore and v0 <= y_i < v0 + Vl, else 0
//   R[i]  = s * (<h_i, wsum> + bsum) (wsum = column sums of W, bsum = sum of
//                                   the bias: sum_j z_ij)
// The target logit is page 1's cross_entropy_kernel step 3 load of
// logits[y]; the row sum feeds the label-smoothing term.  bias and bsum may
// be null (no bias).
// ---------------------------------------------------------------------------
// One row of k_rowdot, computed by one wave.
template <typename T>
__device__ __forceinline__ void rowdot_row(const T* __restrict__ h, const T* __restrict__ W,
                                           const T* __restrict__ bias, int64_t H,
                                           const int64_t* __restrict__ target, int64_t v0,
                                           int64_t Vl, int64_t ignore, float s,
                                           const float* __restrict__ wsum,
                                           const float* __restrict__ bsum,
                                           float* __restrict__ zt, float* __restrict__ R,
                                           int64_t row, int lane) {
  const int64_t y = target[row];
  const int64_t col = y - v0;
  const bool in = (y != ignore) && col >= 0 && col < Vl;
  float a = 0.f, b = 0.f;
  if (!in && wsum == nullptr) {  // nothing to multiply on this row
    if (lane == 0) {
      if (zt != nullptr) zt[row] = 0.f;
      if (R != nullptr) R[row] = bsum != nullptr ? s * *bsum : 0.f;
    }
    return;
  }
  const T* hr = h + row * H;
  const T* wr = W + (in ? col : 0) * H;
  bool done = false;
  if constexpr (sizeof(T) == 2) {
    if (wsum == nullptr && (H & 7) == 0) {  // 16-byte loads: a wave reads 1 KB per step
      for (int64_t k = (int64_t)lane * 8; k < H; k += 512) {
        const bf16x8 xv = *(const bf16x8*)(hr + k), wv = *(const bf16x8*)(wr + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) a += (float)xv[e] * (float)wv[e];
      }
      done = true;
    }
  }
  if (!done)
    for (int64_t k = lane; k < H; k += 64) {
      const float x = to_f32(hr[k]);
      if (in) a += x * to_f32(wr[k]);
      if (wsum != nullptr) b += x * wsum[k];
    }
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane == 0) {
    if (bias != nullptr && in) a += to_f32(bias[col]);
    if (bsum != nullptr) b += *bsum;
    if (zt != nullptr) zt[row] = in ? s * a : 0.f;
    if (R != nullptr) R[row] = s * b;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rowdot(const T* __restrict__ h, const T* __restrict__ W,
                                                const T* __restrict__ bias, int64_t H,
                                                const int64_t* __restrict__ target, int64_t v0,
                                                int64_t Vl, int64_t ignore, float s,
                                                const float* __restrict__ wsum,
                                                const float* __restrict__ bsum, int64_t N,
                                                float* __restrict__ zt, float* __restrict__ R) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < N;
       row += (int64_t)gridDim.x * 4)
    rowdot_row<T>(h, W, bias, H, target, v0, Vl, ignore, s, wsum, bsum, zt, R, row, lane);
}

// ---------------------------------------------------------------------------
// fp32 path: softmax partials over stored logits z [C, ldz]:
// part[t * ldp + i] = (max, sum exp(z - max)) over columns [128 t, 128 t + 128) ∩ [0, V).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_row_partials_f32(const float* __restrict__ z, int64_t ldz,
                                                         int64_t C, int64_t V,
                                                         floatx2* __restrict__ part, int64_t ldp) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (i >= C) return;
  const int64_t j0 = t * 128, j1 = min(V, j0 + 128);
  const float* zr = z + i * ldz;
  float m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) m = fmaxf(m, zr[j]);
  float sum = 0.f;
  for (int64_t j = j0; j < j1; ++j) sum += fast_exp2((zr[j] - m) * kLog2e);
  part[t * ldp + i] = floatx2{m, sum};
}

// ---------------------------------------------------------------------------
// Combine the per-slab partials of each row in a fixed order (page 1: the
// host-side logsumexp over the per-block results of logsumexp_fwd_kernel).
// 256 threads = kRows rows x (256 / kRows) slab groups (below).
//
// R_i (the row sum of the logits) is R[i] when R != nullptr, else the sum of
// rpart over the slabs when rpart != nullptr (fixed order), else 0.
// mode 0 (max-shifted partials (m, S)): lse_i = M + log S, then the loss:
//     l_i   = w_i [(1-eps)(lse_i - zt_i) + eps(lse_i - R_i / Vg)] / p_i   (0 if ignored)
//     coef_i = w_i s / (p_i D)                                            (0 if ignored)
//   (page 1, cross_entropy_kernel step 4 and the label-smoothing combine;
//    the whole smoothed CE is divided by p_i).  w_i = eob_w on rows whose
//   target is the end-of-block token eob >= 0 (the module's forward divides
//   their p_mask by the weight), else 1.  alpha_i = coef_i.
// mode 1 (shard): writes out_m[i] = M, out_s[i] = S (sum relative to M) and,
//   when out_r != nullptr, out_r[i] = R_i.
// mode 2 (partials (S_t, S_t) relative to the reference r_i = zt_i, S_t =
//   sum over slab t of exp(z - r)): a row with some S_t > kRefSumMax is
//   appended to flag_list (flag_count counts them) and nothing else is
//   written for it; otherwise S = sum_t S_t, lse_i = r_i + log S,
//   the loss and coef_i as in mode 0, alpha_i = coef_i / S (so alpha_i e_v =
//   coef_i softmax_v) and the stored E[j, y_i - v0] (= e at the target) is
//   replaced by e - (1 - eps) S, which puts the target term of the gradient
//   into E (page 1, cross_entropy_kernel step 6).
// ---------------------------------------------------------------------------
//
// Rows: chunk row j (< the chunk's row count) is row i = rows[c0 + j] of the
// batch when rows != nullptr (compacted chunk), else i = c0 + j; with jlist
// the rows combined are the chunk rows jlist[q], q < *jcount.  Per-row inputs
// and the lse / rloss / out_* outputs use i; coef_out, alpha_out and tcol
// (when not null) use j: the chunk's coefficient, gradient scale and target
// column (target - v0, or -1 for an ignored row).
struct CombineArgs {
  const floatx2* part;
  const float* rpart;
  int64_t ldp, nT, cmax;
  const int* rows;
  const int* count;
  int64_t c0;
  const int* jlist;
  const int* jcount;
  int mode;
  const int64_t* target;
  const float* p_mask;
  int64_t ignore;
  const float* zt;
  const float* R;
  float eps, Vg, s;
  const float* D;
  int64_t eob;
  float eob_w;
  float* lse_out;
  float* rloss_out;
  float* coef_out;
  float* alpha_out;
  int* tcol;
  int64_t v0;
  bf16* E;
  int64_t ldE;
  int* flag_count;
  int* flag_list;
  float* out_m;
  float* out_s;
  float* out_r;
};

// A block combines kRows rows, each over kGroups = 256 / kRows interleaved
// slab groups (group g takes slabs g, g + kGroups, ...; the group results
// are merged in group order).  32 rows per block read 128-byte pieces of
// each slab row (best for thousands of rows); 8 rows per block give a few
// hundred rows four times the threads per row (measured: the combine of
// 884 rows 23.5 -> 15 us, of 4500 rows 30 -> 38 us).
template <int kRows>
__global__ __launch_bounds__(256) void k_combine_rows(const CombineArgs a) {
  constexpr int kCombineRows = kRows, kCombineGroups = 256 / kRows;
  __shared__ float sm[kCombineGroups][kCombineRows], ss[kCombineGroups][kCombineRows],
      sr[kCombineGroups][kCombineRows];
  const int tx = threadIdx.x % kCombineRows, grp = threadIdx.x / kCombineRows;
  const int64_t C = a.jlist != nullptr ? (int64_t)*a.jcount : chunk_rows(a.count, a.c0, a.cmax);
  const int64_t q = (int64_t)blockIdx.x * kCombineRows + tx;
  const int64_t j = q < C ? (a.jlist != nullptr ? (int64_t)a.jlist[q] : q) : 0;
  const bool ref = a.mode == 2;
  float m = -INFINITY, sum = 0.f, rsum = 0.f;
  auto merge = [&](float m2, float s2) {
    if (ref) {
      m = fmaxf(m, m2);
      sum += s2;
    } else {
      lse_merge(m, sum, m2, s2);
    }
  };
  if (q < C) {
    // slabs grp, grp + G, ... in order (G = kCombineGroups); eight loads in
    // flight per batch
    constexpr int G = kCombineGroups;
    int64_t t = grp;
    for (; t + 7 * G < a.nT; t += 8 * G) {
      floatx2 pv[8];
      float rv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pv[u] = a.part[(t + G * u) * a.ldp + j];
        rv[u] = a.rpart != nullptr ? a.rpart[(t + G * u) * a.ldp + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        merge(pv[u][0], pv[u][1]);
        rsum += rv[u];
      }
    }
    for (; t < a.nT; t += G) {
      const floatx2 pv = a.part[t * a.ldp + j];
      merge(pv[0], pv[1]);
      if (a.rpart != nullptr) rsum += a.rpart[t * a.ldp + j];
    }
  }
  sm[grp][tx] = m;
  ss[grp][tx] = sum;
  sr[grp][tx] = rsum;
  __syncthreads();
  if (grp != 0 || q >= C) return;
  for (int g = 1; g < kCombineGroups; ++g) {
    merge(sm[g][tx], ss[g][tx]);
    rsum += sr[g][tx];
  }
  const int64_t i = a.rows != nullptr ? (int64_t)a.rows[a.c0 + j] : a.c0 + j;
  if (a.mode == 1) {
    a.out_m[i] = m;
    a.out_s[i] = sum;
    if (a.out_r != nullptr) a.out_r[i] = rsum;
    return;
  }
  if (ref && !(m <= kRefSumMax)) {  // the reference is too far below the row's maximum
    a.flag_list[atomicAdd(a.flag_count, 1)] = (int)j;
    return;
  }
  const float lse = ref ? a.zt[i] + logf(sum) : m + logf(sum);
  const bool valid = a.target[i] != a.ignore;
  const float p = (a.p_mask != nullptr && valid) ? a.p_mask[i] : 1.f;
  float l = 0.f, cf = 0.f;
  if (valid) {
    const float rs = (a.R != nullptr) ? a.R[i] : rsum;
    const float wt = (a.eob >= 0 && a.target[i] == a.eob) ? a.eob_w : 1.f;
    l = wt * (((1.f - a.eps) * (lse - a.zt[i]) + a.eps * (lse - rs / a.Vg)) / p);
    cf = wt * (a.s / (p * a.D[0]));
  }
  a.lse_out[i] = valid ? lse : 0.f;
  a.rloss_out[i] = l;
  const int64_t col = valid ? a.target[i] - a.v0 : -1;
  if (a.coef_out != nullptr) a.coef_out[j] = cf;
  if (a.alpha_out != nullptr) a.alpha_out[j] = ref ? cf / sum : cf;
  if (a.tcol != nullptr) a.tcol[j] = (int)col;
  if (ref && a.E != nullptr && valid) {
    bf16* e = a.E + j * a.ldE + col;
    *e = (bf16)((float)*e - (1.f - a.eps) * sum);
  }
}

// coef_j = w_i s / (p_i D), 0 on ignored rows (shard backward, lse given;
// w_i the end-of-block weight as in k_combine_rows), for
// chunk row j -> batch row i as in k_combine_rows; with lsec / tcol also the
// chunk's lse (from the given lse) and target column.
__global__ __launch_bounds__(256) void k_coef_rows(const int64_t* __restrict__ target,
                                                   const float* __restrict__ p_mask, int64_t ignore,
                                                   int64_t cmax, const int* __restrict__ rows,
                                                   const int* __restrict__ count, int64_t c0,
                                                   float s, const float* __restrict__ D,
                                                   int64_t eob, float eob_w,
                                                   float* __restrict__ coef,
                                                   const float* __restrict__ lse_in,
                                                   float* __restrict__ lsec,
                                                   int* __restrict__ tcol, int64_t v0) {
  const int64_t C = chunk_rows(count, c0, cmax);
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= C) return;
  const int64_t i = rows != nullptr ? (int64_t)rows[c0 + j] : c0 + j;
  const bool valid = target[i] != ignore;
  const float p = (p_mask != nullptr && valid) ? p_mask[i] : 1.f;
  const float wt = (valid && eob >= 0 && target[i] == eob) ? eob_w : 1.f;
  coef[j] = valid ? wt * (s / (p * D[0])) : 0.f;
  if (lsec != nullptr) lsec[j] = lse_in[i];
  if (tcol != nullptr) tcol[j] = valid ? (int)(target[i] - v0) : -1;
}

// ---------------------------------------------------------------------------
// dlogits (page 1, cross_entropy_kernel steps 5 and 6): for token i < C and
// vocabulary column j < V of this shard,
//   g_ij = coef_i (exp(z_ij - lse_i) - eps/Vg) - coef_i (1 - eps) [j == y_i - v0]
// and exactly +0 on ignored rows (coef_i == 0), on j >= V and on i >= C.
// Overwrites z [C, ldz] with g (in place) and writes g^T [ldz rows, ldt]
// (token columns up to the grid's extent), both in T.  64 tokens x 64
// columns per block; the grid covers ldz / 64 x ldt / 64 blocks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[e + 4] = b[e];
  }
}
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]};
  *(floatx4*)(p + 4) = floatx4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (bf16)v[e];
  *(bf16x8*)p = a;
}

template <typename T>
__global__ __launch_bounds__(256) void k_gpass(T* __restrict__ z, int64_t ldz, int64_t C, int64_t V,
                                               const float* __restrict__ lse,
                                               const float* __restrict__ coef,
                                               const int64_t* __restrict__ target, int64_t v0,
                                               float eps, float Vg, T* __restrict__ gT, int64_t ldt) {
  // Requires ldz % 64 == 0 (columns j0 .. j0+63 allocated) and ldt % 64 == 0.
  __shared__ float tile[64][65];
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;  // 8 threads x 8 columns per row
  const float epsV = eps / Vg;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int li = ty + pass * 32;
    const int64_t i = i0 + li;
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = 0.f;
    if (i < C) {
      const float cf = coef[i];
      if (cf != 0.f) {
        const float l2 = lse[i] * kLog2e;
        const int64_t yc = target[i] - v0;
        const float tgt = cf * (1.f - eps);
        float zv[8];
        load8(z + i * ldz + j0 + tx * 8, zv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t j = j0 + tx * 8 + e;
          float v = cf * (fast_exp2(__builtin_fmaf(zv[e], kLog2e, -l2)) - epsV);
          if (j == yc) v -= tgt;
          g[e] = (j < V) ? v : 0.f;
        }
      }
      store8(z + i * ldz + j0 + tx * 8, g);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[li][tx * 8 + e] = g[e];
  }
  __syncthreads();
  // transpose out: thread -> vocabulary row j0 + ty (+32), 8 tokens from i0 + tx * 8
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lj = ty + pass * 32;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[tx * 8 + e][lj];
    store8(gT + (j0 + lj) * ldt + i0 + tx * 8, v);
  }
}

// fp32 path: z[i, j] += s * b[j] for i < C, j < V (the bias of F.linear,
// before the logit scale).
__global__ __launch_bounds__(256) void k_add_bias_f32(float* __restrict__ z, int64_t ldz, int64_t C,
                                                      int64_t V, const float* __restrict__ b,
                                                      float s) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= V) return;
  const float sb = s * b[j];
  for (int64_t i = blockIdx.y; i < C; i += gridDim.y) z[i * ldz + j] += sb;
}

// Upstream-gradient scaling (page 1, fused_linear_cross_entropy_backward):
// x[e] = T(float(x[e]) * do) unless do == 1.  Grid-stride over 8-element
// groups (x 16-byte aligned); the tail past a multiple of 8 element by element.
template <typename T>
__global__ __launch_bounds__(256) void k_scale_grad(const float* __restrict__ grad_out,
                                                    T* __restrict__ x, int64_t n) {
  const float d = *grad_out;
  if (d == 1.f) return;
  const int64_t n8 = n / 8;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n8; q += (int64_t)gridDim.x * 256) {
    float v[8];
    load8(x + q * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= d;
    store8(x + q * 8, v);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - n8 * 8) {
    const int64_t e = n8 * 8 + threadIdx.x;
    x[e] = from_f32<T>(to_f32(x[e]) * d);
  }
}

// dH rows of a compacted chunk: out[rows[c0 + j], :] = alpha_j P_j - coef_j
// epsV w for j < C, the chunk's row count, with P_m = sum_s part[s][m][:]
// (s ascending) and w = sum_v W_v: the product P_C of the all-ones row after
// the C rows when extra == 1, else wsum when given, else 0; S =
// choose_splits for C + extra rows, exactly as the dH GEMM chose it (nothing
// to do when it wrote the rows itself).
template <typename Tout>
__global__ __launch_bounds__(256) void k_splitk_scatter(const float* __restrict__ part,
                                                        int max_splits, int64_t k_tiles,
                                                        int64_t cmax, int extra, int64_t H,
                                                        const int* __restrict__ rows,
                                                        const int* __restrict__ count, int64_t c0,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ coef, float epsV,
                                                        const float* __restrict__ wsum,
                                                        Tout* __restrict__ out) {
  const int64_t C = chunk_rows(count, c0, cmax);
  const int64_t Me = C + extra;
  const int S = choose_splits(cdiv(Me, 256) * cdiv(H, 256), k_tiles, max_splits);
  if (S == 1 && extra == 0) return;  // one split: the GEMM wrote the rows itself
  const int64_t MN = Me * H;  // partials [split][Me][H]
  for (int64_t j = blockIdx.x; j < C; j += gridDim.x) {  // chunk rows, grid-strided
    const int64_t dst = (int64_t)rows[c0 + j] * H;
    const float al = alpha[j], ce = (extra || wsum != nullptr) ? coef[j] * epsV : 0.f;
    for (int64_t e = (int64_t)threadIdx.x * 4; e < H; e += 256 * 4) {
      const int64_t src = j * H + e;
      if (e + 4 <= H) {
        floatx4 acc = *(const floatx4*)(part + src);
        for (int s = 1; s < S; ++s) acc += *(const floatx4*)(part + (int64_t)s * MN + src);
        floatx4 ws = floatx4{};
        if (extra)
          for (int s = 0; s < S; ++s) ws += *(const floatx4*)(part + (int64_t)s * MN + C * H + e);
        else if (wsum != nullptr)
          ws = *(const floatx4*)(wsum + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) out[dst + e + k] = from_f32<Tout>(al * acc[k] - ce * ws[k]);
      } else {
        for (int64_t k = 0; e + k < H; ++k) {
          float a = part[src + k], w = 0.f;
          for (int s = 1; s < S; ++s) a += part[(int64_t)s * MN + src + k];
          if (extra)
            for (int s = 0; s < S; ++s) w += part[(int64_t)s * MN + C * H + e + k];
          else if (wsum != nullptr)
            w = wsum[e + k];
          out[dst + e + k] = from_f32<Tout>(al * a - ce * w);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The gradient rows of a chunk formed in place over the stored logits z =
// a + b (bf16, row-major [rows, ldE], ldE % 8 == 0), for chunk rows j < n:
//   E[j, v] = coef_j (exp(s z - lse_i) - eps/Vg) - coef_j (1 - eps) [v == tcol_j]
// for v < V, 0 for V <= v < ldE (page 1, cross_entropy_kernel steps 5 and 6,
// rounded once), and alpha[j] = 1.  Used when label smoothing is large:
// there the smoothing share eps/Vg is most of a flat softmax, and it has to
// be subtracted before the one rounding to bf16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gpass_rows(bf16* __restrict__ E, int64_t ldE, int64_t V,
                                                    const int* __restrict__ count, int64_t c0,
                                                    int64_t cmax, const int* __restrict__ rows,
                                                    const float* __restrict__ lse,
                                                    const float* __restrict__ coef,
                                                    const int* __restrict__ tcol, float eps,
                                                    float Vg, float s, float* __restrict__ alpha) {
  const int64_t n = chunk_rows(count, c0, cmax);
  const float epsV = eps / Vg, sl = s * kLog2e;
  for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int64_t i = rows != nullptr ? (int64_t)rows[c0 + j] : c0 + j;
    const float cf = coef[j], l2 = lse[i] * kLog2e, tg = cf * (1.f - eps);
    const int64_t tc = tcol[j];
    if (blockIdx.x == 0 && threadIdx.x == 0) alpha[j] = 1.f;
    bf16* er = E + j * ldE;
    for (int64_t v0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; v0 < ldE;
         v0 += (int64_t)gridDim.x * 256 * 8) {
      const bf16x8 z = *(const bf16x8*)(er + v0);
      bf16x8 g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = cf * (fast_exp2(__builtin_fmaf((float)z[e], sl, -l2)) - epsV);
        if (v0 + e == tc) x -= tg;
        g[e] = v0 + e < V ? (bf16)x : (bf16)0.f;
      }
      *(bf16x8*)(er + v0) = g;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows the logits GEMM does not write of the chunk's E [rows, ldE] (ldE % 8
// == 0): rows n .. round_up(n + extra, 64) - 1, n = the chunk's row count,
// are zero, except, with extra, row n = 1 in columns < V: its product with W
// in the dH GEMM is sum_v W_v, the smoothing term of every row's dH.  Only
// these rows of E past n are read (dW's K padding, dH's extra row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_e_pad_rows(bf16* __restrict__ E, int64_t ldE, int64_t V,
                                                    const int* __restrict__ count, int64_t c0,
                                                    int64_t cmax, int extra) {
  const int64_t n = chunk_rows(count, c0, cmax);
  const int64_t n_end = round_up(n + extra, 64);
  const int64_t per_row = ldE / 8, units = (n_end - n) * per_row;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * 256) {
    const int64_t row = n + u / per_row, col = (u % per_row) * 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (extra && row == n && col + e < V) ? (bf16)1.f : (bf16)0.f;
    *(bf16x8*)(E + row * ldE + col) = v;
  }
}

// ---------------------------------------------------------------------------
// The B operand of dW for a chunk: hT[c, j] = bf16(alpha_j hc[j, c]) for
// chunk rows j < n (n = the chunk's row count), 0 for n <= j < round_up(n,
// 64); hc = the chunk's gathered rows [>= round_up(n, 64), Cn].  With upart,
// block (x, y) also writes the column sums over its 64 rows of coef_j hc[j, c]
// to upart[(boff + x) * (Cn + 1) + c] and, for y == 0, sum_j coef_j to
// column Cn (fixed order; zeros past n): their sum over the row blocks is
// u = sum_t coef_t h_t, the smoothing term of dW and db.  64 x 64 tiles
// through LDS, 16-byte accesses (Cn % 8 == 0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scale_transpose_bf16(
    const bf16* __restrict__ hc, const int* __restrict__ count, int64_t c0, int64_t cmax,
    int64_t Cn, const float* __restrict__ alpha, const float* __restrict__ coef,
    bf16* __restrict__ hT, int64_t ldd, float* __restrict__ upart, int64_t boff) {
  __shared__ bf16 tile[64][64 + 8];
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  const int64_t n = chunk_rows(count, c0, cmax);
  const int64_t r0 = (int64_t)blockIdx.x * 64, cb = (int64_t)blockIdx.y * 64;
  float* up = upart != nullptr ? upart + (boff + blockIdx.x) * (Cn + 1) : nullptr;
  if (r0 >= round_up(n, 64)) {  // no row of this block exists: zero partials only
    if (up != nullptr) {
      for (int c = threadIdx.x; c < 64; c += 256) up[cb + c] = 0.f;
      if (blockIdx.y == 0 && threadIdx.x == 0) up[Cn] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lr = ty + 32 * p;
    bf16x8 v = bf16x8{};
    if (r0 + lr < n) v = *(const bf16x8*)(hc + (r0 + lr) * Cn + cb + tx * 8);
    *(bf16x8*)&tile[lr][tx * 8] = v;
  }
  __syncthreads();
  float al[8], cf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t r = r0 + tx * 8 + e;
    al[e] = r < n ? alpha[r] : 0.f;
    cf[e] = r < n ? coef[r] : 0.f;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lc = ty + 32 * p;
    bf16x8 v;
    float us = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (float)tile[tx * 8 + e][lc];
      v[e] = (bf16)(al[e] * x);
      us += cf[e] * x;
    }
    *(bf16x8*)(hT + (cb + lc) * ldd + r0 + tx * 8) = v;
    if (up != nullptr) {  // the 8 row groups of this column, added in a fixed order
      us += __shfl_xor(us, 1, 64);
      us += __shfl_xor(us, 2, 64);
      us += __shfl_xor(us, 4, 64);
      if (tx == 0) up[cb + lc] = us;
    }
  }
  if (up != nullptr && blockIdx.y == 0 && threadIdx.x == 0) {
    float cs = 0.f;
    for (int64_t r = r0; r < min(n, r0 + 64); ++r) cs += coef[r];
    up[Cn] = cs;
  }
}

// ---------------------------------------------------------------------------
// db partials of a chunk (page 1: db += c_logits.sum(0)): dbpart[y * ldE + v]
// = sum over the 64 chunk rows j of row block y (j < n) of alpha_j E[j, v],
// for every column v < ldE; zeros for blocks past the rows.  The smoothing
// term is subtracted once at the end (k_db_finish).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_db_partials(const bf16* __restrict__ E, int64_t ldE,
                                                     const int* __restrict__ count, int64_t c0,
                                                     int64_t cmax, const float* __restrict__ alpha,
                                                     float* __restrict__ dbpart) {
  const int64_t n = chunk_rows(count, c0, cmax);
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  if (v >= ldE) return;
  float acc = 0.f;
  for (int64_t r = r0; r < min(n, r0 + 64); ++r) acc += alpha[r] * (float)E[r * ldE + v];
  dbpart[(int64_t)blockIdx.y * ldE + v] = acc;
}

// db[v] = sum_b part[b * ld + v] (b ascending) - epsV * (*csum when csum is
// not null), rounded once to T.
template <typename T>
__global__ __launch_bounds__(256) void k_db_finish(const float* __restrict__ part, int64_t nb,
                                                   int64_t ld, int64_t V,
                                                   const float* __restrict__ csum, float epsV,
                                                   T* __restrict__ out) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float s = 0.f;
  for (int64_t b = 0; b < nb; ++b) s += part[b * ld + v];
  if (csum != nullptr) s -= epsV * *csum;
  out[v] = from_f32<T>(s);
}

// loss = (sum_i rloss[i]) / D, float64 partial sums, fixed tree (page 1:
// loss.sum() of the per-row losses).
__global__ __launch_bounds__(1024) void k_loss_reduce(const float* __restrict__ rloss, int64_t N,
                                                      const float* __restrict__ D,
                                                      float* __restrict__ loss) {
  __shared__ double sh[1024];
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) a += (double)rloss[i];
  sh[threadIdx.x] = a;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(sh[0] / (double)D[0]);
}

__global__ __launch_bounds__(256) void k_fill_u16(uint16_t* __restrict__ p, int64_t n, uint16_t v) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) p[e] = v;
}
__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) p[e] = v;
}

// ---------------------------------------------------------------------------
// fp32 NT GEMM (float32 inputs only): out[m, n] = alpha * sum_k A[m,k] B[n,k]
// (+ out[m, n] if accumulate).  64 x 64 tiles, 4 x 4 per thread, any sizes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_f32_nt(const float* __restrict__ A, int64_t lda,
                                                     int64_t M, const float* __restrict__ B,
                                                     int64_t ldb, int64_t N, int64_t K, float alpha,
                                                     float* __restrict__ out, int64_t ldo,
                                                     int accumulate) {
  __shared__ float As[16][64 + 4], Bs[16][64 + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = threadIdx.x + q * 256;  // 0..1023 -> row idx/16, k idx%16
      const int r = idx >> 4, kk = idx & 15;
      const int64_t ma = m0 + r, nb = n0 + r, k = k0 + kk;
      As[kk][r] = (ma < M && k < K) ? A[ma * lda + k] : 0.f;
      Bs[kk][r] = (nb < N && k < K) ? B[nb * ldb + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[kk][ty * 4 + u];
        b[u] = Bs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + ty * 4 + u, n = n0 + tx * 4 + v;
      if (m < M && n < N) {
        float r = alpha * acc[u][v];
        if (accumulate) r += out[m * ldo + n];
        out[m * ldo + n] = r;
      }
    }
}

}  // namespace fldce
