// libfldce: host side of the C ABI declared in include/fldce.h.
//
// Validation, workspace layout, the row-chunk loop and kernel launches on the
// caller's stream.  No allocation, no host synchronisation.
//
// One chunk of C token rows (page 1, fused_linear_cross_entropy_forward: the
// rows are processed in chunks to bound the [C, V] logits buffer), bf16:
//   1. logits GEMM; its epilogue forms the softmax partials relative to each
//      row's target logit and stores E = exp(z - target logit) (bf16)
//   2. per-row combine -> lse, per-row loss, coefficient s / (p_i D), the row
//      factor alpha = coef / sum E, and the target term put into E
//   3. dH = alpha (E W) - the smoothing term (split-K GEMM over the
//      vocabulary + ordered reduction)
//   4. dW += (alpha h)^T E - the smoothing term (fp32 across chunks, rounded
//      once by the chunk holding the last row)
// so g = alpha E - coef eps / V is never written (for label smoothing above
// 1/2 the logits are stored and one row pass forms g instead).  Before the
// loop: divisor D and the compacted list of rows whose target is not
// ignore_index (only they are multiplied; chunks are taken over that list);
// target logits by per-row dot products.  After it: the loss.  bf16 GEMMs
// read W and E in their own layouts (one via the LDS transpose read); the
// chunk's rows of h are gathered once, row-major and (times alpha)
// transposed.  The fp32 path (float32 inputs) stores z, forms g in place and
// uses plain fp32 GEMMs over transposed copies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/fldce.h"
#include "fldce_common.h"
#include "gemm_bf16.h"
#include "kernels.h"

using namespace fldce;

namespace {

enum Mode { kFwdBwd = 0, kShardPartials = 1, kShardBwd = 2, kFwd = 3 };

constexpr int64_t kZBudgetBytes = int64_t(16) << 30;  // chunk logits + g^T buffers
// bf16: largest vocabulary, and most rows per chunk (the (alpha h)^T operand
// of dW has a row of chunk length; 256 of them must span less than 4 GiB)
constexpr int64_t kMaxVocabBf16 = int64_t(1) << 23;
constexpr int64_t kMaxChunkBf16 = int64_t(1) << 22;
// Label smoothing above which the backward operand is g itself, formed from
// stored logits in one pass, rather than the exponentials E with the
// smoothing share added to the products: that share, eps / V of every entry,
// is more than half of a flat softmax past this point, and subtracting it
// after E is rounded would amplify E's rounding error by 1 / (1 - eps).
constexpr float kFusedSmoothingMax = 0.5f;
// Tile rows per group in the XCD-aware block order (measured best per GEMM at
// the 4B-scale shapes: 4 for logits, 2 for the two backward products).
constexpr int kGroupM = 4;
constexpr int kGroupMBwd = 2;

struct Plan {
  int64_t N = 0, H = 0, V = 0, C = 0, Cp = 0, Vp = 0, nT = 0, nchunks = 0;
  int64_t esz = 0;
  int splits = 1;
  size_t oD = 0, oWT = 0, oColpart = 0, oWsum = 0, oZt = 0, oR = 0, oLse = 0, oRloss = 0,
         oCoef = 0, oAlpha = 0, oPart = 0, oRpart = 0, oZ = 0, oGT = 0, oHT = 0, oDHpart = 0,
         oDW32 = 0, oRows = 0, oCount = 0, oTcol = 0, oBsum = 0, oDbpart = 0, oHC = 0,
         oFlag = 0, oFlist = 0, oUpart = 0, oU = 0, oWcolpart = 0;
  int64_t db_blocks = 0;  // row blocks of db partials (64 rows each, over all chunks)
  int64_t u_blocks = 0;   // row blocks of smoothing-term partials (64 rows each, over all chunks)
  size_t total = 0;
};

size_t take(size_t& cur, size_t bytes) {
  const size_t o = cur;
  cur += (bytes + 255) & ~size_t(255);
  return o;
}

int64_t default_chunk(int64_t N, int64_t V, int64_t esz) {
  const int64_t Vp = round_up(V, 64);
  const int64_t per_row = 2 * esz * Vp;  // bf16: E and room for g-sized data; fp32: z/g and g^T
  if (round_up(std::max<int64_t>(N, 1), 64) * per_row <= kZBudgetBytes) return std::max<int64_t>(N, 1);
  int64_t c = (kZBudgetBytes / per_row) / 256 * 256;
  return std::max<int64_t>(c, 256);
}

// Row blocks of 64 over every chunk of a plan (db and smoothing-term partials).
int64_t row_blocks(int64_t N, int64_t C) {
  int64_t nb = 0;
  for (int64_t c0 = 0; c0 < N; c0 += C) nb += cdiv(std::min(C, N - c0), 64);
  return std::max<int64_t>(nb, 1);
}

Plan make_plan(int mode, int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows) {
  Plan p;
  p.N = N;
  p.H = H;
  p.V = V;
  p.esz = dtype == FLDCE_DTYPE_BF16 ? 2 : 4;
  p.Vp = round_up(V, 64);
  p.nT = cdiv(V, 128);
  const bool bf = dtype == FLDCE_DTYPE_BF16;
  if ((mode == kShardPartials || mode == kFwd) && bf) {
    p.C = std::max<int64_t>(N, 1);  // logits never stored: one pass over all rows
  } else {
    p.C = chunk_rows > 0 ? std::min<int64_t>(chunk_rows, std::max<int64_t>(N, 1))
                         : default_chunk(N, V, p.esz);
    if (bf) p.C = std::min(p.C, kMaxChunkBf16);
  }
  // bf16: one row more than the chunk for the all-ones row of the smoothing term
  p.Cp = round_up(p.C + (bf ? 1 : 0), 64);
  p.nchunks = N > 0 ? cdiv(N, p.C) : 0;
  size_t cur = 0;
  p.oD = take(cur, 256);
  p.oCount = take(cur, 256);
  p.oFlag = take(cur, (size_t)std::max<int64_t>(p.nchunks, 1) * 4);  // flagged rows per chunk
  p.oRows = take(cur, (size_t)std::max<int64_t>(N, 1) * 4);  // compacted row indices
  p.oColpart = take(cur, (size_t)cdiv(V, kColSlab) * H * 4);
  p.oWsum = take(cur, (size_t)H * 4);
  p.oBsum = take(cur, 256);
  if (bf) {
    p.oHC = take(cur, (size_t)p.Cp * H * 2);  // gathered rows of h, the logits B operand
    p.oFlist = take(cur, (size_t)p.C * 4);    // flagged chunk rows
  }
  p.oPart = take(cur, (size_t)p.nT * p.C * 8);
  p.oRpart = take(cur, (size_t)p.nT * p.C * 4);  // per-slab row sums of z (label smoothing)
  if (mode == kShardPartials) {
    if (!bf) p.oZ = take(cur, (size_t)p.C * p.Vp * 4);
    p.total = cur;
    return p;
  }
  if (mode == kFwd) {
    p.oZt = take(cur, (size_t)N * 4);
    p.oR = take(cur, (size_t)N * 4);
    p.oLse = take(cur, (size_t)N * 4);
    p.oRloss = take(cur, (size_t)N * 4);
    if (!bf) p.oZ = take(cur, (size_t)p.C * p.Vp * 4);
    p.total = cur;
    return p;
  }
  if (!bf) p.oWT = take(cur, (size_t)H * p.Vp * p.esz);
  p.oZt = take(cur, (size_t)N * 4);
  p.oR = take(cur, (size_t)N * 4);
  p.oLse = take(cur, (size_t)N * 4);
  p.oRloss = take(cur, (size_t)N * 4);
  p.oCoef = take(cur, (size_t)p.C * 4);
  p.oAlpha = take(cur, (size_t)p.C * 4);
  p.oTcol = take(cur, (size_t)p.C * 4);
  p.oZ = take(cur, (size_t)p.Cp * p.Vp * p.esz);  // bf16: E; fp32: z, then g in place
  if (!bf) p.oGT = take(cur, (size_t)p.Vp * p.Cp * p.esz);
  p.oHT = take(cur, (size_t)H * p.Cp * p.esz);
  if (mode == kFwdBwd) {  // db partials: bf16 per 64 rows of a chunk, fp32 per kColSlab rows
    p.db_blocks = cdiv(std::max<int64_t>(N, 1), 64) + p.nchunks;
    p.oDbpart = take(cur, (size_t)p.db_blocks * p.Vp * 4);
  }
  if (bf) {
    // smoothing-term partials sum_t coef_t h_t (and sum_t coef_t) per 64 rows
    p.u_blocks = row_blocks(N, p.C);
    p.oUpart = take(cur, (size_t)p.u_blocks * (H + 1) * 4);
    p.oU = take(cur, (size_t)(H + 1) * 4);
    p.oWcolpart = take(cur, (size_t)cdiv(V, 256) * H * 4);  // 256-row slabs of sum_v W_v
    // the device picks the split count S for the rows that exist (fewer than
    // C when rows are ignored, plus the all-ones row when eps > 0) and stores
    // S x rows x H partials; reserve the largest such product over every
    // possible number of row tiles
    p.splits = 1;
    size_t part_elems = 0;
    // (choose_splits is 1 from 256 tiles on, so the loop stops there)
    const int64_t tm_max = std::min(cdiv(p.C + 1, kBM), cdiv(256, cdiv(H, kBN)) + 1);
    for (int64_t tm = 1; tm <= tm_max; ++tm) {
      const int S = choose_splits(tm * cdiv(H, kBN), p.Vp / kBK, 8);
      p.splits = std::max(p.splits, S);
      part_elems = std::max(part_elems, (size_t)S * std::min(tm * kBM, p.C + 1) * H);
    }
    p.oDHpart = take(cur, std::max<size_t>(part_elems, 1) * 4);
    // fp32 dW carried across chunks, whole 256 x 256 tiles in the accumulators' layout
    if (p.nchunks > 1)
      p.oDW32 = take(cur, (size_t)cdiv(V, kBM) * cdiv(H, kBN) * kBM * kBN * 4);
  }
  p.total = cur;
  return p;
}

// A dispatch holds fewer than 2^32 work-items per grid dimension: the
// largest 1-D GEMM grid (logits: vocabulary tiles x chunk-row tiles; dH and
// dW in one launch: row tiles x H tiles x splits, rounded up to 8, plus
// vocabulary tiles x H tiles) must fit.
bool grids_fit(const Plan& p, int dtype) {
  if (dtype != FLDCE_DTYPE_BF16) return true;
  const int64_t lim = (int64_t(1) << 32) / kGemmThreads;
  const int64_t tv = cdiv(p.V, kBM), tc = cdiv(std::max<int64_t>(p.C, 1), kBN), th = cdiv(p.H, kBN);
  const int64_t tdh = cdiv(p.C + 1, kBM);  // dH: the chunk's rows and the all-ones row
  return tv * tc < lim && round_up(tdh * th * std::max(p.splits, 1), 8) + tv * th < lim;
}

template <typename K>
void allow_gemm_lds(K kernel) {
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kGemmLds);
}

void set_gemm_attributes() {
  static std::once_flag once;
  std::call_once(once, [] {
    allow_gemm_lds(k_logits_bf16<kEpiMax, kStoreNone, false>);
    allow_gemm_lds(k_logits_bf16<kEpiMax, kStoreNone, true>);
    allow_gemm_lds(k_logits_bf16<kEpiRef, kStoreExp, false>);
    allow_gemm_lds(k_logits_bf16<kEpiRef, kStoreNone, false>);
    allow_gemm_lds(k_logits_bf16<kEpiRef, kStoreRaw, false>);
    allow_gemm_lds(k_logits_bf16<kEpiLse, kStoreExp, false>);
    allow_gemm_lds(k_logits_bf16<kEpiLse, kStoreExp, true>);
    allow_gemm_lds(k_logits_bf16<kEpiNone, kStoreRaw, false>);
    allow_gemm_lds(k_gemm_dh_bf16);
    allow_gemm_lds(k_gemm_dw_bf16<0>);
    allow_gemm_lds(k_gemm_dw_bf16<1>);
    allow_gemm_lds(k_gemm_dw_bf16<3>);
    allow_gemm_lds(k_gemm_dhdw_bf16<1>);
    allow_gemm_lds(k_gemm_dhdw_bf16<3>);
  });
}

// ---------------------------------------------------------------------------
// Device memory of fldce_fwd_noalloc, for callers that cannot allocate: a
// file-scope array each device holds from module load until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the address of each device's copy is
// looked up once per device with hipGetSymbolAddress and kept here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FLDCE_NOALLOC_SCRATCH_BYTES];

// Address of the current device's copy of `scratch` (looked up on the first
// call made on that device).
int scratch_of_current_device(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLDCE_ERR_HIP;
  static std::mutex mu;
  static std::vector<char*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return FLDCE_ERR_HIP;
    ptrs[dev] = static_cast<char*>(ptr);
  }
  *out = ptrs[dev];
  return FLDCE_OK;
}

// ---------------------------------------------------------------------------
// Stage profiling: event pairs recorded on the call's stream.
// ---------------------------------------------------------------------------
enum Stage {
  kPrep = 0, kHT, kLogits, kCombine, kDlogits, kDHGemm, kDHReduce, kDWGemm, kLoss, kFlagged, kDb,
  kBwdGemms, kNumStages
};
const char* const kStageNames[kNumStages] = {
    "prep",      "h_transpose", "logits_gemm", "row_combine",  "dlogits", "dH_gemm",
    "dH_reduce", "dW_gemm",     "loss",        "flagged_rows", "db",      "bwd_gemms"};

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> ev[kNumStages];  // start/end pairs
  size_t used[kNumStages] = {};
  hipEvent_t get(int stage) {
    auto& v = ev[stage];
    if (used[stage] == v.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      v.push_back(e);
    }
    return v[used[stage]++];
  }
};
Profiler g_prof;

// Records a start event on construction and an end event on destruction.
struct StageTimer {
  int stage;
  hipStream_t st;
  bool active;
  StageTimer(int s, hipStream_t stream) : stage(s), st(stream), active(g_prof.on) {
    if (active) {
      hipEvent_t e = g_prof.get(stage);
      if (e) (void)hipEventRecord(e, st);
      else active = false;
    }
  }
  ~StageTimer() {
    if (active) {
      hipEvent_t e = g_prof.get(stage);
      if (e) (void)hipEventRecord(e, st);
    }
  }
};

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Shape range of every entry point: N < 2^28 rows, 0 < V < 2^31, 0 < H <= 2^20.
bool sizes_in_range(int64_t N, int64_t H, int64_t V) {
  return N >= 0 && N < (int64_t(1) << 28) && H > 0 && H <= (int64_t(1) << 20) && V > 0 &&
         V < (int64_t(1) << 31);
}

int check_common(const void* h, const void* W, const int64_t* target, int64_t N, int64_t H,
                 int64_t V, int dtype, float logit_scale) {
  if (!W || (N > 0 && (!h || !target))) return FLDCE_ERR_NULL_POINTER;
  if (dtype != FLDCE_DTYPE_F32 && dtype != FLDCE_DTYPE_BF16) return FLDCE_ERR_BAD_DTYPE;
  if (!sizes_in_range(N, H, V)) return FLDCE_ERR_BAD_SHAPE;
  if (!(logit_scale > 0.f) || !std::isfinite(logit_scale)) return FLDCE_ERR_BAD_ARGUMENT;
  if (dtype == FLDCE_DTYPE_BF16 && H % kBK != 0) return FLDCE_ERR_UNSUPPORTED;
  // bf16 operand tiles are read through buffers: 256 rows of the longest row
  // (V, padded) must span less than 4 GiB
  if (dtype == FLDCE_DTYPE_BF16 && V >= kMaxVocabBf16) return FLDCE_ERR_UNSUPPORTED;
  // fp32 kernels put 4 work-items per vocabulary row on one grid dimension
  if (dtype == FLDCE_DTYPE_F32 && V >= (int64_t(1) << 30)) return FLDCE_ERR_UNSUPPORTED;
  return FLDCE_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? FLDCE_OK : FLDCE_ERR_HIP; }

inline unsigned grid1(int64_t n, int64_t per) { return (unsigned)cdiv(n, per); }
// Grid of a grid-stride kernel over n items, `per` per block.
inline unsigned grid_strided(int64_t n, int64_t per) {
  return (unsigned)std::min<int64_t>(std::max<int64_t>(cdiv(n, per), 1), 65536);
}

void launch_transpose(const float* src, int64_t R, int64_t Cn, int64_t lds, float* dst,
                      int64_t ldd, int64_t Rp, hipStream_t st) {
  dim3 g((unsigned)cdiv(Rp, 64), (unsigned)cdiv(Cn, 64));
  k_transpose<float><<<g, 256, 0, st>>>(src, R, Cn, lds, dst, ldd, Rp);
}

// wsum[c] = sum_j W[j, c] (two ordered passes; fp32 inputs).
void launch_colsum(const float* W, int64_t V, int64_t H, float* colpart, float* wsum,
                   hipStream_t st) {
  dim3 g((unsigned)cdiv(V, kColSlab), (unsigned)cdiv(H, 256));
  k_colsum_slabs<float><<<g, 256, 0, st>>>(W, V, H, colpart);
  k_colsum_finish<float><<<grid1(H, 256), 256, 0, st>>>(colpart, cdiv(V, kColSlab), H, H, wsum);
}

// Everything of the gradient path that fwd_bwd and shard_bwd share.
struct Core {
  const void* h;
  const void* W;
  const void* bias;      // [V] or nullptr
  const int64_t* target;
  const float* p_mask;
  int64_t N, H, V, v0, Vg;
  int dtype;
  int64_t ignore;
  float eps, s;
  const float* lse_in;   // shard: given global lse; nullptr: computed (fwd_bwd)
  float* lse_out;        // fwd_bwd: per-row lse  [N]
  float* rloss_out;      // fwd_bwd: per-row loss [N]
  const float* zt;       // fwd_bwd: target logits [N]
  const float* R;        // fwd_bwd fp32: row sums of z [N] or nullptr
  float* rpart;          // fwd_bwd bf16: per-slab row sums from the logits epilogue, or nullptr
  const float* D;
  const int* rows;       // bf16: compacted row indices (target != ignore), device
  const int* count;      // bf16: their number, device
  void* dH;              // [N, H]: h dtype (fwd_bwd) or fp32 (shard)
  bool dH_f32;
  void* dW;              // [V, H] W dtype
  void* db;              // [V] W dtype or nullptr (fwd_bwd)
  float* dbpart;         // db partials [db_blocks, Vp] when db != nullptr
  int64_t eob;           // end-of-block token (< 0: none) and its weight
  float eob_w;
};

// Row-combine arguments of a chunk common to every mode (mode 0, no chunk outputs).
// The row combine over up to `rows` rows (the block shape by that bound;
// the rows that exist are counted on the device).
void launch_combine(int64_t rows, hipStream_t st, const CombineArgs& a) {
  if (rows >= 4096)
    k_combine_rows<32><<<grid1(rows, 32), 256, 0, st>>>(a);
  else
    k_combine_rows<8><<<grid1(rows, 8), 256, 0, st>>>(a);
}

CombineArgs combine_args(const Core& c, const Plan& p, const floatx2* part, int64_t c0,
                         int64_t cmax) {
  CombineArgs a{};
  a.part = part;
  a.rpart = c.rpart;
  a.ldp = p.C;
  a.nT = p.nT;
  a.cmax = cmax;
  a.rows = c.rows;
  a.count = c.count;
  a.c0 = c0;
  a.mode = 0;
  a.target = c.target;
  a.p_mask = c.p_mask;
  a.ignore = c.ignore;
  a.zt = c.zt;
  a.R = c.R;
  a.eps = c.eps;
  a.Vg = (float)c.Vg;
  a.s = c.s;
  a.D = c.D;
  a.eob = c.eob;
  a.eob_w = c.eob_w;
  a.lse_out = c.lse_out;
  a.rloss_out = c.rloss_out;
  a.v0 = c.v0;
  return a;
}

// Row-combine arguments of a vocabulary shard's partials (mode 1).
CombineArgs shard_combine_args(const floatx2* part, const float* rpart, const Plan& p,
                               int64_t cmax, const int* rows, const int* count, int64_t c0,
                               float* out_m, float* out_s, float* out_r) {
  CombineArgs a{};
  a.part = part;
  a.rpart = rpart;
  a.ldp = p.C;
  a.nT = p.nT;
  a.cmax = cmax;
  a.rows = rows;
  a.count = count;
  a.c0 = c0;
  a.mode = 1;
  a.out_m = out_m;
  a.out_s = out_s;
  a.out_r = out_r;
  return a;
}

// Grid of the logits kernels that run over a device-side list of rows: one
// wave of blocks striding over the tiles (usually the list is empty).
unsigned indirect_grid(int64_t V, int64_t cmax) {
  return (unsigned)std::min<int64_t>(std::max<int64_t>(cdiv(V, kBM) * cdiv(cmax, kBN), 1), 256);
}

// Rows the combine flagged (a logit more than 30 nats above the target
// logit, past the clamp of the reference-relative exponentials): their
// max-shifted partials (logits GEMM over the listed rows), their lse, loss
// and coefficients (row combine over the list) and, when E is wanted, their
// rows of E relative to the lse with the target term.  Launched every time;
// with no flagged row each kernel returns at once.
void run_flagged_rows(const Core& c, const Plan& p, const LogitsArgs& la, const CombineArgs& ca,
                      int* flist, int* nflag, bf16* E, int* tcol, int64_t cmax, hipStream_t st) {
  StageTimer tm(kFlagged, st);
  const unsigned g = indirect_grid(c.V, cmax);
  LogitsArgs f = la;
  f.gidx = flist;
  f.gcount = nflag;
  f.rpart = nullptr;  // the row sums of the main pass stand
  f.E = nullptr;
  k_logits_bf16<kEpiMax, kStoreNone, true><<<g, kGemmThreads, kGemmLds, st>>>(f);
  CombineArgs cb = ca;
  cb.mode = 0;
  cb.jlist = flist;
  cb.jcount = nflag;
  cb.E = nullptr;
  cb.flag_count = nullptr;
  cb.flag_list = nullptr;
  launch_combine(cmax, st, cb);
  if (E == nullptr) return;
  LogitsArgs e = f;
  e.part = nullptr;
  e.ref = c.lse_out;
  e.tcol = tcol;
  e.tsub = 1.f - c.eps;
  e.E = E;
  k_logits_bf16<kEpiLse, kStoreExp, true><<<g, kGemmThreads, kGemmLds, st>>>(e);
}

// per-row stage of a chunk on the fp32 path: lse/loss/coefficients
// (fwd_bwd) or coefficients only (shard backward, lse given).  Returns the
// lse pointer the fp32 dlogits reads.
const float* run_rows_f32(const Core& c, const Plan& p, const floatx2* part, float* coef,
                          int64_t c0, int64_t cmax, hipStream_t st) {
  StageTimer tm(kCombine, st);
  if (c.lse_in == nullptr) {
    CombineArgs a = combine_args(c, p, part, c0, cmax);
    a.coef_out = coef;
    launch_combine(cmax, st, a);
    return c.lse_out + c0;
  }
  k_coef_rows<<<grid1(cmax, 256), 256, 0, st>>>(c.target, c.p_mask, c.ignore, cmax, nullptr,
                                                 nullptr, c0, c.s, c.D, c.eob, c.eob_w, coef,
                                                 c.lse_in, nullptr, nullptr, c.v0);
  return c.lse_in + c0;
}

// bf16: only rows with target != ignore_index are multiplied (compacted on
// the device; kernels read the count, so there is no host synchronisation).
// Per chunk: the chunk's rows of h gathered once; the logits GEMM stores
// E = exp(z - r) relative to each row's target logit r (or to the given lse
// of a vocabulary shard) with the partials of the logsumexp; the row combine
// finishes lse, loss, coef and alpha = coef / sum_v E and puts the target
// term into E; dH = alpha (E W) and dW = (alpha h)^T E read E in place (W
// too, through the LDS transpose), with the label-smoothing term added from
// sum_v W_v (an all-ones row of E) and u = sum_t coef_t h_t.
int run_core_bf16(const Core& c, const Plan& p, char* ws, hipStream_t st) {
  bf16* E = reinterpret_cast<bf16*>(ws + p.oZ);
  bf16* hT = reinterpret_cast<bf16*>(ws + p.oHT);
  bf16* hc = reinterpret_cast<bf16*>(ws + p.oHC);
  float* coef = reinterpret_cast<float*>(ws + p.oCoef);
  int* tcol = reinterpret_cast<int*>(ws + p.oTcol);
  floatx2* part = reinterpret_cast<floatx2*>(ws + p.oPart);
  float* dHpart = reinterpret_cast<float*>(ws + p.oDHpart);
  float* dW32 = reinterpret_cast<float*>(ws + p.oDW32);
  int* nflag = reinterpret_cast<int*>(ws + p.oFlag);
  int* flist = reinterpret_cast<int*>(ws + p.oFlist);
  float* upart = reinterpret_cast<float*>(ws + p.oUpart);
  float* u = reinterpret_cast<float*>(ws + p.oU);
  const bf16* h = static_cast<const bf16*>(c.h);
  const bf16* W = static_cast<const bf16*>(c.W);
  const bf16* bias = static_cast<const bf16*>(c.bias);
  const int64_t H = c.H, V = c.V, Vp = p.Vp;
  const bool given_lse = c.lse_in != nullptr;  // a vocabulary shard's backward
  const bool want_g = c.dH != nullptr || c.dW != nullptr || c.db != nullptr;
  const bool smooth = c.eps > 0.f;
  // Large label smoothing: the logits are stored and one row pass forms g
  // (the smoothing share subtracted before rounding, alpha = 1); otherwise E
  // holds the exponentials and the share is added to the products exactly.
  const bool exact = c.eps > kFusedSmoothingMax;
  // alpha (the row factor of E): coef / sum_v E, or coef itself when E is
  // relative to the lse
  float* alpha = (given_lse && !exact) ? coef : reinterpret_cast<float*>(ws + p.oAlpha);
  const bool fused_smooth = smooth && !exact;
  // sum_v W_v for the smoothing term of dH: from an all-ones row of E with
  // one chunk (free unless the row count is a multiple of 256), else from a
  // column sum of W once per call (an extra row would add a token tile to
  // every full chunk)
  const int extra = (c.dH != nullptr && fused_smooth && p.nchunks == 1) ? 1 : 0;
  float* wsum = nullptr;
  if (c.dH != nullptr && fused_smooth && p.nchunks > 1) {
    StageTimer tm(kPrep, st);
    wsum = reinterpret_cast<float*>(ws + p.oWsum);
    float* colpart = reinterpret_cast<float*>(ws + p.oWcolpart);
    dim3 g((unsigned)cdiv(V, 256), (unsigned)cdiv(H, 2048));
    k_colsum_slabs_bf16<<<g, 256, 0, st>>>(W, V, H, colpart);
    k_colsum_finish<float><<<grid1(H, 256), 256, 0, st>>>(colpart, cdiv(V, 256), H, H, wsum);
  }
  const bool need_u = fused_smooth && (c.dW != nullptr || c.db != nullptr);
  const float epsV = c.eps / (float)c.Vg;
  int64_t db_off = 0, u_off = 0;  // row blocks of db / smoothing-term partials written so far
  if (c.dH != nullptr) {
    StageTimer tm(kPrep, st);
    if (c.dH_f32)
      k_zero_ignored_rows<float><<<grid_strided(c.N, 1), 256, 0, st>>>(c.target, c.N, c.ignore,
                                                               (float*)c.dH, H);
    else
      k_zero_ignored_rows<bf16><<<grid_strided(c.N, 1), 256, 0, st>>>(c.target, c.N, c.ignore,
                                                              (bf16*)c.dH, H);
  }
  for (int64_t ic = 0; ic < p.nchunks; ++ic) {
    const int64_t c0 = ic * p.C;
    const int64_t cmax = std::min(p.C, c.N - c0);  // rows of the chunk if none were ignored
    const int64_t Cpc = round_up(cmax, 64);
    const bool last = ic + 1 == p.nchunks;
    {
      StageTimer tm(kHT, st);
      dim3 g((unsigned)(Cpc / 64), (unsigned)cdiv(H, 64));
      k_transpose_gather_bf16<<<g, 256, 0, st>>>(h, c.rows, c.count, c0, cmax, H, nullptr, 0,
                                                 Cpc, hc);
      if (want_g)
        k_e_pad_rows<<<grid_strided(64 * Vp / 8, 256), 256, 0, st>>>(E, Vp, V, c.count, c0, cmax,
                                                                     extra);
    }
    if (given_lse) {  // coefficients and target columns come first: the epilogue needs them
      StageTimer tm(kCombine, st);
      k_coef_rows<<<grid1(cmax, 256), 256, 0, st>>>(c.target, c.p_mask, c.ignore, cmax, c.rows,
                                                     c.count, c0, c.s, c.D, c.eob, c.eob_w, coef,
                                                     c.lse_in, nullptr, tcol, c.v0);
    }
    LogitsArgs la{};
    la.W = W;
    la.bias = bias;
    la.h = hc;
    la.V = (int)V;
    la.cmax = (int)cmax;
    la.H = (int)H;
    la.s = c.s;
    la.count = c.count;
    la.c0 = c0;
    la.rows = c.rows;
    la.part = part;
    la.rpart = c.rpart;
    la.ldp = p.C;
    la.E = want_g ? E : nullptr;
    la.ldE = Vp;
    la.ref = given_lse ? c.lse_in : c.zt;
    la.tcol = tcol;
    la.tsub = 1.f - c.eps;
    la.group_m = kGroupM;
    {  // 1. logits, E and the logsumexp partials
      StageTimer tm(kLogits, st);
      const int blocks = (int)(cdiv(V, kBM) * cdiv(cmax, kBN));
      if (given_lse && exact)
        k_logits_bf16<kEpiNone, kStoreRaw, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
      else if (given_lse)
        k_logits_bf16<kEpiLse, kStoreExp, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
      else if (want_g && exact)
        k_logits_bf16<kEpiRef, kStoreRaw, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
      else if (want_g)
        k_logits_bf16<kEpiRef, kStoreExp, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
      else  // loss only: E is not stored
        k_logits_bf16<kEpiRef, kStoreNone, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
    }
    if (!given_lse) {  // 2. per-row combine (lse, loss, coef, alpha, target term), flagged rows
      CombineArgs ca = combine_args(c, p, part, c0, cmax);
      ca.mode = 2;
      ca.coef_out = coef;
      ca.alpha_out = alpha;
      ca.tcol = tcol;
      ca.E = exact ? nullptr : la.E;
      ca.ldE = Vp;
      ca.flag_count = nflag + ic;
      ca.flag_list = flist;
      {
        StageTimer tm(kCombine, st);
        launch_combine(cmax, st, ca);
      }
      run_flagged_rows(c, p, la, ca, flist, nflag + ic, exact ? nullptr : la.E, tcol, cmax, st);
    }
    if (!want_g) continue;  // no gradient wanted: the loss needs nothing more
    if (exact) {  // g over the stored logits, rounded once (alpha = 1)
      StageTimer tm(kDlogits, st);
      dim3 g((unsigned)std::min<int64_t>(cdiv(Vp, 2048), 64), (unsigned)std::min<int64_t>(cmax, 4096));
      k_gpass_rows<<<g, 256, 0, st>>>(E, Vp, V, c.count, c0, cmax, c.rows,
                                      given_lse ? c.lse_in : c.lse_out, coef, tcol, c.eps,
                                      (float)c.Vg, c.s, alpha);
    }
    {  // (alpha h)^T for dW, smoothing-term partials
      StageTimer tm(kHT, st);
      dim3 g((unsigned)(Cpc / 64), (unsigned)cdiv(H, 64));
      k_scale_transpose_bf16<<<g, 256, 0, st>>>(hc, c.count, c0, cmax, H, alpha, coef, hT, p.Cp,
                                                need_u ? upart : nullptr, u_off);
      u_off += Cpc / 64;
      // u = sum_t coef_t h_t and sum_t coef_t over the rows so far: after the
      // chunk holding the last row it is final (later blocks add +0), as the
      // dW GEMM of that chunk needs it
      if (need_u && (last || c.count != nullptr))
        k_colsum_finish<float><<<grid1(H + 1, 256), 256, 0, st>>>(upart, u_off, H + 1, H + 1, u);
    }
    // 3. dH (split over the vocabulary, ordered reduction, scattered rows) and
    // 4. dW += (alpha h)^T E (the smoothing term with the final value; with
    // several chunks the final one, found on the device, writes the bf16
    // result).  With several chunks both go in one launch when both are
    // wanted: dW's accumulator traffic then runs beside dH's MFMA work
    // (1024-row chunks at the headline: step 11.35 -> 11.04 ms).  In one
    // chunk, where both are MFMA-bound, separate launches measured as fast
    // or faster (the CUs a partly filled last wave leaves idle are partly
    // paid back by a higher clock under the power limit).
    const int S = p.splits;
    DhArgs da{};
    DwArgs wa{};
    int dh_blocks = 0, dw_blocks = 0;
    if (c.dH != nullptr) {
      da.E = E; da.ldE = Vp; da.M = (int)cmax; da.extra = extra; da.count = c.count; da.c0 = c0;
      da.W = W; da.V = (int)V; da.H = (int)H; da.k_tiles = (int)(Vp / kBK); da.max_splits = S;
      da.out = dHpart; da.group_m = kGroupMBwd; da.dst = c.dH; da.dst_f32 = c.dH_f32 ? 1 : 0;
      da.rows = c.rows; da.alpha = alpha; da.coef = coef; da.wsum = wsum; da.epsV = epsV;
      dh_blocks = (int)(cdiv(cmax + extra, kBM) * cdiv(H, kBN) * S);
    }
    const int dw_mode = p.nchunks == 1 ? 0 : (ic == 0 ? 1 : 3);
    if (c.dW != nullptr) {
      wa.E = E; wa.ldE = Vp; wa.cmax = (int)cmax; wa.count = c.count; wa.c0 = c0; wa.V = (int)V;
      wa.hT = hT; wa.ldh = p.Cp; wa.H = (int)H; wa.out = (bf16*)c.dW; wa.acc32 = dW32;
      wa.group_m = kGroupMBwd; wa.usum = fused_smooth ? u : nullptr; wa.epsV = epsV;
      wa.last_chunk = last ? 1 : 0;
      dw_blocks = (int)(cdiv(V, kBM) * cdiv(H, kBN));
    }
    if (c.dH != nullptr && c.dW != nullptr && p.nchunks > 1) {
      StageTimer tm(kBwdGemms, st);
      const int dhb = (int)round_up(dh_blocks, 8);  // keeps every dW block on its XCD
      auto kern = dw_mode == 1 ? k_gemm_dhdw_bf16<1> : k_gemm_dhdw_bf16<3>;
      kern<<<dhb + dw_blocks, kGemmThreads, kGemmLds, st>>>(da, wa, dhb);
    } else {
      if (c.dH != nullptr) {
        StageTimer tm(kDHGemm, st);
        k_gemm_dh_bf16<<<dh_blocks, kGemmThreads, kGemmLds, st>>>(da);
      }
      if (c.dW != nullptr) {
        StageTimer tm(kDWGemm, st);
        auto kern = dw_mode == 0 ? k_gemm_dw_bf16<0>
                                 : (dw_mode == 1 ? k_gemm_dw_bf16<1> : k_gemm_dw_bf16<3>);
        kern<<<dw_blocks, kGemmThreads, kGemmLds, st>>>(wa);
      }
    }
    if (c.dH != nullptr && (S > 1 || extra)) {
      // (the scatter returns at once when the GEMM wrote the rows itself)
      StageTimer tm(kDHReduce, st);
      const unsigned g = (unsigned)std::min<int64_t>(cmax, 2048);
      if (c.dH_f32)
        k_splitk_scatter<float><<<g, 256, 0, st>>>(dHpart, S, Vp / kBK, cmax, extra, H, c.rows,
                                                   c.count, c0, alpha, coef, epsV, wsum,
                                                   (float*)c.dH);
      else
        k_splitk_scatter<bf16><<<g, 256, 0, st>>>(dHpart, S, Vp / kBK, cmax, extra, H, c.rows,
                                                  c.count, c0, alpha, coef, epsV, wsum,
                                                  (bf16*)c.dH);
    }
    if (c.db != nullptr) {  // 5. db partials: sum_t alpha_t E[t, :] per 64 rows
      StageTimer tm(kDb, st);
      dim3 g((unsigned)cdiv(Vp, 256), (unsigned)(Cpc / 64));
      k_db_partials<<<g, 256, 0, st>>>(E, Vp, c.count, c0, cmax, alpha, c.dbpart + db_off * Vp);
      db_off += Cpc / 64;
    }
  }
  if (c.db != nullptr) {
    StageTimer tm(kDb, st);
    k_db_finish<bf16><<<grid1(V, 256), 256, 0, st>>>(c.dbpart, db_off, Vp, V,
                                                     fused_smooth ? u + H : nullptr, epsV,
                                                     (bf16*)c.db);
  }
  return launch_status();
}

// fp32 inputs: plain fp32 GEMMs over transposed copies.
int run_core_f32(const Core& c, const Plan& p, char* ws, hipStream_t st) {
  float* WT = reinterpret_cast<float*>(ws + p.oWT);
  float* zb = reinterpret_cast<float*>(ws + p.oZ);  // z, then g in place
  float* gT = reinterpret_cast<float*>(ws + p.oGT);
  float* hT = reinterpret_cast<float*>(ws + p.oHT);
  float* coef = reinterpret_cast<float*>(ws + p.oCoef);
  floatx2* part = reinterpret_cast<floatx2*>(ws + p.oPart);
  const float* h = static_cast<const float*>(c.h);
  const float* W = static_cast<const float*>(c.W);
  const int64_t H = c.H, V = c.V, Vp = p.Vp;
  int64_t db_off = 0;  // slabs of db partials written so far
  const bool want_g = c.dH != nullptr || c.dW != nullptr || c.db != nullptr;
  if (c.dH != nullptr) {  // W^T for dH
    StageTimer tm(kPrep, st);
    launch_transpose(W, V, H, H, WT, Vp, Vp, st);
  }
  for (int64_t ic = 0; ic < p.nchunks; ++ic) {
    const int64_t c0 = ic * p.C;
    const int64_t Cc = std::min(p.C, c.N - c0);
    const int64_t Cpc = round_up(Cc, 64);
    const float* hc = h + c0 * H;
    if (c.dW != nullptr) {  // h^T for dW
      StageTimer tm(kHT, st);
      launch_transpose(hc, Cc, H, H, hT, p.Cp, Cpc, st);
    }
    {
      StageTimer tm(kLogits, st);
      dim3 g((unsigned)cdiv(V, 64), (unsigned)cdiv(Cc, 64));
      k_gemm_f32_nt<<<g, 256, 0, st>>>(hc, H, Cc, W, H, V, H, c.s, zb, Vp, 0);
      if (c.bias != nullptr)
        k_add_bias_f32<<<dim3((unsigned)cdiv(V, 256), (unsigned)std::min<int64_t>(Cc, 256)), 256, 0,
                         st>>>(zb, Vp, Cc, V, (const float*)c.bias, c.s);
      if (c.lse_in == nullptr) {
        dim3 g2((unsigned)cdiv(Cc, 64), (unsigned)p.nT);
        k_row_partials_f32<<<g2, 64, 0, st>>>(zb, Vp, Cc, V, part, p.C);
      }
    }
    const float* lse_c = run_rows_f32(c, p, part, coef, c0, Cc, st);
    if (!want_g) continue;  // no gradient wanted: the loss needs nothing more
    {
      StageTimer tm(kDlogits, st);
      dim3 g((unsigned)(Vp / 64), (unsigned)(Cpc / 64));
      k_gpass<float><<<g, 256, 0, st>>>(zb, Vp, Cc, V, lse_c, coef, c.target + c0, c.v0, c.eps,
                                        (float)c.Vg, gT, p.Cp);
      if (c.db != nullptr) {  // column sums of g (now in zb), per kColSlab rows
        dim3 g2((unsigned)cdiv(Cc, kColSlab), (unsigned)cdiv(Vp, 256));
        k_colsum_slabs<float><<<g2, 256, 0, st>>>(zb, Cc, Vp, c.dbpart + db_off * Vp);
        db_off += cdiv(Cc, kColSlab);
      }
    }
    if (c.dH != nullptr) {
      StageTimer tm(kDHGemm, st);
      dim3 g((unsigned)cdiv(H, 64), (unsigned)cdiv(Cc, 64));
      k_gemm_f32_nt<<<g, 256, 0, st>>>(zb, Vp, Cc, WT, Vp, H, V, 1.f, (float*)c.dH + c0 * H, H, 0);
    }
    if (c.dW != nullptr) {
      StageTimer tm(kDWGemm, st);
      dim3 g((unsigned)cdiv(H, 64), (unsigned)cdiv(V, 64));
      k_gemm_f32_nt<<<g, 256, 0, st>>>(gT, p.Cp, V, hT, p.Cp, H, Cpc, 1.f, (float*)c.dW, H,
                                       ic == 0 ? 0 : 1);
    }
  }
  if (c.db != nullptr) {
    StageTimer tm(kDWGemm, st);
    k_colsum_finish<float><<<grid1(V, 256), 256, 0, st>>>(c.dbpart, db_off, Vp, V, (float*)c.db);
  }
  return launch_status();
}

int run_core(const Core& c, const Plan& p, char* ws, hipStream_t st) {
  return c.dtype == FLDCE_DTYPE_BF16 ? run_core_bf16(c, p, ws, st) : run_core_f32(c, p, ws, st);
}

void zero_fill(void* p, int64_t n_elems, int esz, hipStream_t st) {
  if (n_elems <= 0) return;
  const unsigned g = (unsigned)std::min<int64_t>(cdiv(n_elems, 256), 65536);
  if (esz == 2)
    k_fill_u16<<<g, 256, 0, st>>>(static_cast<uint16_t*>(p), n_elems, 0);
  else
    k_fill_f32<<<g, 256, 0, st>>>(static_cast<float*>(p), n_elems, 0.f);
}

// Shared argument checks of the loss entry points.
int check_loss_args(int reduction, float label_smoothing, int64_t eob, float eob_w) {
  if (reduction != FLDCE_REDUCTION_SUM && reduction != FLDCE_REDUCTION_MEAN)
    return FLDCE_ERR_BAD_ARGUMENT;
  if (!(label_smoothing >= 0.f && label_smoothing <= 1.f)) return FLDCE_ERR_BAD_ARGUMENT;
  if (eob >= 0 && !(eob_w >= 0.f && std::isfinite(eob_w))) return FLDCE_ERR_BAD_ARGUMENT;
  return FLDCE_OK;
}

// Target logits and row sums of z for every row (prep of fwd_bwd and fwd):
// bf16 takes the row sums from the logits epilogue (rpart), fp32 from
// <h_i, sum_j W_j> (+ sum_j b_j).
void launch_row_dots(const void* h, const void* W, const void* bias, const int64_t* target,
                     int64_t N, int64_t H, int64_t V, bool bf, int64_t ignore, float s, bool smooth,
                     float* colpart, float* wsum, float* bsum, float* zt, float* R, hipStream_t st) {
  if (bf) {
    k_rowdot<bf16><<<grid_strided(N, 4), 256, 0, st>>>((const bf16*)h, (const bf16*)W, (const bf16*)bias,
                                                 H, target, 0, V, ignore, s, nullptr, nullptr, N,
                                                 zt, nullptr);
    return;
  }
  if (smooth) {
    launch_colsum((const float*)W, V, H, colpart, wsum, st);
    if (bias != nullptr) launch_colsum((const float*)bias, V, 1, colpart, bsum, st);
  }
  k_rowdot<float><<<grid_strided(N, 4), 256, 0, st>>>(
      (const float*)h, (const float*)W, (const float*)bias, H, target, 0, V, ignore, s,
      smooth ? wsum : nullptr, (smooth && bias != nullptr) ? bsum : nullptr, N, zt,
      smooth ? R : nullptr);
}

// Argument checks of the forward-only entry points (everything but the workspace).
int check_fwd_args(const void* h, const void* W, const void* bias, const int64_t* target,
                   const float* p_mask, int64_t N, int64_t H, int64_t V, int dtype,
                   float label_smoothing, float logit_scale, int reduction, int64_t eob_token_id,
                   float eob_weight, const float* loss) {
  int rc = check_common(h, W, target, N, H, V, dtype, logit_scale);
  if (rc != FLDCE_OK) return rc;
  if (!loss) return FLDCE_ERR_NULL_POINTER;
  rc = check_loss_args(reduction, label_smoothing, eob_token_id, eob_weight);
  if (rc != FLDCE_OK) return rc;
  if (!aligned16(h) || !aligned16(W) || !aligned16(bias) || !aligned16(target) ||
      !aligned16(p_mask))
    return FLDCE_ERR_ALIGNMENT;
  return FLDCE_OK;
}

// The forward-only path on a checked call: ws holds at least p.total bytes.
int run_fwd(const Plan& p, const void* h, const void* W, const void* bias, const int64_t* target,
            const float* p_mask, int64_t N, int64_t H, int64_t V, int dtype,
            int64_t ignore_index, float label_smoothing, float logit_scale, int reduction,
            int64_t total, int64_t eob_token_id, float eob_weight, float* loss, float* row_lse,
            float* row_loss, char* ws, hipStream_t st) {
  set_gemm_attributes();
  if (N == 0) {
    zero_fill(loss, 1, 4, st);
    return launch_status();
  }
  float* D = reinterpret_cast<float*>(ws + p.oD);
  const bool smooth = label_smoothing > 0.f;
  const bool bf = dtype == FLDCE_DTYPE_BF16;
  float* colpart = reinterpret_cast<float*>(ws + p.oColpart);
  float* wsum = reinterpret_cast<float*>(ws + p.oWsum);
  float* bsum = reinterpret_cast<float*>(ws + p.oBsum);
  float* zt = reinterpret_cast<float*>(ws + p.oZt);
  float* R = reinterpret_cast<float*>(ws + p.oR);
  float* lse = row_lse ? row_lse : reinterpret_cast<float*>(ws + p.oLse);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + p.oRloss);
  floatx2* part = reinterpret_cast<floatx2*>(ws + p.oPart);
  float* rpart = reinterpret_cast<float*>(ws + p.oRpart);
  int* rows = reinterpret_cast<int*>(ws + p.oRows);
  int* count = reinterpret_cast<int*>(ws + p.oCount);
  int* nflag = reinterpret_cast<int*>(ws + p.oFlag);
  {
    StageTimer tm(kPrep, st);
    if (bf)
      k_prep_rows<<<1, 1024, 0, st>>>(target, N, ignore_index, rows, count, reduction, total, D,
                                      lse, 0.f, rl, 0.f, nullptr, 0.f, nflag, 1);
    else
      k_divisor<<<1, 1024, 0, st>>>(target, N, ignore_index, reduction, total, D);
    launch_row_dots(h, W, bias, target, N, H, V, bf, ignore_index, logit_scale, smooth, colpart,
                    wsum, bsum, zt, R, st);
  }
  Core c{h, W, bias, target, p_mask, N, H, V, 0, V, dtype, ignore_index, label_smoothing,
         logit_scale, nullptr, lse, rl, zt, (smooth && !bf) ? R : nullptr,
         (smooth && bf) ? rpart : nullptr, D, bf ? rows : nullptr, bf ? count : nullptr, nullptr,
         false, nullptr, nullptr, nullptr, eob_token_id, eob_weight};
  if (bf) {  // logits never stored: partials from the GEMM epilogue, valid rows only
    bf16* hc = reinterpret_cast<bf16*>(ws + p.oHC);
    int* flist = reinterpret_cast<int*>(ws + p.oFlist);
    {
      StageTimer tm(kHT, st);
      dim3 g((unsigned)(p.Cp / 64), (unsigned)cdiv(H, 64));
      k_transpose_gather_bf16<<<g, 256, 0, st>>>((const bf16*)h, rows, count, 0, N, H, nullptr, 0,
                                                 p.Cp, hc);
    }
    LogitsArgs la{};
    la.W = (const bf16*)W;
    la.bias = (const bf16*)bias;
    la.h = hc;
    la.V = (int)V;
    la.cmax = (int)N;
    la.H = (int)H;
    la.s = logit_scale;
    la.count = count;
    la.rows = rows;
    la.part = part;
    la.rpart = c.rpart;
    la.ldp = p.C;
    la.ref = zt;
    la.group_m = kGroupM;
    {  // the same partials as the training path, so the loss is bit for bit the same
      StageTimer tm(kLogits, st);
      const int blocks = (int)(cdiv(V, kBM) * cdiv(N, kBN));
      k_logits_bf16<kEpiRef, kStoreNone, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
    }
    CombineArgs ca = combine_args(c, p, part, 0, N);
    ca.mode = 2;
    ca.flag_count = nflag;
    ca.flag_list = flist;
    {
      StageTimer tm(kCombine, st);
      launch_combine(N, st, ca);
    }
    run_flagged_rows(c, p, la, ca, flist, nflag, nullptr, nullptr, N, st);
  } else {  // fp32: z per chunk, row partials, combine
    float* zb = reinterpret_cast<float*>(ws + p.oZ);
    for (int64_t c0 = 0; c0 < N; c0 += p.C) {
      const int64_t Cc = std::min(p.C, N - c0);
      {
        StageTimer tm(kLogits, st);
        dim3 g((unsigned)cdiv(V, 64), (unsigned)cdiv(Cc, 64));
        k_gemm_f32_nt<<<g, 256, 0, st>>>((const float*)h + c0 * H, H, Cc, (const float*)W, H, V,
                                         H, logit_scale, zb, p.Vp, 0);
        if (bias != nullptr)
          k_add_bias_f32<<<dim3((unsigned)cdiv(V, 256), (unsigned)std::min<int64_t>(Cc, 256)), 256,
                           0, st>>>(zb, p.Vp, Cc, V, (const float*)bias, logit_scale);
        dim3 g2((unsigned)cdiv(Cc, 64), (unsigned)p.nT);
        k_row_partials_f32<<<g2, 64, 0, st>>>(zb, p.Vp, Cc, V, part, p.C);
      }
      StageTimer tm(kCombine, st);
      launch_combine(Cc, st, combine_args(c, p, part, c0, Cc));
    }
  }
  {
    StageTimer tm(kLoss, st);
    k_loss_reduce<<<1, 1024, 0, st>>>(rl, N, D, loss);
  }
  return launch_status();
}

}  // namespace

extern "C" {

int fldce_version(void) { return FLDCE_VERSION; }

const char* fldce_status_string(int status) {
  switch (status) {
    case FLDCE_OK: return "ok";
    case FLDCE_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FLDCE_ERR_BAD_SHAPE: return "N, H, V out of range or shard outside the vocabulary";
    case FLDCE_ERR_BAD_DTYPE: return "dtype must be FLDCE_DTYPE_F32 or FLDCE_DTYPE_BF16";
    case FLDCE_ERR_BAD_ARGUMENT: return "reduction, label_smoothing or logit_scale out of range";
    case FLDCE_ERR_WORKSPACE: return "workspace missing or smaller than the size query returns";
    case FLDCE_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case FLDCE_ERR_HIP: return "a HIP kernel launch failed";
    case FLDCE_ERR_UNSUPPORTED:
      return "shape not supported by the bf16 path (H must be a multiple of 64, V below 2^23; "
             "each GEMM grid must hold fewer than 2^32 work-items)";
    case FLDCE_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more than the FLDCE_NOALLOC_SCRATCH_BYTES of the allocation-free "
             "entry point (use fldce_fwd with a workspace)";
    default: return "unknown status";
  }
}

int64_t fldce_default_chunk_rows(int64_t N, int64_t H, int64_t V) {
  (void)H;
  if (N < 0 || V <= 0) return 0;
  return std::min(default_chunk(N, V, 2), kMaxChunkBf16);
}

size_t fldce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows) {
  if (!sizes_in_range(N, H, V) || (dtype != 0 && dtype != 1)) return 0;
  return make_plan(kFwdBwd, N, H, V, dtype, chunk_rows).total;
}

size_t fldce_shard_partials_workspace_size(int64_t N, int64_t H, int64_t V_local, int dtype) {
  if (!sizes_in_range(N, H, V_local) || (dtype != 0 && dtype != 1)) return 0;
  return make_plan(kShardPartials, N, H, V_local, dtype, 0).total;
}

size_t fldce_shard_bwd_workspace_size(int64_t N, int64_t H, int64_t V_local, int dtype,
                                      int64_t chunk_rows) {
  if (!sizes_in_range(N, H, V_local) || (dtype != 0 && dtype != 1)) return 0;
  return make_plan(kShardBwd, N, H, V_local, dtype, chunk_rows).total;
}

int fldce_fwd_bwd(const void* h, const void* W, const int64_t* target, const float* p_mask,
                  int64_t N, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                  float label_smoothing, float logit_scale, int reduction, int64_t total,
                  float* loss, void* dH, void* dW, float* row_lse, float* row_loss,
                  int64_t chunk_rows, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dW || (N > 0 && !dH)) return FLDCE_ERR_NULL_POINTER;  // both gradients are outputs here
  return fldce_fwd_bwd_ex(h, W, nullptr, target, p_mask, N, H, V, dtype, ignore_index,
                          label_smoothing, logit_scale, reduction, total, -1, 1.f, loss, dH, dW,
                          nullptr, row_lse, row_loss, chunk_rows, workspace, workspace_bytes,
                          stream);
}

int fldce_fwd_bwd_ex(const void* h, const void* W, const void* bias, const int64_t* target,
                     const float* p_mask, int64_t N, int64_t H, int64_t V, int dtype,
                     int64_t ignore_index, float label_smoothing, float logit_scale,
                     int reduction, int64_t total, int64_t eob_token_id, float eob_weight,
                     float* loss, void* dH, void* dW, void* db, float* row_lse, float* row_loss,
                     int64_t chunk_rows, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(h, W, target, N, H, V, dtype, logit_scale);
  if (rc != FLDCE_OK) return rc;
  if (!loss) return FLDCE_ERR_NULL_POINTER;  // dH, dW, db: NULL = not wanted
  rc = check_loss_args(reduction, label_smoothing, eob_token_id, eob_weight);
  if (rc != FLDCE_OK) return rc;
  if (chunk_rows < 0) return FLDCE_ERR_BAD_ARGUMENT;
  if (!aligned16(h) || !aligned16(W) || !aligned16(bias) || !aligned16(target) ||
      !aligned16(p_mask) || !aligned16(dH) || !aligned16(dW) || !aligned16(db) ||
      !aligned16(workspace))
    return FLDCE_ERR_ALIGNMENT;
  const Plan p = make_plan(kFwdBwd, N, H, V, dtype, chunk_rows);
  if (!grids_fit(p, dtype)) return FLDCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total) return FLDCE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_gemm_attributes();
  char* ws = static_cast<char*>(workspace);
  float* D = reinterpret_cast<float*>(ws + p.oD);
  const int esz = dtype == FLDCE_DTYPE_BF16 ? 2 : 4;
  if (N == 0) {
    zero_fill(loss, 1, 4, st);
    if (dW != nullptr) zero_fill(dW, V * H, esz, st);
    if (db != nullptr) zero_fill(db, V, esz, st);
    return launch_status();
  }
  const bool smooth = label_smoothing > 0.f;
  float* colpart = reinterpret_cast<float*>(ws + p.oColpart);
  float* wsum = reinterpret_cast<float*>(ws + p.oWsum);
  float* bsum = reinterpret_cast<float*>(ws + p.oBsum);
  float* zt = reinterpret_cast<float*>(ws + p.oZt);
  float* R = reinterpret_cast<float*>(ws + p.oR);
  float* lse = row_lse ? row_lse : reinterpret_cast<float*>(ws + p.oLse);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + p.oRloss);
  const bool bf = dtype == FLDCE_DTYPE_BF16;
  float* rpart = reinterpret_cast<float*>(ws + p.oRpart);
  // row sums of z: bf16 from the logits epilogue, fp32 from <h_i, sum_j W_j>
  int* rows = reinterpret_cast<int*>(ws + p.oRows);
  int* count = reinterpret_cast<int*>(ws + p.oCount);
  float* dbpart = reinterpret_cast<float*>(ws + p.oDbpart);
  Core c{h, W, bias, target, p_mask, N, H, V, 0, V, dtype, ignore_index, label_smoothing,
         logit_scale, nullptr, lse, rl, zt, (smooth && !bf) ? R : nullptr,
         (smooth && bf) ? rpart : nullptr, D, bf ? rows : nullptr, bf ? count : nullptr, dH,
         false, dW, db, dbpart, eob_token_id, eob_weight};
  {
    StageTimer tm(kPrep, st);
    if (bf)
      k_prep_rows<<<1, 1024, 0, st>>>(target, N, ignore_index, rows, count, reduction, total, D,
                                      lse, 0.f, rl, 0.f, nullptr, 0.f,
                                      reinterpret_cast<int*>(ws + p.oFlag), (int)p.nchunks);
    else
      k_divisor<<<1, 1024, 0, st>>>(target, N, ignore_index, reduction, total, D);
    launch_row_dots(h, W, bias, target, N, H, V, bf, ignore_index, logit_scale, smooth, colpart,
                    wsum, bsum, zt, R, st);
  }
  rc = run_core(c, p, ws, st);
  if (rc != FLDCE_OK) return rc;
  {
    StageTimer tm(kLoss, st);
    k_loss_reduce<<<1, 1024, 0, st>>>(rl, N, D, loss);
  }
  return launch_status();
}

size_t fldce_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype) {
  if (!sizes_in_range(N, H, V) || (dtype != 0 && dtype != 1)) return 0;
  return make_plan(kFwd, N, H, V, dtype, 0).total;
}

int fldce_fwd(const void* h, const void* W, const void* bias, const int64_t* target,
              const float* p_mask, int64_t N, int64_t H, int64_t V, int dtype,
              int64_t ignore_index, float label_smoothing, float logit_scale, int reduction,
              int64_t total, int64_t eob_token_id, float eob_weight, float* loss, float* row_lse,
              float* row_loss, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_fwd_args(h, W, bias, target, p_mask, N, H, V, dtype, label_smoothing,
                          logit_scale, reduction, eob_token_id, eob_weight, loss);
  if (rc != FLDCE_OK) return rc;
  if (!aligned16(workspace)) return FLDCE_ERR_ALIGNMENT;
  const Plan p = make_plan(kFwd, N, H, V, dtype, 0);
  if (!grids_fit(p, dtype)) return FLDCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total) return FLDCE_ERR_WORKSPACE;
  return run_fwd(p, h, W, bias, target, p_mask, N, H, V, dtype, ignore_index, label_smoothing,
                 logit_scale, reduction, total, eob_token_id, eob_weight, loss, row_lse, row_loss,
                 static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

int fldce_fwd_noalloc(const void* h, const void* W, const void* bias, const int64_t* target,
                      const float* p_mask, int64_t N, int64_t H, int64_t V, int dtype,
                      int64_t ignore_index, float label_smoothing, float logit_scale,
                      int reduction, int64_t total, int64_t eob_token_id, float eob_weight,
                      float* loss, float* row_lse, float* row_loss, void* stream) {
  int rc = check_fwd_args(h, W, bias, target, p_mask, N, H, V, dtype, label_smoothing,
                          logit_scale, reduction, eob_token_id, eob_weight, loss);
  if (rc != FLDCE_OK) return rc;
  const Plan p = make_plan(kFwd, N, H, V, dtype, 0);
  if (!grids_fit(p, dtype)) return FLDCE_ERR_UNSUPPORTED;
  if (p.total > FLDCE_NOALLOC_SCRATCH_BYTES) return FLDCE_ERR_SCRATCH_TOO_SMALL;
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != FLDCE_OK) return rc;
  return run_fwd(p, h, W, bias, target, p_mask, N, H, V, dtype, ignore_index, label_smoothing,
                 logit_scale, reduction, total, eob_token_id, eob_weight, loss, row_lse, row_loss,
                 ws, static_cast<hipStream_t>(stream));
}

int fldce_scale_grads(const float* grad_out, int dtype, void* dH, int64_t n_dH, void* dW,
                      int64_t n_dW, void* db, int64_t n_db, void* stream) {
  if (!grad_out) return FLDCE_ERR_NULL_POINTER;
  if (dtype != FLDCE_DTYPE_F32 && dtype != FLDCE_DTYPE_BF16) return FLDCE_ERR_BAD_DTYPE;
  if (n_dH < 0 || n_dW < 0 || n_db < 0) return FLDCE_ERR_BAD_SHAPE;
  if ((n_dH > 0 && !dH) || (n_dW > 0 && !dW) || (n_db > 0 && !db)) return FLDCE_ERR_NULL_POINTER;
  if (!aligned16(grad_out) || !aligned16(dH) || !aligned16(dW) || !aligned16(db))
    return FLDCE_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* xs[3] = {dH, dW, db};
  const int64_t ns[3] = {n_dH, n_dW, n_db};
  for (int k = 0; k < 3; ++k) {
    if (ns[k] == 0) continue;
    const unsigned g = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(ns[k], 256 * 8), 8192));
    if (dtype == FLDCE_DTYPE_BF16)
      k_scale_grad<bf16><<<g, 256, 0, st>>>(grad_out, static_cast<bf16*>(xs[k]), ns[k]);
    else
      k_scale_grad<float><<<g, 256, 0, st>>>(grad_out, static_cast<float*>(xs[k]), ns[k]);
  }
  return launch_status();
}

int fldce_shard_partials(const void* h, const void* W_local, const int64_t* target, int64_t N,
                         int64_t H, int64_t V_local, int64_t vocab_start, int dtype,
                         int64_t ignore_index, float logit_scale, float* row_max,
                         float* row_sumexp, float* target_logit, float* row_sumlogit,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(h, W_local, target, N, H, V_local, dtype, logit_scale);
  if (rc != FLDCE_OK) return rc;
  if (N > 0 && (!row_max || !row_sumexp || !target_logit)) return FLDCE_ERR_NULL_POINTER;
  if (vocab_start < 0) return FLDCE_ERR_BAD_SHAPE;
  if (!aligned16(h) || !aligned16(W_local) || !aligned16(target) || !aligned16(workspace))
    return FLDCE_ERR_ALIGNMENT;
  const Plan p = make_plan(kShardPartials, N, H, V_local, dtype, 0);
  if (!grids_fit(p, dtype)) return FLDCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total) return FLDCE_ERR_WORKSPACE;
  if (N == 0) return FLDCE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_gemm_attributes();
  char* ws = static_cast<char*>(workspace);
  floatx2* part = reinterpret_cast<floatx2*>(ws + p.oPart);
  float* rpart = reinterpret_cast<float*>(ws + p.oRpart);
  float* colpart = reinterpret_cast<float*>(ws + p.oColpart);
  float* wsum = reinterpret_cast<float*>(ws + p.oWsum);
  const int64_t V = V_local;
  int* rows = reinterpret_cast<int*>(ws + p.oRows);
  int* count = reinterpret_cast<int*>(ws + p.oCount);
  if (dtype == FLDCE_DTYPE_BF16) {
    // rows with target == ignore_index are skipped: (-inf, 0, 0, 0)
    {
      StageTimer tm(kPrep, st);
      k_prep_rows<<<1, 1024, 0, st>>>(target, N, ignore_index, rows, count, 0, 0, nullptr,
                                      row_max, -INFINITY, row_sumexp, 0.f, row_sumlogit, 0.f);
    }
    const int blocks = (int)(cdiv(V, kBM) * cdiv(N, kBN));
    bf16* hc = reinterpret_cast<bf16*>(ws + p.oHC);
    {
      StageTimer tm(kHT, st);
      dim3 g((unsigned)(p.Cp / 64), (unsigned)cdiv(H, 64));
      k_transpose_gather_bf16<<<g, 256, 0, st>>>((const bf16*)h, rows, count, 0, N, H, nullptr, 0,
                                                 p.Cp, hc);
    }
    {
      StageTimer tm(kLogits, st);
      LogitsArgs la{};
      la.W = (const bf16*)W_local;
      la.h = hc;
      la.V = (int)V;
      la.cmax = (int)N;
      la.H = (int)H;
      la.s = logit_scale;
      la.count = count;
      la.rows = rows;
      la.part = part;
      la.rpart = row_sumlogit ? rpart : nullptr;
      la.ldp = p.C;
      la.group_m = kGroupM;
      k_logits_bf16<kEpiMax, kStoreNone, false><<<blocks, kGemmThreads, kGemmLds, st>>>(la);
    }
    {
      StageTimer tm(kCombine, st);
      launch_combine(N, st,
                     shard_combine_args(part, row_sumlogit ? rpart : nullptr, p, N, rows, count, 0,
                                        row_max, row_sumexp, row_sumlogit));
    }
    StageTimer tm(kPrep, st);
    k_rowdot<bf16><<<grid_strided(N, 4), 256, 0, st>>>((const bf16*)h, (const bf16*)W_local, nullptr, H,
                                                 target, vocab_start, V, ignore_index, logit_scale,
                                                 nullptr, nullptr, N, target_logit, nullptr);
  } else {
    float* zb = reinterpret_cast<float*>(ws + p.oZ);
    for (int64_t c0 = 0; c0 < N; c0 += p.C) {
      const int64_t Cc = std::min(p.C, N - c0);
      dim3 g((unsigned)cdiv(V, 64), (unsigned)cdiv(Cc, 64));
      k_gemm_f32_nt<<<g, 256, 0, st>>>((const float*)h + c0 * H, H, Cc, (const float*)W_local, H,
                                       V, H, logit_scale, zb, p.Vp, 0);
      dim3 g2((unsigned)cdiv(Cc, 64), (unsigned)p.nT);
      k_row_partials_f32<<<g2, 64, 0, st>>>(zb, p.Vp, Cc, V, part, p.C);
      launch_combine(Cc, st, shard_combine_args(
          part, nullptr, p, Cc, nullptr, nullptr, c0, row_max, row_sumexp, nullptr));
    }
    if (row_sumlogit) launch_colsum((const float*)W_local, V, H, colpart, wsum, st);
    k_rowdot<float><<<grid_strided(N, 4), 256, 0, st>>>((const float*)h, (const float*)W_local, nullptr, H,
                                                  target, vocab_start, V, ignore_index, logit_scale,
                                                  row_sumlogit ? wsum : nullptr, nullptr, N,
                                                  target_logit, row_sumlogit);
    // same convention as the bf16 path for rows whose target is ignore_index
    k_ignored_rows_init<<<grid1(N, 256), 256, 0, st>>>(target, N, ignore_index, row_max, -INFINITY,
                                                       row_sumexp, 0.f, row_sumlogit, 0.f);
  }
  return launch_status();
}

int fldce_shard_bwd(const void* h, const void* W_local, const int64_t* target, const float* p_mask,
                    const float* lse, int64_t N, int64_t H, int64_t V_local, int64_t vocab_start,
                    int64_t V_global, int dtype, int64_t ignore_index, float label_smoothing,
                    float logit_scale, int reduction, int64_t total, float* dH_partial,
                    void* dW_local, int64_t chunk_rows, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int rc = check_common(h, W_local, target, N, H, V_local, dtype, logit_scale);
  if (rc != FLDCE_OK) return rc;
  if (!dW_local || (N > 0 && (!dH_partial || !lse))) return FLDCE_ERR_NULL_POINTER;
  if (vocab_start < 0 || V_global < vocab_start + V_local) return FLDCE_ERR_BAD_SHAPE;
  if (reduction != FLDCE_REDUCTION_SUM && reduction != FLDCE_REDUCTION_MEAN)
    return FLDCE_ERR_BAD_ARGUMENT;
  if (!(label_smoothing >= 0.f && label_smoothing <= 1.f)) return FLDCE_ERR_BAD_ARGUMENT;
  if (chunk_rows < 0) return FLDCE_ERR_BAD_ARGUMENT;
  if (!aligned16(h) || !aligned16(W_local) || !aligned16(target) || !aligned16(p_mask) ||
      !aligned16(lse) || !aligned16(dH_partial) || !aligned16(dW_local) || !aligned16(workspace))
    return FLDCE_ERR_ALIGNMENT;
  const Plan p = make_plan(kShardBwd, N, H, V_local, dtype, chunk_rows);
  if (!grids_fit(p, dtype)) return FLDCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total) return FLDCE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_gemm_attributes();
  const int esz = dtype == FLDCE_DTYPE_BF16 ? 2 : 4;
  if (N == 0) {
    zero_fill(dW_local, V_local * H, esz, st);
    return launch_status();
  }
  char* ws = static_cast<char*>(workspace);
  float* D = reinterpret_cast<float*>(ws + p.oD);
  const bool bf = dtype == FLDCE_DTYPE_BF16;
  int* rows = reinterpret_cast<int*>(ws + p.oRows);
  int* count = reinterpret_cast<int*>(ws + p.oCount);
  {
    StageTimer tm(kPrep, st);
    if (bf)
      k_prep_rows<<<1, 1024, 0, st>>>(target, N, ignore_index, rows, count, reduction, total, D,
                                      nullptr, 0.f, nullptr, 0.f, nullptr, 0.f);
    else
      k_divisor<<<1, 1024, 0, st>>>(target, N, ignore_index, reduction, total, D);
  }
  Core c{h, W_local, nullptr, target, p_mask, N, H, V_local, vocab_start, V_global, dtype,
         ignore_index, label_smoothing, logit_scale, lse, nullptr, nullptr, nullptr, nullptr,
         nullptr, D, bf ? rows : nullptr, bf ? count : nullptr, dH_partial, true, dW_local,
         nullptr, nullptr, -1, 1.f};
  return run_core(c, p, ws, st);
}

int fldce_profile_num_stages(void) { return kNumStages; }

const char* fldce_profile_stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

int fldce_profile_begin(void) {
  for (int s = 0; s < kNumStages; ++s) g_prof.used[s] = 0;
  g_prof.on = true;
  return FLDCE_OK;
}

int fldce_profile_end(void) {
  g_prof.on = false;
  return FLDCE_OK;
}

int fldce_profile_read(int stage, double* total_ms, int64_t* launches) {
  if (stage < 0 || stage >= kNumStages) return FLDCE_ERR_BAD_ARGUMENT;
  double sum = 0.0;
  const size_t n = g_prof.used[stage] / 2;
  for (size_t i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_prof.ev[stage][2 * i], g_prof.ev[stage][2 * i + 1]) != hipSuccess)
      return FLDCE_ERR_HIP;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int64_t)n;
  return FLDCE_OK;
}

}  // extern "C"
