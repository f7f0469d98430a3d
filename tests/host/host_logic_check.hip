// Host-side checks of the library's launch logic, run on the CPU (no kernel
// is launched).  The translation unit includes the library source itself, so
// the checks see exactly the code the entry points run:
//   1. tile_coord_of: over a sweep of tile counts, split counts, group sizes
//      and grids sized for more rows than exist, the active blocks cover
//      every (tile row, tile column, split) exactly once, and the 8 XCDs'
//      shares differ by at most one item;
//   2. choose_splits: within [1, max_splits], one split from 256 tiles on,
//      at least 8 K tiles per split;
//   3. make_plan: for every number of rows the device may find in a chunk
//      (any count of non-ignored rows), with and without the all-ones row of
//      the label-smoothing term, the dH GEMM's grid covers its work items,
//      the split-K partials it writes fit the space reserved for them, the
//      rows of E past the chunk's rows fit its allocation, and the
//      smoothing-term partials fit theirs.
// Prints "ok" and exits 0, or prints the first failure and exits 1.
#include "../../lm_head_linear_bf16_amd/csrc/fldce.hip"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

int fail(const char* what, long long a, long long b, long long c, long long d) {
  std::printf("FAIL %s (%lld %lld %lld %lld)\n", what, a, b, c, d);
  return 1;
}

int check_tile_map() {
  for (int tm_grid = 1; tm_grid <= 24; ++tm_grid)
    for (int tiles_n = 1; tiles_n <= 11; ++tiles_n)
      for (int splits = 1; splits <= 8; splits += (splits < 4 ? 1 : 4))
        for (int group_m : {1, 2, 4, 5})
          for (int tiles_m = 0; tiles_m <= tm_grid; ++tiles_m) {
            // grid sized for tm_grid tile rows; the device finds tiles_m
            const int grid = tm_grid * tiles_n * splits;
            const int items = tiles_m * tiles_n * splits;
            std::vector<int> seen((size_t)std::max(items, 1), 0);
            int per_xcd[8] = {};
            for (int bid = 0; bid < grid; ++bid) {
              const TileCoord c = tile_coord_of(bid, tiles_m, tiles_n, splits, group_m);
              if (!c.active) continue;
              if (c.tm < 0 || c.tm >= tiles_m || c.tn < 0 || c.tn >= tiles_n || c.split < 0 ||
                  c.split >= splits)
                return fail("tile_coord_of out of range", bid, tiles_m, tiles_n, splits);
              ++seen[((size_t)c.split * tiles_m + c.tm) * tiles_n + c.tn];
              ++per_xcd[bid % 8];
            }
            for (int i = 0; i < items; ++i)
              if (seen[i] != 1) return fail("tile_coord_of not a bijection", i, tiles_m, tiles_n, splits);
            const int lo = *std::min_element(per_xcd, per_xcd + 8);
            const int hi = *std::max_element(per_xcd, per_xcd + 8);
            if (hi - lo > 1) return fail("tile_coord_of XCD shares unbalanced", lo, hi, items, group_m);
          }
  return 0;
}

int check_choose_splits() {
  for (int64_t tiles = 1; tiles <= 700; ++tiles)
    for (int64_t k_tiles : {1, 7, 8, 40, 71, 297, 2374})
      for (int mx : {1, 2, 4, 8}) {
        const int S = choose_splits(tiles, k_tiles, mx);
        if (S < 1 || S > mx) return fail("choose_splits range", tiles, k_tiles, mx, S);
        if (tiles >= 256 && S != 1) return fail("choose_splits full wave", tiles, k_tiles, mx, S);
        if (S > 1 && k_tiles / S < 8) return fail("choose_splits K per split", tiles, k_tiles, mx, S);
      }
  return 0;
}

int check_plan(int mode, int64_t N, int64_t H, int64_t V, int64_t chunk) {
  const Plan p = make_plan(mode, N, H, V, FLDCE_DTYPE_BF16, chunk);
  const size_t end = p.nchunks > 1 ? p.oDW32 : p.total;
  if (end < p.oDHpart) return fail("plan layout", N, H, V, chunk);
  const size_t reserved = end - p.oDHpart;
  const int64_t th = cdiv(H, kBN), k_tiles = p.Vp / kBK;
  int64_t ublocks = 0;
  for (int64_t ic = 0; ic < p.nchunks; ++ic) {
    const int64_t cmax = std::min(p.C, N - ic * p.C);
    ublocks += cdiv(cmax, 64);
    for (int extra = 0; extra <= 1; ++extra) {  // the all-ones row (label smoothing)
      const int64_t grid = cdiv(cmax + extra, kBM) * th * p.splits;
      for (int64_t n = 0; n <= cmax; ++n) {  // rows the device may find in this chunk
        const int64_t Me = n + extra;
        const int64_t tiles = cdiv(Me, kBM) * th;
        const int S = choose_splits(tiles, k_tiles, p.splits);
        if (tiles * S > grid) return fail("dH grid too small", N, H, n, S);
        const size_t need = (S > 1 || extra) ? (size_t)S * Me * H * 4 : 0;
        if (need > reserved) return fail("dH partials exceed the workspace", N, H, n, (long long)need);
        // E rows written or read past the chunk's rows, and h^T columns
        if (round_up(Me, 64) > p.Cp) return fail("E rows exceed the workspace", N, H, n, p.Cp);
      }
    }
  }
  if (ublocks > p.u_blocks) return fail("smoothing partial blocks", N, H, ublocks, p.u_blocks);
  return 0;
}

}  // namespace

int main() {
  if (check_tile_map()) return 1;
  if (check_choose_splits()) return 1;
  struct Shape { int64_t N, H, V, chunk; };
  const Shape shapes[] = {
      {1, 64, 100, 0},      {300, 64, 1000, 0},   {700, 192, 3001, 256}, {2048, 2560, 151936, 0},
      {8192, 2560, 151936, 0}, {8192, 2560, 151936, 1024}, {5000, 4096, 151936, 2048},
      {3000, 5120, 18992, 0}, {4096, 128, 5000, 1000}, {600, 64 * 40, 7000, 0},
      {797, 320, 3000, 100}, {797, 64, 257, 333}, {1, 64, 1, 0}, {199, 192, 2, 64}};
  for (const Shape& s : shapes)
    for (int mode : {kFwdBwd, kShardBwd})
      if (check_plan(mode, s.N, s.H, s.V, s.chunk)) return 1;
  std::printf("ok\n");
  return 0;
}
