// Host-side tile heuristic for the FP8 GEMM kernels.
//
// The release article ("DeepSeek 开源第三弹 ... DeepGEMM", 优化技术 / 完全 JIT 设计
// and 非对齐块大小) describes a deterministic, autotune-free choice of block sizes,
// and notes that power-of-two blocks can leave compute units idle (its example:
// M=256, N=7168 with 128x128 blocks gives 112 tiles on a 132-unit part, while a
// 112-wide block gives 128).  Here the same idea is applied to 256 CUs: among
// the compiled tile shapes, prefer the one whose tile count fills the chip with
// the least padding, and launch at most (CUs x workgroups per CU) persistent
// workgroups.
#include <algorithm>

#include "dg_internal.hpp"

namespace dg {

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }


// Resident workgroups per CU for each compiled tile shape: the smaller of the
// LDS bound (160 KB per CU) and the occupancy the tile table records.
static int blocks_per_cu_for(int kernel_id) {
  TileConfig tc = tile_config(kernel_id);
  int by_lds = (160 * 1024) / tc.lds_bytes;
  return std::max(1, std::min(tc.blocks_per_cu, by_lds));
}

int plan_slots(int kernel_id, int num_cus) { return num_cus * blocks_per_cu_for(kernel_id); }

// K splitting for the dense and contiguous forms (see split_rule).
static int choose_splits(long long tiles, long long slots, int kb, long long* full) {
  return split_rule(tiles, slots, kb, full);
}

GemmPlan plan_with_kernel(int m, int n, int k, int num_groups, int mode, int num_cus, int kernel_id) {
  GemmPlan plan{};
  plan.skinny_id = -1;
  TileConfig tc = tile_config(kernel_id);
  plan.kernel_id = kernel_id;
  plan.block_m = tc.block_m;
  plan.block_n = tc.block_n;
  plan.tiles_m = cdiv(m, tc.block_m);
  plan.tiles_n = cdiv(n, tc.block_n);
  const bool per_group = mode == MODE_MASKED || mode == MODE_KGROUP;   // every group has its own tile grid
  long long total = (long long)plan.tiles_m * plan.tiles_n * (per_group ? num_groups : 1);
  plan.num_tiles = (int)std::min<long long>(total, 0x7fffffff);
  long long slots = (long long)num_cus * blocks_per_cu_for(kernel_id);
  plan.splits = 1;
  plan.kb_per_split = k / 128;
  plan.full_tiles = plan.num_tiles;
  if (!per_group) {   // (the masked form's split is planned on the device; K-grouped: no split)
    long long full = total;
    plan.splits = choose_splits(total, slots, k / 128, &full);
    plan.kb_per_split = cdiv(k / 128, plan.splits);
    plan.full_tiles = (int)full;
  }
  const long long units = plan.full_tiles + (total - plan.full_tiles) * plan.splits;
  plan.num_workgroups = (int)std::min<long long>(units, slots);
  return plan;
}

GemmPlan plan_fp8_gemm(int m, int n, int k, int num_groups, int mode, int num_cus, int expected_m, int bm_multiple,
                       bool allow_wide) {
  int best_id = -1;
  // rows each group contributes (masked: the expected count if given, else capacity)
  int rows = m;
  if (mode == MODE_MASKED) rows = expected_m > 0 ? std::min(expected_m, m) : m;

  double best_score = -1.0;
  for (int id = 0; id < num_tile_configs(); ++id) {
    TileConfig tc = tile_config(id);
    if (is_wide_tile(id) && (!allow_wide || !wide_serves(id, mode))) continue;
    // the 256x224 tile: from HBM (the timed bench's cold calls) it measured
    // even with 256x256 at K = 16384 and about 2.5 % behind at K = 2048, so it
    // is planned for long K only (with operands resident in the caches it was
    // 4-7 % ahead at both)
    if (id == kTile256x224Id && k < 8192) continue;
    if (mode == MODE_CONTIG && (128 % tc.block_m) != 0) continue;   // blocks must be group-pure
    if (bm_multiple > 0 && tc.block_m % bm_multiple != 0) continue;
    // masked (decode) calls stream every group's B from HBM once per row tile of the
    // group, so a tile shorter than 128 rows re-streams B for groups past its height:
    // measured slower at every expected row count tried (32 groups x 7168 x 7168,
    // masked_m ~ U{0..128}: 64-row tiles 353 us, 128x256 324 us)
    if (mode == MODE_MASKED && m >= 128 && tc.block_m < 128) continue;
    int tm = cdiv(rows, tc.block_m);
    int tn = cdiv(n, tc.block_n);
    long long tiles = (long long)tm * tn * (mode == MODE_MASKED || mode == MODE_KGROUP ? num_groups : 1);
    // useful fraction of the MFMA work (padding in M and N is wasted)
    double util = (double)rows / (tm * tc.block_m) * (double)n / (tn * tc.block_n);
    // wave quantisation: busy fraction of the workgroup slots over the call, in
    // K-block steps (a split tail costs its slice plus about kTailMinGain / 3
    // steps for the partials' round trip)
    int slots = num_cus * blocks_per_cu_for(id);
    const int kb = k / 128;
    long long full = tiles;
    const int splits = mode != MODE_MASKED && mode != MODE_KGROUP ? choose_splits(tiles, slots, kb, &full) : 1;
    const long long units = full + (tiles - full) * splits;
    double fill;
    if (splits > 1 && full > 0) {
      const double steps = (double)(full / slots) * kb + cdiv(kb, splits) + kTailMinGain / 3.0;
      fill = (double)tiles * kb / ((double)slots * steps);
    } else {
      const long long waves = (units + slots - 1) / slots;
      fill = (double)units / (double)(waves * slots);
      if (splits > 1) fill *= 0.8;   // split K writes and re-reads fp32 partials
    }
    // bigger tiles re-read less from L2/HBM: weight by tile area (arithmetic intensity)
    double intensity = (double)tc.block_m * tc.block_n / (tc.block_m + tc.block_n);
    // ... except when every tile is split (skinny M): such calls stream B from
    // HBM, and a deeper copy ring keeps more of it in flight (measured: the
    // 4-slot 64x128 shape beats the 3-slot ones at M = 64 and 128)
    if (splits > 1 && full == 0) intensity = tc.stages;
    // The wide tiles: measured on MI355X against the 256x128 / 128x256 tiles at
    // equal fill (dense, with C), 10-20 % faster from K = 1024 on (fewer copy
    // bytes per matrix instruction, whole-row D stores), even at K = 512, where a
    // tile's fixed costs (pipeline fill, C and D through LDS) weigh most:
    // relative speed about 1.15 kb / (kb + 0.6).  The 128x512 tile measured 0-6 %
    // behind the 256x256 one on dense shapes (its A scales come through a
    // register and cross-lane reads, not LDS), except at K = 512, where the
    // epilogue weighs most and its tile has half the boundaries of the 128x256
    // one, with D and C rows of 1 KB (timed bench, operands from HBM, with C:
    // 4096x32768x512 155 against 164 us; at K = 1024 and 1536 it measured even
    // to 2 % behind).  It serves the contiguous form, whose 128-row groups the
    // 256-row tile would straddle.  The
    // 256x224 tile (N = 7168 in 32 column tiles) runs 28 matrix instructions per
    // barrier instead of 32.
    else if (is_wide_tile(id)) {
      double shape = 1.0;
      if (id == kTile128x512Id && mode == MODE_DENSE) shape = kb == 4 ? 1.1 : 0.97;
      if (id == kTile256x224Id) shape = 0.97;
      intensity = 256.0 * 128.0 / 384.0 * 1.15 * kb / (kb + 0.6) * shape;
    }
    double score = util * fill * intensity;
    // wide tiles store longer rows of D (512 bytes): measured 2-7 % faster than
    // the tall tile of the same area up to K = 8192 (the shorter the K loop, the
    // more the epilogue weighs), and about 1 % slower at K = 16384
    if (k <= 8192 && tc.block_n > tc.block_m && !is_wide_tile(id)) score *= 1.05;
    if (score > best_score + 1e-9) {
      best_score = score;
      best_id = id;
    }
  }
  if (best_id < 0) {
    GemmPlan none{};
    none.kernel_id = -1;
    none.skinny_id = -1;
    return none;
  }
  return plan_with_kernel(m, n, k, num_groups, mode, num_cus, best_id);
}

// Skinny M (all rows of A in one tile).  Such a problem streams B from HBM once;
// the choice is between column-tile widths and K slices.  Each candidate is
// scored with a simple time model (microseconds), from per-phase timestamps of
// the kernel on MI355X:
//   * the chip moves B, A, C and D (and a split plan's partials twice, written
//     by the slices and read by the reduce) at about 5.5 TB/s;
//   * a CU copies its unit's slice of A into LDS at about 20 B/clk, and streams
//     B at about 25 B/clk (bytes in flight over HBM latency);
//   * each K block a unit runs (its slice padded to a multiple of the prefetch
//     depth) costs the waves' reads of A from LDS, about 0.4 us per 64 KB;
//   * a unit costs about 1 us of pipeline fill and drain, a split plan a second
//     launch (about 3 us with its reads).
// Split plans keep every unit in one round of workgroups (at most one partial
// tile per workgroup slot, the bound of the caller's workspace).
GemmPlan plan_skinny(int m, int n, int k, int num_cus, bool has_c, int force_id, int force_splits) {
  GemmPlan best{};
  best.kernel_id = -1;
  best.skinny_id = -1;
  if (m <= 0 || m > 256 || n <= 0 || k <= 0 || num_cus <= 0) return best;
  const int kb = k / 128;
  double best_t = 1e30;
  // the smallest row block that holds every row (two 128-row tiles above 128)
  const int bm_need = m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : 128;
  for (int id = 0; id < num_skinny_configs(); ++id) {
    const SkinnyConfig sc = skinny_config(id);
    if (force_id >= 0 ? id != force_id : sc.block_m != bm_need) continue;
    const int tiles_m = cdiv(m, sc.block_m);
    const int tiles = tiles_m * cdiv(n, sc.block_n);
    for (int s = 1; s <= std::min(16, kb); ++s) {
      const int per = cdiv(kb, s);
      const int splits = cdiv(kb, per);
      if (splits != s) continue;                       // each slice count once
      if (force_splits > 0 && splits != force_splits) continue;
      const long long units = (long long)tiles * splits;
      if (splits > 1 && (units > num_cus || per < 2)) continue;
      const long long rounds = (units + num_cus - 1) / num_cus;
      const double pad = (double)cdiv(per, sc.prefetch) * sc.prefetch;   // blocks a unit runs
      const double a_bytes = (double)std::min(m, sc.block_m) * 128.0 * per;
      const double lds_reads = (double)sc.threads / 64 * sc.block_m * 128.0 * pad;   // every wave reads all of A
      double chip = (double)n * k * tiles_m + (double)m * k + (double)m * n * 2.0 * (has_c ? 2 : 1);
      if (splits > 1) chip += 2.0 * units * sc.block_m * sc.block_n * 4.0;
      const double t_chip = chip / 5.5e6;
      const double t_cu = rounds * (a_bytes / (20.0 * 2400.0) +
                                    std::max((double)sc.block_n * 128.0 * per / (25.0 * 2400.0),
                                             lds_reads / 64e3 * 0.4));
      const double t = std::max(t_chip, t_cu) + rounds * 1.0 + (splits > 1 ? 3.0 : 0.0);
      if (t < best_t - 1e-9) {
        best_t = t;
        best.skinny_id = id;
        best.kernel_id = kSkinnyIdBase + id;
        best.block_m = sc.block_m;
        best.block_n = sc.block_n;
        best.tiles_m = tiles_m;
        best.tiles_n = tiles / tiles_m;
        best.num_tiles = tiles;
        best.splits = splits;
        best.kb_per_split = per;
        best.full_tiles = splits > 1 ? 0 : tiles;
        best.num_workgroups = (int)std::min<long long>(units, num_cus);
      }
    }
  }
  return best;
}

}  // namespace dg
