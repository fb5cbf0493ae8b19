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

GemmPlan plan_fp8_gemm(int m, int n, int k, int num_groups, int mode, int num_cus, int expected_m, int bm_multiple) {
  int best_id = -1;
  // rows each group contributes (masked: the expected count if given, else capacity)
  int rows = m;
  if (mode == MODE_MASKED) rows = expected_m > 0 ? std::min(expected_m, m) : m;

  double best_score = -1.0;
  for (int id = 0; id < num_tile_configs(); ++id) {
    TileConfig tc = tile_config(id);
    if (mode == MODE_CONTIG && (128 % tc.block_m) != 0) continue;   // blocks must be group-pure
    if (bm_multiple > 0 && tc.block_m % bm_multiple != 0) continue;
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
    double score = util * fill * intensity;
    // wide tiles store longer rows of D (512 bytes): measured 2-7 % faster than
    // the tall tile of the same area up to K = 8192 (the shorter the K loop, the
    // more the epilogue weighs), and about 1 % slower at K = 16384
    if (k <= 8192 && tc.block_n > tc.block_m) score *= 1.05;
    if (score > best_score + 1e-9) {
      best_score = score;
      best_id = id;
    }
  }
  if (best_id < 0) {
    GemmPlan none{};
    none.kernel_id = -1;
    return none;
  }
  return plan_with_kernel(m, n, k, num_groups, mode, num_cus, best_id);
}

}  // namespace dg
