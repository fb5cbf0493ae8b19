// Host-side declarations shared by the C-ABI layer, the planner and the kernel
// launchers.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dg {

// MODE_KGROUP: groups along K (each group its own D), with A and B stored [K][..]
enum GemmMode : int { MODE_DENSE = 0, MODE_CONTIG = 1, MODE_MASKED = 2, MODE_KGROUP = 3 };
// Flag or-ed into a mode: A and B scales are packed UE8M0 words (four K blocks
// per int32) instead of fp32, applied by the scaled matrix instruction.
constexpr int MODE_UE8M0 = 4;
// Flag or-ed into a mode: B is stored [K][N], N contiguous (the NN layout).
constexpr int MODE_NN = 8;
// Flag or-ed into a mode: A is stored [K][M], M contiguous (the TN / TT layouts:
// MODE_AT | MODE_NN is TN, MODE_AT alone TT); 128-row A sub-tiles.
constexpr int MODE_AT = 16;

// Arguments of one FP8 block-scaled GEMM launch (dense or grouped).
struct Fp8GemmParams {
  const uint8_t* a;
  const void* sfa;            // fp32 scales, or packed UE8M0 words (MODE_UE8M0)
  const uint8_t* b;
  const void* sfb;
  const uint16_t* c;          // dense only; may be null
  uint16_t* d;
  const int32_t* m_indices;   // contiguous only
  const int32_t* masked_m;    // masked only
  const int32_t* ks;          // K-grouped only: K rows of each group (multiples of 128), on the device
  int m;                      // rows (dense / contiguous) or max_m (masked)
  int n, k;
  int num_groups;             // 1 for dense
  int tiles_m, tiles_n;       // tile grid of one group (masked: over max_m)
  int total_tiles;            // all groups
  int group_m;                // raster: tiles along M visited before moving along N
  int k_rot;                  // K-block rotation step between neighbouring tiles (0: none)
  int splits;                 // K slices per split tile (1: no split)
  int kb_per_split;           // K blocks per slice (the last one may hold fewer)
  int full_tiles;             // tiles [0, full_tiles) of the raster run whole; the rest are split
  float* ws;                  // split K: fp32 partial tiles [(tile - full_tiles) * splits + slice][BM][BN]
  int device_split;           // masked: 0 static tile walk; 1 valid tiles only, split rule applied on the
                              // device (launch the masked reduce after); 2 valid tiles only, no split
};

// Arguments of the skinny-M kernel (all rows of A in one tile; dense NT, fp32 scales).
struct SkinnyParams {
  const uint8_t* a;
  const float* sfa;           // [K/128][M]
  const uint8_t* b;
  const float* sfb;           // [ceil(N/128)][K/128]
  const uint16_t* c;          // may be null
  uint16_t* d;
  float* ws;                  // split K: fp32 partial tiles [(tile * splits + slice)][BM][BN]
  int m, n, k;
  int tiles_m, tiles_n;       // row and column tiles (tile t: row tile t % tiles_m, column tile t / tiles_m)
  int splits;                 // K slices per tile (1: whole tiles, D written directly)
  int kb_per_split;           // K blocks per slice (the last one may hold fewer)
};

// Skinny-M kernel configurations (skinny id indexes this table).
struct SkinnyConfig {
  int block_m, block_n;
  int threads;
  int prefetch;         // K blocks of B in flight per wave (register sets), and of A per chunk
  int lds_bytes;
};
int num_skinny_configs();
SkinnyConfig skinny_config(int id);
hipError_t launch_skinny_gemm(const SkinnyParams& p, int id, int grid, hipStream_t stream);

// Tile shapes compiled into the library (kernel_id indexes this table).
struct TileConfig {
  int block_m, block_n;
  int blocks_per_cu;    // resident workgroups per CU of the compiled kernel
  int threads;          // workgroup size
  int lds_bytes;        // dynamic LDS per workgroup
  int stages;           // LDS ring slots
};
int num_tile_configs();
TileConfig tile_config(int kernel_id);
// The wide tiles (fp8_gemm_wide.hip), NT with fp32 scales only: 256x256 and
// 256x224 (dense), 128x512 (dense and contiguous).  Their copies form (row) * K
// offsets in 32 bits for rows up to a tile past the last.
constexpr int kTile256x256Id = 4, kTile128x512Id = 5, kTile256x224Id = 6;
inline bool is_wide_tile(int kernel_id) { return kernel_id >= kTile256x256Id && kernel_id <= kTile256x224Id; }
inline bool wide_fits(int m, int n, int k) {
  return (long long)(m + 256) * k < (1LL << 32) && (long long)(n + 512) * k < (1LL << 32);
}
// the forms (MODE_*) a wide tile serves
inline bool wide_serves(int kernel_id, int mode) {
  return mode == MODE_DENSE || (kernel_id == kTile128x512Id && mode == MODE_CONTIG);
}
TileConfig wide_tile_config(int kernel_id);
hipError_t launch_fp8_gemm_wide(const Fp8GemmParams& p, int kernel_id, int mode, int grid, hipStream_t stream);

// Device facts the planner and launchers need (cached per device).
struct DeviceInfo {
  int device;
  int num_cus;
  bool ok;
};
DeviceInfo current_device_info();

// Plan for one GEMM call.
struct GemmPlan {
  int kernel_id;
  int block_m, block_n;
  int tiles_m, tiles_n;
  int num_tiles;              // output tiles (all groups)
  int splits;                 // K slices per split tile (dense only; 1: none)
  int kb_per_split;
  int full_tiles;             // tiles computed whole; tiles [full_tiles, num_tiles) are split
  int num_workgroups;
  int skinny_id;              // >= 0: the skinny-M kernel of that configuration (kernel_id is then
                              // kSkinnyIdBase + skinny_id); -1: the square-tile kernel kernel_id
};
constexpr int kSkinnyIdBase = 100;
// The skinny-M plan for a dense NT problem with fp32 scales and m <= 256 rows, in
// row tiles of at most 128 (skinny_id < 0 when the kernel does not apply).  force_id / force_splits >= 0
// pin the configuration / the K slices (for tuning).
GemmPlan plan_skinny(int m, int n, int k, int num_cus, bool has_c, int force_id = -1, int force_splits = -1);
// bm_multiple > 0: only tile shapes whose height is a multiple of it (an A stored
// [K][M] is staged in 128-row sub-tiles)
// allow_wide: the wide tiles may be chosen (NT with fp32 scales, offsets that fit)
GemmPlan plan_fp8_gemm(int m, int n, int k, int num_groups, int mode, int num_cus, int expected_m,
                       int bm_multiple = 0, bool allow_wide = false);
GemmPlan plan_with_kernel(int m, int n, int k, int num_groups, int mode, int num_cus, int kernel_id);
// Resident workgroup slots of a compiled tile shape on num_cus CUs.
int plan_slots(int kernel_id, int num_cus);

// Split K: for every split tile, D = bf16(sum of its ws slices in slice order + C);
// returns a hipError_t.
hipError_t launch_splitk_reduce(const Fp8GemmParams& p, const GemmPlan& plan, int num_cus, hipStream_t stream);
// The same for the device-planned masked form, on the plan the GEMM kernel
// derived from masked_m with `slots` workgroups.
hipError_t launch_masked_splitk_reduce(const Fp8GemmParams& p, const GemmPlan& plan, int slots, hipStream_t stream);

// K splitting rule, shared by the host planner and (for the masked form, whose
// tile count only the device knows) the kernels.  Returns the K slices per
// split tile (1: none) and sets *full to the number of tiles computed whole:
//  * when the tiles cannot fill the workgroup slots (tiles * 2 <= slots) every
//    tile is split, into enough slices to occupy every slot once;
//  * when the last round is partial and at most half full, the whole rounds run
//    unsplit and only the remainder is split, so the last round takes a slice's
//    time instead of a whole tile's; taken only when that saves at least
//    kTailMinGain K blocks per workgroup (the partials' round trip and the
//    second launch cost about that much).
// Slices hold at least four K blocks; at most 16 slices.
constexpr int kTailMinGain = 24;
__host__ __device__ inline int split_rule(long long tiles, long long slots, int kb, long long* full) {
  *full = tiles;
  if (tiles <= 0 || kb < 8) return 1;
  const bool all = tiles * 2 <= slots;
  const long long rem = all ? tiles : tiles % slots;
  if (rem == 0 || rem * 2 > slots) return 1;
  long long s = slots / rem < kb / 4 ? slots / rem : kb / 4;
  s = s < 16 ? s : 16;
  if (s < 2) return 1;
  const int per = (kb + (int)s - 1) / (int)s;
  s = (kb + per - 1) / per;
  if (!all && kb - per < kTailMinGain) return 1;
  *full = tiles - rem;
  return (int)s;
}

// Masked form: output tiles of group g (valid rows rounded up to whole tiles).
__device__ inline int masked_group_tiles(const int32_t* masked_m, int g, int max_m, int bm, int tiles_n) {
  int mm = masked_m[g];
  mm = mm < 0 ? 0 : (mm > max_m ? max_m : mm);
  return (mm + bm - 1) / bm * tiles_n;
}

// Masked form: output tiles of all groups, summed by the 64 lanes of a wave
// in parallel (every lane returns the total).
__device__ inline int masked_total_tiles(const int32_t* masked_m, int groups, int max_m, int bm, int tiles_n) {
  int part = 0;
  for (int g = (int)(threadIdx.x & 63); g < groups; g += 64) part += masked_group_tiles(masked_m, g, max_m, bm, tiles_n);
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  return __builtin_amdgcn_readfirstlane(part);
}

// Raster order of the output tiles (one group): bands of group_m tile rows, walked
// column by column inside a band, tile rows fastest.  Tile index tl -> (tile row, tile column).
__host__ __device__ inline void raster_tile(int tl, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
  const int per_group = group_m * tiles_n;
  const int gi = tl / per_group;
  const int first_m = gi * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int r = tl - gi * per_group;
  *tm = first_m + r % gm;
  *tn = r / gm;
}

// K-grouped form: zeroes D of every group without K rows (before the GEMM).
hipError_t launch_kgroup_zero(const Fp8GemmParams& p, hipStream_t stream);

// Launches the kernel chosen by plan on stream; returns a hipError_t.
hipError_t launch_fp8_gemm(const Fp8GemmParams& p, const GemmPlan& plan, int mode, hipStream_t stream);

// The dense GEMM entry (argument checks, plan, launch) behind dg_fp8_gemm_nt and its
// layout / UE8M0 variants; flags as MODE_* above.  Returns a dg_status.
bool form_mode(int form, int* mode, int* flags);
int dense_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, const uint16_t* c,
                uint16_t* d, int m, int n, int k, void* ws, size_t ws_bytes, void* stream, int flags);

}  // namespace dg
