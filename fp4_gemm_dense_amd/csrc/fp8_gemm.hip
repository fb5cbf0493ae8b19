// Fine-grained-scaled FP8 GEMM for gfx950: D = C + A.B^T (NT), bf16 out.
//
// What is computed follows the DeepGEMM pages: the usage guide
// ("DeepGEMM：统一高性能张量核心 GEMM 计算库编译与使用指南", 五、使用方法) for the
// D = C + A @ B naming, the NT layout and fp32 scale factors, and the release
// article ("DeepSeek 开源第三弹 ... DeepGEMM", DeepGEMM section) for the
// two-level accumulation: the matrix cores reduce one scale block into a fresh
// partial, which is then scaled and added into an fp32 accumulator on the
// vector ALUs.  One kernel template serves the dense, contiguous-grouped and
// masked-grouped forms (release article, 优化技术 / 统一且经过优化的块调度器: one
// scheduler for all of them).
//
// gfx950 design (not the pages' Hopper design):
//   * WM x WN wave64s per workgroup; each wave owns an (MT*16) x (NT*16)
//     sub-tile of 16x16 accumulator blocks, computed transposed (B_nt . A_mt^T)
//     so that a lane's four results lie in one row of D and share one A scale.
//   * Per 128-wide K block, A, B and the A scales are copied by buffer loads
//     straight into a STAGES-deep LDS ring (no registers in between), XOR-
//     swizzled so that fragment reads are free of bank conflicts.  Waits count
//     outstanding memory operations (s_waitcnt vmcnt) instead of draining them.
//   * Each 16x16 block does ONE v_mfma_f32_16x16x128_f8f6f4 per K block into a
//     fresh fp32 partial; the partial is promoted by one FMA per element with
//     sa[row]*sb a few matrix instructions later, so the vector ALU never waits
//     on the matrix core.
//   * Epilogue: C is copied into the ring slots the last two K blocks leave
//     free.  The next tile's first stage is copied into the last block's slot
//     while this tile waits for C (the ring's start moves from tile to tile),
//     its other stages once C has been read, and this tile's stores follow
//     them, draining while the next tile computes.
//   * Persistent workgroups walk a group-M raster of tiles; block ids are
//     remapped so that each XCD (workgroups are dealt round-robin to the 8
//     XCDs) works on a contiguous stretch of the raster and shares its L2.
#include <algorithm>
#include <type_traits>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

// MODE_SF: the form (MODE_DENSE, MODE_CONTIG, MODE_MASKED), plus MODE_UE8M0 for
// packed power-of-two scale factors, which the matrix instruction applies
// itself (no fresh partials, no promotion on the vector ALUs).
template <int MT, int NT, int WM, int WN, int STAGES, int MODE_SF>
__global__ void __launch_bounds__(WM * WN * 64, 1) fp8_gemm_kernel(Fp8GemmParams p) {
  constexpr int MODE = MODE_SF & 3;
  constexpr bool UE = (MODE_SF & MODE_UE8M0) != 0;
  constexpr bool NN = (MODE_SF & MODE_NN) != 0;   // B stored [K][N]
  constexpr bool AT = (MODE_SF & MODE_AT) != 0;   // A stored [K][M]
  constexpr int NW = WM * WN;                 // waves per workgroup
  constexpr int BM = WM * MT * 16;
  constexpr int BN = WN * NT * 16;
  constexpr int A_BYTES = BM * 128;
  constexpr int B_BYTES = BN * 128;
  constexpr int SA_BYTES = BM * 4;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  // Copy waves: in eight-wave tiles only waves 0-3 (one per SIMD) issue the
  // stage copies, so the other wave of each SIMD never stalls on a full memory
  // pipeline between its matrix instructions (measured 1-3 % faster than every
  // wave copying).  Waves w and w + 4 share a SIMD.  Tiles of fewer waves, and
  // an A stored [K][M] (whose doubled copy state would spill), copy with every
  // wave.  Each copy wave copies RA 8-row regions (1 KB) of A, RB of B and SPW A
  // scales per stage.
  constexpr int NCW = NW >= 8 && !AT ? NW / 2 : NW;
  static_assert((BM / 8) % NCW == 0 && (BN / 8) % NCW == 0, "regions must split evenly over the copy waves");
  constexpr int RA = BM / 8 / NCW;
  constexpr int RB = BN / 8 / NCW;
  constexpr int SPW = BM / NCW;
  static_assert(SPW <= 64, "scale copy must fit one instruction per wave");
  constexpr int LPS = RA + RB + 1;            // DMA instructions per copy wave per stage
  // NN: the B slot holds the tile's 128 K rows of BN bytes (columns), as BN/128
  // column halves of 128 rows x 128 bytes, so its copies have the shape of the
  // NT B tile's BN rows of 128 K bytes (8-row x 128-byte regions)
  static_assert(!NN || BN % 128 == 0, "the NN layout uses 128-column B sub-tiles");
  // AT: the A slot holds 128 K rows of BM bytes (rows of D) the same way
  static_assert(!AT || BM % 128 == 0, "an A stored [K][M] uses 128-row sub-tiles");
  // all of a wave's columns lie in one 128-wide B-scale block, so one sb per
  // K block serves the whole wave
  static_assert(128 % (NT * 16) == 0 && (BN % 128 == 0 || 128 % BN == 0), "one B scale per wave");
  static_assert(MT % 4 == 0, "a lane reads its row scales with 16-byte LDS loads");
  constexpr int NBLK = MT * NT;   // 16x16 accumulator blocks per wave
  static_assert(MT <= 4 && STAGES >= 3, "all A fragments of a K block live at once; three or more slots");
  constexpr int LAG = NT;         // matrix instructions between a partial's issue and its promotion (<= NT)
  // Epilogue traffic.  The C tile (BM x BN bf16) is copied into two ring slots
  // that the last two K blocks leave free, in halves of BM/2 rows; each wave
  // copies CPW 1-KB pieces of a half.  A C row holds CPR 16-byte chunks, chunk c
  // of row r sits at position c ^ (r % 16).  D is staged in the same place and
  // layout, and every wave then issues exactly NSTD 16-byte stores of it (NPART
  // 16-byte stores of fp32 partials for a split slice).
  constexpr int CPR = BN / 8;
  constexpr int C_HALF = BM / 2 * BN * 2;
  static_assert(CPR >= 16 && 1024 % (BN * 2) == 0, "C rows must be 256 or 512 bytes");
  static_assert(C_HALF % (NW * 1024) == 0 && C_HALF <= STAGE, "C halves must fit a slot");
  static_assert((BM / 2) % 16 == 0, "a 16-row block must not straddle the C halves");
  constexpr int CPW = C_HALF / (NW * 1024);
  constexpr int NSTD = BM * BN / 8 / (NW * 64);
  static_assert((BM * BN / 8) % (NW * 64) == 0, "D chunks must split evenly over the lanes");
  constexpr int NPART = MT * NT;
  constexpr int NST = NSTD > NPART ? NSTD : NPART;
  static_assert((STAGES - 2) * LPS + NST + CPW < 64, "vmcnt range");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef const __attribute__((address_space(4))) float cfloat;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool cw = NCW == NW || wave < NCW;   // a copy wave (a constant when every wave copies)
  const int wave_m = wave / WN;
  const int wave_n = wave % WN;
  const int lrow = lane & 15;     // operand row / output column inside a 16x16 block
  const int lgrp = lane >> 4;     // K chunk of the operand / row quad of the output

  const int M = p.m, N = p.n, K = p.k;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;
  const int KW = (KB + 3) >> 2;   // packed UE8M0 words per row of scales (four K blocks each)

  // Per-lane LDS read offsets (slot 0); blocks mt / nt add mt*2048 / nt*2048
  // and the slot adds slot*STAGE.  The swizzle depends on row % 16 only.
  const int sw = swz(lrow);
  const uint32_t a_lo = (wave_m * MT * 16 + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const uint32_t a_hi = (wave_m * MT * 16 + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);
  const uint32_t b_lo = A_BYTES + (wave_n * NT * 16 + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const uint32_t b_hi = A_BYTES + (wave_n * NT * 16 + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);
  const uint32_t sa_rd = A_BYTES + B_BYTES + (wave_m * MT * 16 + lrow * MT) * 4;
  // NN B fragments (ds_read_b64_tr_b8).  Within each 16-lane group the read
  // hands lane l byte b of the 8-byte row addressed by lane 2b + (l >= 8),
  // taken at column l % 8.  Lane s addresses K row 32g + 8i + s/2 and the half
  // s % 2 of the block's 16 columns, so lane l receives K 32g + 8i .. +7 of
  // column l: read i gives bytes 8i .. 8i+7 of the lane's 32 K values (the A
  // fragment's K order).  In the slot, 16-byte chunk c of K row r sits at
  // c ^ kt_swz(r): the 8 rows one lane group reads fall on distinct banks, and
  // the rows of the neighbouring group (32 rows on) on the other positions of
  // each half of the banks (measured: the plain r % 8 key left 2-way conflicts).
  // Column chunk q (16 columns) of the tile lies in sub-tile q / 8 at chunk q % 8.
  const uint32_t b_nn_row = A_BYTES + (32 * lgrp + (lrow >> 1)) * 128 + (lrow & 1) * 8;
  const uint32_t a_t_row = (32 * lgrp + (lrow >> 1)) * 128 + (lrow & 1) * 8;   // AT: the same for A
  const int b_nn_sw = kt_swz(32 * lgrp + (lrow >> 1));   // constant over the four reads (rows + 8i)
  const int dma_row = lane >> 3;              // DMA row inside an 8-row region
  const uint32_t a_dst = wave * RA * 1024;
  const uint32_t b_dst = A_BYTES + wave * RB * 1024;
  const uint32_t sa_dst = A_BYTES + B_BYTES + wave * SPW * 4;

  // XCD-aware remap of the persistent block id: workgroups are dealt to the
  // 8 XCDs round-robin, so give XCD x a contiguous stretch of the raster.
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // ---------------- tile decode: tile id -> (group, m0, n0, valid rows) ----------------
  struct Tile {
    int g, m0, n0, rows_valid;
    int kb0, nkb;   // K blocks [kb0, kb0 + nkb) of this work unit (split K: a slice)
    int rot;        // first K block: tiles that share A rows or B rows start at different K
    int part;       // split K: index of this slice's fp32 partial tile in the workspace; -1: whole tile
  };
  // Work units: units [0, full_tiles) are the tiles of the same index, computed
  // whole; unit full_tiles + u is K slice u % splits of tile full_tiles + u / splits.
  int full_tiles = p.full_tiles, splits = p.splits, kb_per_split = p.kb_per_split, total_units = p.total_tiles;
  // Masked form, device-planned: the tiles are those holding valid rows, group
  // after group (group g has ceil(masked_m[g] / BM) tile rows), and the split
  // rule is applied to their count, which only the device knows.  Every
  // workgroup (and the reduce kernel) derives the same plan.
  const bool dev_plan = MODE == MODE_MASKED && p.device_split;
  int mg = 0, mg_base = 0, mg_cnt = 0;   // group cursor of the decode (tile ids only grow)
  if (dev_plan) {
    const int tiles = masked_total_tiles(p.masked_m, p.num_groups, M, BM, p.tiles_n);
    long long full = tiles;
    splits = p.device_split == 1 ? split_rule(tiles, G, KB, &full) : 1;
    full_tiles = (int)full;
    kb_per_split = (KB + splits - 1) / splits;
    total_units = full_tiles + (tiles - full_tiles) * splits;
    mg_cnt = masked_group_tiles(p.masked_m, 0, M, BM, p.tiles_n);
  }
  const bool can_split = splits > 1;
  auto decode = [&](int t, Tile& tile) -> bool {
    tile.kb0 = 0;
    tile.nkb = KB;
    tile.part = -1;
    if (can_split && t >= full_tiles) {
      const int u = t - full_tiles;
      const int sl = u % splits;
      t = full_tiles + u / splits;
      tile.kb0 = sl * kb_per_split;
      tile.nkb = min(kb_per_split, KB - tile.kb0);
      tile.part = u;
    }
    int g = 0, tl = t, tiles_m = p.tiles_m;
    if (dev_plan) {
      while (t >= mg_base + mg_cnt) {
        mg_base += mg_cnt;
        mg_cnt = masked_group_tiles(p.masked_m, ++mg, M, BM, p.tiles_n);
      }
      g = mg;
      tl = t - mg_base;
      tiles_m = mg_cnt / p.tiles_n;
    } else if (MODE == MODE_MASKED || MODE == MODE_KGROUP) {
      const int per = p.tiles_m * p.tiles_n;
      g = t / per;
      tl = t - g * per;
    }
    if (MODE == MODE_KGROUP) {
      // the group's K blocks: after those of the groups before it; counts are
      // rounded down to whole blocks and cut at K (malformed device data stays in
      // bounds).  A group without K rows has no tiles (its D is zeroed apart).
      int kb_start = 0;
      for (int h = 0; h < g; ++h) kb_start += max(p.ks[h], 0) >> 7;
      const int nkb = kb_start < KB ? min(max(p.ks[g], 0) >> 7, KB - kb_start) : 0;
      if (nkb == 0) return false;
      tile.kb0 = kb_start;
      tile.nkb = nkb;
    }
    int tm, tn;
    raster_tile(tl, tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    tile.m0 = tm * BM;
    tile.n0 = tn * BN;
    tile.rot = (tile.part >= 0 || MODE == MODE_KGROUP) ? 0 : (p.k_rot * ((tm + tn) & 7)) % KB;
    tile.rows_valid = M;
    if (MODE == MODE_MASKED) {
      const int mm = p.masked_m[g];
      tile.rows_valid = mm < 0 ? 0 : (mm > M ? M : mm);
      if (tile.m0 >= tile.rows_valid) return false;  // empty tile
    }
    if (MODE == MODE_CONTIG) {
      g = p.m_indices[tile.m0];
      if (g < 0 || g >= p.num_groups) return false;  // padding block
    }
    tile.g = g;
    return true;
  };
  // first tile at or after t with work (all lanes agree: every input is uniform)
  auto next_tile = [&](int& t, Tile& tile) -> bool {
    for (; t < total_units; t += G)
      if (decode(t, tile)) return true;
    return false;
  };

  // ---------------- per-tile DMA state ----------------
  // Buffer resources (SGPRs) for A, B and the A scales of the tile's group; each
  // lane keeps one 32-bit offset per DMA region and the K block advances the
  // scalar offset, so the loop needs no 64-bit address arithmetic.
  v4i rsA, rsB, rsSA;
  cfloat* const SBc = (cfloat*)(uintptr_t)p.sfb;   // constant address space: scalar loads
  typedef const __attribute__((address_space(4))) uint32_t cword;
  cword* const SBw = (cword*)(uintptr_t)p.sfb;      // the same, packed UE8M0 words
  uint32_t a_off[RA], b_off[RB], sa_off = 0;
  // contiguous form: group index of the row of each of the lane's D stores,
  // loaded when the tile is set up and compared after its K loop, when no load
  // is outstanding any more (a later first use would wait for the next tile's
  // copies, issued after these loads)
  int midx[NSTD];
  int rot = 0, kb0_d = 0, nkb_d = 1;   // K range and rotation of the tile whose loads are issued
  int sb_idx = 0;
  auto setup = [&](const Tile& tile) {
    const uint8_t* A = p.a;
    // A scales: fp32 [groups][KB][M], or packed UE8M0 words [groups][M][KW]
    const uint8_t* SA = static_cast<const uint8_t*>(p.sfa);
    const uint8_t* B = p.b;
    const uint32_t sa_bytes = UE ? (uint32_t)M * (uint32_t)KW * 4u : (uint32_t)KB * (uint32_t)M * 4u;
    if (MODE == MODE_MASKED) {
      A += (size_t)tile.g * M * K;
      SA += (size_t)tile.g * sa_bytes;
    }
    if (MODE == MODE_CONTIG || MODE == MODE_MASKED) B += (size_t)tile.g * N * K;   // (K-grouped: one B)
    rot = tile.rot;
    kb0_d = tile.kb0;
    nkb_d = tile.nkb;
    rsA = make_buffer_rsrc(A, (uint32_t)M * (uint32_t)K);
    rsB = make_buffer_rsrc(B, (uint32_t)N * (uint32_t)K);
    rsSA = make_buffer_rsrc(SA, sa_bytes);
    // Region r covers tile rows 8r..8r+7; lane l fills LDS bytes [16l, 16l+16)
    // of it: row 8r + l/8, position l%8, which holds chunk (l%8) ^ swz(row).
    // Rows past the valid ones (ragged edges, masked-off rows) take an
    // out-of-range offset: the copy then reads zeros without a memory request,
    // and their results are never stored.
#pragma unroll
    for (int j = 0; j < RA; ++j) {
      const int row = (wave * RA + j) * 8 + dma_row;
      if constexpr (AT) {   // as B in the NN layout: sub-tile row / 128, K row row % 128
        const int krow = row & 127;
        const int col = tile.m0 + (row >> 7) * 128 + (((lane & 7) ^ kt_swz(krow)) << 4);
        a_off[j] = col < tile.rows_valid ? (uint32_t)krow * (uint32_t)M + (uint32_t)col : kBufferOutOfRange;
      } else {
        a_off[j] = tile.m0 + row < tile.rows_valid
                       ? (uint32_t)(tile.m0 + row) * (uint32_t)K + (((lane & 7) ^ swz(row)) << 4)
                       : kBufferOutOfRange;
      }
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = (wave * RB + j) * 8 + dma_row;
      if constexpr (NN) {
        // region q = row / 8: column sub-tile q / 16, K rows 8 (q % 16) ..; position
        // lane % 8 holds chunk (lane % 8) ^ kt_swz(K row) of the sub-tile's 128 columns
        const int krow = row & 127;
        const int col = tile.n0 + (row >> 7) * 128 + (((lane & 7) ^ kt_swz(krow)) << 4);
        b_off[j] = col < N ? (uint32_t)krow * (uint32_t)N + (uint32_t)col : kBufferOutOfRange;
      } else {
        b_off[j] = tile.n0 + row < N ? (uint32_t)(tile.n0 + row) * (uint32_t)K + (((lane & 7) ^ swz(row)) << 4)
                                     : kBufferOutOfRange;
      }
    }
    {
      // LDS position q of a tile's A scales holds row g*MT*16 + mt*16 + r for
      // q = g*MT*16 + r*MT + mt, so the MT scales a lane needs are adjacent
      const int q = wave * SPW + (lane < SPW ? lane : 0);
      const int g = q / (MT * 16), rem = q % (MT * 16);
      const int row = g * (MT * 16) + (rem % MT) * 16 + rem / MT;
      sa_off = tile.m0 + row < tile.rows_valid ? (uint32_t)(tile.m0 + row) * (UE ? (uint32_t)KW * 4u : 4u)
                                               : kBufferOutOfRange;
    }
    // B-scale element offsets from the kernel argument p.sfb, kept in SGPRs so the
    // per-K-block reads are scalar loads (which vmcnt does not count)
    const int sb_row = UE ? KW : KB;   // scale entries per 128-row block of B
    const int sb_group = (MODE == MODE_CONTIG || MODE == MODE_MASKED) ? tile.g * NB * sb_row : 0;
    sb_idx = __builtin_amdgcn_readfirstlane(sb_group + (min(tile.n0 + wave_n * NT * 16, N - 1) >> 7) * sb_row);
    if constexpr (MODE == MODE_CONTIG) {
#pragma unroll
      for (int j = 0; j < NSTD; ++j) midx[j] = p.m_indices[min(tile.m0 + ((j * NW + wave) * 64 + lane) / CPR, M - 1)];
    }
  };
  auto issue = [&](int kb, uint32_t slot_off) {
    const int kp = __builtin_amdgcn_readfirstlane(kb0_d + (kb + rot < nkb_d ? kb + rot : kb + rot - nkb_d));   // K block in memory
    const uint32_t kofs = (uint32_t)kp * 128u;
    const uint32_t kofs_b = NN ? (uint32_t)kp * 128u * (uint32_t)N : kofs;   // NN: 128 rows of B down
    const uint32_t kofs_a = AT ? (uint32_t)kp * 128u * (uint32_t)M : kofs;
    const uint32_t sofs = UE ? (uint32_t)(kp >> 2) * 4u : (uint32_t)kp * (uint32_t)M * 4u;
#pragma unroll
    for (int j = 0; j < RA; ++j) buf16_to_lds(rsA, a_off[j], kofs_a, smem + slot_off + a_dst + j * 1024);
#pragma unroll
    for (int j = 0; j < RB; ++j) buf16_to_lds(rsB, b_off[j], kofs_b, smem + slot_off + b_dst + j * 1024);
    if (SPW == 64 || lane < SPW) buf4_to_lds(rsSA, sa_off, sofs, smem + slot_off + sa_dst);
  };
  // The same copies one instruction at a time (idx < RA: A region idx, then the
  // B regions), so that a K block's copies can be spread between its matrix
  // instructions; the row-scale copy (issue_sa) goes first.
  auto issue_ab = [&](int idx, int kb, uint32_t slot_off) {
    const int kp = __builtin_amdgcn_readfirstlane(kb0_d + (kb + rot < nkb_d ? kb + rot : kb + rot - nkb_d));
    const uint32_t kofs = (uint32_t)kp * 128u;
    const uint32_t kofs_b = NN ? (uint32_t)kp * 128u * (uint32_t)N : kofs;
    const uint32_t kofs_a = AT ? (uint32_t)kp * 128u * (uint32_t)M : kofs;
#pragma unroll
    for (int j = 0; j < RA; ++j)
      if (idx == j) buf16_to_lds(rsA, a_off[j], kofs_a, smem + slot_off + a_dst + j * 1024);
#pragma unroll
    for (int j = 0; j < RB; ++j)
      if (idx == RA + j) buf16_to_lds(rsB, b_off[j], kofs_b, smem + slot_off + b_dst + j * 1024);
  };
  auto issue_sa = [&](int kb, uint32_t slot_off) {
    const int kp = __builtin_amdgcn_readfirstlane(kb0_d + (kb + rot < nkb_d ? kb + rot : kb + rot - nkb_d));
    const uint32_t sofs = UE ? (uint32_t)(kp >> 2) * 4u : (uint32_t)kp * (uint32_t)M * 4u;
    if (SPW == 64 || lane < SPW) buf4_to_lds(rsSA, sa_off, sofs, smem + slot_off + sa_dst);
  };
  // DMA of half h of the C tile into the slot at slot_off (dense form, whole
  // tiles only: a split tile's C is added when its slices are summed).
  const bool dense_c = MODE == MODE_DENSE && p.c != nullptr;
  bool has_c = false;   // the current tile copies C
  auto issue_c = [&](const Tile& tile, int h, uint32_t slot_off) {
    constexpr int RPI = 1024 / (BN * 2);             // C rows per 1-KB piece
    const v4i rsC = make_buffer_rsrc(p.c, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int q = wave * CPW + j;
      const int rr = h * (BM / 2) + q * RPI + lane / CPR;   // tile row
      const int c = (lane % CPR) ^ (rr & 15);                // C chunk this lane fetches
      const uint32_t off = tile.m0 + rr < M && tile.n0 + c * 8 < N
                               ? ((uint32_t)(tile.m0 + rr) * (uint32_t)N + (uint32_t)(tile.n0 + c * 8)) * 2u
                               : kBufferOutOfRange;
      buf16_to_lds(rsC, off, 0u, smem + slot_off + q * 1024);
    }
  };
  // Waits until stage kb of the ring has landed.  Operations of one wave retire
  // in issue order (loads and stores alike), so stage kb is complete once no
  // more remain than were issued after it: the stages kb+1.. already in flight,
  // the previous tile's stores while kb was a prologue stage (stores_after: 0
  // none, 1 its NSTD stores of D, 2 its NPART stores of a split partial), and
  // the first C half before the last block.
  auto wait_stage = [&](int kb, int KT, int stores_after) {
    const int after = min(STAGES - 2, KT - 1 - kb);
    const int st = kb <= STAGES - 2 ? stores_after : 0;
    const bool ch = STAGES >= 3 && has_c && KT >= 2 && kb == KT - 1;
    auto wait_plus = [&](auto loads_tag) {   // loads_tag: memory loads issued after stage kb
      constexpr int L = decltype(loads_tag)::value;
      if (st == 1) wait_vmcnt<L + NSTD>();
      else if (st == 2) wait_vmcnt<L + NPART>();
      else wait_vmcnt<L>();
    };
    if (STAGES >= 4 && after == 2) wait_plus(std::integral_constant<int, (STAGES >= 4 ? 2 : 0) * LPS>{});
    else if (after == 1) wait_plus(std::integral_constant<int, LPS>{});
    else if (ch) wait_plus(std::integral_constant<int, CPW>{});
    else wait_plus(std::integral_constant<int, 0>{});
  };
  // Stage s of a tile lives in ring slot (s0 + s) % STAGES; s0 moves from tile
  // to tile (the next tile starts in the slot of this tile's last K block).
  int s0 = 0;
  auto slot_of = [&](int i) -> uint32_t { return (uint32_t)(i % STAGES) * (uint32_t)STAGE; };
  // copies of stages [from, to) of the tile set up last
  auto prologue = [&](int from, int to) {
    if (!cw) return;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s >= from && s < to && s < nkb_d) issue(s, slot_of(s0 + s));
  };

  int t = vb;
  Tile cur;
  int stores_after = 0;   // the previous tile's stores issued after this tile's prologue (see wait_stage)
  bool have = next_tile(t, cur);
  if (have) {
    setup(cur);
    prologue(0, STAGES - 1);
  }
  while (have) {
    has_c = dense_c && cur.part < 0;
    v4f acc[MT][NT];       // fp32 accumulators
    v4f part[LAG];         // fresh partials, promoted LAG matrix instructions late
    float sprev = 0.f;     // sa * sb of the previous K block for the last row block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < LAG; ++r) part[r] = v4f{0.f, 0.f, 0.f, 0.f};

    const int KT = cur.nkb;                        // K blocks of this work unit
    const int kb0 = cur.kb0;
    uint32_t rd_slot = slot_of(s0);                // slot of stage kb
    uint32_t wr_slot = slot_of(s0 + STAGES - 1);   // slot of stage kb + STAGES - 1
    // One K block.  STEADY: a later stage is copied in this block, its copy
    // instructions spread between the matrix instructions (a copy that finds
    // the memory pipeline full then stalls the wave while matrix work is
    // queued, instead of before any is); otherwise the C tile may be copied.
    // COPY: the instance a copy wave runs (it issues the stage copies and waits
    // for them); the others only pass the barrier.
    auto kstep = [&](int kb, auto steady_tag, auto copy_tag) {
      constexpr bool COPY = decltype(copy_tag)::value;
      constexpr bool STEADY = decltype(steady_tag)::value && COPY;
      // copies spread over the block (not with streamed A fragments, whose
      // scheduling fences would split the pattern)
      constexpr int ILV = RA + RB;
      constexpr int ILV_STEP = NBLK / ILV > 0 ? NBLK / ILV : NBLK + 1;
      if constexpr (COPY) wait_stage(kb, KT, stores_after);
      block_barrier();
      if (STEADY) {
        issue_sa(kb + STAGES - 1, wr_slot);
        if (ILV_STEP * ILV > NBLK) {
#pragma unroll
          for (int idx = 0; idx < ILV; ++idx) issue_ab(idx, kb + STAGES - 1, wr_slot);
        }
      } else if (has_c) {
        // slot (s0 + KT + h) % STAGES takes half h: free from block KT - 2 + h on
        if (kb == KT - 1) {
          if (KT == 1) issue_c(cur, 0, slot_of(s0 + KT));
          issue_c(cur, 1, slot_of(s0 + KT + 1));
        } else if (kb == KT - 2) {
          issue_c(cur, 0, slot_of(s0 + KT));
        }
      }

      // K block in memory; the B scale of this block is one per wave (its
      // columns share a 128-wide block)
      // (uniform: kept in an SGPR so that the scale load stays scalar and the
      // copies' K offsets need no per-lane handling)
      const int kp = __builtin_amdgcn_readfirstlane(kb0 + (kb + rot < KT ? kb + rot : kb + rot - KT));
      const uint8_t* ra_lo = smem + rd_slot + a_lo;
      const uint8_t* ra_hi = smem + rd_slot + a_hi;
      const uint8_t* rb_lo = smem + rd_slot + b_lo;
      const uint8_t* rb_hi = smem + rd_slot + b_hi;
      const uint8_t* rsa = smem + rd_slot + sa_rd;
      float scur[MT];              // fp32 scales: sa * sb per row block
      int sab[MT], sbb = 0;        // UE8M0: the exponent bytes of this K block
      if constexpr (UE) {
        const int sh = (kp & 3) * 8;
        sbb = (int)((SBw[sb_idx + (kp >> 2)] >> sh) & 0xffu);
#pragma unroll
        for (int q = 0; q < MT / 4; ++q) {
          const v4i sav = *reinterpret_cast<const v4i*>(rsa + 16 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) sab[4 * q + i] = (int)(((uint32_t)sav[i] >> sh) & 0xffu);
        }
      } else {
        const float sbv = SBc[sb_idx + kp];
#pragma unroll
        for (int q = 0; q < MT / 4; ++q) {
          const v4f sav = *reinterpret_cast<const v4f*>(rsa + 16 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) scur[4 * q + i] = sav[i] * sbv;
        }
      }
      auto load_a = [&](int mt) -> v8i {
        if constexpr (AT) {   // transposing reads, as for B in the NN layout
          const int q = wave_m * MT + mt;   // row chunk (16 rows of D) of the tile
          const uint8_t* ra = smem + rd_slot + a_t_row + (q >> 3) * (128 * 128) + (((q & 7) ^ b_nn_sw) << 4);
          v2i r[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = ds_read_tr8_b64(ra + i * 1024);
          return v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(ra_lo + mt * 2048);
          const v4i hi = *reinterpret_cast<const v4i*>(ra_hi + mt * 2048);
          return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      };
      v8i af[MT], bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (NN) {
          const int q = wave_n * NT + nt;   // column chunk of the tile
          const uint8_t* rb = smem + rd_slot + b_nn_row + (q >> 3) * (128 * 128) + (((q & 7) ^ b_nn_sw) << 4);
          v2i r[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = ds_read_tr8_b64(rb + i * 1024);
          bf[nt] = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
        } else {
          v4i lo = *reinterpret_cast<const v4i*>(rb_lo + nt * 2048);
          v4i hi = *reinterpret_cast<const v4i*>(rb_hi + nt * 2048);
          bf[nt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) af[mt] = load_a(mt);
      // The wave computes its tile transposed: block (mt, nt) is B_nt . A_mt^T,
      // so a lane's four results share one row of D (column lrow of the block)
      // and one A scale.  Block j = mt*NT + nt goes into partial register j % LAG;
      // the register's previous partial is promoted first: for j < LAG the one
      // of block j + NBLK - LAG of the previous K block (scale sprev), else the
      // one of block j - LAG of this K block.  A partial is thus read LAG
      // matrix instructions after its issue, so the FMAs never wait on it.
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int j = mt * NT + nt;
          if constexpr (UE) {
            // the matrix core applies both exponents and accumulates in place
            acc[mt][nt] = mfma_scaled_e4m3_16x16x128(bf[nt], sbb, af[mt], sab[mt], acc[mt][nt]);
          } else {
            const int r = j % LAG;
            if (j < LAG) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[MT - 1][j + NT - LAG][i] = fmaf(part[r][i], sprev, acc[MT - 1][j + NT - LAG][i]);
            } else {
              const int pm = (j - LAG) / NT, pn = (j - LAG) % NT;
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[pm][pn][i] = fmaf(part[r][i], scur[pm], acc[pm][pn][i]);
            }
            part[r] = mfma_e4m3_16x16x128(bf[nt], af[mt], v4f{0.f, 0.f, 0.f, 0.f});
          }
          const bool copy_here = STEADY && ILV_STEP * ILV <= NBLK && j % ILV_STEP == ILV_STEP - 1 && j / ILV_STEP < ILV;
          if (copy_here) issue_ab(j / ILV_STEP, kb + STAGES - 1, wr_slot);
          // keep the schedule: the promotion FMAs of block j ride with its matrix
          // instruction, and a copy follows every ILV_STEP-th one
          if constexpr (!UE) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU (promotion)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
          if (copy_here) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 VMEM read (copy)
        }
      }
      if constexpr (!UE) sprev = scur[MT - 1];
      rd_slot = (rd_slot + STAGE == STAGES * STAGE) ? 0u : rd_slot + STAGE;
      wr_slot = (wr_slot + STAGE == STAGES * STAGE) ? 0u : wr_slot + STAGE;
    };
    int kb = 0;
    if (cw) {
#pragma clang loop unroll(disable)
      for (; kb + STAGES - 1 < KT; ++kb) kstep(kb, std::true_type{}, std::true_type{});
#pragma clang loop unroll(disable)
      for (; kb < KT; ++kb) kstep(kb, std::false_type{}, std::true_type{});
    } else {
#pragma clang loop unroll(disable)
      for (; kb < KT; ++kb) kstep(kb, std::false_type{}, std::false_type{});
    }
    // promote the last LAG partials (blocks NBLK - LAG .. NBLK - 1: row MT - 1)
    if constexpr (!UE) {
#pragma unroll
      for (int j = 0; j < LAG; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[MT - 1][NT - LAG + j][i] = fmaf(part[(NBLK - LAG + j) % LAG][i], sprev, acc[MT - 1][NT - LAG + j][i]);
    }
    const Tile done = cur;
    const int c_base = s0 + KT;   // C half h sits in slot (c_base + h) % STAGES

    // The next tile's loads start before this tile's epilogue.  Once every wave
    // has read the last K block, the ring is free but for the two C slots: the
    // next tile's stage 0 goes into the last block's slot and lands while this
    // tile waits for C; its later stages follow once C has been read.  Without
    // C they all go at once.
    uint32_t grp_ok = ~0u;   // contiguous form: bit j, the row of store j is in the tile's group
    if constexpr (MODE == MODE_CONTIG) {
      grp_ok = 0;
#pragma unroll
      for (int j = 0; j < NSTD; ++j) grp_ok |= (midx[j] == done.g ? 1u : 0u) << j;
    }
    t += G;
    have = next_tile(t, cur);
    wait_lgkmcnt0();
    block_barrier();   // every wave is done with the last K block
    const bool whole = done.part < 0;   // D is staged in the C slots (a split slice stores its partial)
    if (have) {
      setup(cur);
      s0 = __builtin_amdgcn_readfirstlane((c_base + STAGES - 1) % STAGES);
      prologue(0, whole ? 1 : STAGES - 1);
    }

    // Epilogue, part 1: D = acc (+ C) rounded to bf16, written over C in LDS.
    // Lane (lgrp, lrow) holds, for block (mt, nt), row mt*16 + lrow and the four
    // columns nt*16 + 4*lgrp .. +3 of the wave's sub-tile: 8 bytes of one row,
    // at the place of the same 8 bytes of C.
    if (has_c) {
      // this wave's C pieces have landed: only the next tile's stage 0 (LPS
      // copies, every tile has at least one K block) was issued after them
      if (have && cw) wait_vmcnt<LPS>();
      else wait_vmcnt<0>();
      block_barrier();   // ... and every other wave's
    }
    // (a split tile's slice stores its fp32 partial instead, below)
#pragma unroll
    for (int mt = 0; mt < (whole ? MT : 0); ++mt) {
      const int rr0 = wave_m * MT * 16 + mt * 16;       // first tile row of the block
      const int h = rr0 >= BM / 2 ? 1 : 0;
      const uint32_t c_row = slot_of(c_base + h) + (uint32_t)(rr0 - h * (BM / 2) + lrow) * (BN * 2) +
                             (uint32_t)((lgrp & 1) << 3);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const v4f v = acc[mt][nt];
        float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
        const int c = (wave_n * NT * 16 + nt * 16 + 4 * lgrp) >> 3;   // chunk; tile row % 16 is lrow
        uint2* const cd = reinterpret_cast<uint2*>(smem + c_row + ((c ^ lrow) << 4));
        if (has_c) {
          const uint2 cv = *cd;
          v0 += __uint_as_float(cv.x << 16);
          v1 += __uint_as_float(cv.x & 0xffff0000u);
          v2 += __uint_as_float(cv.y << 16);
          v3 += __uint_as_float(cv.y & 0xffff0000u);
        }
        *cd = make_uint2(pack_bf16x2_rne(v0, v1), pack_bf16x2_rne(v2, v3));
      }
    }
    if (!whole) {
      // split K: this slice's fp32 partial tile (BM x BN, row-major) goes to
      // workspace tile `part`, 4 consecutive columns = 16 bytes per lane and
      // block.  Rows and columns beyond D are stored too and never read.
      const v4i rsW = make_buffer_rsrc(p.ws + (size_t)done.part * (BM * BN), (uint32_t)(BM * BN * 4));
      const uint32_t off0 = (uint32_t)((wave_m * MT * 16 + lrow) * BN + wave_n * NT * 16 + 4 * lgrp) * 4u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const v4i w = {__float_as_int(acc[mt][nt][0]), __float_as_int(acc[mt][nt][1]),
                         __float_as_int(acc[mt][nt][2]), __float_as_int(acc[mt][nt][3])};
          dg_raw_buffer_store_v4i32(w, rsW, (int)(off0 + (uint32_t)(mt * 16 * BN + nt * 16) * 4u), 0, 0);
        }
      }
    }
    // This tile's stores (D, or a split slice's fp32 partial) follow the next
    // tile's prologue and drain while it computes its first blocks.
    stores_after = whole ? 1 : 2;
    if (!whole) continue;

    // Epilogue, part 2: the staged D, read back as whole rows (16-byte chunk c
    // of tile row rr by one lane; CPR lanes cover a row), then the rest of the
    // next tile's prologue into the freed slots, then exactly NSTD 16-byte
    // stores per wave; masked-off chunks go to an out-of-range offset.
    wait_lgkmcnt0();
    block_barrier();   // D staged by every wave
    v4i dv[NSTD];
#pragma unroll
    for (int j = 0; j < NSTD; ++j) {
      const int idx = (j * NW + wave) * 64 + lane;
      const int rr = idx / CPR, c = idx % CPR;
      const int h = rr >= BM / 2 ? 1 : 0;
      dv[j] = *reinterpret_cast<const v4i*>(smem + slot_of(c_base + h) + (uint32_t)(rr - h * (BM / 2)) * (BN * 2) +
                                            (uint32_t)((c ^ (rr & 15)) << 4));
    }
    wait_lgkmcnt0();
    block_barrier();   // every wave has read D: the C slots are free
    if (have) prologue(1, STAGES - 1);
    const uint16_t* D = p.d;
    if (MODE == MODE_MASKED || MODE == MODE_KGROUP) D += (size_t)done.g * M * N;
    const v4i rsD = make_buffer_rsrc(D, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
    for (int j = 0; j < NSTD; ++j) {
      const int idx = (j * NW + wave) * 64 + lane;
      const int grow = done.m0 + idx / CPR, gcol = done.n0 + (idx % CPR) * 8;
      const bool ok = grow < done.rows_valid && gcol < N && ((grp_ok >> j) & 1u);
      const uint32_t off = ok ? ((uint32_t)grow * (uint32_t)N + (uint32_t)gcol) * 2u : kBufferOutOfRange;
      dg_raw_buffer_store_v4i32(dv[j], rsD, (int)off, 0, kStoreNonTemporal);
    }
  }
}

// split K: 8 consecutive fp32 columns of one row summed over the slices in
// slice order (slice s at w + s * stride4 float4s).  The loads of four slices
// are issued before any is added: one load at a time left the reduce bound by
// memory latency.
__device__ __forceinline__ void sum_slices(const float4* w, int splits, size_t stride4, float4& lo, float4& hi) {
  lo = w[0];
  hi = w[1];
  int s = 1;
  for (; s + 4 <= splits; s += 4) {
    float4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = w[(s + u) * stride4];
      b[u] = w[(s + u) * stride4 + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lo.x += a[u].x; lo.y += a[u].y; lo.z += a[u].z; lo.w += a[u].w;
      hi.x += b[u].x; hi.y += b[u].y; hi.z += b[u].z; hi.w += b[u].w;
    }
  }
  for (; s < splits; ++s) {
    const float4 a = w[s * stride4], b = w[s * stride4 + 1];
    lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
    hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
  }
}

// ---------------------------------------------------------------------------
// split K: for every split tile, the sum of its slices' fp32 partials (in slice
// order), plus C, rounded to bf16
// ---------------------------------------------------------------------------
// One thread per 8 consecutive columns of one row of a split tile.  Split tile
// i (raster tile full_tiles + i) keeps slice s at workspace tile i * splits + s,
// each bm x bn fp32, row-major.  Contiguous form (m_indices given): a padding
// block's tile was never computed and rows of other groups are not written.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws,
                                                            const uint16_t* __restrict__ c, uint16_t* d, int m,
                                                            int n, int splits, int full_tiles, int split_tiles,
                                                            int bm, int bn, int tiles_m, int tiles_n, int group_m,
                                                            const int32_t* __restrict__ m_indices, int groups) {
  const int per_row = bn / 8;
  const long long per_tile = (long long)bm * per_row;
  const long long total = per_tile * split_tiles;
  const size_t tile_elems = (size_t)bm * bn;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int st = (int)(i / per_tile);
    const int q = (int)(i - (long long)st * per_tile);
    const int r = q / per_row, c8 = q - r * per_row;
    int tm, tn;
    raster_tile(full_tiles + st, tiles_m, tiles_n, group_m, &tm, &tn);
    const int row = tm * bm + r, col = tn * bn + c8 * 8;
    if (row >= m || col >= n) continue;
    if (m_indices) {
      const int g = m_indices[tm * bm];
      if (g < 0 || g >= groups || m_indices[row] != g) continue;
    }
    const float4* w = reinterpret_cast<const float4*>(ws + (size_t)st * splits * tile_elems + (size_t)r * bn + c8 * 8);
    float4 lo, hi;
    sum_slices(w, splits, tile_elems / 4, lo, hi);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const size_t o8 = ((size_t)row * n + col) / 8;   // n % 16 == 0: 16-byte aligned
    if (c) {
      const uint4 cv = reinterpret_cast<const uint4*>(c)[o8];
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] += __uint_as_float(cw[j] << 16);
        v[2 * j + 1] += __uint_as_float(cw[j] & 0xffff0000u);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2_rne(v[2 * j], v[2 * j + 1]);
    reinterpret_cast<uint4*>(d)[o8] = uint4{o[0], o[1], o[2], o[3]};
  }
}

hipError_t launch_splitk_reduce(const Fp8GemmParams& p, const GemmPlan& plan, int num_cus, hipStream_t stream) {
  const int split_tiles = plan.num_tiles - plan.full_tiles;
  const long long threads = (long long)plan.block_m * (plan.block_n / 8) * split_tiles;
  const int grid = (int)std::min<long long>((threads + 255) / 256, (long long)num_cus * 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, stream, p.ws, p.c, p.d, p.m, p.n, plan.splits,
                     plan.full_tiles, split_tiles, plan.block_m, plan.block_n, p.tiles_m, p.tiles_n, p.group_m,
                     p.m_indices, p.num_groups);
  return hipGetLastError();
}

// Masked form, device-planned: the same plan as the GEMM kernel (valid tiles
// of all groups in group order, split rule over their count on `slots`
// workgroups).  Work item = 8 rows of one split tile (one thread per 8
// columns for bn = 256), so a split tile's partials are summed by many
// workgroups at once.
__global__ void __launch_bounds__(256) masked_splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* d,
                                                                   const int32_t* __restrict__ masked_m,
                                                                   int groups, int max_m, int n, int kb, int bm,
                                                                   int bn, int tiles_n, int group_m, int slots) {
  const int tiles = masked_total_tiles(masked_m, groups, max_m, bm, tiles_n);
  long long full = tiles;
  const int splits = split_rule(tiles, slots, kb, &full);
  if (splits <= 1) return;
  const int split_tiles = tiles - (int)full;
  const int per_row = bn / 8;
  const int rows_per_item = 256 / per_row;
  const int items_per_tile = bm / rows_per_item;
  const size_t tile_elems = (size_t)bm * bn;
  int mg = 0, base = 0, cnt = masked_group_tiles(masked_m, 0, max_m, bm, tiles_n);
  for (int it = blockIdx.x; it < split_tiles * items_per_tile; it += gridDim.x) {
    const int st = it / items_per_tile;
    const int t = (int)full + st;
    while (t >= base + cnt) {
      base += cnt;
      cnt = masked_group_tiles(masked_m, ++mg, max_m, bm, tiles_n);
    }
    int tm, tn;
    raster_tile(t - base, cnt / tiles_n, tiles_n, group_m, &tm, &tn);
    int mm = masked_m[mg];
    mm = mm < 0 ? 0 : (mm > max_m ? max_m : mm);
    const int r = (it - st * items_per_tile) * rows_per_item + (int)threadIdx.x / per_row;
    const int c8 = (int)threadIdx.x % per_row;
    const int row = tm * bm + r, col = tn * bn + c8 * 8;
    if (r >= bm || row >= mm || col >= n) continue;
    const float4* w = reinterpret_cast<const float4*>(ws + (size_t)st * splits * tile_elems + (size_t)r * bn + c8 * 8);
    float4 lo, hi;
    sum_slices(w, splits, tile_elems / 4, lo, hi);
    const uint4 o = {pack_bf16x2_rne(lo.x, lo.y), pack_bf16x2_rne(lo.z, lo.w), pack_bf16x2_rne(hi.x, hi.y),
                     pack_bf16x2_rne(hi.z, hi.w)};
    uint16_t* dg = d + (size_t)mg * max_m * n;
    reinterpret_cast<uint4*>(dg)[((size_t)row * n + col) / 8] = o;
  }
}

// K-grouped form: the GEMM has no tiles for a group without K rows, whose D is
// zero; this writes it (groups with K rows return at once).  Same rounding and
// cut of the counts as the GEMM's decode.
__global__ void __launch_bounds__(256) kgroup_zero_kernel(const int32_t* __restrict__ ks, uint16_t* d, int m, int n,
                                                          int kb_total) {
  const int g = blockIdx.y;
  int kb_start = 0;
  for (int h = 0; h < g; ++h) kb_start += max(ks[h], 0) >> 7;
  const int nkb = kb_start < kb_total ? min(max(ks[g], 0) >> 7, kb_total - kb_start) : 0;
  if (nkb > 0) return;
  uint4* dg = reinterpret_cast<uint4*>(d + (size_t)g * m * n);
  const size_t vecs = (size_t)m * n / 8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < vecs; i += (size_t)gridDim.x * 256)
    dg[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_kgroup_zero(const Fp8GemmParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kgroup_zero_kernel, dim3(64, p.num_groups), dim3(256), 0, stream, p.ks, p.d, p.m, p.n,
                     p.k / 128);
  return hipGetLastError();
}

hipError_t launch_masked_splitk_reduce(const Fp8GemmParams& p, const GemmPlan& plan, int slots, hipStream_t stream) {
  hipLaunchKernelGGL(masked_splitk_reduce_kernel, dim3(slots), dim3(256), 0, stream, p.ws, p.d, p.masked_m,
                     p.num_groups, p.m, p.n, p.k / 128, plan.block_m, plan.block_n, p.tiles_n, p.group_m, slots);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tile-config table and launcher
// ---------------------------------------------------------------------------

// id, MT, NT, WM, WN, STAGES, workgroups per CU.  Every shape runs eight waves,
// two per SIMD, so that one wave's LDS waits and barrier are covered by the other
// wave's matrix instructions (measured: the 128x128 and 64x128 shapes ran 15-20 %
// and up to 9 % slower as four waves of twice the width).
#define DG_TILE_CONFIGS(X)    \
  X(0, 4, 4, 4, 2, 3, 1)      \
  X(1, 4, 4, 2, 4, 3, 1)      \
  X(2, 4, 2, 2, 4, 3, 1)      \
  X(3, 4, 1, 1, 8, 4, 1)

static const TileConfig kTileConfigs[] = {
#define X(id, MT, NT, WM, WN, ST, OCC) {WM * MT * 16, WN * NT * 16, OCC, WM * WN * 64,                     \
                                        ST * ((WM * MT * 16 + WN * NT * 16) * 128 + WM * MT * 16 * 4), ST},
    DG_TILE_CONFIGS(X)
#undef X
};

// ids 0-3: this file's template; ids 4-6: the 256x256, 128x512 and 256x224 tiles of fp8_gemm_wide.hip
int num_tile_configs() { return (int)(sizeof(kTileConfigs) / sizeof(kTileConfigs[0])) + 3; }
TileConfig tile_config(int id) { return is_wide_tile(id) ? wide_tile_config(id) : kTileConfigs[id]; }

template <int MODE>
static hipError_t launch_mode(const Fp8GemmParams& p, int kernel_id, int grid, hipStream_t stream) {
  switch (kernel_id) {
#define X(id, MT, NT, WM, WN, ST, OCC)                                                              \
  case id: {                                                                                      \
    if constexpr (((MODE & MODE_NN) != 0 && (WN * NT * 16) % 128 != 0) ||                           \
                  ((MODE & MODE_AT) != 0 && (WM * MT * 16) % 128 != 0))                             \
      return hipErrorInvalidValue;                                                                \
    else {                                                                                        \
    const TileConfig& tc = kTileConfigs[id];                                                      \
    static const hipError_t attr = hipFuncSetAttribute(                                           \
        reinterpret_cast<const void*>(&fp8_gemm_kernel<MT, NT, WM, WN, ST, MODE>),                \
        hipFuncAttributeMaxDynamicSharedMemorySize, tc.lds_bytes);                                \
    if (attr != hipSuccess) return attr;                                                          \
    hipLaunchKernelGGL((fp8_gemm_kernel<MT, NT, WM, WN, ST, MODE>), dim3(grid), dim3(tc.threads), \
                       tc.lds_bytes, stream, p);                                                  \
    break;                                                                                        \
    }                                                                                             \
  }
    DG_TILE_CONFIGS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const Fp8GemmParams& p, const GemmPlan& plan, int mode, hipStream_t stream) {
  if (plan.num_workgroups <= 0) return hipSuccess;
  const int g = plan.num_workgroups, id = plan.kernel_id;
  if (is_wide_tile(id)) return launch_fp8_gemm_wide(p, id, mode, g, stream);
  switch (mode) {
    case MODE_DENSE: return launch_mode<MODE_DENSE>(p, id, g, stream);
    case MODE_CONTIG: return launch_mode<MODE_CONTIG>(p, id, g, stream);
    case MODE_MASKED: return launch_mode<MODE_MASKED>(p, id, g, stream);
    case MODE_DENSE | MODE_UE8M0: return launch_mode<MODE_DENSE | MODE_UE8M0>(p, id, g, stream);
    case MODE_CONTIG | MODE_UE8M0: return launch_mode<MODE_CONTIG | MODE_UE8M0>(p, id, g, stream);
    case MODE_MASKED | MODE_UE8M0: return launch_mode<MODE_MASKED | MODE_UE8M0>(p, id, g, stream);
    case MODE_DENSE | MODE_NN: return launch_mode<MODE_DENSE | MODE_NN>(p, id, g, stream);
    case MODE_CONTIG | MODE_NN: return launch_mode<MODE_CONTIG | MODE_NN>(p, id, g, stream);
    case MODE_DENSE | MODE_AT | MODE_NN: return launch_mode<MODE_DENSE | MODE_AT | MODE_NN>(p, id, g, stream);
    case MODE_DENSE | MODE_AT: return launch_mode<MODE_DENSE | MODE_AT>(p, id, g, stream);
    case MODE_KGROUP | MODE_AT | MODE_NN: return launch_mode<MODE_KGROUP | MODE_AT | MODE_NN>(p, id, g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
