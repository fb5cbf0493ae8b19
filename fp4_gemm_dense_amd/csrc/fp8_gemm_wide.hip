// Fine-grained-scaled FP8 GEMM for gfx950 on wide tiles: D = C + A.B^T (NT),
// fp32 scales, bf16 out.  Three tiles: 256x256 and 256x224 (dense form) and
// 128x512 (dense and M-grouped contiguous forms), for problems large enough to
// fill the chip with them.
//
// What is computed is the dense GEMM of the usage guide ("DeepGEMM：统一高性能张量
// 核心 GEMM 计算库编译与使用指南", 五、使用方法) and its M-grouped contiguous form,
// with the two-level accumulation of the release article ("DeepSeek 开源第三弹 ...
// DeepGEMM", DeepGEMM section): one matrix instruction per 128-wide K block into
// a fresh fp32 partial, promoted on the vector ALUs by sa * sb -- exactly as the
// tiles of fp8_gemm.hip, in the same per-element order.
//
// Why a second kernel: every K block of a tile is copied from L2 into LDS by
// LDS-DMA loads, and on gfx950 the copy path (texture address unit, LDS writes)
// and the matrix cores are both about half busy on the 128x256 tile, which moves
// 48 KB per 16 matrix instructions per wave.  A 256x256 tile moves 64 KB per 32:
// a third fewer copy bytes and a quarter fewer LDS fragment bytes per matrix
// instruction, half the barriers per instruction.  Its price is the LDS: a stage
// is 65 KB (80 KB for 128x512), so the ring has two slots, and the stage copies
// of K block kb + 1 are issued right after block kb's barrier (one block of
// lead).
//   * 8 waves, each a 64 x 128 (64 x 112) sub-tile of 16x16 blocks (MT = 4 row
//     blocks, NT = 8 or 7 column blocks), computed transposed (B_nt . A_mt^T) so
//     that a lane's four results lie in one row of D and share one A scale;
//   * the four A fragments of a K block are read once, the B fragments one at a
//     time, each feeding four matrix instructions (the register file holds 128
//     accumulators per lane, which the promotion FMAs need in VGPRs);
//   * tile boundaries: the next unit's first stage is copied during this unit's
//     last K block (or, with C, right after it, the last block copying half of
//     C instead); D leaves through a free LDS slot half a tile at a time, as
//     bf16 (plus C, staged there in the same layout), and is stored from there
//     in whole rows (1024 bytes per store instruction).
//   * split K (a partial last round) writes fp32 partial tiles to the caller's
//     workspace, summed by the split-K reduce kernel of fp8_gemm.hip.
#include <algorithm>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

namespace {
// The value x, opaque to the compiler: expressions of it are evaluated where
// they are written.  Lane-dependent offsets that are needed only at a tile's
// edges are derived from an opaque lane id there, so that the compiler cannot
// hoist them out of the loops and hold them in registers through the K loop,
// whose working set (accumulators, fragments, partials) fills the register file.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

extern "C" __device__ int dg_raw_buffer_load_i32(v4i rsrc, int voffset, int soffset,
                                                 int aux) __asm("llvm.amdgcn.raw.buffer.load.i32");

constexpr int W_MT = 4, W_NW = 8;   // a wave: 64 rows (4 blocks of 16) of the tile; eight waves
constexpr int W_LAG = 4;        // matrix instructions between a partial's issue and its promotion
constexpr int W_CPH = 8;        // copy (and store) instructions per wave per half tile of C or D

// The tile shapes: 256 x 256 (4 x 2 waves of 64 x 128), 128 x 512 (2 x 4 waves
// of 64 x 128) and 256 x 224 (4 x 2 waves of 64 x 112).  A stage holds the A and
// B tiles of one K block (and, for 256 rows, the A scales); two stages fill 130
// KB or all 160 KB of LDS, so for 128 rows the A scales of the next K block are
// loaded into a register instead (one row per lane) and handed to the lanes that
// need them by cross-lane reads.  The 224-wide tile copies and stages B and D as
// if 256 wide (rows and columns past 224 read and write nothing); a wave's 112
// columns may span two 128-column blocks of B scales.
template <int BM, int BN_>
struct WideShape {
  static constexpr int BN = BN_;
  static constexpr int WN = BN == 512 ? 4 : 2, WM = W_NW / WN;   // waves along N and M
  static constexpr int WC = BN / WN, NT = WC / 16;               // a wave's columns and 16-column blocks
  static constexpr int BNP = BN == 224 ? 256 : BN;               // B rows copied, D columns staged
  static constexpr int RA = BM / 64, RB = BNP / 64;              // 1-KB copy regions of A, B per wave per stage
  static constexpr bool SA_LDS = BM == 256;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BNP * 128, SA_BYTES = SA_LDS ? BM * 4 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int LPS = RA + RB + 1;                        // memory instructions per wave per stage
  static constexpr int ROWB = BNP * 2;                           // bytes of a staged C / D row
  static constexpr int RPC = 1024 / ROWB;                        // staged rows per copy instruction
  static constexpr bool SPLIT_SB = WC % 128 != 0;                // a wave's columns may span two scale blocks
  static_assert(LDS <= 160 * 1024 && LPS <= W_MT * NT && WC % 16 == 0, "tile shape");
};
}  // namespace

// MODE: MODE_DENSE (C optional) or, for 128 rows, MODE_CONTIG (groups of rows
// padded to 128, each with its own B; no C).
template <int BM, int BN, int MODE>
__global__ void __launch_bounds__(512, 1) fp8_gemm_wide_kernel(Fp8GemmParams p) {
  using S = WideShape<BM, BN>;
  constexpr int WN = S::WN, WC = S::WC, NT = S::NT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef const __attribute__((address_space(4))) float cfloat;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / WN, wave_n = wave % WN;
  const int M = p.m, N = p.n, K = p.k;
  const int KB = K >> 7;

  // XCD-aware remap of the persistent block id (workgroups are dealt to the 8
  // XCDs round-robin; XCD x takes a contiguous stretch of the raster)
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Work units: [0, full_tiles) whole tiles; then unit full_tiles + u is K slice
  // u % splits of tile full_tiles + u / splits.  Contiguous form: a tile whose
  // first row is padding (group index out of range) is skipped.
  struct Unit {
    int m0, n0, kb0, nkb, part, g;
  };
  auto decode = [&](int t, Unit& w) -> bool {
    w.kb0 = 0;
    w.nkb = KB;
    w.part = -1;
    if (p.splits > 1 && t >= p.full_tiles) {
      const int u = t - p.full_tiles;
      w.kb0 = (u % p.splits) * p.kb_per_split;
      w.nkb = min(p.kb_per_split, KB - w.kb0);
      w.part = u;
      t = p.full_tiles + u / p.splits;
    }
    int tm, tn;
    raster_tile(t, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    w.m0 = tm * BM;
    w.n0 = tn * BN;
    w.g = 0;
    if constexpr (MODE == MODE_CONTIG) {
      w.g = p.m_indices[w.m0];
      if (w.g < 0 || w.g >= p.num_groups) return false;
    }
    return true;
  };
  // the first unit at or after t with work
  auto next_unit = [&](int& t, Unit& w) -> bool {
    for (; t < p.total_tiles; t += G)
      if (decode(t, w)) return true;
    return false;
  };

  const v4i rsA = make_buffer_rsrc(p.a, (uint32_t)M * (uint32_t)K);
  const v4i rsSA = make_buffer_rsrc(p.sfa, (uint32_t)KB * (uint32_t)M * 4u);
  cfloat* const SBc = (cfloat*)(uintptr_t)p.sfb;
  const int NB = (N + 127) >> 7;   // 128-column blocks of B scales per group

  // Per-lane copy offsets of the unit whose stages are being copied.  Region j of
  // a wave's A (B) copies covers tile rows 8 (RA wave + j) .. + 7 (RB for B);
  // lane l fills 16 bytes of row 8 (..) + l / 8 at position l % 8, which holds
  // chunk (l % 8) ^ swz(row).  swz depends on the row modulo 16 only, so regions
  // j and j + 2 (16 rows apart) share a lane's chunk and two offsets per operand
  // serve all regions.  A row past M (N) lies past the end of A (B): the
  // buffer's range check makes it read zeros (its results are never stored).
  // Row scales, 256 rows: position q = g * 64 + r * 4 + mt of the slot's scale
  // area holds row g * 64 + mt * 16 + r, so a lane's four scales are adjacent;
  // waves w and w + 4 copy the same 64 positions (identical bytes), so that every
  // lane of every wave issues the same instructions.  128 rows: lane l loads the
  // scale of the wave's row l into a register (one coalesced load of 256 bytes);
  // a row past M reads another K block's scale or zero, harmlessly.
  uint32_t a_off[2], b_off[2], sa_off = 0;
  v4i rsB = make_buffer_rsrc(p.b, (uint32_t)N * (uint32_t)K);
  float sa_nx = 0.f;   // 128 rows: the scale of the lane's row in the next K block
  int cp_kb0 = 0;   // first K block of that unit
  auto setup_copies = [&](const Unit& w) {
    cp_kb0 = w.kb0;
    if constexpr (MODE == MODE_CONTIG)
      rsB = make_buffer_rsrc(p.b + (size_t)w.g * (size_t)N * (size_t)K, (uint32_t)N * (uint32_t)K);
    const int ln = opaque(lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ra = (wave * S::RA + e) * 8 + (ln >> 3), rb = (wave * S::RB + e) * 8 + (ln >> 3);
      a_off[e] = (uint32_t)(w.m0 + ra) * (uint32_t)K + (uint32_t)(((ln & 7) ^ swz(ra)) << 4);
      b_off[e] = wave * S::RB * 8 < BN ? (uint32_t)(w.n0 + rb) * (uint32_t)K + (uint32_t)(((ln & 7) ^ swz(rb)) << 4)
                                       : kBufferOutOfRange;   // (224 wide: the last wave's rows are past the tile)
    }
    if constexpr (S::SA_LDS) {
      const int row = (wave & 3) * 64 + (ln & 3) * 16 + (ln >> 2);
      sa_off = w.m0 + row < M ? (uint32_t)(w.m0 + row) * 4u : kBufferOutOfRange;
    } else {
      sa_off = (uint32_t)(w.m0 + wave_m * 64 + ln) * 4u;
    }
  };
  // Memory instruction idx of stage s (within the unit's K range) of the unit
  // set up last, into the slot at byte offset slot: A regions, then B regions,
  // then the A scales (a copy into LDS, or a load into a register).
  auto issue = [&](int idx, int s, uint32_t slot) {
    const uint32_t kofs = (uint32_t)(cp_kb0 + s) * 128u;
    if (idx < S::RA) {
      const uint32_t off = a_off[idx & 1] + (uint32_t)(idx >> 1) * 16u * (uint32_t)K;
      buf16_to_lds(rsA, off, kofs, smem + slot + (wave * S::RA + idx) * 1024);
    } else if (idx < S::RA + S::RB) {
      const int j = idx - S::RA;
      const uint32_t off = b_off[j & 1] + (uint32_t)(j >> 1) * 16u * (uint32_t)K;
      buf16_to_lds(rsB, off, kofs, smem + slot + S::A_BYTES + (wave * S::RB + j) * 1024);
    } else if constexpr (S::SA_LDS) {
      buf4_to_lds(rsSA, sa_off, (uint32_t)(cp_kb0 + s) * (uint32_t)M * 4u,
                  smem + slot + S::A_BYTES + S::B_BYTES + (wave & 3) * 256);
    } else {
      sa_nx = __int_as_float(dg_raw_buffer_load_i32(rsSA, (int)sa_off, (int)((uint32_t)(cp_kb0 + s) * (uint32_t)M * 4u), 0));
    }
  };
  // C of a whole tile (dense form) is staged through a free LDS slot, half a
  // tile at a time: half h holds row blocks 2h and 2h + 1 of every wave row,
  // WM * 32 rows of BN * 2 bytes; half row q = 32 wm + 16 i + r is tile row
  // 64 wm + 16 (2h + i) + r and keeps its 16-byte chunk c at position c ^ r, so
  // that the 16 rows a wave reads at once fall on distinct banks.  Copy j (0-7)
  // of wave w fills the 1024 bytes at (8 w + j) KB: one row, or two (lanes 0-31
  // and 32-63).  Elements past M or N read zeros (they are never stored).
  const v4i rsC = make_buffer_rsrc(p.c, (uint32_t)M * (uint32_t)N * 2u);
  // (half row, position) of copy j's lane ln
  auto staged_q = [&](int j, int ln) -> int { return S::RPC == 1 ? wave * 8 + j : (wave * 8 + j) * 2 + (ln >> 5); };
  auto staged_row = [&](int q, int h) -> int { return (q >> 5) * 64 + (2 * h + ((q >> 4) & 1)) * 16 + (q & 15); };
  auto staged_col = [&](int q, int ln) -> int { return (((S::RPC == 1 ? ln : ln & 31) ^ (q & 15)) << 3); };
  // (a staged column past the tile's width holds nothing)
  auto issue_c = [&](int j, int h, const Unit& w, uint32_t slot) {
    const int ln = opaque(lane);
    const int q = staged_q(j, ln);
    const int tc = staged_col(q, ln);
    const int row = w.m0 + staged_row(q, h), col = w.n0 + tc;
    const uint32_t off =
        row < M && col < N && tc < BN ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 2u : kBufferOutOfRange;
    buf16_to_lds(rsC, off, 0u, smem + slot + (wave * 8 + j) * 1024);
  };

  int t = vb;
  Unit cur;
  if (!next_unit(t, cur)) return;
  setup_copies(cur);
  // The ring: stage s of a unit sits in slot s0 ^ (s & 1); K block kb copies
  // stage kb + 1 into the other slot right after its barrier (every wave is then
  // done with stage kb - 1, which that slot held), and the last K block copies
  // the next unit's stage 0, or the first half of C, which then goes first.
  uint32_t s0 = 0;
#pragma unroll
  for (int idx = 0; idx < S::LPS; ++idx) issue(idx, 0, 0u);
  bool stores_pending = false;   // the previous unit's stores were issued after this unit's stage 0

  while (true) {
    const int KT = cur.nkb;
    const int kb0 = cur.kb0;
    // B scales: the wave's first 128-column block, and (224 wide) the next one,
    // which column blocks nt >= nt_split fall in
    const int bcol0 = cur.n0 + wave_n * WC;
    const int blk0 = min(bcol0, N - 1) >> 7;
    const int sb_idx = __builtin_amdgcn_readfirstlane((cur.g * NB + blk0) * KB + kb0);
    const int sb_idx1 = __builtin_amdgcn_readfirstlane((cur.g * NB + min(blk0 + 1, NB - 1)) * KB + kb0);
    const int nt_split = __builtin_amdgcn_readfirstlane(S::SPLIT_SB ? min(NT, ((blk0 + 1) * 128 - bcol0) >> 4) : NT);
    int t_next = t + G;
    Unit nxt{};
    const bool have_next = next_unit(t_next, nxt);
    const bool c_lds = MODE == MODE_DENSE && cur.part < 0 && p.c != nullptr;   // C is added (through LDS)

    // LDS fragment read offsets (slot 0; block mt / nt adds mt * 2048 / nt *
    // 2048), derived anew for every unit so that they need no register through
    // the tile boundary
    const int lf = opaque(lane);
    const int fr = lf & 15, fg = lf >> 4, sw = swz(fr);
    const uint32_t a_lo = (wave_m * 64 + fr) * 128 + (((2 * fg) ^ sw) << 4);
    const uint32_t a_hi = (wave_m * 64 + fr) * 128 + (((2 * fg + 1) ^ sw) << 4);
    const uint32_t b_lo = S::A_BYTES + (wave_n * WC + fr) * 128 + (((2 * fg) ^ sw) << 4);
    const uint32_t b_hi = S::A_BYTES + (wave_n * WC + fr) * 128 + (((2 * fg + 1) ^ sw) << 4);
    const uint32_t sa_rd = S::A_BYTES + S::B_BYTES + (wave_m * 64 + fr * 4) * 4;

    v4f acc[W_MT][NT];
#pragma unroll
    for (int mt = 0; mt < W_MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
    v4f part[W_LAG];
#pragma unroll
    for (int r = 0; r < W_LAG; ++r) part[r] = v4f{0.f, 0.f, 0.f, 0.f};
    float sprev[W_MT] = {0.f, 0.f, 0.f, 0.f};

    // One K block from the slot at byte offset rd; copy(j) issues what goes
    // after matrix instruction j (one memory instruction after each of the first
    // LPS).  Block j = nt * MT + mt goes into partial register j % LAG (= mt);
    // the register's previous partial, of block (nt - 1, mt) -- for nt = 0 block
    // (NT - 1, mt) of the previous K block, scale sprev -- is promoted first.
    auto kblock = [&](int kb, uint32_t rd, auto&& copy) {
      // Stage kb has landed once no more than the copies and stores issued after
      // it remain (a wave's memory operations retire in issue order): at kb = 0
      // the previous unit's last stores (16 of D's; a split unit's 32 partial
      // stores are waited for down to 16), later nothing (stage kb was the last
      // thing issued, in block kb - 1).
      if (kb == 0 && stores_pending) wait_vmcnt<2 * W_CPH>();
      else wait_vmcnt<0>();
      block_barrier();
      const float sbv = SBc[sb_idx + kb];
      const float sbv1 = S::SPLIT_SB ? SBc[sb_idx1 + kb] : sbv;
      float sav[W_MT];
      if constexpr (S::SA_LDS) {
        const v4f v = *reinterpret_cast<const v4f*>(smem + rd + sa_rd);
#pragma unroll
        for (int i = 0; i < W_MT; ++i) sav[i] = v[i];
      } else {
        // row block i of the lane's rows: the wave's row 16 i + (lane % 16)
#pragma unroll
        for (int i = 0; i < W_MT; ++i) sav[i] = __shfl(sa_nx, 16 * i + (lane & 15), 64);
      }
      // the promotion scale of row block i in column blocks before / from nt_split
      float scur[W_MT], scur1[W_MT];
#pragma unroll
      for (int i = 0; i < W_MT; ++i) {
        scur[i] = sav[i] * sbv;
        scur1[i] = S::SPLIT_SB ? sav[i] * sbv1 : scur[i];
      }
      v8i af[W_MT];
#pragma unroll
      for (int mt = 0; mt < W_MT; ++mt) {
        const v4i lo = *reinterpret_cast<const v4i*>(smem + rd + a_lo + mt * 2048);
        const v4i hi = *reinterpret_cast<const v4i*>(smem + rd + a_hi + mt * 2048);
        af[mt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const v4i lo = *reinterpret_cast<const v4i*>(smem + rd + b_lo + nt * 2048);
        const v4i hi = *reinterpret_cast<const v4i*>(smem + rd + b_hi + nt * 2048);
        const v8i bf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int mt = 0; mt < W_MT; ++mt) {
          const int j = nt * W_MT + mt;
          if (nt == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][NT - 1][i] = fmaf(part[mt][i], sprev[mt], acc[mt][NT - 1][i]);
          } else {
            const float sc = S::SPLIT_SB && nt - 1 >= nt_split ? scur1[mt] : scur[mt];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt - 1][i] = fmaf(part[mt][i], sc, acc[mt][nt - 1][i]);
          }
          part[mt] = mfma_e4m3_16x16x128(bf, af[mt], v4f{0.f, 0.f, 0.f, 0.f});
          if (j < S::LPS) copy(j);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU (promotion)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
          if (j < S::LPS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 VMEM (copy)
        }
      }
#pragma unroll
      for (int i = 0; i < W_MT; ++i) sprev[i] = S::SPLIT_SB && NT - 1 >= nt_split ? scur1[i] : scur[i];
    };

#pragma clang loop unroll(disable)
    for (int kb = 0; kb < KT - 1; ++kb) {
      const uint32_t wr = (s0 ^ (uint32_t)((kb + 1) & 1)) * (uint32_t)S::STAGE;
      kblock(kb, (s0 ^ (uint32_t)(kb & 1)) * (uint32_t)S::STAGE, [&](int j) { issue(j, kb + 1, wr); });
    }
    // the last K block: into the other slot goes half 0 of C, else the next
    // unit's stage 0
    const uint32_t last_slot = (s0 ^ (uint32_t)((KT - 1) & 1)) * (uint32_t)S::STAGE;
    const uint32_t other_slot = last_slot ^ (uint32_t)S::STAGE;
    const bool copy_next = have_next && !c_lds;
    if (copy_next) setup_copies(nxt);
    kblock(KT - 1, last_slot, [&](int j) {
      if (c_lds) {
        if (j < W_CPH) issue_c(j, 0, cur, other_slot);
      } else if (copy_next) {
        issue(j, 0, other_slot);
      }
    });
    // promote the last K block's last column blocks
#pragma unroll
    for (int mt = 0; mt < W_MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][NT - 1][i] = fmaf(part[mt][i], sprev[mt], acc[mt][NT - 1][i]);

    // ---------------- tile boundary ----------------
    const Unit done = cur;
    const bool whole = done.part < 0;
    const int ln = opaque(lane);
    const v4i rsD = make_buffer_rsrc(p.d, (uint32_t)M * (uint32_t)N * 2u);
    // LDS address of a lane's four values of (row block 2h + i, column block nt)
    // in a staged half tile (C's layout)
    auto cd_addr = [&](int i, int nt, uint32_t slot) -> uint32_t {
      const int q = wave_m * 32 + i * 16 + (ln & 15);
      const int c = (wave_n * WC >> 3) + 2 * nt + (ln >> 5);   // the lane's 16-byte chunk of the row
      return slot + q * S::ROWB + ((c ^ (ln & 15)) << 4) + ((ln >> 4) & 1) * 8;
    };
    // half h of D as bf16 into the half tile staged at slot (over C, plus C)
    auto stage_d = [&](int h, bool add_c, uint32_t slot) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t addr = cd_addr(i, nt, slot);
          const v4f a = acc[2 * h + i][nt];
          float v0 = a[0], v1 = a[1], v2 = a[2], v3 = a[3];
          if (add_c) {
            const v2i cv = *reinterpret_cast<const v2i*>(smem + addr);
            v0 += __uint_as_float((uint32_t)cv.x << 16);
            v1 += __uint_as_float((uint32_t)cv.x & 0xffff0000u);
            v2 += __uint_as_float((uint32_t)cv.y << 16);
            v3 += __uint_as_float((uint32_t)cv.y & 0xffff0000u);
          }
          *reinterpret_cast<v2i*>(smem + addr) = v2i{(int)pack_bf16x2_rne(v0, v1), (int)pack_bf16x2_rne(v2, v3)};
        }
    };
    // a staged half tile's rows into registers (copy j's place of issue_c), then
    // to D: every store instruction writes whole rows (1024 bytes), so the lines
    // are whole and the non-temporal hint lets them leave L2 first (stores of
    // 32 bytes in each of 16 rows, straight from the accumulators, measured 5-25 %
    // slower: partial lines, and a wave's stores stall its next tile's K loop).
    // Contiguous form: a row outside the tile's group (padding) is not written.
    v4i drow[W_CPH];
    auto read_d = [&](uint32_t slot) {
#pragma unroll
      for (int j = 0; j < W_CPH; ++j) drow[j] = *reinterpret_cast<const v4i*>(smem + slot + (wave * 8 + j) * 1024 + ln * 16);
    };
    auto store_d = [&](int h) {
#pragma unroll
      for (int j = 0; j < W_CPH; ++j) {
        const int q = staged_q(j, ln);
        const int tc = staged_col(q, ln);
        const int row = done.m0 + staged_row(q, h), col = done.n0 + tc;
        bool ok = row < M && col < N && tc < BN;
        if constexpr (MODE == MODE_CONTIG) ok = ok && p.m_indices[row] == done.g;   // (row is uniform: RPC = 1)
        const uint32_t off = ok ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 2u : kBufferOutOfRange;
        dg_raw_buffer_store_v4i32(drow[j], rsD, (int)off, 0, kStoreNonTemporal);
      }
    };
    if (c_lds) {
      // Half 0 of C is in the other slot; the next unit's stage 0 goes into this
      // one once every wave is done with it.  Each half of D is formed over its
      // half of C in place (a lane reads and writes the same bytes), read back
      // in rows and stored; half 1 of C is copied into the other slot once every
      // wave has read half 0 of D, ahead of half 0's stores.  (The next unit's
      // first K block copies its stage 1 into the other slot after its barrier,
      // which every wave reaches only after reading half 1 of D.)
      wait_lgkmcnt0();
      block_barrier();
      if (have_next) {
        setup_copies(nxt);
#pragma unroll
        for (int idx = 0; idx < S::LPS; ++idx) issue(idx, 0, last_slot);
        wait_vmcnt<S::LPS>();   // half 0 has landed (only the next stage 0 was issued after it)
      } else {
        wait_vmcnt<0>();
      }
      block_barrier();
      stage_d(0, true, other_slot);
      wait_lgkmcnt0();
      block_barrier();   // half 0 of D is staged
      read_d(other_slot);
      wait_lgkmcnt0();
      block_barrier();   // every wave has read it: the slot takes half 1 of C
#pragma unroll
      for (int j = 0; j < W_CPH; ++j) issue_c(j, 1, done, other_slot);
      store_d(0);
      wait_vmcnt<W_CPH>();   // half 1 of C has landed (only half 0's stores were issued after it)
      block_barrier();
      stage_d(1, true, other_slot);
      wait_lgkmcnt0();
      block_barrier();
      read_d(other_slot);
      store_d(1);
    } else if (whole) {
      // D leaves through the last K block's slot (the next unit's stage 0 is in
      // the other one); the next unit's first K block copies its stage 1 into
      // this slot after its barrier, which every wave reaches only after
      // reading half 1 of D
      wait_lgkmcnt0();
      block_barrier();
      stage_d(0, false, last_slot);
      wait_lgkmcnt0();
      block_barrier();
      read_d(last_slot);
      wait_lgkmcnt0();
      block_barrier();
      store_d(0);
      stage_d(1, false, last_slot);
      wait_lgkmcnt0();
      block_barrier();
      read_d(last_slot);
      store_d(1);
    } else {
      // fp32 partial tile of this slice: ws[part][BM][BN], row-major (partials
      // past M or N, or of padding rows, are written too: the reduce reads only
      // valid ones)
      const v4i rsW = make_buffer_rsrc(p.ws + (size_t)done.part * (BM * BN), (uint32_t)(BM * BN * 4));
      const int w_lane = ((wave_m * 64 + (ln & 15)) * BN + wave_n * WC + 4 * (ln >> 4)) * 4;
#pragma unroll
      for (int mt = 0; mt < W_MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const v4i w = {__float_as_int(acc[mt][nt][0]), __float_as_int(acc[mt][nt][1]),
                         __float_as_int(acc[mt][nt][2]), __float_as_int(acc[mt][nt][3])};
          dg_raw_buffer_store_v4i32(w, rsW, w_lane, (mt * 16 * BN + nt * 16) * 4, 0);
        }
    }
    if (!have_next) break;
    t = t_next;
    cur = nxt;
    // the next unit's stage 0 sits in the last block's slot when C was staged,
    // else in the other one
    s0 = (c_lds ? last_slot : other_slot) / (uint32_t)S::STAGE;
    stores_pending = true;
  }
  wait_vmcnt<0>();
}

TileConfig wide_tile_config(int kernel_id) {
  if (kernel_id == kTile256x256Id) return TileConfig{256, 256, 1, W_NW * 64, WideShape<256, 256>::LDS, 2};
  if (kernel_id == kTile256x224Id) return TileConfig{256, 224, 1, W_NW * 64, WideShape<256, 224>::LDS, 2};
  return TileConfig{128, 512, 1, W_NW * 64, WideShape<128, 512>::LDS, 2};
}

template <int BM, int BN, int MODE>
static hipError_t launch_wide(const Fp8GemmParams& p, int grid, hipStream_t stream) {
  constexpr int lds = WideShape<BM, BN>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fp8_gemm_wide_kernel<BM, BN, MODE>), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fp8_gemm_wide_kernel<BM, BN, MODE>), dim3(grid), dim3(W_NW * 64), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm_wide(const Fp8GemmParams& p, int kernel_id, int mode, int grid, hipStream_t stream) {
  if (!wide_fits(p.m, p.n, p.k)) return hipErrorInvalidValue;
  if (kernel_id == kTile256x256Id && mode == MODE_DENSE) return launch_wide<256, 256, MODE_DENSE>(p, grid, stream);
  if (kernel_id == kTile256x224Id && mode == MODE_DENSE) return launch_wide<256, 224, MODE_DENSE>(p, grid, stream);
  if (kernel_id == kTile128x512Id && mode == MODE_DENSE) return launch_wide<128, 512, MODE_DENSE>(p, grid, stream);
  if (kernel_id == kTile128x512Id && mode == MODE_CONTIG) return launch_wide<128, 512, MODE_CONTIG>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace dg
