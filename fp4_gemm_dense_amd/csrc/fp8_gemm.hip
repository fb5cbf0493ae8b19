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
//   * 256 threads = 4 wave64s laid out WM x WN; each wave owns an
//     (MT*16) x (NT*16) sub-tile of 16x16 accumulator blocks.
//   * Per 128-wide K block: A and B tiles (BM x 128 and BN x 128 bytes) are
//     staged through a double-buffered, XOR-swizzled LDS ring with 16-byte
//     coalesced global loads prefetched one block ahead into registers.
//   * Each 16x16 block does ONE v_mfma_f32_16x16x128_f8f6f4 per K block into a
//     fresh fp32 partial, promoted by one FMA per element with sa[row]*sb.
//   * Persistent workgroups walk a group-M raster of tiles; block ids are
//     remapped so that each XCD (workgroups are dealt round-robin to the 8
//     XCDs) works on a contiguous stretch of the raster and shares its L2.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

template <int MT, int NT, int WM, int WN, int STAGES, int MODE>
__global__ void __launch_bounds__(WM * WN * 64, 1) fp8_gemm_kernel(Fp8GemmParams p) {
  constexpr int NW = WM * WN;                 // waves per workgroup
  constexpr int BM = WM * MT * 16;
  constexpr int BN = WN * NT * 16;
  constexpr int A_BYTES = BM * 128;
  constexpr int B_BYTES = BN * 128;
  constexpr int SA_BYTES = BM * 4;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  // Each wave copies RA 8-row regions (1 KB) of A, RB of B and SPW A scales per stage.
  static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "regions must split evenly over waves");
  constexpr int RA = BM / 8 / NW;
  constexpr int RB = BN / 8 / NW;
  constexpr int SPW = BM / NW;
  static_assert(SPW <= 64, "scale copy must fit one instruction per wave");
  constexpr int LPS = RA + RB + 1;            // DMA instructions per wave per stage
  // the 16 columns of every accumulator block lie in one 128-wide B-scale block;
  // when all of a wave's columns do, one sb serves the whole wave
  constexpr bool ONE_SB = (128 % (NT * 16) == 0) && (BN % 128 == 0 || 128 % BN == 0);

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef const __attribute__((address_space(4))) float cfloat;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / WN;
  const int wave_n = wave % WN;
  const int lrow = lane & 15;     // operand row / output column inside a 16x16 block
  const int lgrp = lane >> 4;     // K chunk of the operand / row quad of the output

  const int M = p.m, N = p.n, K = p.k;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;

  // Per-lane LDS read offsets (slot 0); blocks mt / nt add mt*2048 / nt*2048
  // and the slot adds slot*STAGE.  The swizzle depends on row % 16 only.
  const int sw = swz(lrow);
  const uint32_t a_lo = (wave_m * MT * 16 + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const uint32_t a_hi = (wave_m * MT * 16 + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);
  const uint32_t b_lo = A_BYTES + (wave_n * NT * 16 + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const uint32_t b_hi = A_BYTES + (wave_n * NT * 16 + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);
  const uint32_t sa_rd = A_BYTES + B_BYTES + (wave_m * MT * 16 + 4 * lgrp) * 4;
  // Per-lane DMA row inside an 8-row region; the swizzled chunk depends on the
  // tile row's bit 3 as well, i.e. on the region's parity.
  const int dma_row = lane >> 3;

  // XCD-aware remap of the persistent block id: workgroups are dealt to the
  // 8 XCDs round-robin, so give XCD x a contiguous stretch of the raster.
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int t = vb; t < p.total_tiles; t += G) {
    // ---------------- tile -> (group, tm, tn) ----------------
    int g = 0, tl = t;
    if (MODE == MODE_MASKED) {
      const int per = p.tiles_m * p.tiles_n;
      g = t / per;
      tl = t - g * per;
    }
    const int per_group = p.group_m * p.tiles_n;
    const int gi = tl / per_group;
    const int first_m = gi * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int r = tl - gi * per_group;
    const int tm = first_m + r % gm;
    const int tn = r / gm;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    int rows_valid = M;      // rows that may be stored
    if (MODE == MODE_MASKED) {
      int mm = p.masked_m[g];
      rows_valid = mm < 0 ? 0 : (mm > M ? M : mm);
      if (m0 >= rows_valid) continue;           // empty tile: the whole workgroup skips it
    }
    if (MODE == MODE_CONTIG) {
      g = p.m_indices[m0];
      if (g < 0 || g >= p.num_groups) continue; // padding block
    }

    const uint8_t* A = p.a;
    const float* SA = p.sfa;
    const uint8_t* B = p.b;
    const float* SB = p.sfb;
    if (MODE == MODE_MASKED) {
      A += (size_t)g * M * K;
      SA += (size_t)g * KB * M;
    }
    if (MODE != MODE_DENSE) {
      B += (size_t)g * N * K;
      SB += (size_t)g * NB * KB;
    }

    // ---------------- DMA sources of this wave ----------------
    // A region (wave*RA + j) covers tile rows 8*(wave*RA+j) .. +7; lane l fills
    // LDS bytes [16l, 16l+16) of it: row + l/8, position l%8, which holds
    // logical chunk (l%8) ^ swz(row).  Offsets are 32-bit, relative to A / B.
    uint32_t a_off[RA], b_off[RB];
#pragma unroll
    for (int j = 0; j < RA; ++j) {
      const int row = (wave * RA + j) * 8 + dma_row;
      a_off[j] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K + (((lane & 7) ^ swz(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = (wave * RB + j) * 8 + dma_row;
      b_off[j] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)K + (((lane & 7) ^ swz(row)) << 4);
    }
    const uint32_t sa_off = (uint32_t)min(m0 + wave * SPW + (lane < SPW ? lane : 0), M - 1) * 4;
    const uint32_t a_dst = wave * RA * 1024;
    const uint32_t b_dst = A_BYTES + wave * RB * 1024;
    const uint32_t sa_dst = A_BYTES + B_BYTES + wave * SPW * 4;

    auto issue = [&](int kb, uint32_t slot_off) {
      const uint8_t* ak = A + (size_t)kb * 128;
      const uint8_t* bk = B + (size_t)kb * 128;
      const uint8_t* sk = reinterpret_cast<const uint8_t*>(SA + (size_t)kb * M);
#pragma unroll
      for (int j = 0; j < RA; ++j) dma16_to_lds(ak + a_off[j], smem + slot_off + a_dst + j * 1024);
#pragma unroll
      for (int j = 0; j < RB; ++j) dma16_to_lds(bk + b_off[j], smem + slot_off + b_dst + j * 1024);
      if (SPW == 64 || lane < SPW) dma4_to_lds(sk + sa_off, smem + slot_off + sa_dst);
    };

    // B-scale indices are wave-uniform; reading them through the constant
    // address space makes the per-K-block reads scalar loads (not counted by vmcnt)
    cfloat* SBc = (cfloat*)(uintptr_t)(SB);
    int sb_idx[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      sb_idx[nt] = __builtin_amdgcn_readfirstlane((min(n0 + wave_n * NT * 16 + nt * 16, N - 1) >> 7) * KB);

    v4f acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

    // prologue: stages 0 .. STAGES-2 in flight
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KB) issue(s, s * STAGE);

    uint32_t rd_slot = 0;                          // slot of stage kb
    uint32_t wr_slot = (STAGES - 1) * STAGE;       // slot of stage kb + STAGES - 1
    for (int kb = 0; kb < KB; ++kb) {
      // stage kb has landed once at most (#stages issued after it) DMA ops remain
      const int after = min(STAGES - 2, KB - 1 - kb);
      if (STAGES >= 4 && after >= 2) wait_vmcnt<(STAGES >= 4 ? 2 : 0) * LPS>();
      else if (STAGES >= 3 && after >= 1) wait_vmcnt<(STAGES >= 3 ? 1 : 0) * LPS>();
      else wait_vmcnt<0>();
      block_barrier();
      if (kb + STAGES - 1 < KB) issue(kb + STAGES - 1, wr_slot);

      float sbv[NT];
      if (ONE_SB) {
        const float s0 = SBc[sb_idx[0] + kb];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sbv[nt] = s0;
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sbv[nt] = SBc[sb_idx[nt] + kb];
      }
      const uint8_t* ra_lo = smem + rd_slot + a_lo;
      const uint8_t* ra_hi = smem + rd_slot + a_hi;
      const uint8_t* rb_lo = smem + rd_slot + b_lo;
      const uint8_t* rb_hi = smem + rd_slot + b_hi;
      const uint8_t* rsa = smem + rd_slot + sa_rd;
      v4f sa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sa[mt] = *reinterpret_cast<const v4f*>(rsa + mt * 64);
      v8i af[MT], bf[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4i lo = *reinterpret_cast<const v4i*>(ra_lo + mt * 2048);
        v4i hi = *reinterpret_cast<const v4i*>(ra_hi + mt * 2048);
        af[mt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        v4i lo = *reinterpret_cast<const v4i*>(rb_lo + nt * 2048);
        v4i hi = *reinterpret_cast<const v4i*>(rb_hi + nt * 2048);
        bf[nt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
      if (ONE_SB) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sa[mt] *= sbv[0];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          v4f part = mfma_e4m3_16x16x128(af[mt], bf[nt], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sc = ONE_SB ? sa[mt][i] : sa[mt][i] * sbv[nt];
            acc[mt][nt][i] = fmaf(part[i], sc, acc[mt][nt][i]);
          }
        }
      }
      rd_slot = (rd_slot + STAGE == STAGES * STAGE) ? 0u : rd_slot + STAGE;
      wr_slot = (wr_slot + STAGE == STAGES * STAGE) ? 0u : wr_slot + STAGE;
    }
    block_barrier();   // every wave is done with the LDS ring before the next tile refills it

    // ---------------- epilogue: + C, bf16 RNE, predicated stores ----------------
    uint16_t* D = p.d;
    if (MODE == MODE_MASKED) D += (size_t)g * M * N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int grow = m0 + wave_m * MT * 16 + mt * 16 + 4 * lgrp + i;
        bool row_ok = grow < rows_valid;
        if (MODE == MODE_CONTIG && row_ok) row_ok = p.m_indices[grow] == g;
        if (!row_ok) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = n0 + wave_n * NT * 16 + nt * 16 + lrow;
          if (col >= N) continue;
          float v = acc[mt][nt][i];
          if (MODE == MODE_DENSE && p.c != nullptr) v += bf16_to_f32(p.c[(size_t)grow * N + col]);
          D[(size_t)grow * N + col] = f32_to_bf16_rne(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tile-config table and launcher
// ---------------------------------------------------------------------------

// id, MT, NT, WM, WN, STAGES, workgroups per CU
#define DG_TILE_CONFIGS(X)    \
  X(0, 4, 4, 4, 2, 3, 1)      \
  X(1, 4, 4, 2, 4, 3, 1)      \
  X(2, 4, 4, 2, 2, 3, 1)      \
  X(3, 4, 2, 1, 4, 4, 1)

static const TileConfig kTileConfigs[] = {
#define X(id, MT, NT, WM, WN, ST, OCC) {WM * MT * 16, WN * NT * 16, OCC, WM * WN * 64, \
                                        ST * ((WM * MT * 16 + WN * NT * 16) * 128 + WM * MT * 16 * 4)},
    DG_TILE_CONFIGS(X)
#undef X
};

int num_tile_configs() { return (int)(sizeof(kTileConfigs) / sizeof(kTileConfigs[0])); }
TileConfig tile_config(int id) { return kTileConfigs[id]; }

template <int MODE>
static hipError_t launch_mode(const Fp8GemmParams& p, int kernel_id, int grid, hipStream_t stream) {
  switch (kernel_id) {
#define X(id, MT, NT, WM, WN, ST, OCC)                                                              \
  case id: {                                                                                      \
    const TileConfig& tc = kTileConfigs[id];                                                      \
    static const hipError_t attr = hipFuncSetAttribute(                                           \
        reinterpret_cast<const void*>(&fp8_gemm_kernel<MT, NT, WM, WN, ST, MODE>),                \
        hipFuncAttributeMaxDynamicSharedMemorySize, tc.lds_bytes);                                \
    if (attr != hipSuccess) return attr;                                                          \
    hipLaunchKernelGGL((fp8_gemm_kernel<MT, NT, WM, WN, ST, MODE>), dim3(grid), dim3(tc.threads), \
                       tc.lds_bytes, stream, p);                                                  \
    break;                                                                                        \
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
  switch (mode) {
    case MODE_DENSE: return launch_mode<MODE_DENSE>(p, plan.kernel_id, plan.num_workgroups, stream);
    case MODE_CONTIG: return launch_mode<MODE_CONTIG>(p, plan.kernel_id, plan.num_workgroups, stream);
    case MODE_MASKED: return launch_mode<MODE_MASKED>(p, plan.kernel_id, plan.num_workgroups, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
