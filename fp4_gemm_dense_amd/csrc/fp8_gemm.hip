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

template <int MT, int NT, int WM, int WN, int MODE>
__global__ void __launch_bounds__(256, 1) fp8_gemm_kernel(Fp8GemmParams p) {
  constexpr int BM = WM * MT * 16;
  constexpr int BN = WN * NT * 16;
  constexpr int A_BYTES = BM * 128;
  constexpr int B_BYTES = BN * 128;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_CHUNKS = BM * 8;    // 16-byte chunks per A tile
  constexpr int B_CHUNKS = BN * 8;
  constexpr int A_LD = (A_CHUNKS + 255) / 256;
  constexpr int B_LD = (B_CHUNKS + 255) / 256;
  static_assert(WM * WN == 4, "four waves per workgroup");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave / WN;
  const int wave_n = wave % WN;
  const int lrow = lane & 15;     // operand row / output column inside a 16x16 block
  const int lgrp = lane >> 4;     // K chunk of the operand / row quad of the output

  const int M = p.m, N = p.n, K = p.k;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;

  // XCD-aware remap of the persistent block id.
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
      if (m0 >= rows_valid) continue;           // empty tile: whole block skips
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

    // ---------------- global -> register staging ----------------
    v4i ra[A_LD], rb[B_LD];
    const v4i* a_src[A_LD];
    const v4i* b_src[B_LD];
    int a_dst[A_LD], b_dst[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      int ch = tid + i * 256;
      int row = ch >> 3, c = ch & 7;
      if (ch >= A_CHUNKS) row = 0;
      int gr = min(m0 + row, M - 1);
      a_src[i] = reinterpret_cast<const v4i*>(A + (size_t)gr * K + c * 16);
      a_dst[i] = row * 128 + ((c ^ swz(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      int ch = tid + i * 256;
      int row = ch >> 3, c = ch & 7;
      if (ch >= B_CHUNKS) row = 0;
      int gc = min(n0 + row, N - 1);
      b_src[i] = reinterpret_cast<const v4i*>(B + (size_t)gc * K + c * 16);
      b_dst[i] = A_BYTES + row * 128 + ((c ^ swz(row)) << 4);
    }
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        if (A_CHUNKS % 256 == 0 || tid + i * 256 < A_CHUNKS) ra[i] = a_src[i][kb * 8];
#pragma unroll
      for (int i = 0; i < B_LD; ++i)
        if (B_CHUNKS % 256 == 0 || tid + i * 256 < B_CHUNKS) rb[i] = b_src[i][kb * 8];
    };
    auto lstore = [&](int buf) {
      uint8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        if (A_CHUNKS % 256 == 0 || tid + i * 256 < A_CHUNKS) *reinterpret_cast<v4i*>(base + a_dst[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_LD; ++i)
        if (B_CHUNKS % 256 == 0 || tid + i * 256 < B_CHUNKS) *reinterpret_cast<v4i*>(base + b_dst[i]) = rb[i];
    };

    // per-lane scale addresses
    int sa_row[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sa_row[mt][i] = min(m0 + wave_m * MT * 16 + mt * 16 + 4 * lgrp + i, M - 1);
    int sb_blk[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      sb_blk[nt] = (min(n0 + wave_n * NT * 16 + nt * 16, N - 1) >> 7) * KB;

    v4f acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < KB) gload(kb + 1);

      float sa[MT][4], sb[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[mt][i] = SA[(size_t)kb * M + sa_row[mt][i]];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sb[nt] = SB[sb_blk[nt] + kb];

      const uint8_t* sA = smem + cur * STAGE_BYTES;
      const uint8_t* sB = sA + A_BYTES;
      v8i af[MT], bf[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wave_m * MT * 16 + mt * 16 + lrow;
        const uint8_t* rp = sA + row * 128;
        const int s = swz(row);
        v4i lo = *reinterpret_cast<const v4i*>(rp + (((2 * lgrp) ^ s) << 4));
        v4i hi = *reinterpret_cast<const v4i*>(rp + (((2 * lgrp + 1) ^ s) << 4));
        af[mt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int row = wave_n * NT * 16 + nt * 16 + lrow;
        const uint8_t* rp = sB + row * 128;
        const int s = swz(row);
        v4i lo = *reinterpret_cast<const v4i*>(rp + (((2 * lgrp) ^ s) << 4));
        v4i hi = *reinterpret_cast<const v4i*>(rp + (((2 * lgrp + 1) ^ s) << 4));
        bf[nt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          v4f part = mfma_e4m3_16x16x128(af[mt], bf[nt], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(part[i], sa[mt][i] * sb[nt], acc[mt][nt][i]);
        }
      }

      if (kb + 1 < KB) lstore(cur ^ 1);
      __syncthreads();
    }

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

// id, MT, NT, WM, WN, waves per SIMD reached by the compiled kernel
#define DG_TILE_CONFIGS(X) \
  X(0, 4, 4, 2, 2, 1)      \
  X(1, 2, 4, 2, 2, 2)      \
  X(2, 2, 2, 2, 2, 3)

static const TileConfig kTileConfigs[] = {
#define X(id, MT, NT, WM, WN, OCC) {WM * MT * 16, WN * NT * 16, OCC},
    DG_TILE_CONFIGS(X)
#undef X
};

int num_tile_configs() { return (int)(sizeof(kTileConfigs) / sizeof(kTileConfigs[0])); }
TileConfig tile_config(int id) { return kTileConfigs[id]; }

template <int MODE>
static hipError_t launch_mode(const Fp8GemmParams& p, int kernel_id, int grid, hipStream_t stream) {
  switch (kernel_id) {
#define X(id, MT, NT, WM, WN, OCC)                                                            \
  case id:                                                                                    \
    hipLaunchKernelGGL((fp8_gemm_kernel<MT, NT, WM, WN, MODE>), dim3(grid), dim3(256), 0, stream, p); \
    break;
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
