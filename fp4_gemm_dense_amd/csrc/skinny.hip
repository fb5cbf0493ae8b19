// Skinny-M fine-grained-scaled FP8 GEMM for gfx950: D = C + A.B^T (NT), bf16 out.
//
// What is computed is the dense GEMM of the usage guide ("DeepGEMM：统一高性能张量
// 核心 GEMM 计算库编译与使用指南", 五、使用方法) with the two-level accumulation of
// the release article ("DeepSeek 开源第三弹 ... DeepGEMM", DeepGEMM section): one
// matrix instruction per 128-wide K block into a fresh fp32 partial, promoted on
// the vector ALUs by sa * sb.  The release article's featured shape is of this
// kind (M=128, N=2112, K=7168, 性能), and its update news (其他更新) swaps A and B
// for skinny problems so that the large operand takes the matrix unit's wide side.
//
// gfx950 design for problems with few rows (M <= 128): such a GEMM streams B
// (N x K bytes) from HBM once and is bound by how many bytes each CU keeps in
// flight, not by the matrix cores.  So the roles of the operands differ from the
// square-tile kernel:
//   * a tile holds BM = 16 * MT rows of A (all of them when M <= BM) and
//     BN = 16 * NT columns per wave; the waves split N and share A;
//   * B, the large operand, goes straight from HBM into registers: each wave
//     loads its own 16 * NT rows of B, P K blocks ahead, into P register sets
//     (no LDS round trip, and P * NW * NT * 2 KB of B in flight per CU);
//   * A, the small shared operand, is copied into LDS in chunks of P K blocks
//     (buffer_load ... lds) through two chunk buffers, so the waves meet at one
//     barrier per P blocks and otherwise stream B independently;
//   * K is split into slices when the column tiles alone cannot fill the chip;
//     a slice writes its fp32 partial tile into the caller's workspace and the
//     split-K reduce kernel sums the slices in slice order (plus C).
// The K loop is straight-line over groups of P blocks (the register set of a
// block is a compile-time index); a slice is padded to a multiple of P with
// blocks whose loads use a null buffer resource (no memory traffic) and whose
// promotion weight is zero.
#include <algorithm>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

template <int MT, int NT, int NW, int P>
__global__ void __launch_bounds__(NW * 64, 1) skinny_gemm_kernel(SkinnyParams p) {
  constexpr int BM = MT * 16;
  constexpr int BN = NW * NT * 16;
  constexpr int A_BLK = BM * 128;               // LDS bytes of A per K block
  constexpr int RG = BM / 8;                    // 1 KB regions (8 rows x 128 bytes) per K block
  constexpr int LB = 2 * NT;                    // B loads per wave per K block
  // A goes through two chunk buffers of P K blocks each: A rows, then the row
  // scales (copied 64 at a time); a 1 KB area takes the copies a wave issues
  // beyond a chunk's real ones, so that every wave issues the same count
  constexpr int CH_A = P * A_BLK;
  constexpr int CH_SA_OPS = (P * BM + 63) / 64;
  constexpr int CH_BYTES = CH_A + CH_SA_OPS * 256;
  constexpr uint32_t DUMMY = 2 * CH_BYTES;
  constexpr int RA = (P * RG + NW - 1) / NW;    // region copies per wave per chunk
  constexpr int RS = (CH_SA_OPS + NW - 1) / NW; // scale copies per wave per chunk
  constexpr int CC = RA + RS;                   // copies per wave per chunk
  static_assert((P - 1) * LB + CC < 64 && P * LB < 64, "vmcnt range");
  static_assert(MT == 1 || MT == 2 || MT % 4 == 0, "row scales are read 1, 2 or 4 at a time");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef const __attribute__((address_space(4))) float cfloat;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15;    // operand row / output column inside a 16 x 16 block
  const int lgrp = lane >> 4;    // K chunk of the operand / row quad of the output
  const int sw = swz(lrow);

  const int M = p.m, N = p.n, K = p.k;
  const int KB = K >> 7;
  const int tiles_m = p.tiles_m, tiles_n = p.tiles_n, splits = p.splits, kbps = p.kb_per_split;
  const int tiles = tiles_m * tiles_n;
  const int total = tiles * splits;

  const v4i rsA = make_buffer_rsrc(p.a, (uint32_t)M * (uint32_t)K);
  const v4i rsSA = make_buffer_rsrc(p.sfa, (uint32_t)KB * (uint32_t)M * 4u);
  const v4i rsB = make_buffer_rsrc(p.b, (uint32_t)N * (uint32_t)K);
  const v4i rsNull = make_buffer_rsrc(p.b, 0u);   // every access out of range: zeros, no request
  cfloat* const SBc = (cfloat*)(uintptr_t)p.sfb;

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so XCD x
  // takes a contiguous stretch of units; units are slice-major, so the units an
  // XCD runs at once share their K slices of A in its L2.
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int u = vb; u < total; u += G) {
    // unit u: K slice u / tiles of tile u % tiles; tiles are column-major (row
    // tile fastest), as the split-K reduce walks them
    const int t = u % tiles, sl = u / tiles;
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows = min(BM, M - m0);          // valid rows of the tile
    const int kb0 = sl * kbps;
    const int nkb = min(kbps, KB - kb0);
    const int nch = (nkb + P - 1) / P;         // chunks of P blocks (the last one padded)
    const bool whole = splits == 1;
    const int col0 = n0 + wave * (NT * 16);   // the wave's first column
    // one B scale per wave and K block: its 16 * NT columns lie in one 128-row block of B
    const int sb_idx = __builtin_amdgcn_readfirstlane((min(col0, N - 1) >> 7) * KB + kb0);

    uint32_t b_off[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = col0 + nt * 16 + lrow;
      b_off[nt] = row < N ? (uint32_t)row * (uint32_t)K + (uint32_t)(lgrp << 4) : kBufferOutOfRange;
    }

    // every wave is done with the previous unit's A before it is overwritten
    block_barrier();

    // C of a whole tile, fetched first and added in the epilogue.  Lane (lgrp,
    // lrow) of block (mt, nt) holds row mt * 16 + lrow, columns nt * 16 + 4 lgrp
    // .. + 3 of the wave's strip.
    v2i creg[MT][NT];
    const bool has_c = whole && p.c != nullptr;
    if (has_c) {
      const v4i rsC = make_buffer_rsrc(p.c, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row = mt * 16 + lrow, col = col0 + nt * 16 + 4 * lgrp;
          const uint32_t off = (row < rows && col < N)
                                   ? ((uint32_t)(m0 + row) * (uint32_t)N + (uint32_t)col) * 2u
                                   : kBufferOutOfRange;
          creg[mt][nt] = dg_raw_buffer_load_v2i32(rsC, (int)off, 0, 0);
        }
    }

    // Copies of chunk c (K blocks cP .. cP + P - 1 of the slice) into buffer c % 2:
    // region o of the chunk (the wave's j-th is o = j * NW + wave) is block o / RG,
    // rows 8 (o % RG) ..; lane l fills bytes [16 l, 16 l + 16): row 8 (o % RG) + l / 8,
    // position l % 8, which holds chunk (l % 8) ^ swz(row).  Scale copy q moves
    // entries 64 q .. of the chunk's [block][BM] scales.  Copies past the slice (or
    // past the chunk) read nothing and land in the dummy area; rows past the tile
    // read zeros.
    auto copy_chunk = [&](int c) {
      const uint32_t buf = (uint32_t)(c & 1) * (uint32_t)CH_BYTES;
#pragma unroll
      for (int j = 0; j < RA; ++j) {
        const int o = j * NW + wave;
        const int kb = c * P + o / RG, rg = o % RG;
        const bool real = o < P * RG && kb < nkb;
        const int row = rg * 8 + (lane >> 3);
        const uint32_t off = row < rows
                                 ? (uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)(((lane & 7) ^ swz(row)) << 4)
                                 : kBufferOutOfRange;
        buf16_to_lds(real ? rsA : rsNull, off, real ? (uint32_t)(kb0 + kb) * 128u : 0u,
                     smem + (real ? buf + (uint32_t)(o / RG) * A_BLK + (uint32_t)rg * 1024u : DUMMY));
      }
#pragma unroll
      for (int j = 0; j < RS; ++j) {
        const int q = j * NW + wave;
        const int e = q * 64 + lane;             // entry blk * BM + pos of the chunk
        const int blk = e / BM, pos = e % BM;
        const int row = (pos % MT) * 16 + pos / MT;
        const int kb = c * P + blk;
        const bool real = q < CH_SA_OPS;
        const uint32_t off = (blk < P && kb < nkb && row < rows)
                                 ? (uint32_t)(kb0 + kb) * (uint32_t)M * 4u + (uint32_t)(m0 + row) * 4u
                                 : kBufferOutOfRange;
        buf4_to_lds(real ? rsSA : rsNull, off, 0u, smem + (real ? buf + (uint32_t)CH_A + (uint32_t)q * 256u : DUMMY));
      }
    };
    copy_chunk(0);
    asm volatile("" ::: "memory");

    // B of the first P K blocks (a padding block past the slice reads nothing)
    v8i bset[P][NT];
    auto issue_b = [&](int s, auto set_tag) {
      constexpr int js = decltype(set_tag)::value;
      const bool real = s < nkb;
      const v4i& rb = real ? rsB : rsNull;
      const uint32_t kofs = (uint32_t)(kb0 + (real ? s : 0)) * 128u;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // K chunks lgrp (bytes 16 lgrp ..) and lgrp + 4 (bytes 64 + 16 lgrp ..) of
        // the block: any K order common to both operands gives the same sum, and
        // this one reads 64 contiguous bytes of a row per instruction
        const v4i lo = dg_raw_buffer_load_v4i32(rb, (int)b_off[nt], (int)kofs, 0);
        const v4i hi = dg_raw_buffer_load_v4i32(rb, (int)(b_off[nt] + 64u), (int)kofs, 0);
        bset[js][nt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    };
    static_for<P>([&](auto jt) {
      issue_b(decltype(jt)::value, jt);
      asm volatile("" ::: "memory");
    });

    v4f acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

    // the B scale of the next K block is loaded one block ahead (scalar loads)
    float sb_next = SBc[sb_idx];
    for (int c = 0; c < nch; ++c) {
      // chunk c has landed once no more than the B loads issued after its copies
      // are outstanding; the barrier makes every wave's copies visible and frees
      // the other buffer (every wave is done with chunk c - 1), which takes chunk c + 1
      wait_vmcnt<P * LB>();
      block_barrier();
      copy_chunk(c + 1);
      asm volatile("" ::: "memory");
      const uint32_t buf = (uint32_t)(c & 1) * (uint32_t)CH_BYTES;
      static_for<P>([&](auto jt) {
        constexpr int j = decltype(jt)::value;
        const int kb = c * P + j;
        const bool real = kb < nkb;
        const int kr = real ? j : 0;             // a padding block reads the chunk's first block, weight 0
        const float wgt = real ? sb_next : 0.f;
        sb_next = SBc[sb_idx + (kb + 1 < nkb ? kb + 1 : 0)];
        float s[MT];
        const uint8_t* srd = smem + buf + CH_A + (uint32_t)kr * (BM * 4) + lrow * MT * 4;
        if constexpr (MT % 4 == 0) {
#pragma unroll
          for (int q = 0; q < MT / 4; ++q) {
            const v4f v = *reinterpret_cast<const v4f*>(srd + 16 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[4 * q + i] = v[i] * wgt;
          }
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) s[mt] = reinterpret_cast<const float*>(srd)[mt] * wgt;
        }
        // A fragments of the block, read one row block ahead of the matrix instructions
        const uint8_t* ablk = smem + buf + (uint32_t)kr * A_BLK + (uint32_t)lrow * 128u;
        auto read_a = [&](int mt) -> v8i {
          const uint8_t* ar = ablk + (uint32_t)mt * 2048u;
          const v4i lo = *reinterpret_cast<const v4i*>(ar + ((lgrp ^ sw) << 4));
          const v4i hi = *reinterpret_cast<const v4i*>(ar + (((lgrp + 4) ^ sw) << 4));
          return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        };
        v8i af[2];
        af[0] = read_a(0);
        // B of block kb has landed once no more than the later blocks' loads and
        // the next chunk's copies are outstanding
        wait_vmcnt<(P - 1) * LB + CC>();
        v4f part[2][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt + 1 < MT) af[(mt + 1) & 1] = read_a(mt + 1);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            part[mt & 1][nt] = mfma_e4m3_16x16x128(bset[j][nt], af[mt & 1], v4f{0.f, 0.f, 0.f, 0.f});
          if (mt > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[mt - 1][nt][i] = fmaf(part[(mt - 1) & 1][nt][i], s[mt - 1], acc[mt - 1][nt][i]);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[MT - 1][nt][i] = fmaf(part[(MT - 1) & 1][nt][i], s[MT - 1], acc[MT - 1][nt][i]);
        // this wave is done with register set j: refill it with block kb + P
        issue_b(kb + P, jt);
      });
    }

    if (!whole) {
      // fp32 partial tile of this slice: ws[(t * splits + sl)][BM][BN], row-major
      const v4i rsW = make_buffer_rsrc(p.ws + (size_t)(t * splits + sl) * (BM * BN), (uint32_t)(BM * BN * 4));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t off =
              (uint32_t)((mt * 16 + lrow) * BN + wave * NT * 16 + nt * 16 + 4 * lgrp) * 4u;
          const v4i w = {__float_as_int(acc[mt][nt][0]), __float_as_int(acc[mt][nt][1]),
                         __float_as_int(acc[mt][nt][2]), __float_as_int(acc[mt][nt][3])};
          dg_raw_buffer_store_v4i32(w, rsW, (int)off, 0, 0);
        }
    } else {
      const v4i rsD = make_buffer_rsrc(p.d, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row = mt * 16 + lrow, col = col0 + nt * 16 + 4 * lgrp;
          float v0 = acc[mt][nt][0], v1 = acc[mt][nt][1], v2 = acc[mt][nt][2], v3 = acc[mt][nt][3];
          if (has_c) {
            const v2i cv = creg[mt][nt];
            v0 += __uint_as_float((uint32_t)cv.x << 16);
            v1 += __uint_as_float((uint32_t)cv.x & 0xffff0000u);
            v2 += __uint_as_float((uint32_t)cv.y << 16);
            v3 += __uint_as_float((uint32_t)cv.y & 0xffff0000u);
          }
          const uint32_t off = (row < rows && col < N)
                                   ? ((uint32_t)(m0 + row) * (uint32_t)N + (uint32_t)col) * 2u
                                   : kBufferOutOfRange;
          const v2i w = {(int)pack_bf16x2_rne(v0, v1), (int)pack_bf16x2_rne(v2, v3)};
          dg_raw_buffer_store_v2i32(w, rsD, (int)off, 0, kStoreNonTemporal);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// configurations and launcher
// ---------------------------------------------------------------------------

// id, MT, NT, NW, P
#define DG_SKINNY_CONFIGS(X) \
  X(0, 1, 1, 8, 8)           \
  X(1, 2, 1, 8, 8)           \
  X(2, 4, 1, 8, 8)           \
  X(3, 8, 1, 8, 4)           \
  X(4, 4, 1, 4, 8)           \
  X(5, 8, 1, 4, 4)           \
  X(6, 4, 1, 6, 8)           \
  X(7, 8, 1, 6, 4)           \
  X(8, 4, 2, 8, 6)           \
  X(9, 2, 2, 8, 6)           \
  X(10, 8, 1, 7, 4)          \
  X(11, 4, 1, 7, 8)          \
  X(12, 8, 2, 7, 4)

// LDS of a configuration: two chunk buffers of P K blocks (A rows and scales) and
// the 1 KB area of the surplus copies
#define DG_SKINNY_LDS(MT, P) (2 * ((P) * (MT) * 16 * 128 + ((P) * (MT) * 16 + 63) / 64 * 256) + 1024)
static const SkinnyConfig kSkinnyConfigs[] = {
#define X(id, MT, NT, NW, P) {MT * 16, NW * NT * 16, NW * 64, P, DG_SKINNY_LDS(MT, P)},
    DG_SKINNY_CONFIGS(X)
#undef X
};

int num_skinny_configs() { return (int)(sizeof(kSkinnyConfigs) / sizeof(kSkinnyConfigs[0])); }
SkinnyConfig skinny_config(int id) { return kSkinnyConfigs[id]; }

hipError_t launch_skinny_gemm(const SkinnyParams& p, int id, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const SkinnyConfig sc = kSkinnyConfigs[id];

  switch (id) {
#define X(i, MT, NT, NW, P)                                                                             \
  case i: {                                                                                             \
    static const hipError_t attr = hipFuncSetAttribute(                                                 \
        reinterpret_cast<const void*>(&skinny_gemm_kernel<MT, NT, NW, P>),                              \
        hipFuncAttributeMaxDynamicSharedMemorySize, sc.lds_bytes);                                      \
    if (attr != hipSuccess) return attr;                                                                \
    hipLaunchKernelGGL((skinny_gemm_kernel<MT, NT, NW, P>), dim3(grid), dim3(sc.threads),               \
                       sc.lds_bytes, stream, p);                                                        \
    return hipGetLastError();                                                                           \
  }
    DG_SKINNY_CONFIGS(X)
#undef X
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
