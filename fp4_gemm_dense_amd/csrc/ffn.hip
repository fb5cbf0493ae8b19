// FP8 x FP4 expert FFN for gfx950: the single-GPU compute share of the fused
// MoE layer.
//
// What is computed follows the news page on the DeepGEMM update ("DeepSeek 发布
// DeepGEMM 重大更新：Mega MoE 融合算子与 FP4 精度支持"): in section "Mega MoE" each
// expert runs linear1 -> SwiGLU -> linear2 and the results are combined; in
// section "FP4 精度支持" activations are FP8, weights are FP4 with UE8M0 scale
// factors packed four to an int32.  Dispatch and combine across GPUs are not
// part of this library: tokens, their top-k expert ids and weights arrive on
// this GPU and only the local experts are computed.
//
// gfx950 design (four kernels on one stream, no host synchronisation):
//   1. route   (one workgroup): per-expert pair counts, starts, and a pair list
//              (token of each pair; pair index of each (token, slot)).
//   2. linear1 (persistent): for each (expert, 64-row block of its pairs,
//              128 intermediate columns) the gathered e4m3 token rows times the
//              matching 128 gate rows and 128 up rows of W1 with
//              v_mfma_scale_f32_16x16x128_f8f6f4 (A e4m3, B e2m1; both UE8M0
//              scales applied by the matrix core per 32-element K chunk), then in
//              registers: s = silu(gate) * up, per-row 128-column amax across the
//              four waves (LDS), power-of-two scale, e4m3 round-to-nearest-even;
//              writes the e4m3 intermediate and its UE8M0 exponents.
//   3. linear2 (persistent): (expert, 64-row block, 256 output columns) of the
//              intermediate times W2 with the same scaled MFMA; writes fp32 per pair.
//   4. combine: y[t] = sum over slots j (in order) of w[t,j] * o[pair(t,j)], bf16.
// Operand tiles and their scale words are staged through a 3-stage LDS ring with
// global_load_lds (the token gather happens in the DMA addresses).
#include "../../include/dg.h"
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

constexpr int FFN_MAX_EXPERTS = 256;
constexpr int FFN_BM = 64;          // pair rows per tile
constexpr int FFN_BROWS = 256;      // weight rows per tile (128 gate + 128 up, or 256 outputs)
constexpr int FFN_STAGES = 3;
constexpr int FFN_THREADS = 256;

struct FfnParams {
  const uint8_t* x;
  const int32_t* x_sf;
  const int32_t* topk_idx;
  const float* topk_w;
  const uint8_t* w1;
  const int32_t* w1_sf;
  const uint8_t* w2;
  const int32_t* w2_sf;
  uint16_t* y;
  int T, k, E, offset, H, I;
  int sq_stride;        // bytes per intermediate-scale row (I/128 rounded up to 4)
  int32_t* cnt;         // [E]
  int32_t* start;       // [E+1]
  int32_t* pair_token;  // [T*k]
  int32_t* pair_of;     // [T*k]
  uint8_t* q;           // [T*k, I]
  uint8_t* sq;          // [T*k, sq_stride]
  float* o;             // [T*k, H]
};

struct FfnLayout {
  size_t cnt, start, pair_token, pair_of, q, sq, o, total;
  int sq_stride;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace regions (all 256-byte aligned); P_max = T*k bounds the number of
// (token, slot) pairs routed to local experts for any routing.
static bool ffn_layout(int T, int k, int E, int H, int I, FfnLayout* L) {
  if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return false;
  size_t P = (size_t)T * k;
  L->sq_stride = ((I / 128) + 3) & ~3;
  size_t off = 0;
  L->cnt = off;        off = align256(off + (size_t)E * 4);
  L->start = off;      off = align256(off + (size_t)(E + 1) * 4);
  L->pair_token = off; off = align256(off + P * 4);
  L->pair_of = off;    off = align256(off + P * 4);
  L->q = off;          off = align256(off + P * (size_t)I);
  L->sq = off;         off = align256(off + P * (size_t)L->sq_stride);
  L->o = off;          off = align256(off + P * (size_t)H * 4);
  L->total = off;
  return true;
}

// ---------------------------------------------------------------------------
// 1. routing
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) ffn_route_kernel(FfnParams p) {
  __shared__ int cnt[FFN_MAX_EXPERTS];
  __shared__ int cur[FFN_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int total = p.T * p.k;
  for (int e = tid; e < p.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < total; i += blockDim.x) {
    const int e = p.topk_idx[i] - p.offset;
    if (e >= 0 && e < p.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int e = 0; e < p.E; ++e) {
      p.start[e] = s;
      cur[e] = s;
      p.cnt[e] = cnt[e];
      s += cnt[e];
    }
    p.start[p.E] = s;
  }
  __syncthreads();
  // The order of pairs inside an expert does not affect any result: each pair's
  // output row depends only on its token, and the combine sums slots in order.
  for (int i = tid; i < total; i += blockDim.x) {
    const int e = p.topk_idx[i] - p.offset;
    int pr = -1;
    if (e >= 0 && e < p.E) {
      pr = atomicAdd(&cur[e], 1);
      p.pair_token[pr] = i / p.k;
    }
    p.pair_of[i] = pr;
  }
}

// ---------------------------------------------------------------------------
// 2./3. grouped FP8 x FP4 GEMM (linear1 with SwiGLU + requant, or linear2)
// ---------------------------------------------------------------------------

// 64-byte rows of FP4 weights: 4 chunks of 16 bytes; chunk c of row r sits at
// position c ^ swzb(r) (conflict-free for 16 consecutive rows; depends on r % 16).
__device__ __forceinline__ int swzb(int r) { return ((r >> 1) ^ ((r >> 3) & 1)) & 3; }

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Smallest e with 448 * 2^e >= amax (amax > 0): with amax = f * 2^x, f in [0.5, 1),
// e = x - 9 when f <= 0.875 (448 = 0.875 * 2^9), else x - 8.  0 for amax == 0.
__device__ __forceinline__ int pow2_exponent_448(float amax) {
  if (!(amax > 0.f)) return 0;
  int x;
  const float f = frexpf(amax, &x);
  return f <= 0.875f ? x - 9 : x - 8;
}

// float (|v| <= 448, finite) -> e4m3fn code, round to nearest even.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float m = fabsf(v);
  uint32_t code;
  if (m < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    code = (uint32_t)rintf(m * 512.0f);        // 0..8 (8 is the smallest normal, 0x08)
  } else {
    uint32_t u = __float_as_uint(m);
    u += 0x7ffffu + ((u >> 20) & 1u);          // round the 23-bit mantissa to 3 bits
    code = (u >> 20) - (120u << 3);            // rebias the exponent from 127 to 7
  }
  return sign | code;
}

template <int MODE>   // 1: linear1 (+ SwiGLU + requant), 2: linear2 (fp32 out)
__global__ void __launch_bounds__(FFN_THREADS, 2) ffn_gemm_kernel(FfnParams p) {
  constexpr int A_BYTES = FFN_BM * 128;            // e4m3, 128 K per row
  constexpr int B_BYTES = FFN_BROWS * 64;          // e2m1, 128 K per row
  constexpr int SA_BYTES = FFN_BM * 4;             // one scale word per row
  constexpr int SB_BYTES = FFN_BROWS * 4;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  constexpr int OFF_B = A_BYTES, OFF_SA = A_BYTES + B_BYTES, OFF_SB = OFF_SA + SA_BYTES;
  constexpr int LPS = 2 + 4 + 1 + 1;               // DMA instructions per wave per stage
  __shared__ __attribute__((aligned(16))) uint8_t smem[FFN_STAGES * STAGE];
  __shared__ int tile_base[FFN_MAX_EXPERTS + 1];
  __shared__ float red[4][FFN_BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;

  const int H = p.H, I = p.I, E = p.E;
  const int K = MODE == 1 ? H : I;
  const int KB = K >> 7;
  const int tiles_n = MODE == 1 ? I / 128 : (H + FFN_BROWS - 1) / FFN_BROWS;

  // device-side tile enumeration: expert e owns tiles_m(e) * tiles_n tiles,
  // ordered (n-tile, m-tile) so consecutive tiles share a weight tile
  if (tid == 0) {
    int s = 0;
    for (int e = 0; e < E; ++e) {
      tile_base[e] = s;
      s += ((p.cnt[e] + FFN_BM - 1) / FFN_BM) * tiles_n;
    }
    tile_base[E] = s;
  }
  __syncthreads();
  const int total = tile_base[E];

  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Per-lane LDS read offsets.  In the F8F6F4 instruction an e4m3 operand lane
  // (row, g) holds K [16g, 16g+16) in its first 16 bytes and K [64+16g, 64+16g+16)
  // in the next 16, while an e2m1 operand lane (col, g) holds K [32g, 32g+32)
  // contiguously (low nibble first); so the e4m3 lane reads 16-byte chunks g and
  // g + 4 of its 128-byte row.
  const int sw = swz(lrow);
  const uint32_t a_lo = lrow * 128 + ((lgrp ^ sw) << 4);
  const uint32_t a_hi = lrow * 128 + (((lgrp + 4) ^ sw) << 4);
  // weight rows read by this wave: linear1 gate rows 32w..32w+31 (nt 0,1) and
  // up rows 128+32w.. (nt 2,3); linear2 rows 64w + 16nt
  uint32_t b_rd[4], sb_rd[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int row = MODE == 1 ? ((nt < 2 ? 0 : 128) + wave * 32 + (nt & 1) * 16 + lrow) : (wave * 64 + nt * 16 + lrow);
    b_rd[nt] = OFF_B + row * 64 + ((lgrp ^ swzb(row)) << 4);
    sb_rd[nt] = OFF_SB + row * 4;
  }
  const int dma_arow = lane >> 3;   // A: 8 rows x 128 B per 1 KB region
  const int dma_brow = lane >> 2;   // B: 16 rows x 64 B per 1 KB region

  for (int t = vb; t < total; t += G) {
    // ---------------- tile -> (expert, m-tile, n-tile) ----------------
    int lo = 0, hi = E - 1;
    while (lo < hi) {                            // last e with tile_base[e] <= t
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int cnt_e = p.cnt[e];
    const int tm_e = (cnt_e + FFN_BM - 1) / FFN_BM;
    const int local = t - tile_base[e];
    const int tn = local / tm_e;
    const int tm = local - tn * tm_e;
    const int row0 = p.start[e] + tm * FFN_BM;        // first pair of the tile
    const int rows = min(FFN_BM, cnt_e - tm * FFN_BM); // valid pairs in the tile
    const int last_pair = p.start[e] + cnt_e - 1;

    // ---------------- DMA sources ----------------
    const uint8_t* a_src[2];
    const uint8_t* sa_src;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = (wave * 2 + j) * 8 + dma_arow;
      const int pr = min(row0 + r, last_pair);
      const int chunk = ((lane & 7) ^ swz(r)) << 4;
      if (MODE == 1) a_src[j] = p.x + (size_t)p.pair_token[pr] * H + chunk;
      else a_src[j] = p.q + (size_t)pr * I + chunk;
    }
    {
      const int r = wave * 16 + (lane & 15);
      const int pr = min(row0 + r, last_pair);
      if (MODE == 1) sa_src = reinterpret_cast<const uint8_t*>(p.x_sf + (size_t)p.pair_token[pr] * (H / 512));
      else sa_src = p.sq + (size_t)pr * p.sq_stride;
    }
    const uint8_t* b_src[4];
    const uint8_t* sb_src;
    const size_t wrow_bytes = MODE == 1 ? (size_t)(H / 2) : (size_t)(I / 2);
    const size_t wsf_words = MODE == 1 ? (size_t)(H / 128) : (size_t)(I / 128);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (wave * 4 + j) * 16 + dma_brow;                // tile weight row
      size_t wr;                                                    // expert-local weight row
      if (MODE == 1) wr = (r < 128 ? 0 : I) + tn * 128 + (r & 127);
      else wr = min(tn * FFN_BROWS + r, H - 1);
      const size_t erows = MODE == 1 ? (size_t)2 * I : (size_t)H;
      const uint8_t* wb = MODE == 1 ? p.w1 : p.w2;
      b_src[j] = wb + ((size_t)e * erows + wr) * wrow_bytes + (((lane & 3) ^ swzb(r)) << 4);
    }
    {
      const int r = wave * 64 + lane;
      size_t wr;
      if (MODE == 1) wr = (r < 128 ? 0 : I) + tn * 128 + (r & 127);
      else wr = min(tn * FFN_BROWS + r, H - 1);
      const size_t erows = MODE == 1 ? (size_t)2 * I : (size_t)H;
      const int32_t* ws = MODE == 1 ? p.w1_sf : p.w2_sf;
      sb_src = reinterpret_cast<const uint8_t*>(ws + ((size_t)e * erows + wr) * wsf_words);
    }

    auto issue = [&](int kb, uint32_t slot) {
      uint8_t* base = smem + slot;
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16_to_lds(a_src[j] + kb * 128, base + (wave * 2 + j) * 1024);
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_to_lds(b_src[j] + kb * 64, base + OFF_B + (wave * 4 + j) * 1024);
      // A scale word: four 128-blocks per word for x_sf / sq; lanes 16..63 idle
      if (lane < 16) dma4_to_lds(sa_src + (kb >> 2) * 4, base + OFF_SA + wave * 64);
      dma4_to_lds(sb_src + kb * 4, base + OFF_SB + wave * 256);
    };

    v4f acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < FFN_STAGES - 1; ++s)
      if (s < KB) issue(s, s * STAGE);

    uint32_t rd = 0, wr = (FFN_STAGES - 1) * STAGE;
    for (int kb = 0; kb < KB; ++kb) {
      if (kb + 1 < KB) wait_vmcnt<LPS>();
      else wait_vmcnt<0>();
      block_barrier();
      if (kb + FFN_STAGES - 1 < KB) issue(kb + FFN_STAGES - 1, wr);

      const uint8_t* sbase = smem + rd;
      const int byte_sel = (kb & 3) * 8;
      int sa_s[4];
      v8i af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(sbase + OFF_SA + (mt * 16 + lrow) * 4);
        sa_s[mt] = (int)((w >> byte_sel) & 0xffu);
        v4i l4 = *reinterpret_cast<const v4i*>(sbase + a_lo + mt * 2048);
        v4i h4 = *reinterpret_cast<const v4i*>(sbase + a_hi + mt * 2048);
        af[mt] = v8i{l4.x, l4.y, l4.z, l4.w, h4.x, h4.y, h4.z, h4.w};
      }
      int sb_s[4];
      v8i bfr[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(sbase + sb_rd[nt]);
        sb_s[nt] = (int)((w >> (8 * lgrp)) & 0xffu);
        v4i b4 = *reinterpret_cast<const v4i*>(sbase + b_rd[nt]);
        bfr[nt] = v8i{b4.x, b4.y, b4.z, b4.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = mfma_scaled_e4m3_e2m1_16x16x128(af[mt], sa_s[mt], bfr[nt], sb_s[nt], acc[mt][nt]);

      rd = (rd + STAGE == FFN_STAGES * STAGE) ? 0u : rd + STAGE;
      wr = (wr + STAGE == FFN_STAGES * STAGE) ? 0u : wr + STAGE;
    }
    block_barrier();   // the ring is free before the next tile's prologue

    if (MODE == 2) {
      // fp32 output rows of the pairs
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + 4 * lgrp + i;
          if (r >= rows) continue;
          float* orow = p.o + (size_t)(row0 + r) * H;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const int col = tn * FFN_BROWS + wave * 64 + nt * 16 + lrow;
            if (col < H) orow[col] = acc[mt][nt][i];
          }
        }
    } else {
      // SwiGLU in registers: gate blocks nt = 0,1 pair with up blocks nt = 2,3
      float s[4][2][4];
      float rmax[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float m = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float v = silu_f32(acc[mt][h][i]) * acc[mt][h + 2][i];
            s[mt][h][i] = v;
            m = fmaxf(m, fabsf(v));
          }
          // max over the 16 lanes holding this row's columns (lanes differ in lrow)
#pragma unroll
          for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
          rmax[mt][i] = m;
        }
      if (lrow == 0) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave][mt * 16 + 4 * lgrp + i] = rmax[mt][i];
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + 4 * lgrp + i;
          const float amax = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
          const int ex = pow2_exponent_448(amax);
          if (r >= rows) continue;
          const size_t pr = (size_t)(row0 + r);
          uint8_t* qrow = p.q + pr * I + tn * 128;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = wave * 32 + h * 16 + lrow;
            qrow[col] = (uint8_t)e4m3_rne(ldexpf(s[mt][h][i], -ex));
          }
          if (wave == 0 && lrow == 0) p.sq[pr * p.sq_stride + tn] = (uint8_t)(ex + 127);
        }
      __syncthreads();   // red[] is reused by the next tile
    }
  }
}

// ---------------------------------------------------------------------------
// 4. combine: y[t] = bf16( sum_j w[t,j] * o[pair(t,j)] ), slots in order
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) ffn_combine_kernel(FfnParams p) {
  const int t = blockIdx.y;
  const int c8 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c8 >= p.H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < p.k; ++j) {
    const int pr = p.pair_of[(size_t)t * p.k + j];
    if (pr < 0) continue;
    const float w = p.topk_w[(size_t)t * p.k + j];
    const v4f* src = reinterpret_cast<const v4f*>(p.o + (size_t)pr * p.H + c8);
    const v4f v0 = src[0], v1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = fmaf(w, v0[i], acc[i]);
      acc[4 + i] = fmaf(w, v1[i], acc[4 + i]);
    }
  }
  v4i out;
  out.x = (int)f32_to_bf16_rne(acc[0]) | ((int)f32_to_bf16_rne(acc[1]) << 16);
  out.y = (int)f32_to_bf16_rne(acc[2]) | ((int)f32_to_bf16_rne(acc[3]) << 16);
  out.z = (int)f32_to_bf16_rne(acc[4]) | ((int)f32_to_bf16_rne(acc[5]) << 16);
  out.w = (int)f32_to_bf16_rne(acc[6]) | ((int)f32_to_bf16_rne(acc[7]) << 16);
  *reinterpret_cast<v4i*>(p.y + (size_t)t * p.H + c8) = out;
}

static hipError_t launch_ffn(FfnParams& p, int num_cus, hipStream_t stream) {
  hipLaunchKernelGGL(ffn_route_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = num_cus * 2;
  hipLaunchKernelGGL(ffn_gemm_kernel<1>, dim3(grid), dim3(FFN_THREADS), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_gemm_kernel<2>, dim3(grid), dim3(FFN_THREADS), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 cgrid((p.H / 8 + 255) / 256, p.T);
  hipLaunchKernelGGL(ffn_combine_kernel, cgrid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dg

using namespace dg;

extern "C" {

size_t dg_fp8_fp4_expert_ffn_workspace_bytes(int num_tokens, int num_topk, int num_local_experts, int hidden,
                                             int intermediate) {
  FfnLayout L;
  if (!ffn_layout(num_tokens, num_topk, num_local_experts, hidden, intermediate, &L)) return 0;
  return L.total;
}

int dg_fp8_fp4_expert_ffn(const uint8_t* x, const int32_t* x_sf, const int32_t* topk_idx, const float* topk_w,
                          const uint8_t* w1, const int32_t* w1_sf, const uint8_t* w2, const int32_t* w2_sf,
                          uint16_t* y, int T, int k, int E, int expert_offset, int H, int I, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    if (!x || !x_sf || !topk_idx || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !y || !workspace)
      return DG_ERR_INVALID_ARG;
    if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return DG_ERR_INVALID_ARG;
    if (H % 512 != 0 || I % 128 != 0 || E > FFN_MAX_EXPERTS) return DG_ERR_UNSUPPORTED;
    if ((long long)T * k > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;
    uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w1) |
                   reinterpret_cast<uintptr_t>(w2) | reinterpret_cast<uintptr_t>(y);
    if ((al & 15) || (reinterpret_cast<uintptr_t>(x_sf) & 3) || (reinterpret_cast<uintptr_t>(topk_idx) & 3) ||
        (reinterpret_cast<uintptr_t>(topk_w) & 3) || (reinterpret_cast<uintptr_t>(w1_sf) & 3) ||
        (reinterpret_cast<uintptr_t>(w2_sf) & 3))
      return DG_ERR_INVALID_ARG;
    FfnLayout L;
    ffn_layout(T, k, E, H, I, &L);
    if (workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return DG_ERR_INVALID_ARG;
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    FfnParams p{};
    p.x = x; p.x_sf = x_sf; p.topk_idx = topk_idx; p.topk_w = topk_w;
    p.w1 = w1; p.w1_sf = w1_sf; p.w2 = w2; p.w2_sf = w2_sf; p.y = y;
    p.T = T; p.k = k; p.E = E; p.offset = expert_offset; p.H = H; p.I = I;
    p.sq_stride = L.sq_stride;
    p.cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
    p.start = reinterpret_cast<int32_t*>(ws + L.start);
    p.pair_token = reinterpret_cast<int32_t*>(ws + L.pair_token);
    p.pair_of = reinterpret_cast<int32_t*>(ws + L.pair_of);
    p.q = ws + L.q;
    p.sq = ws + L.sq;
    p.o = reinterpret_cast<float*>(ws + L.o);
    int cus = dg_get_num_cus();
    if (cus <= 0) cus = di.num_cus;
    hipError_t e = launch_ffn(p, cus, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? DG_OK : DG_ERR_HIP;
  } catch (...) {
    return DG_ERR_HIP;
  }
}

}  // extern "C"
