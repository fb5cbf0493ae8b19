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
//   2. linear1 (persistent, 8 waves): for each (expert, 128-row block of its
//              pairs, 128 intermediate columns) the gathered e4m3 token rows times
//              the matching 128 gate rows and 128 up rows of W1 with
//              v_mfma_scale_f32_16x16x128_f8f6f4 (A e4m3, B e2m1; both UE8M0
//              scales applied by the matrix core per 32-element K chunk), then in
//              registers: s = silu(gate) * up, per-row 128-column amax across the
//              two waves sharing the row (LDS), power-of-two scale, e4m3
//              round-to-nearest-even; writes the e4m3 intermediate and its UE8M0
//              exponents.
//   3. linear2 (persistent): (expert, 128-row block, 256 output columns) of the
//              intermediate times W2 with the same scaled MFMA; writes fp32 per pair,
//              except for a token with a single local pair, whose output row it
//              forms itself (bf16 of w * o, the combine's arithmetic for one slot).
//   4. combine: y[t] = sum over slots j (in order) of w[t,j] * o[pair(t,j)], bf16,
//              for the tokens with no local pair or with two or more.
// Activations and weight-scale words are staged per 128-wide K block through a
// 4-slot LDS ring, the weights per pair of K blocks through a 2-slot ring, and
// the activation-scale words (four K blocks each) through a ring of their own,
// all with LDS-DMA loads (the token gather happens in the DMA addresses).  The
// weight-scale words are K-block-major (written once by the weight
// pre-transform).  Each K block's operand fragments are read into registers
// during the previous block.  The same GEMM kernel also serves the exported
// M-grouped FP8 x FP4 GEMM (contiguous and masked forms, bf16 out).
#include <type_traits>

#include "../../include/dg.h"
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

constexpr int FFN_MAX_EXPERTS = 256;

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
  int32_t* pair_single; // [T*k]: (token, slot) entry of a pair that is its token's only local pair, else -1
  uint8_t* q;           // [T*k, I]
  uint8_t* sq;          // [T*k, sq_stride]
  float* o;             // [T*k, H]
  // standalone M-grouped FP8 x FP4 GEMM (modes 3, 4): D = A_rows . B_g^T in bf16,
  // A = x / x_sf, B = w2 / w2_sf
  int gm, gn, gk;       // rows of A (masked: groups * max_m), N, K
  int groups, max_m;
  const int32_t* m_indices;   // contiguous: group of each row (-1: padding)
  const int32_t* masked_m;    // masked: valid rows per group
  uint16_t* d;
};

struct FfnLayout {
  size_t cnt, start, pair_token, pair_of, q, sq, o, pair_single, total;
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
  L->pair_single = off; off = align256(off + P * 4);
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
  const int nt = blockDim.x;
  // The entries are read RU per thread at a time, all loads issued before any
  // is used (one workgroup: the loop is bound by load latency, not bandwidth).
  // When one batch covers every entry (T * k <= 32768) the second pass reuses
  // the ids the first one read.
  constexpr int RU = 32;
  const bool one_batch = total <= RU * nt;
  int ev[RU];
  for (int e = tid; e < p.E; e += nt) cnt[e] = 0;
  __syncthreads();
  for (int base = 0; base < total; base += RU * nt) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int i = base + u * nt + tid;
      ev[u] = i < total ? p.topk_idx[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int e = ev[u] - p.offset;
      if (base + u * nt + tid < total && e >= 0 && e < p.E) atomicAdd(&cnt[e], 1);
    }
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
  // A pair whose token has no other local pair is marked (its entry index): its
  // token's output row is then formed by linear2.  With k dividing 64 a token's k
  // entries sit in k consecutive lanes of one wave (entry i = base + u * nt + tid,
  // base and u * nt multiples of 64), so one ballot counts them; otherwise the
  // token's entries are read again.
  const bool wave_tokens = 64 % p.k == 0 && nt % 64 == 0;   // (k is then a power of two)
  const int lane = tid & 63;
  const int ksh = wave_tokens ? __builtin_ctz((unsigned)p.k) : 0;
  const int first = wave_tokens ? lane & ~(p.k - 1) : 0;   // the lane of the token's first entry
  const unsigned long long kmask = p.k >= 64 ? ~0ull : (1ull << p.k) - 1ull;
  for (int base = 0; base < total; base += RU * nt) {
    if (!one_batch) {
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int i = base + u * nt + tid;
        ev[u] = i < total ? p.topk_idx[i] : 0;
      }
    }
    // in chunks of CH entries: the pair indices first (the LDS atomics go out
    // back to back), then the stores
    constexpr int CH = 8;
#pragma unroll
    for (int c = 0; c < RU; c += CH) {
      int pr[CH];
#pragma unroll
      for (int v = 0; v < CH; ++v) {
        const int i = base + (c + v) * nt + tid;
        const int e = ev[c + v] - p.offset;
        pr[v] = i < total && e >= 0 && e < p.E ? atomicAdd(&cur[e], 1) : -1;
      }
#pragma unroll
      for (int v = 0; v < CH; ++v) {
        const int i = base + (c + v) * nt + tid;
        int nloc = 0;
        if (wave_tokens) nloc = __popcll((__ballot(pr[v] >= 0) >> first) & kmask);   // (uniform: every lane)
        if (i >= total) continue;
        if (pr[v] >= 0) {
          const int t = wave_tokens ? i >> ksh : i / p.k;
          p.pair_token[pr[v]] = t;
          if (!wave_tokens) {
            for (int j = 0; j < p.k; ++j) {
              const int e2 = p.topk_idx[t * p.k + j] - p.offset;
              nloc += (e2 >= 0 && e2 < p.E) ? 1 : 0;
            }
          }
          p.pair_single[pr[v]] = nloc == 1 ? i : -1;
        }
        p.pair_of[i] = pr[v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2./3. grouped FP8 x FP4 GEMM (linear1 with SwiGLU + requant, or linear2)
// ---------------------------------------------------------------------------

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

// Tile of the grouped GEMM: 128 pair rows x 256 weight rows, 8 waves as 4 x 2,
// each wave 32 rows x 128 weight rows (2 x 8 blocks of 16 x 16).  Each block is
// computed transposed (W_nt . X_mt^T, the FP4 weights as the instruction's first
// operand), so a lane's four results are four consecutive weight rows (output
// columns) of one pair row.  Operand tiles and their scale words go through LDS
// rings by buffer loads; the K position advances the scalar offset only:
//  * per 128-wide K block (4-slot ring): the activation tile and the scale
//    words of both operands;
//  * per pair of K blocks (2-slot ring): the FP4 weight tile.  A weight row
//    holds 64 bytes per K block, so copying two blocks at once makes every copy
//    request a whole 128-byte line (half-line requests move about a third fewer
//    bytes per CU and cycle).
constexpr int FFN_WM = 4, FFN_WN = 2, FFN_MT = 2, FFN_NT = 8;
constexpr int FFN_BM = FFN_WM * FFN_MT * 16;      // 128 pair rows per tile
constexpr int FFN_BN = FFN_WN * FFN_NT * 16;      // 256 weight rows per tile
constexpr int FFN_STAGES = 4;                     // K-block slots (activations, weight scales)
constexpr int FFN_BSTAGES = 2;                    // K-block-pair slots (weights)
constexpr int FFN_SASLOTS = 4;                    // activation-scale slots (four K blocks each)
constexpr int FFN_THREADS = 512;
constexpr int FFN_A_BYTES = FFN_BM * 128;         // e4m3, 128 K per row
constexpr int FFN_SB_BYTES = FFN_BN * 4;          // one weight-scale word per row
constexpr int FFN_STAGE = FFN_A_BYTES + FFN_SB_BYTES;
constexpr int FFN_BPAIR = FFN_BN * 128;           // e2m1, 256 K per row
constexpr int FFN_SASLOT = FFN_BM * 4;            // one activation-scale word per row
constexpr int FFN_LDS = FFN_STAGES * FFN_STAGE + FFN_BSTAGES * FFN_BPAIR + FFN_SASLOTS * FFN_SASLOT;

// MODE 1: linear1 (+ SwiGLU + requant); 2: linear2 (fp32 out); 3 / 4: the
// standalone masked / contiguous M-grouped GEMM (bf16 out).
template <int MODE>
__global__ void __launch_bounds__(FFN_THREADS, 1) ffn_gemm_kernel(FfnParams p) {
  constexpr int NW = FFN_WM * FFN_WN;
  constexpr int MT = FFN_MT, NT = FFN_NT, STAGES = FFN_STAGES, STAGE = FFN_STAGE;
  constexpr int OFF_SB = FFN_A_BYTES;
  constexpr int BRING = FFN_STAGES * FFN_STAGE;    // start of the weight-pair ring
  constexpr int SARING = BRING + FFN_BSTAGES * FFN_BPAIR;   // start of the activation-scale ring
  constexpr int RA = FFN_BM / 8 / NW;              // A regions (8 rows x 128 B) per wave per K block
  constexpr int RB = FFN_BN / 8 / NW;              // B regions (8 rows x 128 B) per wave per K-block pair
  constexpr int SAQ = FFN_BM / 4 / NW;             // A scale words per wave per quarter slot
  constexpr int SBW = FFN_BN / NW;                 // B scale words per wave
  static_assert(SAQ >= 1 && SAQ <= 64 && SBW <= 64, "one scale copy per wave");
  // An activation-scale word holds the exponents of four K blocks, so the words
  // of K-block group q = kb / 4 (all tile rows) are copied once, into slot q % 4
  // of their own ring, a quarter of the rows at a time: staging K block kn
  // copies quarter kn % 4 of group kn / 4 + 1, so group q is complete once K
  // block 4q is (group 0 is copied at the start of the tile).  Weight-scale
  // words (one per row and K block, K-block-major) travel with their K block.
  // Copy instructions per wave: LA per K block (two scale words, A regions),
  // LB more per K-block pair (B regions).  Past the end of a tile's K range the
  // same instructions are issued with out-of-range offsets (they read nothing),
  // so the counts, and the waits below, never change.
  constexpr int LA = RA + 2, LB = RB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int tile_base[FFN_MAX_EXPERTS + 1];
  __shared__ float red[FFN_WN][FFN_BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / FFN_WN;
  const int wave_n = wave % FFN_WN;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;

  constexpr bool GEMM = MODE >= 3;
  const int H = p.H, I = p.I;
  const int E = MODE == 3 ? p.groups : p.E;         // row lists: experts, or masked groups
  const int K = GEMM ? p.gk : (MODE == 1 ? H : I);
  const int KB = K >> 7;
  const int NOUT = GEMM ? p.gn : H;                 // output row length (modes 2-4)
  // H % 512 == 0; the GEMM forms allow N % 16 == 0 (a last, partial column tile)
  const int tiles_n = MODE == 1 ? I / 128 : (NOUT + FFN_BN - 1) / FFN_BN;
  const int tiles_m4 = (p.gm + FFN_BM - 1) / FFN_BM;        // contiguous form: 128-row blocks
  // rows of row list e (expert pairs, or a masked group's valid rows) and where they start
  auto list_cnt = [&](int e) -> int {
    if (MODE == 3) {
      const int mm = p.masked_m[e];
      return mm < 0 ? 0 : (mm > p.max_m ? p.max_m : mm);
    }
    return p.cnt[e];
  };
  auto list_start = [&](int e) -> int { return MODE == 3 ? e * p.max_m : p.start[e]; };

  // device-side tile enumeration: row list e owns tiles_m(e) * tiles_n tiles,
  // ordered (n-tile, m-tile) so that consecutive tiles share a weight tile; the
  // contiguous form walks (n-tile, 128-row block) and skips padding blocks
  if (MODE != 4 && tid == 0) {
    int s = 0;
    for (int e = 0; e < E; ++e) {
      tile_base[e] = s;
      s += ((list_cnt(e) + FFN_BM - 1) / FFN_BM) * tiles_n;
    }
    tile_base[E] = s;
  }
  __syncthreads();
  const int total = MODE == 4 ? tiles_m4 * tiles_n : tile_base[E];

  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Per-lane LDS read offsets.  An e4m3 operand lane (row, g) of the F8F6F4
  // instruction holds K [16g, 16g+16) and [64+16g, 64+16g+16), so it reads the
  // 16-byte chunks g and g+4 of its 128-byte row; an e2m1 lane (row, g) holds
  // K [32g, 32g+32): chunk g of its 64-byte row.
  const int sw = swz(lrow);
  const uint32_t a_lo = (wave_m * MT * 16 + lrow) * 128 + ((lgrp ^ sw) << 4);
  const uint32_t a_hi = (wave_m * MT * 16 + lrow) * 128 + (((lgrp + 4) ^ sw) << 4);
  const uint32_t sa_rd = SARING + (wave_m * MT * 16 + lrow) * 4;
  // weight rows of block nt: linear1 gate rows 64*wn + 16nt (nt < 4) and the
  // matching up rows 128 + 64*wn + 16(nt-4); linear2 output rows 128*wn + 16nt.
  // A weight row in the pair ring holds 8 chunks of 16 bytes (chunks 0-3: the
  // even K block, 4-7: the odd one), chunk c at position c ^ swz(row); an e2m1
  // lane (row, g) reads chunk g of its K block.
  uint32_t b_rd[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = MODE == 1 ? ((nt < 4 ? 0 : 128) + wave_n * 64 + (nt & 3) * 16 + lrow)
                              : (wave_n * 128 + nt * 16 + lrow);
    b_rd[nt] = row * 128;
  }
  const uint32_t b_ch[2] = {(uint32_t)((lgrp ^ sw) << 4), (uint32_t)(((4 + lgrp) ^ sw) << 4)};
  const uint32_t sb_rd0 = OFF_SB + (MODE == 1 ? wave_n * 64 + lrow : wave_n * 128 + lrow) * 4;

  const uint8_t* a_base = MODE == 2 ? p.q : p.x;
  const size_t a_rows = MODE == 1 ? (size_t)p.T : (GEMM ? (size_t)p.gm : (size_t)p.T * p.k);
  // bytes per A-scale row: one word per four K blocks
  const uint32_t sa_stride = MODE == 1 ? (uint32_t)(H / 512) * 4u
                                       : (MODE == 2 ? (uint32_t)p.sq_stride : (uint32_t)((KB + 3) / 4) * 4u);
  const v4i rsA = make_buffer_rsrc(a_base, (uint32_t)(a_rows * (size_t)K));
  const v4i rsSA = make_buffer_rsrc(MODE == 2 ? (const void*)p.sq : (const void*)p.x_sf,
                                    (uint32_t)(a_rows * sa_stride));
  const uint32_t wrow_bytes = (uint32_t)K / 2;
  const uint32_t e_rows = MODE == 1 ? 2u * I : (uint32_t)NOUT;
  const uint32_t wsf_kb_bytes = e_rows * 4u;        // weight-scale words of one K block (K-block-major)

  for (int t = vb; t < total; t += G) {
    // ---------------- tile -> (row list / group e, m-tile, n-tile) ----------------
    int e, tn, row0, rows, last_pair;
    if (MODE == 4) {
      int tm;
      raster_tile(t, tiles_m4, tiles_n, 8, &tm, &tn);
      row0 = tm * FFN_BM;
      e = p.m_indices[row0];
      if (e < 0 || e >= p.groups) continue;       // padding block (uniform: skip the tile)
      rows = min(FFN_BM, p.gm - row0);
      last_pair = p.gm - 1;
    } else {
      int lo = 0, hi = E - 1;
      while (lo < hi) {                          // last e with tile_base[e] <= t
        const int mid = (lo + hi + 1) >> 1;
        if (tile_base[mid] <= t) lo = mid; else hi = mid - 1;
      }
      e = lo;
      const int cnt_e = list_cnt(e);
      const int tm_e = (cnt_e + FFN_BM - 1) / FFN_BM;
      int tm;
      raster_tile(t - tile_base[e], tm_e, tiles_n, 8, &tm, &tn);
      row0 = list_start(e) + tm * FFN_BM;        // first row (pair) of the tile
      rows = min(FFN_BM, cnt_e - tm * FFN_BM);   // valid rows in the tile
      last_pair = list_start(e) + cnt_e - 1;
    }

    // linear2: the (token, slot) entry of each of the lane's rows if it is its
    // token's only local pair, else -1 (read before this tile's copies)
    int single[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = wave_m * MT * 16 + mt * 16 + lrow;
      single[mt] = MODE == 2 && r < rows ? p.pair_single[row0 + r] : -1;
    }

    // ---------------- copy sources (per-lane offsets, scalar K offsets) ----------------
    const uint8_t* wb = MODE == 1 ? p.w1 : p.w2;
    const int32_t* wsf = MODE == 1 ? p.w1_sf : p.w2_sf;
    const v4i rsB = make_buffer_rsrc(wb + (size_t)e * e_rows * wrow_bytes, e_rows * wrow_bytes);
    const v4i rsSB = make_buffer_rsrc(wsf + (size_t)e * e_rows * (K / 128), e_rows * (uint32_t)(K / 128) * 4u);
    uint32_t a_off[RA], b_off[RB], sa_off[4], sb_off;
#pragma unroll
    for (int j = 0; j < RA; ++j) {
      const int r = (wave * RA + j) * 8 + (lane >> 3);
      const int pr = min(row0 + r, last_pair);
      const uint32_t src_row = MODE == 1 ? (uint32_t)p.pair_token[pr] : (uint32_t)pr;
      a_off[j] = src_row * (uint32_t)K + (((lane & 7) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int r = (wave * RB + j) * 8 + (lane >> 3);             // tile weight row
      const uint32_t wr = MODE == 1 ? (uint32_t)((r < 128 ? 0 : I) + tn * 128 + (r & 127))
                                    : (uint32_t)(tn * FFN_BN + r);
      b_off[j] = wr < e_rows ? wr * wrow_bytes + (((lane & 7) ^ swz(r)) << 4) : kBufferOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {                 // scale-word quarter j: rows j*BM/4 + wave*SAQ + lane
      const int r = j * (FFN_BM / 4) + wave * SAQ + (lane < SAQ ? lane : 0);
      const int pr = min(row0 + r, last_pair);
      sa_off[j] = MODE == 1 ? (uint32_t)p.pair_token[pr] * sa_stride : (uint32_t)pr * sa_stride;
    }
    {
      const int r = wave * SBW + (lane < SBW ? lane : 0);
      const uint32_t wr = MODE == 1 ? (uint32_t)((r < 128 ? 0 : I) + tn * 128 + (r & 127))
                                    : (uint32_t)(tn * FFN_BN + r);
      sb_off = wr < e_rows ? wr * 4u : kBufferOutOfRange;   // rows past N: a partial last tile
    }
    const int NPAIR = (KB + 1) >> 1;
    // activation-scale quarter j of K-block group q into its slot (q beyond the K range: read nothing)
    // (j is a compile-time quarter so that sa_off stays in registers)
    auto issue_sa = [&](int q, auto j_tag) {
      constexpr int j = decltype(j_tag)::value;
      const bool live = q * 4 < KB;
      if (SAQ == 64 || lane < SAQ)
        buf4_to_lds(rsSA, live ? sa_off[j] : kBufferOutOfRange, (uint32_t)(live ? q : 0) * 4u,
                    smem + SARING + (q & 3) * FFN_SASLOT + (j * (FFN_BM / 4) + wave * SAQ) * 4);
    };
    // scale copies that travel with K block kb (staged into A-ring slot `slot`;
    // kb >= KB: read nothing); kb % 4 == decltype(j_tag)::value
    auto issue_scales = [&](int kb, uint32_t slot, auto j_tag) {
      issue_sa((kb >> 2) + 1, j_tag);
      const bool live = kb < KB;
      if (SBW == 64 || lane < SBW)
        buf4_to_lds(rsSB, live ? sb_off : kBufferOutOfRange, (uint32_t)(live ? kb : 0) * wsf_kb_bytes,
                    smem + slot + OFF_SB + wave * SBW * 4);
    };
    auto issue_a = [&](int j, int kb, uint32_t slot) {
      const bool live = kb < KB;
      buf16_to_lds(rsA, live ? a_off[j] : kBufferOutOfRange, (uint32_t)(live ? kb : 0) * 128u,
                   smem + slot + (wave * RA + j) * 1024);
    };
    // copies of K-block pair pp into pair slot `bslot` (pp >= NPAIR: read nothing)
    auto issue_b = [&](int j, int pp, uint32_t bslot) {
      const bool live = pp < NPAIR;
      buf16_to_lds(rsB, live ? b_off[j] : kBufferOutOfRange, (uint32_t)(live ? pp : 0) * 128u,
                   smem + BRING + bslot + (wave * RB + j) * 1024);
    };

    v4f acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

    // Operand fragments live in two register sets: block kb multiplies set
    // kb % 2, read from LDS during block kb - 1, while it reads K block kb + 1
    // into the other set.  The LDS reads thus never hold up the matrix
    // instructions, and a block's barrier also certifies that every wave has
    // read stage kb, whose A slot is then refilled (with K block kb + 4).
    v8i af[2][MT], bfr[2][NT];
    uint32_t saw[2][MT], sbw[2][NT];   // scale words; the exponent byte is taken at use
    // Part `part` of the fragments of K block kb (kb % 4 == PH) into set PH % 2:
    // parts 0 .. MT-1 the A fragments (two 16-byte reads each), MT .. MT+NT-1
    // the B fragments, then the A scale words and the B scale words.
    constexpr int NPARTS = MT + NT + 2;
    auto read_part = [&](int kb, auto ph_tag, auto part_tag) {
      constexpr int PH = decltype(ph_tag)::value, S = PH & 1, P = decltype(part_tag)::value;
      const uint8_t* sbase = smem + PH * STAGE;
      if constexpr (P < MT) {
        const v4i l4 = *reinterpret_cast<const v4i*>(sbase + a_lo + P * 2048);
        const v4i h4 = *reinterpret_cast<const v4i*>(sbase + a_hi + P * 2048);
        af[S][P] = v8i{l4.x, l4.y, l4.z, l4.w, h4.x, h4.y, h4.z, h4.w};
      } else if constexpr (P < MT + NT) {
        const uint8_t* bbase = smem + BRING + (uint32_t)((PH >> 1) & 1) * FFN_BPAIR + b_ch[S];
        const v4i b4 = *reinterpret_cast<const v4i*>(bbase + b_rd[P - MT]);
        bfr[S][P - MT] = v8i{b4.x, b4.y, b4.z, b4.w, 0, 0, 0, 0};
      } else if constexpr (P == MT + NT) {
        const uint8_t* sabase = smem + (uint32_t)((kb >> 2) & 3) * FFN_SASLOT;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) saw[S][mt] = *reinterpret_cast<const uint32_t*>(sabase + sa_rd + mt * 64);
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row_off = MODE == 1 ? ((nt < 4 ? 0 : 128) + (nt & 3) * 16) : nt * 16;
          sbw[S][nt] = *reinterpret_cast<const uint32_t*>(sbase + sb_rd0 + row_off * 4);
        }
      }
    };
    auto read_frags = [&](int kb, auto ph_tag) {
      static_for<NPARTS>([&](auto part_tag) { read_part(kb, ph_tag, part_tag); });
    };

    // Prologue: activation-scale group 0, weight pair 0, K blocks 0 and 1,
    // weight pair 1, K blocks 2 and 3; then K block 0's fragments.  Block kb
    // copies K block kb + 4 (into the slot of K block kb) and, when kb is odd,
    // weight pair (kb + 3) / 2 (into the slot of pair (kb - 1) / 2, whose last
    // K block was read in block kb - 1).
    static_assert(STAGES == 4, "four A-ring slots: the slot of K block kb is kb % 4");
    issue_sa(0, std::integral_constant<int, 0>{});
    issue_sa(0, std::integral_constant<int, 1>{});
    issue_sa(0, std::integral_constant<int, 2>{});
    issue_sa(0, std::integral_constant<int, 3>{});
#pragma unroll
    for (int j = 0; j < RB; ++j) issue_b(j, 0, 0);
    issue_scales(0, 0u, std::integral_constant<int, 0>{});
#pragma unroll
    for (int j = 0; j < RA; ++j) issue_a(j, 0, 0u);
    issue_scales(1, (uint32_t)STAGE, std::integral_constant<int, 1>{});
#pragma unroll
    for (int j = 0; j < RA; ++j) issue_a(j, 1, (uint32_t)STAGE);
#pragma unroll
    for (int j = 0; j < RB; ++j) issue_b(j, 1, (uint32_t)FFN_BPAIR);
    issue_scales(2, 2u * STAGE, std::integral_constant<int, 2>{});
#pragma unroll
    for (int j = 0; j < RA; ++j) issue_a(j, 2, 2u * STAGE);
    issue_scales(3, 3u * STAGE, std::integral_constant<int, 3>{});
#pragma unroll
    for (int j = 0; j < RA; ++j) issue_a(j, 3, 3u * STAGE);
    wait_vmcnt<3 * LA + LB>();   // K block 0, pair 0 and scale group 0 have landed
    block_barrier();
    read_frags(0, std::integral_constant<int, 0>{});

    // One K block; PH = kb % 4.  The copy instructions are spread between the
    // matrix instructions (a copy that finds the memory pipeline full stalls the
    // wave; spread out, matrix work is queued meanwhile), pinned with scheduling
    // group barriers: the scale words first, then the A regions, then (odd
    // blocks) the weight pair.
    auto kstep = [&](int kb, auto ph_tag) {
      constexpr int PH = decltype(ph_tag)::value, S = PH & 1;
      constexpr bool ODD = (PH & 1) != 0;
      constexpr int ILV = RA + (ODD ? RB : 0);
      constexpr int ILV_STEP = (MT * NT) / ILV;
      // K block kb + 1 (and its weight pair) has landed once at most this many
      // copies remain (a wave's loads retire in issue order):
      //  * even kb: K block kb + 1 and its pair were copied in block kb - 3 (the
      //    pair last); younger are blocks kb - 2 (LA) and kb - 1 (LA + LB);
      //  * odd kb >= 3: the pair of K block kb + 1 was the last copy of block
      //    kb - 2; younger is block kb - 1 (LA);
      //  * kb = 1: pair 1 came before the prologue's K blocks 2 and 3 and block
      //    0's copies (K block 2 is older than K block 3).
      if (ODD) {
        if (kb == 1) wait_vmcnt<2 * LA>();
        else wait_vmcnt<LA>();
      } else {
        wait_vmcnt<2 * LA + LB>();
      }
      wait_lgkmcnt0();   // this wave's reads of K block kb are done ...
      block_barrier();   // ... and every wave's: its slot can be refilled
      const int kn = kb + 4;                       // K block copied in this block
      const int pn = (kb + 3) >> 1;                // weight pair copied in this block (odd kb)
      constexpr uint32_t wr = PH * STAGE;
      constexpr uint32_t bwr = (uint32_t)(((PH + 3) >> 1) & 1) * FFN_BPAIR;
      issue_scales(kn, wr, std::integral_constant<int, PH>{});

      constexpr int byte_sel = PH * 8;
      int sa_s[MT], sb_s[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sa_s[mt] = (int)((saw[S][mt] >> byte_sel) & 0xffu);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sb_s[nt] = (int)((sbw[S][nt] >> (8 * lgrp)) & 0xffu);
      // matrix instruction j is followed by read part j of K block kb + 1 (the
      // LDS reads spread over the block keep them off the barrier's critical
      // path) and, every ILV_STEP-th, by one copy
      static_for<MT * NT>([&](auto j_tag) {
        constexpr int j = decltype(j_tag)::value, mt = j / NT, nt = j % NT;
        acc[mt][nt] = mfma_scaled_e2m1_e4m3_16x16x128(bfr[S][nt], sb_s[nt], af[S][mt], sa_s[mt], acc[mt][nt]);
        constexpr bool copy_here = j % ILV_STEP == ILV_STEP - 1 && j / ILV_STEP < ILV;
        if constexpr (j < NPARTS) read_part(kb + 1, std::integral_constant<int, (PH + 1) & 3>{}, j_tag);
        if constexpr (copy_here) {
          constexpr int idx = j / ILV_STEP;
          if constexpr (idx < RA) issue_a(idx, kn, wr);
          else issue_b(idx - RA, pn, bwr);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // 1 MFMA
        if constexpr (j < NPARTS)
          __builtin_amdgcn_sched_group_barrier(0x100, j < MT ? 2 : (j < MT + NT ? 1 : (j == MT + NT ? 1 : 4)), 0);
        if constexpr (copy_here) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // then 1 copy
      });
    };
#pragma clang loop unroll(disable)
    for (int kb = 0; kb < KB; kb += 4) {
      kstep(kb, std::integral_constant<int, 0>{});
      if (kb + 1 < KB) kstep(kb + 1, std::integral_constant<int, 1>{});
      if (kb + 2 < KB) kstep(kb + 2, std::integral_constant<int, 2>{});
      if (kb + 3 < KB) kstep(kb + 3, std::integral_constant<int, 3>{});
    }
    wait_vmcnt<0>();   // the trailing copies (of nothing) have retired
    wait_lgkmcnt0();   // and the last block's reads (of K block KB)
    block_barrier();   // the ring is free before the next tile's prologue

    if (GEMM) {
      // bf16 D rows: 4 consecutive columns (8 bytes) per lane and block; contiguous
      // form: only rows of this block's group (padding rows keep their contents)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = wave_m * MT * 16 + mt * 16 + lrow;
        if (r >= rows) continue;
        if (MODE == 4 && p.m_indices[row0 + r] != e) continue;
        uint16_t* drow = p.d + (size_t)(row0 + r) * NOUT + tn * FFN_BN + wave_n * 128 + 4 * lgrp;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (tn * FFN_BN + wave_n * 128 + nt * 16 >= NOUT) break;   // columns past N (N % 16 == 0)
          const v4f v = acc[mt][nt];
          *reinterpret_cast<uint2*>(drow + nt * 16) = uint2{pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3])};
        }
      }
    } else if (MODE == 2) {
      // fp32 output rows of the pairs: 4 consecutive columns (16 bytes) per lane
      // and block; the only local pair of a token gives that token's bf16 output
      // row instead, w * o rounded once as the combine does for a single slot
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = wave_m * MT * 16 + mt * 16 + lrow;
        if (r >= rows) continue;
        const int col = tn * FFN_BN + wave_n * 128 + 4 * lgrp;
        if (single[mt] >= 0) {
          const float w = p.topk_w[single[mt]];
          uint16_t* yrow = p.y + (size_t)(single[mt] / p.k) * H + col;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const v4f v = acc[mt][nt];
            *reinterpret_cast<uint2*>(yrow + nt * 16) =
                uint2{pack_bf16x2_rne(fmaf(w, v[0], 0.f), fmaf(w, v[1], 0.f)),
                      pack_bf16x2_rne(fmaf(w, v[2], 0.f), fmaf(w, v[3], 0.f))};
          }
        } else {
          float* orow = p.o + (size_t)(row0 + r) * H + col;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<v4f*>(orow + nt * 16) = acc[mt][nt];
        }
      }
    } else {
      // SwiGLU in registers: gate block nt pairs with up block nt + 4 (same columns)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = wave_m * MT * 16 + mt * 16 + lrow;
        float sv[4][4];
        float m = 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = silu_f32(acc[mt][nt][i]) * acc[mt][nt + 4][i];
            sv[nt][i] = v;
            m = fmaxf(m, fabsf(v));
          }
        // this wave's 64 columns of the row sit in the four lanes lrow + 16g
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lgrp == 0) red[wave_n][r] = m;
        __syncthreads();
        const float amax = fmaxf(red[0][r], red[1][r]);
        const int ex = pow2_exponent_448(amax);
        if (r < rows) {
          const size_t pr = (size_t)(row0 + r);
          uint8_t* qrow = p.q + pr * I + tn * 128 + wave_n * 64 + 4 * lgrp;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) w |= e4m3_rne(ldexpf(sv[nt][i], -ex)) << (8 * i);
            *reinterpret_cast<uint32_t*>(qrow + nt * 16) = w;
          }
          if (wave_n == 0 && lgrp == 0) p.sq[pr * p.sq_stride + tn] = (uint8_t)(ex + 127);
        }
        __syncthreads();   // red[] is rewritten by the next row block
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4. combine: y[t] = bf16( sum_j w[t,j] * o[pair(t,j)] ), slots in order (a
// token with exactly one local pair has its row from linear2)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) ffn_combine_kernel(FfnParams p) {
  const int t = blockIdx.y;
  const int c8 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c8 >= p.H) return;
  int nloc = 0;
  for (int j = 0; j < p.k; ++j) nloc += p.pair_of[(size_t)t * p.k + j] >= 0 ? 1 : 0;
  if (nloc == 1) return;
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
  out.x = (int)pack_bf16x2_rne(acc[0], acc[1]);
  out.y = (int)pack_bf16x2_rne(acc[2], acc[3]);
  out.z = (int)pack_bf16x2_rne(acc[4], acc[5]);
  out.w = (int)pack_bf16x2_rne(acc[6], acc[7]);
  *reinterpret_cast<v4i*>(p.y + (size_t)t * p.H + c8) = out;
}

static hipError_t launch_ffn(FfnParams& p, int num_cus, hipStream_t stream) {
  hipLaunchKernelGGL(ffn_route_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static const hipError_t attr1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_kernel<1>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, FFN_LDS);
  static const hipError_t attr2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_kernel<2>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, FFN_LDS);
  if (attr1 != hipSuccess) return attr1;
  if (attr2 != hipSuccess) return attr2;
  const int grid = num_cus;
  hipLaunchKernelGGL(ffn_gemm_kernel<1>, dim3(grid), dim3(FFN_THREADS), FFN_LDS, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_gemm_kernel<2>, dim3(grid), dim3(FFN_THREADS), FFN_LDS, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 cgrid((p.H / 8 + 255) / 256, p.T);
  hipLaunchKernelGGL(ffn_combine_kernel, cgrid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// weight pre-transform: packed UE8M0 weight-scale words [G][N][KB] -> [G][KB][N]
// (K-block-major), 64 x 64 words at a time through LDS so that both the reads
// (along K) and the writes (along N) are contiguous
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) fp4_sf_transpose_kernel(const int32_t* in, int32_t* out, int n, int kb) {
  __shared__ int32_t tile[64][65];
  const size_t gbase = (size_t)blockIdx.z * n * kb;
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4)
    if (n0 + r < n && k0 + tx < kb) tile[r][tx] = in[gbase + (size_t)(n0 + r) * kb + k0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4)
    if (k0 + r < kb && n0 + tx < n) out[gbase + (size_t)(k0 + r) * n + n0 + tx] = tile[tx][r];
}

}  // namespace dg

using namespace dg;

static hipError_t launch_gemm4(FfnParams& p, bool masked, int num_cus, hipStream_t stream) {
  static const hipError_t attr3 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_kernel<3>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, FFN_LDS);
  static const hipError_t attr4 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_kernel<4>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, FFN_LDS);
  if (attr3 != hipSuccess) return attr3;
  if (attr4 != hipSuccess) return attr4;
  if (masked)
    hipLaunchKernelGGL(ffn_gemm_kernel<3>, dim3(num_cus), dim3(FFN_THREADS), FFN_LDS, stream, p);
  else
    hipLaunchKernelGGL(ffn_gemm_kernel<4>, dim3(num_cus), dim3(FFN_THREADS), FFN_LDS, stream, p);
  return hipGetLastError();
}

// Checks shared by the two exported forms; rows = rows of A (and D).
static int gemm4_check(const uint8_t* a, const int32_t* a_sf, const uint8_t* b, const int32_t* b_sf,
                       const int32_t* meta, uint16_t* d, long long rows, int n, int k, int groups) {
  if (!a || !a_sf || !b || !b_sf || !meta || !d) return DG_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || k <= 0 || groups <= 0) return DG_ERR_INVALID_ARG;
  if (k % 128 != 0 || n % 16 != 0) return DG_ERR_UNSUPPORTED;
  const long long lim = 1LL << 31;
  if (rows * k > lim || (long long)n * (k / 2) > lim || rows * 4LL * ((k / 128 + 3) / 4) > lim ||
      (long long)n * (k / 128) * 4 > lim)
    return DG_ERR_UNSUPPORTED;
  const uintptr_t al16 = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                         reinterpret_cast<uintptr_t>(d);
  const uintptr_t al4 = reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf) |
                        reinterpret_cast<uintptr_t>(meta);
  if ((al16 & 15) || (al4 & 3)) return DG_ERR_INVALID_ARG;
  return DG_OK;
}

extern "C" {

int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const uint8_t* a, const int32_t* a_sf, const uint8_t* b,
                                            const int32_t* b_sf, const int32_t* m_indices, uint16_t* d,
                                            int m, int n, int k, int num_groups, void* stream) {
  try {
    const int st = gemm4_check(a, a_sf, b, b_sf, m_indices, d, m, n, k, num_groups);
    if (st != DG_OK) return st;
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    FfnParams p{};
    p.x = a; p.x_sf = a_sf; p.w2 = b; p.w2_sf = b_sf; p.d = d; p.m_indices = m_indices;
    p.gm = m; p.gn = n; p.gk = k; p.groups = num_groups;
    int cus = dg_get_num_cus();
    if (cus <= 0) cus = di.num_cus;
    const hipError_t e = launch_gemm4(p, false, cus, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? DG_OK : DG_ERR_HIP;
  } catch (...) {
    return DG_ERR_HIP;
  }
}

int dg_m_grouped_fp8_fp4_gemm_nt_masked(const uint8_t* a, const int32_t* a_sf, const uint8_t* b,
                                        const int32_t* b_sf, const int32_t* masked_m, uint16_t* d,
                                        int num_groups, int max_m, int n, int k, int expected_m,
                                        void* stream) {
  (void)expected_m;
  try {
    if (max_m <= 0) return DG_ERR_INVALID_ARG;
    const int st = gemm4_check(a, a_sf, b, b_sf, masked_m, d, (long long)num_groups * max_m, n, k, num_groups);
    if (st != DG_OK) return st;
    if (num_groups > FFN_MAX_EXPERTS) return DG_ERR_UNSUPPORTED;
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    FfnParams p{};
    p.x = a; p.x_sf = a_sf; p.w2 = b; p.w2_sf = b_sf; p.d = d; p.masked_m = masked_m;
    p.gm = num_groups * max_m; p.gn = n; p.gk = k; p.groups = num_groups; p.max_m = max_m;
    int cus = dg_get_num_cus();
    if (cus <= 0) cus = di.num_cus;
    const hipError_t e = launch_gemm4(p, true, cus, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? DG_OK : DG_ERR_HIP;
  } catch (...) {
    return DG_ERR_HIP;
  }
}

int dg_transform_fp4_weight_sf(const int32_t* sf, int32_t* sf_t, int num_groups, int n, int k, void* stream) {
  try {
    if (!sf || !sf_t || num_groups <= 0 || n <= 0 || k <= 0) return DG_ERR_INVALID_ARG;
    if (k % 128 != 0) return DG_ERR_UNSUPPORTED;
    if (num_groups > 65535) return DG_ERR_UNSUPPORTED;
    const size_t bytes = (size_t)num_groups * n * (k / 128) * 4;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(sf), lo_t = reinterpret_cast<uintptr_t>(sf_t);
    if (((lo | lo_t) & 3) || (lo < lo_t + bytes && lo_t < lo + bytes)) return DG_ERR_INVALID_ARG;
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    const int kb = k / 128;
    hipLaunchKernelGGL(fp4_sf_transpose_kernel, dim3((n + 63) / 64, (kb + 63) / 64, num_groups), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), sf, sf_t, n, kb);
    return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
  } catch (...) {
    return DG_ERR_HIP;
  }
}

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
    // the GEMM kernels address x, the intermediate and one expert's weights
    // through buffer resources with 32-bit offsets
    const long long lim = 1LL << 31;
    if ((long long)T * H > lim || (long long)T * k * I > lim || (long long)T * k * ((I / 128 + 3) & ~3) > lim ||
        (long long)I * H > lim)
      return DG_ERR_UNSUPPORTED;
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
    p.pair_single = reinterpret_cast<int32_t*>(ws + L.pair_single);
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
