// Device-side helpers shared by the gfx950 kernels: vector types, the CDNA4
// F8F6F4 matrix-core builtins, bf16 rounding, and the LDS swizzle.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>

namespace dg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Operand formats of the F8F6F4 matrix instructions (cbsz/blgp fields).
enum MfmaFmt : int { FMT_E4M3 = 0, FMT_E5M2 = 1, FMT_E2M3 = 2, FMT_E3M2 = 3, FMT_E2M1 = 4 };

// 16x16x128 e4m3 x e4m3 -> fp32.  A lane holds 32 K-consecutive bytes of one
// row (lane % 16) of A / column of B, K chunk (lane / 16); the 16x16 result has
// rows 4*(lane/16) + i (i = 0..3) and column lane % 16 in element i.
// With zero scale operands the compiler emits the unscaled instruction.
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT_E4M3, FMT_E4M3, 0, 0, 0, 0);
}

// ds_read_b64_tr_b8: a transposing LDS read of 8 bytes per lane (lane layout
// documented where it is used).  lds points into shared memory.
__device__ __forceinline__ v2i ds_read_tr8_b64(const uint8_t* lds) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(const_cast<uint8_t*>(lds)));
}

// 16x16x128 e4m3 x e4m3 with hardware block scales: each lane supplies one
// UE8M0 byte for its operand row's K chunk of A and one for B.
__device__ __forceinline__ v4f mfma_scaled_e4m3_16x16x128(const v8i& a, int sa, const v8i& b, int sb,
                                                          const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT_E4M3, FMT_E4M3, 0, sa, 0, sb);
}

// 16x16x128 e4m3 (A) x e2m1 (B) with hardware block scales: each lane supplies
// one UE8M0 byte for its 32-element K chunk of A and one for its chunk of B
// (byte 0 of the given word).  B's 32 FP4 values occupy the low 4 dwords.
__device__ __forceinline__ v4f mfma_scaled_e4m3_e2m1_16x16x128(const v8i& a, int sa, const v8i& b,
                                                               int sb, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT_E4M3, FMT_E2M1, 0, sa, 0, sb);
}

// The same instruction with the operands the other way round: A e2m1 (FP4,
// low 4 dwords), B e4m3; scale bytes as above.
__device__ __forceinline__ v4f mfma_scaled_e2m1_e4m3_16x16x128(const v8i& a, int sa, const v8i& b,
                                                               int sb, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT_E2M1, FMT_E4M3, 0, sa, 0, sb);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Two fp32 -> two bf16 (lo in bits 15:0), one v_cvt_pk_bf16_f32.  Round to nearest
// even; for every non-NaN input the result equals f32_to_bf16_rne bit for bit
// (denormals and overflow to infinity included).  A NaN stays a quiet NaN with
// its payload's top bits (not the canonical 0x7fc0).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// LDS layout of a K-block tile: each row is 128 bytes = 8 chunks of 16 bytes;
// chunk c of row r lives at position c ^ swz(r).  swz spreads any 8 (and any 16)
// consecutive rows that read the same logical chunk over distinct bank groups,
// and depends only on r % 16, so rows r and r + 16k share one pattern (their
// addresses differ by a constant that fits an instruction offset).
__device__ __forceinline__ int swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

// Chunk swizzle of a K-row-major tile (an operand stored with K outermost) read
// with the transposing loads: K row r holds its 16-byte chunk c at c ^ kt_swz(r).
// It depends on r % 8 and bit 5 of r only, so rows r and r + 8i share it.
__device__ __forceinline__ int kt_swz(int r) { return (r & 7) ^ ((r >> 5) & 1); }

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1, in order: a loop
// whose index is a compile-time constant in the body (register arrays indexed by
// it stay in registers, and `if constexpr` can select per iteration).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Waits until at most n vector-memory operations of this wave are outstanding.
// (gfx9 encoding: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at max.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Waits until every LDS access of this wave has completed (lgkmcnt 0; vmcnt
// and expcnt left at max).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence __syncthreads() implies: the
// fence would wait for every outstanding load, including the LDS-DMA loads of
// later pipeline stages.  The empty asm keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource for raw (stride 0) buffer accesses: base address, size in
// bytes (accesses at or beyond it read 0), and the gfx9 format word.
__device__ __forceinline__ v4i make_buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// LLVM's raw buffer load into LDS: lane l's `size` bytes from
// base + voffset(l) + soffset + offset land at lds + l * size (lds wave-uniform).
extern "C" __device__ void dg_raw_buffer_load_lds(v4i rsrc, __attribute__((address_space(3))) uint32_t* lds,
                                                  int size, int voffset, int soffset, int offset,
                                                  int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ void buf16_to_lds(const v4i& rsrc, uint32_t voff, uint32_t soff, void* lds_base) {
  dg_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)lds_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void buf4_to_lds(const v4i& rsrc, uint32_t voff, uint32_t soff, void* lds_base) {
  dg_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)lds_base, 4, (int)voff, (int)soff, 0, 0);
}

// LLVM's raw buffer store of 8 bytes per lane at base + voffset(l) + soffset.
// A lane whose offset lies at or beyond the resource's size stores nothing, so
// a masked-off lane passes an out-of-range offset instead of branching, and
// every lane of the wave always issues exactly one store instruction.
extern "C" __device__ void dg_raw_buffer_store_v2i32(v2i data, v4i rsrc, int voffset, int soffset,
                                                     int aux) __asm("llvm.amdgcn.raw.buffer.store.v2i32");
extern "C" __device__ void dg_raw_buffer_store_v4i32(v4i data, v4i rsrc, int voffset, int soffset,
                                                     int aux) __asm("llvm.amdgcn.raw.buffer.store.v4i32");
constexpr uint32_t kBufferOutOfRange = 0x80000000u;   // valid with resources below 2 GiB
// Cache policy of a buffer access (the intrinsics' aux operand): non-temporal.
// The GEMMs' bf16 outputs are written once and never read back by the kernel, so
// they are stored with it and evict first from L2, which the copies of A and B
// need (measured: masked grouped GEMM 3-8 % faster; fp32 split-K partials, which
// the reduce reads back, keep the default policy).
constexpr int kStoreNonTemporal = 2;

// LLVM's raw buffer loads into registers: lane l reads base + voffset(l) + soffset;
// a lane whose offset lies at or beyond the resource's size reads zeros and sends
// no memory request.
extern "C" __device__ v4i dg_raw_buffer_load_v4i32(v4i rsrc, int voffset, int soffset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
extern "C" __device__ v2i dg_raw_buffer_load_v2i32(v4i rsrc, int voffset, int soffset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.v2i32");

// Direct global -> LDS copies: lane l's 16 (or 4) bytes land at
// lds_base + 16*l (or 4*l).  lds_base must be the same for the whole wave.
__device__ __forceinline__ void dma16_to_lds(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 4, 0, 0);
}

}  // namespace dg
