// C-ABI entry points (declared in include/dg.h): argument validation, device
// facts, tile planning and kernel launch.  Validation runs on the host before
// any HIP call; no exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/dg.h"
#include "dg_internal.hpp"

namespace dg {

static std::atomic<int> g_cu_cap{0};
static std::mutex g_dev_mu;
struct DevCache {
  bool probed = false;
  bool ok = false;
  int num_cus = 0;
};
static DevCache g_dev_cache[64];

DeviceInfo current_device_info() {
  DeviceInfo info{-1, 0, false};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return info;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevCache& c = g_dev_cache[dev];
  if (!c.probed) {
    c.probed = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      c.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      c.num_cus = prop.multiProcessorCount;
    } else {
      (void)hipGetLastError();
    }
  }
  info.device = dev;
  info.ok = c.ok;
  info.num_cus = c.num_cus;
  return info;
}

static int effective_cus(const DeviceInfo& di) {
  int cap = g_cu_cap.load();
  if (cap <= 0) {
    const char* env = std::getenv("DG_NUM_CUS");
    if (env) cap = std::atoi(env);
  }
  if (cap > 0 && cap < di.num_cus) return cap;
  return di.num_cus;
}

static bool log_enabled() {
  const char* env = std::getenv("DG_LOG");
  return env && env[0] == '1';
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels address A, B, C and D (one group's share of them) through buffer
// resources with 32-bit offsets and park masked-off stores at offset 2^31, so
// each of these operands must span at most 2 GiB.
static bool fits_buffer(long long rows, long long cols, long long elem_bytes) {
  return rows * cols * elem_bytes <= (1LL << 31);
}
static bool operands_fit(int m, int n, int k) {
  return fits_buffer(m, k, 1) && fits_buffer(n, k, 1) && fits_buffer(m, n, 2);
}

// Split-K workspace: one fp32 buffer per (device, stream), grown on demand and
// kept until the process ends, so calls on one stream reuse it in stream order.
static std::mutex g_ws_mu;
static std::map<std::pair<int, void*>, std::pair<void*, size_t>> g_ws;

static float* split_workspace(int dev, hipStream_t stream, size_t bytes, hipError_t* err) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto& e = g_ws[{dev, reinterpret_cast<void*>(stream)}];
  if (e.second < bytes) {
    if (e.first) {
      // earlier calls on this stream may still read the old buffer
      hipError_t r = hipStreamSynchronize(stream);
      if (r == hipSuccess) r = hipFree(e.first);
      e = {nullptr, 0};
      if (r != hipSuccess) {
        *err = r;
        return nullptr;
      }
    }
    void* ptr = nullptr;
    hipError_t r = hipMalloc(&ptr, bytes);
    if (r != hipSuccess) {
      *err = r;
      return nullptr;
    }
    e = {ptr, bytes};
  }
  return static_cast<float*>(e.first);
}

// flags: MODE_UE8M0 and / or MODE_NN, or-ed into the form's mode at launch
static int run_fp8_gemm(Fp8GemmParams& p, int mode, int expected_m, void* stream, const char* name,
                        int flags = 0) {
  DeviceInfo di = current_device_info();
  if (!di.ok) return DG_ERR_NO_DEVICE;
  int cus = effective_cus(di);
  const int bm_multiple = (flags & MODE_AT) ? 128 : 0;   // A stored [K][M]: 128-row sub-tiles
  // K-grouped: plan for a group's mean K
  const int k_plan = mode == MODE_KGROUP ? std::max(128, p.k / p.num_groups / 128 * 128) : p.k;
  GemmPlan plan = plan_fp8_gemm(p.m, p.n, k_plan, p.num_groups, mode, cus, expected_m, bm_multiple);
  if (plan.kernel_id < 0) return DG_ERR_UNSUPPORTED;
  // DG_FORCE_KERNEL=<id>: override the heuristic's tile choice (for tuning)
  if (const char* fk = std::getenv("DG_FORCE_KERNEL")) {
    int id = std::atoi(fk);
    if (id >= 0 && id < num_tile_configs() &&
        !(mode == MODE_CONTIG && (128 % tile_config(id).block_m) != 0) &&
        !(bm_multiple > 0 && tile_config(id).block_m % bm_multiple != 0))
      plan = plan_with_kernel(p.m, p.n, p.k, p.num_groups, mode, cus, id);
  }
  p.tiles_m = plan.tiles_m;
  p.tiles_n = plan.tiles_n;
  p.splits = plan.splits;
  p.kb_per_split = plan.kb_per_split;
  p.full_tiles = plan.full_tiles;
  p.total_tiles = (int)std::min<long long>(
      (long long)plan.full_tiles + (long long)(plan.num_tiles - plan.full_tiles) * plan.splits, 0x7fffffff);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // Masked form: the kernel walks only the tiles holding valid rows, spread
  // evenly over one full set of workgroup slots, and over long K splits a small
  // last round along K (decided on the device from masked_m; the reduce kernel
  // re-derives the same plan and does nothing when there is no split).
  int masked_slots = 0;
  p.device_split = 0;
  if (mode == MODE_MASKED) {
    masked_slots = plan_slots(plan.kernel_id, cus);
    plan.num_workgroups = masked_slots;
    p.device_split = p.k / 128 >= 4 + kTailMinGain ? 1 : 2;
  }
  if (p.device_split == 1) {
    // at most one partial tile per workgroup slot
    const size_t ws_bytes = (size_t)masked_slots * plan.block_m * plan.block_n * 4;
    hipError_t werr = hipSuccess;
    p.ws = split_workspace(di.device, hs, ws_bytes, &werr);
    if (!p.ws) return DG_ERR_HIP;
  }
  if (plan.splits > 1) {
    // one fp32 block_m x block_n partial per slice of every split tile (at most
    // one per workgroup slot, so a few tens of MB at most)
    const size_t ws_bytes = (size_t)(plan.num_tiles - plan.full_tiles) * plan.splits * plan.block_m * plan.block_n * 4;
    hipError_t werr = hipSuccess;
    p.ws = split_workspace(di.device, hs, ws_bytes, &werr);
    if (!p.ws) return DG_ERR_HIP;
  }
  // raster band: the 32 tiles an XCD runs at once share the fewest A and B rows
  // as a 4 x 8 block of 256 x 128 tiles (1024 + 1024 rows) or an 8 x 4 block of
  // 128 x 256 ones; long K loops gain most from the L2 reuse
  p.group_m = (plan.block_m == 256 && plan.block_n == 128 && p.k >= 4096) ? 4 : 8;
  if (const char* gm = std::getenv("DG_GROUP_M")) p.group_m = std::max(1, std::atoi(gm));   // raster band (tuning)
  // DG_KROT=<s>: K-block rotation step between neighbouring tiles (tuning)
  p.k_rot = 0;
  if (const char* kr = std::getenv("DG_KROT")) p.k_rot = std::max(0, std::atoi(kr));
  if (log_enabled())
    std::fprintf(stderr, "[dg] %s m=%d n=%d k=%d groups=%d -> tile %dx%d (kernel %d), %d tiles (%d whole, the rest "
                 "x %d K slices), %d workgroups\n", name, p.m, p.n, p.k, p.num_groups, plan.block_m, plan.block_n,
                 plan.kernel_id, plan.num_tiles, plan.full_tiles, plan.splits, plan.num_workgroups);
  hipError_t e = launch_fp8_gemm(p, plan, mode | flags, hs);
  if (e == hipSuccess && plan.splits > 1) e = launch_splitk_reduce(p, plan, cus, hs);
  if (e == hipSuccess && p.device_split == 1) e = launch_masked_splitk_reduce(p, plan, masked_slots, hs);
  return e == hipSuccess ? DG_OK : DG_ERR_HIP;
}

}  // namespace dg

using namespace dg;

// The three forms; ue8m0 selects packed UE8M0 scale words instead of fp32 scales.
static int dense_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, const uint16_t* c,
                       uint16_t* d, int m, int n, int k, void* stream, int flags) {
  try {
    if (!a || !sfa || !b || !sfb || !d) return DG_ERR_INVALID_ARG;
    if (m <= 0 || n <= 0 || k <= 0) return DG_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sfa, 4) || !aligned(sfb, 4) ||
        (c && !aligned(c, 16)))
      return DG_ERR_INVALID_ARG;
    if (k % 128 != 0 || n % 16 != 0 || !operands_fit(m, n, k)) return DG_ERR_UNSUPPORTED;
    if ((flags & MODE_AT) && m % 16 != 0) return DG_ERR_UNSUPPORTED;   // A's K rows: whole 16-byte chunks
    Fp8GemmParams p{};
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.c = c; p.d = d;
    p.m = m; p.n = n; p.k = k; p.num_groups = 1;
    const char* name = (flags & MODE_AT) ? ((flags & MODE_NN) ? "fp8_gemm_tn" : "fp8_gemm_tt")
                       : (flags & MODE_NN) ? "fp8_gemm_nn"
                       : ((flags & MODE_UE8M0) ? "fp8_gemm_nt_ue8m0" : "fp8_gemm_nt");
    return run_fp8_gemm(p, MODE_DENSE, 0, stream, name, flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

static int contiguous_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                            const int32_t* m_indices, uint16_t* d, int m, int n, int k, int num_groups, void* stream,
                            int flags) {
  try {
    if (!a || !sfa || !b || !sfb || !m_indices || !d) return DG_ERR_INVALID_ARG;
    if (m <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sfa, 4) || !aligned(sfb, 4) ||
        !aligned(m_indices, 4))
      return DG_ERR_INVALID_ARG;
    if (k % 128 != 0 || n % 16 != 0 || !operands_fit(m, n, k)) return DG_ERR_UNSUPPORTED;
    Fp8GemmParams p{};
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.m_indices = m_indices;
    p.m = m; p.n = n; p.k = k; p.num_groups = num_groups;
    const char* name = (flags & MODE_NN) ? "m_grouped_fp8_gemm_nn_contiguous"
                                         : ((flags & MODE_UE8M0) ? "m_grouped_fp8_gemm_nt_contiguous_ue8m0"
                                                                 : "m_grouped_fp8_gemm_nt_contiguous");
    return run_fp8_gemm(p, MODE_CONTIG, 0, stream, name, flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

static int masked_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                        const int32_t* masked_m, uint16_t* d, int num_groups, int max_m, int n, int k, int expected_m,
                        void* stream, int flags) {
  try {
    if (!a || !sfa || !b || !sfb || !masked_m || !d) return DG_ERR_INVALID_ARG;
    if (num_groups <= 0 || max_m <= 0 || n <= 0 || k <= 0) return DG_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sfa, 4) || !aligned(sfb, 4) ||
        !aligned(masked_m, 4))
      return DG_ERR_INVALID_ARG;
    if (k % 128 != 0 || n % 16 != 0 || !operands_fit(max_m, n, k)) return DG_ERR_UNSUPPORTED;
    // the whole tile grid must be addressable with 32-bit tile ids
    long long tiles = (long long)num_groups * ((max_m + 15) / 16) * ((n + 15) / 16);
    if (tiles > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;
    Fp8GemmParams p{};
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.masked_m = masked_m;
    p.m = max_m; p.n = n; p.k = k; p.num_groups = num_groups;
    return run_fp8_gemm(p, MODE_MASKED, expected_m, stream,
                        (flags & MODE_UE8M0) ? "m_grouped_fp8_gemm_nt_masked_ue8m0" : "m_grouped_fp8_gemm_nt_masked",
                        flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

extern "C" {

int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, stream, 0);
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, stream, 0);
}

int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                    const float* sfb, const int32_t* masked_m, uint16_t* d,
                                    int num_groups, int max_m, int n, int k, int expected_m,
                                    void* stream) {
  return masked_entry(a, sfa, b, sfb, masked_m, d, num_groups, max_m, n, k, expected_m, stream, 0);
}

int dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, stream, MODE_NN);
}

int dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, stream, MODE_AT | MODE_NN);
}

int dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, stream, MODE_AT);
}

int dg_m_grouped_fp8_gemm_nn_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, stream, MODE_NN);
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b, const int32_t* sfb,
                         const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, stream, MODE_UE8M0);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                              const int32_t* sfb, const int32_t* m_indices, uint16_t* d,
                                              int m, int n, int k, int num_groups, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, stream, MODE_UE8M0);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                          const int32_t* sfb, const int32_t* masked_m, uint16_t* d,
                                          int num_groups, int max_m, int n, int k, int expected_m,
                                          void* stream) {
  return masked_entry(a, sfa, b, sfb, masked_m, d, num_groups, max_m, n, k, expected_m, stream, MODE_UE8M0);
}

int dg_k_grouped_fp8_gemm_tn_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                        const int32_t* ks, uint16_t* d, int m, int n, int k, int num_groups,
                                        void* stream) {
  try {
    if (!a || !sfa || !b || !sfb || !ks || !d) return DG_ERR_INVALID_ARG;
    if (m <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sfa, 4) || !aligned(sfb, 4) ||
        !aligned(ks, 4))
      return DG_ERR_INVALID_ARG;
    if (k % 128 != 0 || n % 16 != 0 || m % 16 != 0 || !operands_fit(m, n, k)) return DG_ERR_UNSUPPORTED;
    if (num_groups > 65535) return DG_ERR_UNSUPPORTED;
    const long long tiles = (long long)num_groups * ((m + 15) / 16) * ((n + 15) / 16);
    if (tiles > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    Fp8GemmParams p{};
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.ks = ks;
    p.m = m; p.n = n; p.k = k; p.num_groups = num_groups;
    const hipError_t e = launch_kgroup_zero(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return DG_ERR_HIP;
    return run_fp8_gemm(p, MODE_KGROUP, 0, stream, "k_grouped_fp8_gemm_tn_contiguous", MODE_AT | MODE_NN);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int dg_set_num_cus(int n) {
  if (n < 0) return DG_ERR_INVALID_ARG;
  if (n > 0) {
    DeviceInfo di = current_device_info();
    if (di.ok && n > di.num_cus) return DG_ERR_INVALID_ARG;
  }
  g_cu_cap.store(n);
  return DG_OK;
}

int dg_get_num_cus(void) {
  DeviceInfo di = current_device_info();
  if (di.num_cus <= 0) return 0;
  return effective_cus(di);
}

int dg_num_tiles(int m, int n, int block_m, int block_n) {
  if (m <= 0 || n <= 0 || block_m <= 0 || block_n <= 0) return 0;
  return ((m + block_m - 1) / block_m) * ((n + block_n - 1) / block_n);
}

static int query_plan(int m, int n, int k, int num_groups, int mode, int num_cus, dg_plan* out) {
  if (!out || m <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERR_INVALID_ARG;
  if (k % 128 != 0 || n % 16 != 0) return DG_ERR_UNSUPPORTED;
  if (num_cus <= 0) {
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    num_cus = effective_cus(di);
  }
  GemmPlan p = plan_fp8_gemm(m, n, k, num_groups, mode, num_cus, 0);
  out->block_m = p.block_m;
  out->block_n = p.block_n;
  out->num_tiles = p.num_tiles;
  out->num_workgroups = p.num_workgroups;
  out->kernel_id = p.kernel_id;
  out->splits = p.splits;
  out->full_tiles = p.full_tiles;
  return DG_OK;
}

int dg_query_plan(int m, int n, int k, int num_groups, int num_cus, dg_plan* out) {
  return query_plan(m, n, k, num_groups, num_groups > 1 ? MODE_MASKED : MODE_DENSE, num_cus, out);
}

int dg_query_plan_contiguous(int m, int n, int k, int num_groups, int num_cus, dg_plan* out) {
  return query_plan(m, n, k, num_groups, MODE_CONTIG, num_cus, out);
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported shape";
    case DG_ERR_HIP: return "HIP runtime error";
    case DG_ERR_NO_DEVICE: return "no gfx950 device";
  }
  return "unknown status";
}

}  // extern "C"
