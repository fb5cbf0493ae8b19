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

// Host-side decisions of one GEMM call: the tile plan (with the tuning
// overrides), the raster, and the bytes of caller workspace the plan needs.
struct CallPlan {
  GemmPlan plan;
  int masked_slots;   // masked form: workgroups of the device-planned walk
  size_t ws_bytes;    // split-K partial tiles (0: the plan does not split)
};

static CallPlan plan_call(Fp8GemmParams& p, int mode, int expected_m, int flags, int cus) {
  CallPlan cp{};
  const int bm_multiple = (flags & MODE_AT) ? 128 : 0;   // A stored [K][M]: 128-row sub-tiles
  // K-grouped: plan for a group's mean K
  const int k_plan = mode == MODE_KGROUP ? std::max(128, p.k / p.num_groups / 128 * 128) : p.k;
  GemmPlan plan = plan_fp8_gemm(p.m, p.n, k_plan, p.num_groups, mode, cus, expected_m, bm_multiple,
                                flags == 0 && wide_fits(p.m, p.n, p.k));
  if (plan.kernel_id < 0) {
    cp.plan = plan;
    return cp;
  }
  // DG_FORCE_KERNEL=<id>: override the heuristic's tile choice (for tuning)
  const char* fk = std::getenv("DG_FORCE_KERNEL");
  if (fk) {
    int id = std::atoi(fk);
    if (id >= 0 && id < num_tile_configs() &&
        !(is_wide_tile(id) && (!wide_serves(id, mode) || flags != 0 || !wide_fits(p.m, p.n, p.k))) &&
        !(mode == MODE_CONTIG && (128 % tile_config(id).block_m) != 0) &&
        !(bm_multiple > 0 && tile_config(id).block_m % bm_multiple != 0))
      plan = plan_with_kernel(p.m, p.n, p.k, p.num_groups, mode, cus, id);
  }
  // Skinny M (dense NT, fp32 scales, m <= 128): the streaming kernel with all rows
  // of A in one tile.  DG_FORCE_SKINNY=<id>[,<splits>] pins its configuration
  // (for tuning); DG_FORCE_KERNEL keeps the square-tile kernel.
  if (mode == MODE_DENSE && flags == 0 && !fk) {
    int force_id = -1, force_splits = -1;
    if (const char* fs = std::getenv("DG_FORCE_SKINNY")) {
      force_id = std::atoi(fs);
      if (const char* comma = std::strchr(fs, ',')) force_splits = std::atoi(comma + 1);
    }
    // Up to 128 rows the skinny kernel always applies.  Up to 256 rows it is taken
    // only where the square-tile plan leaves more than a tenth of the workgroup
    // slots idle in its last round and the skinny plan's column width (any
    // multiple of 16, 112 among them) fills at least 95 % of them: the release
    // article's case of non-power-of-two BLOCK_N (优化技术 / 非对齐块大小).  (C is
    // not part of the choice: the workspace query, which has no C, plans the same.)
    if (p.m <= 256 || force_id >= 0) {
      const GemmPlan sk = plan_skinny(p.m, p.n, p.k, cus, false, force_id, force_splits);
      auto fill = [&](const GemmPlan& g) {
        const long long units = (long long)g.full_tiles + (long long)(g.num_tiles - g.full_tiles) * g.splits;
        const long long rounds = (units + cus - 1) / cus;
        return rounds > 0 ? (double)units / ((double)rounds * cus) : 0.0;
      };
      if (sk.skinny_id >= 0 &&
          (p.m <= 128 || force_id >= 0 || (fill(plan) < 0.9 && fill(sk) >= 0.95)))
        plan = sk;
    }
  }
  p.tiles_m = plan.tiles_m;
  p.tiles_n = plan.tiles_n;
  p.splits = plan.splits;
  p.kb_per_split = plan.kb_per_split;
  p.full_tiles = plan.full_tiles;
  p.total_tiles = (int)std::min<long long>(
      (long long)plan.full_tiles + (long long)(plan.num_tiles - plan.full_tiles) * plan.splits, 0x7fffffff);
  // Masked form: the kernel walks only the tiles holding valid rows, spread
  // evenly over one full set of workgroup slots, and over long K splits a small
  // last round along K (decided on the device from masked_m; the reduce kernel
  // re-derives the same plan and does nothing when there is no split).
  p.device_split = 0;
  const size_t tile_bytes = (size_t)plan.block_m * plan.block_n * 4;
  if (mode == MODE_MASKED) {
    cp.masked_slots = plan_slots(plan.kernel_id, cus);
    plan.num_workgroups = cp.masked_slots;
    p.device_split = p.k / 128 >= 4 + kTailMinGain ? 1 : 2;
    // the device's split rule yields at most one partial tile per workgroup slot
    if (p.device_split == 1) cp.ws_bytes = (size_t)cp.masked_slots * tile_bytes;
  } else if (plan.splits > 1) {
    // one partial per slice of every split tile (at most one per workgroup slot)
    cp.ws_bytes = (size_t)(plan.num_tiles - plan.full_tiles) * plan.splits * tile_bytes;
  }
  // raster band: the 32 tiles an XCD runs at once share the fewest A and B rows
  // as a 4 x 8 block of 256 x 128 tiles (1024 + 1024 rows) or an 8 x 4 block of
  // 128 x 256 ones; long K loops gain most from the L2 reuse
  p.group_m = (plan.block_m == 256 && plan.block_n == 128 && p.k >= 4096) ? 4 : 8;
  if (const char* gm = std::getenv("DG_GROUP_M")) p.group_m = std::max(1, std::atoi(gm));   // raster band (tuning)
  if (plan.skinny_id >= 0) p.group_m = std::max(1, plan.tiles_m);   // skinny tiles are column-major
  // DG_KROT=<s>: K-block rotation step between neighbouring tiles (tuning)
  p.k_rot = 0;
  if (const char* kr = std::getenv("DG_KROT")) p.k_rot = std::max(0, std::atoi(kr));
  cp.plan = plan;
  return cp;
}

// flags: MODE_UE8M0, MODE_NN and / or MODE_AT, or-ed into the form's mode at launch
static int run_fp8_gemm(Fp8GemmParams& p, int mode, int expected_m, void* workspace, size_t workspace_bytes,
                        void* stream, const char* name, int flags = 0) {
  DeviceInfo di = current_device_info();
  if (!di.ok) return DG_ERR_NO_DEVICE;
  const int cus = effective_cus(di);
  CallPlan cp = plan_call(p, mode, expected_m, flags, cus);
  const GemmPlan& plan = cp.plan;
  if (plan.kernel_id < 0) return DG_ERR_UNSUPPORTED;
  if (cp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < cp.ws_bytes || !aligned(workspace, 16)) return DG_ERR_INVALID_ARG;
    p.ws = static_cast<float*>(workspace);
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[dg] %s m=%d n=%d k=%d groups=%d -> tile %dx%d (kernel %d), %d tiles (%d whole, the rest "
                 "x %d K slices), %d workgroups, workspace %zu bytes\n", name, p.m, p.n, p.k, p.num_groups,
                 plan.block_m, plan.block_n, plan.kernel_id, plan.num_tiles, plan.full_tiles, plan.splits,
                 plan.num_workgroups, cp.ws_bytes);
  hipError_t e;
  if (plan.skinny_id >= 0) {
    SkinnyParams sp{};
    sp.a = p.a; sp.sfa = static_cast<const float*>(p.sfa); sp.b = p.b; sp.sfb = static_cast<const float*>(p.sfb);
    sp.c = p.c; sp.d = p.d; sp.ws = p.ws;
    sp.m = p.m; sp.n = p.n; sp.k = p.k;
    sp.tiles_m = plan.tiles_m; sp.tiles_n = plan.tiles_n;
    sp.splits = plan.splits; sp.kb_per_split = plan.kb_per_split;
    e = launch_skinny_gemm(sp, plan.skinny_id, plan.num_workgroups, hs);
  } else {
    e = launch_fp8_gemm(p, plan, mode | flags, hs);
  }
  if (e == hipSuccess && plan.splits > 1 && mode != MODE_MASKED) e = launch_splitk_reduce(p, plan, cus, hs);
  if (e == hipSuccess && p.device_split == 1) e = launch_masked_splitk_reduce(p, plan, cp.masked_slots, hs);
  return e == hipSuccess ? DG_OK : DG_ERR_HIP;
}

// The three forms; ue8m0 selects packed UE8M0 scale words instead of fp32 scales.
// Kernel mode and layout/scale flags of a dg_gemm_form (false: not a form with a plan).
bool form_mode(int form, int* mode, int* flags) {
  switch (form) {
    case DG_FORM_NT: *mode = MODE_DENSE; *flags = 0; return true;
    case DG_FORM_NN: *mode = MODE_DENSE; *flags = MODE_NN; return true;
    case DG_FORM_TN: *mode = MODE_DENSE; *flags = MODE_AT | MODE_NN; return true;
    case DG_FORM_TT: *mode = MODE_DENSE; *flags = MODE_AT; return true;
    case DG_FORM_NT_UE8M0: *mode = MODE_DENSE; *flags = MODE_UE8M0; return true;
    case DG_FORM_CONTIGUOUS_NT: *mode = MODE_CONTIG; *flags = 0; return true;
    case DG_FORM_CONTIGUOUS_NN: *mode = MODE_CONTIG; *flags = MODE_NN; return true;
    case DG_FORM_CONTIGUOUS_NT_UE8M0: *mode = MODE_CONTIG; *flags = MODE_UE8M0; return true;
    case DG_FORM_MASKED_NT: *mode = MODE_MASKED; *flags = 0; return true;
    case DG_FORM_MASKED_NT_UE8M0: *mode = MODE_MASKED; *flags = MODE_UE8M0; return true;
  }
  return false;
}

int dense_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, const uint16_t* c,
                       uint16_t* d, int m, int n, int k, void* ws, size_t ws_bytes, void* stream, int flags) {
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
    return run_fp8_gemm(p, MODE_DENSE, 0, ws, ws_bytes, stream, name, flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

}  // namespace dg

using namespace dg;

static int contiguous_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                            const int32_t* m_indices, uint16_t* d, int m, int n, int k, int num_groups, void* ws,
                            size_t ws_bytes, void* stream, int flags) {
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
    return run_fp8_gemm(p, MODE_CONTIG, 0, ws, ws_bytes, stream, name, flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

static int masked_entry(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                        const int32_t* masked_m, uint16_t* d, int num_groups, int max_m, int n, int k, int expected_m,
                        void* ws, size_t ws_bytes, void* stream, int flags) {
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
    return run_fp8_gemm(p, MODE_MASKED, expected_m, ws, ws_bytes, stream,
                        (flags & MODE_UE8M0) ? "m_grouped_fp8_gemm_nt_masked_ue8m0" : "m_grouped_fp8_gemm_nt_masked",
                        flags);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

extern "C" {

int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, workspace, workspace_bytes, stream, 0);
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, workspace, workspace_bytes, stream, 0);
}

int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                    const float* sfb, const int32_t* masked_m, uint16_t* d,
                                    int num_groups, int max_m, int n, int k, int expected_m,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return masked_entry(a, sfa, b, sfb, masked_m, d, num_groups, max_m, n, k, expected_m, workspace, workspace_bytes,
                      stream, 0);
}

int dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, workspace, workspace_bytes, stream, MODE_NN);
}

int dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, workspace, workspace_bytes, stream, MODE_AT | MODE_NN);
}

int dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, workspace, workspace_bytes, stream, MODE_AT);
}

int dg_m_grouped_fp8_gemm_nn_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, workspace, workspace_bytes, stream,
                          MODE_NN);
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b, const int32_t* sfb,
                         const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return dense_entry(a, sfa, b, sfb, c, d, m, n, k, workspace, workspace_bytes, stream, MODE_UE8M0);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                              const int32_t* sfb, const int32_t* m_indices, uint16_t* d,
                                              int m, int n, int k, int num_groups, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return contiguous_entry(a, sfa, b, sfb, m_indices, d, m, n, k, num_groups, workspace, workspace_bytes, stream,
                          MODE_UE8M0);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                          const int32_t* sfb, const int32_t* masked_m, uint16_t* d,
                                          int num_groups, int max_m, int n, int k, int expected_m,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  return masked_entry(a, sfa, b, sfb, masked_m, d, num_groups, max_m, n, k, expected_m, workspace, workspace_bytes,
                      stream, MODE_UE8M0);
}

size_t dg_fp8_gemm_workspace_bytes(int form, int m, int n, int k, int num_groups, int expected_m, int num_cus) {
  try {
    if (m <= 0 || n <= 0 || k <= 0 || num_groups <= 0 || k % 128 != 0 || n % 16 != 0) return 0;
    int mode, flags;
    if (!dg::form_mode(form, &mode, &flags)) return 0;
    if (mode == MODE_DENSE) num_groups = 1;
    if (num_cus <= 0) {
      DeviceInfo di = current_device_info();
      if (!di.ok) return 0;
      num_cus = effective_cus(di);
    }
    Fp8GemmParams p{};
    p.m = m; p.n = n; p.k = k; p.num_groups = num_groups;
    const CallPlan cp = plan_call(p, mode, expected_m, flags, num_cus);
    return cp.plan.kernel_id < 0 ? 0 : cp.ws_bytes;
  } catch (...) {
    return 0;
  }
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
    return run_fp8_gemm(p, MODE_KGROUP, 0, nullptr, 0, stream, "k_grouped_fp8_gemm_tn_contiguous", MODE_AT | MODE_NN);
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

static int query_plan(int m, int n, int k, int num_groups, int mode, int num_cus, dg_plan* out, int flags = 0,
                      int expected_m = 0) {
  if (!out || m <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERR_INVALID_ARG;
  if (k % 128 != 0 || n % 16 != 0) return DG_ERR_UNSUPPORTED;
  if (num_cus <= 0) {
    DeviceInfo di = current_device_info();
    if (!di.ok) return DG_ERR_NO_DEVICE;
    num_cus = effective_cus(di);
  }
  Fp8GemmParams p{};
  p.m = m; p.n = n; p.k = k; p.num_groups = num_groups;
  const GemmPlan pl = plan_call(p, mode, expected_m, flags, num_cus).plan;
  if (pl.kernel_id < 0) return DG_ERR_UNSUPPORTED;
  out->block_m = pl.block_m;
  out->block_n = pl.block_n;
  out->num_tiles = pl.num_tiles;
  out->num_workgroups = pl.num_workgroups;
  out->kernel_id = pl.kernel_id;
  out->splits = pl.splits;
  out->full_tiles = pl.full_tiles;
  return DG_OK;
}

int dg_query_plan(int m, int n, int k, int num_groups, int num_cus, dg_plan* out) {
  return query_plan(m, n, k, num_groups, num_groups > 1 ? MODE_MASKED : MODE_DENSE, num_cus, out);
}

int dg_query_plan_contiguous(int m, int n, int k, int num_groups, int num_cus, dg_plan* out) {
  return query_plan(m, n, k, num_groups, MODE_CONTIG, num_cus, out);
}

int dg_query_plan_form(int form, int m, int n, int k, int num_groups, int expected_m, int num_cus, dg_plan* out) {
  try {
    int mode, flags;
    if (!dg::form_mode(form, &mode, &flags)) return DG_ERR_INVALID_ARG;
    return query_plan(m, n, k, mode == MODE_DENSE ? 1 : num_groups, mode, num_cus, out, flags, expected_m);
  } catch (...) {
    return DG_ERR_HIP;
  }
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported shape";
    case DG_ERR_HIP: return "HIP runtime error";
    case DG_ERR_NO_DEVICE: return "no gfx950 device";
    case DG_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
