// FP8 x FP4 expert FFN: host entry points (kernels follow in this file).
#include "../../include/dg.h"
#include "dg_internal.hpp"

namespace dg {

struct FfnLayout {
  size_t counts, pair_token, pair_of, q, sq, o, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions (all 256-byte aligned):
//   counts     (3E + 2) int32   per-expert pair counts, starts and cursors
//   pair_token P_max int32      token of each (token, slot) pair, grouped by expert
//   pair_of    T*k int32        pair index of each (token, slot), -1 if not local
//   q          P_max x I bytes  requantised SwiGLU output (e4m3)
//   sq         P_max x I/128    its UE8M0 exponents
//   o          P_max x H fp32   linear2 output per pair
// P_max = T*k bounds the pair count for any routing.
static bool ffn_layout(int T, int k, int E, int H, int I, FfnLayout* L) {
  if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return false;
  size_t P = (size_t)T * k;
  size_t off = 0;
  L->counts = off;     off = align256(off + (size_t)(3 * E + 2) * 4);
  L->pair_token = off; off = align256(off + P * 4);
  L->pair_of = off;    off = align256(off + (size_t)T * k * 4);
  L->q = off;          off = align256(off + P * I);
  L->sq = off;         off = align256(off + P * (I / 128));
  L->o = off;          off = align256(off + P * H * 4);
  L->total = off;
  return true;
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
  (void)expert_offset;
  (void)stream;
  if (!x || !x_sf || !topk_idx || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !y || !workspace)
    return DG_ERR_INVALID_ARG;
  if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return DG_ERR_INVALID_ARG;
  if (H % 512 != 0 || I % 128 != 0) return DG_ERR_UNSUPPORTED;
  FfnLayout L;
  ffn_layout(T, k, E, H, I, &L);
  if (workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return DG_ERR_INVALID_ARG;
  return DG_ERR_UNSUPPORTED;
}

}  // extern "C"
