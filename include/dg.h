/*
 * dg.h -- C ABI of the MI355X (gfx950) fine-grained-scaled FP8 / FP8xFP4 GEMM library.
 *
 * Operations (sources are the DeepGEMM pages):
 *   - dense NT GEMM D = C + A.B^T with e4m3 operands and fp32 block scales
 *     (usage guide "DeepGEMM：统一高性能张量核心 GEMM 计算库编译与使用指南",
 *      section 五、使用方法 / 基础非分组 FP8 GEMM: naming D = C + A @ B, NT layout,
 *      fp32 scale factors on SM90);
 *   - the M-grouped contiguous and masked forms for MoE experts
 *     (same page, 分组 GEMM（MoE）: grouping along M only, N and K shared);
 *   - the FP8xFP4 expert FFN, the single-GPU compute share of the fused MoE layer
 *     (news page "DeepSeek 发布 DeepGEMM 重大更新：Mega MoE 融合算子与 FP4 精度支持",
 *      sections Mega MoE and FP4 精度支持: linear1 -> SwiGLU -> linear2 -> combine,
 *      FP4 weights with UE8M0 scales packed four per int32).
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to dense row-major arrays (last index
 *     contiguous).  Sizes are element counts.  Operand and output pointers must
 *     be 16-byte aligned; scale pointers 4-byte aligned.
 *   - The caller owns every buffer, including outputs and workspaces (the
 *     Mega MoE call of the update news page writes a caller-allocated y).  The
 *     library keeps only host-side state (a device-property cache and the CU
 *     cap) and never allocates or frees device memory.  Scratch memory a call
 *     needs (the FP8 GEMMs' split-K partial tiles, the FFN's routing lists and
 *     intermediates) comes from a caller workspace whose size a query function
 *     returns; its contents on entry are ignored.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     There is no host read of device data and no host synchronisation, so
 *     every call may be captured in a HIP graph.  Calls that share a workspace
 *     must be ordered (the same stream, or synchronised streams).
 *   - e4m3 means OCP e4m3fn (bias 7, max 448, NaN = 0x7F/0xFF).  bf16 values
 *     are passed as their uint16 bit patterns.  Outputs are rounded from fp32
 *     to bf16 with round-to-nearest-even (a NaN result stays a quiet NaN).
 *   - Every function returns a dg_status.  Arguments are validated on the host
 *     before any HIP call; on an error nothing is enqueued and nothing is
 *     written.  No C++ exception crosses this boundary and the library never
 *     aborts, so a caller can fall back to another path.
 *   - Malformed device metadata cannot cause out-of-bounds access: group ids
 *     outside [0, num_groups) are treated as -1 (row skipped) and masked_m
 *     values are clamped to [0, max_m].
 *   - Scale layouts are part of the interface (the explainer page
 *     "算子与编译器：DeepGEMM：FP8 GEMM 与 Mega-MoE", section 难点解释, treats the
 *     scale layout as API semantics): A's scales are stored K-block-major so the
 *     scales of one K block for consecutive rows are contiguous.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, misalignment, small workspace */
  DG_ERR_UNSUPPORTED = 2,   /* shape outside what the kernels support (e.g. K % 128 != 0)   */
  DG_ERR_HIP = 3,           /* a HIP runtime error while launching                            */
  DG_ERR_NO_DEVICE = 4,     /* no usable gfx950 device is current                             */
  DG_ERR_SCRATCH_LIMIT = 5  /* dg_fp8_gemm_nt_noalloc: the plan needs more than its static scratch */
} dg_status;

/*
 * Dense NT GEMM: d[m][n] = bf16( c[m][n] + sum_k A[m][k] * B[n][k] ), where the
 * dequantised operands are A[m][k] = e4m3(a[m][k]) * sfa[k/128][m] and
 * B[n][k] = e4m3(b[n][k]) * sfb[n/128][k/128].  Accumulation is fp32: each 128-wide
 * K block is reduced by the matrix cores into a fresh fp32 partial that is then
 * scaled by sfa*sfb and added to the fp32 accumulator.
 *
 *   a    [m, k]               e4m3 codes
 *   sfa  [k/128, m]           fp32, one scale per row per 128-wide K block
 *   b    [n, k]               e4m3 codes (B is stored N x K: the "T" of NT)
 *   sfb  [ceil(n/128), k/128] fp32, one scale per 128x128 block
 *   c    [m, n]               bf16, or NULL for C = 0 (16-byte aligned)
 *   d    [m, n]               bf16 output (may alias c only if identical)
 *   workspace, workspace_bytes
 *        device scratch of at least dg_fp8_gemm_workspace_bytes(DG_FORM_NT, m, n, k, 1, 0, 0)
 *        bytes, 16-byte aligned; may be NULL when that is 0.  Too small (or NULL when
 *        needed): DG_ERR_INVALID_ARG, nothing enqueued.
 * Requirements: m, n, k > 0; k % 128 == 0; n % 16 == 0; m*k, n*k and 2*m*n
 *   (the bytes of A, B and D) at most 2^31, else DG_ERR_UNSUPPORTED.
 */
int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The dense NT GEMM for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, arguments (without the workspace), kernels and results as
 * dg_fp8_gemm_nt, with the split-K partial tiles in a static device buffer of
 * this library instead of a caller workspace.  The buffer holds 24 MiB per GPU
 * (a file-scope device array: each GPU the library runs on keeps its copy until
 * the process ends); a problem whose plan needs more (dg_fp8_gemm_workspace_bytes
 * with DG_FORM_NT above 24 MiB) is rejected with DG_ERR_SCRATCH_LIMIT before
 * anything is enqueued.  The call allocates nothing: no hipMalloc, no allocating
 * library routine.  All calls on one GPU share the buffer and its contents are
 * left from the last call (nothing in it needs clearing), so calls that may
 * overlap in time on one GPU -- on different streams without ordering -- race.
 */
int dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream);

/*
 * M-grouped GEMM, contiguous layout (prefill / training forward).  Rows of all
 * groups are concatenated along M; group g's rows are padded up to a multiple of
 * dg_get_mk_alignment_for_contiguous_layout() and the padding rows carry group
 * index -1.  For every row r with g = m_indices[r] in [0, num_groups):
 *   d[r][n] = bf16( sum_k A[r][k] * B_g[n][k] )
 * Rows with m_indices[r] == -1 (or out of range) are NOT written.  Each
 * 128-row-aligned block of rows must belong to one group (or be padding); a row
 * whose index differs from its block's first row is not written either.
 *
 *   a         [m, k]                            e4m3
 *   sfa       [k/128, m]                        fp32
 *   b         [num_groups, n, k]                e4m3
 *   sfb       [num_groups, ceil(n/128), k/128]  fp32
 *   m_indices [m]                               int32, device memory
 *   d         [m, n]                            bf16
 *   workspace as dg_fp8_gemm_nt, sized by DG_FORM_CONTIGUOUS_NT
 * Requirements: m, n, k, num_groups > 0; k % 128 == 0; n % 16 == 0; m*k, n*k and
 *   2*m*n at most 2^31 (B: one group), else DG_ERR_UNSUPPORTED.
 */
int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * M-grouped GEMM, masked layout (decode).  Each group has a fixed-capacity
 * buffer of max_m rows, of which the first masked_m[g] are valid:
 *   d[g][r][n] = bf16( sum_k A_g[r][k] * B_g[n][k] )   for r < masked_m[g]
 * Rows r >= masked_m[g] are NOT written.  masked_m lives in device memory and
 * is never read by the host.  expected_m is an optional host-side hint of the
 * typical masked_m (<= 0: unknown) used only to choose tile sizes.
 *
 *   a        [num_groups, max_m, k]            e4m3
 *   sfa      [num_groups, k/128, max_m]        fp32
 *   b        [num_groups, n, k]                e4m3
 *   sfb      [num_groups, ceil(n/128), k/128]  fp32
 *   masked_m [num_groups]                      int32, device memory
 *   d        [num_groups, max_m, n]            bf16
 *   workspace as dg_fp8_gemm_nt, sized by DG_FORM_MASKED_NT with m = max_m
 * Requirements: num_groups, max_m, n, k > 0; k % 128 == 0; n % 16 == 0; per group,
 *   max_m*k, n*k and 2*max_m*n at most 2^31, else DG_ERR_UNSUPPORTED.
 */
int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                    const float* sfb, const int32_t* masked_m, uint16_t* d,
                                    int num_groups, int max_m, int n, int k, int expected_m,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * NN layout (usage guide "DeepGEMM：统一高性能张量核心 GEMM 计算库编译与使用指南",
 * 五、使用方法 / 基础非分组 FP8 GEMM: the newer architecture takes the NT, TN, NN and
 * TT layouts; 分组 GEMM（MoE）: the contiguous grouped form in NN for the training
 * backward pass): B is stored K-major, not transposed, so D = C + A @ B with
 *   b    [k, n]          e4m3, n contiguous (grouped: [num_groups, k, n])
 * and every other argument, scale layout (sfb stays [ceil(n/128)][k/128], indexed
 * by n-block then k-block), requirement and row rule as in dg_fp8_gemm_nt and
 * dg_m_grouped_fp8_gemm_nt_contiguous (workspace sized by DG_FORM_NN and
 * DG_FORM_CONTIGUOUS_NN).  The kernel reads B's tiles with gfx950's transposing
 * LDS loads.
 */
int dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream);
int dg_m_grouped_fp8_gemm_nn_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, const int32_t* m_indices, uint16_t* d,
                                        int m, int n, int k, int num_groups, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * TN and TT layouts (same usage-guide passage): A is stored [k, m], m contiguous,
 * so D[i][j] = C[i][j] + sum_k A[k][i] * B(k, j), with B stored [k, n] (TN) or
 * [n, k] (TT).  sfa stays [k/128][m] (one scale per row of D per 128-wide K
 * block), sfb [ceil(n/128)][k/128].  Both read A's tiles with the transposing
 * LDS loads (in 128-row sub-tiles).  Requirements as dg_fp8_gemm_nt plus
 * m % 16 == 0; workspace sized by DG_FORM_TN and DG_FORM_TT.
 */
int dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream);
int dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The same three GEMMs with packed UE8M0 scale factors instead of fp32 ones
 * (usage guide "DeepGEMM：统一高性能张量核心 GEMM 计算库编译与使用指南", 五、使用方法 /
 * 基础非分组 FP8 GEMM: the older architecture takes fp32 scale factors, the newer
 * one power-of-two scale factors packed four to an int32).  The scale granularity is that of
 * the fp32 forms (A per row per 128-wide K block, B per 128x128 block); a scale is
 * 2^(e - 127) for the exponent byte e.  Byte i (from the least significant) of
 * word j holds K block 4j + i.  The matrix instruction applies both exponents
 * exactly, so D is the fp32 sum of exact products rounded once to bf16 (no
 * separate promotion step).
 *   dg_fp8_gemm_nt_ue8m0:               sfa [m, ceil(k/512)], sfb [ceil(n/128), ceil(k/512)], c optional
 *   dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0:
 *                                       sfa [m, ceil(k/512)], sfb [num_groups, ceil(n/128), ceil(k/512)]
 *   dg_m_grouped_fp8_gemm_nt_masked_ue8m0:
 *                                       sfa [num_groups, max_m, ceil(k/512)], sfb as contiguous
 * All other arguments, requirements, row rules (padding rows, rows past masked_m
 * not written) and errors are those of the fp32-scale form (workspace sized by
 * DG_FORM_NT_UE8M0, DG_FORM_CONTIGUOUS_NT_UE8M0, DG_FORM_MASKED_NT_UE8M0).
 * Exponent byte 255 (NaN scale) gives NaN results.
 */
int dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b, const int32_t* sfb,
                         const uint16_t* c, uint16_t* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, void* stream);
int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                              const int32_t* sfb, const int32_t* m_indices, uint16_t* d,
                                              int m, int n, int k, int num_groups, void* workspace,
                                              size_t workspace_bytes, void* stream);
int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                                          const int32_t* sfb, const int32_t* masked_m, uint16_t* d,
                                          int num_groups, int max_m, int n, int k, int expected_m,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace of the FP8 GEMM entry points above.  Skinny problems (and the
 * partial last round of some large ones) are split along K: each slice of a
 * split tile sums a range of 128-wide K blocks into an fp32 partial tile, and a
 * second kernel adds a tile's partials in slice order (plus C) and rounds to
 * bf16.  The partials live in the caller's workspace.  This returns the bytes
 * the call with these sizes needs (0: the plan does not split, and workspace may
 * be NULL), for the entry point named by `form`:
 *   dense forms:   m, n, k of the call; num_groups and expected_m ignored
 *   contiguous:    m = total rows of the layout, num_groups
 *   masked:        m = max_m, num_groups, expected_m as passed to the call
 * num_cus: the CU count the call will run with (<= 0: the current cap of the
 * current device; > 0: host-only, no HIP call).  The need never exceeds one
 * fp32 block_m x block_n tile per workgroup slot (dg_query_plan).  Returns 0 for
 * invalid sizes, whose calls then fail with their own status.
 */
typedef enum dg_gemm_form {
  DG_FORM_NT = 0,                   /* dg_fp8_gemm_nt */
  DG_FORM_NN = 1,                   /* dg_fp8_gemm_nn */
  DG_FORM_TN = 2,                   /* dg_fp8_gemm_tn */
  DG_FORM_TT = 3,                   /* dg_fp8_gemm_tt */
  DG_FORM_NT_UE8M0 = 4,             /* dg_fp8_gemm_nt_ue8m0 */
  DG_FORM_CONTIGUOUS_NT = 5,        /* dg_m_grouped_fp8_gemm_nt_contiguous */
  DG_FORM_CONTIGUOUS_NN = 6,        /* dg_m_grouped_fp8_gemm_nn_contiguous */
  DG_FORM_CONTIGUOUS_NT_UE8M0 = 7,  /* dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 */
  DG_FORM_MASKED_NT = 8,            /* dg_m_grouped_fp8_gemm_nt_masked */
  DG_FORM_MASKED_NT_UE8M0 = 9       /* dg_m_grouped_fp8_gemm_nt_masked_ue8m0 */
} dg_gemm_form;
size_t dg_fp8_gemm_workspace_bytes(int form, int m, int n, int k, int num_groups, int expected_m,
                                   int num_cus);

/*
 * Weight pre-transform for the FP8 x FP4 entry points (news page "DeepSeek 发布
 * DeepGEMM 重大更新：Mega MoE 融合算子与 FP4 精度支持": section FP4 精度支持, the
 * weight pre-transform tool, and section Mega MoE, whose expert weights are
 * converted once to the layout the fused kernel reads).  Here the E2M1 weight
 * bytes keep their row-major layout and the packed UE8M0 scale words are made
 * K-block-major:
 *   sf_t[g][kb][r] = sf[g][r][kb]     sf [num_groups, n, k/128] -> sf_t [num_groups, k/128, n]
 * so that the scale words of one K block of a weight tile are one contiguous run.
 * dg_fp8_fp4_expert_ffn (w1_sf, w2_sf) and the M-grouped FP8 x FP4 GEMMs (b_sf)
 * take the transformed words; the transform is meant to run once per weight set.
 *   sf, sf_t  device buffers, 4-byte aligned, not overlapping (DG_ERR_INVALID_ARG)
 * Requirements: k % 128 == 0, num_groups <= 65535 (else DG_ERR_UNSUPPORTED).
 * Enqueued on stream; no host synchronisation.
 */
int dg_transform_fp4_weight_sf(const int32_t* sf, int32_t* sf_t, int num_groups, int n, int k,
                               void* stream);

/*
 * Bytes of device workspace dg_fp8_fp4_expert_ffn needs for these sizes
 * (routing lists, the requantised intermediate and per-pair outputs).
 * Returns 0 for invalid sizes.
 */
size_t dg_fp8_fp4_expert_ffn_workspace_bytes(int num_tokens, int num_topk, int num_local_experts,
                                             int hidden, int intermediate);

/*
 * Single-GPU FP8 x FP4 expert FFN over the local experts
 * [expert_offset, expert_offset + num_local_experts):
 *   for each token t and slot j with e = topk_idx[t][j] - expert_offset in range:
 *     h = e4m3(x[t]) * 2^(x_sf exponent per 128)
 *     u = h . W1_e^T                       (W1_e = E2M1 * UE8M0 per 1x32, [2I, H])
 *     s = silu(u[0:I]) * u[I:2I]           (gate rows first, then up rows)
 *     q, sq = e4m3 requantisation of s per 1x128 with scale 2^ceil(log2(amax/448))
 *     o = (q * sq) . W2_e^T                (W2_e = E2M1 * UE8M0 per 1x32, [H, I])
 *     y[t] += topk_w[t][j] * o
 *   y = bf16(y), with y[t] = 0 for tokens without a local hit.  Every row of y is written.
 *
 *   x         [T, H]            e4m3 activations
 *   x_sf      [T, H/512]        int32, four UE8M0 scales per word (1x128 blocks);
 *                               byte i (from the least significant) of word j is block 4j+i
 *   topk_idx  [T, num_topk]     int32 global expert ids (any value; out-of-range ids ignored)
 *   topk_w    [T, num_topk]     fp32
 *   w1        [E, 2I, H/2]      E2M1 pairs; element 2i in the low nibble of byte i
 *   w1_sf     [E, H/128, 2I]    int32, four UE8M0 scales per word (1x32 blocks; byte i of
 *                               word [e][kb][r] is K 128kb+32i..+32 of row r), K-block-major
 *                               as dg_transform_fp4_weight_sf writes it
 *   w2        [E, H, I/2]       E2M1 pairs
 *   w2_sf     [E, I/128, H]     int32, K-block-major likewise
 *   y         [T, H]            bf16 output
 *   workspace device buffer of at least dg_fp8_fp4_expert_ffn_workspace_bytes(...) bytes,
 *             256-byte aligned; its contents on entry are ignored
 * Requirements: T, num_topk, E > 0; E <= 256; H % 512 == 0; I % 128 == 0; T*H,
 *   T*num_topk*I and I*H at most 2^31 (else DG_ERR_UNSUPPORTED).
 */
int dg_fp8_fp4_expert_ffn(const uint8_t* x, const int32_t* x_sf, const int32_t* topk_idx,
                          const float* topk_w, const uint8_t* w1, const int32_t* w1_sf,
                          const uint8_t* w2, const int32_t* w2_sf, uint16_t* y, int num_tokens,
                          int num_topk, int num_local_experts, int expert_offset, int hidden,
                          int intermediate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * M-grouped FP8 x FP4 GEMM, the FFN's GEMM form exported on its own (news page
 * "DeepSeek 发布 DeepGEMM 重大更新：Mega MoE 融合算子与 FP4 精度支持", section FP4
 * 精度支持: FP8 activations times FP4 weights; usage guide, 分组 GEMM（MoE）, for the
 * contiguous and masked layouts).  The block scales are applied by the matrix
 * cores; there is no C input and no split along K.
 *   D[r] = bf16( sum_k A[r,k] 2^(ea(r, k/128)) * B_g[n,k] 2^(eb(g, n, k/32)) )
 * with g the group of row r.
 *   a      e4m3 rows, 16-byte aligned
 *   a_sf   int32, ceil(k/512) words per row, four UE8M0 exponents per word (1x128
 *          blocks; byte i of word j is block 4j+i), 4-byte aligned
 *   b      [num_groups, n, k/2] E2M1 pairs (element 2i in the low nibble of byte i), 16-byte aligned
 *   b_sf   [num_groups, k/128, n] int32, four UE8M0 exponents per word (1x32 blocks),
 *          K-block-major as dg_transform_fp4_weight_sf writes it
 *   d      bf16 rows of n, 16-byte aligned
 * Requirements: n % 16 == 0; k % 128 == 0; (rows of A) * k, n * k / 2 and
 *   (rows of A) * 4 * ceil(k/512) at most 2^31 (else DG_ERR_UNSUPPORTED).
 *
 * Contiguous: a [m, k], a_sf [m, ceil(k/512)], m_indices [m] (group of each row,
 * -1 for padding; groups padded to 128 rows, so each 128-row block holds one
 * group), d [m, n]; only rows of a group are written.
 */
int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const uint8_t* a, const int32_t* a_sf, const uint8_t* b,
                                            const int32_t* b_sf, const int32_t* m_indices, uint16_t* d,
                                            int m, int n, int k, int num_groups, void* stream);

/*
 * Masked: a [num_groups, max_m, k], a_sf [num_groups, max_m, ceil(k/512)],
 * masked_m [num_groups] (valid rows per group, clamped to [0, max_m]),
 * d [num_groups, max_m, n]; rows r < masked_m[g] of group g are written, no other.
 * num_groups <= 256.  expected_m is accepted for symmetry with the FP8 form and
 * unused: the kernel walks only the tiles that hold valid rows.
 */
int dg_m_grouped_fp8_fp4_gemm_nt_masked(const uint8_t* a, const int32_t* a_sf, const uint8_t* b,
                                        const int32_t* b_sf, const int32_t* masked_m, uint16_t* d,
                                        int num_groups, int max_m, int n, int k, int expected_m,
                                        void* stream);

/*
 * K-grouped GEMM in the TN layout, contiguous (usage guide
 * "DeepGEMM：统一高性能张量核心 GEMM 计算库编译与使用指南", 分组 GEMM（MoE）: the
 * K-axis grouped form of the training backward pass, e.g. each expert's weight
 * gradient): the K rows (tokens) are split into consecutive groups and each group
 * has its own output:
 *   d[g][i][j] = bf16( sum over k in group g of A[k][i] * B[k][j] )
 *   a    [k, m]            e4m3, m contiguous; sfa [k/128][m] fp32
 *   b    [k, n]            e4m3, n contiguous; sfb [ceil(n/128)][k/128] fp32
 *   ks   [num_groups]      int32 on the device: K rows of each group, multiples of
 *                          128 (the contiguous layout pads each group to 128 rows;
 *                          padding rows should hold zeros), in order; read only on
 *                          the device.  Counts are rounded down to multiples of 128
 *                          and cut at k.
 *   d    [num_groups, m, n] bf16, every element written (0 for a group without rows)
 * No C input.  Requirements: m % 16 == 0, n % 16 == 0, k % 128 == 0, m*k, n*k and
 * 2*m*n at most 2^31, num_groups <= 65535 (else DG_ERR_UNSUPPORTED).
 */
int dg_k_grouped_fp8_gemm_tn_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                        const int32_t* ks, uint16_t* d, int m, int n, int k, int num_groups,
                                        void* stream);

/* Row alignment of each group in the contiguous layout (usage guide, 工具函数). Returns 128. */
int dg_get_mk_alignment_for_contiguous_layout(void);

/*
 * Cap the number of compute units the persistent kernels use (usage guide, 工具函数:
 * the SM-count setter/getter).  1 <= n <= CUs of the current device; n = 0 restores
 * the default (all CUs).  Returns DG_OK or DG_ERR_INVALID_ARG.  dg_get_num_cus
 * returns the cap in force (the device's CU count when none is set, or 0 when no
 * device is visible).
 */
int dg_set_num_cus(int n);
int dg_get_num_cus(void);

/*
 * The tile plan the heuristic picks for an M x N x K problem split over
 * num_groups groups (1 for dense), on num_cus compute units (<= 0: current cap).
 * Host-only: no HIP call is made when num_cus > 0.  Fills block_m, block_n,
 * the number of output tiles, the K slices per split tile, the tiles computed
 * whole and the number of workgroups launched.  Dense problems may be split
 * along K: when the tiles cannot fill the chip (skinny M) every tile is split,
 * and when the last round of tiles would leave at least half of the workgroup
 * slots idle over a long K loop, only that round's tiles are (partials in the
 * caller's workspace, see dg_fp8_gemm_workspace_bytes).
 * The masked form's tile list depends on masked_m, which only the device
 * reads: its kernel walks just the tiles that hold valid rows, spread evenly
 * over the workgroups, and for K >= 3584 applies the same split rule to their
 * count on the device (a second kernel then sums the split tiles).  For it this
 * function reports the tile shape and splits = 1.
 * Exposed so callers can log the choice (DG_LOG=1 prints it on every call).
 */
typedef struct dg_plan {
  int block_m;
  int block_n;
  int num_tiles;        /* output tiles */
  int num_workgroups;
  int kernel_id;        /* 0-3: the 256x128, 128x256, 128x128, 64x128 tiles; 4: the 256x256 tile
                           and 6: the 256x224 tile (dense NT with fp32 scales only); 5: the 128x512
                           tile (dense and contiguous NT with fp32 scales); >= 100: the skinny-M
                           kernel */
  int splits;           /* K slices per split tile (dense only; 1: no split) */
  int full_tiles;       /* tiles computed whole; the other num_tiles - full_tiles are split */
} dg_plan;
int dg_query_plan(int m, int n, int k, int num_groups, int num_cus, dg_plan* out);

/* The same for the M-grouped contiguous form (dg_m_grouped_fp8_gemm_nt_contiguous):
 * m is the total row count of the layout, num_groups the groups.  Its tiles may
 * be split along K by the same rule (padding blocks are skipped).  Host-only
 * when num_cus > 0. */
int dg_query_plan_contiguous(int m, int n, int k, int num_groups, int num_cus, dg_plan* out);

/* The plan of the call of a given form (a dg_gemm_form value, as for
 * dg_fp8_gemm_workspace_bytes), with that form's arguments: the forms differ
 * in the kernels they may take (the skinny-M kernel of the dense NT form with
 * fp32 scales, for one), so this is the query to use for any form but plain
 * dense NT.  An unknown form returns DG_ERR_INVALID_ARG.  Host-only when
 * num_cus > 0. */
int dg_query_plan_form(int form, int m, int n, int k, int num_groups, int expected_m, int num_cus, dg_plan* out);

/* Number of output tiles for a tile shape: ceil(m/block_m) * ceil(n/block_n). Host-only. */
int dg_num_tiles(int m, int n, int block_m, int block_n);

/* Static description of a status code. */
const char* dg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
