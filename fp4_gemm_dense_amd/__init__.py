"""Python binding of the gfx950 fine-grained-scaled FP8 / FP8xFP4 GEMM library.

Argument marshalling only: every function here checks dtypes, shapes and
devices of torch tensors, then calls the C ABI of ``libdg.so`` (declared in
``include/dg.h``) with raw device pointers and torch's current HIP stream.
All arithmetic runs in the library's HIP kernels; there is no fallback path.
If the library is not built, ``load_library()`` raises.

The ``dg_*`` functions mirror the C entry points one to one (outputs are
caller-allocated).  ``fp8_gemm_nt`` etc. are convenience wrappers that allocate
the output, as in the pages' Python API (usage guide, 五、使用方法).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")
_lib = None

DG_OK = 0
STATUS_NAMES = {0: "DG_OK", 1: "DG_ERR_INVALID_ARG", 2: "DG_ERR_UNSUPPORTED", 3: "DG_ERR_HIP",
                4: "DG_ERR_NO_DEVICE", 5: "DG_ERR_SCRATCH_LIMIT"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "dg_fp8_gemm_nt": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_gemm_nt_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_gemm_nt_masked": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_fp8_gemm_nn": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "dg_fp8_gemm_tn": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "dg_k_grouped_fp8_gemm_tn_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "dg_fp8_gemm_tt": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_gemm_nn_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_fp8_gemm_nt_ue8m0": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_m_grouped_fp8_fp4_gemm_nt_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "dg_m_grouped_fp8_fp4_gemm_nt_masked": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "dg_transform_fp4_weight_sf": (_I, [_P, _P, _I, _I, _I, _P]),
    "dg_fp8_fp4_expert_ffn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "dg_fp8_fp4_expert_ffn": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "dg_fp8_gemm_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "dg_fp8_gemm_nt_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "dg_get_mk_alignment_for_contiguous_layout": (_I, []),
    "dg_set_num_cus": (_I, [_I]),
    "dg_get_num_cus": (_I, []),
    "dg_query_plan": (_I, [_I, _I, _I, _I, _I, _P]),
    "dg_query_plan_contiguous": (_I, [_I, _I, _I, _I, _I, _P]),
    "dg_query_plan_form": (_I, [_I, _I, _I, _I, _I, _I, _I, _P]),
    "dg_num_tiles": (_I, [_I, _I, _I, _I]),
    "dg_status_string": (ctypes.c_char_p, [_I]),
}


class DgPlan(ctypes.Structure):
    _fields_ = [("block_m", _I), ("block_n", _I), ("num_tiles", _I), ("num_workgroups", _I),
                ("kernel_id", _I), ("splits", _I), ("full_tiles", _I)]


class DgError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} "
                         f"({_lib.dg_status_string(status).decode() if _lib else '?'})")


def load_library(path=LIB_PATH):
    """Load libdg.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fp4_gemm_dense_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def lib():
    return load_library()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn, status):
    if status != DG_OK:
        raise DgError(fn, status)


def _req(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")


_U8 = torch.uint8
_BF = (torch.int16, torch.bfloat16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16, torch.bfloat16)


def _req_bf16(t, shape, name):
    if t.dtype not in _BF:
        raise TypeError(f"{name}: expected bf16 (or its int16 bit view), got {t.dtype}")
    _req(t, t.dtype, shape, name)


def _nb(n):
    return (n + 127) // 128


# dg_gemm_form (include/dg.h): which FP8 GEMM entry point a workspace query is for
FORM_NT, FORM_NN, FORM_TN, FORM_TT, FORM_NT_UE8M0 = 0, 1, 2, 3, 4
FORM_CONTIGUOUS_NT, FORM_CONTIGUOUS_NN, FORM_CONTIGUOUS_NT_UE8M0 = 5, 6, 7
FORM_MASKED_NT, FORM_MASKED_NT_UE8M0 = 8, 9


def dg_fp8_gemm_workspace_bytes(form, m, n, k, num_groups=1, expected_m=0, num_cus=0):
    """Bytes of workspace the FP8 GEMM entry point `form` needs for these sizes (0: none)."""
    return int(lib().dg_fp8_gemm_workspace_bytes(int(form), m, n, k, num_groups, int(expected_m), int(num_cus)))


def _workspace(form, m, n, k, num_groups, expected_m, device, workspace):
    """(pointer, bytes) of the workspace for one call: the caller's uint8 tensor, or a
    new one from torch's caching allocator when none is given and the plan needs one."""
    if workspace is not None:
        _req(workspace, _U8, (workspace.numel(),), "workspace")
        return _ptr(workspace), workspace.numel(), workspace
    need = dg_fp8_gemm_workspace_bytes(form, m, n, k, num_groups, expected_m)
    if need == 0:
        return None, 0, None
    ws = torch.empty(need, dtype=_U8, device=device)
    return _ptr(ws), need, ws


# ----------------------------------------------------------------------------
# C entry points (caller-allocated outputs)
# ----------------------------------------------------------------------------

def dg_fp8_gemm_nt(a, sfa, b, sfb, c, d, workspace=None):
    """d = c + a . b^T (see include/dg.h).  a/b uint8 e4m3, sfa [K/128, M], sfb [ceil(N/128), K/128].
    workspace: optional uint8 device tensor for the split-K partials (allocated here when needed
    and not given)."""
    L = lib()
    M, K = a.shape
    N = b.shape[0]
    _req(a, _U8, (M, K), "a")
    _req(b, _U8, (N, K), "b")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(sfb, torch.float32, (_nb(N), K // 128), "sfb")
    if c is not None:
        _req_bf16(c, (M, N), "c")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_NT, M, N, K, 1, 0, a.device, workspace)
    _check("dg_fp8_gemm_nt", L.dg_fp8_gemm_nt(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(c), _ptr(d),
                                              M, N, K, wp, wn, _stream(a)))
    return d


def dg_fp8_gemm_nt_noalloc(a, sfa, b, sfb, c, d):
    """d = c + a . b^T like dg_fp8_gemm_nt, with the split-K partials in the library's static
    per-GPU scratch buffer (24 MiB): the call allocates nothing.  Calls that overlap in time
    on one GPU race on that buffer."""
    L = lib()
    M, K = a.shape
    N = b.shape[0]
    _req(a, _U8, (M, K), "a")
    _req(b, _U8, (N, K), "b")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(sfb, torch.float32, (_nb(N), K // 128), "sfb")
    if c is not None:
        _req_bf16(c, (M, N), "c")
    _req_bf16(d, (M, N), "d")
    _check("dg_fp8_gemm_nt_noalloc", L.dg_fp8_gemm_nt_noalloc(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(c),
                                                              _ptr(d), M, N, K, _stream(a)))
    return d


def dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, m_indices, d, workspace=None):
    L = lib()
    M, K = a.shape
    G, N = b.shape[0], b.shape[1]
    _req(a, _U8, (M, K), "a")
    _req(b, _U8, (G, N, K), "b")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(sfb, torch.float32, (G, _nb(N), K // 128), "sfb")
    _req(m_indices, torch.int32, (M,), "m_indices")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_CONTIGUOUS_NT, M, N, K, G, 0, a.device, workspace)
    _check("dg_m_grouped_fp8_gemm_nt_contiguous",
           L.dg_m_grouped_fp8_gemm_nt_contiguous(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(m_indices),
                                                 _ptr(d), M, N, K, G, wp, wn, _stream(a)))
    return d


def dg_m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, masked_m, d, expected_m=0, workspace=None):
    L = lib()
    G, max_m, K = a.shape
    N = b.shape[1]
    _req(a, _U8, (G, max_m, K), "a")
    _req(b, _U8, (G, N, K), "b")
    _req(sfa, torch.float32, (G, K // 128, max_m), "sfa")
    _req(sfb, torch.float32, (G, _nb(N), K // 128), "sfb")
    _req(masked_m, torch.int32, (G,), "masked_m")
    _req_bf16(d, (G, max_m, N), "d")
    wp, wn, _keep = _workspace(FORM_MASKED_NT, max_m, N, K, G, expected_m, a.device, workspace)
    _check("dg_m_grouped_fp8_gemm_nt_masked",
           L.dg_m_grouped_fp8_gemm_nt_masked(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(masked_m), _ptr(d),
                                             G, max_m, N, K, int(expected_m), wp, wn, _stream(a)))
    return d


def dg_fp8_gemm_nn(a, sfa, b, sfb, c, d, workspace=None):
    """d = c + a . b with b stored [K, N] (NN layout)."""
    L = lib()
    M, K = a.shape
    N = b.shape[1]
    _req(a, _U8, (M, K), "a")
    _req(b, _U8, (K, N), "b")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(sfb, torch.float32, (_nb(N), K // 128), "sfb")
    if c is not None:
        _req_bf16(c, (M, N), "c")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_NN, M, N, K, 1, 0, a.device, workspace)
    _check("dg_fp8_gemm_nn", L.dg_fp8_gemm_nn(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(c), _ptr(d),
                                              M, N, K, wp, wn, _stream(a)))
    return d


def _dense_layout(name, form, a, sfa, b, sfb, c, d, a_km, b_kn, workspace):
    L = lib()
    if a_km:
        K, M = a.shape
    else:
        M, K = a.shape
    N = b.shape[1] if b_kn else b.shape[0]
    _req(a, _U8, (K, M) if a_km else (M, K), "a")
    _req(b, _U8, (K, N) if b_kn else (N, K), "b")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(sfb, torch.float32, (_nb(N), K // 128), "sfb")
    if c is not None:
        _req_bf16(c, (M, N), "c")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(form, M, N, K, 1, 0, a.device, workspace)
    _check(name, getattr(L, name)(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(c), _ptr(d), M, N, K, wp, wn,
                                  _stream(a)))
    return d


def dg_fp8_gemm_tn(a, sfa, b, sfb, c, d, workspace=None):
    """d = c + a^T b with a stored [K, M] and b stored [K, N] (TN layout)."""
    return _dense_layout("dg_fp8_gemm_tn", FORM_TN, a, sfa, b, sfb, c, d, True, True, workspace)


def dg_fp8_gemm_tt(a, sfa, b, sfb, c, d, workspace=None):
    """d = c + a^T b^T with a stored [K, M] and b stored [N, K] (TT layout)."""
    return _dense_layout("dg_fp8_gemm_tt", FORM_TT, a, sfa, b, sfb, c, d, True, False, workspace)


def dg_k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, ks, d):
    """d[g] = a[rows of g]^T . b[rows of g] with a stored [K, M], b [K, N], groups along K (ks on the device)."""
    L = lib()
    K, M = a.shape
    N = b.shape[1]
    G = ks.shape[0]
    _req(a, _U8, (K, M), "a")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(b, _U8, (K, N), "b")
    _req(sfb, torch.float32, (_nb(N), K // 128), "sfb")
    _req(ks, torch.int32, (G,), "ks")
    _req_bf16(d, (G, M, N), "d")
    _check("dg_k_grouped_fp8_gemm_tn_contiguous",
           L.dg_k_grouped_fp8_gemm_tn_contiguous(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(ks), _ptr(d),
                                                 M, N, K, G, _stream(a)))
    return d


def dg_m_grouped_fp8_gemm_nn_contiguous(a, sfa, b, sfb, m_indices, d, workspace=None):
    """Contiguous grouped form with each group's b stored [K, N]."""
    L = lib()
    M, K = a.shape
    G, N = b.shape[0], b.shape[2]
    _req(a, _U8, (M, K), "a")
    _req(sfa, torch.float32, (K // 128, M), "sfa")
    _req(b, _U8, (G, K, N), "b")
    _req(sfb, torch.float32, (G, _nb(N), K // 128), "sfb")
    _req(m_indices, torch.int32, (M,), "m_indices")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_CONTIGUOUS_NN, M, N, K, G, 0, a.device, workspace)
    _check("dg_m_grouped_fp8_gemm_nn_contiguous",
           L.dg_m_grouped_fp8_gemm_nn_contiguous(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(m_indices), _ptr(d),
                                                 M, N, K, G, wp, wn, _stream(a)))
    return d


def _kw(K):
    return (K // 128 + 3) // 4


def dg_fp8_gemm_nt_ue8m0(a, sfa, b, sfb, c, d, workspace=None):
    L = lib()
    M, K = a.shape
    N = b.shape[0]
    _req(a, _U8, (M, K), "a")
    _req(sfa, torch.int32, (M, _kw(K)), "sfa")
    _req(b, _U8, (N, K), "b")
    _req(sfb, torch.int32, (_nb(N), _kw(K)), "sfb")
    if c is not None:
        _req_bf16(c, (M, N), "c")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_NT_UE8M0, M, N, K, 1, 0, a.device, workspace)
    _check("dg_fp8_gemm_nt_ue8m0",
           L.dg_fp8_gemm_nt_ue8m0(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(c),
                                  _ptr(d), M, N, K, wp, wn, _stream(a)))
    return d


def dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(a, sfa, b, sfb, m_indices, d, workspace=None):
    L = lib()
    M, K = a.shape
    G, N = b.shape[0], b.shape[1]
    _req(a, _U8, (M, K), "a")
    _req(sfa, torch.int32, (M, _kw(K)), "sfa")
    _req(b, _U8, (G, N, K), "b")
    _req(sfb, torch.int32, (G, _nb(N), _kw(K)), "sfb")
    _req(m_indices, torch.int32, (M,), "m_indices")
    _req_bf16(d, (M, N), "d")
    wp, wn, _keep = _workspace(FORM_CONTIGUOUS_NT_UE8M0, M, N, K, G, 0, a.device, workspace)
    _check("dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
           L.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(m_indices),
                                                       _ptr(d), M, N, K, G, wp, wn, _stream(a)))
    return d


def dg_m_grouped_fp8_gemm_nt_masked_ue8m0(a, sfa, b, sfb, masked_m, d, expected_m=0, workspace=None):
    L = lib()
    G, max_m, K = a.shape
    N = b.shape[1]
    _req(a, _U8, (G, max_m, K), "a")
    _req(sfa, torch.int32, (G, max_m, _kw(K)), "sfa")
    _req(b, _U8, (G, N, K), "b")
    _req(sfb, torch.int32, (G, _nb(N), _kw(K)), "sfb")
    _req(masked_m, torch.int32, (G,), "masked_m")
    _req_bf16(d, (G, max_m, N), "d")
    wp, wn, _keep = _workspace(FORM_MASKED_NT_UE8M0, max_m, N, K, G, expected_m, a.device, workspace)
    _check("dg_m_grouped_fp8_gemm_nt_masked_ue8m0",
           L.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(masked_m),
                                                   _ptr(d), G, max_m, N, K, int(expected_m), wp, wn, _stream(a)))
    return d


def dg_m_grouped_fp8_fp4_gemm_nt_contiguous(a, a_sf, b, b_sf, m_indices, d):
    L = lib()
    M, K = a.shape
    G, N = b.shape[0], b.shape[1]
    _req(a, _U8, (M, K), "a")
    _req(a_sf, torch.int32, (M, (K // 128 + 3) // 4), "a_sf")
    _req(b, _U8, (G, N, K // 2), "b")
    _req(b_sf, torch.int32, (G, K // 128, N), "b_sf")
    _req(m_indices, torch.int32, (M,), "m_indices")
    _req_bf16(d, (M, N), "d")
    _check("dg_m_grouped_fp8_fp4_gemm_nt_contiguous",
           L.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(m_indices),
                                                     _ptr(d), M, N, K, G, _stream(a)))
    return d


def dg_m_grouped_fp8_fp4_gemm_nt_masked(a, a_sf, b, b_sf, masked_m, d, expected_m=0):
    L = lib()
    G, max_m, K = a.shape
    N = b.shape[1]
    _req(a, _U8, (G, max_m, K), "a")
    _req(a_sf, torch.int32, (G, max_m, (K // 128 + 3) // 4), "a_sf")
    _req(b, _U8, (G, N, K // 2), "b")
    _req(b_sf, torch.int32, (G, K // 128, N), "b_sf")
    _req(masked_m, torch.int32, (G,), "masked_m")
    _req_bf16(d, (G, max_m, N), "d")
    _check("dg_m_grouped_fp8_fp4_gemm_nt_masked",
           L.dg_m_grouped_fp8_fp4_gemm_nt_masked(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(masked_m),
                                                 _ptr(d), G, max_m, N, K, int(expected_m), _stream(a)))
    return d


def dg_transform_fp4_weight_sf(sf, sf_t=None):
    """Packed UE8M0 weight-scale words [G, N, K/128] -> K-block-major [G, K/128, N] (new tensor
    unless sf_t is given)."""
    G, N, KB = sf.shape
    _req(sf, torch.int32, (G, N, KB), "sf")
    if sf_t is None:
        sf_t = torch.empty(G, KB, N, dtype=torch.int32, device=sf.device)
    _req(sf_t, torch.int32, (G, KB, N), "sf_t")
    _check("dg_transform_fp4_weight_sf",
           lib().dg_transform_fp4_weight_sf(_ptr(sf), _ptr(sf_t), G, N, KB * 128, _stream(sf)))
    return sf_t


def dg_fp8_fp4_expert_ffn_workspace_bytes(num_tokens, num_topk, num_local_experts, hidden, intermediate):
    return int(lib().dg_fp8_fp4_expert_ffn_workspace_bytes(num_tokens, num_topk, num_local_experts,
                                                            hidden, intermediate))


def dg_fp8_fp4_expert_ffn(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, expert_offset, workspace):
    L = lib()
    T, H = x.shape
    k = topk_idx.shape[1]
    E, I2 = w1.shape[0], w1.shape[1]
    I = I2 // 2
    _req(x, _U8, (T, H), "x")
    _req(x_sf, torch.int32, (T, H // 512), "x_sf")
    _req(topk_idx, torch.int32, (T, k), "topk_idx")
    _req(topk_w, torch.float32, (T, k), "topk_w")
    _req(w1, _U8, (E, 2 * I, H // 2), "w1")
    _req(w1_sf, torch.int32, (E, H // 128, 2 * I), "w1_sf")
    _req(w2, _U8, (E, H, I // 2), "w2")
    _req(w2_sf, torch.int32, (E, I // 128, H), "w2_sf")
    _req_bf16(y, (T, H), "y")
    _req(workspace, _U8, (workspace.numel(),), "workspace")
    _check("dg_fp8_fp4_expert_ffn",
           L.dg_fp8_fp4_expert_ffn(_ptr(x), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_w), _ptr(w1), _ptr(w1_sf),
                                   _ptr(w2), _ptr(w2_sf), _ptr(y), T, k, E, int(expert_offset), H, I,
                                   _ptr(workspace), workspace.numel(), _stream(x)))
    return y


def dg_get_mk_alignment_for_contiguous_layout():
    return int(lib().dg_get_mk_alignment_for_contiguous_layout())


def dg_set_num_cus(n):
    _check("dg_set_num_cus", lib().dg_set_num_cus(int(n)))


def dg_get_num_cus():
    return int(lib().dg_get_num_cus())


def dg_query_plan(m, n, k, num_groups=1, num_cus=0):
    p = DgPlan()
    _check("dg_query_plan", lib().dg_query_plan(m, n, k, num_groups, num_cus, ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in DgPlan._fields_}


def dg_query_plan_contiguous(m, n, k, num_groups, num_cus=0):
    p = DgPlan()
    _check("dg_query_plan_contiguous",
           lib().dg_query_plan_contiguous(m, n, k, num_groups, num_cus, ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in DgPlan._fields_}


def dg_query_plan_form(form, m, n, k, num_groups=1, expected_m=0, num_cus=0):
    """The plan of a call of the given form (FORM_* constant)."""
    p = DgPlan()
    _check("dg_query_plan_form",
           lib().dg_query_plan_form(form, m, n, k, num_groups, expected_m, num_cus, ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in DgPlan._fields_}


def dg_num_tiles(m, n, block_m, block_n):
    return int(lib().dg_num_tiles(m, n, block_m, block_n))


# ----------------------------------------------------------------------------
# allocating conveniences (the pages' Python-style API)
# ----------------------------------------------------------------------------

def fp8_gemm_nt(a, sfa, b, sfb, c=None):
    """Returns a new bf16 tensor d = c + a . b^T."""
    d = torch.empty(a.shape[0], b.shape[0], dtype=torch.bfloat16, device=a.device)
    if c is not None and c.dtype == torch.int16:
        d = d.view(torch.int16)
    return dg_fp8_gemm_nt(a, sfa, b, sfb, c, d)


def m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, m_indices, out=None):
    d = out if out is not None else torch.empty(a.shape[0], b.shape[1], dtype=torch.bfloat16, device=a.device)
    return dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, m_indices, d)


def m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, masked_m, expected_m=0, out=None):
    d = out if out is not None else torch.empty(a.shape[0], a.shape[1], b.shape[1], dtype=torch.bfloat16,
                                                device=a.device)
    return dg_m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, masked_m, d, expected_m)


def transform_weights_for_expert_ffn(l1_weights, l2_weights):
    """(w1, w1_sf), (w2, w2_sf) with row-major scale words -> the same pairs with the scale
    words K-block-major, the layout dg_fp8_fp4_expert_ffn reads; the E2M1 bytes are unchanged."""
    (w1, w1_sf), (w2, w2_sf) = l1_weights, l2_weights
    return (w1, dg_transform_fp4_weight_sf(w1_sf)), (w2, dg_transform_fp4_weight_sf(w2_sf))


def fp8_fp4_expert_ffn(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, expert_offset=0, workspace=None):
    T, H = x.shape
    E, I2 = w1.shape[0], w1.shape[1]
    nbytes = dg_fp8_fp4_expert_ffn_workspace_bytes(T, topk_idx.shape[1], E, H, I2 // 2)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    return dg_fp8_fp4_expert_ffn(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, expert_offset, workspace)


def dg_status_string(status):
    return lib().dg_status_string(int(status)).decode()
