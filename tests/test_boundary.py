"""Host-side checks of the C-ABI library: it loads, exports every symbol that
include/dg.h declares, and rejects invalid arguments before any HIP call.
No compute is launched here (these tests run without a GPU)."""

import ctypes
import json
import os
import re

import pytest

import fp4_gemm_dense_amd as dgm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dgm.load_library()
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
    # the binding wraps every one of them under the same name
    for name in names:
        assert callable(getattr(dgm, name)), name


def test_status_strings_and_constants():
    lib = dgm.load_library()
    for s in range(5):
        assert lib.dg_status_string(s)
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128


def test_tile_count_golden_from_pages():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "tile_counts.json")))
    for c in g["cases"]:
        assert dgm.dg_num_tiles(c["m"], c["n"], c["block_m"], c["block_n"]) == c["tiles"]
        assert c["tiles"] <= c["units"]


def test_planner_reproduces_the_pages_non_power_of_two_block_n():
    """The release article's example as a planner decision: M=256, N=7168 on 132
    compute units, where 128-wide tiles leave 20 units idle (112 tiles) and the
    112-wide tile occupies 128.  With K short enough that splitting K does not pay,
    the planner takes 128 x 112 tiles, one per workgroup."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "tile_counts.json")))
    pow2, npow2 = g["cases"]
    units = npow2["units"]
    for k in (512, 1024, 1536):
        p = dgm.dg_query_plan(npow2["m"], npow2["n"], k, 1, units)
        assert (p["block_m"], p["block_n"]) == (npow2["block_m"], npow2["block_n"]), p
        assert p["num_tiles"] == npow2["tiles"] and p["splits"] == 1, p
        assert p["num_workgroups"] == npow2["tiles"] <= units
        assert p["num_tiles"] > pow2["tiles"]
    # on 256 units the same problem keeps the square-tile kernel, whose tiles fill
    # the chip well enough; up to 128 rows non-power-of-two widths are ordinary
    # choices (e.g. the 96-wide tile)
    assert dgm.dg_query_plan(256, 7168, 1024, 1, 256)["kernel_id"] < 100
    widths = {dgm.dg_query_plan(m, n, k, 1, 256)["block_n"] for m, n, k in
              [(64, 24576, 1536), (128, 2112, 7168), (64, 7168, 16384), (192, 7168, 4096)]}
    assert widths & {96, 112, 224}, widths


A16 = 0x10000   # fake 16-byte-aligned "device" addresses: never dereferenced on the host


@pytest.mark.parametrize("args,status", [
    ((0, A16, A16, A16, 0, A16, 64, 64, 128), 1),          # null a
    ((A16, A16, A16, A16, 0, A16, 0, 64, 128), 1),         # m = 0
    ((A16, A16, A16, A16, 0, A16, 64, -1, 128), 1),        # n < 0
    ((A16 + 4, A16, A16, A16, 0, A16, 64, 64, 128), 1),    # misaligned a
    ((A16, A16 + 2, A16, A16, 0, A16, 64, 64, 128), 1),    # misaligned sfa
    ((A16, A16, A16, A16, 0, A16, 64, 64, 100), 2),        # K % 128 != 0
    ((A16, A16, A16, A16, 0, A16, 64, 40, 128), 2),        # N % 16 != 0
    ((A16, A16, A16, A16, 0, A16, 1 << 21, 64, 1152), 2),  # A above 2 GiB (32-bit buffer offsets)
    ((A16, A16, A16, A16, 0, A16, 64, 1 << 21, 1152), 2),  # B above 2 GiB
    ((A16, A16, A16, A16, 0, A16, 1 << 15, (1 << 15) + 16, 128), 2),  # D above 2 GiB
    ((A16, A16, A16, A16, 0, A16, 1 << 15, 1 << 15, 128), -1),  # D of exactly 2 GiB: accepted
])
def test_dense_argument_validation(args, status):
    lib = dgm.load_library()
    got = lib.dg_fp8_gemm_nt(*args, None, 0, None)
    if status < 0:
        # passes validation; without a gfx950 device the call stops at the device check
        assert got in (0, 4)
    else:
        assert got == status


def test_fp8_fp4_grouped_argument_validation():
    lib = dgm.load_library()
    f = lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous
    assert f(A16, A16, A16, A16, 0, A16, 256, 256, 128, 4, None) == 1           # null m_indices
    assert f(A16, A16, A16, A16, A16, A16, 256, 256, 128, 0, None) == 1         # no groups
    assert f(A16 + 8, A16, A16, A16, A16, A16, 256, 256, 128, 4, None) == 1     # misaligned a
    assert f(A16, A16 + 2, A16, A16, A16, A16, 256, 256, 128, 4, None) == 1     # misaligned a_sf
    assert f(A16, A16, A16, A16, A16, A16, 256, 264, 128, 4, None) == 2         # N % 16
    assert f(A16, A16, A16, A16, A16, A16, 256, 272, 128, 4, None) in (0, 4)    # partial column tile: valid
    assert f(A16, A16, A16, A16, A16, A16, 256, 256, 200, 4, None) == 2         # K % 128
    assert f(A16, A16, A16, A16, A16, A16, 1 << 21, 256, 1152, 4, None) == 2    # A above 2 GiB
    assert f(A16, A16, A16, A16, A16, A16, 256, 256, 128, 4, None) in (0, 4)    # valid: device check
    g = lib.dg_m_grouped_fp8_fp4_gemm_nt_masked
    assert g(A16, A16, A16, A16, 0, A16, 4, 256, 256, 128, 0, None) == 1        # null masked_m
    assert g(A16, A16, A16, A16, A16, A16, 4, 0, 256, 128, 0, None) == 1        # max_m = 0
    assert g(A16, A16, A16, A16, A16, A16, 300, 64, 256, 128, 0, None) == 2     # more than 256 groups
    assert g(A16, A16, A16, A16, A16, A16, 4, 256, 256, 128, 0, None) in (0, 4)


def test_transform_fp4_weight_sf_argument_validation():
    lib = dgm.load_library()
    t = lib.dg_transform_fp4_weight_sf
    far = A16 + (1 << 24)
    assert t(0, far, 2, 256, 512, None) == 1                                     # null input
    assert t(A16, far, 0, 256, 512, None) == 1                                   # no groups
    assert t(A16 + 2, far, 2, 256, 512, None) == 1                               # misaligned
    assert t(A16, A16 + 64, 2, 256, 512, None) == 1                              # output overlaps input
    assert t(A16, far, 2, 256, 500, None) == 2                                   # K % 128
    assert t(A16, far, 70000, 1, 128, None) == 2                                 # grid z limit
    assert t(A16, far, 2, 256, 512, None) in (0, 4)                              # valid: device check


def test_grouped_and_ffn_argument_validation():
    lib = dgm.load_library()
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert f(A16, A16, A16, A16, 0, A16, 256, 64, 128, 4, None, 0, None) == 1            # null m_indices
    assert f(A16, A16, A16, A16, A16, A16, 256, 64, 128, 0, None, 0, None) == 1          # no groups
    assert f(A16, A16, A16, A16, A16, A16, 256, 64, 384 + 1, 4, None, 0, None) == 2
    g = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert g(A16, A16, A16, A16, 0, A16, 4, 256, 64, 128, 0, None, 0, None) == 1         # null masked_m
    assert g(A16, A16, A16, A16, A16, A16, 4, 0, 64, 128, 0, None, 0, None) == 1         # max_m = 0
    assert g(A16, A16, A16, A16, A16, A16, 4, 256, 72, 128, 0, None, 0, None) == 2       # N % 16
    assert g(A16, A16, A16, A16, A16, A16, 4, 1 << 15, (1 << 15) + 16, 128, 0, None, 0, None) == 2  # D > 2 GiB
    h = lib.dg_fp8_fp4_expert_ffn
    ws = lib.dg_fp8_fp4_expert_ffn_workspace_bytes(64, 8, 4, 512, 256)
    assert lib.dg_fp8_fp4_expert_ffn_workspace_bytes(0, 8, 4, 512, 256) == 0
    common = (A16, A16, A16, A16, A16, A16, A16, A16, A16)
    assert h(*common, 64, 8, 4, 0, 500, 256, A16, ws, None) == 2                # H % 512
    assert h(*common, 64, 8, 4, 0, 512, 200, A16, ws, None) == 2                # I % 128
    assert h(*common, 64, 8, 4, 0, 512, 256, A16, max(ws, 1) - 1, None) in (1, 2)  # workspace too small
    assert h(*common, 64, 0, 4, 0, 512, 256, A16, ws, None) == 1                # no slots
    assert h(0, *common[1:], 64, 8, 4, 0, 512, 256, A16, ws, None) == 1         # null x


def test_set_num_cus_rejects_negative():
    lib = dgm.load_library()
    assert lib.dg_set_num_cus(-3) == 1
    assert lib.dg_set_num_cus(0) == 0


def test_planner_is_host_only_and_fills_the_chip():
    # with an explicit CU count the plan needs no device
    for (m, n, k) in [(4096, 7168, 2048), (4096, 2112, 7168), (64, 32768, 512), (128, 2112, 7168)]:
        p = dgm.dg_query_plan(m, n, k, 1, 256)
        assert p["num_tiles"] == dgm.dg_num_tiles(m, n, p["block_m"], p["block_n"])
        assert p["splits"] >= 1
        assert 0 < p["num_workgroups"] <= max(p["num_tiles"] * p["splits"], 1)
        assert p["num_workgroups"] <= 256 * 4
    # skinny M: the 17 output tiles of a 128 x 2112 x 7168 problem are split along
    # K so that the work units fill the chip; K slices hold whole 128-wide blocks
    p = dgm.dg_query_plan(128, 2112, 7168, 1, 256)
    assert p["splits"] > 1 and p["num_tiles"] * p["splits"] > 128
    assert p["splits"] <= 7168 // 128 // 4
    assert p["full_tiles"] == 0, "skinny M splits every tile"
    # ... on the skinny-M kernel with all 128 rows of A in one tile, so that B (15 MB,
    # the bulk of the call's bytes) streams from HBM once
    assert p["kernel_id"] >= 100 and p["block_m"] == 128 and p["num_tiles"] == -(-2112 // p["block_n"])
    # a problem that already fills the chip is not split: 4096 x 7168 x 2048 has a
    # half-empty last round, but 16 K blocks are too few to gain from splitting it
    p = dgm.dg_query_plan(4096, 7168, 2048, 1, 256)
    assert p["splits"] == 1 and p["full_tiles"] == p["num_tiles"]
    # whole rounds need no split either
    p = dgm.dg_query_plan(4096, 4096, 7168, 1, 256)
    assert p["num_tiles"] % 256 == 0 and p["splits"] == 1


@pytest.mark.parametrize("m,n,k", [(3072, 6144, 16384), (4096, 2112, 7168), (2304, 3840, 4096)])
def test_planner_splits_only_the_last_partial_round(m, n, k):
    """Long K with a partial last round: the whole rounds run unsplit and only the
    remainder is split, into slices that together fit in one round (the first
    shape on the 256 x 256 tile: 288 tiles, 32 of them split)."""
    slots = 256
    p = dgm.dg_query_plan(m, n, k, 1, slots)
    tiles, full, s = p["num_tiles"], p["full_tiles"], p["splits"]
    assert s > 1, p
    assert full % slots == 0 and 0 < tiles - full <= slots // 2
    assert (tiles - full) * s <= slots
    assert p["num_workgroups"] == slots
    kb = k // 128
    per = -(-kb // s)
    assert per >= 4 and kb - per >= 24   # slices of >= 4 K blocks; the tail gains >= 24 blocks


def test_planner_split_tail_with_a_cu_cap():
    # the same rule on a capped part: 40 tiles (256 x 128 or 128 x 256) on 32
    # CUs leave a remainder of 8, split 4 ways over K = 128 * 32
    p = dgm.dg_query_plan(1280, 1024, 128 * 32, 1, 32)
    if p["block_m"] * p["block_n"] == 256 * 128:
        assert p["full_tiles"] == 32 and p["splits"] == 4
    assert p["full_tiles"] % 32 == 0 or p["full_tiles"] == p["num_tiles"]


def test_split_rule_mirror_matches_the_planner():
    """The host mirror of the split rule used by the masked-form GPU tests agrees
    with the library's dense plans (same rule, whole-tile count known on the host)."""
    from tests.test_gpu_splitk import _split_rule
    for (m, n, k, cus) in [(4096, 7168, 16384, 256), (4096, 2112, 7168, 256), (2304, 3840, 4096, 256),
                           (4096, 7168, 2048, 256), (128, 2112, 7168, 256), (1280, 1024, 4096, 32),
                           (64, 7168, 16384, 256), (1100, 1040, 7680, 32), (1300, 1040, 4608, 48)]:
        p = dgm.dg_query_plan(m, n, k, 1, cus)
        if p["kernel_id"] >= 100:
            continue   # skinny M: its own plan (test_skinny_plans_fill_one_round)
        s, full = _split_rule(p["num_tiles"], cus, k // 128)
        assert (s, full) == (p["splits"], p["full_tiles"]), (m, n, k, cus, p)


def test_contiguous_plan_query_is_host_only_and_may_split():
    # 33280 rows (8 groups padded to 128) x 4096 x 7168 on 256 CUs: 4160 tiles of
    # 128 x 256, the last 64 split along K
    p = dgm.dg_query_plan_contiguous(33280, 4096, 7168, 8, 256)
    assert p["block_m"] <= 128 and 128 % p["block_m"] == 0   # blocks stay group-pure
    assert p["num_tiles"] == dgm.dg_num_tiles(33280, 4096, p["block_m"], p["block_n"])
    assert p["splits"] > 1 and p["full_tiles"] % 256 == 0 and p["full_tiles"] < p["num_tiles"]
    p = dgm.dg_query_plan_contiguous(33280, 7168, 2048, 8, 256)
    assert p["splits"] == 1 and p["full_tiles"] == p["num_tiles"]


# ---------------------------------------------------------------------------
# split-K workspace: sized by a host-only query, bounded by one fp32 partial
# tile per workgroup slot, never allocated by the library
# ---------------------------------------------------------------------------
_DENSE_FORMS = [dgm.FORM_NT, dgm.FORM_NN, dgm.FORM_TN, dgm.FORM_TT, dgm.FORM_NT_UE8M0]
_CONFIG_SHAPES = [(128, 2112, 7168)] + [(m, n, k) for m in (64, 4096) for (n, k) in
                                       [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168),
                                        (7168, 2048)]]


def _check_ws_bound(form, m, n, k, groups, cus, expected_m=0):
    ws = dgm.dg_fp8_gemm_workspace_bytes(form, m, n, k, groups, expected_m, cus)
    if form in _DENSE_FORMS or form in (dgm.FORM_CONTIGUOUS_NT, dgm.FORM_CONTIGUOUS_NN,
                                        dgm.FORM_CONTIGUOUS_NT_UE8M0):
        q = dgm.dg_query_plan_form(form, m, n, k, groups, expected_m, cus)
        split_tiles = q["num_tiles"] - q["full_tiles"]
        want = split_tiles * q["splits"] * q["block_m"] * q["block_n"] * 4 if q["splits"] > 1 else 0
        assert ws == want, (form, m, n, k, q, ws)
        assert split_tiles * q["splits"] <= cus, "at most one partial tile per workgroup slot"
    # the bound every plan respects: one fp32 partial of the largest tile per slot
    assert ws <= cus * 256 * 256 * 4, (form, m, n, k, groups, ws)
    return ws


def test_form_plan_query_names_each_forms_kernel():
    """dg_query_plan_form plans each form as its call does: NT with fp32 scales takes
    the skinny-M kernel for short M, the UE8M0 and transposed layouts keep the square
    kernel; NT and contiguous NT agree with the older queries; a bad form is refused."""
    for (m, n, k) in _CONFIG_SHAPES:
        assert dgm.dg_query_plan_form(dgm.FORM_NT, m, n, k, 1, 0, 256) == dgm.dg_query_plan(m, n, k, 1, 256)
        for form in (dgm.FORM_NN, dgm.FORM_TN, dgm.FORM_TT, dgm.FORM_NT_UE8M0):
            assert dgm.dg_query_plan_form(form, m, n, k, 1, 0, 256)["kernel_id"] < 100, (form, m, n, k)
    assert dgm.dg_query_plan_form(dgm.FORM_NT, 64, 4096, 7168, 1, 0, 256)["kernel_id"] >= 100
    for (n, k) in [(4096, 7168), (7168, 2048)]:
        assert (dgm.dg_query_plan_form(dgm.FORM_CONTIGUOUS_NT, 33280, n, k, 8, 0, 256)
                == dgm.dg_query_plan_contiguous(33280, n, k, 8, 256))
    with pytest.raises(RuntimeError):
        dgm.dg_query_plan_form(99, 128, 128, 128, 1, 0, 256)


def test_wide_tile_is_dense_nt_only(monkeypatch):
    """The 256 x 256 and 256 x 224 tiles (kernels 4, 6) serve the dense NT form
    with fp32 scales only, the 128 x 512 tile (kernel 5) that and the contiguous
    NT form: pinned
    on another form the pin is ignored; pinned on NT it is planned, with its
    workspace (split K) counted like any other tile's; a shape whose row offsets
    would pass 2^32 bytes keeps the square tiles."""
    for kid in (4, 5, 6):
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kid))
        for form in (dgm.FORM_NN, dgm.FORM_TN, dgm.FORM_TT, dgm.FORM_NT_UE8M0):
            assert dgm.dg_query_plan_form(form, 1024, 1024, 1024, 1, 0, 256)["kernel_id"] != kid, form
        for form in (dgm.FORM_CONTIGUOUS_NN, dgm.FORM_CONTIGUOUS_NT_UE8M0):
            assert dgm.dg_query_plan_form(form, 1024, 1024, 1024, 4, 0, 256)["kernel_id"] != kid, form
        assert dgm.dg_query_plan_form(dgm.FORM_MASKED_NT, 256, 1024, 1024, 8, 128, 256)["kernel_id"] != kid
        p = dgm.dg_query_plan_form(dgm.FORM_NT, 1000, 1040, 2048, 1, 0, 256)
        assert p["kernel_id"] == kid
        _check_ws_bound(dgm.FORM_NT, 1000, 1040, 2048, 1, 256)
    monkeypatch.setenv("DG_FORCE_KERNEL", "5")
    p = dgm.dg_query_plan_form(dgm.FORM_CONTIGUOUS_NT, 1024, 1024, 1024, 4, 0, 256)
    assert (p["kernel_id"], p["block_m"], p["block_n"]) == (5, 128, 512)
    for kid in (4, 6):
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kid))
        assert dgm.dg_query_plan_form(dgm.FORM_CONTIGUOUS_NT, 1024, 1024, 1024, 4, 0, 256)["kernel_id"] != kid
    monkeypatch.setenv("DG_FORCE_KERNEL", "4")
    p = dgm.dg_query_plan_form(dgm.FORM_NT, 1000, 1040, 2048, 1, 0, 256)
    assert (p["kernel_id"], p["block_m"], p["block_n"], p["num_tiles"]) == (4, 256, 256, 4 * 5)
    _check_ws_bound(dgm.FORM_NT, 1000, 1040, 2048, 1, 256)
    assert dgm.dg_query_plan_form(dgm.FORM_NT, 4096, 4096, 7168, 1, 0, 256)["splits"] == 1
    # (m + 256) * k must stay below 2^32: 2^31 bytes of A and B at K = 2^24 do not
    assert dgm.dg_query_plan_form(dgm.FORM_NT, 128, 128, 1 << 24, 1, 0, 256)["kernel_id"] != 4
    assert dgm.dg_query_plan_form(dgm.FORM_NT, 128, 128, 1 << 22, 1, 0, 256)["kernel_id"] == 4


def test_workspace_query_matches_the_plan_and_the_bound():
    for (m, n, k) in _CONFIG_SHAPES:
        for form in _DENSE_FORMS:
            _check_ws_bound(form, m, n, k, 1, 256)
    assert dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, 128, 2112, 7168, 1, 0, 256) > 0   # skinny: split
    assert dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, 4096, 4096, 7168, 1, 0, 256) == 0  # whole rounds
    # grouped configurations: 8 groups padded to 128 (contiguous), 32 x 256 (masked)
    for (n, k) in [(4096, 7168), (7168, 2048)]:
        for form in (dgm.FORM_CONTIGUOUS_NT, dgm.FORM_CONTIGUOUS_NN, dgm.FORM_CONTIGUOUS_NT_UE8M0):
            _check_ws_bound(form, 33280, n, k, 8, 256)
        for form in (dgm.FORM_MASKED_NT, dgm.FORM_MASKED_NT_UE8M0):
            ws = _check_ws_bound(form, 256, n, k, 32, 256, expected_m=128)
            p = dgm.dg_query_plan(256, n, k, 32, 256)
            assert ws in (0, 256 * p["block_m"] * p["block_n"] * 4)


def test_workspace_query_random_shapes_fit_the_bound():
    import numpy as np
    rng = np.random.default_rng(2024)
    for _ in range(1000):
        m = int(rng.integers(1, 8193))
        n = int(rng.integers(1, 2049)) * 16
        k = int(rng.integers(1, 161)) * 128
        cus = int(rng.choice([256, 255, 200, 128, 80, 32, 7, 1]))
        form = int(rng.integers(0, 10))
        groups = int(rng.integers(1, 33))
        if form >= dgm.FORM_MASKED_NT:
            _check_ws_bound(form, min(m, 1024), n, k, groups, cus, expected_m=int(rng.integers(0, 300)))
        elif form >= dgm.FORM_CONTIGUOUS_NT:
            _check_ws_bound(form, (m + 127) // 128 * 128, n, k, groups, cus)
        else:
            if form in (dgm.FORM_TN, dgm.FORM_TT):
                m = (m + 15) // 16 * 16
            _check_ws_bound(form, m, n, k, 1, cus)


def test_workspace_query_rejects_invalid_sizes():
    for args in [(dgm.FORM_NT, 0, 64, 128), (dgm.FORM_NT, 64, 40, 128), (dgm.FORM_NT, 64, 64, 100), (99, 64, 64, 128)]:
        assert dgm.dg_fp8_gemm_workspace_bytes(*args, 1, 0, 256) == 0
