"""Stream behaviour of the C ABI on the GPU: calls enqueue on the caller's stream without
host synchronisation or allocation, so they can be captured into a HIP graph and replayed,
and calls on different streams may run at the same time (each call's split-K workspace is
the caller's).

Each replay is checked bit for bit against an eager call of the same inputs, with eager
work on the same buffers between the replays.
"""

import numpy as np
import pytest
import torch

import synth
from tests.helpers import bits

pytestmark = pytest.mark.gpu


def _dense_call(dg, g, d):
    dg.dg_fp8_gemm_nt(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)


@pytest.mark.parametrize("M,N,K", [(512, 1024, 1024),     # whole tiles
                                   (64, 2112, 7168)])      # split along K: workspace + reduce kernel
def test_dense_graph_capture_replays_match_eager(dg, M, N, K):
    g = synth.gen_dense(M, N, K, seed=M + N + K, backend="torch", device="cuda")
    d_ref = torch.empty(M, N, dtype=torch.int16, device="cuda")
    _dense_call(dg, g, d_ref)
    torch.cuda.synchronize()
    want = bits(d_ref)
    s = torch.cuda.Stream()
    d = torch.empty(M, N, dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        _dense_call(dg, g, d)
    for rep in range(3):
        d.fill_(-1)                      # eager work on the output between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), want), f"replay {rep} differs from the eager result"


def test_graph_replay_after_a_larger_eager_split_call(dg):
    """A captured split call keeps its own workspace: a larger split call run eagerly on
    the same stream after the capture (its own, larger workspace) does not disturb the
    replays, which match the eager result bit for bit."""
    small, large = (16, 512, 8192), (128, 2112, 7168)
    gs = synth.gen_dense(*small, seed=31, backend="torch", device="cuda")
    gl = synth.gen_dense(*large, seed=32, backend="torch", device="cuda")
    for shp in (small, large):
        assert dg.dg_fp8_gemm_workspace_bytes(dg.FORM_NT, *shp) > 0, "both calls must split along K"
    assert dg.dg_fp8_gemm_workspace_bytes(dg.FORM_NT, *large) > dg.dg_fp8_gemm_workspace_bytes(dg.FORM_NT, *small)
    want_s = torch.empty(small[0], small[1], dtype=torch.int16, device="cuda")
    want_l = torch.empty(large[0], large[1], dtype=torch.int16, device="cuda")
    _dense_call(dg, gs, want_s)
    _dense_call(dg, gl, want_l)
    torch.cuda.synchronize()
    ws_s, ws_l = bits(want_s), bits(want_l)
    s = torch.cuda.Stream()
    d = torch.empty(small[0], small[1], dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        _dense_call(dg, gs, d)
    dl = torch.empty(large[0], large[1], dtype=torch.int16, device="cuda")
    for rep in range(3):
        with torch.cuda.stream(s):
            dl.fill_(-1)
            _dense_call(dg, gl, dl)          # larger split call, eager, same stream
            d.fill_(-1)
            graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), ws_s), f"replay {rep} differs from the eager result"
        assert np.array_equal(bits(dl), ws_l), f"eager large call {rep} differs"


def test_masked_graph_capture_replays_match_eager(dg):
    """The masked form reads masked_m only on the device: new counts written into the
    same buffer between replays change what each replay computes."""
    G, max_m, N, K = 6, 192, 512, 4096
    g = synth.gen_masked(G, max_m, N, K, seed=77, masked_m=[0, 192, 5, 100, 129, 64],
                         backend="torch", device="cuda")
    mm = g["masked_m"]
    s = torch.cuda.Stream()
    d = torch.full((G, max_m, N), -1, dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        dg.dg_m_grouped_fp8_gemm_nt_masked(g["a"], g["sfa"], g["b"], g["sfb"], mm, d, 128)
    for rep, counts in enumerate([[0, 192, 5, 100, 129, 64], [3, 0, 192, 1, 64, 128], [0, 192, 5, 100, 129, 64]]):
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        d_ref = torch.full((G, max_m, N), -1, dtype=torch.int16, device="cuda")
        dg.dg_m_grouped_fp8_gemm_nt_masked(g["a"], g["sfa"], g["b"], g["sfb"], mm, d_ref, 128)
        d.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), bits(d_ref)), f"replay {rep} (masked_m {counts}) differs from eager"


def test_ffn_graph_capture_replays_match_eager(dg):
    gen = synth.gen_ffn(T=96, H=512, I=256, num_local=4, num_experts=8, topk=4, seed=21)
    t = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in gen.items()}
    (w1, w1_sf), (w2, w2_sf) = dg.transform_weights_for_expert_ffn((t["w1"], t["w1_sf"]), (t["w2"], t["w2_sf"]))
    T, H = t["x"].shape
    ws = torch.zeros(dg.dg_fp8_fp4_expert_ffn_workspace_bytes(T, 4, 4, H, 256), dtype=torch.uint8, device="cuda")

    def call(y):
        dg.dg_fp8_fp4_expert_ffn(t["x"], t["x_sf"], t["topk_idx"], t["topk_w"], w1, w1_sf, w2, w2_sf, y, 0, ws)
    y_ref = torch.empty(T, H, dtype=torch.int16, device="cuda")
    call(y_ref)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call(y)
    for rep in range(3):
        y.fill_(-1)
        ws.fill_(0xAB)                   # the workspace's contents on entry are ignored
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(y_ref)), f"FFN replay {rep} differs from eager"


def test_two_streams_concurrently_match_single_stream(dg):
    """Split-K calls on two streams at once (each call with its own workspace) give the
    single-stream results."""
    shapes = [(64, 2112, 7168), (96, 4096, 7168)]
    gens = [synth.gen_dense(M, N, K, seed=500 + M, backend="torch", device="cuda") for M, N, K in shapes]
    refs = []
    for (M, N, K), g in zip(shapes, gens):
        d = torch.empty(M, N, dtype=torch.int16, device="cuda")
        _dense_call(dg, g, d)
        torch.cuda.synchronize()
        refs.append(bits(d))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((M, N), -1, dtype=torch.int16, device="cuda") for M, N, _ in shapes]
    torch.cuda.synchronize()
    for it in range(4):
        for s, g, d in zip(streams, gens, outs):
            with torch.cuda.stream(s):
                _dense_call(dg, g, d)
    torch.cuda.synchronize()
    for ref, d in zip(refs, outs):
        assert np.array_equal(bits(d), ref)
