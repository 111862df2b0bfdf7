"""The library on the caller's stream and inside a captured HIP graph.

Every entry point queues its kernels on the stream it is handed and allocates
nothing, so a caller can run it on a side stream or capture a whole step
(forward, key-split forward, backward) into a graph and replay it.  Each
replay below gets new inputs copied into the captured buffers, runs between
eager work and synchronisations, and must give exactly the bits of the eager
calls on the same inputs."""
import numpy as np
import pytest

from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

SHAPE = (2, 4, 700, 128)          # B, H, N, d: several tiles and a ragged tail


def _bf(seed):
    x = np.random.default_rng(seed).standard_normal(SHAPE, dtype=np.float32)
    return upload(W.bf16_bits_to_f32(W.bf16_bits_rne(x)), "bf16")


def _eager(fa, torch, q, k, v, g, ws_split, ws_bwd):
    o, lse = fa.fwd(q, k, v, causal=True)
    o2, lse2 = fa.fwd_splitkv(q, k, v, causal=True, num_splits=3, workspace=ws_split)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=True, workspace=ws_bwd)
    return [o, lse, o2, lse2, dq, dk, dv]


def _same_bits(torch, a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_side_stream_matches_default_stream():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("side stream: fa_fwd B=%d H=%d N=%d d=%d causal" % SHAPE)
    q, k, v = _bf(1), _bf(2), _bf(3)
    o0, l0 = fa.fwd(q, k, v, causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = fa.fwd(q, k, v, causal=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert _same_bits(torch, o0, o1) and _same_bits(torch, l0, l1)


def test_graph_replays_match_eager():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, N, d = SHAPE
    note("graph capture: fa_fwd, fa_fwd_splitkv (3 chunks), fa_bwd; B=%d H=%d N=%d d=%d causal" % SHAPE)
    q, k, v, g = _bf(11), _bf(12), _bf(13), _bf(14)
    ws_split = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, d, 3), dtype=torch.uint8, device="cuda")
    ws_bwd = torch.empty(max(1, fa.fa_bwd_workspace_size(B, H, N, d)), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(q)
    lse2 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    # warm up on a side stream, as capture wants
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _eager(fa, torch, q, k, v, g, ws_split, ws_bwd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.fwd_splitkv(q, k, v, causal=True, num_splits=3, workspace=ws_split, out=o2, lse=lse2)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=True, workspace=ws_bwd)
    captured = [o, lse, o2, lse2, dq, dk, dv]

    names = ("O", "LSE", "split O", "split LSE", "dQ", "dK", "dV")
    for rep in range(4):
        for t, seed in zip((q, k, v, g), (100 * rep + 21, 100 * rep + 22, 100 * rep + 23, 100 * rep + 24)):
            t.copy_(_bf(seed))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in captured]
        # eager work between replays, then the eager reference
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()
        want = _eager(fa, torch, q, k, v, g, ws_split, ws_bwd)
        torch.cuda.synchronize()
        same = [_same_bits(torch, a, b) for a, b in zip(got, want)]
        note("replay %d: bitwise equal to eager: %s" % (rep, dict(zip(names, same))))
        assert all(same), "replay %d differs from the eager calls" % rep
