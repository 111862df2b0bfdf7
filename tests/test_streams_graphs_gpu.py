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


def test_graph_replays_match_eager_grouped_and_fp8():
    """The same for a grouped-K/V-head step: fa_fwd_gqa with 4 key chunks,
    fa_bwd_gqa (its per-head fp32 shares and group sum live in the
    workspace), and the fp8 quantizers followed by fa_fwd_fp8_gqa."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, Hkv, N, d = 1, 8, 2, 500, 128
    note("graph capture: fa_fwd_gqa (4 chunks), fa_bwd_gqa, fp8 quantizers + fa_fwd_fp8_gqa; "
         "B=%d H=%d Hkv=%d N=%d d=%d causal" % (B, H, Hkv, N, d))

    def bf(seed, heads):
        x = np.random.default_rng(seed).standard_normal((B, heads, N, d), dtype=np.float32)
        return upload(W.bf16_bits_to_f32(W.bf16_bits_rne(x)), "bf16")

    q, k, v, g = bf(51, H), bf(52, Hkv), bf(53, Hkv), bf(54, H)
    ws_f = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, d, 4), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(fa.fa_bwd_gqa_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        fa.fwd_gqa(q, k, v, causal=True, num_splits=4, workspace=ws_f, out=o, lse=lse)
        grads = fa.bwd_gqa(q, k, v, o, lse, g, causal=True, workspace=ws_b)
        q8, qs = fa.quantize_qk_fp8(q)
        k8, ks = fa.quantize_qk_fp8(k)
        v8t, vs = fa.quantize_v_fp8(v)
        o8, l8 = fa.fwd_fp8(q8, qs, k8, ks, v8t, vs, causal=True)
        return [o, lse] + list(grads) + [o8, l8]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep in range(3):
        for t, seed, heads in zip((q, k, v, g), (100 * rep + 61, 100 * rep + 62, 100 * rep + 63, 100 * rep + 64),
                                  (H, Hkv, Hkv, H)):
            t.copy_(bf(seed, heads))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in captured]
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()
        want = step()
        torch.cuda.synchronize()
        same = [_same_bits(torch, a, b) for a, b in zip(got, want)]
        note("replay %d: bitwise equal to eager: %s" % (rep, same))
        assert all(same), "replay %d differs from the eager calls" % rep


def test_concurrent_host_threads():
    """The library keeps no state between calls: two host threads, each on
    its own stream, call fa_fwd, fa_fwd_gqa (key split) and fa_bwd at the same
    time, and every result equals the one computed alone."""
    torch = torch_or_skip()
    import threading
    import io_aware_softmax_fwd_amd as fa
    note("concurrent host threads: fa_fwd, fa_fwd_gqa (3 chunks), fa_bwd on two streams")
    probs = []
    for t in range(2):
        q, k, v, g = _bf(300 + 4 * t), _bf(301 + 4 * t), _bf(302 + 4 * t), _bf(303 + 4 * t)
        probs.append((q, k, v, g))

    def run(q, k, v, g, stream=None):
        o, lse = fa.fwd(q, k, v, causal=True, stream=stream)
        o2, lse2 = fa.fwd_gqa(q, k[:, :2].contiguous(), v[:, :2].contiguous(), causal=True, num_splits=3,
                              stream=stream)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=True, stream=stream)
        return [o, lse, o2, lse2, dq, dk, dv]

    alone = [run(*p) for p in probs]
    torch.cuda.synchronize()
    results = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    results[i] = run(*probs[i], stream=s.cuda_stream)
            s.synchronize()
        except Exception as e:   # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert all(_same_bits(torch, a, b) for a, b in zip(results[i], alone[i])), "thread %d differs" % i
