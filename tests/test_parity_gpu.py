"""Parity of the HIP path with the fp64 oracle, through the C entry points."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, run, torch_or_skip, upload

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale)


def _as(x, dtype):
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x)) if dtype == "bf16" else x.astype(np.float32)


# ---------------------------------------------------------------- small, full
SMALL = [
    # (B, H, N, d, causal) -- several tiles plus ragged tails
    (1, 1, 1, 64, False), (1, 1, 1, 128, True), (1, 2, 63, 64, True),
    (1, 2, 65, 128, False), (2, 3, 300, 64, False), (2, 3, 300, 64, True),
    (1, 2, 513, 128, True), (1, 2, 513, 128, False), (1, 1, 1000, 64, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,d,causal", SMALL)
def test_small_shapes_full(dtype, B, H, N, d, causal):
    torch_or_skip()
    case = "small %s B=%d H=%d N=%d d=%d causal=%d" % (dtype, B, H, N, d, causal)
    note(case)
    seed = 100 * N + d + causal
    q = _as(_rand((B, H, N, d), seed + 1), dtype)
    k = _as(_rand((B, H, N, d), seed + 2), dtype)
    v = _as(_rand((B, H, N, d), seed + 3), dtype)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run(q, k, v, scale, causal, dtype)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(O, L, O_ref, L_ref, dtype, case)


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_parity(cfg):
    torch = torch_or_skip()
    w = W.WORKLOADS[cfg]
    note("workload C%d: %s" % (cfg, w.describe()))
    x = W.make_inputs(w)
    O, L = run(x["q"], x["k"], x["v"], w.scale, w.causal, w.dtype)
    if w.B * w.H * w.N <= 16384:
        O_ref, L_ref = oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal)
        assert_close(O, L, O_ref, L_ref, w.dtype, "C%d all rows" % cfg)
    else:
        rows = W.sample_rows(w, 384, seed=cfg)
        O_ref, L_ref = oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal, rows=rows)
        Of = O.reshape(-1, w.d)[rows]
        Lf = L.reshape(-1)[rows]
        assert_close(Of, Lf, O_ref, L_ref, w.dtype, "C%d %d sampled rows" % (cfg, len(rows)))
    del torch


# ------------------------------------------------------ the worked example
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_example(dtype):
    """notes section 8: scores (1.414, 0.707, 0.707), v = (1, 0, 1)."""
    torch_or_skip()
    with open(os.path.join(GOLD, "hand_example.json")) as f:
        g = json.load(f)
    d = 64
    q = np.zeros((1, 1, 3, d), np.float32)
    k = np.zeros((1, 1, 3, d), np.float32)
    v = np.zeros((1, 1, 3, d), np.float32)
    q[..., 0] = 1.0
    k[0, 0, :, 0] = g["scores"]
    v[0, 0, :, 0] = g["values"]
    q, k, v = _as(q, dtype), _as(k, dtype), _as(v, dtype)
    for causal in (False, True):
        O, L = run(q, k, v, 1.0, causal, dtype)
        O_ref, L_ref = oracle.attention_c(q, k, v, 1.0, causal)
        assert_close(O, L, O_ref, L_ref, dtype, "hand example %s causal=%d" % (dtype, causal))
        pr = g["printed"]
        tol = 5e-4 if dtype == "f32" else 1e-2
        if not causal:
            assert abs(O[0, 0, 2, 0] - pr["merged_O"]) < tol
        else:
            assert O[0, 0, 0, 0] == 1.0
            assert abs(O[0, 0, 1, 0] - pr["block1_O"]) < tol


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_and_row0(causal):
    torch_or_skip()
    B, H, N, d = 1, 4, 777, 128
    q = _as(_rand((B, H, N, d), 1, 2.0), "bf16")
    k = _as(_rand((B, H, N, d), 2, 2.0), "bf16")
    cvec = _as(_rand((d,), 3), "bf16")
    v = np.broadcast_to(cvec, (B, H, N, d)).copy()
    O, L = run(q, k, v, 0.125, causal, "bf16")
    # each output row is a convex combination of identical rows
    assert np.abs(O - cvec).max() <= 2e-2 * np.abs(cvec).max()
    if causal:
        vr = _as(_rand((B, H, N, d), 4), "bf16")
        O, L = run(q, k, vr, 0.125, True, "bf16")
        assert np.array_equal(O[:, :, 0], vr[:, :, 0].astype(np.float64))
        ref = 0.125 * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
        assert np.abs(L[:, :, 0] - ref).max() < 1e-3


def test_key_permutation_and_determinism():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, N, d = 2, 2, 640, 64
    q = _as(_rand((B, H, N, d), 5), "bf16")
    k = _as(_rand((B, H, N, d), 6), "bf16")
    v = _as(_rand((B, H, N, d), 7), "bf16")
    perm = np.random.default_rng(8).permutation(N)
    O1, L1 = run(q, k, v, 0.125, False, "bf16")
    O2, L2 = run(q, k[:, :, perm].copy(), v[:, :, perm].copy(), 0.125, False, "bf16")
    assert np.abs(O1 - O2).max() <= 2e-2 * np.abs(O1).max()
    assert np.abs(L1 - L2).max() <= 1e-3
    # bitwise determinism: same inputs, repeated launches
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    outs = []
    for _ in range(3):
        o, lse = fa.fwd(qd, kd, vd, scale=0.125, causal=True)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    for o, lse in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(lse.view(np.int32), outs[0][1].view(np.int32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_writes_outside_outputs(dtype):
    """O and LSE are placed inside larger buffers filled with a sentinel; the
    kernel must leave everything outside [B,H,N,d] / [B,H,N] untouched."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, N, d = 1, 3, 333, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = upload(_as(_rand((B, H, N, d), 9), dtype), dtype)
    k = upload(_as(_rand((B, H, N, d), 10), dtype), dtype)
    v = upload(_as(_rand((B, H, N, d), 11), dtype), dtype)
    pad = 4096
    obuf = torch.full((B * H * N * d + 2 * pad,), 7.0, dtype=tdt, device="cuda")
    lbuf = torch.full((B * H * N + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    f = fa.fa_fwd if dtype == "bf16" else fa.fa_fwd_f32
    st = f(q.data_ptr(), k.data_ptr(), v.data_ptr(), obuf[pad:].data_ptr(), lbuf[pad:].data_ptr(),
           B, H, N, d, 0.088, 1, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ob, lb = obuf.float().cpu().numpy(), lbuf.cpu().numpy()
    assert np.all(ob[:pad] == 7.0) and np.all(ob[pad + B * H * N * d:] == 7.0)
    assert np.all(lb[:pad] == 7.0) and np.all(lb[pad + B * H * N:] == 7.0)
    assert np.all(np.isfinite(ob[pad:pad + B * H * N * d]))


# ------------------------------------------- d = 64 with 256-row tiles
@pytest.mark.parametrize("B,H,N,causal", [(1, 64, 2000, True), (2, 32, 1900, False)])
def test_d64_wide_tiles_full(B, H, N, causal):
    """d = 64 problems with at least 512 tiles of 256 rows run two 32-row
    blocks per wave; ragged last tiles, causal diagonals, every row against
    the oracle."""
    torch_or_skip()
    d = 64
    note("d=64 wide tiles: B=%d H=%d N=%d causal=%d" % (B, H, N, causal))
    q, k, v = (_as(_rand((B, H, N, d), 600 + N + t), "bf16") for t in range(3))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run(q, k, v, scale, causal, "bf16")
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", "d=64 wide tiles B=%d H=%d N=%d causal=%d" % (B, H, N, causal))
