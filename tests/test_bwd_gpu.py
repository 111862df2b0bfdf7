"""Parity of the attention backward (fa_bwd) with the fp64 oracle.

Every case runs the forward pass on the GPU (fa_fwd) for O and LSE, then
fa_bwd, and compares dQ, dK and dV with the oracle's gradients of the same
bf16 inputs.  Bound, per gradient: max |dX - dX_ref| <= 2e-2 * max |dX_ref|
(the bf16 bound of the forward's O: inputs, probabilities and dS are rounded
to bf16 for the products, accumulation is fp32).
"""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2


def _bf(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _run(q, k, v, g, scale, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    qd, kd, vd, gd = (upload(x, "bf16") for x in (q, k, v, g))
    o, lse = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, gd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def _check(got, ref, what, inputs=None, scale=None):
    """BWD_TOL relative to each gradient's largest reference element.  A
    gradient that is exactly zero (dQ when every row sees one key: P = 1, so
    dS = dP - D = 0) has no scale of its own; there the kernel's dP (matrix
    core) and D (dot products) are two differently ordered fp32 sums of the
    same d products, and their difference times scale * K is allowed up to
    d * 2^-16 * scale * max|dO| * max|V| * max|K| (inputs = (q, k, v, dO))."""
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(a)), "%s %s: non-finite" % (what, name)
        err, mx = float(np.abs(a - b).max()), float(np.abs(b).max())
        bound = BWD_TOL * mx
        if mx == 0.0 and inputs is not None:
            q, k, v, g = inputs
            bound = q.shape[-1] * 2.0 ** -16 * scale * np.abs(g).max() * np.abs(v).max() * np.abs(k).max()
        note("%s %s: max|err|=%.3e  max|ref|=%.3e  bound=%.3e" % (what, name, err, mx, bound))
        assert err <= bound, "%s %s: %.3e > %.3e" % (what, name, err, bound)


CASES = [
    # (B, H, N, d, causal)
    (1, 2, 64, 64, False),
    (1, 2, 64, 64, True),
    (2, 3, 200, 64, True),
    (1, 2, 257, 128, True),
    (1, 1, 1, 128, True),
    (1, 1, 1, 64, False),
    (1, 2, 130, 128, False),
    (2, 2, 333, 64, False),
    (1, 1, 500, 128, True),
    (1, 1, 1000, 128, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", CASES)
def test_bwd_matches_oracle(B, H, N, d, causal):
    case = "bwd B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal)
    note(case)
    seed = 5 * N + d + 7 * H + causal
    q, k, v, g = (_bf((B, H, N, d), seed + t) for t in range(4))
    scale = float(np.float32(1 / math.sqrt(d)))
    got = _run(q, k, v, g, scale, causal)
    ref = oracle.attention_bwd_c(q, k, v, g, scale, causal)
    _check(got, ref, case, (q, k, v, g), scale)


# The cases above have at most 128 workgroups per kernel, so the backward
# runs as one fused launch (bwd_fused_kernel); with many heads the same
# shapes go through the two separate kernels.
WIDE_CASES = [
    # (B, H, N, d, causal): more than 128 query tiles of 128 rows in all
    (1, 130, 1, 128, True),
    (1, 64, 257, 128, True),
    (2, 40, 200, 64, True),
    (1, 72, 130, 64, False),
    (1, 130, 64, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", WIDE_CASES)
def test_bwd_two_kernel_path_matches_oracle(B, H, N, d, causal):
    case = "bwd two-kernel B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal)
    note(case)
    seed = 11 * N + d + 3 * H + causal
    q, k, v, g = (_bf((B, H, N, d), seed + t) for t in range(4))
    scale = float(np.float32(1 / math.sqrt(d)))
    got = _run(q, k, v, g, scale, causal)
    ref = oracle.attention_bwd_c(q, k, v, g, scale, causal)
    _check(got, ref, case, (q, k, v, g), scale)


@pytest.mark.parametrize("N,d,causal", [(200, 64, True), (333, 128, False)])
def test_bwd_fused_and_two_kernel_paths_agree(N, d, causal):
    """Heads are independent: the first heads of a many-head call (two
    kernels) must equal, bit for bit, the same heads run alone (one fused
    launch)."""
    torch = torch_or_skip()
    note("bwd fused vs two-kernel N=%d d=%d causal=%d" % (N, d, causal))
    H = 136
    q, k, v, g = (_bf((1, H, N, d), 60 + N + t) for t in range(4))
    wide = _run(q, k, v, g, 0.125, causal)
    few = _run(q[:, :2].copy(), k[:, :2].copy(), v[:, :2].copy(), g[:, :2].copy(), 0.125, causal)
    for a, b in zip(wide, few):
        assert np.array_equal(a[:, :2], b)


def test_bwd_deterministic():
    """No atomics: two launches give identical bits."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    q, k, v, g = (upload(_bf((2, 4, 300, 128), 90 + t), "bf16") for t in range(4))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, g, causal=True)
    b = fa.bwd(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cfg,heads", [(2, None), (3, [0, 63]), (4, [0, 5, 31]), (5, [0, 2, 15])])
def test_bwd_workload_shapes(cfg, heads):
    """The forward workloads' shapes and input recipes (dO drawn N(0,1) with
    seed 1000*cfg + 6); the larger ones are checked on the listed heads
    (C3 on every head in test_zy_full_rows_gpu.py)."""
    torch_or_skip()
    w = W.WORKLOADS[cfg]
    note("bwd workload C%d: %s heads=%s" % (cfg, w.describe(), heads))
    x = W.make_inputs(w)
    g = _bf((w.B, w.H, w.N, w.d), 1000 * cfg + 6)
    got = _run(x["q"], x["k"], x["v"], g, w.scale, w.causal)
    ref = oracle.attention_bwd_c(x["q"], x["k"], x["v"], g, w.scale, w.causal, heads=heads)
    if heads is not None:
        got = [a.reshape(w.B * w.H, w.N, w.d)[heads] for a in got]
    _check(got, ref, "C%d" % cfg)
