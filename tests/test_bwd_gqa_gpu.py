"""Backward pass with grouped K/V heads (fa_bwd_gqa) against the oracle.

A K/V head shared by G query heads enters the forward once per query head,
so its gradient is the sum of the gradients the G copies would get.  The
oracle side is written that way: the oracle's square backward on K/V with
every head repeated G times, then dK and dV summed over each group; dQ is
the repeated problem's dQ unchanged.  On the GPU, dQ must also equal bit for
bit fa_bwd run on the repeated K/V (the dQ kernel reads the shared head in
place of its copy), and Hkv == H must give exactly fa_bwd's results."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import note, torch_or_skip, upload

pytestmark = pytest.mark.gpu


def _bf(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _close(name, got, ref, case):
    err, mx = float(np.abs(got - ref).max()), float(np.abs(ref).max())
    note("fa_bwd_gqa %s %s: max|err|=%.3e max|ref|=%.3e" % (name, case, err, mx))
    assert err <= 2e-2 * mx, "fa_bwd_gqa %s %s: %.3e > %.3e" % (name, case, err, 2e-2 * mx)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (1, 8, 2, 300, 128, True),
    (2, 4, 1, 200, 64, False),
    (1, 6, 3, 513, 64, True),
    (1, 16, 2, 129, 128, False),
    # more than 128 query tiles of 128 rows: the two separate kernels (the
    # cases above run as one fused launch)
    (1, 144, 8, 130, 64, True),
    (2, 72, 24, 200, 128, False),
])
def test_bwd_gqa_matches_oracle(B, H, Hkv, N, d, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    G = H // Hkv
    case = "B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (B, H, Hkv, N, d, causal)
    note("fa_bwd_gqa " + case)
    seed = 100 * H + 10 * Hkv + N + d
    q, k, v, g = _bf((B, H, N, d), seed), _bf((B, Hkv, N, d), seed + 1), _bf((B, Hkv, N, d), seed + 2), \
        _bf((B, H, N, d), seed + 3)
    scale = float(np.float32(1 / math.sqrt(d)))
    qd, kd, vd, gd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), upload(g, "bf16")
    o, lse = fa.fwd_gqa(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd_gqa(qd, kd, vd, o, lse, gd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dQ, dKr, dVr = oracle.attention_bwd_c(q, kr, vr, g, scale, causal)
    dK = dKr.reshape(B, Hkv, G, N, d).sum(axis=2)
    dV = dVr.reshape(B, Hkv, G, N, d).sum(axis=2)
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    _close("dQ", f64(dq), dQ, case)
    _close("dK", f64(dk), dK, case)
    _close("dV", f64(dv), dV, case)
    # dQ reads the shared head exactly as the repeated problem reads its copy
    kdr = kd.repeat_interleave(G, dim=1).contiguous()
    vdr = vd.repeat_interleave(G, dim=1).contiguous()
    dq2, _, _ = fa.bwd(qd, kdr, vdr, o, lse, gd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2), "dQ differs from the repeated-head backward"


def test_bwd_gqa_with_one_query_head_per_kv_head_is_fa_bwd():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, N, d = 2, 4, 333, 128
    note("fa_bwd_gqa Hkv == H against fa_bwd B=%d H=%d N=%d d=%d causal" % (B, H, N, d))
    q, k, v, g = (upload(_bf((B, H, N, d), 40 + t), "bf16") for t in range(4))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, g, causal=True)
    b = fa.bwd_gqa(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
