"""Seeded random shapes through every bf16 entry point against the oracle.

The parity tests elsewhere pick their shapes by hand (tile edges, ragged
tails, packed heads, more chunks than tiles).  Here a fixed seed draws 96
further problems over the whole argument space: d in {64, 128}; causal or
not; 1, 2 or 4 K/V heads shared by 1 to 8 query heads each; 1 to 700 keys
and queries (queries at most the keys when causal, as the entry points
require); 1 to 8 key chunks; one or two batches; inputs scaled so that some
rows' scores are far from 1.  Each problem runs through fa_fwd_gqa, the
square multi-head ones also through fa_fwd, fa_fwd_splitkv and (the
even-numbered ones) fa_bwd, the even-numbered square grouped ones through
fa_bwd_gqa, and every output is compared element by element with the fp64
oracle at the bf16 tolerances."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, torch_or_skip, upload

pytestmark = pytest.mark.gpu


def _problems(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        hkv = int(rng.choice([1, 2, 4]))
        mha = rng.random() < 0.35          # one query head per K/V head, Nq = Nk
        g = 1 if mha else int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.choice([1, 2]))
        nk = int(rng.integers(1, 701))
        square = mha or rng.random() < 0.3
        nq = nk if square else (int(rng.integers(1, nk + 1)) if causal else int(rng.integers(1, 701)))
        splits = int(rng.choice([1, 1, 2, 3, 5, 8]))
        amp = float(rng.choice([1.0, 1.0, 4.0]))
        out.append((i, B, hkv * g, hkv, nq, nk, d, causal, splits, amp))
    return out


def _bf(shape, rng, amp):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(amp)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _np(o, lse):
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("i,B,H,Hkv,Nq,Nk,d,causal,splits,amp", _problems())
def test_random_shape(i, B, H, Hkv, Nq, Nk, d, causal, splits, amp):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    case = "random #%d: B=%d H=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d splits=%d amp=%g" % (
        i, B, H, Hkv, Nq, Nk, d, causal, splits, amp)
    note(case)
    rng = np.random.default_rng(9000 + i)
    q = _bf((B, H, Nq, d), rng, amp)
    k = _bf((B, Hkv, Nk, d), rng, amp)
    v = _bf((B, Hkv, Nk, d), rng, 1.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    o, lse = fa.fwd_gqa(qd, kd, vd, scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    assert_close(*_np(o, lse), O_ref, L_ref, "bf16", "fa_fwd_gqa " + case)
    if Nq != Nk:
        return
    if Hkv != H:
        if i % 2 == 0:
            _check_bwd(fa, torch, fa.bwd_gqa, q, k, v, qd, kd, vd, o, lse, rng, scale, causal, case)
        return
    o, lse = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert_close(*_np(o, lse), O_ref, L_ref, "bf16", "fa_fwd " + case)
    o2, lse2 = fa.fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    assert_close(*_np(o2, lse2), O_ref, L_ref, "bf16", "fa_fwd_splitkv " + case)
    if i % 2 == 0:
        _check_bwd(fa, torch, fa.bwd, q, k, v, qd, kd, vd, o, lse, rng, scale, causal, case)


def _check_bwd(fa, torch, fn, q, k, v, qd, kd, vd, o, lse, rng, scale, causal, case):
    """Gradients through fn against the oracle's: the square backward on K/V
    repeated once per query head of a group, dK and dV summed per group."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    g = _bf((B, H, N, d), rng, 1.0)
    dq, dk, dv = fn(qd, kd, vd, o, lse, upload(g, "bf16"), scale=scale, causal=causal)
    torch.cuda.synchronize()
    dQ, dKr, dVr = oracle.attention_bwd_c(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), g, scale,
                                          causal)
    ref = (dQ, dKr.reshape(B, Hkv, G, N, d).sum(axis=2), dVr.reshape(B, Hkv, G, N, d).sum(axis=2))
    for name, t, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = t.float().cpu().numpy().astype(np.float64)
        err, mx = float(np.abs(got - r).max()), float(np.abs(r).max())
        note("%s %s %s: max|err|=%.3e max|ref|=%.3e" % (fn.__name__, name, case, err, mx))
        assert err <= 2e-2 * mx, "%s %s %s" % (fn.__name__, name, case)
