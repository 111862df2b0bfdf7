"""Helpers for the GPU tests: upload the seeded inputs, run the library
through its C entry points, and compare with the oracle at the stated
tolerances."""
import sys

import numpy as np
import pytest

import io_aware_softmax_fwd_amd as fa

# Tolerances (max over the compared elements; max|O| is the oracle's):
#   fp32 inputs: |dO| <= 1e-5 max|O|, |dLSE| <= 1e-5 max|LSE|
#   bf16 inputs: |dO| <= 2e-2 max|O|, |dLSE| <= 1e-2 (absolute)
TOL = {"f32": (1e-5, 1e-5, "rel"), "bf16": (2e-2, 1e-2, "abs")}


def torch_or_skip():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(x, dtype):
    """numpy float32 values (already representable in `dtype`) -> device tensor."""
    import torch
    if dtype == "bf16":
        from io_aware_softmax_fwd_amd import workloads as W
        bits = W.bf16_bits_rne(x)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def run(q, k, v, scale, causal, dtype):
    """Run fa_fwd / fa_fwd_f32 on host arrays; returns float64 (O, LSE)."""
    import torch
    qd, kd, vd = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    o, lse = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def errors(O, L, O_ref, L_ref):
    return (float(np.abs(O - O_ref).max()), float(np.abs(O_ref).max()),
            float(np.abs(L - L_ref).max()), float(np.abs(L_ref).max()))


def assert_close(O, L, O_ref, L_ref, dtype, what=""):
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), what + ": non-finite output"
    eo, mo, el, ml = errors(O, L, O_ref, L_ref)
    to, tl, kind = TOL[dtype]
    lse_bound = tl * ml if kind == "rel" else tl
    note("%s: max|dO|=%.3e (bound %.3e)  max|dLSE|=%.3e (bound %.3e)"
         % (what, eo, to * mo, el, lse_bound))
    assert eo <= to * mo, "%s: O error %.3e > %.3e" % (what, eo, to * mo)
    assert el <= lse_bound, "%s: LSE error %.3e > %.3e" % (what, el, lse_bound)
