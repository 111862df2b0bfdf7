"""Element offsets at and past 2^31.

Every [B, H, N, d] tensor of these problems holds 2^31 elements (B = 2,
H = 16384, N = 512, d = 128), so the rows of the second half sit at element
offsets that a 32-bit index would wrap.  The heads repeat one seeded block of
64 heads, so head h must give exactly the bits of head h mod 64, and the first
64 heads must match the oracle at the bf16 tolerances.  The entry points run
as their callers use them: fa_fwd, fa_fwd_splitkv (fp32 partials past 2^32
elements) and fa_bwd."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

H0, N, D = 64, 512, 128
B, REP = 2, 256                 # heads per batch: 64 * 256 = 16384
SCALE = float(np.float32(1 / math.sqrt(D)))


def _block(seed):
    x = np.random.default_rng(seed).standard_normal((1, H0, N, D), dtype=np.float32)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _big(x):
    t = upload(x, "bf16").repeat(B, REP, 1, 1)
    assert t.is_contiguous() and t.numel() == 1 << 31
    return t


def _same_as_first_block(t, what):
    """Every 64-head block of t (flattened over batch and heads) equals the
    first one bit for bit."""
    torch = torch_or_skip()
    blocks = t.reshape(B * REP, H0, -1)
    bits = blocks.view(torch.int16) if blocks.dtype == torch.bfloat16 else blocks.view(torch.int32)
    same = torch.equal(bits, bits[:1].expand_as(bits))
    note("%s: all %d head blocks identical: %s" % (what, B * REP, same))
    assert same, what + ": a repeated head block differs"


def _first_block(t):
    return t.reshape(B * REP, H0, N, -1)[0].float().cpu().numpy().astype(np.float64)[None]


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_and_splitkv_past_2_31(causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("offsets past 2^31: forward B=%d H=%d N=%d d=%d causal=%d" % (B, H0 * REP, N, D, causal))
    q0, k0, v0 = (_block(7100 + 10 * causal + t) for t in range(3))
    q, k, v = _big(q0), _big(k0), _big(v0)
    O_ref, L_ref = oracle.attention_c(q0, k0, v0, SCALE, causal)
    o, lse = fa.fwd(q, k, v, scale=SCALE, causal=causal)
    torch.cuda.synchronize()
    _same_as_first_block(o, "fa_fwd O")
    _same_as_first_block(lse, "fa_fwd LSE")
    assert_close(_first_block(o), _first_block(lse)[..., 0], O_ref, L_ref, "bf16", "fa_fwd first block")
    del o, lse
    splits = 2
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H0 * REP, N, D, splits), dtype=torch.uint8,
                     device="cuda")
    o, lse = fa.fwd_splitkv(q, k, v, scale=SCALE, causal=causal, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    del ws
    _same_as_first_block(o, "fa_fwd_splitkv O")
    _same_as_first_block(lse, "fa_fwd_splitkv LSE")
    assert_close(_first_block(o), _first_block(lse)[..., 0], O_ref, L_ref, "bf16", "fa_fwd_splitkv first block")
    del o, lse, q, k, v
    torch.cuda.empty_cache()


def test_bwd_past_2_31():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("offsets past 2^31: backward B=%d H=%d N=%d d=%d causal=1" % (B, H0 * REP, N, D))
    q0, k0, v0, g0 = (_block(7200 + t) for t in range(4))
    q, k, v, g = _big(q0), _big(k0), _big(v0), _big(g0)
    o, lse = fa.fwd(q, k, v, scale=SCALE, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    del o, lse, q, k, v, g
    heads = [0, 1, 63]
    ref = oracle.attention_bwd_c(q0, k0, v0, g0, SCALE, True, heads=heads)
    for name, t, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _same_as_first_block(t, "fa_bwd " + name)
        got = _first_block(t)[0, heads]        # [heads, N, d], as the oracle returns them
        want = r
        err, mx = float(np.abs(got - want).max()), float(np.abs(want).max())
        note("fa_bwd %s first block heads %s: max|err|=%.3e  max|ref|=%.3e" % (name, heads, err, mx))
        assert err <= 2e-2 * mx, "fa_bwd %s: %.3e > %.3e" % (name, err, 2e-2 * mx)
    del dq, dk, dv
    torch.cuda.empty_cache()
