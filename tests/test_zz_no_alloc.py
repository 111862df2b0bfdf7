"""The allocation-free key-split entry point (fa_fwd_splitkv_noalloc)
against the workspace one (fa_fwd_splitkv) through the C interface: two
calls in a row on one GPU, the second smaller than the first, each bit for
bit equal to fa_fwd_splitkv with the same split count, and within the bf16
tolerances of the fp64 oracle.  The static scratch keeps the first call's
partials when the second starts, so the second call's agreement shows that
nothing of them is read."""
import numpy as np
import pytest

import oracle

from gpu_util import assert_close, note, torch_or_skip

pytestmark = pytest.mark.gpu


def _inputs(torch, B, H, Nq, Nk, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, H, Nq, d), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, Nk, d), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, Nk, d), device="cuda", generator=g).to(torch.bfloat16)
    return q, k, v


def _run_both(torch, fa, B, H, Nq, Nk, d, causal, splits, seed):
    q, k, v = _inputs(torch, B, H, Nq, Nk, d, seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    stream = torch.cuda.current_stream().cuda_stream
    o1 = torch.empty_like(q)
    l1 = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, Nq, d, splits), dtype=torch.uint8, device="cuda")
    st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(), B, H, Nq,
                           Nk, d, scale, causal, splits, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, fa.fa_strerror(st)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), B,
                                   H, Nq, Nk, d, scale, causal, splits, stream)
    assert st == 0, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return q, k, v, scale, (o1, l1), (o2, l2)


@pytest.mark.parametrize("first,second", [
    # (B, H, Nq, Nk, d, causal, splits): a decoding step over many chunks,
    # then a smaller multi-row call with fewer chunks and a ragged key tail
    ((1, 32, 1, 70000, 128, 1, 64), (2, 4, 100, 3000, 64, 0, 5)),
])
def test_noalloc_matches_workspace_call(first, second):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    for i, (B, H, Nq, Nk, d, causal, splits) in enumerate((first, second)):
        case = "noalloc call %d: B=%d H=%d Nq=%d Nk=%d d=%d causal=%d splits=%d" % (
            i + 1, B, H, Nq, Nk, d, causal, splits)
        note(case)
        assert fa.fa_fwd_splitkv_workspace_size(B, H, Nq, d, splits) <= fa.fa_fwd_splitkv_noalloc_max_bytes()
        q, k, v, scale, (o1, l1), (o2, l2) = _run_both(torch, fa, B, H, Nq, Nk, d, causal, splits, 900 + i)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), case + ": O differs"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), case + ": LSE differs"
        O_ref, L_ref = oracle.attention_c(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                          v.float().cpu().numpy(), scale, bool(causal))
        assert_close(o2.float().cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64),
                     O_ref, L_ref, "bf16", case)


def test_noalloc_rejects_oversized_call_before_launch():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, Nq, Nk, d, splits = 1, 16, 1024, 4096, 128, 4
    q, k, v = _inputs(torch, B, H, Nq, Nk, d, 5)
    o = torch.full_like(q, 3.0)
    lse = torch.zeros((B, H, Nq), dtype=torch.float32, device="cuda")
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                                   Nq, Nk, d, 0.088, 0, splits, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o.float() == 3.0).all())
