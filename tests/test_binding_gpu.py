"""The high-level binding rejects mismatched tensors before any launch.

Every wrong buffer below is at least as large as the right one, so even a
check that let it through could not make a kernel read or write outside an
allocation.  After the rejected calls, the same call with correct tensors
must still run and agree with the default-allocated result."""
import numpy as np
import pytest

from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

SHAPE = (1, 2, 200, 64)


def _bf(seed, shape=SHAPE):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return upload(W.bf16_bits_to_f32(W.bf16_bits_rne(x)), "bf16")


def test_fwd_rejects_mismatched_outputs():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("binding checks: fwd")
    q, k, v = _bf(1), _bf(2), _bf(3)
    B, H, N, d = SHAPE
    bad = [
        (dict(out=torch.empty(SHAPE, dtype=torch.float32, device="cuda")), TypeError),
        (dict(out=torch.empty((B, H, N + 1, d), dtype=torch.bfloat16, device="cuda")), ValueError),
        (dict(lse=torch.empty((B, H, N), dtype=torch.float64, device="cuda")), TypeError),
        (dict(lse=torch.empty((B, H, N + 3), dtype=torch.float32, device="cuda")), ValueError),
    ]
    for kw, err in bad:
        with pytest.raises(err):
            fa.fwd(q, k, v, **kw)
    with pytest.raises(ValueError):
        fa.fwd(q, k.transpose(2, 3).contiguous().transpose(2, 3), v)
    with pytest.raises(TypeError):
        fa.fwd(q, k.float(), v)
    o1, l1 = fa.fwd(q, k, v)
    o2 = torch.empty_like(q)
    l2 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_gqa_bwd_reject_mismatched_tensors():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("binding checks: fwd_splitkv, fwd_gqa, bwd")
    q, k, v, g = _bf(11), _bf(12), _bf(13), _bf(14)
    B, H, N, d = SHAPE
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, num_splits=2,
                       out=torch.empty((B, H, N + 1, d), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):
        fa.fwd_splitkv(q, k, v, num_splits=2, lse=torch.empty((B, H, N), dtype=torch.float64, device="cuda"))
    k1, v1 = _bf(15, (B, 1, N, d)), _bf(16, (B, 1, N, d))
    with pytest.raises(ValueError):
        fa.fwd_gqa(q, k1, v1, lse=torch.empty((B, H, N + 5), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_gqa(q, k1, _bf(17, (B, 1, N + 1, d)))
    o, lse = fa.fwd(q, k, v)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, torch.empty((B, H, N + 1), dtype=torch.float32, device="cuda"), g)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o.transpose(2, 3).contiguous().transpose(2, 3), lse, g)
    o2, l2 = fa.fwd_splitkv(q, k, v, num_splits=2)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(o2.float()).all()


def test_fwd_fp8_rejects_mismatched_quantized_buffers():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    note("binding checks: fwd_fp8")
    B, H, N, d = 1, 2, 256, 128
    q, k, v = _bf(21, (B, H, N, d)), _bf(22, (B, H, N, d)), _bf(23, (B, H, N, d))
    q8, qs = fa.quantize_qk_fp8(q)
    k8, ks = fa.quantize_qk_fp8(k)
    v8t, vs = fa.quantize_v_fp8(v)
    big_k8 = torch.zeros((B, H, N + 64, d), dtype=torch.uint8, device="cuda")
    big_ks = torch.zeros((B, H, N + 64, d // 32), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_fp8(q8, qs, big_k8, ks, v8t, vs)
    with pytest.raises(ValueError):
        fa.fwd_fp8(q8, qs, k8, big_ks, v8t, vs)
    with pytest.raises(TypeError):
        fa.fwd_fp8(q8, qs, k8, ks, v8t.view(torch.int16), vs)
    with pytest.raises(TypeError):
        fa.fwd_fp8(q8.view(torch.int8), qs, k8, ks, v8t, vs)
    o, lse = fa.fwd_fp8(q8, qs, k8, ks, v8t, vs)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
