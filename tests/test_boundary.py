"""The C boundary on a host without a GPU: the library loads, exports every
function include/fa_fwd.h declares, and rejects bad arguments on the host
before any HIP call (no launch happens, so fake device addresses are safe)."""
import ctypes
import os
import re
import subprocess

import pytest

import io_aware_softmax_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    fa.load()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert hasattr(fa.load(), name)


def test_status_enum_matches_header():
    text = open(HEADER).read()
    for name, val in re.findall(r"(FA_\w+)\s*=\s*(\d+)", text):
        assert getattr(fa, name) == int(val), name


A = 0x10000          # fake, 16-byte aligned "device" addresses; never touched
MB = 1 << 20


def _call(fn, **kw):
    args = dict(q=A, k=A + 8 * MB, v=A + 16 * MB, o=A + 24 * MB, lse=A + 32 * MB,
                B=1, H=2, N=64, d=64, scale=0.125, causal=0, stream=None)
    args.update(kw)
    return fn(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"],
              args["N"], args["d"], args["scale"], args["causal"], args["stream"])


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(k=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=-1), fa.FA_ERR_SHAPE), (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 10, N=1 << 10, d=128), fa.FA_ERR_SHAPE),
    (dict(N=1 << 23, d=128), fa.FA_ERR_SHAPE),
    # 2^31 heads of one row: 2^37 elements, but one workgroup per head
    (dict(B=1 << 16, H=1 << 15, N=1, d=64), fa.FA_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 15, N=7, d=64), fa.FA_ERR_SHAPE),
    # 2^24 groups of 32 rows: a launch would exceed 2^32 threads
    (dict(B=1, H=1 << 14, N=1 << 15, d=64), fa.FA_ERR_SHAPE),
    (dict(B=2, H=1 << 13, N=(1 << 15) - 31, d=64), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED_D), (dict(d=96), fa.FA_ERR_UNSUPPORTED_D),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED_D),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=-0.5), fa.FA_ERR_SCALE),
    (dict(scale=float("inf")), fa.FA_ERR_SCALE), (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(causal=2), fa.FA_ERR_CAUSAL), (dict(causal=-1), fa.FA_ERR_CAUSAL),
    (dict(q=A + 2), fa.FA_ERR_ALIGN), (dict(lse=A + 32 * MB + 4), fa.FA_ERR_ALIGN),
    (dict(o=A), fa.FA_ERR_ALIAS), (dict(lse=A + 24 * MB + 64), fa.FA_ERR_ALIAS),
    (dict(o=A + 16 * MB + 32), fa.FA_ERR_ALIAS),
])
def test_bad_arguments_rejected_on_host(fn, kw, status):
    assert _call(fn, **kw) == status


def test_strerror_covers_every_status():
    codes = [int(v) for _, v in re.findall(r"(FA_\w+)\s*=\s*(\d+)", open(HEADER).read())]
    assert sorted(codes) == list(range(len(codes)))
    seen = set()
    for s in codes:
        msg = fa.fa_strerror(s)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == len(codes)
    assert fa.fa_strerror(12345) == "unknown status"


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(fa.binding, "_lib", None)
    monkeypatch.setattr(fa.binding, "LIB_PATH", "/nonexistent/libfa_fwd.so")
    with pytest.raises(ImportError):
        fa.binding.fa_fwd(A, A, A, A, A, 1, 1, 1, 64, 1.0, 0, None)


def _split_call(**kw):
    args = dict(q=A, k=A + 8 * MB, v=A + 16 * MB, o=A + 24 * MB, lse=A + 32 * MB,
                B=1, H=2, Nq=64, Nk=128, d=64, scale=0.125, causal=0, splits=2,
                ws=A + 64 * MB, ws_bytes=1 << 24, stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                             args["H"], args["Nq"], args["Nk"], args["d"], args["scale"],
                             args["causal"], args["splits"], args["ws"], args["ws_bytes"],
                             args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(Nq=0), fa.FA_ERR_SHAPE), (dict(Nk=0), fa.FA_ERR_SHAPE),
    (dict(causal=1, Nq=129, Nk=128), fa.FA_ERR_SHAPE),
    # 256 chunks x 1024 heads x 64 query tiles = 2^24 workgroups of 256 threads
    (dict(H=1 << 10, Nq=1 << 13, Nk=1 << 13, splits=256), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED_D), (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(causal=3), fa.FA_ERR_CAUSAL),
    (dict(splits=0), fa.FA_ERR_SPLITS), (dict(splits=257), fa.FA_ERR_SPLITS),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 64 * MB + 8), fa.FA_ERR_ALIGN), (dict(v=A + 16 * MB + 4), fa.FA_ERR_ALIGN),
    (dict(ws=A + 24 * MB), fa.FA_ERR_ALIAS), (dict(o=A + 8 * MB), fa.FA_ERR_ALIAS),
])
def test_splitkv_bad_arguments_rejected_on_host(kw, status):
    assert _split_call(**kw) == status


def test_splitkv_workspace_size_and_split_choice():
    # o part: splits*rows*d*4 rounded to 256, then lse part rounded to 256
    rows = 2 * 8 * 1024
    assert fa.fa_fwd_splitkv_workspace_size(2, 8, 1024, 64, 4) == 4 * rows * 64 * 4 + 4 * rows * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 128, 3) == 1536 + 256
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 96, 3) == 0
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 64, 0) == 0
    # big grids need no split; small grids and long key runs get more
    assert fa.fa_fwd_splitkv_num_splits(1, 32, 16384, 16384, 256) == 1
    # 128 row blocks of 16 tiles: two workgroups per CU, chunks of 4 tiles
    assert fa.fa_fwd_splitkv_num_splits(2, 8, 1024, 1024, 256) == 4
    # decoding 8 heads over 512 tiles: two per CU, 64 chunks of 8 tiles
    assert fa.fa_fwd_splitkv_num_splits(1, 8, 1, 32768, 256) == 64
    # 32 heads over 2048 tiles: two per CU (16 chunks), doubled while chunks keep 16 tiles
    assert fa.fa_fwd_splitkv_num_splits(1, 32, 1, 131072, 256) == 32
    assert fa.fa_fwd_splitkv_num_splits(1, 32, 1, 32768, 256) == 32
    assert fa.fa_fwd_splitkv_num_splits(1, 32, 1, 4096, 256) == 16
    # one head over 2048 tiles: one per CU, chunks of 8 tiles
    assert fa.fa_fwd_splitkv_num_splits(1, 1, 1, 131072, 256) == 256
    # one head over 512 tiles: chunks of 4 tiles at most
    assert fa.fa_fwd_splitkv_num_splits(1, 1, 1, 32768, 256) == 128
    assert fa.fa_fwd_splitkv_num_splits(1, 1, 1, 64, 256) == 1


def _gqa_call(**kw):
    args = dict(q=A, k=A + 8 * MB, v=A + 16 * MB, o=A + 24 * MB, lse=A + 32 * MB,
                B=1, H=8, Hkv=2, Nq=16, Nk=128, d=64, scale=0.125, causal=0, splits=2,
                ws=A + 64 * MB, ws_bytes=1 << 24, stream=None)
    args.update(kw)
    return fa.fa_fwd_gqa(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                         args["H"], args["Hkv"], args["Nq"], args["Nk"], args["d"], args["scale"],
                         args["causal"], args["splits"], args["ws"], args["ws_bytes"],
                         args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(k=None), fa.FA_ERR_NULL),
    (dict(Hkv=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE),
    (dict(Hkv=3), fa.FA_ERR_HEADS), (dict(H=8, Hkv=16), fa.FA_ERR_HEADS),
    (dict(causal=1, Nq=129, Nk=128), fa.FA_ERR_SHAPE),
    # the query rows of one K/V head must stay below 2^31
    (dict(H=1 << 12, Hkv=1, Nq=1 << 19, Nk=1 << 19, splits=1), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED_D), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(causal=2), fa.FA_ERR_CAUSAL),
    (dict(splits=0), fa.FA_ERR_SPLITS), (dict(splits=300), fa.FA_ERR_SPLITS),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 64 * MB + 4), fa.FA_ERR_ALIGN), (dict(lse=A + 32 * MB + 8), fa.FA_ERR_ALIGN),
    (dict(ws=A + 8 * MB), fa.FA_ERR_ALIAS), (dict(lse=A + 16 * MB), fa.FA_ERR_ALIAS),
    # with one split the workspace is not used, so it is not checked; the
    # error that remains is the alias of o with k
    (dict(splits=1, ws=None, ws_bytes=0, o=A + 8 * MB), fa.FA_ERR_ALIAS),
])
def test_gqa_bad_arguments_rejected_on_host(kw, status):
    assert _gqa_call(**kw) == status


def test_gqa_split_choice():
    # grouped heads of a decoding step share one tile per K/V head
    assert fa.fa_fwd_gqa_num_splits(1, 32, 8, 1, 32768, 1, 256) == 64
    assert fa.fa_fwd_gqa_num_splits(1, 32, 8, 1, 131072, 1, 256) == 128
    assert fa.fa_fwd_gqa_num_splits(1, 32, 2, 1, 131072, 1, 256) == 128
    assert fa.fa_fwd_gqa_num_splits(1, 32, 1, 1, 131072, 1, 256) == 256
    assert fa.fa_fwd_gqa_num_splits(1, 32, 8, 1, 2048, 1, 256) == 8
    # Hkv == H agrees with the multi-head choice
    for args in ((2, 8, 1024, 1024), (1, 8, 1, 32768), (1, 32, 16384, 16384), (3, 5, 77, 900)):
        B, H, Nq, Nk = args
        for causal in (0, 1):
            assert (fa.fa_fwd_gqa_num_splits(B, H, H, Nq, Nk, causal, 256)
                    == fa.fa_fwd_splitkv_num_splits(B, H, Nq, Nk, 256))
    # a long causal prefill over 8 K/V heads fills the GPU without a split
    assert fa.fa_fwd_gqa_num_splits(1, 32, 8, 16384, 16384, 1, 256) == 1
    # bad arguments give 1
    assert fa.fa_fwd_gqa_num_splits(1, 6, 4, 1, 100, 0, 256) == 1
    assert fa.fa_fwd_gqa_num_splits(0, 6, 3, 1, 100, 0, 256) == 1


def _bwd_call(**kw):
    args = dict(q=A, k=A + 8 * MB, v=A + 16 * MB, o=A + 24 * MB, dout=A + 32 * MB,
                lse=A + 40 * MB, dq=A + 48 * MB, dk=A + 56 * MB, dv=A + 64 * MB,
                B=1, H=2, N=64, d=64, scale=0.125, causal=0, ws=A + 72 * MB, ws_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return fa.fa_bwd(args["q"], args["k"], args["v"], args["o"], args["dout"], args["lse"],
                     args["dq"], args["dk"], args["dv"], args["B"], args["H"], args["N"], args["d"],
                     args["scale"], args["causal"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(dout=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(dq=None), fa.FA_ERR_NULL), (dict(dv=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(N=1 << 23, d=128), fa.FA_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 15, N=1, d=64), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED_D), (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(causal=5), fa.FA_ERR_CAUSAL),
    (dict(dk=A + 56 * MB + 2), fa.FA_ERR_ALIGN), (dict(ws=A + 72 * MB + 8), fa.FA_ERR_ALIGN),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(dq=A), fa.FA_ERR_ALIAS), (dict(dk=A + 48 * MB), fa.FA_ERR_ALIAS),
    (dict(dv=A + 40 * MB), fa.FA_ERR_ALIAS), (dict(ws=A + 64 * MB), fa.FA_ERR_ALIAS),
    (dict(dq=A + 32 * MB + 64), fa.FA_ERR_ALIAS),
    (dict(H=1 << 14, N=1 << 15), fa.FA_ERR_SHAPE),
])
def test_bwd_bad_arguments_rejected_on_host(kw, status):
    assert _bwd_call(**kw) == status


def test_bwd_workspace_size():
    assert fa.fa_bwd_workspace_size(2, 8, 1024, 64) == 2 * 8 * 1024 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 3, 128) == 256
    assert fa.fa_bwd_workspace_size(1, 1, 3, 80) == 0
    assert fa.fa_bwd_workspace_size(0, 1, 3, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fa.FA_ERR_NULL), (dict(xs=None), fa.FA_ERR_NULL), (dict(rows=0), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED_D), (dict(x8=A + 8 * MB + 4), fa.FA_ERR_ALIGN),
    (dict(rows=1 << 30, d=128), fa.FA_ERR_SHAPE), (dict(rows=1 << 31, d=64), fa.FA_ERR_SHAPE),
    (dict(x8=A + 64), fa.FA_ERR_ALIAS), (dict(xs=A + 8 * MB + 128), fa.FA_ERR_ALIAS),
])
def test_quantize_qk_fp8_bad_arguments(kw, status):
    a = dict(x=A, rows=64, d=64, x8=A + 8 * MB, xs=A + 16 * MB, stream=None)
    a.update(kw)
    assert fa.fa_quantize_qk_fp8(a["x"], a["rows"], a["d"], a["x8"], a["xs"], a["stream"]) == status


@pytest.mark.parametrize("kw,status", [
    (dict(v=None), fa.FA_ERR_NULL), (dict(vs=None), fa.FA_ERR_NULL), (dict(BH=0), fa.FA_ERR_SHAPE),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED_D),
    (dict(vs=A + 16 * MB + 2), fa.FA_ERR_ALIGN), (dict(v8t=A + 32), fa.FA_ERR_ALIAS),
    # 2^14 heads x 2^10 tiles x 256 threads = 2^32 threads
    (dict(BH=1 << 14, N=1 << 16), fa.FA_ERR_SHAPE),
])
def test_quantize_v_fp8_bad_arguments(kw, status):
    a = dict(v=A, BH=2, N=100, d=128, v8t=A + 8 * MB, vs=A + 16 * MB, stream=None)
    a.update(kw)
    assert fa.fa_quantize_v_fp8(a["v"], a["BH"], a["N"], a["d"], a["v8t"], a["vs"], a["stream"]) == status


def test_fp8_v_sizes():
    assert fa.fa_fp8_v_bytes(2, 100, 128) == 2 * 2 * 128 * 64
    assert fa.fa_fp8_v_scale_bytes(2, 100, 128) == 2 * 2 * 2 * 128
    assert fa.fa_fp8_v_bytes(1, 64, 64) == 64 * 64 and fa.fa_fp8_v_bytes(1, 64, 80) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q8=None), fa.FA_ERR_NULL), (dict(vs=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(d=256), fa.FA_ERR_UNSUPPORTED_D),
    (dict(B=1 << 16, H=1 << 15, N=1), fa.FA_ERR_SHAPE),
    (dict(scale=-1.0), fa.FA_ERR_SCALE), (dict(causal=3), fa.FA_ERR_CAUSAL),
    (dict(ks=A + 24 * MB + 1), fa.FA_ERR_ALIGN), (dict(o=A + 8 * MB), fa.FA_ERR_ALIAS),
    (dict(lse=A + 40 * MB + 16), fa.FA_ERR_ALIAS), (dict(lse=A + 48 * MB), fa.FA_ERR_ALIAS),
])
def test_fwd_fp8_bad_arguments(kw, status):
    a = dict(q8=A, qs=A + 8 * MB, k8=A + 16 * MB, ks=A + 24 * MB, v8t=A + 32 * MB, vs=A + 40 * MB,
             o=A + 48 * MB, lse=A + 56 * MB, B=1, H=2, N=64, d=64, scale=0.125, causal=0, stream=None)
    a.update(kw)
    assert fa.fa_fwd_fp8(a["q8"], a["qs"], a["k8"], a["ks"], a["v8t"], a["vs"], a["o"], a["lse"], a["B"],
                         a["H"], a["N"], a["d"], a["scale"], a["causal"], a["stream"]) == status


def test_binding_tensor_checks_on_host():
    """The binding's tensor check (used by every high-level function before a
    launch) on CPU tensors: type, device, contiguity, dtype, shape, size."""
    import torch
    from io_aware_softmax_fwd_amd.binding import _check
    cpu = torch.device("cpu")
    t = torch.zeros((2, 3, 4, 64), dtype=torch.bfloat16)
    _check("t", t, cpu, torch.bfloat16, (2, 3, 4, 64), min_bytes=t.numel() * 2)
    with pytest.raises(TypeError):
        _check("t", [1, 2], cpu)
    with pytest.raises(ValueError, match="live on"):
        _check("t", t, torch.device("cuda", 0))
    with pytest.raises(ValueError, match="contiguous"):
        _check("t", t.transpose(2, 3), cpu)
    with pytest.raises(TypeError, match="bfloat16"):
        _check("t", t.float(), cpu, torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        _check("t", t, cpu, torch.bfloat16, (2, 3, 5, 64))
    with pytest.raises(ValueError, match="bytes"):
        _check("t", t, cpu, min_bytes=t.numel() * 2 + 1)


def _bwd_gqa_call(**kw):
    a = dict(q=A, k=A + 8 * MB, v=A + 12 * MB, o=A + 16 * MB, dout=A + 24 * MB, lse=A + 32 * MB,
             dq=A + 40 * MB, dk=A + 48 * MB, dv=A + 52 * MB, B=1, H=4, Hkv=2, N=512, d=128,
             scale=0.125, causal=1, ws=A + 64 * MB, ws_bytes=16 * MB, stream=None)
    a.update(kw)
    return fa.fa_bwd_gqa(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                         a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["ws"],
                         a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), fa.FA_ERR_HEADS), (dict(Hkv=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE),
    (dict(k=None), fa.FA_ERR_NULL), (dict(dv=None), fa.FA_ERR_NULL),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED_D),
    (dict(ws_bytes=1024), fa.FA_ERR_WORKSPACE),
    # k, v, dk, dv are [B, Hkv, N, d]: 256 KB each here
    (dict(dk=A + 8 * MB + 128 * 1024), fa.FA_ERR_ALIAS), (dict(dv=A + 48 * MB + 4096), fa.FA_ERR_ALIAS),
    (dict(ws=A + 40 * MB + 64), fa.FA_ERR_ALIAS),
])
def test_bwd_gqa_bad_arguments_rejected_on_host(kw, status):
    assert _bwd_gqa_call(**kw) == status


def test_bwd_gqa_workspace_size():
    d_part = (1 * 4 * 512 * 4 + 255) // 256 * 256
    assert fa.fa_bwd_gqa_workspace_size(1, 4, 4, 512, 128) == fa.fa_bwd_workspace_size(1, 4, 512, 128) == d_part
    # per-query-head fp32 partial dK and dV for a shared K/V head
    assert fa.fa_bwd_gqa_workspace_size(1, 4, 2, 512, 128) == d_part + 2 * 4 * 512 * 128 * 4
    assert fa.fa_bwd_gqa_workspace_size(1, 4, 3, 512, 128) == 0
    assert fa.fa_bwd_gqa_workspace_size(1, 4, 2, 512, 80) == 0


def test_fwd_fp8_gqa_checks_on_host():
    a = dict(q8=A, qs=A + 8 * MB, k8=A + 16 * MB, ks=A + 24 * MB, v8t=A + 32 * MB, vs=A + 40 * MB,
             o=A + 48 * MB, lse=A + 56 * MB, B=1, H=4, Hkv=2, N=64, d=64, scale=0.125, causal=0, stream=None)
    call = lambda **kw: fa.fa_fwd_fp8_gqa(*[dict(a, **kw)[n] for n in (
        "q8", "qs", "k8", "ks", "v8t", "vs", "o", "lse", "B", "H", "Hkv", "N", "d", "scale", "causal", "stream")])
    assert call(Hkv=3) == fa.FA_ERR_HEADS
    assert call(Hkv=0) == fa.FA_ERR_SHAPE
    assert call(k8=None) == fa.FA_ERR_NULL
    # K codes of B*Hkv*N rows (8 KB here): an output 4 KB in overlaps them
    assert call(o=A + 16 * MB + 4096) == fa.FA_ERR_ALIAS


def _noalloc_call(**kw):
    args = dict(q=A, k=A + 8 * MB, v=A + 16 * MB, o=A + 24 * MB, lse=A + 32 * MB,
                B=1, H=2, Nq=64, Nk=128, d=64, scale=0.125, causal=0, splits=2, stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                     args["B"], args["H"], args["Nq"], args["Nk"], args["d"],
                                     args["scale"], args["causal"], args["splits"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(Nq=0), fa.FA_ERR_SHAPE), (dict(causal=1, Nq=129, Nk=128), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED_D), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(causal=3), fa.FA_ERR_CAUSAL),
    (dict(splits=0), fa.FA_ERR_SPLITS), (dict(splits=257), fa.FA_ERR_SPLITS),
    (dict(v=A + 16 * MB + 4), fa.FA_ERR_ALIGN), (dict(o=A + 8 * MB), fa.FA_ERR_ALIAS),
    # partials of 4 splits x 16384 rows x 128 dims x 4 B = 32 MiB, plus the
    # LSE part: one byte too many for the 32 MiB scratch
    (dict(B=1, H=16, Nq=1024, Nk=4096, d=128, splits=4, q=A, k=A + 64 * MB, v=A + 128 * MB,
          o=A + 192 * MB, lse=A + 256 * MB), fa.FA_ERR_SCRATCH),
])
def test_noalloc_bad_arguments_rejected_on_host(kw, status):
    assert _noalloc_call(**kw) == status


def test_noalloc_scratch_limit():
    cap = fa.fa_fwd_splitkv_noalloc_max_bytes()
    assert cap == 32 << 20
    # the largest decoding call of the test suite fits, with room to spare
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 1, 128, 256) <= cap
    assert fa.fa_fwd_splitkv_workspace_size(1, 16, 1024, 128, 4) > cap
