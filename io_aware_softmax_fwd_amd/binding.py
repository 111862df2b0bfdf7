"""ctypes binding of libfa_fwd.so (declared in include/fa_fwd.h).

Argument marshalling only: every step of the attention forward pass runs in
the library's HIP kernels.  There is no fallback: if the library is missing
or cannot be loaded, every call raises.

Low level (same names and arguments as the C functions, raw pointers):
    fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> status
    fa_fwd_f32(...)                                            -> status
    fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal,
                   num_splits, workspace, workspace_bytes, stream) -> status
    fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits)     -> bytes
    fa_fwd_splitkv_num_splits(B, H, Nq, Nk, num_cus)           -> count
    fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale,
                           causal, num_splits, stream)         -> status
    fa_fwd_splitkv_noalloc_max_bytes()                         -> bytes
    fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal,
               num_splits, workspace, workspace_bytes, stream) -> status
    fa_fwd_gqa_num_splits(B, H, Hkv, Nq, Nk, causal, num_cus)  -> count
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
           workspace, workspace_bytes, stream)                 -> status
    fa_bwd_workspace_size(B, H, N, d)                          -> bytes
    fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale,
               causal, workspace, workspace_bytes, stream)     -> status
    fa_bwd_gqa_workspace_size(B, H, Hkv, N, d)                 -> bytes
    fa_quantize_qk_fp8(x, rows, d, x8, xs, stream)             -> status
    fa_quantize_qk_fp8_rotated(x, rows, d, signs, x8, xs, stream) -> status
    fa_quantize_v_fp8(v, BH, N, d, v8t, vs, stream)            -> status
    fa_fp8_v_bytes(BH, N, d), fa_fp8_v_scale_bytes(BH, N, d)   -> bytes
    fa_fwd_fp8(q8, qs, k8, ks, v8t, vs, o, lse, B, H, N, d, scale, causal,
               stream)                                         -> status
    fa_fwd_fp8_gqa(q8, qs, k8, ks, v8t, vs, o, lse, B, H, Hkv, N, d, scale,
                   causal, stream)                             -> status
    fa_strerror(status)                                        -> str
High level (torch tensors on a ROCm device):
    fwd(q, k, v, scale=None, causal=False, out=None, lse=None) -> (o, lse)
    fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=None,
                workspace=None)                                -> (o, lse)
    fwd_gqa(q, k, v, scale=None, causal=False, num_splits=1,
            workspace=None)                                    -> (o, lse)
    bwd(q, k, v, o, lse, dout, scale=None, causal=False,
        workspace=None)                                        -> (dq, dk, dv)
    bwd_gqa(q, k, v, o, lse, dout, scale=None, causal=False,
            workspace=None)                                    -> (dq, dk, dv)
    quantize_qk_fp8(x, signs=None, rotate=False)               -> (x8, xs)
    quantize_v_fp8(v)                                          -> (v8t, vs)
    fwd_fp8(q8, qs, k8, ks, v8t, vs, scale=None, causal=False) -> (o, lse)
The high-level functions check every tensor they are given (type, device,
dtype, shape, contiguity) before any launch, so a mismatched buffer raises
TypeError or ValueError instead of being read or written out of bounds.
"""
import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_UNSUPPORTED_D = 3
FA_ERR_SCALE = 4
FA_ERR_ALIGN = 5
FA_ERR_HIP = 6
FA_ERR_CAUSAL = 7
FA_ERR_ALIAS = 8
FA_ERR_WORKSPACE = 9
FA_ERR_SPLITS = 10
FA_ERR_HEADS = 11
FA_ERR_SCRATCH = 12

EXPORTED = ("fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
            "fa_fwd_splitkv_num_splits", "fa_fwd_splitkv_noalloc", "fa_fwd_splitkv_noalloc_max_bytes",
            "fa_fwd_gqa", "fa_fwd_gqa_num_splits", "fa_bwd",
            "fa_bwd_workspace_size", "fa_bwd_gqa", "fa_bwd_gqa_workspace_size", "fa_quantize_qk_fp8", "fa_quantize_qk_fp8_rotated", "fa_quantize_v_fp8", "fa_fp8_v_bytes",
            "fa_fp8_v_scale_bytes", "fa_fwd_fp8", "fa_fwd_fp8_gqa", "fa_strerror")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed: %s (status %d)" % (what, fa_strerror(status), status))
        self.status = status


def _check(name, t, device, dtype=None, shape=None, min_bytes=None):
    """Raise unless t is a contiguous torch tensor on `device` with the given
    dtype and shape (or at least min_bytes bytes)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s must live on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s" % (name, tuple(shape)))
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s must hold at least %d bytes" % (name, min_bytes))


def _gpu_device(name, t):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must live on the GPU" % name)
    return t.device


def load():
    """Load libfa_fwd.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libfa_fwd.so not found at %s; build it with "
            "`python -m io_aware_softmax_fwd_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    for name in ("fa_fwd", "fa_fwd_f32"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 +
                                   [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p])
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int] * 5
    lib.fa_fwd_splitkv_num_splits.restype = ctypes.c_int
    lib.fa_fwd_splitkv_num_splits.argtypes = [ctypes.c_int] * 5
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 +
                                           [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
    lib.fa_fwd_splitkv_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_noalloc_max_bytes.argtypes = []
    lib.fa_fwd_gqa.restype = ctypes.c_int
    lib.fa_fwd_gqa.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                               [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_void_p])
    lib.fa_fwd_gqa_num_splits.restype = ctypes.c_int
    lib.fa_fwd_gqa_num_splits.argtypes = [ctypes.c_int] * 7
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int] * 4 +
                           [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                            ctypes.c_void_p])
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_size.argtypes = [ctypes.c_int] * 4
    lib.fa_bwd_gqa.restype = ctypes.c_int
    lib.fa_bwd_gqa.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 +
                               [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p])
    lib.fa_bwd_gqa_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_gqa_workspace_size.argtypes = [ctypes.c_int] * 5
    lib.fa_quantize_qk_fp8.restype = ctypes.c_int
    lib.fa_quantize_qk_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_quantize_qk_fp8_rotated.restype = ctypes.c_int
    lib.fa_quantize_qk_fp8_rotated.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_quantize_v_fp8.restype = ctypes.c_int
    lib.fa_quantize_v_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for name in ("fa_fp8_v_bytes", "fa_fp8_v_scale_bytes"):
        f = getattr(lib, name)
        f.restype = ctypes.c_size_t
        f.argtypes = [ctypes.c_int] * 3
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 4 +
                               [ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
    lib.fa_fwd_fp8_gqa.restype = ctypes.c_int
    lib.fa_fwd_fp8_gqa.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 5 +
                                   [ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    return load().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, workspace,
                   workspace_bytes, stream):
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits,
                                 workspace, workspace_bytes, stream)


def fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits):
    return int(load().fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits))


def fa_fwd_splitkv_num_splits(B, H, Nq, Nk, num_cus):
    return int(load().fa_fwd_splitkv_num_splits(B, H, Nq, Nk, num_cus))


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, stream):
    return load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits,
                                         stream)


def fa_fwd_splitkv_noalloc_max_bytes():
    return int(load().fa_fwd_splitkv_noalloc_max_bytes())


def fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, num_splits, workspace,
               workspace_bytes, stream):
    return load().fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, num_splits,
                             workspace, workspace_bytes, stream)


def fa_fwd_gqa_num_splits(B, H, Hkv, Nq, Nk, causal, num_cus):
    return int(load().fa_fwd_gqa_num_splits(B, H, Hkv, Nq, Nk, causal, num_cus))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace,
           workspace_bytes, stream):
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace,
                         workspace_bytes, stream)


def fa_bwd_workspace_size(B, H, N, d):
    return int(load().fa_bwd_workspace_size(B, H, N, d))


def fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace,
               workspace_bytes, stream):
    return load().fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal,
                             workspace, workspace_bytes, stream)


def fa_bwd_gqa_workspace_size(B, H, Hkv, N, d):
    return int(load().fa_bwd_gqa_workspace_size(B, H, Hkv, N, d))


def fa_quantize_qk_fp8(x, rows, d, x8, xs, stream):
    return load().fa_quantize_qk_fp8(x, rows, d, x8, xs, stream)


def fa_quantize_qk_fp8_rotated(x, rows, d, signs, x8, xs, stream):
    return load().fa_quantize_qk_fp8_rotated(x, rows, d, signs, x8, xs, stream)


def fa_quantize_v_fp8(v, BH, N, d, v8t, vs, stream):
    return load().fa_quantize_v_fp8(v, BH, N, d, v8t, vs, stream)


def fa_fp8_v_bytes(BH, N, d):
    return int(load().fa_fp8_v_bytes(BH, N, d))


def fa_fp8_v_scale_bytes(BH, N, d):
    return int(load().fa_fp8_v_scale_bytes(BH, N, d))


def fa_fwd_fp8(q8, qs, k8, ks, v8t, vs, o, lse, B, H, N, d, scale, causal, stream):
    return load().fa_fwd_fp8(q8, qs, k8, ks, v8t, vs, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_fp8_gqa(q8, qs, k8, ks, v8t, vs, o, lse, B, H, Hkv, N, d, scale, causal, stream):
    return load().fa_fwd_fp8_gqa(q8, qs, k8, ks, v8t, vs, o, lse, B, H, Hkv, N, d, scale, causal, stream)


def fa_strerror(status):
    return load().fa_strerror(int(status)).decode()


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """Attention forward of torch tensors q, k, v [B,H,N,d] (bf16 or fp32,
    contiguous, on the GPU).  Queues the kernel on `stream` (default: torch's
    current stream) and returns (o, lse); o has q's dtype, lse is fp32 [B,H,N].
    """
    import torch
    dev = _gpu_device("q", q)
    _check("q", q, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("k", k), ("v", v)):
        _check(name, t, dev, q.dtype, q.shape)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("out", out, dev, q.dtype, q.shape)
    _check("lse", lse, dev, torch.float32, (B, H, N))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    f = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = f(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
           B, H, N, d, float(scale), int(bool(causal)), stream)
    if st != FA_OK:
        raise FaError(st, f.__name__)
    return out, lse


def fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=None, workspace=None,
                out=None, lse=None, stream=None):
    """Key-split attention forward of bf16 torch tensors: q [B,H,Nq,d],
    k and v [B,H,Nk,d] (contiguous, on the GPU).  num_splits defaults to the
    library's suggestion for this GPU; workspace (a uint8 device tensor) is
    allocated here if not given.  Returns (o, lse)."""
    import torch
    dev = _gpu_device("q", q)
    _check("q", q, dev, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    B, H, Nq, d = q.shape
    _gpu_device("k", k)
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Nk, d]")
    Nk = k.shape[2]
    for name, t in (("k", k), ("v", v)):
        _check(name, t, dev, torch.bfloat16, (B, H, Nk, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = fa_fwd_splitkv_num_splits(B, H, Nq, Nk, cus)
    need = fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check("out", out, dev, torch.bfloat16, q.shape)
    _check("lse", lse, dev, torch.float32, (B, H, Nq))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, Nq, Nk, d, float(scale), int(bool(causal)), int(num_splits),
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv")
    return out, lse


def fwd_gqa(q, k, v, scale=None, causal=False, num_splits=1, workspace=None,
            out=None, lse=None, stream=None):
    """Grouped-K/V-head attention forward of bf16 torch tensors: q [B,H,Nq,d],
    k and v [B,Hkv,Nk,d] with Hkv dividing H (contiguous, on the GPU).
    num_splits=None takes the library's suggestion for this GPU; with more
    than one split a workspace (uint8 device tensor) is allocated here if not
    given.  Returns (o, lse)."""
    import torch
    dev = _gpu_device("q", q)
    _check("q", q, dev, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    B, H, Nq, d = q.shape
    _gpu_device("k", k)
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, Nk, d]")
    Hkv, Nk = k.shape[1], k.shape[2]
    for name, t in (("k", k), ("v", v)):
        _check(name, t, dev, torch.bfloat16, (B, Hkv, Nk, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = fa_fwd_gqa_num_splits(B, H, Hkv, Nq, Nk, int(bool(causal)), cus)
    ws_ptr, ws_bytes = None, 0
    if num_splits > 1:
        if workspace is None:
            need = fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check("workspace", workspace, dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check("out", out, dev, torch.bfloat16, q.shape)
    _check("lse", lse, dev, torch.float32, (B, H, Nq))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), int(num_splits),
                    ws_ptr, ws_bytes, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_gqa")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None):
    """Attention backward of bf16 torch tensors q, k, v, o, dout [B,H,N,d] and
    the forward's lse [B,H,N] (fp32), all contiguous on the GPU.  Returns
    (dq, dk, dv) as bf16 tensors; the workspace (uint8 device tensor) is
    allocated here if not given."""
    import torch
    dev = _gpu_device("q", q)
    _check("q", q, dev, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(name, t, dev, torch.bfloat16, q.shape)
    B, H, N, d = q.shape
    _check("lse", lse, dev, torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(1, fa_bwd_workspace_size(B, H, N, d)), dtype=torch.uint8,
                                device=q.device)
    _check("workspace", workspace, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                float(scale), int(bool(causal)), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def bwd_gqa(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None):
    """Backward pass with grouped K/V heads: q, o, dout [B,H,N,d] and k, v
    [B,Hkv,N,d] bf16 (Hkv dividing H), lse [B,H,N] fp32 from the forward, all
    contiguous on the GPU.  Returns (dq [B,H,N,d], dk and dv [B,Hkv,N,d]) as
    bf16; the workspace (uint8 device tensor) is allocated here if not given."""
    import torch
    dev = _gpu_device("q", q)
    _check("q", q, dev, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("o", o), ("dout", dout)):
        _check(name, t, dev, torch.bfloat16, q.shape)
    _gpu_device("k", k)
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, N, d]")
    Hkv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        _check(name, t, dev, torch.bfloat16, (B, Hkv, N, d))
    _check("lse", lse, dev, torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(1, fa_bwd_gqa_workspace_size(B, H, Hkv, N, d)), dtype=torch.uint8,
                                device=q.device)
    _check("workspace", workspace, dev)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                    float(scale), int(bool(causal)), workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_gqa")
    return dq, dk, dv


def _bf16_4d(name, t):
    import torch
    _check(name, t, _gpu_device(name, t), torch.bfloat16)
    if t.dim() != 4:
        raise ValueError("%s must be [B, H, N, d]" % name)


def quantize_qk_fp8(x, stream=None, rotate=False, signs=None):
    """MX fp8 quantization of a bf16 [B,H,N,d] Q or K: returns (codes uint8
    [B,H,N,d], E8M0 scales uint8 [B,H,N,d/32]).  rotate=True quantizes the
    rows rotated by diag(signs) H_d (fa_quantize_qk_fp8_rotated); signs is
    then None or an int8 tensor of d entries on the same device."""
    import torch
    _bf16_4d("x", x)
    B, H, N, d = x.shape
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    xs = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    if rotate:
        sp = None
        if signs is not None:
            _check("signs", signs, x.device, torch.int8, (d,))
            sp = signs.data_ptr()
        st = fa_quantize_qk_fp8_rotated(x.data_ptr(), B * H * N, d, sp, x8.data_ptr(), xs.data_ptr(), stream)
        name = "fa_quantize_qk_fp8_rotated"
    else:
        if signs is not None:
            raise ValueError("signs are only used with rotate=True")
        st = fa_quantize_qk_fp8(x.data_ptr(), B * H * N, d, x8.data_ptr(), xs.data_ptr(), stream)
        name = "fa_quantize_qk_fp8"
    if st != FA_OK:
        raise FaError(st, name)
    return x8, xs


def quantize_v_fp8(v, stream=None):
    """MX fp8 quantization of a bf16 [B,H,N,d] V into the transposed tile
    layout: returns (codes uint8, scales uint8), flat buffers of
    fa_fp8_v_bytes / fa_fp8_v_scale_bytes bytes."""
    import torch
    _bf16_4d("v", v)
    B, H, N, d = v.shape
    v8t = torch.empty(fa_fp8_v_bytes(B * H, N, d), dtype=torch.uint8, device=v.device)
    vs = torch.empty(fa_fp8_v_scale_bytes(B * H, N, d), dtype=torch.uint8, device=v.device)
    if stream is None:
        stream = torch.cuda.current_stream(v.device).cuda_stream
    st = fa_quantize_v_fp8(v.data_ptr(), B * H, N, d, v8t.data_ptr(), vs.data_ptr(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_quantize_v_fp8")
    return v8t, vs


def fwd_fp8(q8, qs, k8, ks, v8t, vs, scale=None, causal=False, stream=None):
    """fp8 attention forward of quantized inputs (as returned by
    quantize_qk_fp8 and quantize_v_fp8); q8 gives the [B,H,N,d] shape and
    k8 [B,Hkv,N,d] the K/V heads (Hkv dividing H; Hkv < H reads each K/V head
    for H/Hkv query heads).  Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    import torch
    dev = _gpu_device("q8", q8)
    _check("q8", q8, dev, torch.uint8)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    if d not in (64, 128):
        raise ValueError("head dimension must be 64 or 128")
    _gpu_device("k8", k8)
    if k8.dim() != 4:
        raise ValueError("k8 must be [B, Hkv, N, d]")
    Hkv = k8.shape[1]
    _check("k8", k8, dev, torch.uint8, (B, Hkv, N, d))
    _check("qs", qs, dev, torch.uint8, (B, H, N, d // 32))
    _check("ks", ks, dev, torch.uint8, (B, Hkv, N, d // 32))
    _check("v8t", v8t, dev, torch.uint8, min_bytes=fa_fp8_v_bytes(B * Hkv, N, d))
    _check("vs", vs, dev, torch.uint8, min_bytes=fa_fp8_v_scale_bytes(B * Hkv, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    st = fa_fwd_fp8_gqa(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(), v8t.data_ptr(),
                        vs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d, float(scale),
                        int(bool(causal)), stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_gqa")
    return o, lse
