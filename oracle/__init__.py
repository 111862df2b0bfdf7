"""fp64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (io_aware_softmax_fwd_amd): neither imports the other.

What it computes, for every (b, h, i) with Q of layout [B, H, Nq, d] and
K, V of layout [B, Hkv, Nk, d] (Nq == Nk == N for the square problem;
Hkv == H for ordinary multi-head attention, else query head h reads K/V
head h // (H // Hkv)):

    s_j   = scale * <q_i, k_j>          j in J_i = {0..Nk-1}, or, if causal,
                                        {0..i + Nk - Nq} (the last query lines
                                        up with the last key; needs Nq <= Nk)
    m     = max_j s_j
    l     = sum_j exp(s_j - m)
    O_i   = sum_j exp(s_j - m) v_j / l
    LSE_i = m + ln(l)

That is the plain three-step attention (zzszmyf.github.io notes
"FlashAttention 原理是什么", section 2; aiqz.cc Flash Attention IO article,
section 标准注意力瓶颈) with the max-subtracted softmax of the cf-1.com
write-up, section 3.1.  The method is exact up to rounding (notes,
section 5.1 and Theorem 1 in section 7.2), so the oracle is that definition
written out, in IEEE double.

Entry points
  attention_c(q, k, v, scale, causal, rows=None)  -- the C oracle (OpenMP)
  attention_np(q, k, v, scale, causal)            -- the same definition with
                                                     a numpy matmul per head
  online_merge_deferred(s, v, bounds)             -- running-max merge that
        divides once at the end (aiqz.cc article, section 在线Softmax算法;
        cf-1.com write-up, section 3.2)
  online_merge_normalized(s, v, bounds)           -- merge keeping O normalized
        after each block, with block-local max (notes, section 5)
  attention_bwd_c(q, k, v, dO, scale, causal, heads=None)
                                                  -- gradients dQ, dK, dV of
        the square problem for an upstream gradient dO (C, OpenMP)
  attention_bwd_np(q, k, v, dO, scale, causal)    -- the same gradients as
        numpy matrix products

Backward: the pages give the strategy (keep the row statistics, rebuild S
and P from Q, K, V in the backward pass; notes, section 6) but no formulas.
The gradients are the chain rule through O = P V, P = row-softmax(S),
S = scale Q K^T over the visible pairs:
    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
    dQ = scale dS K,  dK = scale dS^T Q.

The two merge forms are here only to pin the claim that a block-by-block
merge reproduces the whole-row softmax; the oracle itself never merges.
Pins for every function live in tests/test_oracle_pins.py.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_attn_f64.restype = ctypes.c_int
        lib.oracle_attn_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attn_bwd_f64.restype = ctypes.c_int
        lib.oracle_attn_bwd_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    """OpenMP threads the C oracle uses (OMP_NUM_THREADS / affinity)."""
    return int(_load().oracle_max_threads())


def _as_f32(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 4:
        raise ValueError("expected a [B, H, N, d] array")
    return x


def attention_c(q, k, v, scale, causal, rows=None):
    """fp64 attention of float32 inputs: q [B,H,Nq,d], k and v [B,Hkv,Nk,d].

    rows: optional 1-D array of flat query-row indices r = (b*H + h)*Nq + i.
    Returns (O, LSE) as float64: O [B,H,Nq,d] and LSE [B,H,Nq] when rows is
    None, else O [len(rows), d] and LSE [len(rows)].
    """
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3] \
            or q.shape[1] % k.shape[1] != 0:
        raise ValueError("q [B,H,Nq,d], k and v [B,Hkv,Nk,d] with Hkv dividing H expected")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    if rows is None:
        nrows = B * H * Nq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64).ravel()
        nrows = rows_arr.size
    O = np.empty((nrows, d), dtype=np.float64)
    LSE = np.empty((nrows,), dtype=np.float64)
    rc = _load().oracle_attn_f64(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Hkv, Nq, Nk, d,
        float(scale), int(bool(causal)),
        None if rows_arr is None else rows_arr.ctypes.data, nrows,
        O.ctypes.data, LSE.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_attn_f64 failed with code %d" % rc)
    if rows is None:
        return O.reshape(B, H, Nq, d), LSE.reshape(B, H, Nq)
    return O, LSE


def attention_np(q, k, v, scale, causal, block_rows=1024):
    """The same definition as attention_c, written with numpy fp64 matmuls.

    Row blocks only bound memory; each row's softmax is taken whole.  Grouped
    K/V heads are expanded by repeating each one H // Hkv times.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    if k.shape[1] != H:
        k = np.repeat(k, H // k.shape[1], axis=1)
        v = np.repeat(v, H // v.shape[1], axis=1)
    Nk = k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    O = np.empty((B, H, Nq, d))
    LSE = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, block_rows):
                r1 = min(Nq, r0 + block_rows)
                s = float(scale) * (q[b, h, r0:r1] @ k[b, h].T)   # [rows, Nk]
                if causal:
                    keep = np.arange(Nk)[None, :] <= (np.arange(r0, r1) + (Nk - Nq))[:, None]
                    s = np.where(keep, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                O[b, h, r0:r1] = (p @ v[b, h]) / l
                LSE[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    return O, LSE


def attention_bwd_c(q, k, v, dO, scale, causal, heads=None):
    """fp64 gradients of the square attention problem: q, k, v, dO are
    float32 [B,H,N,d].  heads: optional flat (b*H + h) indices to compute.
    Returns (dQ, dK, dV) float64, [B,H,N,d] each when heads is None, else
    [len(heads), N, d]."""
    q, k, v, dO = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dO)
    if not (q.shape == k.shape == v.shape == dO.shape):
        raise ValueError("q, k, v, dO must share one [B,H,N,d] shape")
    B, H, N, d = q.shape
    if heads is None:
        nh, harr = B * H, None
    else:
        harr = np.ascontiguousarray(heads, dtype=np.int64).ravel()
        nh = harr.size
    dQ = np.empty((nh, N, d))
    dK = np.empty((nh, N, d))
    dV = np.empty((nh, N, d))
    rc = _load().oracle_attn_bwd_f64(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dO.ctypes.data, B, H, N, d, float(scale),
        int(bool(causal)), None if harr is None else harr.ctypes.data, nh,
        dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd_f64 failed with code %d" % rc)
    if heads is None:
        return dQ.reshape(B, H, N, d), dK.reshape(B, H, N, d), dV.reshape(B, H, N, d)
    return dQ, dK, dV


def attention_bwd_np(q, k, v, dO, scale, causal):
    """The same gradients as attention_bwd_c with whole-head numpy matrices
    (small problems only: one N x N matrix per head)."""
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    B, H, N, d = q.shape
    dQ, dK, dV = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = dO[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dV[b, h] = p.T @ dO[b, h]
            dQ[b, h] = float(scale) * (ds @ k[b, h])
            dK[b, h] = float(scale) * (ds.T @ q[b, h])
    return dQ, dK, dV


def _blocks(n, bounds):
    edges = [0] + list(bounds) + [n]
    for a, b in zip(edges[:-1], edges[1:]):
        if b > a:
            yield a, b


def online_merge_deferred(s, v, bounds):
    """Block-by-block softmax-weighted sum of one score row, dividing once.

    s: scores [n]; v: values [n, d]; bounds: increasing split points.
    Running state (m, l, acc) starts at (-inf, 0, 0).  For each block:
      m_new = max(m, max s_blk);  r = exp(m - m_new)
      l   <- r*l   + sum exp(s_blk - m_new)
      acc <- r*acc + sum exp(s_blk - m_new) v_blk
    and O = acc / l at the end (aiqz.cc article, section 在线Softmax算法).
    Returns (O [d], l, m) with l relative to the final m.
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(s), -1)
    m, l = -np.inf, 0.0
    acc = np.zeros(v.shape[1])
    for a, b in _blocks(len(s), bounds):
        m_new = max(m, float(s[a:b].max()))
        r = np.exp(m - m_new)
        p = np.exp(s[a:b] - m_new)
        l = r * l + p.sum()
        acc = r * acc + p @ v[a:b]
        m = m_new
    return acc / l, l, m


def online_merge_normalized(s, v, bounds, trace=None):
    """Block merge that keeps O normalized after every block.

    Per block: block-local max mt, Pt = exp(s_blk - mt), lt = sum Pt, then
      m'  = max(m, mt)
      l'  = exp(m - m') l + exp(mt - m') lt
      O'  = (exp(m - m') l O + exp(mt - m') Pt v_blk) / l'
    (zzszmyf.github.io notes, section 5 update equations).  If `trace` is a
    list, (m, l, O) after each block is appended to it.
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(s), -1)
    m, l = -np.inf, 0.0
    O = np.zeros(v.shape[1])
    for a, b in _blocks(len(s), bounds):
        mt = float(s[a:b].max())
        pt = np.exp(s[a:b] - mt)
        lt = pt.sum()
        m_new = max(m, mt)
        a_old = np.exp(m - m_new) if l > 0 else 0.0
        a_new = np.exp(mt - m_new)
        l_new = a_old * l + a_new * lt
        O = (a_old * l * O + a_new * (pt @ v[a:b])) / l_new
        m, l = m_new, l_new
        if trace is not None:
            trace.append((m, l, O.copy()))
    return O, l, m
