"""Seeded synthetic inputs for the attention forward pass.

This module holds no attention arithmetic: it only draws Q, K, V and rounds
them to the storage type.  The GPU tests, the benchmark and the oracle tests
all take their inputs from here, so the device and the CPU oracle see
bit-identical values.

Recipe (one per workload):
  * generator: numpy.random.default_rng(seed).standard_normal(shape, float32),
    seed = 1000*cfg + t with t = 1 (Q), 2 (K), 3 (V), 4 (amplified Q rows),
    5 (amplified K rows);
  * "amplified" workloads multiply, for every (b, h), round(0.01*N) distinct
    seeded rows of Q and, separately, of K by 8 (exact in bf16) to force
    frequent running-max rescales; V is left alone;
  * bf16 workloads round the float32 draw to bfloat16 with round-to-nearest-
    even, and the oracle receives those rounded values widened to float32.
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    cfg: int            # 1-based id
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    amplify: bool = False

    @property
    def scale(self) -> float:
        """1/sqrt(d) as the float32 value handed to the library."""
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the throughput metric's count)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once (input dtype), LSE fp32."""
        n = self.B * self.H * self.N
        return 4 * n * self.d * self.elem_bytes + 4 * n

    def describe(self) -> str:
        return ("B=%d H=%d N=%d d=%d %s %s%s" % (
            self.B, self.H, self.N, self.d, self.dtype,
            "causal" if self.causal else "non-causal",
            ", 1% rows x8" if self.amplify else ""))


WORKLOADS = {
    1: Workload(1, "small_f32", 1, 1, 256, 64, "f32", False),
    2: Workload(2, "bf16_n1k_d64", 2, 8, 1024, 64, "bf16", False),
    3: Workload(3, "bf16_n4k_d128_causal", 4, 16, 4096, 128, "bf16", True),
    4: Workload(4, "bf16_n16k_d128_causal_amplified", 1, 32, 16384, 128, "bf16", True, True),
    5: Workload(5, "bf16_n32749_d64_tail", 1, 16, 32749, 64, "bf16", False),
}


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN is not expected here (the draws are finite).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exactly equal float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def _amplified_rows(seed, B, H, N):
    """For each (b, h): round(0.01*N) distinct row indices, seeded."""
    rng = np.random.default_rng(seed)
    n_amp = int(round(0.01 * N))
    return [[rng.choice(N, size=n_amp, replace=False) for _ in range(H)] for _ in range(B)]


def make_inputs(w, seed_base=None):
    """Draw (q, k, v) for workload `w` (a Workload or its id).

    Returns a dict with
      'q', 'k', 'v'      float32 arrays [B,H,N,d] holding the exact values the
                         library receives (bf16-rounded for bf16 workloads);
      'q_bits', ...      uint16 bf16 bit patterns (bf16 workloads only);
      'workload'         the Workload.
    """
    if isinstance(w, int):
        w = WORKLOADS[w]
    base = 1000 * w.cfg if seed_base is None else int(seed_base)
    shape = (w.B, w.H, w.N, w.d)
    q = _draw(base + 1, shape)
    k = _draw(base + 2, shape)
    v = _draw(base + 3, shape)
    if w.amplify:
        for arr, t in ((q, 4), (k, 5)):
            rows = _amplified_rows(base + t, w.B, w.H, w.N)
            for b in range(w.B):
                for h in range(w.H):
                    arr[b, h, rows[b][h], :] *= np.float32(8.0)
    out = {"workload": w}
    if w.dtype == "bf16":
        for name, arr in (("q", q), ("k", k), ("v", v)):
            bits = bf16_bits_rne(arr)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
    else:
        out.update(q=q, k=k, v=v)
    return out


def sample_rows(w, count, seed=7):
    """Flat row indices r = (b*H + h)*N + i spread over the workload:
    the first and last row of every head, the last tile's rows, and seeded
    random rows; sorted and unique."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    heads = w.B * w.H
    picks = []
    for bh in range(heads):
        picks += [bh * w.N, bh * w.N + w.N - 1]
    tail = np.arange(max(0, w.N - 3), w.N)
    picks += list(tail + (heads - 1) * w.N)
    extra = max(0, count - len(picks))
    picks += list(rng.integers(0, heads * w.N, size=extra))
    return np.unique(np.asarray(picks, dtype=np.int64))
