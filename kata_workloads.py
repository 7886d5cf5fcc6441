"""Seeded synthetic inputs and the workload table, shared by the tests, the smoke check and
the benchmark.

This module draws and shapes inputs only; it holds none of the attention arithmetic.  Both
the GPU path and the CPU oracle receive exactly the tensors built here (the oracle upcasts
them to float64).

Recipe (every workload): numpy PCG64 seeded with SeedSequence([workload_id, seed, T]);
float32 N(0, 1) drawn in the order q, k, v, dO, each as one C-order (B, T, H, D) array;
rows L2-normalized over the last dimension in float32 (workload 1: k only; the others: q and
k); then cast to bfloat16 by round-to-nearest-even (torch CPU) unless the workload is
float32.  Shapes follow the pages' kernel workloads: the 340M model's attention layer
(16 heads of width 64 at context 2048, from the KATA README's model description), a
quadratic/chunked crossover sweep, and long-context throughput at 131k tokens (the abstract's
operating point).  No dataset or benchmark suite is involved.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "DECODE", "SWEEP_T", "CROSSOVER_T", "make_inputs",
           "sweep_workload"]


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    T: int
    p: int
    dv: int
    chunk: int
    dtype: torch.dtype
    normalize_q: bool = True
    T_values: tuple = field(default=())

    @property
    def tokens(self):
        return self.B * self.H * self.T


WORKLOADS = {
    1: Workload(1, "tiny_fp32", B=1, H=1, T=256, p=8, dv=16, chunk=32,
                dtype=torch.float32, normalize_q=False),
    2: Workload(2, "layer340m", B=8, H=16, T=2048, p=16, dv=64, chunk=64,
                dtype=torch.bfloat16),
    3: Workload(3, "crossover_p32", B=4, H=16, T=16384, p=32, dv=64, chunk=64,
                dtype=torch.bfloat16, T_values=(1024, 4096, 8192, 16384)),
    4: Workload(4, "long_context_131k", B=1, H=16, T=131072, p=16, dv=64, chunk=64,
                dtype=torch.bfloat16),
    5: Workload(5, "training_4k", B=8, H=16, T=4096, p=16, dv=64, chunk=64,
                dtype=torch.bfloat16),
}

# Decode: one new token for each of 512 sequences of 16 heads, p=16, d_v=64 (a serving batch
# whose 545 MB of fp32 state exceeds the 256 MB Infinity Cache, so every step streams the
# state from HBM).
DECODE = Workload(6, "decode_b512", B=512, H=16, T=1, p=16, dv=64, chunk=64,
                  dtype=torch.bfloat16)

# Throughput sweep at p=16, d_v=64, 16 heads, with B*T held at 131072 head-positions.
SWEEP_T = (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)

# Sequence lengths of the quadratic/chunked crossover workload (B=4, H=16, p=32).
CROSSOVER_T = (1024, 4096, 8192, 16384)


def sweep_workload(T):
    return Workload(100 + SWEEP_T.index(T), f"sweep_T{T}", B=131072 // T, H=16, T=T, p=16,
                    dv=64, chunk=64, dtype=torch.bfloat16)


def _normalize_rows(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def make_inputs(w, seed=0, T=None, B=None, H=None, with_dO=False):
    """Return CPU tensors (q, k, v[, dO]) of dtype w.dtype, shaped (B, T, H, D).

    T/B/H override the workload's sizes (used for small slices of a workload's recipe).
    """
    T = w.T if T is None else T
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.wid, seed, T])))
    q = rng.standard_normal((B, T, H, w.p), dtype=np.float32)
    k = rng.standard_normal((B, T, H, w.p), dtype=np.float32)
    v = rng.standard_normal((B, T, H, w.dv), dtype=np.float32)
    dO = rng.standard_normal((B, T, H, w.dv), dtype=np.float32) if with_dO else None
    k = _normalize_rows(k)
    if w.normalize_q:
        q = _normalize_rows(q)
    out = [torch.from_numpy(x).to(w.dtype) for x in (q, k, v)]
    if with_dO:
        out.append(torch.from_numpy(dO).to(w.dtype))
    return tuple(out)
