"""Seeded synthetic inputs for the GEMM workloads.

This module holds no GEMM arithmetic: it only draws matrices from a seeded
CPU ``torch.Generator`` and casts them (round-to-nearest-even) to the stored
dtype.  Both the oracle-side tests and the GPU-side tests and benchmark take
their inputs from here, so the two sides read the same bits.

Distributions (per workload):

* ``"uniform"``  -- i.i.d. U(-1, 1)
* ``"normal"``   -- i.i.d. N(0, 1)
* ``"normal_k"`` -- i.i.d. N(0, 1) / sqrt(K)   (``scale_k`` gives K)
* ``"int2"``     -- i.i.d. integers uniform in {-2, ..., 2}

Seeds follow ``1000 * workload + role`` with role 1 = A, 2 = B, 3 = C_in;
integer twins add 100.
"""
from __future__ import annotations

import math

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def seed_for(workload: int, role: str, integer_twin: bool = False) -> int:
    return 1000 * workload + {"A": 1, "B": 2, "C": 3}[role] + (100 if integer_twin else 0)


def draw(rows: int, cols: int, dist: str, seed: int, dtype: str = "f32", *, ld: int | None = None,
         scale_k: int | None = None) -> torch.Tensor:
    """A rows x cols CPU tensor of ``dtype``; with ``ld > cols`` it is a view
    into a rows x ld buffer (the padding holds a recognisable fill value)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    width = cols if ld is None else ld
    if width < cols:
        raise ValueError("ld must be >= cols")
    shape = (rows, width)
    if dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "normal_k":
        x = torch.randn(shape, generator=g, dtype=torch.float32) / math.sqrt(max(scale_k or 1, 1))
    elif dist == "int2":
        x = torch.randint(-2, 3, shape, generator=g, dtype=torch.int32).to(torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if width > cols:
        x[:, cols:] = 1.0e30 if dtype == "f32" else 3.0e4  # never read by a correct GEMM
    x = x.to(DTYPES[dtype])
    return x[:, :cols] if width > cols else x


def as_numpy_bits(t: torch.Tensor):
    """Stored bits of a CPU tensor as numpy (float32, or uint16 for f16/bf16),
    keeping the row stride (leading dimension)."""
    import numpy as np
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        base = t.view(torch.int16)
        return base.numpy().view(np.uint16)
    if t.dtype == torch.float64:
        return t.numpy()
    raise TypeError(t.dtype)


# ---- the named workloads (shapes, layouts, scalars and input recipes) ----------
# ta/tb: False = op(X) is the stored matrix, True = its transpose.  "TN" (A
# stored M x K, B stored N x K) is ta=False, tb=True.
WORKLOADS = {
    "fp32_nn_256": dict(wid=1, in_dtype="f32", c_dtype="f32", M=256, N=256, K=256, ta=False,
                        tb=False, alpha=1.0, beta=0.0, dist="uniform"),
    "fp32_nn_4092": dict(wid=2, in_dtype="f32", c_dtype="f32", M=4092, N=4092, K=4092, ta=False,
                         tb=False, alpha=1.5, beta=0.5, dist="uniform"),
    "fp32_nn_8192x8192x4096": dict(wid=3, in_dtype="f32", c_dtype="f32", M=8192, N=8192, K=4096,
                                   ta=False, tb=False, alpha=1.0, beta=0.0, dist="normal"),
    **{f"fp16_tn_{n}": dict(wid=4, in_dtype="f16", c_dtype="f16", M=n, N=n, K=n, ta=False,
                            tb=True, alpha=1.0, beta=0.0, dist="normal_k")
       for n in (2048, 4096, 8192, 16384)},
    "bf16_nn_4096x11008x4096": dict(wid=5, in_dtype="bf16", c_dtype="f32", M=4096, N=11008,
                                    K=4096, ta=False, tb=False, alpha=1.0, beta=1.0,
                                    dist="uniform"),
    "bf16_nn_127x4096x4095": dict(wid=5, in_dtype="bf16", c_dtype="f32", M=127, N=4096, K=4095,
                                  ta=False, tb=False, alpha=1.0, beta=1.0, dist="uniform"),
}



# ---- tuning shapes ----------------------------------------------------------
# Square problems (2048^3, 4096^3, 8192^3) for every layout / output-type class that
# the named workloads leave out, so that the tuning table has a rule for each
# class: fp32 NT/TN/TT; fp16 with fp16 C in NN/TN/TT; fp16 with fp32 C and
# bf16 with bf16 C in all four layouts; bf16 with fp32 C in NT/TN/TT.  Inputs
# as in the named workloads of the same input type (fp32 N(0,1), 16-bit
# N(0,1)/sqrt(K)); alpha = 1, beta = 0; seeds from workload number 9.  Names
# carry the operation flags (opNT: ta = N, tb = T, the layout the pages call
# "TN" and the fp16 workloads use).
def _tuning_shapes():
    out = {}
    covered = {("f32", "f32", False, False), ("f16", "f16", False, True), ("bf16", "f32", False, False)}
    for ind, cd in (("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "f32"), ("bf16", "bf16")):
        for ta in (False, True):
            for tb in (False, True):
                if (ind, cd, ta, tb) in covered:
                    continue
                for n in (2048, 4096, 8192):
                    name = f"{ind}{'' if cd == ind else '_c' + cd}_op{'NT'[ta]}{'NT'[tb]}_{n}"
                    out[name] = dict(wid=9, in_dtype=ind, c_dtype=cd, M=n, N=n, K=n, ta=ta, tb=tb,
                                     alpha=1.0, beta=0.0, dist="normal" if ind == "f32" else "normal_k")
    return out


TUNING_SHAPES = _tuning_shapes()


def workload_inputs(name: str, integer_twin: bool = False):
    """(A, B, C_in) CPU tensors of a named workload (or tuning shape); C_in is
    None when beta == 0.

    A is stored M x K (K x M if ta), B stored K x N (N x K if tb); C_in is
    M x N in the output dtype.  The integer twin draws every matrix from
    {-2..2} with seeds offset by 100."""
    w = WORKLOADS[name] if name in WORKLOADS else TUNING_SHAPES[name]
    M, N, K = w["M"], w["N"], w["K"]
    sa = (K, M) if w["ta"] else (M, K)
    sb = (N, K) if w["tb"] else (K, N)
    dist = "int2" if integer_twin else w["dist"]
    A = draw(*sa, dist, seed_for(w["wid"], "A", integer_twin), w["in_dtype"], scale_k=K)
    B = draw(*sb, dist, seed_for(w["wid"], "B", integer_twin), w["in_dtype"], scale_k=K)
    C = None
    if w["beta"] != 0.0:
        cdist = "int2" if integer_twin else "uniform"
        C = draw(M, N, cdist, seed_for(w["wid"], "C", integer_twin), w["c_dtype"])
    return A, B, C
