"""Comparison helpers used by the parity tests (host-side, fp64).

* ``within_bound`` -- element-wise |C - C_ref| <= tol*(|alpha||a_i||b_j| + |beta||C_in_ij|),
  the error model for random inputs (tol 1e-5 for fp32, 4e-3 for fp16/bf16
  inputs); a_i is row i of op(A), b_j column j of op(B).
* ``freivalds`` -- a whole-matrix probabilistic check: for a random +-1
  vector x, (C x)_i must match (alpha op(A) (op(B) x) + beta C_in x)_i within
  sum_j |x_j| bound_ij = sum_j bound_ij.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3}


def within_bound(got, ref, tol, alpha, beta, a_norms, b_norms, c_in=None):
    """Return (ok, worst ratio |err|/bound, index of the worst element)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = abs(alpha) * np.outer(a_norms, b_norms)
    if beta != 0.0 and c_in is not None:
        bound = bound + abs(beta) * np.abs(np.asarray(c_in, dtype=np.float64))
    bound = tol * bound
    err = np.abs(got - ref)
    if not np.all(np.isfinite(got)):
        bad = np.argwhere(~np.isfinite(got))[0]
        return False, float("inf"), tuple(bad)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    idx = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else ()
    worst = float(ratio[idx]) if ratio.size else 0.0
    return bool(worst <= 1.0), worst, idx


def freivalds(C, opA, opB, tol, alpha, beta, c_in=None, seed=0, rounds=2):
    """fp64 Freivalds check of C ~= alpha opA opB + beta c_in.  opA (M x K),
    opB (K x N) and c_in are fp64 arrays of the exact stored values."""
    rng = np.random.default_rng(seed)
    M, N = C.shape
    a_norms = np.sqrt(np.einsum("ik,ik->i", opA, opA))
    b_norms = np.sqrt(np.einsum("kj,kj->j", opB, opB))
    b_sum = b_norms.sum()
    for _ in range(rounds):
        x = rng.choice([-1.0, 1.0], size=N)
        lhs = C @ x
        rhs = alpha * (opA @ (opB @ x))
        slack = tol * abs(alpha) * a_norms * b_sum
        if beta != 0.0:
            rhs = rhs + beta * (c_in @ x)
            slack = slack + tol * abs(beta) * np.abs(c_in).sum(axis=1)
        # fp64 evaluation error of the check itself is far below tol-level slack
        if not np.all(np.abs(lhs - rhs) <= slack + 1e-9 * (np.abs(rhs) + 1)):
            return False
    return True
