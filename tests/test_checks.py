"""The parity checkers catch errors planted in oracle results (CPU only)."""
import numpy as np

import oracle
from checks import TOL, freivalds, within_bound


def _case(seed=0, M=48, N=40, K=300):
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ref = oracle.gemm(A, B, alpha=1.5, beta=0.5, C=C)
    return A, B, C, ref


def test_within_bound_accepts_fp32_rounding_and_rejects_planted_error():
    A, B, C, ref = _case()
    an, bn = oracle.row_norms(A, "f32"), oracle.col_norms(B, "f32")
    rounded = oracle.round_to(ref, "f32")
    ok, worst, _ = within_bound(rounded, ref, TOL["f32"], 1.5, 0.5, an, bn, C)
    assert ok and worst < 0.1
    bad = rounded.astype(np.float64).copy()
    bad[7, 9] += 1e-3 * np.abs(ref).max()
    ok, _, idx = within_bound(bad, ref, TOL["f32"], 1.5, 0.5, an, bn, C)
    assert not ok and idx == (7, 9)
    nan = rounded.astype(np.float64).copy()
    nan[1, 2] = np.nan
    assert not within_bound(nan, ref, TOL["f32"], 1.5, 0.5, an, bn, C)[0]


def test_freivalds_accepts_good_and_rejects_planted_errors():
    A, B, C, ref = _case(1)
    opA, opB, cin = A.astype(np.float64), B.astype(np.float64), C.astype(np.float64)
    good = oracle.round_to(ref, "f32").astype(np.float64)
    assert freivalds(good, opA, opB, TOL["f32"], 1.5, 0.5, cin)
    # a dropped k term, a sign slip and a transposed operand all fail
    dropped = oracle.gemm(A[:, :-1], B[:-1], alpha=1.5, beta=0.5, C=C)
    assert not freivalds(dropped, opA, opB, TOL["f32"], 1.5, 0.5, cin)
    flipped = good.copy()
    flipped[3] = -flipped[3]
    assert not freivalds(flipped, opA, opB, TOL["f32"], 1.5, 0.5, cin)
    no_beta = oracle.gemm(A, B, alpha=1.5)
    assert not freivalds(no_beta, opA, opB, TOL["f32"], 1.5, 0.5, cin)
