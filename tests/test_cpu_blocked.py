"""The blocked CPU baseline computes the same GEMM as the oracle (within the
fp32 error bound; exactly on integer data), so the time it reports is the
time of the right computation."""
import numpy as np
import pytest

import cpu_gemm
import gemm_inputs as gi
import oracle
from checks import within_bound


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_blocked_matches_oracle(in_dtype, ta, tb):
    M, N, K = 37, 70, 300   # ragged against MR, NR and KC
    for dist, exact in (("int2", True), ("uniform", False)):
        A = gi.draw(*((K, M) if ta else (M, K)), dist, 5, in_dtype)
        B = gi.draw(*((N, K) if tb else (K, N)), dist, 6, in_dtype)
        C = gi.draw(M, N, dist, 7, "f32")
        An, Bn, Cn = gi.as_numpy_bits(A), gi.as_numpy_bits(B), gi.as_numpy_bits(C)
        ref = oracle.gemm(An, Bn, a_dtype=in_dtype, trans_a=ta, trans_b=tb, alpha=1.5, beta=0.5,
                          C=Cn, c_dtype="f32", M=M, N=N, K=K)
        got = cpu_gemm.gemm_rows(An, Bn, in_dtype=in_dtype, ta=ta, tb=tb, M=M, N=N, K=K, alpha=1.5,
                                 beta=0.5, Cin=Cn, threads=3)
        if exact:
            assert np.array_equal(got.astype(np.float64), ref)
        else:
            an = oracle.row_norms(An, in_dtype, trans=ta)
            bn = oracle.col_norms(Bn, in_dtype, trans=tb)
            ok, worst, idx = within_bound(got.astype(np.float64), ref, 1e-5, 1.5, 0.5, an, bn, Cn.astype(np.float64))
            assert ok, (worst, idx)


def test_row_slab_and_threads():
    M, N, K = 50, 40, 64
    A = gi.as_numpy_bits(gi.draw(M, K, "int2", 8, "f32"))
    B = gi.as_numpy_bits(gi.draw(K, N, "int2", 9, "f32"))
    full = cpu_gemm.gemm_rows(A, B, in_dtype="f32", ta=False, tb=False, M=M, N=N, K=K, threads=1)
    part = cpu_gemm.gemm_rows(A, B, in_dtype="f32", ta=False, tb=False, M=M, N=N, K=K,
                              rows=(13, 41), threads=4)
    assert np.array_equal(full[13:41], part)
    assert np.array_equal(full.astype(np.float64), A.astype(np.float64) @ B.astype(np.float64))
