"""Non-finite inputs (IEEE 754 arithmetic in C = alpha * op(A) op(B) + beta * C):
a NaN in row i of op(A) makes row i of C NaN; an infinity in op(B) gives
+Inf, -Inf or NaN (inf - inf, 0 * inf) down its column, by the signs of
its partners; everything else stays finite and exact.  Which of NaN, +Inf,
-Inf or a finite value an output is does not depend on the order of the
sum (integer data keep every finite partial sum exact and far from
overflow), so every configuration, both entry points and every layout must
give exactly the oracle's classes, and bit-exact values where finite.  NaN
payloads are not compared."""
import numpy as np
import pytest

import gemm_inputs as gi
from gpu_helpers import SK_WS_BYTES, log, oracle_full, out_as_f64, run_gpu, stored_shapes

pytestmark = pytest.mark.gpu

M, N, K = 304, 264, 200  # multiples of 8, so every stored layout takes the 16-byte-load tiles; ragged against them


def _plant(A, B, ta, tb):
    """NaN at op(A)[5, 7]; op(A)[:, 11] = 1 and op(B)[11, 13] = +Inf (column 13
    +Inf except in rows holding a NaN); op(B)[20, 40] = -Inf with op(A)[:, 20]
    the int2 draw (its zeros make 0 * inf = NaN, its signs pick +-Inf);
    op(B)[150, 250] = +Inf and op(B)[151, 250] = -Inf (inf - inf = NaN
    wherever both partners are non-zero)."""
    A, B = A.clone(), B.clone()
    a = A.t() if ta else A     # op(A) view, M x K
    b = B.t() if tb else B     # op(B) view, K x N
    a[5, 7] = float("nan")
    a[:, 11] = 1.0
    b[11, 13] = float("inf")
    b[20, 40] = -float("inf")
    b[150, 250] = float("inf")
    b[151, 250] = -float("inf")
    return A, B


def _classes(x: np.ndarray):
    return np.where(np.isnan(x), 0, np.where(np.isposinf(x), 1, np.where(np.isneginf(x), 2, 3)))


def _check(got, ref, c_dtype, what):
    import oracle
    have = out_as_f64(got, c_dtype)
    want = oracle.widen(oracle.round_to(ref, c_dtype), c_dtype)
    hc, wc = _classes(have), _classes(want)
    if not np.array_equal(hc, wc):
        i, j = np.argwhere(hc != wc)[0]
        raise AssertionError(f"{what}: class mismatch at ({i},{j}): got {have[i, j]!r} want {want[i, j]!r}")
    fin = wc == 3
    assert np.array_equal(have[fin], want[fin]), f"{what}: finite values differ"
    return int((wc == 0).sum()), int((wc == 1).sum()), int((wc == 2).sum())


@pytest.mark.parametrize("in_dtype,c_dtype", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)],
                         ids=["NN", "NT", "TN", "TT"])
def test_nonfinite_inputs_every_config(in_dtype, c_dtype, ta, tb):
    import dense_gemm_12_amd as mg
    sa, sb = stored_shapes(M, N, K, ta, tb)
    A = gi.draw(*sa, "int2", 7100, in_dtype)
    B = gi.draw(*sb, "int2", 7101, in_dtype)
    C = gi.draw(M, N, "int2", 7102, c_dtype)
    A, B = _plant(A, B, ta, tb)
    ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
    counts = None
    for cfg in [-1] + list(range(mg.num_configs(in_dtype))):
        name = "plan" if cfg < 0 else mg.config_name(in_dtype, cfg)
        ws = SK_WS_BYTES if name.endswith("_sk") else None
        what = f"{name} {in_dtype}->{c_dtype} ta={ta} tb={tb}"
        log("case " + what)
        try:
            got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, c_dtype=c_dtype, config=cfg,
                          workspace_bytes=ws)
        except mg.MgemmError as e:
            # the few-row tile stores only k-contiguous A
            if e.status == mg.MG_EUNSUPPORTED and ta and "_64x" in name:
                continue
            raise
        c = _check(got, ref, c_dtype, what)
        counts = counts or c
        assert c == counts
    nan, pinf, ninf = counts
    assert nan >= N and pinf > 0 and ninf > 0, counts  # every planted case is present


@pytest.mark.parametrize("in_dtype,c_dtype", [("f32", "f32"), ("bf16", "f32")])
def test_nonfinite_inputs_split_k(in_dtype, c_dtype):
    """The same through gemm_ex: fp32 partials of each K range summed by
    the reduction kernel keep the classes."""
    A = gi.draw(M, K, "int2", 7200, in_dtype)
    B = gi.draw(K, N, "int2", 7201, in_dtype)
    C = gi.draw(M, N, "int2", 7202, c_dtype)
    A, B = _plant(A, B, False, False)
    ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=False, in_dtype=in_dtype, c_dtype=c_dtype)
    for splits in (2, 3, 4):
        what = f"split-K {splits} {in_dtype}->{c_dtype}"
        log("case " + what)
        got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=False, c_dtype=c_dtype,
                      workspace_bytes=splits * M * N * 4 + (1 << 20), splits=splits)
        _check(got, ref, c_dtype, what)
