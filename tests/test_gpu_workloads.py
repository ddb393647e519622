"""GPU parity on the named workloads at their full sizes, in the launch
configuration the benchmark times (the planner's choice).

The 2048^3 tuning shapes (every layout and output-type class the workloads
leave out, each run on the tuned rule for its class) get the same checks.

Small workloads are compared with the full oracle; large ones with the oracle
on sampled rows, columns and corner blocks (element for element) plus a
whole-matrix Freivalds check.  Integer twins of every workload are checked
bit-exactly (sampled) and with an exact integer Freivalds check.
"""
import zlib

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import (assert_bit_exact, assert_within, freivalds_stream, log, oracle_cols,
                         oracle_full, oracle_rows, out_as_f64, run_gpu, sample_plan, _sub)

pytestmark = pytest.mark.gpu

FULL_ORACLE_MAX_MACS = 3e9
SIGNIFICAND_BITS = {"f32": 24, "f16": 11, "bf16": 8}


def _check_workload(name, integer_twin):
    w = gi.WORKLOADS[name] if name in gi.WORKLOADS else gi.TUNING_SHAPES[name]
    M, N, K = w["M"], w["N"], w["K"]
    kw = dict(alpha=w["alpha"], beta=w["beta"], ta=w["ta"], tb=w["tb"], in_dtype=w["in_dtype"],
              c_dtype=w["c_dtype"])
    what = f"{name}{' int' if integer_twin else ''}"
    log(f"workload {what}: generating inputs")
    A, B, C = gi.workload_inputs(name, integer_twin)
    # the benchmark's launch configuration: through gemm_ex with the
    # planner's workspace when it asks for one (split-K, repacking, stream-K)
    import dense_gemm_12_amd as mg
    codes = mg.DTYPE_CODES
    ws = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]), M, N, K,
                           A.stride(0), B.stride(0))
    log(f"workload {what}: GPU run (workspace {ws} bytes)")
    got = run_gpu(A, B, C, alpha=w["alpha"], beta=w["beta"], ta=w["ta"], tb=w["tb"],
                  c_dtype=w["c_dtype"], workspace_bytes=ws if ws else None, splits=0)
    c = w["c_dtype"]
    if M * N * K <= FULL_ORACLE_MAX_MACS:
        log(f"workload {what}: full oracle")
        ref = oracle_full(A, B, C, **kw)
        if integer_twin:
            assert_bit_exact(got, ref, c, what)
        else:
            assert_within(out_as_f64(got, c), ref, A=A, B=B, Cin=C, what=what, **kw)
        return
    rows, cols, blocks = sample_plan(M, N, seed=zlib.crc32(name.encode()) % 1000)
    log(f"workload {what}: oracle on {len(rows)} rows, {len(cols)} cols, {len(blocks)} blocks")
    ref_r = oracle_rows(A, B, C, rows, **kw)
    ref_c = oracle_cols(A, B, C, cols, **kw)
    got_r = _sub(got, rows, 0)
    got_c = _sub(got, cols, 1)
    if integer_twin:
        assert_bit_exact(got_r, ref_r, c, what + " rows")
        assert_bit_exact(got_c, ref_c, c, what + " cols")
    else:
        assert_within(out_as_f64(got_r, c), ref_r, A=A, B=B, Cin=C, rows=rows, what=what + " rows",
                      **kw)
        assert_within(out_as_f64(got_c, c), ref_c, A=A, B=B, Cin=C, cols=cols, what=what + " cols",
                      **kw)
    for (r0, r1, c0, c1) in blocks:
        rr, cc = list(range(r0, r1)), list(range(c0, c1))
        As = _sub(A, rr, 1 if w["ta"] else 0)
        Bs = _sub(B, cc, 0 if w["tb"] else 1)
        Cs = C[r0:r1, c0:c1].contiguous() if C is not None else None
        ref_b = oracle_full(As, Bs, Cs, **kw)
        got_b = got[r0:r1, c0:c1].contiguous()
        if integer_twin:
            assert_bit_exact(got_b, ref_b, c, what + f" block {r0},{c0}")
        else:
            assert_within(out_as_f64(got_b, c), ref_b, A=A, B=B, Cin=C, rows=rr, cols=cc,
                          what=what + f" block {r0},{c0}", **kw)
    # Integer sums are exact in C only while they fit its significand; rounding
    # is monotonic and 2^p is representable, so |C| < 2^p everywhere shows that
    # nothing was rounded.  Otherwise (e.g. bf16 C, K = 2048) the rounded
    # outputs get the tolerance form; the samples above stayed bit-exact.
    exact = integer_twin and float(got.float().abs().max()) < 2.0 ** SIGNIFICAND_BITS[c]
    log(f"workload {what}: Freivalds ({'exact' if exact else 'within the bound'})")
    freivalds_stream(got, A, B, C, exact=exact, **kw)


@pytest.mark.parametrize("integer_twin", [False, True], ids=["random", "int"])
@pytest.mark.parametrize("name", list(gi.WORKLOADS))
def test_workload(name, integer_twin):
    _check_workload(name, integer_twin)


@pytest.mark.parametrize("integer_twin", [False, True], ids=["random", "int"])
@pytest.mark.parametrize("name", [n for n, w in gi.TUNING_SHAPES.items() if w["M"] == 2048])
def test_tuned_layout_class(name, integer_twin):
    _check_workload(name, integer_twin)
