"""Seeded random problems against the oracle, bit-exact on integer data:
random M, N, K (ragged against every tile), storage layouts, leading-dimension
padding, base addresses off by one element, alpha/beta and output types,
through the plain entry point (planner's choice) and through gemm_ex with a
workspace (split-K and operand repacking).  All GPU work goes through the
C ABI."""
import numpy as np
import pytest

import gemm_inputs as gi
from gpu_helpers import assert_bit_exact, log, oracle_full, run_gpu, stored_shapes

pytestmark = pytest.mark.gpu

C_TYPES = {"f32": ["f32"], "f16": ["f16", "f32"], "bf16": ["bf16", "f32"]}
ALPHAS = (1.0, 1.5, -2.0, 0.5)
BETAS = (0.0, 1.0, 0.5, -1.0)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_random_problems_bit_exact(in_dtype):
    rng = np.random.default_rng({"f32": 71, "f16": 72, "bf16": 73}[in_dtype])
    for case in range(14):
        M, N = (int(x) for x in rng.integers(1, 640, size=2))
        K = int(rng.integers(1, 900))
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        pad = int(rng.integers(0, 10)) if rng.random() < 0.5 else 0
        off = int(rng.integers(0, 2))
        alpha = float(rng.choice(ALPHAS))
        beta = float(rng.choice(BETAS))
        c_dtype = str(rng.choice(C_TYPES[in_dtype]))
        use_ws = bool(rng.integers(2))
        what = (f"{in_dtype}->{c_dtype} case {case}: {M}x{N}x{K} ta={int(ta)} tb={int(tb)} pad={pad} off={off} "
                f"a={alpha} b={beta} ws={use_ws}")
        log("case " + what)
        sa, sb = stored_shapes(M, N, K, ta, tb)
        seed = 5000 + 10 * case
        A = gi.draw(*sa, "int2", seed, in_dtype, ld=sa[1] + pad if pad else None)
        B = gi.draw(*sb, "int2", seed + 1, in_dtype, ld=sb[1] + pad if pad else None)
        C = gi.draw(M, N, "int2", seed + 2, c_dtype)
        es = 4 if in_dtype == "f32" else 2
        ws = ((sa[0] * (sa[1] + pad + 8) + sb[0] * (sb[1] + pad + 8)) * es + 4096 + 64 * M * N * 4) if use_ws \
            else None
        got = run_gpu(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb, c_dtype=c_dtype,
                      offset_elems=off, workspace_bytes=ws, splits=0)
        ref = oracle_full(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb,
                          in_dtype=in_dtype, c_dtype=c_dtype)
        assert_bit_exact(got, ref, c_dtype, what)
