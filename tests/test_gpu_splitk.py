"""Split-K GEMM (gemm_ex with a caller workspace) against the oracle.

Integer data keeps every partial sum exact in fp32, so a split result must
equal the oracle bit for bit whatever the split; random data must stay
within the error bound and be identical on repeated runs (the partials are
summed in a fixed order).  Every configuration runs split, on every layout.
All GPU work goes through the C ABI.
"""
import itertools

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import (SK_WS_BYTES, assert_bit_exact, assert_within, bits, log, oracle_full, out_as_f64,
                         run_gpu, stored_shapes)

pytestmark = pytest.mark.gpu

LAYOUTS = list(itertools.product([False, True], repeat=2))  # (ta, tb)
C_TYPES = {"f32": ["f32"], "f16": ["f16", "f32"], "bf16": ["bf16", "f32"]}


def make(M, N, K, ta, tb, in_dtype, c_dtype, dist, seed):
    sa, sb = stored_shapes(M, N, K, ta, tb)
    return (gi.draw(*sa, dist, seed, in_dtype), gi.draw(*sb, dist, seed + 1, in_dtype),
            gi.draw(M, N, dist, seed + 2, c_dtype))


def check(M, N, K, ta, tb, in_dtype, c_dtype, *, alpha, beta, dist, seed, splits, ws_bytes=None,
          config=-1):
    what = (f"{in_dtype}->{c_dtype} ta={int(ta)} tb={int(tb)} M={M} N={N} K={K} a={alpha} "
            f"b={beta} {dist} splits={splits} cfg={config}")
    log("case " + what)
    A, B, C = make(M, N, K, ta, tb, in_dtype, c_dtype, dist, seed)
    ws = ws_bytes if ws_bytes is not None else max(splits, 1) * M * N * 4
    got = run_gpu(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb,
                  c_dtype=c_dtype, config=config, workspace_bytes=ws, splits=splits)
    ref = oracle_full(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb,
                      in_dtype=in_dtype, c_dtype=c_dtype)
    if dist == "int2":
        assert_bit_exact(got, ref, c_dtype, what)
    else:
        assert_within(out_as_f64(got, c_dtype), ref, A=A, B=B, Cin=C, alpha=alpha, beta=beta,
                      ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype, what=what)
    return got


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_every_config_split_integer_bit_exact(in_dtype):
    """Every configuration, forced to 3 K ranges, on every layout and output
    type: ragged M, N against every tile and K not a multiple of the range."""
    import dense_gemm_12_amd as mg
    for cfg in range(mg.num_configs(in_dtype)):
        name = mg.config_name(in_dtype, cfg)
        # element-load variants also take the odd shape they exist for
        shapes = [(200, 136, 520)] + ([(201, 135, 521)] if name.startswith("elemAB") else [])
        for (M, N, K) in shapes:
            for (ta, tb) in LAYOUTS:
                for c_dtype in C_TYPES[in_dtype]:
                    try:
                        # stream-K configurations ignore the split count and need their own workspace
                        check(M, N, K, ta, tb, in_dtype, c_dtype, alpha=1.5, beta=0.5, dist="int2",
                              seed=31, splits=3, config=cfg,
                              ws_bytes=SK_WS_BYTES if name.endswith("_sk") else None)
                    except mg.MgemmError as e:
                        assert e.status == mg.MG_EUNSUPPORTED, (name, e)
                        log(f"  {name}: unsupported for this layout/alignment")


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("splits", [2, 5, 16])
def test_split_counts_random_within_bound(in_dtype, splits):
    c_dtype = "f32" if in_dtype != "f16" else "f16"
    for (ta, tb) in LAYOUTS:
        check(96, 160, 1000, ta, tb, in_dtype, c_dtype, alpha=1.0, beta=0.0, dist="uniform", seed=41,
              splits=splits)


def test_split_is_deterministic_and_beta_zero_ignores_c():
    """Same arguments twice: identical bits.  beta = 0 with NaN in C and in
    the workspace on entry: no NaN comes out."""
    import dense_gemm_12_amd as mg
    M, N, K = 127, 512, 4095
    A, B, _ = make(M, N, K, False, False, "bf16", "f32", "uniform", 51)
    runs = [run_gpu(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype="f32",
                    workspace_bytes=8 * M * N * 4, splits=8) for _ in range(2)]
    assert torch.equal(runs[0].view(torch.int32), runs[1].view(torch.int32))
    assert not torch.isnan(runs[0]).any()
    ref = oracle_full(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=False, in_dtype="bf16",
                      c_dtype="f32")
    assert_within(out_as_f64(runs[0], "f32"), ref, A=A, B=B, Cin=None, alpha=1.0, beta=0.0, ta=False,
                  tb=False, in_dtype="bf16", c_dtype="f32", what="bf16 127x512x4095 split 8")
    assert mg.load() is not None


def test_auto_split_respects_small_workspace():
    """splits = 0 with room for only 2 partials must still be correct, and
    with no workspace it is the plain kernel."""
    M, N, K = 64, 256, 2048
    for ws in (0, 2 * M * N * 4, 3 * M * N * 4 - 4):
        check(M, N, K, False, True, "f16", "f16", alpha=1.0, beta=0.0, dist="int2", seed=61,
              splits=0, ws_bytes=ws)


def test_forced_split_needs_workspace():
    import dense_gemm_12_amd as mg
    M, N, K = 64, 128, 512
    with pytest.raises(mg.MgemmError) as e:
        check(M, N, K, False, False, "f32", "f32", alpha=1.0, beta=0.0, dist="int2", seed=71,
              splits=4, ws_bytes=4 * M * N * 4 - 16)
    assert e.value.status == mg.MG_EINVAL


@pytest.mark.parametrize("integer_twin", [False, True])
def test_c5b_workload_auto_split(integer_twin):
    """bf16 NN 127x4096x4095 with fp32 C and beta = 1 (odd K: A rows are not
    16-byte aligned) through the planner's split choice, against the full
    oracle."""
    import dense_gemm_12_amd as mg
    name = "bf16_nn_127x4096x4095"
    w = gi.WORKLOADS[name]
    A, B, C = gi.workload_inputs(name, integer_twin=integer_twin)
    M, N, K = w["M"], w["N"], w["K"]
    ws = mg.workspace_size(mg.MG_BF16, mg.MG_F32, mg.MG_N, mg.MG_N, M, N, K, K, N)
    log(f"case {name} int={integer_twin} workspace {ws} bytes")
    assert ws >= 2 * M * N * 4, "the planner should split this problem"
    got = run_gpu(A, B, C, alpha=w["alpha"], beta=w["beta"], ta=False, tb=False, c_dtype="f32",
                  workspace_bytes=ws, splits=0)
    ref = oracle_full(A, B, C, alpha=w["alpha"], beta=w["beta"], ta=False, tb=False,
                      in_dtype="bf16", c_dtype="f32")
    if integer_twin:
        assert_bit_exact(got, ref, "f32", name)
    else:
        assert_within(out_as_f64(got, "f32"), ref, A=A, B=B, Cin=C, alpha=w["alpha"], beta=w["beta"],
                      ta=False, tb=False, in_dtype="bf16", c_dtype="f32", what=name)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_repacked_operands_integer_bit_exact(in_dtype):
    """Operands 16-byte loads cannot read (odd contiguous extent, odd pitch,
    base off by one element) are repacked into the workspace and run on the
    vector tiles, split or not: every layout, bit-exact on integer data."""
    import dense_gemm_12_amd as mg
    c_dtype = "f32" if in_dtype != "bf16" else "bf16"
    for (M, N, K), pad, off in (((127, 256, 1023), 0, 0), ((100, 90, 301), 3, 0), ((64, 72, 200), 0, 1)):
        for (ta, tb) in LAYOUTS:
            what = f"repack {in_dtype} ta={int(ta)} tb={int(tb)} {M}x{N}x{K} pad={pad} off={off}"
            log("case " + what)
            sa, sb = stored_shapes(M, N, K, ta, tb)
            A = gi.draw(*sa, "int2", 131, in_dtype, ld=sa[1] + pad if pad else None)
            B = gi.draw(*sb, "int2", 132, in_dtype, ld=sb[1] + pad if pad else None)
            C = gi.draw(M, N, "int2", 133, c_dtype)
            es = 4 if in_dtype == "f32" else 2
            ws = (sa[0] * (sa[1] + 8) + sb[0] * (sb[1] + 8)) * es + 4096 + 16 * M * N * 4
            got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, c_dtype=c_dtype, offset_elems=off,
                          workspace_bytes=ws, splits=0)
            ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
            assert_bit_exact(got, ref, c_dtype, what)
    assert mg.load() is not None


def _bench_workspace_workloads():
    """Named workloads the benchmark runs through gemm_ex with a workspace
    (the planner would split or repack them), small enough for the full
    oracle."""
    import dense_gemm_12_amd as mg
    out = []
    for name, w in gi.WORKLOADS.items():
        if w["M"] * w["N"] * w["K"] > 3e9:
            continue
        codes = mg.DTYPE_CODES
        lda = w["M"] if w["ta"] else w["K"]
        ldb = w["K"] if w["tb"] else w["N"]
        if mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]),
                             w["M"], w["N"], w["K"], lda, ldb) > 0:
            out.append(name)
    return out


@pytest.mark.parametrize("integer_twin", [False, True], ids=["random", "int"])
@pytest.mark.parametrize("name", _bench_workspace_workloads())
def test_bench_workspace_launches(name, integer_twin):
    """Each such workload in the benchmark's launch configuration (gemm_ex,
    the planner's split count and configuration) against the full oracle."""
    import dense_gemm_12_amd as mg
    w = gi.WORKLOADS[name]
    A, B, C = gi.workload_inputs(name, integer_twin=integer_twin)
    M, N, K = w["M"], w["N"], w["K"]
    codes = mg.DTYPE_CODES
    ws = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]), M, N, K,
                           A.stride(0), B.stride(0))
    log(f"case {name} int={integer_twin} workspace {ws} bytes")
    got = run_gpu(A, B, C, alpha=w["alpha"], beta=w["beta"], ta=w["ta"], tb=w["tb"], c_dtype=w["c_dtype"],
                  workspace_bytes=ws, splits=0)
    kw = dict(alpha=w["alpha"], beta=w["beta"], ta=w["ta"], tb=w["tb"], in_dtype=w["in_dtype"],
              c_dtype=w["c_dtype"])
    ref = oracle_full(A, B, C, **kw)
    if integer_twin:
        assert_bit_exact(got, ref, w["c_dtype"], name)
    else:
        assert_within(out_as_f64(got, w["c_dtype"]), ref, A=A, B=B, Cin=C, what=name, **kw)
