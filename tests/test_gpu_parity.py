"""GPU parity at oracle-sized shapes: every kernel configuration, every
storage layout and output type, integer data (bit-exact) and random data
(error bound), ragged tails, and the degenerate cases.

All GPU work goes through the C ABI (dense_gemm_12_amd -> libmgemm.so).
"""
import itertools

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import (SK_WS_BYTES, assert_bit_exact, assert_within, log, oracle_full, out_as_f64,
                         run_gpu, stored_shapes)

pytestmark = pytest.mark.gpu

LAYOUTS = list(itertools.product([False, True], repeat=2))  # (ta, tb)
C_TYPES = {"f32": ["f32"], "f16": ["f16", "f32"], "bf16": ["bf16", "f32"]}


def make(M, N, K, ta, tb, in_dtype, c_dtype, dist, seed, ld_pad=0):
    sa, sb = stored_shapes(M, N, K, ta, tb)
    A = gi.draw(*sa, dist, seed, in_dtype, ld=sa[1] + ld_pad if ld_pad else None)
    B = gi.draw(*sb, dist, seed + 1, in_dtype, ld=sb[1] + ld_pad if ld_pad else None)
    C = gi.draw(M, N, dist, seed + 2, c_dtype)
    return A, B, C


def check(M, N, K, ta, tb, in_dtype, c_dtype, *, alpha, beta, dist, seed, config=-1, ld_pad=0,
          offset=0, ldc=None, stream=None):
    what = (f"{in_dtype}->{c_dtype} ta={int(ta)} tb={int(tb)} M={M} N={N} K={K} a={alpha} "
            f"b={beta} {dist} cfg={config} pad={ld_pad} off={offset}")
    log("case " + what)
    A, B, C = make(M, N, K, ta, tb, in_dtype, c_dtype, dist, seed, ld_pad)
    got = run_gpu(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb,
                  c_dtype=c_dtype, config=config, offset_elems=offset, ldc=ldc, stream=stream)
    ref = oracle_full(A, B, C if beta != 0 else None, alpha=alpha, beta=beta, ta=ta, tb=tb,
                      in_dtype=in_dtype, c_dtype=c_dtype)
    if dist == "int2":
        assert_bit_exact(got, ref, c_dtype, what)
    else:
        assert_within(out_as_f64(got, c_dtype), ref, A=A, B=B, Cin=C, alpha=alpha, beta=beta,
                      ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype, what=what)
    return got


def test_mfma_layout_probe_identity():
    """B = I: C must equal A exactly (row/column placement of every lane)."""
    import dense_gemm_12_amd as mg
    for dt in ("f32", "f16", "bf16"):
        M, K = 96, 80
        a = torch.arange(M * K, dtype=torch.float32).reshape(M, K) % 251 - 125
        A = a.to(gi.DTYPES[dt])
        B = torch.eye(K, dtype=gi.DTYPES[dt])
        ctype = "f32"
        got = run_gpu(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype=ctype)
        assert torch.equal(got, A.float()), dt
        # identity on the left, TN storage
        got = run_gpu(torch.eye(K, dtype=gi.DTYPES[dt]), A, None, alpha=1.0, beta=0.0, ta=False,
                      tb=True, c_dtype=ctype)
        assert torch.equal(got, A.float().t()), dt
    assert mg.load() is not None


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_every_config_every_layout_integer_bit_exact(in_dtype):
    """Forced configurations.  Every configuration runs on a shape whose
    operands are 16-byte loadable but ragged against every tile; the
    all-element-load configuration also runs on an odd shape."""
    import dense_gemm_12_amd as mg
    n = mg.num_configs(in_dtype)
    for (ta, tb) in LAYOUTS:
        for c_dtype in C_TYPES[in_dtype]:
            for (M, N, K), only_elem_ab in (((296, 272, 200), False), ((300, 270, 201), True)):
                A, B, C = make(M, N, K, ta, tb, in_dtype, c_dtype, "int2", 11)
                ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, in_dtype=in_dtype,
                                  c_dtype=c_dtype)
                for cfg in range(n):
                    name = mg.config_name(in_dtype, cfg)
                    if only_elem_ab and not name.startswith("elemAB"):
                        continue
                    what = f"{name} ta={ta} tb={tb} c={c_dtype} {M}x{N}x{K}"
                    log("case " + what)
                    # stream-K configurations run only with a workspace (through gemm_ex)
                    ws = SK_WS_BYTES if name.endswith("_sk") else None
                    try:
                        got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, c_dtype=c_dtype,
                                      config=cfg, workspace_bytes=ws)
                    except mg.MgemmError as e:
                        # only the few-row tiles lack a layout: a k-major A of 64 rows
                        assert e.status == mg.MG_EUNSUPPORTED and ta and "_64x" in name, (what, e)
                        log(f"  {name}: no k-major A layout")
                        continue
                    assert_bit_exact(got, ref, c_dtype, what)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_every_config_beta_ragged_row_of_vector_and_tail_c(in_dtype):
    """beta != 0 with N % 4 != 0 inside a row pitch that allows vector C
    accesses (ldc = 272): in every tile's last column block a row mixes
    vector accesses (their C values loaded ahead of the row's stores) with
    element-wise tail accesses.  Integer data, bit-exact; the padding columns
    of C must stay untouched."""
    import dense_gemm_12_amd as mg
    M, N, K, ldc = 296, 270, 200, 272
    for c_dtype in C_TYPES[in_dtype]:
        A, B, C = make(M, N, K, False, True, in_dtype, c_dtype, "int2", 23)
        ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=True, in_dtype=in_dtype, c_dtype=c_dtype)
        for cfg in range(mg.num_configs(in_dtype)):
            name = mg.config_name(in_dtype, cfg)
            what = f"{name} TN c={c_dtype} {M}x{N}x{K} ldc={ldc}"
            log("case " + what)
            ws = SK_WS_BYTES if name.endswith("_sk") else None
            got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=True, c_dtype=c_dtype, config=cfg,
                          ldc=ldc, workspace_bytes=ws)
            assert_bit_exact(got, ref, c_dtype, what)


@pytest.mark.parametrize("in_dtype", ["f16", "bf16"])
def test_every_16bit_config_long_k_integer_bit_exact(in_dtype):
    """Forced 16-bit configurations with K from one slice to many trips
    around the deepest LDS ring (odd and even slice counts, a ragged last
    slice), in the two headline layouts (TN with 16-bit C, NN with fp32 C and
    beta = 1) and their mirror images."""
    import dense_gemm_12_amd as mg
    n = mg.num_configs(in_dtype)
    cases = [(False, True, in_dtype), (False, False, "f32"), (True, True, in_dtype), (True, False, "f32")]
    for (ta, tb, c_dtype) in cases:
        for K in (32, 64, 96, 544, 1000):
            M, N = 264, 392
            A, B, C = make(M, N, K, ta, tb, in_dtype, c_dtype, "int2", 31 + K)
            ref = oracle_full(A, B, C, alpha=1.0, beta=1.0, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
            for cfg in range(n):
                name = mg.config_name(in_dtype, cfg)
                if not name.startswith(("dma", "ws")):
                    continue
                what = f"{name} ta={ta} tb={tb} c={c_dtype} {M}x{N}x{K}"
                log("case " + what)
                ws = SK_WS_BYTES if name.endswith("_sk") else None
                try:
                    got = run_gpu(A, B, C, alpha=1.0, beta=1.0, ta=ta, tb=tb, c_dtype=c_dtype, config=cfg,
                                  workspace_bytes=ws)
                except mg.MgemmError as e:
                    assert e.status == mg.MG_EUNSUPPORTED and ta and "_64x" in name, (what, e)
                    continue
                assert_bit_exact(got, ref, c_dtype, what)


def test_forced_vector_config_refuses_unaligned_problem():
    import dense_gemm_12_amd as mg
    A, B, C = make(64, 70, 64, False, False, "f16", "f16", "int2", 12)
    with pytest.raises(mg.MgemmError) as e:
        run_gpu(A, B, C, alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype="f16",
                config=mg.config_id("f16", "mfma_f16_128x128x64_w2x2"))
    assert e.value.status == mg.MG_EUNSUPPORTED


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_random_data_within_bound(in_dtype, ta, tb):
    for c_dtype in C_TYPES[in_dtype]:
        check(517, 389, 1000, ta, tb, in_dtype, c_dtype, alpha=1.0, beta=0.0, dist="uniform",
              seed=21)
        check(264, 520, 333 if in_dtype != "f32" else 331, ta, tb, in_dtype, c_dtype, alpha=1.5,
              beta=0.5, dist="normal", seed=22)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_tail_sweep(in_dtype):
    """Dimensions around every tile and chunk boundary, including 1."""
    sizes = [1, 2, 3, 7, 8, 15, 16, 17, 31, 33, 63, 65, 127, 129, 255, 257]
    rng = np.random.default_rng(5)
    c_dtype = C_TYPES[in_dtype][0]
    for t in range(24):
        M, N, K = (int(rng.choice(sizes)) for _ in range(3))
        ta, tb = LAYOUTS[t % 4]
        check(M, N, K, ta, tb, in_dtype, c_dtype, alpha=1.0, beta=1.0, dist="int2", seed=100 + t)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_misaligned_and_padded_operands(in_dtype):
    c_dtype = C_TYPES[in_dtype][-1]
    for off in (1, 3):
        for (ta, tb) in LAYOUTS:
            check(130, 99, 75, ta, tb, in_dtype, c_dtype, alpha=1.0, beta=0.5, dist="int2",
                  seed=300 + off, offset=off)
    for (ta, tb) in LAYOUTS:
        check(200, 136, 96, ta, tb, in_dtype, c_dtype, alpha=1.5, beta=0.5, dist="int2", seed=310,
              ld_pad=8)
        check(200, 136, 96, ta, tb, in_dtype, c_dtype, alpha=1.5, beta=0.5, dist="int2", seed=311,
              ld_pad=5, ldc=141)


def test_degenerate_cases():
    # K == 0 and alpha == 0: C = beta * C, A/B not read
    for in_dtype in ("f32", "f16", "bf16"):
        c_dtype = C_TYPES[in_dtype][0]
        check(33, 65, 0, False, False, in_dtype, c_dtype, alpha=1.0, beta=-2.0, dist="int2", seed=1)
        check(33, 65, 17, False, True, in_dtype, c_dtype, alpha=0.0, beta=0.5, dist="int2", seed=2)
        # beta == 0 with NaN-filled C: NaN never propagates
        got = run_gpu(*make(70, 40, 30, False, False, in_dtype, c_dtype, "int2", 3)[:2], None,
                      alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype=c_dtype)
        assert not torch.isnan(got.float()).any()
        # alpha == 0 and beta == 0 -> zeros, even over NaN
        got = run_gpu(*make(70, 40, 30, False, False, in_dtype, c_dtype, "int2", 4)[:2], None,
                      alpha=0.0, beta=0.0, ta=False, tb=False, c_dtype=c_dtype)
        assert torch.all(got.float() == 0)


def test_empty_problems_leave_c_untouched():
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    C = torch.full((5, 7), 3.0, device=dev)
    A = torch.ones((0, 4), device=dev)
    B = torch.ones((4, 7), device=dev)
    mg.gemm(A, B, C[:0], alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


def test_non_default_stream_and_determinism():
    s = torch.cuda.Stream()
    A, B, C = make(700, 600, 512, False, True, "f16", "f16", "normal", 40)
    r1 = run_gpu(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=True, c_dtype="f16", stream=s)
    r2 = run_gpu(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=True, c_dtype="f16")
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    A, B, C = make(513, 515, 517, False, False, "f32", "f32", "uniform", 41)
    r1 = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=False, c_dtype="f32")
    r2 = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=False, tb=False, c_dtype="f32")
    assert torch.equal(r1.view(torch.int32), r2.view(torch.int32))


def test_nn_and_tn_storage_agree_bitwise():
    """The same op(B) stored K x N (NN) or N x K (TN) gives identical bits."""
    M, N, K = 384, 320, 640
    for in_dtype in ("f16", "bf16", "f32"):
        A = gi.draw(M, K, "normal", 50, in_dtype)
        B = gi.draw(K, N, "normal", 51, in_dtype)
        Bt = B.t().contiguous()
        c = C_TYPES[in_dtype][-1]
        r_nn = run_gpu(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype=c)
        r_tn = run_gpu(A, Bt, None, alpha=1.0, beta=0.0, ta=False, tb=True, c_dtype=c)
        ref = oracle_full(A, B, None, alpha=1.0, beta=0.0, ta=False, tb=False, in_dtype=in_dtype,
                          c_dtype=c)
        assert_within(out_as_f64(r_nn, c), ref, A=A, B=B, Cin=None, alpha=1.0, beta=0.0, ta=False,
                      tb=False, in_dtype=in_dtype, c_dtype=c, what="nn")
        assert torch.equal(r_nn.float(), r_tn.float()), in_dtype
