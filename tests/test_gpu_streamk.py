"""Stream-K configurations (_sk: persistent workgroups share the slice
iterations of all tiles; a tile split between workgroups is finished by the
last contributor from fp32 partials summed in k order) against the oracle,
through gemm_ex with a workspace.

Shapes are chosen so that tiles are split between two, several and many
workgroups (long K with many tiles, short K with few tiles, a ragged last
slice and ragged tile edges).  Integer data must match bit for bit; random
data must be within the bound and bitwise identical across repeated calls
(the partial sums are added in a fixed order, whichever workgroup finishes
last), also when the workspace holds stale counters and partials from an
earlier call."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import (SK_WS_BYTES, assert_bit_exact, assert_within, log, oracle_full, out_as_f64, run_gpu,
                         stored_shapes)

pytestmark = pytest.mark.gpu

SHAPES = [
    # (M, N, K): tiles x slices vs 256 workgroups
    (1024, 2816, 4096),   # 44 tiles x 64 slices: ~11 slices per workgroup, 6 contributors per tile
    (2560, 2560, 2048),   # 100 tiles x 32 slices: tiles split 2-3 ways at uneven points
    (600, 520, 333),      # ragged edges, ragged last slice, 9 tiles x 6 slices: 54 one-slice workgroups
    (4096, 4352, 1024),   # 272 tiles x 16 slices: just over one round
]


def _sk_configs(in_dtype):
    import dense_gemm_12_amd as mg
    return [i for i in range(mg.num_configs(in_dtype)) if mg.config_name(in_dtype, i).endswith("_sk")]


def _make(M, N, K, ta, tb, in_dtype, c_dtype, dist, seed):
    sa, sb = stored_shapes(M, N, K, ta, tb)
    return (gi.draw(*sa, dist, seed, in_dtype), gi.draw(*sb, dist, seed + 1, in_dtype),
            gi.draw(M, N, "uniform" if dist != "int2" else "int2", seed + 2, c_dtype))


@pytest.mark.parametrize("in_dtype,c_dtype,ta,tb", [("bf16", "f32", False, False), ("f16", "f16", False, True),
                                                     ("bf16", "bf16", True, True), ("f16", "f32", True, False)])
def test_streamk_integer_bit_exact(in_dtype, c_dtype, ta, tb):
    import dense_gemm_12_amd as mg
    cfgs = _sk_configs(in_dtype)
    assert cfgs, "no stream-K configuration built"
    for (M, N, K) in SHAPES:
        A, B, C = _make(M, N, K, ta, tb, in_dtype, c_dtype, "int2", 4000 + K)
        ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
        for cfg in cfgs:
            what = f"{mg.config_name(in_dtype, cfg)} {in_dtype}->{c_dtype} ta={ta} tb={tb} {M}x{N}x{K}"
            log("case " + what)
            got = run_gpu(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=tb, c_dtype=c_dtype, config=cfg,
                          workspace_bytes=SK_WS_BYTES)
            assert_bit_exact(got, ref, c_dtype, what)


def test_streamk_random_within_bound_and_repeatable():
    """bf16 NN with fp32 C and beta = 1 (the shape class of the
    4096 x 11008 x 4096 workload): within the bound, and bitwise identical on
    three calls with one workspace (stale counters and partials between
    calls) and with a fresh one."""
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    for (M, N, K) in SHAPES[:2]:
        A, B, C = _make(M, N, K, False, False, "bf16", "f32", "uniform", 4100 + K)
        Ad, Bd = A.to(dev), B.to(dev)
        for cfg in _sk_configs("bf16"):
            log(f"case {mg.config_name('bf16', cfg)} random {M}x{N}x{K}")
            ws = torch.empty(SK_WS_BYTES, dtype=torch.uint8, device=dev)
            outs = []
            for rep in range(4):
                if rep == 3:
                    ws = torch.full((SK_WS_BYTES,), 0x7F, dtype=torch.uint8, device=dev)
                Cd = C.to(dev)
                mg.gemm(Ad, Bd, Cd, alpha=1.0, beta=1.0, config=cfg, workspace=ws)
                torch.cuda.synchronize()
                outs.append(Cd.cpu())
            for o in outs[1:]:
                assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32)), "stream-K is not repeatable"
            ref = oracle_full(A, B, C, alpha=1.0, beta=1.0, ta=False, tb=False, in_dtype="bf16", c_dtype="f32")
            assert_within(out_as_f64(outs[0], "f32"), ref, A=A, B=B, Cin=C, alpha=1.0, beta=1.0, ta=False,
                          tb=False, in_dtype="bf16", c_dtype="f32", what=f"stream-K {M}x{N}x{K}")


def test_streamk_needs_its_workspace():
    """Forced without a workspace, or with one too small, a stream-K
    configuration is refused before anything runs; the planner given a
    small workspace falls back to another configuration."""
    import dense_gemm_12_amd as mg
    cfg = _sk_configs("bf16")[0]
    A, B, C = _make(512, 512, 512, False, False, "bf16", "f32", "int2", 4200)
    for ws in (None, 1 << 20):
        with pytest.raises(mg.MgemmError) as e:
            run_gpu(A, B, C, alpha=1.0, beta=0.0, ta=False, tb=False, c_dtype="f32", config=cfg,
                    workspace_bytes=ws)
        assert e.value.status == mg.MG_EUNSUPPORTED
