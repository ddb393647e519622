"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

The entry points launch only on the caller's stream and record no memset,
so a capture holds exactly their kernels.  Each case captures one call,
replays the graph several times with eager work in between (C is restored
from a copy before every replay), and requires every replay to equal the
eager call bit for bit; the eager call itself is checked against the
oracle.
"""
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import SK_WS_BYTES, assert_bit_exact, log, oracle_full

pytestmark = pytest.mark.gpu

CASES = [
    # (label, workload or shape, through gemm_ex with a workspace, forced configuration)
    ("fp16 TN 300x260x200 plain", ("f16", "f16", False, True, 300, 260, 200, 1.0, 0.0), False, None),
    ("fp32 NN 256^3 split-K", "fp32_nn_256", True, None),
    ("bf16 NN 127x4096x4095 repack + split-K", "bf16_nn_127x4096x4095", True, None),
    ("fp32 NN 190x170x160 beta=0.5 plain", ("f32", "f32", False, False, 190, 170, 160, 1.5, 0.5), False, None),
    # stream-K: a counter-zeroing kernel, then the persistent tile kernel with its last-arriver fixup
    ("bf16 NN 1024x2816x1024 beta=0.5 stream-K", ("bf16", "f32", False, False, 1024, 2816, 1024, 1.0, 0.5), True,
     "dma_bf16_256x256x64_s2_w2x4_sk"),
]


def _inputs(spec):
    if isinstance(spec, str):
        w = gi.WORKLOADS[spec]
        A, B, C = gi.workload_inputs(spec, integer_twin=True)
        return (w["in_dtype"], w["c_dtype"], w["ta"], w["tb"], w["alpha"], w["beta"], A, B, C)
    ind, cd, ta, tb, M, N, K, alpha, beta = spec
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    A = gi.draw(*sa, "int2", 61, ind)
    B = gi.draw(*sb, "int2", 62, ind)
    C = gi.draw(M, N, "int2", 63, cd) if beta != 0.0 else None
    return (ind, cd, ta, tb, alpha, beta, A, B, C)


@pytest.mark.parametrize("label,spec,use_ws,cfg_name", CASES, ids=[c[0] for c in CASES])
def test_captured_call_replays_match_eager(label, spec, use_ws, cfg_name):
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    ind, cd, ta, tb, alpha, beta, A, B, C = _inputs(spec)
    M = A.shape[1] if ta else A.shape[0]
    N = B.shape[0] if tb else B.shape[1]
    K = A.shape[0] if ta else A.shape[1]
    Ad, Bd = A.to(dev), B.to(dev)
    C0 = (C if C is not None else torch.zeros((M, N), dtype=gi.DTYPES[cd])).to(dev)
    Cd = C0.clone()
    ws = None
    cfg = -1 if cfg_name is None else mg.config_id(ind, cfg_name)
    if use_ws:
        codes = mg.DTYPE_CODES
        nbytes = (SK_WS_BYTES if cfg_name is not None else
                  mg.workspace_size(codes[ind], codes[cd], int(ta), int(tb), M, N, K, Ad.stride(0), Bd.stride(0)))
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    log(f"case {label}: eager")

    def call():
        mg.gemm(Ad, Bd, Cd, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb, workspace=ws, config=cfg)

    call()
    torch.cuda.synchronize()
    eager = Cd.clone()
    ref = oracle_full(A, B, C, alpha=alpha, beta=beta, ta=ta, tb=tb, in_dtype=ind, c_dtype=cd)
    assert_bit_exact(eager.cpu(), ref, cd, label + " (eager)")

    log(f"case {label}: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream, as torch asks
        Cd.copy_(C0)
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        Cd.copy_(C0)  # eager work between replays
        Cd.add_(0)
        torch.cuda.synchronize()
        log(f"case {label}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Cd.view(torch.int16 if Cd.element_size() == 2 else torch.int32),
                           eager.view(torch.int16 if eager.element_size() == 2 else torch.int32)), \
            f"{label}: replay {r} differs from the eager call"
