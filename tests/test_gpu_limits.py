"""The largest leading dimension the library accepts (2^21 elements, so a
tile's 256 rows span up to 255 x 2^23 bytes < 2^31 in the kernels' 32-bit
buffer offsets), on every input type and both storage orders of A, against
the oracle (bit-exact on integer data).  The operands live in wide device
buffers whose padding holds NaN, which a correct kernel never reads."""
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import assert_bit_exact, log, oracle_full

pytestmark = pytest.mark.gpu

MAX_LD = 1 << 21


def _wide(t: torch.Tensor, ld: int, dev):
    """Device copy of a host matrix as a view with row pitch ld (NaN padding)."""
    rows, cols = t.shape
    buf = torch.full((rows, ld), float("nan"), dtype=t.dtype, device=dev)
    buf[:, :cols].copy_(t.to(dev))
    return buf[:, :cols]


@pytest.mark.parametrize("in_dtype,c_dtype", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("ta", [False, True], ids=["A_MxK", "A_KxM"])
def test_maximum_leading_dimension(in_dtype, c_dtype, ta):
    """The planner on M = 300 (A stored K x M then has rows that are not whole
    16-byte chunks, so it takes the element-wise loads), and every forced
    256 x 256 DMA tile on M = 304, where all operands take 16-byte loads."""
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    N, K = 264, 96
    names = [mg.config_name(in_dtype, i) for i in range(mg.num_configs(in_dtype))]
    cases = [("plan", 300)] + [(n, 304) for n in names
                               if n.startswith("dma_") and "_256x256" in n and not n.endswith("_sk")]
    for name, M in cases:
        sa = (K, M) if ta else (M, K)
        A = gi.draw(*sa, "int2", 6000, in_dtype)
        B = gi.draw(K, N, "int2", 6001, in_dtype)
        C = gi.draw(M, N, "int2", 6002, c_dtype)
        ref = oracle_full(A, B, C, alpha=1.5, beta=0.5, ta=ta, tb=False, in_dtype=in_dtype, c_dtype=c_dtype)
        Ad, Bd = _wide(A, MAX_LD, dev), _wide(B, MAX_LD, dev)
        assert Ad.stride(0) == MAX_LD and Bd.stride(0) == MAX_LD
        cfg = -1 if name == "plan" else mg.config_id(in_dtype, name)
        log(f"case max ld {in_dtype}->{c_dtype} ta={ta} M={M} {name}")
        Cd = C.to(dev)
        mg.gemm(Ad, Bd, Cd, alpha=1.5, beta=0.5, trans_a=ta, config=cfg)
        torch.cuda.synchronize()
        assert_bit_exact(Cd.cpu(), ref, c_dtype, f"max ld {in_dtype} ta={ta} M={M} {name}")
        del Ad, Bd, Cd
        torch.cuda.empty_cache()


def test_leading_dimension_above_the_maximum_is_refused():
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    A = torch.zeros((4, MAX_LD + 8), dtype=torch.float16, device=dev)[:, :8]
    B = torch.zeros((8, 8), dtype=torch.float16, device=dev)
    C = torch.zeros((4, 8), dtype=torch.float16, device=dev)
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm(A, B, C)
    assert e.value.status == mg.MG_EUNSUPPORTED
