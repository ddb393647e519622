"""Pins for the CPU oracle: checks against what the mathematics and the
problem statement fix, never against the oracle itself.

The GEMM definition (C = alpha*op(A)*op(B) + beta*C, row-major) is the one in
"SGEMM CUDA代码学习" (problem definition section), "CUDA GEMM：从基础写法到工程优化"
(opening definition, section 1) and the worklog's Kernel 1.  Each pin below is
chosen so that a plausible slip in the oracle (a dropped or extra term, a
wrong sign, a swapped index, a transposed operand, a mis-rounded conversion,
a mis-read leading dimension) fails at least one of them.
"""
import itertools
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- formats --

def test_f16_widen_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.widen(bits, "f16")
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_bf16_widen_exhaustive_is_upper_half_of_fp32():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle.widen(bits.astype(np.uint16), "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_f16_round_matches_numpy_on_random_and_edges():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        np.array([0.0, -0.0, 65504.0, 65519.999, 65520.0, 65536.0, -65520.0, 1e10,
                  2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -24, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11),
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1e-30]),
    ])
    ref = x.astype(np.float16).view(np.uint16)
    got = oracle.round_to(x, "f16")
    assert np.array_equal(ref, got)


def test_bf16_round_ties_to_even_exhaustive():
    """Every midpoint between consecutive positive finite bf16 values rounds to
    the one with an even last bit; a nudge either side rounds to the nearer."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    v = oracle.widen(bits, "bf16")
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2.0  # exact in fp64
    got = oracle.round_to(mid, "bf16")
    even = np.where((bits[:-1] & 1) == 0, bits[:-1], bits[1:])
    assert np.array_equal(got, even)
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(oracle.round_to(mid - eps, "bf16"), bits[:-1])
    assert np.array_equal(oracle.round_to(mid + eps, "bf16"), bits[1:])
    # negative side mirrors the positive side
    assert np.array_equal(oracle.round_to(-mid - eps, "bf16"), bits[1:] | 0x8000)
    # overflow: halfway above the largest finite goes to +inf (0x7f80)
    big = v[-1] + (v[-1] - v[-2]) / 2.0
    assert oracle.round_to(np.array([big]), "bf16")[0] == 0x7F80


def test_bf16_round_matches_torch_for_fp32_representable_values():
    """For values that are exact in fp32, one rounding fp64->bf16 equals
    torch's fp32->bf16 rounding (nearest-even)."""
    g = torch.Generator().manual_seed(3)
    x32 = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)
    ref = x32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to(x32.numpy().astype(np.float64), "bf16")
    assert np.array_equal(ref, got)


def test_f32_round_is_single_rounding():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000)
    assert np.array_equal(oracle.round_to(x, "f32"), x.astype(np.float32))


# ------------------------------------------------------------- definition --

def _frac_gemm(opA, opB, alpha, beta, C):
    M = len(opA)
    K = len(opA[0]) if M else 0
    N = len(opB[0]) if opB else (len(C[0]) if C else 0)
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = sum((opA[i][k] * opB[k][j] for k in range(K)), Fraction(0))
            row.append(alpha * s + (beta * C[i][j] if beta != 0 else 0))
        out.append(row)
    return out


def _store(op, trans):
    """Stored row-major matrix whose op() is `op` (list of lists of Fractions)."""
    arr = np.array([[float(v) for v in r] for r in op], dtype=np.float64).reshape(len(op), -1)
    return np.ascontiguousarray(arr.T if trans else arr)


@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], repeat=2)))
def test_brute_force_tiny_shapes_exact_rationals(ta, tb):
    """All M, N, K in 0..3 with dyadic values: the fp64 oracle is exact there,
    so it must equal exact rational arithmetic element for element."""
    rnd = random.Random(11 + 2 * ta + tb)
    dy = lambda: Fraction(rnd.randint(-16, 16), 8)
    for M, N, K in itertools.product(range(4), repeat=3):
        for alpha, beta in [(Fraction(1), Fraction(0)), (Fraction(3, 2), Fraction(1, 2)),
                            (Fraction(-1, 4), Fraction(-2)), (Fraction(0), Fraction(3))]:
            opA = [[dy() for _ in range(K)] for _ in range(M)]
            opB = [[dy() for _ in range(N)] for _ in range(K)]
            C = [[dy() for _ in range(N)] for _ in range(M)]
            ref = _frac_gemm(opA, opB, alpha, beta, C)
            A = _store(opA, ta).astype(np.float32) if M * K else np.zeros((1, 1), np.float32)
            B = _store(opB, tb).astype(np.float32) if K * N else np.zeros((1, 1), np.float32)
            Cn = np.array([[float(v) for v in r] for r in C], dtype=np.float32).reshape(M, N)
            got = oracle.gemm(A, B, trans_a=ta, trans_b=tb, alpha=float(alpha),
                              beta=float(beta), C=Cn if M * N else None, M=M, N=N, K=K)
            assert got.shape == (M, N)
            for i in range(M):
                for j in range(N):
                    assert Fraction(got[i, j]) == ref[i][j], (M, N, K, i, j)


def test_hand_worked_2x3x4():
    """A small product worked by hand from the definition."""
    A = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float32)          # 2 x 3
    B = np.array([[1, 0, -1, 2], [0, 1, 1, 0], [2, -1, 0, 1]], dtype=np.float32)  # 3 x 4
    # row 0: [1+0+6, 0+2-3, -1+2+0, 2+0+3] = [7, -1, 1, 5]
    # row 1: [4+0+12, 0+5-6, -4+5+0, 8+0+6] = [16, -1, 1, 14]
    want = np.array([[7, -1, 1, 5], [16, -1, 1, 14]], dtype=np.float64)
    assert np.array_equal(oracle.gemm(A, B), want)
    Cin = np.ones((2, 4), np.float32)
    assert np.array_equal(oracle.gemm(A, B, alpha=2.0, beta=-1.0, C=Cin), 2 * want - 1)


def _int_mats(M, N, K, seed, dtype="f32"):
    A = gi.draw(M, K, "int2", seed, dtype)
    B = gi.draw(K, N, "int2", seed + 1, dtype)
    C = gi.draw(M, N, "int2", seed + 2, "f32")
    return gi.as_numpy_bits(A), gi.as_numpy_bits(B), gi.as_numpy_bits(C)


def test_identity():
    rng = np.random.default_rng(2)
    K, N = 37, 29
    I = np.eye(K, dtype=np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    Cin = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    assert np.array_equal(oracle.gemm(I, B), B.astype(np.float64))
    got = oracle.gemm(I, B, alpha=1.5, beta=0.5, C=Cin)
    assert np.array_equal(got, 1.5 * B.astype(np.float64) + 0.5 * Cin.astype(np.float64))
    # identity on the right
    A = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    assert np.array_equal(oracle.gemm(A, I), A.astype(np.float64))


def test_permutation_rows_and_columns():
    rng = np.random.default_rng(3)
    M, N, K = 23, 31, 23
    perm = rng.permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1
    B = rng.standard_normal((K, N)).astype(np.float32)
    assert np.array_equal(oracle.gemm(P, B), B[perm].astype(np.float64))
    # permutation on the right permutes columns of A
    K2 = 31
    A = rng.standard_normal((M, K2)).astype(np.float32)
    perm2 = rng.permutation(K2)
    Q = np.zeros((K2, K2), np.float32)
    Q[perm2, np.arange(K2)] = 1  # (A Q)[:, j] = A[:, perm2[j]]
    assert np.array_equal(oracle.gemm(A, Q), A[:, perm2].astype(np.float64))


def test_rank_one_closed_form():
    rng = np.random.default_rng(4)
    M, N, K = 19, 27, 41
    u = rng.integers(-3, 4, M).astype(np.float32)
    v = rng.integers(-3, 4, N).astype(np.float32)
    A = np.repeat(u[:, None], K, axis=1)  # op(A) = u 1^T
    B = np.repeat(v[None, :], K, axis=0)  # op(B) = 1 v^T
    Cin = rng.integers(-5, 6, (M, N)).astype(np.float32)
    got = oracle.gemm(A, B, alpha=1.5, beta=-0.5, C=Cin)
    want = 1.5 * K * np.outer(u, v).astype(np.float64) - 0.5 * Cin
    assert np.array_equal(got, want)
    # the transposed storage of the same operands gives the same result
    got_t = oracle.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), trans_a=True,
                        trans_b=True, alpha=1.5, beta=-0.5, C=Cin)
    assert np.array_equal(got_t, want)


def test_linearity_in_alpha_beta_integer_data():
    A, B, C = _int_mats(45, 38, 67, 500)
    base = oracle.gemm(A, B)
    for alpha, beta in [(1.5, 0.5), (-2.0, 1.0), (0.25, -3.0)]:
        got = oracle.gemm(A, B, alpha=alpha, beta=beta, C=C)
        assert np.array_equal(got, alpha * base + beta * C.astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_transpose_storage_equivalence(dtype):
    A, B, _ = _int_mats(33, 26, 51, 600, dtype)
    ref = oracle.gemm(A, B, a_dtype=dtype)
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    assert np.array_equal(oracle.gemm(A, Bt, a_dtype=dtype, trans_b=True), ref)
    assert np.array_equal(oracle.gemm(At, B, a_dtype=dtype, trans_a=True), ref)
    assert np.array_equal(oracle.gemm(At, Bt, a_dtype=dtype, trans_a=True, trans_b=True), ref)


def test_integer_data_matches_exact_integer_product():
    """Integer data: fp64 sums are exact, so the oracle equals numpy's int64 product."""
    for dtype in ["f32", "f16", "bf16"]:
        A, B, C = _int_mats(70, 90, 300, 700, dtype)
        Ai = oracle.widen(A, dtype).astype(np.int64)
        Bi = oracle.widen(B, dtype).astype(np.int64)
        want = Ai @ Bi
        assert np.array_equal(oracle.gemm(A, B, a_dtype=dtype), want.astype(np.float64))


def test_leading_dimension_padding_is_never_read():
    """Matrices that are views into wider buffers (ld > row length) whose
    padding holds huge values give the same result as contiguous copies."""
    for dtype in ["f32", "bf16"]:
        A = gi.draw(21, 13, "int2", 800, dtype, ld=20)
        B = gi.draw(13, 17, "int2", 801, dtype, ld=29)
        C = gi.draw(21, 17, "int2", 802, "f32", ld=24)
        An, Bn, Cn = gi.as_numpy_bits(A), gi.as_numpy_bits(B), gi.as_numpy_bits(C)
        got = oracle.gemm(An, Bn, a_dtype=dtype, alpha=1.5, beta=0.5, C=Cn)
        want = oracle.gemm(np.ascontiguousarray(An), np.ascontiguousarray(Bn), a_dtype=dtype,
                           alpha=1.5, beta=0.5, C=np.ascontiguousarray(Cn))
        assert np.array_equal(got, want)
        assert np.all(np.abs(got) < 1e4)


def test_beta_zero_never_reads_c_and_alpha_zero_never_reads_ab():
    A, B, C = _int_mats(9, 11, 13, 900)
    Cnan = np.full((9, 11), np.nan, np.float32)
    assert not np.isnan(oracle.gemm(A, B, beta=0.0, C=Cnan)).any()
    Anan = np.full_like(A, np.nan)
    got = oracle.gemm(Anan, B, alpha=0.0, beta=2.0, C=C)
    assert np.array_equal(got, 2.0 * C.astype(np.float64))
    # K == 0: C = beta * C_in
    got = oracle.gemm(np.zeros((9, 0), np.float32), np.zeros((0, 11), np.float32), alpha=1.0,
                      beta=-1.0, C=C, M=9, N=11, K=0)
    assert np.array_equal(got, -C.astype(np.float64))


def test_rows_slab_and_element_agree_with_full():
    rng = np.random.default_rng(5)
    A = rng.uniform(-1, 1, (40, 57)).astype(np.float32)
    B = rng.uniform(-1, 1, (57, 35)).astype(np.float32)
    C = rng.uniform(-1, 1, (40, 35)).astype(np.float32)
    full = oracle.gemm(A, B, alpha=1.5, beta=0.5, C=C)
    slab = oracle.gemm(A, B, alpha=1.5, beta=0.5, C=C, rows=(13, 29))
    assert np.array_equal(slab, full[13:29])
    for (i, j) in [(0, 0), (39, 34), (17, 5)]:
        e = oracle.element(A, B, i, j, alpha=1.5, beta=0.5, C=C)
        assert e == full[i, j]


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((64, 200)).astype(np.float32)
    B = rng.standard_normal((200, 48)).astype(np.float32)
    assert np.array_equal(oracle.gemm(A, B, threads=1), oracle.gemm(A, B, threads=7))


def test_random_fp32_within_textbook_error_of_float32_product():
    """Independent cross-check on random data: numpy's float64 matmul (a
    library routine) agrees with the oracle to fp64 rounding."""
    rng = np.random.default_rng(8)
    A = rng.uniform(-1, 1, (50, 300)).astype(np.float32)
    B = rng.uniform(-1, 1, (300, 60)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    got = oracle.gemm(A, B)
    bound = 300 * 2.0 ** -52 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64))
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], repeat=2)))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_padded_storage_every_layout_matches_exact_integer_product(ta, tb, dtype):
    """Every layout with leading dimensions larger than the stored row length
    (a transposed A stored K x M with lda > M, a transposed B stored N x K
    with ldb > K, and the plain forms), padding filled with huge values: the
    result equals the exact int64 product of the stored values, computed by
    numpy from explicit transposes of contiguous copies.  Reading lda as M
    (or ldb as K) for a transposed operand picks up the padding or the wrong
    elements and fails."""
    M, N, K = 11, 9, 14
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    A = gi.draw(*sa, "int2", 810, dtype, ld=sa[1] + 5)
    B = gi.draw(*sb, "int2", 811, dtype, ld=sb[1] + 3)
    C = gi.draw(M, N, "int2", 812, "f32", ld=N + 2)
    An, Bn, Cn = gi.as_numpy_bits(A), gi.as_numpy_bits(B), gi.as_numpy_bits(C)
    assert An.strides[0] // An.itemsize == sa[1] + 5 and Bn.strides[0] // Bn.itemsize == sb[1] + 3
    got = oracle.gemm(An, Bn, a_dtype=dtype, trans_a=ta, trans_b=tb, alpha=2.0, beta=-1.0, C=Cn)
    Ai = oracle.widen(np.ascontiguousarray(An), dtype).astype(np.int64)
    Bi = oracle.widen(np.ascontiguousarray(Bn), dtype).astype(np.int64)
    opA = np.ascontiguousarray(Ai.T) if ta else Ai
    opB = np.ascontiguousarray(Bi.T) if tb else Bi
    want = 2 * (opA @ opB) - np.ascontiguousarray(Cn).astype(np.int64)
    assert np.array_equal(got, want.astype(np.float64))


# ------------------------------------------------- tolerance norms (pins) --

def test_row_and_col_norms_closed_forms_every_storage_order():
    """row_norms / col_norms define every tolerance bound, so they are pinned
    to closed forms: a row of op(A) made of K copies of v has 2-norm |v|*sqrt(K);
    a column of op(B) made of K copies of w has |w|*sqrt(K); Pythagorean rows
    (3, 4) and (1, 2, 2) have norms 5 and 3 exactly.  Each is checked for
    both storage orders, so summing over the wrong axis, a missing square
    root or a constant factor fails."""
    K = 37
    v = np.array([1.0, -2.0, 0.5, 3.0, 0.0, -0.25], np.float32)   # M = 6 rows of op(A)
    w = np.array([2.0, -1.0, 0.125, 4.0], np.float32)              # N = 4 columns of op(B)
    opA = np.repeat(v[:, None], K, axis=1)                          # M x K
    opB = np.repeat(w[None, :], K, axis=0)                          # K x N
    for dtype, conv in (("f32", lambda x: x), ("f16", lambda x: x.astype(np.float16)),
                        ("bf16", lambda x: (x.view(np.uint32) >> 16).astype(np.uint16))):
        a = conv(opA)
        b = conv(opB)
        want_a = np.abs(v.astype(np.float64)) * np.sqrt(K)
        want_b = np.abs(w.astype(np.float64)) * np.sqrt(K)
        assert np.allclose(oracle.row_norms(a, dtype), want_a, rtol=1e-15, atol=0)
        assert np.allclose(oracle.row_norms(np.ascontiguousarray(a.T), dtype, trans=True), want_a,
                           rtol=1e-15, atol=0)
        assert np.allclose(oracle.col_norms(b, dtype), want_b, rtol=1e-15, atol=0)
        assert np.allclose(oracle.col_norms(np.ascontiguousarray(b.T), dtype, trans=True), want_b,
                           rtol=1e-15, atol=0)
    pyth = np.array([[3, 4, 0], [1, 2, 2]], np.float32)
    assert np.array_equal(oracle.row_norms(pyth, "f32"), [5.0, 3.0])
    assert np.array_equal(oracle.row_norms(np.ascontiguousarray(pyth.T), "f32", trans=True), [5.0, 3.0])
    assert np.array_equal(oracle.col_norms(np.ascontiguousarray(pyth.T), "f32"), [5.0, 3.0])
    assert np.array_equal(oracle.col_norms(pyth, "f32", trans=True), [5.0, 3.0])


def test_norms_of_padded_views_ignore_the_padding():
    """A stored matrix inside a wider buffer (padding = 1e30) has the norms of
    its contiguous copy, in both storage orders."""
    A = gi.draw(7, 5, "uniform", 820, "f32", ld=9)
    An = gi.as_numpy_bits(A)
    want_rows = np.sqrt((np.ascontiguousarray(An).astype(np.float64) ** 2).sum(axis=1))
    want_cols = np.sqrt((np.ascontiguousarray(An).astype(np.float64) ** 2).sum(axis=0))
    assert np.allclose(oracle.row_norms(An, "f32"), want_rows, rtol=1e-15, atol=0)
    assert np.allclose(oracle.col_norms(An, "f32"), want_cols, rtol=1e-15, atol=0)
    assert np.allclose(oracle.row_norms(An, "f32", trans=True), want_cols, rtol=1e-15, atol=0)
    assert np.allclose(oracle.col_norms(An, "f32", trans=True), want_rows, rtol=1e-15, atol=0)
