"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle (full, or sampled rows/columns/blocks + Freivalds).

Expected values always come from ``oracle`` on the same seeded inputs; the
GPU result is only ever the thing being checked.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gemm_inputs as gi
import oracle
from checks import TOL, within_bound

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor):
    return gi.as_numpy_bits(t)


def stored_shapes(M, N, K, ta, tb):
    return ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))


GUARD = 256  # bytes after a split-K workspace that the library must not touch
# Workspace large enough for any stream-K configuration (2 partial-tile slots
# of 256 x 256 floats per workgroup of one 256-CU round, plus tile counters).
SK_WS_BYTES = 2 * 256 * 256 * 256 * 4 + (1 << 20)


def run_gpu(A, B, Cin, *, alpha, beta, ta, tb, c_dtype, config=-1, ldc=None, stream=None,
            offset_elems=0, workspace_bytes=None, splits=0):
    """Copy host tensors to the GPU, run the library's GEMM, return C on the host.

    ``ldc`` > N places C inside a wider buffer; ``offset_elems`` shifts every
    operand's base address by that many elements (misalignment tests).
    ``workspace_bytes`` (with ``splits``) runs the split-K entry point with a
    workspace of that size, pre-filled with 0xff bytes (NaN as fp32) and
    followed by GUARD bytes that must come back untouched."""
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")

    def up(t):
        if offset_elems == 0 and t.is_contiguous():
            return t.to(dev)
        rows, cols = t.shape
        ld = t.stride(0) if rows > 1 else cols
        buf = torch.empty(offset_elems + rows * max(ld, 1) + 8, dtype=t.dtype, device=dev)
        buf.fill_(float("nan") if t.dtype != torch.int16 else 0)
        view = buf[offset_elems:offset_elems + rows * ld].view(rows, ld)[:, :cols] if rows * ld else \
            buf[offset_elems:offset_elems].view(rows, cols)
        view.copy_(t.to(dev))
        return view

    Ad, Bd = up(A), up(B)
    M = A.shape[1] if ta else A.shape[0]
    N = B.shape[0] if tb else B.shape[1]
    Cin_t = Cin if Cin is not None else torch.full((M, N), float("nan"), dtype=TORCH[c_dtype])
    Cbig = None
    if ldc is not None and ldc > N:
        # C inside a wider buffer whose extra columns hold a sentinel
        Cbig = torch.full((M, ldc), 7.0, dtype=TORCH[c_dtype])
        Cbig[:, :N] = Cin_t
        Cbig = Cbig.to(dev)
        Cd = Cbig[:, :N]
    else:
        Cd = up(Cin_t)
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())  # uploads ran on the current stream
    ws = None
    if workspace_bytes is not None:
        ws_all = torch.full((workspace_bytes + GUARD,), 0xFF, dtype=torch.uint8, device=dev)
        ws_all[workspace_bytes:] = 0xAB
        ws = ws_all[:workspace_bytes]
    mg.gemm(Ad, Bd, Cd, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb, config=config,
            stream=stream, workspace=ws, splits=splits)
    torch.cuda.synchronize()
    if ws is not None:
        assert torch.all(ws_all[workspace_bytes:] == 0xAB).item(), "GEMM wrote past its workspace"
    if Cbig is not None:
        assert torch.all(Cbig[:, N:].float() == 7.0).item(), "GEMM wrote outside C's columns"
    return Cd.cpu()


def out_as_f64(C: torch.Tensor, c_dtype: str) -> np.ndarray:
    return oracle.widen(bits(C.contiguous()), c_dtype)


def oracle_full(A, B, Cin, *, alpha, beta, ta, tb, in_dtype, c_dtype):
    return oracle.gemm(bits(A), bits(B), a_dtype=in_dtype, trans_a=ta, trans_b=tb, alpha=alpha,
                       beta=beta, C=None if Cin is None else bits(Cin), c_dtype=c_dtype,
                       M=A.shape[1] if ta else A.shape[0], N=B.shape[0] if tb else B.shape[1],
                       K=A.shape[0] if ta else A.shape[1])


def assert_bit_exact(got: torch.Tensor, ref64: np.ndarray, c_dtype: str, what: str):
    want = oracle.round_to(ref64, c_dtype)
    have = bits(got.contiguous())
    if c_dtype == "f32":
        have = have.view(np.uint32)
        want = want.view(np.uint32)
    if not np.array_equal(have, want):
        idx = np.argwhere(have != want)
        i, j = idx[0]
        raise AssertionError(f"{what}: {len(idx)} mismatches, first at ({i},{j}): "
                             f"got {out_as_f64(got, c_dtype)[i, j]!r} want {ref64[i, j]!r}")


def assert_within(got64, ref64, *, A, B, Cin, alpha, beta, ta, tb, in_dtype, c_dtype, what,
                  rows=None, cols=None):
    an = oracle.row_norms(bits(A), in_dtype, trans=ta)
    bn = oracle.col_norms(bits(B), in_dtype, trans=tb)
    if rows is not None:
        an = an[rows]
    if cols is not None:
        bn = bn[cols]
    cin = None
    if beta != 0.0 and Cin is not None:
        cin = oracle.widen(bits(Cin), c_dtype)
        if rows is not None:
            cin = cin[rows]
        if cols is not None:
            cin = cin[:, cols]
    ok, worst, idx = within_bound(got64, ref64, TOL[in_dtype], alpha, beta, an, bn, cin)
    assert ok, f"{what}: error/bound = {worst:.3g} at {idx}"
    return worst


def sample_plan(M, N, seed, n_lines=64, block=256, band=128):
    """Deterministic sample: rows and columns at random, at least one random
    row in every ``band``-row band and one random column in every
    ``band``-column band (so every tile of 128 or more rows and columns has
    sampled elements, and a tile left unwritten cannot escape the
    element-wise check), the four corner blocks and the last partial tile
    rows/cols."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n_lines, M), replace=False).tolist())
    cols = set(rng.choice(N, size=min(n_lines, N), replace=False).tolist())
    rows |= {int(rng.integers(b, min(M, b + band))) for b in range(0, M, band)}
    cols |= {int(rng.integers(b, min(N, b + band))) for b in range(0, N, band)}
    rows |= set(range(max(0, M - 3), M)) | {0}
    cols |= set(range(max(0, N - 3), N)) | {0}
    blocks = []
    for r0 in (0, max(0, M - block)):
        for c0 in (0, max(0, N - block)):
            blocks.append((r0, min(M, r0 + block), c0, min(N, c0 + block)))
    return sorted(rows), sorted(cols), blocks


def _sub(t: torch.Tensor, idx, axis):
    """Rows or columns (axis) of a stored CPU tensor as a contiguous copy."""
    idx_t = torch.as_tensor(idx, dtype=torch.long)
    return t.index_select(axis, idx_t).contiguous()


def oracle_rows(A, B, Cin, rows, *, alpha, beta, ta, tb, in_dtype, c_dtype):
    """Oracle on the rows `rows` of C (all columns)."""
    As = _sub(A, rows, 1 if ta else 0)
    Cs = _sub(Cin, rows, 0) if (beta != 0.0 and Cin is not None) else None
    return oracle_full(As, B, Cs, alpha=alpha, beta=beta, ta=ta, tb=tb, in_dtype=in_dtype,
                       c_dtype=c_dtype)


def oracle_cols(A, B, Cin, cols, *, alpha, beta, ta, tb, in_dtype, c_dtype):
    """Oracle on the columns `cols` of C (all rows)."""
    Bs = _sub(B, cols, 0 if tb else 1)
    Cs = _sub(Cin, cols, 1) if (beta != 0.0 and Cin is not None) else None
    return oracle_full(A, Bs, Cs, alpha=alpha, beta=beta, ta=ta, tb=tb, in_dtype=in_dtype,
                       c_dtype=c_dtype)


# Unit roundoff of each output type (half an ulp at 1).
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# Hoeffding multiplier: a sum sum_j e_j x_j with fixed |e_j| <= b_j and
# independent random signs x_j exceeds T * sqrt(sum_j b_j^2) with probability
# at most 2 exp(-T^2 / 2) < 3e-14 for T = 8.
HOEFFDING_T = 8.0


def freivalds_stream(C: torch.Tensor, A, B, Cin, *, alpha, beta, ta, tb, in_dtype, c_dtype,
                     seed=0, exact=False, chunk=2048, rounds=2, extra_rel=0.0, acc_terms=None):
    """Whole-matrix Freivalds check in fp64, streaming over row chunks so
    that large operands never exist in fp64 all at once.

    For random +-1 vectors x (drawn here, after C was computed, so they are
    independent of its error E = C - C_ref), (C x)_i is compared with the
    exact (alpha op(A) (op(B) x) + beta C_in x)_i.  If every |E_ij| <= b_ij,
    Hoeffding's inequality bounds |(E x)_i| by HOEFFDING_T * sqrt(sum_j b_ij^2)
    except with probability < 3e-14 per row and vector; a larger difference
    fails.  Two per-element bounds b_ij are checked:

    * the stated tolerance tol * (|alpha| |a_i| |b_j| + |beta| |C_in,ij|);
    * the worst-case rounding error of fp32 accumulation (any summation order
      of n terms is within gamma_n = n u / (1 - n u) of sum |terms|, u = 2^-24;
      Higham, Accuracy and Stability of Numerical Algorithms, section 3.1),
      bounded with Cauchy-Schwarz by gamma * (|alpha| |a_i| |b_j| +
      |beta| |C_in,ij|), plus the output rounding u_C |C_ij|.  ``acc_terms``
      is n (default K + 66: the K products, up to 64 split-K partials, alpha
      and beta, each rounded at most once); ``extra_rel`` adds an
      error relative to |a_i| |b_j| for paths that approximate the products
      (fp32 through split fp16).  This is what catches a plausible but wrong
      result (a zeroed tile, C left as C_in) when the stated tolerance is
      loose next to |C| (16-bit inputs at large K).

    ``exact``: integer data, where every fp64 quantity is an exact integer,
    so equality is required."""
    rng = np.random.default_rng(seed)
    M, N = C.shape
    K = A.shape[0] if ta else A.shape[1]
    X = rng.choice([-1.0, 1.0], size=(N, rounds))
    # Y = op(B) X (K x rounds), and the column norms of op(B)
    Y = np.zeros((K, rounds))
    bn2 = np.zeros(N)
    Bb = bits(B)
    for s in range(0, Bb.shape[0], chunk):
        blk = oracle.widen(Bb[s:s + chunk], in_dtype)
        if tb:   # stored N x K: rows are columns of op(B)
            Y += blk.T @ X[s:s + chunk]
            bn2[s:s + chunk] += np.sum(blk * blk, axis=1)
        else:    # stored K x N
            Y[s:s + chunk] = blk @ X
            bn2 += np.sum(blk * blk, axis=0)
    bn = np.sqrt(bn2)
    sum_bn, sum_bn2 = bn.sum(), bn2.sum()
    Ab = bits(A)
    lhs = np.zeros((M, rounds))
    rhs = np.zeros((M, rounds))
    an2 = np.zeros(M)
    c_abs = np.zeros(M)       # sum_j |C_ij|
    c_sq = np.zeros(M)        # sum_j C_ij^2
    Cb = bits(C.contiguous())
    for s in range(0, M, chunk):
        e = min(M, s + chunk)
        c = oracle.widen(Cb[s:e], c_dtype)
        if not np.all(np.isfinite(c)):
            bad = np.argwhere(~np.isfinite(c))[0]
            raise AssertionError(f"Freivalds: non-finite C at ({s + bad[0]}, {bad[1]})")
        lhs[s:e] = c @ X
        c_abs[s:e] = np.abs(c).sum(axis=1)
        c_sq[s:e] = (c * c).sum(axis=1)
    if ta:
        for s in range(0, Ab.shape[0], chunk):   # stored K x M
            blk = oracle.widen(Ab[s:s + chunk], in_dtype)
            rhs += blk.T @ Y[s:s + chunk]
            an2 += np.sum(blk * blk, axis=0)
    else:
        for s in range(0, M, chunk):
            blk = oracle.widen(Ab[s:s + chunk], in_dtype)
            rhs[s:s + chunk] = blk @ Y
            an2[s:s + chunk] = np.sum(blk * blk, axis=1)
    an = np.sqrt(an2)
    rhs *= alpha
    aa = abs(alpha)
    # sum_j (|alpha| a_i n_j + |beta| |cin_ij|)^2 and sum_j of the same term
    g_sq = aa * aa * an2 * sum_bn2
    g_abs = aa * an * sum_bn
    if beta != 0.0:
        Cib = bits(Cin)
        ab = abs(beta)
        for s in range(0, M, chunk):
            e = min(M, s + chunk)
            ci = oracle.widen(Cib[s:e], c_dtype)
            rhs[s:e] += beta * (ci @ X)
            cia = np.abs(ci)
            g_sq[s:e] += 2.0 * aa * ab * an[s:e] * (cia @ bn) + ab * ab * (cia * cia).sum(axis=1)
            g_abs[s:e] += ab * cia.sum(axis=1)
    diff = np.abs(lhs - rhs)
    if exact:
        bad = np.nonzero(np.any(diff != 0, axis=1))[0]
        assert bad.size == 0, f"Freivalds (exact) failed on {bad.size} rows, first row {bad[0]}"
        return
    # error of the fp64 evaluation of the check itself
    u64 = 2.0 ** -53
    eval_slack = (N + K + 8) * 2 * u64 * (g_abs + c_abs)
    stated = HOEFFDING_T * TOL[in_dtype] * np.sqrt(g_sq) + eval_slack
    bad = np.nonzero(np.any(diff > stated[:, None], axis=1))[0]
    assert bad.size == 0, (f"Freivalds (stated tolerance) failed on {bad.size} rows, first row {bad[0]}: "
                           f"|diff| {diff[bad[0]].max():.4g} > {stated[bad[0]]:.4g}")
    n = (K + 66) if acc_terms is None else acc_terms
    u = 2.0 ** -24
    gamma = n * u / (1.0 - n * u) + extra_rel
    uc = UNIT_ROUNDOFF[c_dtype] * (1.0 + 2.0 ** -10)
    # (x + y)^2 <= 2 x^2 + 2 y^2 for the two parts of the element bound
    derived = HOEFFDING_T * np.sqrt(2.0 * gamma * gamma * g_sq + 2.0 * uc * uc * c_sq) + eval_slack
    bad = np.nonzero(np.any(diff > derived[:, None], axis=1))[0]
    assert bad.size == 0, (f"Freivalds (fp32-accumulation bound) failed on {bad.size} rows, first row "
                           f"{bad[0]}: |diff| {diff[bad[0]].max():.4g} > {derived[bad[0]]:.4g}")
