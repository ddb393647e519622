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


def sample_plan(M, N, seed, n_lines=64, block=256):
    """Deterministic sample: rows and columns at random, the four corner
    blocks and the last partial tile rows/cols are all included."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n_lines, M), replace=False).tolist())
    cols = set(rng.choice(N, size=min(n_lines, N), replace=False).tolist())
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


def freivalds_stream(C: torch.Tensor, A, B, Cin, *, alpha, beta, ta, tb, in_dtype, c_dtype,
                     seed=0, exact=False, chunk=2048):
    """Freivalds check in fp64 with a +-1 vector, streaming over row chunks
    so that large operands never exist in fp64 all at once.

    ``exact``: integer data, where every fp64 quantity is an exact integer,
    so equality is required."""
    rng = np.random.default_rng(seed)
    M, N = C.shape
    K = A.shape[0] if ta else A.shape[1]
    x = rng.choice([-1.0, 1.0], size=N)
    # y = op(B) x  (K-vector), and column norms of op(B) (for the slack)
    y = np.zeros(K)
    bn2 = np.zeros(N)
    Bb = bits(B)
    for s in range(0, Bb.shape[0], chunk):
        blk = oracle.widen(Bb[s:s + chunk], in_dtype)
        if tb:   # stored N x K: rows are columns of op(B)
            y += blk.T @ x[s:s + chunk]
            bn2[s:s + chunk] += np.sum(blk * blk, axis=1)
        else:    # stored K x N
            y[s:s + chunk] = blk @ x
            bn2 += np.sum(blk * blk, axis=0)
    bsum = np.sqrt(bn2).sum()
    Ab = bits(A)
    lhs = np.zeros(M)
    rhs = np.zeros(M)
    an2 = np.zeros(M)
    Cb = bits(C.contiguous())
    for s in range(0, M, chunk):
        e = min(M, s + chunk)
        c = oracle.widen(Cb[s:e], c_dtype)
        lhs[s:e] = c @ x
    if ta:
        for s in range(0, Ab.shape[0], chunk):   # stored K x M
            blk = oracle.widen(Ab[s:s + chunk], in_dtype)
            rhs += blk.T @ y[s:s + chunk]
            an2 += np.sum(blk * blk, axis=0)
    else:
        for s in range(0, M, chunk):
            blk = oracle.widen(Ab[s:s + chunk], in_dtype)
            rhs[s:s + chunk] = blk @ y
            an2[s:s + chunk] = np.sum(blk * blk, axis=1)
    rhs *= alpha
    slack = TOL[in_dtype] * abs(alpha) * np.sqrt(an2) * bsum
    if beta != 0.0:
        Cib = bits(Cin)
        for s in range(0, M, chunk):
            ci = oracle.widen(Cib[s:s + chunk], c_dtype)
            rhs[s:s + chunk] += beta * (ci @ x)
            slack[s:s + chunk] += TOL[in_dtype] * abs(beta) * np.abs(ci).sum(axis=1)
    if exact:
        bad = np.nonzero(lhs != rhs)[0]
    else:
        bad = np.nonzero(np.abs(lhs - rhs) > slack + 1e-9 * (np.abs(rhs) + 1.0))[0]
    assert bad.size == 0, f"Freivalds failed on {bad.size} rows, first row {bad[0]}"
