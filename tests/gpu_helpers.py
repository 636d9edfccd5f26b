"""Helpers for the GPU parity tests: device transfer, oracle reference on whole
blocks or sampled rows, and the tolerance rule.

Tolerance rule for floating-point outputs (Y, T, dX, dA, dB), against the
fp64 oracle on the same bf16 inputs:
    ||got - ref||_F / ||ref||_F <= 1e-2   and   max|got - ref| <= 3e-2 * max|ref|.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_F = 1e-2
MAX_ABS = 3e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def dev_f32(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        t.bfloat16).cuda()


def host_bf16_bits(x) -> np.ndarray:
    t = torch()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def host_bf16_f64(x) -> np.ndarray:
    return oracle.bf16_bits_to_f64(host_bf16_bits(x))


def host(x) -> np.ndarray:
    return x.cpu().numpy()


def f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def metrics(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mref = np.abs(ref).max() if ref.size else 0.0
    mabs = np.abs(err).max() if err.size else 0.0
    return rel, mabs, mref


def assert_close(got, ref, name: str):
    rel, mabs, mref = metrics(got, ref)
    log(f"  {name}: relF={rel:.3e} maxerr={mabs:.3e} maxref={mref:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if mref == 0.0:
        assert mabs == 0.0, f"{name}: expected exact zeros, max err {mabs}"
        return
    assert rel <= REL_F, f"{name}: relative Frobenius error {rel:.3e} > {REL_F}"
    assert mabs <= MAX_ABS * mref, f"{name}: max error {mabs:.3e} > {MAX_ABS} * {mref:.3e}"


class OracleWeight:
    """The oracle's NF4 + double-quant view of a base weight W [N, K].

    absmax and the 8-bit constants are computed over the whole tensor (the mean
    is global); 4-bit codes and dequantised values can be produced for a subset
    of rows or of 64-column blocks, since blocks never straddle rows."""

    def __init__(self, W: np.ndarray, full: bool = True):
        self.W = np.ascontiguousarray(W, dtype=np.float32)
        self.N, self.K = W.shape
        self.kb = self.K // 64
        self.absmax = oracle.absmax_blocks(self.W, 64)
        self.codes8, self.scales, self.mean = oracle.double_quant(self.absmax, 256)
        self.a_hat = oracle.dequant_absmax(self.codes8, self.scales, self.mean, 256)
        self._full = None
        if full:
            codes4, _ = oracle.quantize_nf4(self.W, 64)
            self.codes4 = codes4
            self.packed = oracle.pack_nibbles(codes4)
            _, wb = oracle.dequant_codes(codes4, self.a_hat, 64)
            self._full = wb.reshape(self.N, self.K)

    def w_bf16(self) -> np.ndarray:
        assert self._full is not None
        return self._full

    def rows_bf16(self, rows) -> np.ndarray:
        rows = np.asarray(rows)
        if self._full is not None:
            return self._full[rows]
        sub = self.W[rows]
        c4, _ = oracle.quantize_nf4(sub, 64)
        blk = (rows[:, None] * self.kb + np.arange(self.kb)[None, :]).reshape(-1)
        _, wb = oracle.dequant_codes(c4, self.a_hat[blk], 64)
        return wb.reshape(len(rows), self.K)

    def colblocks_bf16(self, kblocks) -> np.ndarray:
        """Dequantised W[:, cols] for the 64-wide column blocks listed (all rows)."""
        kblocks = np.asarray(kblocks)
        cols = (kblocks[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        if self._full is not None:
            return self._full[:, cols]
        sub = np.ascontiguousarray(self.W[:, cols])
        c4, _ = oracle.quantize_nf4(sub, 64)
        blk = (np.arange(self.N)[:, None] * self.kb + kblocks[None, :]).reshape(-1)
        _, wb = oracle.dequant_codes(c4, self.a_hat[blk], 64)
        return wb.reshape(self.N, len(cols))


def sample_rows(M: int, count: int, seed: int = 0, tile: int = 128) -> np.ndarray:
    """Rows to check: first, last, both sides of every tile edge, then random."""
    s = {0, M - 1}
    for e in range(tile, M, tile):
        s.update({e - 1, e})
    g = np.random.default_rng(seed)
    while len(s) < min(count, M):
        s.add(int(g.integers(0, M)))
    return np.array(sorted(s))
