"""LoRA dropout on the adapter input (oracle side) -- TEST INFRASTRUCTURE ONLY.

Every training recipe on the pages sets ``lora_dropout=0.05`` ([AG] code
block; [LC] the code under 实现要点; [SB] "A QLoRA setup in outline";
[LI] §3, "Production QLoRA Configuration with Hugging Face PEFT").  In
the LoRA layer that setting drops elements of the input of the down
projection A only; the frozen base sees the undropped input:

    Y  = X W_hat^T + s (Xd A^T) B^T,      Xd = D(X)
    D(x) = x * scale  where the element is kept,  0 where it is dropped,
    scale = 1 / (1 - p).

Readings (the pages give only p):
  * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator,
    so that any element's draw is a pure function of (seed, element index).
    Element i of the row-major X [M, K] uses word i % 4 of
    Philox4x32-10(counter = (g mod 2^32, g div 2^32, 0, 0),
                  key = (seed mod 2^32, seed div 2^32)),  g = i div 4.
  * Keep rule: keep iff word >= t, t = floor(p * 2^32) (an exact integer
    comparison; P(drop) = t / 2^32).
  * scale = fp32(1 / (1 - p)) (the quotient in fp64, rounded once); a kept
    element is Xd = bf16(fp32(x * scale)) with round to nearest even, a dropped
    one is +0.  Xd is the bf16 tensor that feeds A, as in a framework where
    the dropout output is a tensor of the compute type.
  * Backward: the dropout is a fixed elementwise scaling of X once the mask is
    drawn, so dX picks up s (U A) * mask * scale, and dA = s U^T Xd,
    dB = s dY^T (Xd A^T).
"""
from __future__ import annotations

import numpy as np

from .nf4 import f32_to_bf16_bits
from .qlora import lora_scale, _f64

# Philox constants from the published definition: the two round multipliers
# and the two Weyl increments of the key, for 32-bit and 64-bit words.
PHILOX_M32 = (0xD2511F53, 0xCD9E8D57)
PHILOX_W32 = (0x9E3779B9, 0xBB67AE85)
PHILOX_M64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W64 = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox(ctr, key, width: int = 32, rounds: int = 10):
    """Philox4xW-R on Python integers: four counter words, two key words.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as double-width
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    The key is bumped by the Weyl constants between rounds."""
    M, Wk = (PHILOX_M32, PHILOX_W32) if width == 32 else (PHILOX_M64, PHILOX_W64)
    mask = (1 << width) - 1
    c = [int(x) & mask for x in ctr]
    k = [int(x) & mask for x in key]
    for rnd in range(rounds):
        if rnd:
            k = [(k[0] + Wk[0]) & mask, (k[1] + Wk[1]) & mask]
        p0, p1 = M[0] * c[0], M[1] * c[2]
        c = [(p1 >> width) ^ c[1] ^ k[0], p1 & mask, (p0 >> width) ^ c[3] ^ k[1], p0 & mask]
    return c


def philox4x32_words(seed: int, groups: np.ndarray) -> np.ndarray:
    """Philox4x32-10 outputs for counters (g lo, g hi, 0, 0), key = seed: the
    same round function as ``philox`` evaluated on numpy uint64 arrays (every
    product of two 32-bit words fits in 64 bits).  Returns uint32 [len, 4]."""
    g = np.asarray(groups, dtype=np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    c0, c1 = g & m32, g >> np.uint64(32)
    c2 = np.zeros_like(g)
    c3 = np.zeros_like(g)
    k0, k1 = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W32[0]) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W32[1]) & 0xFFFFFFFF
        p0 = np.uint64(PHILOX_M32[0]) * c0
        p1 = np.uint64(PHILOX_M32[1]) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & m32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & m32)
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """t = floor(p 2^32): keep iff the element's 32-bit word >= t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("p must lie in [0, 1)")
    return int(np.floor(np.float64(p) * 4294967296.0))


def dropout_scale(p: float) -> np.float32:
    """fp32(1 / (1 - p)), the fp64 quotient rounded once."""
    return np.float32(1.0 / (1.0 - np.float64(p)))


def dropout_mask(M: int, K: int, p: float, seed: int, rows=None) -> np.ndarray:
    """Keep mask (bool [len(rows), K]) of X [M, K]; ``rows`` selects rows
    (default: all).  Element (m, k) has index i = m K + k."""
    rows = np.arange(M) if rows is None else np.asarray(rows)
    idx = (rows.astype(np.int64)[:, None] * K + np.arange(K, dtype=np.int64)[None, :]).reshape(-1)
    words = philox4x32_words(seed, idx // 4)          # one generator call per element
    w = words[np.arange(idx.size), idx % 4]
    return (w.astype(np.uint64) >= np.uint64(dropout_threshold(p))).reshape(len(rows), K)


def dropout_apply(X_bits: np.ndarray, mask: np.ndarray, p: float) -> np.ndarray:
    """Xd bf16 bits: bf16(fp32(x * scale)) where kept, +0 where dropped."""
    x = (np.asarray(X_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    y = (x * dropout_scale(p)).astype(np.float32)
    out = f32_to_bf16_bits(y)
    return np.where(mask, out, np.uint16(0)).astype(np.uint16)


def pack_mask(mask: np.ndarray) -> np.ndarray:
    """Bit i % 32 of word i // 32 holds element i of the flattened mask."""
    flat = np.asarray(mask, dtype=bool).reshape(-1)
    n = -(-flat.size // 32) * 32
    bits = np.zeros(n, dtype=np.uint64)
    bits[:flat.size] = flat
    return (bits.reshape(-1, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)


def forward_dropout(X, Xd, W_hat, A, B, alpha: float, r: int):
    """Y = X W^T + s (Xd A^T) B^T in fp64; returns (Y, T = Xd A^T)."""
    X, Xd, W_hat, A, B = _f64(X), _f64(Xd), _f64(W_hat), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    T = Xd @ A.T
    return X @ W_hat.T + s * (T @ B.T), T


def backward_dropout(dY, Xd, mask, p: float, W_hat, A, B, alpha: float, r: int):
    """(dX, dA, dB) of forward_dropout with the mask held fixed, in fp64."""
    dY, Xd, W_hat, A, B = _f64(dY), _f64(Xd), _f64(W_hat), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    U = dY @ B
    keep = np.asarray(mask, dtype=np.float64) * np.float64(dropout_scale(p))
    dX = dY @ W_hat + s * (U @ A) * keep
    dA = s * (U.T @ Xd)
    dB = s * (dY.T @ (Xd @ A.T))
    return dX, dA, dB
