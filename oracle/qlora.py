"""The QLoRA linear layer, forward and backward, in fp64 (oracle side).

Forward ([LC] 方法与公式, the one displayed equation):

    h = dequant(W0_NF4) x + (alpha / r) B A x

written for a batch of row vectors X [M, K]:

    Y = X W_hat^T + s (X A^T) B^T,     s = alpha / r,

with W_hat [N, K] the dequantised base weight in the compute type (bf16),
A [r, K] and B [N, r] the bf16 adapters.  Backward: gradients flow through
the frozen quantised base into the adapters only; W0 itself never receives an
update ([AG] opening paragraph; [LC] 方法与公式, text under the equation;
[SB] "Quantized base plus LoRA"; [AU] Precisie box).  With dY = dL/dY:

    dX = dY W_hat + s (dY B) A
    dA = s (dY B)^T X
    dB = s dY^T (X A^T)

These are the plain derivatives of the forward; there is no dW0.

Readings: the matmul operands are the exact values of the bf16 inputs and of
the bf16 dequantised weight; everything is evaluated in fp64 without
intermediate rounding; s = fp32(alpha / r).  The SiLU-gated glue used by the
MLP configurations is not on the pages (they only name gate/up/down
projections as LoRA targets, [AG] code block); it is the textbook
silu(g) = g * sigmoid(g).
"""
from __future__ import annotations

import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r, evaluated in fp32 ([LC] 方法与公式: the alpha/r factor)."""
    return float(np.float32(alpha) / np.float32(r))


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def forward(X, W_hat, A, B, alpha: float, r: int):
    """Y = X W^T + s (X A^T) B^T in fp64.  Returns (Y, T) with T = X A^T."""
    X, W_hat, A, B = _f64(X), _f64(W_hat), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    T = X @ A.T
    Y = X @ W_hat.T + s * (T @ B.T)
    return Y, T


def backward(dY, X, W_hat, A, B, alpha: float, r: int):
    """(dX, dA, dB) of the forward above, in fp64."""
    dY, X, W_hat, A, B = _f64(dY), _f64(X), _f64(W_hat), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    U = dY @ B                     # [M, r]
    T = X @ A.T                    # [M, r]
    dX = dY @ W_hat + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def silu_mul_forward(G, Up):
    """H = silu(G) * Up, silu(g) = g * sigmoid(g)."""
    G, Up = _f64(G), _f64(Up)
    return G * _sigmoid(G) * Up


def silu_mul_backward(dH, G, Up):
    """(dG, dUp) of H = silu(G) * Up."""
    dH, G, Up = _f64(dH), _f64(G), _f64(Up)
    sg = _sigmoid(G)
    dsilu = sg * (1.0 + G * (1.0 - sg))
    return dH * Up * dsilu, dH * G * sg


def mlp_forward(X, gate, up, down):
    """Gated MLP of three QLoRA linears.  Each of gate/up/down is a dict with
    keys W_hat, A, B, alpha, r.  Returns Y and the saved activations."""
    G, _ = forward(X, gate["W_hat"], gate["A"], gate["B"], gate["alpha"], gate["r"])
    Up, _ = forward(X, up["W_hat"], up["A"], up["B"], up["alpha"], up["r"])
    H = silu_mul_forward(G, Up)
    Y, _ = forward(H, down["W_hat"], down["A"], down["B"], down["alpha"], down["r"])
    return Y, dict(G=G, Up=Up, H=H)


def mlp_backward(dY, X, saved, gate, up, down):
    """Gradients of the gated MLP: dX and (dA, dB) of each linear."""
    dH, dA_d, dB_d = backward(dY, saved["H"], down["W_hat"], down["A"], down["B"],
                              down["alpha"], down["r"])
    dG, dUp = silu_mul_backward(dH, saved["G"], saved["Up"])
    dXg, dA_g, dB_g = backward(dG, X, gate["W_hat"], gate["A"], gate["B"],
                               gate["alpha"], gate["r"])
    dXu, dA_u, dB_u = backward(dUp, X, up["W_hat"], up["A"], up["B"],
                               up["alpha"], up["r"])
    return dXg + dXu, dict(gate=(dA_g, dB_g), up=(dA_u, dB_u), down=(dA_d, dB_d))


# ---------------------------------------------------------------------------
# Merging the adapter into the dequantised base (serving path)
# ---------------------------------------------------------------------------

def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 once (round to nearest, ties to even), as
    uint16 bits.  Values are finite and normal in bf16 (|x| >= 2^-126)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)                   # 8 significant bits, half to even
    r = np.ldexp(q, e - 8)                   # exactly representable in bf16
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def merge(W_hat, A, B, alpha: float, r: int):
    """W_merged = W_hat + s B A in fp64, s = fp32(alpha / r).

    After training the adapter can be folded into the base for serving; for a
    4-bit base the base must first be dequantised, and the merged weight then
    carries the quantisation error of the base ([LC] 与 baseline 对比 table,
    row 部署合并, and 实现要点, the item on merging with care; [AU] FAQ, the
    question on inference; [SB] "Quantized base plus LoRA").  W_hat is the
    bf16 dequantised weight [N, K]; the exact result is returned (round it
    with f64_to_bf16_bits for the bf16 merged weight)."""
    W_hat, A, B = _f64(W_hat), _f64(A), _f64(B)
    return W_hat + lora_scale(alpha, r) * (B @ A)
