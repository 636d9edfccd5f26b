"""Seeded synthetic inputs for the QLoRA linear layer (shared by tests, bench and smoke).

This module only draws random numbers and rounds them to the storage types the
layer takes (fp32 base weights, bf16 activations and adapters).  It contains none
of the method's arithmetic: no codebook, no quantisation, no matmul.  Both the
CPU oracle and the HIP path receive exactly the arrays produced here.

Distributions follow the pages' premise that weights are roughly zero-mean
normal (aigrafen "QLoRA", list item 1 on NF4; llm-compass "QLoRA", section
方法与公式, item 1).  Shapes mirror the 7B (d=4096) and 65B (d=8192) models the
pages name, with the LoRA settings r=16, alpha=32 of the pages' configuration
listings (aigrafen "QLoRA", code block; learn-interview-questions §3).

Seeds: every tensor gets its own stream,
``numpy.random.default_rng(SeedSequence([seed, cfg_id, tensor_id]))``.
N(mu, sigma) means standard deviation sigma.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# tensor ids inside one config (stable: changing them changes every input)
T_W, T_X, T_A, T_B, T_DY, T_XO = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Linear:
    """One quantised linear W0 [N, K] (out x in) with a rank-r adapter."""
    name: str
    N: int
    K: int
    r: int
    alpha: float
    w_std: float = 0.02
    outlier_frac: float = 0.0      # fraction of Student-t(3)*outlier_scale weights
    outlier_scale: float = 0.05


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    M: int
    linears: List[Linear]
    kind: str                # "linear" | "mlp" | "decoder" | "gemv"
    backward: bool = True


def workloads() -> Dict[str, Workload]:
    """The five configurations (sizes in the docstring of each entry)."""
    c1 = Workload(1, "c1_linear_256", 16,
                  [Linear("w", 256, 256, 8, 16.0)], "linear")
    c2 = Workload(2, "c2_linear_4096", 2048,
                  [Linear("w", 4096, 4096, 16, 32.0)], "linear")
    c3 = Workload(3, "c3_mlp_11008", 4096,
                  [Linear("gate", 11008, 4096, 64, 128.0),
                   Linear("up", 11008, 4096, 64, 128.0),
                   Linear("down", 4096, 11008, 64, 128.0)], "mlp")
    c4 = Workload(4, "c4_gemv_28672x8192", 16,
                  [Linear("w", 28672, 8192, 16, 32.0, w_std=0.015)], "gemv",
                  backward=False)
    mix = dict(outlier_frac=0.01, outlier_scale=0.05)
    c5 = Workload(5, "c5_decoder_8192", 4096,
                  [Linear("q", 8192, 8192, 16, 32.0, **mix),
                   Linear("k", 8192, 8192, 16, 32.0, **mix),
                   Linear("v", 8192, 8192, 16, 32.0, **mix),
                   Linear("o", 8192, 8192, 16, 32.0, **mix),
                   Linear("gate", 22016, 8192, 16, 32.0, **mix),
                   Linear("up", 22016, 8192, 16, 32.0, **mix),
                   Linear("down", 8192, 22016, 16, 32.0, **mix)], "decoder")
    return {w.name: w for w in (c1, c2, c3, c4, c5)}


def rng(seed: int, cfg_id: int, tensor_id: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_id, sub]))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even) and return the uint16 bits.

    Input preparation only: the layer's activations and adapters are bf16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight(seed: int, cfg_id: int, lin_index: int, lin: Linear) -> np.ndarray:
    """Base weight W0 [N, K] fp32."""
    g = rng(seed, cfg_id, T_W, lin_index)
    w = g.standard_normal((lin.N, lin.K), dtype=np.float32) * np.float32(lin.w_std)
    if lin.outlier_frac > 0:
        mask = g.random((lin.N, lin.K), dtype=np.float32) < lin.outlier_frac
        cnt = int(mask.sum())
        t = g.standard_t(3, size=cnt).astype(np.float32) * np.float32(lin.outlier_scale)
        w[mask] = t
    return w


def adapters(seed: int, cfg_id: int, lin_index: int, lin: Linear):
    """LoRA A [r, K] ~ U(-1/sqrt(K), 1/sqrt(K)), B [N, r] ~ N(0, 0.01), as bf16 bits."""
    ga = rng(seed, cfg_id, T_A, lin_index)
    gb = rng(seed, cfg_id, T_B, lin_index)
    lim = 1.0 / math.sqrt(lin.K)
    a = ga.uniform(-lim, lim, size=(lin.r, lin.K)).astype(np.float32)
    b = (gb.standard_normal((lin.N, lin.r), dtype=np.float32) * np.float32(0.01))
    return round_to_bf16_bits(a), round_to_bf16_bits(b)


def activations(seed: int, cfg_id: int, M: int, K: int, tensor_id: int = T_X, sub: int = 0):
    """X [M, K] ~ N(0, 1) as bf16 bits."""
    g = rng(seed, cfg_id, tensor_id, sub)
    return round_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))


def grad_output(seed: int, cfg_id: int, M: int, N: int, sub: int = 0):
    """dY [M, N] ~ N(0, 1) as bf16 bits."""
    g = rng(seed, cfg_id, T_DY, sub)
    return round_to_bf16_bits(g.standard_normal((M, N), dtype=np.float32))


def linear_case(seed: int, M: int, N: int, K: int, r: int, alpha: float,
                w_std: float = 0.02, cfg_id: int = 100, outlier_frac: float = 0.0):
    """A single linear case of arbitrary shape (for parity sweeps over odd sizes)."""
    lin = Linear("w", N, K, r, alpha, w_std=w_std, outlier_frac=outlier_frac)
    w = weight(seed, cfg_id, 0, lin)
    a, b = adapters(seed, cfg_id, 0, lin)
    x = activations(seed, cfg_id, M, K)
    dy = grad_output(seed, cfg_id, M, N)
    return dict(W=w, A=a, B=b, X=x, dY=dy, M=M, N=N, K=K, r=r, alpha=alpha)
