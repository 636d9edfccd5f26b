"""GPU parity for adapter ranks that are not multiples of 8 and for scalings
s = alpha / r that are not powers of two, against the fp64 oracle.

The layer's s = alpha / r multiplies the adapter branch (llm-compass "QLoRA",
方法与公式, the equation); the pages' configurations use r = 16, alpha = 32
(s = 2), so every other test here would pass with s folded in exactly.  A
rank that is not a multiple of 8 runs on zero-padded adapter copies inside
the library; these cases check that the padding adds nothing and that T, dA
and dB come back cut to the caller's rank.  The one-hot output gradient
(dY = e_i e_j^T) reads back single rows: dX[i] = W_hat[j] + s B[j] A, every
other row of dX zero, dB row j = s T[i], dA = s B[j]^T X[i].
"""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import (OracleWeight, assert_close, dev_bf16, dev_f32, f64, host,
                         host_bf16_bits, host_bf16_f64, log)

pytestmark = pytest.mark.gpu


def run_gpu(case):
    t = pytest.importorskip("torch")
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Y, T = q.linear_fwd(X, qw, A, B, case["alpha"])
    dX, dA, dB = q.linear_bwd(dY, X, qw, A, B, case["alpha"], T=T)
    t.cuda.synchronize()
    return dict(Y=host_bf16_f64(Y), T=host_bf16_f64(T), dX=host_bf16_f64(dX),
                dA=host(dA).astype(np.float64), dB=host(dB).astype(np.float64))


def oracle_full(case, Wh=None):
    if Wh is None:
        Wh = f64(OracleWeight(case["W"]).w_bf16())
    X, A, B, dY = (f64(case[k]) for k in ("X", "A", "B", "dY"))
    Y, T = oracle.forward(X, Wh, A, B, case["alpha"], case["r"])
    dX, dA, dB = oracle.backward(dY, X, Wh, A, B, case["alpha"], case["r"])
    return dict(Y=Y, T=T, dX=dX, dA=dA, dB=dB)


CASES = [
    # (M, N, K, r, alpha): s = alpha / r
    (16, 256, 256, 1, 2.0),        # r = 1, small-M forward
    (4, 512, 1024, 4, 16.0),       # r = 4, small-M forward
    (1, 200, 192, 12, 16.0),       # r = 12 (s = 4/3), one token
    (130, 384, 320, 12, 16.0),     # r = 12 (s = 4/3), tiled, ragged tails
    (300, 512, 704, 24, 10.0),     # r = 24 (a multiple of 8, unpadded), s = 5/12
    (257, 520, 704, 3, 7.0),       # r = 3, s = 7/3, two adapter steps of padding
    (100, 4096, 4096, 12, 16.0),   # r = 12 with the 8-way split contraction
    (1024, 512, 768, 5, 9.0),      # r = 5, s = 9/5, backward on the once-dequantised weight
    (64, 256, 512, 255, 100.0),    # r = 255 (the largest rank that pads), s = 100/255
]


@pytest.mark.parametrize("M,N,K,r,alpha", CASES)
def test_rank_and_scale_parity(M, N, K, r, alpha):
    log(f"[rank] M={M} N={N} K={K} r={r} alpha={alpha} s={alpha / r:.6f}")
    case = wl.linear_case(31, M, N, K, r, alpha)
    got = run_gpu(case)
    assert got["T"].shape == (M, r) and got["dA"].shape == (r, K) and got["dB"].shape == (N, r)
    compare = oracle_full(case)
    for n in ("Y", "T", "dX", "dA", "dB"):
        assert_close(got[n], compare[n], f"r{r} {n}")


@pytest.mark.parametrize("M,r,alpha", [(8, 16, 32.0), (64, 12, 16.0), (1024, 12, 16.0)])
def test_one_hot_output_gradient_reads_back_rows(M, r, alpha):
    """dY = e_i e_j^T: dX row i is W_hat[j] + s B[j] A and every other row is
    zero; dB row j is s T[i] and every other row zero; dA = s B[j]^T X[i]."""
    t = pytest.importorskip("torch")
    N, K = 256, 512
    i, j = M // 3, 201
    case = wl.linear_case(32, M, N, K, r, alpha)
    dY = np.zeros((M, N), dtype=np.float32)
    dY[i, j] = 1.0
    case["dY"] = wl.round_to_bf16_bits(dY)
    got = run_gpu(case)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    s = oracle.lora_scale(alpha, r)
    X, A, B = f64(case["X"]), f64(case["A"]), f64(case["B"])
    others = np.arange(M) != i
    assert np.all(got["dX"][others] == 0.0), "dX rows other than i"
    assert_close(got["dX"][i], Wh[j] + s * (B[j] @ A), "dX[i]")
    rows = np.arange(N) != j
    assert np.all(got["dB"][rows] == 0.0), "dB rows other than j"
    assert_close(got["dB"][j], s * (X[i] @ A.T), "dB[j]")
    assert_close(got["dA"], s * np.outer(B[j], X[i]), "dA")
    t.cuda.synchronize()


def test_mlp_with_unpadded_and_padded_ranks_equals_the_composition():
    """Gate r = 12 and up r = 8: the MLP calls run the two padded layer calls
    and the gating, so they equal that composition bit for bit."""
    t = pytest.importorskip("torch")
    M, I, K = 40, 264, 320
    cg = wl.linear_case(33, M, I, K, 12, 16.0)
    cu = wl.linear_case(34, M, I, K, 8, 16.0)
    X = dev_bf16(cg["X"])
    dH = dev_bf16(cg["dY"])
    lin = []
    for c in (cg, cu):
        lin.append((q.quantize(dev_f32(c["W"])), dev_bf16(c["A"]), dev_bf16(c["B"]), c["alpha"]))
    G, U, H, Tg, Tu = q.mlp_fwd(X, lin[0], lin[1])
    dX, (dAg, dBg), (dAu, dBu), dG, dU = q.mlp_bwd(dH, X, lin[0], lin[1], G, U, Tg, Tu)
    G2, Tg2 = q.linear_fwd(X, *lin[0])
    U2, Tu2 = q.linear_fwd(X, *lin[1])
    H2 = q.silu_mul_fwd(G2, U2)
    dG2, dU2 = q.silu_mul_bwd(dH, G2, U2)
    dX2, dAg2, dBg2 = q.linear_bwd(dG2, X, *lin[0], T=Tg2)
    _, dAu2, dBu2 = q.linear_bwd(dU2, X, *lin[1], T=Tu2, accumulate_into=dX2)
    t.cuda.synchronize()
    for name, a, b in (("G", G, G2), ("U", U, U2), ("H", H, H2), ("Tg", Tg, Tg2),
                       ("Tu", Tu, Tu2), ("dG", dG, dG2), ("dU", dU, dU2), ("dX", dX, dX2)):
        assert np.array_equal(host_bf16_bits(a), host_bf16_bits(b)), name
    for name, a, b in (("dAg", dAg, dAg2), ("dBg", dBg, dBg2), ("dAu", dAu, dAu2),
                       ("dBu", dBu, dBu2)):
        assert np.array_equal(host(a), host(b)), name


def test_dropout_layer_with_rank_4():
    t = pytest.importorskip("torch")
    M, N, K, r, alpha, p, seed = 70, 256, 320, 4, 10.0, 0.05, 123
    case = wl.linear_case(35, M, N, K, r, alpha)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Xd, mask = q.dropout(X, p, seed)
    Y, T = q.linear_fwd_dropout(X, Xd, qw, A, B, alpha)
    dX, dA, dB = q.linear_bwd_dropout(dY, Xd, mask, p, qw, A, B, alpha, T=T)
    t.cuda.synchronize()
    keep = oracle.dropout_mask(M, K, p, seed)
    Xdo = oracle.dropout_apply(case["X"], keep, p)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    Yr, Tr = oracle.forward_dropout(f64(case["X"]), f64(Xdo), Wh, f64(case["A"]), f64(case["B"]),
                                    alpha, r)
    dXr, dAr, dBr = oracle.backward_dropout(f64(case["dY"]), f64(Xdo), keep, p, Wh,
                                            f64(case["A"]), f64(case["B"]), alpha, r)
    for n, g, ref in (("Y", host_bf16_f64(Y), Yr), ("T", host_bf16_f64(T), Tr),
                      ("dX", host_bf16_f64(dX), dXr), ("dA", host(dA), dAr),
                      ("dB", host(dB), dBr)):
        assert_close(g, ref, f"dropout r4 {n}")


@pytest.mark.parametrize("r,alpha", [(12, 16.0), (1, 3.0)])
def test_merge_with_unaligned_rank(r, alpha):
    """B [N, r] rows are not 16-byte aligned when r % 8 != 0."""
    from test_gpu_merge import check_merge
    t = pytest.importorskip("torch")
    case = wl.linear_case(36, 16, 136, 320, r, alpha)
    qw = q.quantize(dev_f32(case["W"]))
    out = q.merge(qw, dev_bf16(case["A"]), dev_bf16(case["B"]), alpha)
    t.cuda.synchronize()
    check_merge(host_bf16_bits(out), OracleWeight(case["W"]).w_bf16(), case["A"], case["B"],
                alpha, r, f"merge r{r}")
