"""GPU parity of LoRA dropout on the adapter input: the Philox mask and the
dropped input Xd bit for bit against the oracle (integer decisions, one
bf16 rounding), and the layer's forward and backward with dropout against
the fp64 oracle under the layer's tolerances.  Shapes take the fused
forward and dX kernels, the tile-engine fallbacks (K / 64 not a multiple of
4, N not a multiple of 256) and the small-M forward; the full c2 shape is
checked on sampled tokens."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import (OracleWeight, assert_close, dev_bf16, dev_f32, f64, host,
                         host_bf16_bits, host_bf16_f64, log, sample_rows)

pytestmark = pytest.mark.gpu


def gpu_dropout(X_bits, p, seed):
    t = pytest.importorskip("torch")
    Xd, mask = q.dropout(dev_bf16(X_bits), p, seed)
    t.cuda.synchronize()
    return host_bf16_bits(Xd), host(mask).view(np.uint32)


@pytest.mark.parametrize("M,K,p,seed", [
    (1, 32, 0.05, 0), (5, 96, 0.05, 1), (130, 256, 0.05, 2**40 + 7), (64, 512, 0.5, 3),
    (33, 64, 0.9, 4), (16, 4096, 0.0, 5), (300, 1024, 0.05, 2**64 - 1)])
def test_mask_and_dropped_input_bit_exact(M, K, p, seed):
    log(f"[dropout] M={M} K={K} p={p} seed={seed}")
    X = wl.activations(seed % 1000, 31, M, K)
    Xd, words = gpu_dropout(X, p, seed)
    keep = oracle.dropout_mask(M, K, p, seed)
    assert np.array_equal(words, oracle.pack_mask(keep)), "mask"
    assert np.array_equal(Xd, oracle.dropout_apply(X, keep, p)), "Xd"


def test_mask_full_c2_bit_exact():
    M, K, p, seed = 2048, 4096, 0.05, 123456789
    X = wl.activations(0, 2, M, K)
    Xd, words = gpu_dropout(X, p, seed)
    keep = oracle.dropout_mask(M, K, p, seed)
    assert np.array_equal(words, oracle.pack_mask(keep))
    assert np.array_equal(Xd, oracle.dropout_apply(X, keep, p))
    log(f"  kept fraction {keep.mean():.5f}")


CASES = [
    # (M, N, K, r, alpha): fused fwd + fused dX; fallback dX (N % 256); fallback fwd (K / 64 = 3);
    # small-M forward (GEMV, K / 64 a multiple of 16); small-M forward generic
    (300, 512, 256, 16, 32.0),
    (200, 200, 512, 16, 32.0),
    (130, 256, 192, 8, 16.0),
    (4, 384, 1024, 16, 32.0),
    (13, 256, 320, 24, 48.0),
]


def run_case(case, p, seed, accumulate=False):
    t = pytest.importorskip("torch")
    M, K = case["M"], case["K"]
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Xd, mask = q.dropout(X, p, seed)
    Y, T = q.linear_fwd_dropout(X, Xd, qw, A, B, case["alpha"])
    acc = None
    if accumulate:
        acc = dev_bf16(wl.activations(seed % 97, 77, M, K))
        acc0 = host_bf16_f64(acc).copy()
    dX, dA, dB = q.linear_bwd_dropout(dY, Xd, mask, p, qw, A, B, case["alpha"], T=T,
                                      accumulate_into=acc)
    t.cuda.synchronize()
    out = dict(Y=host_bf16_f64(Y), T=host_bf16_f64(T), dX=host_bf16_f64(dX), dA=host(dA),
               dB=host(dB), Xd=host_bf16_bits(Xd))
    if accumulate:
        out["acc0"] = acc0
    return out


@pytest.mark.parametrize("M,N,K,r,alpha", CASES)
def test_layer_with_dropout_parity(M, N, K, r, alpha):
    p, seed = 0.05, 1000 + M
    log(f"[dropout layer] M={M} N={N} K={K} r={r}")
    case = wl.linear_case(51, M, N, K, r, alpha)
    got = run_case(case, p, seed)
    keep = oracle.dropout_mask(M, K, p, seed)
    Xd = oracle.dropout_apply(case["X"], keep, p)
    assert np.array_equal(got["Xd"], Xd)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    Yr, Tr = oracle.forward_dropout(f64(case["X"]), f64(Xd), Wh, f64(case["A"]), f64(case["B"]),
                                    alpha, r)
    dXr, dAr, dBr = oracle.backward_dropout(f64(case["dY"]), f64(Xd), keep, p, Wh, f64(case["A"]),
                                            f64(case["B"]), alpha, r)
    assert_close(got["Y"], Yr, "Y")
    assert_close(got["T"], Tr, "T")
    assert_close(got["dX"], dXr, "dX")
    assert_close(got["dA"], dAr, "dA")
    assert_close(got["dB"], dBr, "dB")
    # the mask acts on the adapter part of dX only: where an element is
    # dropped, dX equals dY W_hat there
    base = f64(case["dY"]) @ Wh
    assert_close(got["dX"][~keep], base[~keep], "dX at dropped elements")


@pytest.mark.parametrize("M,N,K,r,alpha", [CASES[0], CASES[1]])
def test_dropout_backward_accumulates(M, N, K, r, alpha):
    p, seed = 0.05, 7
    case = wl.linear_case(52, M, N, K, r, alpha)
    got = run_case(case, p, seed, accumulate=True)
    keep = oracle.dropout_mask(M, K, p, seed)
    Xd = oracle.dropout_apply(case["X"], keep, p)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    dXr, _, _ = oracle.backward_dropout(f64(case["dY"]), f64(Xd), keep, p, Wh, f64(case["A"]),
                                        f64(case["B"]), alpha, r)
    assert_close(got["dX"], got["acc0"] + dXr, "dX accumulated")


def test_p_zero_matches_the_plain_layer():
    """p = 0 keeps everything with scale 1, so Xd = X bit for bit and the
    forward, T, dA and dB equal the plain layer's bit for bit (same kernels,
    same inputs); dX adds the adapter term separately, so it agrees within
    rounding."""
    t = pytest.importorskip("torch")
    case = wl.linear_case(53, 300, 512, 256, 16, 32.0)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Xd, mask = q.dropout(X, 0.0, 9)
    Y1, T1 = q.linear_fwd_dropout(X, Xd, qw, A, B, 32.0)
    dX1, dA1, dB1 = q.linear_bwd_dropout(dY, Xd, mask, 0.0, qw, A, B, 32.0, T=T1)
    Y0, T0 = q.linear_fwd(X, qw, A, B, 32.0)
    dX0, dA0, dB0 = q.linear_bwd(dY, X, qw, A, B, 32.0, T=T0)
    t.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(Xd), case["X"])
    for a, b in ((Y1, Y0), (T1, T0)):
        assert np.array_equal(host_bf16_bits(a), host_bf16_bits(b))
    for a, b in ((dA1, dA0), (dB1, dB0)):
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))
    assert_close(host_bf16_f64(dX1), host_bf16_f64(dX0), "dX p=0")


def test_full_c2_with_dropout_sampled_tokens():
    t = pytest.importorskip("torch")
    w = wl.workloads()["c2_linear_4096"]
    lin = w.linears[0]
    M, K, N, p, seed = w.M, lin.K, lin.N, 0.05, 2024
    log(f"[dropout full] {w.name}")
    W = wl.weight(0, w.cfg_id, 0, lin)
    A, B = wl.adapters(0, w.cfg_id, 0, lin)
    X = wl.activations(0, w.cfg_id, M, K)
    dY = wl.grad_output(0, w.cfg_id, M, N)
    qw = q.quantize(dev_f32(W))
    Xg, Ag, Bg, dYg = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    Xd, mask = q.dropout(Xg, p, seed)
    Y, T = q.linear_fwd_dropout(Xg, Xd, qw, Ag, Bg, lin.alpha)
    dX, dA, dB = q.linear_bwd_dropout(dYg, Xd, mask, p, qw, Ag, Bg, lin.alpha, T=T)
    t.cuda.synchronize()
    rows = sample_rows(M, 24, seed=3, tile=256)
    keep = oracle.dropout_mask(M, K, p, seed, rows=rows)
    Xd_r = oracle.dropout_apply(X[rows], keep, p)
    assert np.array_equal(host_bf16_bits(Xd)[rows], Xd_r)
    Wh = f64(OracleWeight(W).w_bf16())
    Yr, _ = oracle.forward_dropout(f64(X[rows]), f64(Xd_r), Wh, f64(A), f64(B), lin.alpha, lin.r)
    dXr, _, _ = oracle.backward_dropout(f64(dY[rows]), f64(Xd_r), keep, p, Wh, f64(A), f64(B),
                                        lin.alpha, lin.r)
    assert_close(host_bf16_f64(Y)[rows], Yr, "Y[sampled tokens]")
    assert_close(host_bf16_f64(dX)[rows], dXr, "dX[sampled tokens]")
