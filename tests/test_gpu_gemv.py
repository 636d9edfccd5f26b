"""GPU parity of the small-M forward (M <= 16 tokens) on the shapes that take
the K-split kernel: K of 2048, 4096 or 8192 (4, 8 or 16 blocks per wave),
one to several groups of 16 rows per workgroup, ragged last row groups, the
two-block MFMA form (M <= 8) and the one-block form (9 <= M <= 16), ranks
that are and are not multiples of 16, and the dropout variant whose adapter
input differs from X.  Y and T against the fp64 oracle within
||err||_F/||ref||_F <= 1e-2 and max|err| <= 3e-2 max|ref|."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import (OracleWeight, assert_close, dev_bf16, dev_f32, f64, host_bf16_bits,
                         host_bf16_f64, log)

pytestmark = pytest.mark.gpu

CASES = [
    # (M, N, K, r, alpha)
    (1, 4360, 4096, 16, 32.0),    # two row groups per workgroup, ragged last group
    (2, 1000, 8192, 12, 16.0),    # 16 blocks per wave, one row group, ragged
    (3, 520, 2048, 1, 2.0),       # 4 blocks per wave, r = 1
    (5, 4112, 4096, 40, 80.0),    # last workgroup holds one row group
    (8, 200, 2048, 16, 32.0),     # largest M of the two-block form, 13 workgroups
    (9, 1000, 8192, 256, 512.0),  # r = 256 (beyond the split kernel's adapter tiles)
    (13, 8232, 2048, 8, 16.0),    # three row groups per workgroup
    (16, 4104, 4096, 16, 32.0),   # full one-block form
    (7, 520, 4096, 64, 128.0),    # r = 64: four adapter tiles
    (12, 1000, 2048, 24, 48.0),   # r = 24 (two tiles, the second half empty), one-block form
    (4, 200, 8192, 40, 60.0),     # r = 40, s = 1.5
]


def run(case, dropout_p=None, seed=7):
    t = pytest.importorskip("torch")
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B = (dev_bf16(case[k]) for k in ("X", "A", "B"))
    if dropout_p is None:
        Y, T = q.linear_fwd(X, qw, A, B, case["alpha"])
        Xd = None
    else:
        Xd, _ = q.dropout(X, dropout_p, seed)
        Y, T = q.linear_fwd_dropout(X, Xd, qw, A, B, case["alpha"])
    t.cuda.synchronize()
    return Y, T, Xd


@pytest.mark.parametrize("M,N,K,r,alpha", CASES)
def test_small_m_forward_parity(M, N, K, r, alpha):
    log(f"[gemv] M={M} N={N} K={K} r={r}")
    case = wl.linear_case(41, M, N, K, r, alpha)
    Y, T, _ = run(case)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    Yr, Tr = oracle.forward(f64(case["X"]), Wh, f64(case["A"]), f64(case["B"]), alpha, r)
    assert_close(host_bf16_f64(T), Tr, "T")
    assert_close(host_bf16_f64(Y), Yr, "Y")


def test_small_m_forward_with_dropout():
    M, N, K, r, alpha, p = 6, 520, 4096, 16, 32.0, 0.05
    case = wl.linear_case(42, M, N, K, r, alpha)
    Y, T, Xd = run(case, dropout_p=p)
    keep = oracle.dropout_mask(M, K, p, 7)
    Xdo = oracle.dropout_apply(case["X"], keep, p)
    assert np.array_equal(host_bf16_bits(Xd), Xdo)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    Yr, Tr = oracle.forward_dropout(f64(case["X"]), f64(Xdo), Wh, f64(case["A"]),
                                    f64(case["B"]), alpha, r)
    assert_close(host_bf16_f64(T), Tr, "T (dropped input)")
    assert_close(host_bf16_f64(Y), Yr, "Y")


def test_small_m_forward_is_deterministic():
    case = wl.linear_case(43, 4, 4112, 8192, 16, 32.0)
    a = run(case)
    b = run(case)
    assert np.array_equal(host_bf16_bits(a[0]), host_bf16_bits(b[0]))
    assert np.array_equal(host_bf16_bits(a[1]), host_bf16_bits(b[1]))
