"""GPU parity of the layer with an unquantised bf16 base weight
(qlora_linear_fwd_bf16 / qlora_linear_bwd_bf16) against the fp64 oracle with
W_hat = W: the forward on the dX kernel's forward form, the backward on the
same kernels as the NF4 weight with the dequantisation switched off, and the
tile engine for the shapes they do not take.  Tolerances as for the NF4
layer: ||err||_F / ||ref||_F <= 1e-2 and max|err| <= 3e-2 max|ref|."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import assert_close, dev_bf16, f64, host, host_bf16_f64, log

pytestmark = pytest.mark.gpu

CASES = [
    # (M, N, K, r, alpha)
    (16, 256, 256, 8, 16.0),
    (5, 200, 192, 16, 32.0),      # small M, ragged N: tile engine for both GEMMs
    (130, 384, 320, 64, 128.0),   # forward on the tile engine (K / 64 = 5)
    (300, 512, 704, 40, 80.0),    # dX kernel, ragged M, K % 128 == 64
    (520, 264, 768, 72, 144.0),   # forward kernel, ragged M and N
    (272, 768, 1280, 136, 272.0), # both dedicated kernels, r > 128
]


@pytest.mark.parametrize("M,N,K,r,alpha", CASES)
def test_linear_bf16_parity(M, N, K, r, alpha):
    t = pytest.importorskip("torch")
    log(f"[bf16 linear] M={M} N={N} K={K} r={r}")
    case = wl.linear_case(31, M, N, K, r, alpha)
    Wb = wl.round_to_bf16_bits(case["W"])
    X, A, B, dY, W = (dev_bf16(v) for v in (case["X"], case["A"], case["B"], case["dY"], Wb))
    Y, T = q.linear_fwd(X, W, A, B, alpha)
    dX, dA, dB = q.linear_bwd(dY, X, W, A, B, alpha, T=T)
    t.cuda.synchronize()
    Wh = f64(Wb)
    Xf, Af, Bf, dYf = (f64(case[k]) for k in ("X", "A", "B", "dY"))
    Yr, Tr = oracle.forward(Xf, Wh, Af, Bf, alpha, r)
    dXr, dAr, dBr = oracle.backward(dYf, Xf, Wh, Af, Bf, alpha, r)
    assert_close(host_bf16_f64(Y), Yr, "Y")
    assert_close(host_bf16_f64(T), Tr, "T")
    assert_close(host_bf16_f64(dX), dXr, "dX")
    assert_close(host(dA).astype(np.float64), dAr, "dA")
    assert_close(host(dB).astype(np.float64), dBr, "dB")


@pytest.mark.parametrize("M", [300, 2100])
def test_bf16_weight_equal_to_dequantised_nf4_gives_same_bits(M):
    """Feeding the bf16 path the dequantised NF4 weight must give exactly what
    the NF4 path computes in the backward, where both run the same kernels
    (the NF4 path decoding inside its tiles at 300 tokens, into a bf16 copy
    first at 2100), and the same T.  The forwards run different kernels (NF4:
    decode in registers; bf16: the dX kernel's forward form), whose
    contraction orders differ: Y agrees within the layer's tolerance."""
    t = pytest.importorskip("torch")
    case = wl.linear_case(32, M, 512, 1024, 16, 32.0)
    qw = q.quantize(t.from_numpy(case["W"]).cuda())
    Wd = q.nf4_dequant(qw)
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Yq, Tq = q.linear_fwd(X, qw, A, B, 32.0)
    Yb, Tb = q.linear_fwd(X, Wd, A, B, 32.0)
    dXq, dAq, dBq = q.linear_bwd(dY, X, qw, A, B, 32.0, T=Tq)
    dXb, dAb, dBb = q.linear_bwd(dY, X, Wd, A, B, 32.0, T=Tb)
    t.cuda.synchronize()
    assert_close(host_bf16_f64(Yb), host_bf16_f64(Yq), "Y")
    for n, a, b in (("T", Tq, Tb), ("dX", dXq, dXb), ("dA", dAq, dAb), ("dB", dBq, dBb)):
        assert t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a,
                       b.view(t.int16) if b.dtype == t.bfloat16 else b), n
