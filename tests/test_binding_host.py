"""Host-side checks of the Python binding (no GPU, nothing launched).

The kernels size their buffer ranges from the call's sizes, not from the
tensors, so the binding must refuse any tensor of the wrong dtype, shape or
layout, outputs included, before it reaches the library.  CPU tensors of the
right dtype and shape are refused too (not on a HIP device), so every case
here raises ValueError without a GPU.
"""
import pytest
import torch

import bit_nf4_quantized_07_amd as q

M, K, N, R = 16, 256, 128, 8
bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8


def _qw(N=N, K=K):
    nb = N * K // 64
    return q.QuantizedWeight(torch.zeros(N * K // 2, dtype=u8), torch.zeros(nb, dtype=u8),
                             torch.zeros((nb + 255) // 256, dtype=f32), torch.zeros(1, dtype=f32),
                             N, K)


def _args():
    return dict(X=torch.zeros(M, K, dtype=bf), qw=_qw(), A=torch.zeros(R, K, dtype=bf),
                B=torch.zeros(N, R, dtype=bf))


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_linear_fwd_refuses_bad_tensors():
    a = _args()
    f = lambda **kw: q.linear_fwd(kw.get("X", a["X"]), kw.get("qw", a["qw"]), kw.get("A", a["A"]),
                                  kw.get("B", a["B"]), 16.0, out=kw.get("out"),
                                  T_out=kw.get("T_out"))
    _raises("X: dtype", f, X=torch.zeros(M, K, dtype=torch.float16))
    _raises("A: shape", f, A=torch.zeros(R, K + 64, dtype=bf))
    _raises("B: shape", f, B=torch.zeros(N, R + 1, dtype=bf))
    _raises("B: dtype", f, B=torch.zeros(N, R, dtype=f32))
    _raises("out: shape", f, out=torch.zeros(M, N - 8, dtype=bf))
    _raises("out: dtype", f, out=torch.zeros(M, N, dtype=f32))
    _raises("T_out: shape", f, T_out=torch.zeros(M, R + 8, dtype=bf))
    _raises("X: not contiguous", f, X=torch.zeros(K, M, dtype=bf).t())
    _raises("codes: shape", f, qw=a["qw"]._replace(codes=torch.zeros(3, dtype=u8)))
    _raises("weight has K", f, qw=_qw(K=512))
    _raises("not on a CUDA", f)          # right dtypes and shapes, but host memory


def test_linear_bwd_refuses_bad_tensors():
    a = _args()
    dY = torch.zeros(M, N, dtype=bf)
    f = lambda **kw: q.linear_bwd(kw.get("dY", dY), a["X"], a["qw"], a["A"], a["B"], 16.0,
                                  T=kw.get("T"), dX_out=kw.get("dX_out"),
                                  dA_out=kw.get("dA_out"), dB_out=kw.get("dB_out"),
                                  accumulate_into=kw.get("acc"))
    _raises("dY: shape", f, dY=torch.zeros(M, N + 8, dtype=bf))
    _raises("dY: dtype", f, dY=torch.zeros(M, N, dtype=f32))
    _raises("T: shape", f, T=torch.zeros(M, R + 1, dtype=bf))
    _raises("dX: shape", f, dX_out=torch.zeros(M, K - 64, dtype=bf))
    _raises("dX: dtype", f, acc=torch.zeros(M, K, dtype=f32))
    _raises("dA: dtype", f, dA_out=torch.zeros(R, K, dtype=bf))
    _raises("dB: shape", f, dB_out=torch.zeros(N, R + 8, dtype=f32))
    _raises("not on a CUDA", f)


def test_dropout_and_mlp_refuse_bad_tensors():
    a = _args()
    X, Xd = a["X"], torch.zeros(M, K, dtype=bf)
    _raises("Xd: shape", q.dropout, X, 0.05, 1, Xd_out=torch.zeros(M, K + 64, dtype=bf))
    _raises("mask", q.dropout, X, 0.05, 1, mask_out=torch.zeros(3, dtype=torch.int32))
    _raises("mask", q.linear_bwd_dropout, torch.zeros(M, N, dtype=bf), Xd,
            torch.zeros(M * K // 32, dtype=torch.int64), 0.05, a["qw"], a["A"], a["B"], 16.0)
    _raises("Xd: dtype", q.linear_fwd_dropout, X, Xd.float(), a["qw"], a["A"], a["B"], 16.0)
    gate = (a["qw"], a["A"], a["B"], 16.0)
    up = (_qw(N=2 * N), a["A"], torch.zeros(2 * N, R, dtype=bf), 16.0)
    _raises("differ in shape", q.mlp_fwd, X, gate, up)
    _raises("A: shape", q.mlp_fwd, X, gate, (a["qw"], torch.zeros(R, 2 * K, dtype=bf), a["B"], 16.0))
    G = torch.zeros(M, N, dtype=bf)
    T = torch.zeros(M, R, dtype=bf)
    _raises("dH: shape", q.mlp_bwd, torch.zeros(M, N + 8, dtype=bf), X, gate, gate, G, G, T, T)
    _raises("Tu: shape", q.mlp_bwd, G, X, gate, gate, G, G, T, torch.zeros(M, R + 1, dtype=bf))


def test_quantize_and_merge_refuse_bad_tensors():
    a = _args()
    _raises("W: dtype", q.nf4_quantize, torch.zeros(N, K, dtype=bf))
    _raises("W: a 2-D", q.nf4_quantize, torch.zeros(N * K, dtype=f32))
    _raises("absmax: dtype", q.double_quant, torch.zeros(64, dtype=bf))
    _raises("B: shape", q.merge, a["qw"], a["A"], torch.zeros(N + 8, R, dtype=bf), 16.0)
    _raises("out: shape", q.merge, a["qw"], a["A"], a["B"], 16.0,
            out=torch.zeros(N, K + 64, dtype=bf))
    _raises("Up: shape", q.silu_mul_fwd, torch.zeros(8, 16, dtype=bf), torch.zeros(8, 24, dtype=bf))


class _FakeStream:
    def __init__(self, handle):
        self.cuda_stream = handle


def test_default_workspace_is_per_device_and_stream():
    """Calls on different streams never share scratch memory by default."""
    s1, s2 = _FakeStream(0x1000), _FakeStream(0x2000)
    w1 = q.default_workspace("cuda:0", s1)
    assert q.default_workspace("cuda:0", s1) is w1
    assert q.default_workspace("cuda:0", _FakeStream(0x1000)) is w1
    assert q.default_workspace("cuda:0", s2) is not w1
    assert q.default_workspace("cuda:1", s1) is not w1
    assert q.default_workspace(torch.device("cuda", 0), s1) is w1
