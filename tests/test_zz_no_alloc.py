"""GPU check of qlora_linear_bwd_noalloc, the backward whose scratch memory is
a static device array instead of a caller workspace: called through the C ABI
twice in a row (the second call smaller, so it runs on what the first left in
the array), each time bit-identical to qlora_linear_bwd with a workspace on
the same inputs (the same kernels, in the same order)."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import qlora_workloads as wl
from gpu_helpers import dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu


def _noalloc(lib, dY, X, qw, A, B, alpha, T, dX, dA, dB, stream):
    M, K = X.shape
    return lib.qlora_linear_bwd_noalloc(
        dY.data_ptr(), X.data_ptr(), M, K, qw.N, qw.packed.data_ptr(), qw.codes.data_ptr(),
        qw.scales.data_ptr(), qw.mean.data_ptr(), A.data_ptr(), B.data_ptr(), A.shape[0],
        float(alpha), T.data_ptr(), dX.data_ptr(), dA.data_ptr(), dB.data_ptr(), 0, stream)


# (M, N, K, r, alpha): the first uses the once-dequantised weight copy (from
# 1024 tokens) and 16-way adapter-gradient splits; the second is smaller, with
# a rank that is padded and the 8-way split dX.
CALLS = [(1024, 2048, 2048, 16, 32.0), (100, 1024, 1024, 12, 16.0)]


def test_noalloc_backward_equals_the_workspace_backward():
    t = pytest.importorskip("torch")
    lib = q.load_library()
    for i, (M, N, K, r, alpha) in enumerate(CALLS):
        need = lib.qlora_workspace_bytes(M, K, N, r, 1)
        log(f"[noalloc] call {i}: M={M} N={N} K={K} r={r}, workspace need {need} bytes")
        assert 0 < need <= q.NOALLOC_SCRATCH_BYTES
        case = wl.linear_case(61 + i, M, N, K, r, alpha)
        qw = q.quantize(dev_f32(case["W"]))
        X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
        _, T = q.linear_fwd(X, qw, A, B, alpha)
        dX1, dA1, dB1 = q.linear_bwd(dY, X, qw, A, B, alpha, T=T)
        dX2 = t.full_like(dX1, float("nan"))
        dA2 = t.full_like(dA1, float("nan"))
        dB2 = t.full_like(dB1, float("nan"))
        stream = t.cuda.current_stream().cuda_stream
        assert _noalloc(lib, dY, X, qw, A, B, alpha, T, dX2, dA2, dB2, stream) == q.OK
        t.cuda.synchronize()
        for name, a, b in (("dX", dX1, dX2), ("dA", dA1, dA2), ("dB", dB1, dB2)):
            ab = a.contiguous().view(t.int16 if a.dtype == t.bfloat16 else t.int32).cpu().numpy()
            bb = b.contiguous().view(t.int16 if b.dtype == t.bfloat16 else t.int32).cpu().numpy()
            assert np.array_equal(ab, bb), f"call {i}: {name} differs"
