"""HIP graph capture of the layer's forward and backward.  A call of the
library makes no allocation, memset or synchronisation of its own (the
scratch memory is the caller's workspace), so a caller can capture a whole
training step of the layer in a graph (torch.cuda.graph) and replay it.  The
step is captured once and replayed three times; before each replay the
program's own eager work overwrites every output, and each replay must give
the eager step's bits."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import qlora_workloads as wl
from gpu_helpers import dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K,r", [
    (16, 256, 256, 8),      # the 16-token 256 x 256 layer
    (1, 512, 1024, 16),     # small-M forward (T partials + weight stream)
    (300, 512, 704, 40),    # tiled forward, split dX contraction, padded rank
])
def test_captured_step_replays_the_eager_bits(M, N, K, r):
    t = pytest.importorskip("torch")
    log(f"[graph] M={M} N={N} K={K} r={r}")
    alpha = 2.0 * r
    case = wl.linear_case(21, M, N, K, r, alpha)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    ws = q.Workspace("cuda")
    ws.get(max(q.workspace_bytes(M, K, N, r, b) for b in (False, True)))
    outs = dict(Y=t.empty(M, N, dtype=t.bfloat16, device="cuda"),
                T=t.empty(M, r, dtype=t.bfloat16, device="cuda"),
                dX=t.empty(M, K, dtype=t.bfloat16, device="cuda"),
                dA=t.empty(r, K, dtype=t.float32, device="cuda"),
                dB=t.empty(N, r, dtype=t.float32, device="cuda"))

    def step():
        q.linear_fwd(X, qw, A, B, alpha, out=outs["Y"], T_out=outs["T"], workspace=ws)
        q.linear_bwd(dY, X, qw, A, B, alpha, T=outs["T"], dX_out=outs["dX"], dA_out=outs["dA"],
                     dB_out=outs["dB"], workspace=ws)

    step()
    t.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):   # warm-up on the capture's kind of stream
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    t.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for k, v in outs.items():
            a = v.view(t.int16 if v.dtype == t.bfloat16 else t.int32).cpu().numpy()
            b = ref[k].view(t.int16 if v.dtype == t.bfloat16 else t.int32).cpu().numpy()
            assert np.array_equal(a, b), f"replay {rep}: {k}"
