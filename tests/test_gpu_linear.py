"""GPU parity of the QLoRA linear layer (forward and backward) against the fp64
oracle, within  ||err||_F/||ref||_F <= 1e-2  and  max|err| <= 3e-2 max|ref|.

Shapes span several tiles with ragged tails in every dimension; the small-M
(GEMV) path and the tiled path are both covered; the full-size configurations
are checked on sampled rows (Y, dX) and completely (dA, dB)."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import (OracleWeight, assert_close, dev_bf16, dev_f32, f64, host,
                         host_bf16_f64, log, metrics, sample_rows)

pytestmark = pytest.mark.gpu


def run_gpu(case, T_saved=True, need_dX=True):
    t = pytest.importorskip("torch")
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Y, T = q.linear_fwd(X, qw, A, B, case["alpha"], save_T=True)
    dX, dA, dB = q.linear_bwd(dY, X, qw, A, B, case["alpha"], T=T if T_saved else None,
                              need_dX=need_dX)
    t.cuda.synchronize()
    return dict(Y=host_bf16_f64(Y), T=host_bf16_f64(T), dX=None if dX is None else host_bf16_f64(dX),
                dA=host(dA).astype(np.float64), dB=host(dB).astype(np.float64))


def oracle_full(case):
    ow = OracleWeight(case["W"])
    Wh = f64(ow.w_bf16())
    X, A, B, dY = (f64(case[k]) for k in ("X", "A", "B", "dY"))
    Y, T = oracle.forward(X, Wh, A, B, case["alpha"], case["r"])
    dX, dA, dB = oracle.backward(dY, X, Wh, A, B, case["alpha"], case["r"])
    return dict(Y=Y, T=T, dX=dX, dA=dA, dB=dB)


def compare(got, ref, tag, names=("Y", "T", "dX", "dA", "dB")):
    for n in names:
        if got.get(n) is not None:
            assert_close(got[n], ref[n], f"{tag} {n}")


CASES = [
    # (M, N, K, r, alpha)
    (16, 256, 256, 8, 16.0),      # configuration 1
    (1, 8, 64, 8, 16.0),          # smallest legal
    (5, 200, 192, 16, 32.0),      # GEMV path, ragged N
    (17, 264, 576, 24, 24.0),     # first tiled M, ragged everything
    (100, 136, 128, 8, 8.0),
    (130, 384, 320, 64, 128.0),   # two M tiles, ragged tail
    (257, 520, 704, 136, 272.0),  # r > 128: two adapter tiles
    (384, 1024, 1024, 16, 32.0),
    # shapes that take the dedicated forward / dX kernels with ragged edges
    (520, 264, 768, 72, 144.0),   # forward kernel: ragged M and N, r = 72
    (300, 512, 704, 40, 80.0),    # dX kernel: ragged M, K % 128 == 64
    (272, 768, 1280, 136, 272.0), # both kernels, r = 136 (nine adapter steps)
    # few tiles: both kernels split the contraction 8 ways (fp32 partials and
    # the fixed-order reduce)
    (100, 4096, 4096, 16, 32.0),
]


@pytest.mark.parametrize("M,N,K,r,alpha", CASES)
def test_linear_parity(M, N, K, r, alpha):
    log(f"[linear] M={M} N={N} K={K} r={r} alpha={alpha}")
    case = wl.linear_case(7, M, N, K, r, alpha)
    got = run_gpu(case)
    ref = oracle_full(case)
    compare(got, ref, f"M{M}N{N}K{K}r{r}")


def test_config1_adapter_term_is_significant():
    """The adapter term must matter at the tolerance: dropping it fails the check
    (otherwise the parity test could not see a broken LoRA path)."""
    w = wl.workloads()["c1_linear_256"]
    lin = w.linears[0]
    case = dict(W=wl.weight(0, 1, 0, lin), X=wl.activations(0, 1, w.M, lin.K),
                dY=wl.grad_output(0, 1, w.M, lin.N), r=lin.r, alpha=lin.alpha)
    case["A"], case["B"] = wl.adapters(0, 1, 0, lin)
    ref = oracle_full(case)
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    base = f64(case["X"]) @ Wh.T
    rel, _, _ = metrics(base, ref["Y"])
    log(f"  adapter share of ||Y||: {rel:.3e}")
    assert rel > 3 * 1e-2
    got = run_gpu(case)
    compare(got, ref, "config1")


def test_saved_T_or_recomputed_give_same_bits():
    case = wl.linear_case(3, 130, 256, 512, 16, 32.0)
    a = run_gpu(case, T_saved=True)
    b = run_gpu(case, T_saved=False)
    for n in ("dX", "dA", "dB"):
        assert np.array_equal(a[n], b[n]), n


def test_backward_is_deterministic():
    case = wl.linear_case(4, 300, 512, 1024, 16, 32.0)
    a, b = run_gpu(case), run_gpu(case)
    for n in ("Y", "dX", "dA", "dB"):
        assert np.array_equal(a[n], b[n]), n


def test_special_cases():
    """B = 0: Y is the base product alone and dA = 0.  A = 0: dB = 0, T = 0."""
    for M in (4, 64):
        case = wl.linear_case(5, M, 128, 256, 16, 32.0)
        c0 = dict(case, B=np.zeros_like(case["B"]))
        got, ref = run_gpu(c0), oracle_full(c0)
        compare(got, ref, f"B=0 M{M}", names=("Y", "dX", "dB"))
        assert np.all(got["dA"] == 0)
        c1 = dict(case, A=np.zeros_like(case["A"]))
        got, ref = run_gpu(c1), oracle_full(c1)
        compare(got, ref, f"A=0 M{M}", names=("Y", "dX", "dA"))
        assert np.all(got["dB"] == 0) and np.all(got["T"] == 0)


@pytest.mark.parametrize("K", [128, 256])
def test_identity_input_reads_weight_layout(K):
    """X = I (M = K): Y = W_hat^T + s (B A)^T, checked element-wise.  K = 256
    takes the dedicated forward kernel (permuted contraction order)."""
    N = K
    case = wl.linear_case(6, K, N, K, 16, 32.0)
    eye = np.eye(K, dtype=np.float32)
    case["X"] = wl.round_to_bf16_bits(eye)
    got, ref = run_gpu(case), oracle_full(case)
    compare(got, ref, "X=I", names=("Y",))


def test_accumulate_dx():
    t = pytest.importorskip("torch")
    case = wl.linear_case(8, 64, 256, 512, 16, 32.0)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    base = dev_bf16(wl.activations(9, 100, 64, 512))
    acc = base.clone()
    q.linear_bwd(dY, X, qw, A, B, 32.0, accumulate_into=acc)
    dX, _, _ = q.linear_bwd(dY, X, qw, A, B, 32.0)
    t.cuda.synchronize()
    want = host_bf16_f64(base) + host_bf16_f64(dX)
    assert_close(host_bf16_f64(acc), want, "accumulated dX")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_matches_tiled_path(M):
    """The small-M path and the tiled path agree (both against the oracle)."""
    case = wl.linear_case(10, M, 512, 1024, 16, 32.0)
    ref = oracle_full(case)
    got = run_gpu(case)
    compare(got, ref, f"gemv M{M}", names=("Y", "T"))
    # same rows embedded in a batch of 32 go through the tiled path
    big = dict(case)
    big["X"] = np.concatenate([case["X"], wl.activations(11, 100, 32 - M, 1024)])
    big["dY"] = np.concatenate([case["dY"], wl.grad_output(11, 100, 32 - M, 512)])
    gb = run_gpu(big)
    assert_close(gb["Y"][:M], ref["Y"], f"tiled rows M{M}")


@pytest.mark.parametrize("N,K", [(512, 768), (1024, 320)])
def test_dequant_once_dx_equals_in_tile_decode(N, K):
    """From 1024 tokens the backward dequantises the weight once and runs the
    dX kernel on the bf16 copy; below, every tile decodes the NF4 bytes.  dX
    rows depend on their own dY row only, so the first 512 rows of a
    1024-token backward must equal a 512-token backward of those rows bit for
    bit (dA, dB sum over tokens and differ).  At these shapes both token
    counts split the contraction over N into the same ranges (4 steps of 64),
    so the sums run in the same order."""
    t = pytest.importorskip("torch")
    case = wl.linear_case(12, 1024, N, K, 16, 32.0)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    for mask_p in (None, 0.05):
        if mask_p is None:
            dX_big, _, _ = q.linear_bwd(dY, X, qw, A, B, 32.0)
            dX_small, _, _ = q.linear_bwd(dY[:512].contiguous(), X[:512].contiguous(), qw, A, B, 32.0)
        else:
            Xd, mask = q.dropout(X, mask_p, 77)
            dX_big, _, _ = q.linear_bwd_dropout(dY, Xd, mask, mask_p, qw, A, B, 32.0)
            dX_small, _, _ = q.linear_bwd_dropout(dY[:512].contiguous(), Xd[:512].contiguous(),
                                                  mask[:512 * K // 32].contiguous(), mask_p, qw, A,
                                                  B, 32.0)
        t.cuda.synchronize()
        a = dX_big[:512].contiguous().view(t.int16).cpu().numpy()
        b = dX_small.view(t.int16).cpu().numpy()
        assert np.array_equal(a, b), f"dropout={mask_p}"


def test_wide_dx_tile_matches_narrow_tile_and_oracle():
    """Once 256 x 256 tiles of dX fill the device, the dX kernel on the bf16
    weight copy takes four 128 x 128 waves per tile instead of eight 64 x 64
    ones.  Both run the same MFMAs on every accumulator in the same order
    (contraction blocks of 16 in increasing order, then the adapter steps), so
    the first 1024 rows of a 4136-token backward (wide tile: 17 x 17 tiles,
    ragged in tokens and features) equal a 1024-token backward of those rows
    (eight-wave tile) bit for bit, also when accumulating into dX; sampled
    rows, the ragged last token tile among them, against the oracle."""
    t = pytest.importorskip("torch")
    M, N, K, small = 4136, 1024, 4160, 1024
    log(f"[wide dX] M={M} N={N} K={K}")
    case = wl.linear_case(13, M, N, K, 16, 32.0)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    base = dev_bf16(wl.activations(14, 100, M, K))
    dX_big, _, _ = q.linear_bwd(dY, X, qw, A, B, 32.0)
    dX_small, _, _ = q.linear_bwd(dY[:small].contiguous(), X[:small].contiguous(), qw, A, B, 32.0)
    acc_big = base.clone()
    q.linear_bwd(dY, X, qw, A, B, 32.0, accumulate_into=acc_big)
    acc_small = base[:small].clone()
    q.linear_bwd(dY[:small].contiguous(), X[:small].contiguous(), qw, A, B, 32.0,
                 accumulate_into=acc_small)
    t.cuda.synchronize()
    bits = lambda v: v.contiguous().view(t.int16).cpu().numpy()
    assert np.array_equal(bits(dX_big[:small]), bits(dX_small)), "dX wide vs eight-wave tile"
    assert np.array_equal(bits(acc_big[:small]), bits(acc_small)), "accumulated dX"
    rows = np.unique(np.concatenate([sample_rows(M, 24, seed=5), np.arange(M - 40, M)]))
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    dYr = f64(case["dY"])[rows]
    s = oracle.lora_scale(32.0, 16)
    ref = dYr @ Wh + s * ((dYr @ f64(case["B"])) @ f64(case["A"]))
    assert_close(host_bf16_f64(dX_big)[rows], ref, "dX sampled rows")
    assert_close(host_bf16_f64(acc_big)[rows], host_bf16_f64(base)[rows] + ref, "accumulated dX rows")


def test_wide_forward_matches_narrow_tile_and_oracle():
    """Once 256 x 256 tiles of Y fill the device, the forward dequantises the
    weight once and runs the wide bf16 tile on the copy instead of the
    256-token tile that decodes in registers.  Both run the same MFMAs on the
    same operands in the same order, so the first 1280 rows of a 4136-token
    forward (17 x 16 wide tiles, ragged in tokens and outputs) equal a
    1280-token forward of those rows (256-token tile, no split) bit for bit;
    sampled rows, the ragged last token tile among them, against the oracle."""
    t = pytest.importorskip("torch")
    M, N, K, small = 4136, 3848, 1024, 1280
    log(f"[wide fwd] M={M} N={N} K={K}")
    case = wl.linear_case(15, M, N, K, 16, 32.0)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B = (dev_bf16(case[k]) for k in ("X", "A", "B"))
    Y_big, T_big = q.linear_fwd(X, qw, A, B, 32.0, save_T=True)
    Y_small, T_small = q.linear_fwd(X[:small].contiguous(), qw, A, B, 32.0, save_T=True)
    t.cuda.synchronize()
    bits = lambda v: v.contiguous().view(t.int16).cpu().numpy()
    assert np.array_equal(bits(T_big[:small]), bits(T_small)), "T next to the dequantisation"
    assert np.array_equal(bits(Y_big[:small]), bits(Y_small)), "Y wide vs 256-token tile"
    rows = np.unique(np.concatenate([sample_rows(M, 24, seed=6, tile=256), np.arange(M - 40, M)]))
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    Xr = f64(case["X"])[rows]
    Tr = Xr @ f64(case["A"]).T
    ref = Xr @ Wh.T + oracle.lora_scale(32.0, 16) * (Tr @ f64(case["B"]).T)
    assert_close(host_bf16_f64(Y_big)[rows], ref, "Y sampled rows")
    assert_close(host_bf16_f64(T_big)[rows], Tr, "T sampled rows")


def test_wide_forward_alone_when_k_is_an_odd_multiple_of_128():
    """K = 384 (a multiple of 128 but not of 256): the register-decoded tile
    does not take it, so at 4096 tokens x 4096 outputs (256 tiles of
    256 x 256) the wide tile on the dequantised copy covers every column
    alone.  Sampled rows of Y and T against the oracle, with r = 24 (the
    adapter term's steps of 16 end in a partial one), and the backward's dX
    on the same rows."""
    t = pytest.importorskip("torch")
    M, N, K, r, alpha = 4096, 4096, 384, 24, 48.0
    log(f"[wide fwd, K % 256 == 128] M={M} N={N} K={K} r={r}")
    case = wl.linear_case(17, M, N, K, r, alpha)
    qw = q.quantize(dev_f32(case["W"]))
    X, A, B, dY = (dev_bf16(case[k]) for k in ("X", "A", "B", "dY"))
    Y, T = q.linear_fwd(X, qw, A, B, alpha, save_T=True)
    dX, dA, dB = q.linear_bwd(dY, X, qw, A, B, alpha, T=T)
    t.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(M, 24, seed=8, tile=256), np.arange(M - 8, M)]))
    Wh = f64(OracleWeight(case["W"]).w_bf16())
    s = oracle.lora_scale(alpha, r)
    Xr = f64(case["X"])[rows]
    Tr = Xr @ f64(case["A"]).T
    ref = Xr @ Wh.T + s * (Tr @ f64(case["B"]).T)
    assert_close(host_bf16_f64(Y)[rows], ref, "Y sampled rows")
    assert_close(host_bf16_f64(T)[rows], Tr, "T sampled rows")
    dYr = f64(case["dY"])[rows]
    refdx = dYr @ Wh + s * ((dYr @ f64(case["B"])) @ f64(case["A"]))
    assert_close(host_bf16_f64(dX)[rows], refdx, "dX sampled rows")


# ---------------------------- full-size configs ------------------------------

def _full_linear(cfg, idx, M=None, rows=48):
    t = pytest.importorskip("torch")
    w = wl.workloads()[cfg]
    lin = w.linears[idx]
    M = M or w.M
    log(f"[full] {cfg}/{lin.name} M={M} N={lin.N} K={lin.K} r={lin.r}")
    W = wl.weight(0, w.cfg_id, idx, lin)
    A, B = wl.adapters(0, w.cfg_id, idx, lin)
    X = wl.activations(0, w.cfg_id, M, lin.K, sub=idx)
    dY = wl.grad_output(0, w.cfg_id, M, lin.N, sub=idx)
    qw = q.quantize(dev_f32(W))
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    Y, T = q.linear_fwd(Xd, qw, Ad, Bd, lin.alpha)
    got = dict(Y=host_bf16_f64(Y), T=host_bf16_f64(T))
    if w.backward:
        dX, dA, dB = q.linear_bwd(dYd, Xd, qw, Ad, Bd, lin.alpha, T=T)
        got.update(dX=host_bf16_f64(dX), dA=host(dA).astype(np.float64),
                   dB=host(dB).astype(np.float64))
    t.cuda.synchronize()
    del qw, Xd, dYd
    ow = OracleWeight(W, full=False)
    s = oracle.lora_scale(lin.alpha, lin.r)
    Xf, Af, Bf, dYf = f64(X), f64(A), f64(B), f64(dY)
    # The oracle's own forward on the sampled weight rows (the layer restricted
    # to those output columns): Y[:, ncol] and the whole of T.
    ncol = sample_rows(lin.N, rows, seed=2)
    Wr = f64(ow.rows_bf16(ncol))
    Yref, Tref = oracle.forward(Xf, Wr, Af, Bf[ncol], lin.alpha, lin.r)
    assert_close(got["T"], Tref, "T")
    assert_close(got["Y"][:, ncol], Yref, "Y[:, sampled]")
    if not w.backward:
        return
    # dA and dB whole, from their definitions
    U = dYf @ Bf
    assert_close(got["dA"], s * (U.T @ Xf), "dA")
    assert_close(got["dB"], s * (dYf.T @ Tref), "dB")
    # The oracle's backward on restricted operands: with the input features
    # cut to sampled 64-column blocks it gives dX and dA on those columns
    # (U = dY B is unchanged); with the output features cut to the sampled
    # weight rows it gives dB on those rows (T = X A^T is unchanged).
    kb = np.unique(np.concatenate([[0, lin.K // 64 - 1],
                                   np.random.default_rng(3).integers(0, lin.K // 64, 6)]))
    Wc = f64(ow.colblocks_bf16(kb))
    cols = (kb[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    dXc, dAc, _ = oracle.backward(dYf, Xf[:, cols], Wc, Af[:, cols], Bf, lin.alpha, lin.r)
    assert_close(got["dX"][:, cols], dXc, "dX[:, sampled]")
    assert_close(got["dA"][:, cols], dAc, "dA[:, sampled]")
    _, _, dBr = oracle.backward(dYf[:, ncol], Xf, Wr, Af, Bf[ncol], lin.alpha, lin.r)
    assert_close(got["dB"][ncol], dBr, "dB[sampled]")


def test_full_config2():
    _full_linear("c2_linear_4096", 0)


@pytest.mark.parametrize("idx", [0, 2])
def test_full_config3_linears(idx):
    _full_linear("c3_mlp_11008", idx)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_full_config4_gemv(M):
    _full_linear("c4_gemv_28672x8192", 0, M=M, rows=256)


@pytest.mark.parametrize("idx", [0, 4, 6])
def test_full_config5_linears(idx):
    _full_linear("c5_decoder_8192", idx)
