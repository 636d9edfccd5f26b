"""Host-only checks of the C ABI (no GPU needed, no kernel is launched).

* libqlora.so loads and exports every function include/qlora.h declares;
* the Python binding declares the same set;
* the codebooks the kernels embed equal the oracle's bit for bit;
* every invalid argument is rejected with its status code.  Validation runs
  before any launch, so fake (never dereferenced) device addresses suffice.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

if not os.path.exists(q.LIB_PATH):
    pytest.skip("libqlora.so not built", allow_module_level=True)

lib = q.load_library()
D = 0x7f0000000000           # fake 16-byte aligned "device" address (never touched)
MIS = D + 4                   # misaligned


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", txt, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q.SIGNATURES), "binding and header disagree"


def test_codebooks_match_oracle_bits():
    got = np.array(q.codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    got8 = np.array(q.dq_levels(), dtype=np.float32)
    assert np.array_equal(got8.view(np.uint32), oracle.dq_codebook().view(np.uint32))


def test_float8_table_matches_oracle_bits():
    got = np.array(q.dq_float8_levels(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.dq_float8_codebook().view(np.uint32))


def test_second_level_table_validation():
    lv = (ctypes.c_float * 253)(*q.dq_float8_levels())
    bad = (ctypes.c_float * 3)(0.0, -1.0, 1.0)
    P = ctypes.cast(lv, ctypes.c_void_p)
    B = ctypes.cast(bad, ctypes.c_void_p)
    dq, ad, dt = lib.double_quant_table, lib.absmax_dequant, lib.dequant_tables
    assert dq(D, 100, 256, None, 253, D, D, D, None) == q.ERR_NULL
    assert dq(D, 100, 256, P, 1, D, D, D, None) == q.ERR_ARG          # too few levels
    assert dq(D, 100, 256, P, 257, D, D, D, None) == q.ERR_ARG
    assert dq(D, 100, 256, B, 3, D, D, D, None) == q.ERR_ARG          # not ascending
    assert dq(D, 100, 128, P, 253, D, D, D, None) == q.ERR_UNSUPPORTED
    assert dq(D, 0, 256, P, 253, D, D, D, None) == q.ERR_SHAPE
    assert dq(D, 100, 256, P, 253, D, D, MIS, None) == q.ERR_ALIGN
    assert ad(D, D, D, 100, 256, P, 253, None, None) == q.ERR_NULL
    assert ad(D, D, D, 100, 256, B, 3, D, None) == q.ERR_ARG
    assert ad(D, D, D, 100, 256, P, 253, MIS, None) == q.ERR_ALIGN
    assert dt(D, D, D, D, 4, 64, 64, 256, None, P, 253, None, None) == q.ERR_NULL
    assert dt(D, D, D, D, 4, 64, 64, 256, None, B, 3, D, None) == q.ERR_ARG
    assert dt(D, D, D, D, 4, 65, 64, 256, None, P, 253, D, None) == q.ERR_SHAPE
    assert dt(D, D, D, D, 4, 64, 64, 256, B, P, 253, D, None) == q.ERR_ARG   # levels4 read as 16


def test_strerror_and_version():
    for code in range(0, -9, -1):
        s = lib.qlora_strerror(code).decode()
        assert s and s != "unknown status"
    assert lib.qlora_strerror(5).decode() == "unknown status"
    assert lib.qlora_version() >= 100


def test_quantize_validation():
    f = lib.nf4_quantize
    assert f(None, 4, 64, 64, D, D, None) == q.ERR_NULL
    assert f(D, 4, 64, 32, D, D, None) == q.ERR_UNSUPPORTED
    assert f(D, 4, 100, 64, D, D, None) == q.ERR_SHAPE
    assert f(D, 0, 64, 64, D, D, None) == q.ERR_SHAPE
    assert f(D, -3, 64, 64, D, D, None) == q.ERR_SHAPE
    assert f(MIS, 4, 64, 64, D, D, None) == q.ERR_ALIGN
    assert f(D, 4, 64, 64, D, MIS, None) == q.ERR_ALIGN


def test_double_quant_and_dequant_validation():
    assert lib.double_quant(D, 100, 256, D, D, None, None) == q.ERR_NULL
    assert lib.double_quant(D, 100, 128, D, D, D, None) == q.ERR_UNSUPPORTED
    assert lib.double_quant(D, 0, 256, D, D, D, None) == q.ERR_SHAPE
    assert lib.double_quant(D, 100, 256, D, D, MIS, None) == q.ERR_ALIGN
    f = lib.nf4_dequant
    assert f(D, D, D, D, 4, 64, 64, 256, None, None) == q.ERR_NULL
    assert f(D, D, D, D, 4, 64, 64, 512, D, None) == q.ERR_UNSUPPORTED
    assert f(D, D, D, D, 4, 65, 64, 256, D, None) == q.ERR_SHAPE
    assert f(D, D, D, MIS, 4, 64, 64, 256, D, None) == q.ERR_ALIGN


def _fwd(**kw):
    a = dict(X=D, M=16, K=256, N=256, packed=D, codes=D, scales=D, mean=D, A=D, B=D, r=8,
             alpha=16.0, Y=D, T=None, ws=D, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.qlora_linear_fwd(a["X"], a["M"], a["K"], a["N"], a["packed"], a["codes"],
                                a["scales"], a["mean"], a["A"], a["B"], a["r"], a["alpha"],
                                a["Y"], a["T"], a["ws"], a["wsb"], a["stream"])


def _fwd_bf16(**kw):
    a = dict(X=D, M=16, K=256, N=256, W=D, A=D, B=D, r=8, alpha=16.0, Y=D, T=None, ws=D,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.qlora_linear_fwd_bf16(a["X"], a["M"], a["K"], a["N"], a["W"], a["A"], a["B"],
                                     a["r"], a["alpha"], a["Y"], a["T"], a["ws"], a["wsb"],
                                     a["stream"])


def _bwd(**kw):
    a = dict(dY=D, X=D, M=16, K=256, N=256, packed=D, codes=D, scales=D, mean=D, A=D, B=D,
             r=8, alpha=16.0, T=None, dX=D, dA=D, dB=D, flags=0, ws=D, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.qlora_linear_bwd(a["dY"], a["X"], a["M"], a["K"], a["N"], a["packed"],
                                a["codes"], a["scales"], a["mean"], a["A"], a["B"], a["r"],
                                a["alpha"], a["T"], a["dX"], a["dA"], a["dB"], a["flags"],
                                a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", [_fwd, _bwd])
def test_linear_validation(fn):
    assert fn(X=None) == q.ERR_NULL
    assert fn(mean=None) == q.ERR_NULL
    assert fn(M=0) == q.ERR_SHAPE
    assert fn(K=96) == q.ERR_SHAPE          # K % 64
    assert fn(N=260) == q.ERR_SHAPE         # N % 8
    assert fn(r=0) == q.ERR_SHAPE
    assert fn(r=-3) == q.ERR_SHAPE
    assert fn(r=257) == q.ERR_SHAPE
    assert fn(r=264) == q.ERR_SHAPE
    assert fn(alpha=float("nan")) == q.ERR_ARG
    assert fn(A=MIS) == q.ERR_ALIGN
    assert fn(ws=None, wsb=0) == q.ERR_WORKSPACE
    assert fn(wsb=16) == q.ERR_WORKSPACE
    assert fn(ws=MIS) == q.ERR_ALIGN


@pytest.mark.parametrize("fn", [_fwd, _bwd])
def test_any_rank_from_1_to_256_is_accepted_up_to_the_workspace(fn):
    """Every rank in [1, 256] passes validation: with a workspace too small
    by one byte the call stops at the workspace check (so nothing else was
    refused), and ranks that are not multiples of 8 need room for the
    zero-padded adapter copies."""
    M, K, N = 16, 256, 256
    is_bwd = 1 if fn is _bwd else 0
    for r in (1, 4, 7, 8, 12, 24, 100, 255, 256):
        need = lib.qlora_workspace_bytes(M, K, N, r, is_bwd)
        assert need > 0, r
        assert fn(r=r, wsb=need - 1) == q.ERR_WORKSPACE, r
    # padding: r = 12 runs as 16 with room for padded A, B, T (and dA, dB)
    pad = 16 * K * 2 + N * 16 * 2 + M * 16 * 2 + (16 * K * 4 + N * 16 * 4 if is_bwd else 0)
    assert (lib.qlora_workspace_bytes(M, K, N, 12, is_bwd)
            >= lib.qlora_workspace_bytes(M, K, N, 16, is_bwd) + pad)


def _timing():
    t = q.TimingC()
    return ctypes.byref(t)


def test_timed_entry_points_validate_like_the_plain_calls():
    ff, fb = lib.qlora_linear_fwd_timed, lib.qlora_linear_bwd_timed
    fwd = [D, 16, 256, 256, D, D, D, D, D, D, 8, 16.0, D, None, D, 1 << 30, None]
    bwd = [D, D, 16, 256, 256, D, D, D, D, D, D, 8, 16.0, None, D, D, D, 0, D, 1 << 30, None]
    for t in (None, _timing()):
        for i, v, code in ((0, None, q.ERR_NULL), (2, 96, q.ERR_SHAPE), (10, 0, q.ERR_SHAPE),
                           (11, float("nan"), q.ERR_ARG), (15, 16, q.ERR_WORKSPACE)):
            a = list(fwd)
            a[i] = v
            assert ff(*a, t) == code, (i, v)
        for i, v, code in ((0, None, q.ERR_NULL), (3, 96, q.ERR_SHAPE), (11, 257, q.ERR_SHAPE),
                           (17, 2, q.ERR_ARG), (19, 16, q.ERR_WORKSPACE)):
            a = list(bwd)
            a[i] = v
            assert fb(*a, t) == code, (i, v)


def test_noalloc_backward_refuses_shapes_beyond_its_static_scratch():
    """qlora_linear_bwd_noalloc validates like qlora_linear_bwd and refuses, before
    anything is launched, a backward that needs more scratch than the static
    array holds (here the 65B-shaped 22016 x 8192 layer at 4096 tokens)."""
    f = lib.qlora_linear_bwd_noalloc
    big = (D, D, 4096, 8192, 22016, D, D, D, D, D, D, 16, 32.0, None, D, D, D, 0, None)
    assert lib.qlora_workspace_bytes(4096, 8192, 22016, 16, 1) > q.NOALLOC_SCRATCH_BYTES
    assert f(*big) == q.ERR_SCRATCH
    assert lib.qlora_strerror(q.ERR_SCRATCH).decode() != "unknown status"
    ok = list(big)
    ok[2], ok[3], ok[4] = 64, 256, 256
    bad = list(ok); bad[0] = None
    assert f(*bad) == q.ERR_NULL
    bad = list(ok); bad[11] = 0
    assert f(*bad) == q.ERR_SHAPE
    bad = list(ok); bad[17] = 2
    assert f(*bad) == q.ERR_ARG


def test_linear_output_validation():
    assert _fwd(Y=None) == q.ERR_NULL
    assert _fwd(T=MIS) == q.ERR_ALIGN
    assert _bwd(dA=None) == q.ERR_NULL
    assert _bwd(dB=None) == q.ERR_NULL
    assert _bwd(flags=2) == q.ERR_ARG
    assert _bwd(dX=MIS) == q.ERR_ALIGN


def test_workspace_sizes():
    assert lib.qlora_workspace_bytes(16, 256, 256, 8, 0) > 0
    assert lib.qlora_workspace_bytes(2048, 4096, 4096, 16, 1) > 0
    assert lib.qlora_workspace_bytes(0, 256, 256, 8, 0) == 0
    assert lib.qlora_workspace_bytes(16, 100, 256, 8, 0) == 0
    assert lib.qlora_workspace_bytes(16, 256, 256, 0, 1) == 0
    assert lib.qlora_workspace_bytes(16, 256, 256, 257, 1) == 0
    # the backward needs room for U and T at least
    assert lib.qlora_workspace_bytes(2048, 4096, 4096, 16, 1) >= 2 * 2048 * 16 * 2
    # from 1024 tokens on it also holds the once-dequantised bf16 weight
    big, small = lib.qlora_workspace_bytes(1024, 4096, 4096, 16, 1), lib.qlora_workspace_bytes(1023, 4096, 4096, 16, 1)
    assert big - small >= 2 * 4096 * 4096
    assert small < 2 * 4096 * 4096


def test_forward_workspace_holds_the_weight_copy_for_wide_shapes():
    """Once 256 x 256 tiles of Y alone fill the device (256 of them), the
    forward dequantises the weight once into the workspace (bf16, 2 N K
    bytes) and runs the wide tile on that copy; below that it decodes in the
    tile and needs no copy."""
    K, N = 4096, 4096
    wide = lib.qlora_workspace_bytes(4096, K, N, 16, 0)    # 16 x 16 tiles
    narrow = lib.qlora_workspace_bytes(4095, K, N, 16, 0)  # 16 x 16 tiles too
    assert wide >= 2 * N * K and narrow >= 2 * N * K
    below = lib.qlora_workspace_bytes(3840, K, N, 16, 0)   # 15 x 16 tiles
    assert below < 2 * N * K
    # 22016 outputs of 8192 inputs: 4096 tokens fill the device (16 x 86)
    assert lib.qlora_workspace_bytes(4096, 8192, 22016, 64, 0) >= 2 * 22016 * 8192
    # a weight copy of 2 GiB or more is not made (32-bit buffer offsets)
    assert lib.qlora_workspace_bytes(4096, 16384, 65536, 16, 0) < 2 * 65536 * 16384


def test_workspace_holds_the_split_partials():
    """With fewer than 128 output tiles (256 tokens x 128 outputs) the forward
    and dX kernels split their contraction so that about 256 workgroups run,
    and the workspace holds one fp32 [M, N] (forward) or [M, K] (dX) partial
    per split; from 128 tiles on they run in one pass."""
    K = N = 4096
    splits = 8   # 256 tokens: 32 tiles, 256 / 32 = 8 splits of 8 K-steps
    assert lib.qlora_workspace_bytes(256, K, N, 16, 0) >= splits * 256 * N * 4
    assert lib.qlora_workspace_bytes(256, K, N, 16, 1) >= splits * 256 * K * 4
    # 128 and 256 tiles: no partials (T, U and the adapter-gradient splits only,
    # and the bf16 weight copy in the backward)
    assert lib.qlora_workspace_bytes(1024, K, N, 16, 0) < 1024 * N * 4
    assert lib.qlora_workspace_bytes(2048, K, N, 16, 0) < 2048 * N * 4
    assert lib.qlora_workspace_bytes(1024, K, N, 16, 1) < 2 * N * K + 1024 * K * 4


def test_split_partials_are_reserved_only_where_a_split_runs():
    """Only the NF4 register-decode forward splits its contraction; the
    bf16-base forward needs T alone, and a backward without dX needs no dX
    partials.  A misaligned workspace of the right size gets past the size
    check and stops at the alignment check (no launch), one byte less stops
    at the size check."""
    K = N = 4096
    M, r = 256, 16
    t_only = M * r * 2                       # T, the bf16 forward's whole need
    assert _fwd_bf16(M=M, K=K, N=N, r=r, ws=MIS, wsb=t_only) == q.ERR_ALIGN
    assert _fwd_bf16(M=M, K=K, N=N, r=r, ws=MIS, wsb=t_only - 1) == q.ERR_WORKSPACE
    assert _fwd(M=M, K=K, N=N, r=r, ws=MIS, wsb=t_only) == q.ERR_WORKSPACE   # NF4: partials
    full = lib.qlora_workspace_bytes(M, K, N, r, 1)
    dx_parts = 8 * M * K * 4                 # 8 splits of the dX contraction
    assert _bwd(M=M, K=K, N=N, r=r, dX=None, ws=MIS, wsb=full - dx_parts) == q.ERR_ALIGN
    assert _bwd(M=M, K=K, N=N, r=r, ws=MIS, wsb=full - dx_parts) == q.ERR_WORKSPACE


def test_silu_validation():
    assert lib.silu_mul_fwd(D, None, 64, D, None) == q.ERR_NULL
    assert lib.silu_mul_fwd(D, D, 60, D, None) == q.ERR_SHAPE
    assert lib.silu_mul_fwd(D, D, 64, MIS, None) == q.ERR_ALIGN
    assert lib.silu_mul_bwd(D, D, D, 64, D, None, None) == q.ERR_NULL
    assert lib.silu_mul_bwd(D, D, D, 0, D, D, None) == q.ERR_SHAPE


def test_linear_size_limits():
    """Operands of 2 GiB or more are refused (32-bit buffer offsets)."""
    assert _fwd(M=1 << 18, K=1 << 12) == q.ERR_SHAPE          # X = 2 GiB
    assert _fwd(M=1 << 18, N=1 << 12) == q.ERR_SHAPE          # Y = 2 GiB
    assert _bwd(M=1 << 18, N=1 << 12) == q.ERR_SHAPE          # dY = 2 GiB
    assert _fwd(N=1 << 16, K=1 << 16) == q.ERR_SHAPE          # packed = 2 GiB


def test_merge_validation():
    f = lib.qlora_merge
    ok = (D, D, D, D, 256, 128, 64, 256, D, D, 16, 32.0, D, None)   # valid: never called as is

    def call(**kw):
        a = list(ok)
        names = ["packed", "codes", "scales", "mean", "N", "K", "bs", "dqbs", "A", "B", "r",
                 "alpha", "out", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)
    assert call(out=None) == q.ERR_NULL
    assert call(A=None) == q.ERR_NULL
    assert call(bs=32) == q.ERR_UNSUPPORTED
    assert call(dqbs=128) == q.ERR_UNSUPPORTED
    assert call(K=100) == q.ERR_SHAPE
    assert call(N=12) == q.ERR_SHAPE
    assert call(r=0) == q.ERR_SHAPE
    assert call(r=264) == q.ERR_SHAPE
    assert call(alpha=float("nan")) == q.ERR_ARG
    assert call(B=MIS) == q.ERR_ALIGN
    assert call(out=MIS) == q.ERR_ALIGN


def _fl16(vals):
    return ctypes.cast((ctypes.c_float * 16)(*vals), ctypes.c_void_p)


def test_codebook_validation():
    good = [float(v) for v in oracle.int4_codebook()]
    bad_order = list(good)
    bad_order[3], bad_order[4] = bad_order[4], bad_order[3]
    dup = list(good)
    dup[5] = dup[4]
    nan = list(good)
    nan[0] = float("nan")
    fq, fd = lib.codebook_quantize, lib.codebook_dequant
    assert fq(D, 4, 64, 64, None, D, D, None) == q.ERR_NULL
    for lv in (bad_order, dup, nan):
        assert fq(D, 4, 64, 64, _fl16(lv), D, D, None) == q.ERR_ARG
        assert fd(D, D, D, D, 4, 64, 64, 256, _fl16(lv), D, None) == q.ERR_ARG
    assert fq(None, 4, 64, 64, _fl16(good), D, D, None) == q.ERR_NULL
    assert fq(D, 4, 100, 64, _fl16(good), D, D, None) == q.ERR_SHAPE
    assert fq(D, 4, 64, 32, _fl16(good), D, D, None) == q.ERR_UNSUPPORTED
    assert fq(D, 4, 64, 64, _fl16(good), MIS, D, None) == q.ERR_ALIGN
    assert fd(D, D, D, D, 4, 64, 64, 256, None, D, None) == q.ERR_NULL
    assert fd(D, D, D, D, 4, 64, 64, 128, _fl16(good), D, None) == q.ERR_UNSUPPORTED
    assert fd(D, D, D, D, 4, 64, 64, 256, _fl16(good), MIS, None) == q.ERR_ALIGN


def test_dropout_validation():
    f = lib.lora_dropout
    assert f(None, 4, 64, 0.05, 1, D, D, None) == q.ERR_NULL
    assert f(D, 4, 64, 0.05, 1, D, None, None) == q.ERR_NULL
    assert f(D, 4, 48, 0.05, 1, D, D, None) == q.ERR_SHAPE        # K % 32
    assert f(D, 0, 64, 0.05, 1, D, D, None) == q.ERR_SHAPE
    assert f(D, 1 << 18, 1 << 12, 0.05, 1, D, D, None) == q.ERR_SHAPE   # X = 2 GiB
    for p in (1.0, -0.01, float("nan"), 2.0):
        assert f(D, 4, 64, p, 1, D, D, None) == q.ERR_ARG
    assert f(MIS, 4, 64, 0.05, 1, D, D, None) == q.ERR_ALIGN
    assert f(D, 4, 64, 0.05, 1, D, MIS, None) == q.ERR_ALIGN


def test_linear_dropout_validation():
    ff, fb = lib.qlora_linear_fwd_dropout, lib.qlora_linear_bwd_dropout
    fwd_ok = [D, D, 64, 256, 256, D, D, D, D, D, D, 16, 32.0, D, D, D, 1 << 30, None]
    bwd_ok = [D, D, D, 0.05, 64, 256, 256, D, D, D, D, D, D, 16, 32.0, D, D, D, D, 0, D,
              1 << 30, None]

    def call(f, base, changes):
        a = list(base)
        for k, v in changes.items():
            a[k] = v
        return f(*a)
    assert call(ff, fwd_ok, {1: None}) == q.ERR_NULL          # Xd
    assert call(ff, fwd_ok, {1: MIS}) == q.ERR_ALIGN
    assert call(ff, fwd_ok, {3: 100}) == q.ERR_SHAPE          # K % 64
    assert call(ff, fwd_ok, {0: None}) == q.ERR_NULL          # X
    assert call(fb, bwd_ok, {2: None}) == q.ERR_NULL          # mask
    assert call(fb, bwd_ok, {2: MIS}) == q.ERR_ALIGN
    assert call(fb, bwd_ok, {3: 1.0}) == q.ERR_ARG            # p
    assert call(fb, bwd_ok, {3: float("nan")}) == q.ERR_ARG
    assert call(fb, bwd_ok, {1: None}) == q.ERR_NULL          # Xd
    assert call(fb, bwd_ok, {19: 4}) == q.ERR_ARG             # unknown flag
    assert call(fb, bwd_ok, {20: None}) == q.ERR_WORKSPACE


def test_mlp_fwd_validation():
    f = lib.qlora_mlp_fwd
    good = q.LoraLinearC(D, D, D, D, D, D, 16, 32.0)

    def call(gate=good, up=good, M=64, K=256, I=512, G=D, U=D, H=D, Tg=D, Tu=D, ws=D,
             wsb=1 << 30):
        gp = None if gate is None else ctypes.byref(gate)
        upp = None if up is None else ctypes.byref(up)
        return f(D, M, K, I, gp, upp, G, U, H, Tg, Tu, ws, wsb, None)
    assert call(gate=None) == q.ERR_NULL
    assert call(up=None) == q.ERR_NULL
    assert call(up=q.LoraLinearC(D, D, D, D, D, D, 0, 32.0)) == q.ERR_SHAPE      # r < 1
    assert call(gate=q.LoraLinearC(D, None, D, D, D, D, 16, 32.0)) == q.ERR_NULL
    assert call(up=q.LoraLinearC(D, D, D, D, D, D, 16, float("inf"))) == q.ERR_ARG
    assert call(K=100) == q.ERR_SHAPE
    assert call(I=12) == q.ERR_SHAPE
    assert call(H=None) == q.ERR_NULL
    assert call(Tu=None) == q.ERR_NULL
    assert call(U=MIS) == q.ERR_ALIGN
    assert call(M=4, ws=None, wsb=0) == q.ERR_WORKSPACE      # small M needs workspace
    # the fused gate/up kernel (M > 16, whole ranks) needs none; a rank that
    # is not a multiple of 8 runs the padded composition, which does
    assert call(up=q.LoraLinearC(D, D, D, D, D, D, 12, 32.0), ws=None, wsb=0) == q.ERR_WORKSPACE


def test_mlp_bwd_validation():
    f = lib.qlora_mlp_bwd
    good = q.LoraLinearC(D, D, D, D, D, D, 16, 32.0)

    def call(gate=good, up=good, K=256, I=512, dH=D, dX=D, dAu=D, flags=0, ws=D, wsb=1 << 30):
        gp = None if gate is None else ctypes.byref(gate)
        upp = None if up is None else ctypes.byref(up)
        return f(dH, D, 64, K, I, gp, upp, D, D, D, D, D, D, dX, D, D, dAu, D, flags, ws, wsb, None)
    assert call(gate=None) == q.ERR_NULL
    assert call(up=q.LoraLinearC(D, D, D, D, D, D, 264, 32.0)) == q.ERR_SHAPE
    assert call(K=96) == q.ERR_SHAPE
    assert call(dH=None) == q.ERR_NULL
    assert call(dAu=None) == q.ERR_NULL
    assert call(flags=2) == q.ERR_ARG
    assert call(dX=MIS) == q.ERR_ALIGN
    assert call(ws=None) == q.ERR_WORKSPACE
    assert call(wsb=16) == q.ERR_WORKSPACE
