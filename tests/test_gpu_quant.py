"""GPU parity of the storage kernels: nf4_quantize, double_quant and
nf4_dequant must reproduce the oracle bit for bit."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import OracleWeight, dev_f32, host, host_bf16_bits, log

pytestmark = pytest.mark.gpu


def gpu_quant(W):
    t = dev_f32(W)
    packed, absmax = q.nf4_quantize(t)
    codes, scales, mean = q.double_quant(absmax)
    qw = q.QuantizedWeight(packed, codes, scales, mean, W.shape[0], W.shape[1])
    return qw, absmax


def check_full(W, name):
    log(f"[quant] {name} shape={W.shape}")
    qw, absmax = gpu_quant(W)
    deq = q.nf4_dequant(qw)
    ow = OracleWeight(W)
    assert np.array_equal(host(absmax).view(np.uint32), ow.absmax.view(np.uint32)), "absmax"
    assert np.array_equal(host(qw.packed), ow.packed), "packed"
    assert np.array_equal(host(qw.codes), ow.codes8), "dq codes"
    assert np.array_equal(host(qw.scales).view(np.uint32), ow.scales.view(np.uint32)), "scales"
    assert host(qw.mean)[0].view(np.uint32) == np.float32(ow.mean).view(np.uint32), "mean"
    assert np.array_equal(host_bf16_bits(deq), ow.w_bf16()), "dequant bf16"


SHAPES = [(1, 64), (3, 64), (40, 192), (7, 1024), (300, 64), (256, 256), (129, 4160)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_storage_bit_exact_small(N, K):
    W = wl.weight(0, 100, N * 10000 + K, wl.Linear("w", N, K, 8, 16.0))
    check_full(W, f"N={N} K={K}")


def test_storage_bit_exact_config1_and_2():
    for cfg in ("c1_linear_256", "c2_linear_4096"):
        w = wl.workloads()[cfg]
        lin = w.linears[0]
        check_full(wl.weight(0, w.cfg_id, 0, lin), cfg)


@pytest.mark.parametrize("N,K", [(4100, 4096), (262244, 64)])
def test_storage_bit_exact_many_groups(N, K):
    """More than 1024 groups of 256 constants take the two-launch mean; the
    second shape ends with a partial group of 100 constants."""
    W = wl.weight(0, 100, N * 10000 + K, wl.Linear("w", N, K, 8, 16.0))
    check_full(W, f"N={N} K={K}")


def test_storage_special_blocks():
    """Zero blocks, exact ties at representable midpoints, +-absmax, -0.0,
    subnormal and tiny values."""
    q4 = oracle.nf4_codebook().astype(np.float64)
    mids = [(q4[i] + q4[i + 1]) / 2 for i in range(15)]
    ties = [np.float32(m) for m in mids if float(np.float32(m)) == m]
    assert len(ties) == 4
    rows = []
    z = np.zeros(64, np.float32); rows.append(z)                          # all zero
    b = np.zeros(64, np.float32); b[0] = 1.0
    for i, t in enumerate(ties):
        b[1 + 3 * i] = t
        b[2 + 3 * i] = np.nextafter(t, np.float32(2))
        b[3 + 3 * i] = np.nextafter(t, np.float32(-2))
    rows.append(b)                                                        # ties, absmax 1
    c = np.full(64, -0.0, np.float32); c[5] = -3.5; c[6] = 3.5; rows.append(c)   # +-absmax
    d = np.full(64, 1e-45, np.float32); d[0] = 1e-38; d[1] = -1e-40; rows.append(d)  # tiny
    e = np.linspace(-1, 1, 64).astype(np.float32) * np.float32(0.02); rows.append(e)
    W = np.stack(rows * 52)[:256].reshape(-1, 256)                        # 64 rows of 256
    check_full(W, "special blocks")


def test_storage_equal_constants():
    """Every block has absmax 0.5: the mean is 0.5, every centred constant is 0,
    every second-level scale is 0 and every 8-bit code is the zero code."""
    g = np.random.default_rng(3)
    W = (g.uniform(-0.4, 0.4, (48, 512))).astype(np.float32)
    W[:, ::64] = 0.5
    check_full(W, "equal constants")


@pytest.mark.parametrize("cfg,idx", [("c3_mlp_11008", 0), ("c3_mlp_11008", 2),
                                     ("c4_gemv_28672x8192", 0), ("c5_decoder_8192", 0),
                                     ("c5_decoder_8192", 4)])
def test_storage_full_size_sampled(cfg, idx):
    """Full-size weights: absmax and all double-quant outputs everywhere,
    packed nibbles and dequantised bf16 on sampled rows."""
    w = wl.workloads()[cfg]
    lin = w.linears[idx]
    log(f"[quant-full] {cfg}/{lin.name} {lin.N}x{lin.K}")
    W = wl.weight(0, w.cfg_id, idx, lin)
    qw, absmax = gpu_quant(W)
    deq = q.nf4_dequant(qw)
    ow = OracleWeight(W, full=False)
    assert np.array_equal(host(absmax).view(np.uint32), ow.absmax.view(np.uint32)), "absmax"
    assert np.array_equal(host(qw.codes), ow.codes8), "dq codes"
    assert np.array_equal(host(qw.scales).view(np.uint32), ow.scales.view(np.uint32)), "scales"
    assert host(qw.mean)[0].view(np.uint32) == np.float32(ow.mean).view(np.uint32), "mean"
    rows = np.unique(np.concatenate([[0, 1, lin.N - 1],
                                     np.random.default_rng(1).integers(0, lin.N, 61)]))
    c4, _ = oracle.quantize_nf4(W[rows], 64)
    packed_rows = host(qw.packed).reshape(lin.N, lin.K // 2)[rows]
    assert np.array_equal(packed_rows.reshape(-1), oracle.pack_nibbles(c4)), "packed rows"
    deq_rows = host_bf16_bits(deq).reshape(lin.N, lin.K)[rows]
    assert np.array_equal(deq_rows, ow.rows_bf16(rows)), "dequant rows"


def _oracle_boundaries():
    """For each NF4 level i < 15, the largest fp32 value the oracle maps to a
    level <= i, found by bisection over fp32 values ordered as integers."""
    q4 = oracle.nf4_codebook()

    def key_to_f(k):   # monotone integer key -> fp32
        b = np.uint32(k) if k >= 0 else (np.uint32(-k) | np.uint32(0x80000000))
        return np.array([b], np.uint32).view(np.float32)[0]

    lo_k, hi_k = -0x3F800000, 0x3F800000      # -1.0 .. +1.0
    out = []
    for i in range(15):
        lo, hi = lo_k, hi_k                   # invariant: code(lo) <= i < code(hi)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            c = oracle.nearest_index(np.array([key_to_f(mid)], np.float32), q4)[0]
            lo, hi = (mid, hi) if c <= i else (lo, mid)
        out.append(key_to_f(lo))
    return np.array(out, np.float32)


def test_exhaustive_fp32_sweep():
    """Every fp32 n in [-1, 1] goes through nf4_quantize (blocks with absmax
    exactly 1.0 hold the sweep values, so n = w) and must get the oracle's code."""
    t = pytest.importorskip("torch")
    bounds = t.from_numpy(_oracle_boundaries()).cuda()
    npos = 0x3F800000 + 1                     # +0 .. +1.0
    per_block = 63
    chunk_blocks = 1 << 21
    done = 0
    for sign in (0, 1):
        start = 0
        while start < npos:
            nb = min(chunk_blocks, (npos - start + per_block - 1) // per_block)
            idx = t.arange(start, start + nb * per_block, dtype=t.int64, device="cuda")
            idx = t.clamp(idx, max=npos - 1)      # pad the last block with repeats of 1.0
            bits = (idx - (1 << 31) if sign else idx).to(t.int32)   # sign bit set for sign=1
            vals = bits.view(t.float32).view(nb, per_block)
            W = t.cat([t.ones(nb, 1, device="cuda"), vals], dim=1).contiguous()
            packed, absmax = q.nf4_quantize(W.view(nb, 64))
            assert bool((absmax == 1.0).all())
            codes = t.stack([packed >> 4, packed & 15], dim=1).view(nb, 64)
            want = t.bucketize(vals, bounds, right=False).to(t.uint8)
            assert bool((codes[:, 0] == 15).all())
            bad = (codes[:, 1:] != want)
            if bool(bad.any()):
                i = int(bad.reshape(-1).nonzero()[0][0])
                raise AssertionError(f"mismatch at sweep index {start + i} sign {sign}")
            start += nb * per_block
            done += nb * per_block
        log(f"  sweep sign={sign} done ({done} values)")
    assert done >= 2 * npos
