"""GPU parity of the double quantisation with a second-level table passed as
data (double_quant_table, absmax_dequant, dequant_tables): bit-exact against
the oracle for the 8-bit-float table, and with the linear table equal to the
layer's own double_quant.  Shapes: a partial last group of 256, a group whose
constants are all equal (scale 0), the heavy-tailed 65B-shaped weight."""
import numpy as np
import pytest

import bit_nf4_quantized_07_amd as q
import oracle
import qlora_workloads as wl
from gpu_helpers import dev_f32, host, host_bf16_bits, log

pytestmark = pytest.mark.gpu


def _absmax_cases():
    g = np.random.default_rng(11)
    a = np.abs(g.standard_normal(5 * 256 + 77)).astype(np.float32) * np.float32(0.02)
    a[256:512] = np.float32(0.03)                         # one group with scale 0
    b = np.abs(g.standard_t(3, 4 * 256)).astype(np.float32) * np.float32(0.05)
    return {"ragged": a, "heavy_tail": b}


@pytest.mark.parametrize("name", ["ragged", "heavy_tail"])
def test_double_quant_table_bit_exact(name):
    t = pytest.importorskip("torch")
    a = _absmax_cases()[name]
    f8 = oracle.dq_float8_codebook()
    d = dev_f32(a)
    c, s, mu = q.double_quant_table(d, f8.tolist())
    ah = q.absmax_dequant(c, s, mu, f8.tolist())
    cl, sl, ml = q.double_quant_table(d, oracle.dq_codebook().tolist())
    c0, s0, m0 = q.double_quant(d)
    t.cuda.synchronize()
    rc, rs, rmu = oracle.double_quant(a, 256, levels=f8)
    assert np.array_equal(host(c), rc), "codes"
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32)), "scales"
    assert host(mu).view(np.uint32)[0] == np.float32(rmu).view(np.uint32), "mean"
    rah = oracle.dequant_absmax(rc, rs, rmu, 256, levels=f8)
    assert np.array_equal(host(ah).view(np.uint32), rah.view(np.uint32)), "a_hat"
    # the linear table through the same kernels gives the layer's own codes
    assert np.array_equal(host(cl), host(c0)) and np.array_equal(host(sl), host(s0))
    assert host(ml)[0] == host(m0)[0]


def test_dequant_tables_bit_exact():
    t = pytest.importorskip("torch")
    lin = wl.Linear("w", 136, 512, 8, 16.0, outlier_frac=0.01)
    W = wl.weight(3, 120, 0, lin)
    f8 = oracle.dq_float8_codebook()
    packed, absmax = q.nf4_quantize(dev_f32(W))
    codes, scales, mean = q.double_quant_table(absmax, f8.tolist())
    qw = q.QuantizedWeight(packed, codes, scales, mean, lin.N, lin.K)
    for levels4 in (None, oracle.int4_codebook()):
        if levels4 is None:
            out = q.dequant_tables(qw, f8.tolist())
            c4, _ = oracle.quantize_nf4(W, 64)
        else:
            p4, a4 = q.codebook_quantize(dev_f32(W), levels4.tolist())
            c8, s8, m8 = q.double_quant_table(a4, f8.tolist())
            out = q.dequant_tables(q.QuantizedWeight(p4, c8, s8, m8, lin.N, lin.K), f8.tolist(),
                                   levels4=levels4.tolist())
            c4, _ = oracle.quantize_blocks(W, levels4, 64)
        t.cuda.synchronize()
        ab = oracle.absmax_blocks(W, 64)
        rc, rs, rmu = oracle.double_quant(ab, 256, levels=f8)
        ah = oracle.dequant_absmax(rc, rs, rmu, 256, levels=f8)
        _, wb = oracle.dequant_codes(c4.reshape(-1), ah, 64, levels=levels4)
        assert np.array_equal(host_bf16_bits(out).reshape(-1), wb.reshape(-1)), levels4 is None


def test_float8_table_on_the_65b_weight():
    """Relative reconstruction error of the block constants, linear vs float
    second level, on the 65B-shaped weight with Student-t outliers: reported,
    and the float table must not be worse at the median."""
    t = pytest.importorskip("torch")
    w = wl.workloads()["c5_decoder_8192"]
    lin = w.linears[4]
    W = wl.weight(0, w.cfg_id, 4, lin)
    _, absmax = q.nf4_quantize(dev_f32(W))
    del W
    out = {}
    for name, lv in (("linear", oracle.dq_codebook()), ("float8", oracle.dq_float8_codebook())):
        c, s, mu = q.double_quant_table(absmax, lv.tolist())
        ah = q.absmax_dequant(c, s, mu, lv.tolist())
        rel = ((ah - absmax).abs() / absmax.clamp_min(1e-30)).double()
        out[name] = (float(((ah - absmax).double().norm() / absmax.double().norm()).item()),
                     float(rel.median().item()), float(rel.max().item()))
    t.cuda.synchronize()
    log(f"  a_hat relative error (Frobenius, median, max): {out}")
    assert out["float8"][1] <= out["linear"][1]
