"""NF4 storage of the frozen base weight, written from the pages (oracle side).

Every step follows the description of QLoRA's storage format:

* 4-bit NormalFloat: 16 levels placed at quantiles of the standard normal so
  that each bin receives the same expected share of normally distributed
  weights ([AG] list item 1; [AU] "Hoe het werkt", NF4 box; [LC] 方法与公式
  item 1; [LI] §2).
* Blockwise absmax: weights are quantised in blocks of (for example) 64, each
  block carrying its own scale constant ([LC] 方法与公式 item 1).
* Double quantisation: the per-block fp32 constants are themselves quantised
  to 8 bits, cutting their cost from about 0.5 to about 0.13 bit per parameter
  ([AG] list item 2; [AU] Dubbele Quantisatie box; [LC] 方法与公式 item 2;
  [LI] §1 innovation tree).
* On-the-fly dequantisation to the 16-bit compute type before the matmul
  ([AU] "QLoRA DATASTROOM" box; [LC] 直觉与动机 and 方法与公式).

Where the pages leave a step open the reading taken is stated at that step;
every reading is also listed in the design notes of the repository.
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

# ---------------------------------------------------------------------------
# Codebooks
# ---------------------------------------------------------------------------

#: Extreme probability of the NF4 quantiles.  Reading: the pages fix 16 levels
#: at normal quantiles with an exact zero and range [-1, 1]; Phi^-1(1) is
#: infinite, so the outermost quantile sits at the midpoint of the two tail
#: masses 1/(2*15) and 1/(2*16), i.e. delta = 1 - (1/30 + 1/32)/2.
NF4_DELTA = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def _nf4_levels_f64(inv_cdf) -> list:
    """The 16 NF4 levels in fp64, using the supplied inverse normal CDF.

    Positive side: 8 quantiles evenly spaced in probability between 1/2
    (excluded: that is the zero level) and delta.  Negative side: 7 quantiles
    evenly spaced between 1/2 (excluded) and delta, mirrored.  Zero is added
    exactly.  Everything is divided by Phi^-1(delta) so that the range is
    exactly [-1, 1].  16 is even and zero must be exact, so one side has to
    carry one more level; the positive side does (reading, see module doc).
    """
    z = inv_cdf(NF4_DELTA)
    pos = [inv_cdf(NF4_DELTA - i * (NF4_DELTA - 0.5) / 8.0) / z for i in range(8)]
    neg = [-inv_cdf(NF4_DELTA - j * (NF4_DELTA - 0.5) / 7.0) / z for j in range(7)]
    return sorted(neg + [0.0] + pos)


def nf4_codebook() -> np.ndarray:
    """Q4[0..15] as fp32: levels evaluated in fp64, rounded once (RNE) to fp32.

    [LC] 方法与公式 item 1 (quantile quantisation of a zero-mean normal, equal
    expected count per bin); [AU] NF4 box (16 levels); [LI] §2.
    """
    lv = _nf4_levels_f64(NormalDist().inv_cdf)
    return np.array(lv, dtype=np.float64).astype(np.float32)


def dq_codebook() -> np.ndarray:
    """Q8[0..254] as fp32, the 8-bit code for the centred block constants.

    The pages only say the constants are re-quantised to 8 bits ([AU] Dubbele
    Quantisatie box; [LC] 方法与公式 item 2).  Reading (the plainest one):
    symmetric linear levels (i - 127)/127, i = 0..254, each the correctly
    rounded fp32 quotient; code byte = index, byte 255 unused.
    """
    i = np.arange(255, dtype=np.float32)
    return (i - np.float32(127.0)) / np.float32(127.0)


def fp8_e4m3_values() -> np.ndarray:
    """Every finite value of the 8-bit float with one sign bit, 4 exponent bits
    (bias 7) and 3 mantissa bits, no infinities and one NaN pattern per sign
    (exponent and mantissa all ones), decoded from its bit fields in fp64:
    exponent 0 gives the subnormals m / 8 * 2^-6, exponent e > 0 the normal
    values (1 + m / 8) * 2^(e - 7).  Sorted, +0 and -0 counted once: 253
    values from -448 to 448."""
    vals = set()
    for b in range(256):
        sign, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue                               # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals.add(-v if sign else v)
    return np.array(sorted(vals), dtype=np.float64)


def dq_float8_codebook() -> np.ndarray:
    """Q8F[0..252] as fp32: an 8-bit float code for the centred block constants.

    The pages give only the width of the second level, 8 bits ([AU] Dubbele
    Quantisatie box; [LC] 方法与公式 item 2).  This table is the other reading
    of "8-bit" next to the linear code: the finite values of the 8-bit float
    above (4 exponent, 3 mantissa bits), divided by the largest one (448) so
    that the levels span the normalised range [-1, 1] with an exact zero,
    each quotient evaluated in fp64 and rounded once to fp32.  Its levels are
    dense near zero and sparse near +-1, so small constants in a group with
    one large outlier keep their relative precision.  Code byte = index
    (0..252, zero at 126); bytes 253..255 unused.
    """
    return (fp8_e4m3_values() / 448.0).astype(np.float32)


def int4_codebook() -> np.ndarray:
    """Uniform 4-bit codebook for the comparison the pages draw with NF4:
    16 levels spaced evenly over the absmax-normalised range [-1, 1] ([LI] §2,
    standard uniform INT4 puts its bins at equal linear intervals; [LC] 方法与
    公式 item 1, uniform INT4 wastes levels in the tails).  Reading: levels
    -1 + 2 i / 15, i = 0..15, each evaluated in fp64 and rounded once to
    fp32.  Same packing, blocks and absmax constants as NF4."""
    return (-1.0 + 2.0 * np.arange(16, dtype=np.float64) / 15.0).astype(np.float32)


def nearest_index(values: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level, ties to the LOWER index (deterministic).

    Brute force: distance to every level, argmin (numpy returns the first of
    equal minima).  ``values`` and ``levels`` are fp32; the distances are taken
    in fp64, where the difference of two fp32 numbers of comparable size is
    exact, and where it is not (a tiny value) the competing distances differ by
    far more than the rounding.  Reading: the pages say "nearest level" only
    implicitly (quantile bins); the tie rule is the build's.
    """
    v = np.asarray(values, dtype=np.float32).astype(np.float64).reshape(-1)
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    step = 1 << 20
    for s in range(0, v.size, step):
        d = np.abs(v[s:s + step, None] - lv[None, :])
        out[s:s + step] = np.argmin(d, axis=1).astype(np.uint8)
    return out.reshape(np.shape(values))


# ---------------------------------------------------------------------------
# 4-bit blockwise quantisation
# ---------------------------------------------------------------------------

def absmax_blocks(w: np.ndarray, blocksize: int = 64) -> np.ndarray:
    """Per-block max |w| in fp32 ([LC] 方法与公式 item 1: one constant per block).

    Blocks are consecutive runs of ``blocksize`` elements of the row-major
    flattened weight; a final partial block uses the elements present.
    """
    flat = np.asarray(w, dtype=np.float32).reshape(-1)
    nb = -(-flat.size // blocksize)
    out = np.empty(nb, dtype=np.float32)
    full = flat.size // blocksize
    if full:
        out[:full] = np.abs(flat[:full * blocksize].reshape(full, blocksize)).max(axis=1)
    if nb > full:
        out[full] = np.abs(flat[full * blocksize:]).max()
    return out


def quantize_nf4(w: np.ndarray, blocksize: int = 64):
    """W0 fp32 -> (codes uint8 [numel], absmax fp32 [nblocks]).

    n = w / absmax (IEEE fp32 division, correctly rounded), code = nearest NF4
    level.  A block whose absmax is 0 holds only zeros; its codes are the zero
    level (index 7).  Non-finite weights are rejected.
    """
    return quantize_blocks(w, nf4_codebook(), blocksize)


def quantize_blocks(w: np.ndarray, levels: np.ndarray, blocksize: int = 64):
    """Blockwise absmax quantisation onto any ascending 16-level codebook:
    n = w / absmax as above (n = 0 in an all-zero block), code = nearest level
    with ties to the lower index.  quantize_nf4 is this with the NF4 levels."""
    flat = np.asarray(w, dtype=np.float32).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite weights")
    a = absmax_blocks(flat, blocksize)
    per_elem = np.repeat(a, blocksize)[:flat.size]
    with np.errstate(divide="ignore", invalid="ignore"):
        n = np.where(per_elem > 0, flat / np.where(per_elem > 0, per_elem, np.float32(1)),
                     np.float32(0)).astype(np.float32)
    codes = nearest_index(n, levels)
    return codes, a


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte; element 2j goes in the HIGH nibble.

    The pages only say the weights are stored as 4-bit values (about half a
    byte per parameter, [LC] 与 baseline 对比 table).  Nibble order is the
    build's reading.
    """
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        raise ValueError("odd number of codes")
    return ((c[0::2] << 4) | (c[1::2] & 0x0F)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


# ---------------------------------------------------------------------------
# Double quantisation of the block constants
# ---------------------------------------------------------------------------

def _fixed_order_sum(a: np.ndarray, group: int) -> float:
    """fp64 sum in a fixed two-level order: a sequential sum inside each group of
    ``group`` consecutive values, then a sequential sum of the group sums in
    index order.  (np.add.accumulate is a strict left-to-right scan.)"""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    sums = []
    for s in range(0, a64.size, group):
        sums.append(float(np.add.accumulate(a64[s:s + group])[-1]))
    total = 0.0
    for v in sums:
        total = total + v
    return total


def double_quant(absmax: np.ndarray, dq_blocksize: int = 256, levels=None):
    """absmax fp32 [nb] -> (codes uint8 [nb], scales fp32 [ceil(nb/256)], mean fp32).

    [AU] Dubbele Quantisatie box / [LC] 方法与公式 item 2: the constants are
    quantised again to 8 bits.  Readings (the pages give no more detail):
      * one mean mu per tensor, subtracted first: mu = fp32(S / nb), S the
        fixed two-level fp64 sum of the constants;
      * centred c_b = fp32(a_b - mu);
      * one fp32 second-level scale per 256 consecutive constants,
        s_g = max |c_b| over the group;
      * 8-bit code = nearest level of the linear codebook to fp32(c_b / s_g),
        ties to the lower index; a group with s_g = 0 gets the zero code 127.
    ``levels`` replaces the linear codebook (e.g. dq_float8_codebook()); the
    code of a group with s_g = 0 is then the index of its zero level.
    """
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    mu = np.float32(_fixed_order_sum(a, dq_blocksize) / float(nb))
    c = (a - mu).astype(np.float32)
    ng = -(-nb // dq_blocksize)
    scales = np.empty(ng, dtype=np.float32)
    n2 = np.zeros(nb, dtype=np.float32)
    for g in range(ng):
        seg = c[g * dq_blocksize:(g + 1) * dq_blocksize]
        s = np.float32(np.abs(seg).max())
        scales[g] = s
        if s > 0:
            n2[g * dq_blocksize:(g + 1) * dq_blocksize] = (seg / s).astype(np.float32)
    codes = nearest_index(n2, dq_codebook() if levels is None else levels)
    return codes, scales, mu


def dequant_absmax(codes: np.ndarray, scales: np.ndarray, mean, dq_blocksize: int = 256,
                   levels=None):
    """a_hat_b = fp32( fp32(Q8[code_b] * s_g) + mu ): two separately rounded fp32 ops
    (Q8 the linear codebook, or ``levels``)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    q8 = dq_codebook() if levels is None else np.asarray(levels, dtype=np.float32)
    s = np.repeat(np.asarray(scales, dtype=np.float32), dq_blocksize)[:c.size]
    prod = (q8[c] * s).astype(np.float32)
    return (prod + np.float32(mean)).astype(np.float32)


# ---------------------------------------------------------------------------
# Dequantisation to the compute type
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bits.

    bf16 is the compute type on every page that names one ([AG] code block;
    [LC] 实现要点; [LI] §3).  Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = (u >> 16) & 1
    return ((u + 0x7FFF + keep) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return ((np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16)
            .view(np.float32).astype(np.float64))


def dequant_nf4(packed: np.ndarray, codes: np.ndarray, scales: np.ndarray, mean,
                N: int, K: int, blocksize: int = 64, dq_blocksize: int = 256, levels8=None):
    """(packed, 8-bit codes, scales, mean) -> (w_hat fp32 [N,K], bf16 bits [N,K]).

    w_hat = fp32(Q4[nibble] * a_hat_block); the bf16 weight fed to the matmul is
    RNE(w_hat) ([AU] DATASTROOM box: dequantise per layer, on the fly;
    [LC] 直觉与动机: back to bf16 for the matrix product).
    """
    nib = unpack_nibbles(packed)[:N * K]
    a_hat = dequant_absmax(codes, scales, mean, dq_blocksize, levels=levels8)
    w_hat, wb = dequant_codes(nib, a_hat, blocksize)
    return w_hat.reshape(N, K), wb.reshape(N, K)


def dequant_codes(codes4: np.ndarray, a_hat: np.ndarray, blocksize: int = 64, levels=None):
    """4-bit codes [nblk*blocksize] and the decoded constant of each of their
    blocks [nblk] -> (w_hat fp32, bf16 bits), w_hat = fp32(Q4[code] * a_hat).
    ``levels`` is the 16-level codebook (default NF4).

    Works on any whole-block subset of a weight (blocks are independent)."""
    lv = nf4_codebook() if levels is None else np.asarray(levels, dtype=np.float32)
    c = np.asarray(codes4, dtype=np.uint8).reshape(-1)
    per_elem = np.repeat(np.asarray(a_hat, dtype=np.float32), blocksize)[:c.size]
    w_hat = (lv[c] * per_elem).astype(np.float32)
    return w_hat, f32_to_bf16_bits(w_hat)


# ---------------------------------------------------------------------------
# Storage accounting
# ---------------------------------------------------------------------------

def bits_per_param(numel: int, blocksize: int = 64, dq_blocksize: int = 256,
                   double: bool = True) -> float:
    """Storage cost per parameter from the actual buffer sizes.

    Without double quantisation: 4-bit codes + one fp32 constant per block.
    With it: 4-bit codes + one 8-bit code per block + one fp32 scale per
    dq-group + one fp32 mean per tensor.
    """
    nb = -(-numel // blocksize)
    bits = 4.0 * numel
    if double:
        ng = -(-nb // dq_blocksize)
        bits += 8.0 * nb + 32.0 * ng + 32.0
    else:
        bits += 32.0 * nb
    return bits / numel
