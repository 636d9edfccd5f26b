"""CPU oracle for the QLoRA NF4 linear layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy code written from the pages' description
of QLoRA.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The HIP library never calls, links or loads
anything here, and nothing here imports the HIP package: the two sides share
only the seeded input generators in ``qlora_workloads``.

Pages cited (titles as printed on each page):
  [AG] aigrafen.se "QLoRA"
  [AU] auryth.ai glossary "QLoRA" (Dutch)
  [LC] llm-compass "QLoRA" (brenchcc.github.io, Chinese)
  [SB] skillbyai "QLoRA: Fine-Tuning on One Consumer GPU"
  [LI] learn-interview-questions "QLoRA (Quantized Low-Rank Adaptation):
       4-bit NormalFloat (NF4) & Paged Optimizers"
Outside the pages: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011) for the dropout mask.

Functions and what pins them (tests/test_oracle_*.py):
  nf4_codebook      three independent inverse-normal routes, equal-probability
                    spacing of the quantiles, structure (-1, 0, +1 exact)
  nearest_index     exact rational arithmetic on tiny inputs; midpoint search
  quantize_nf4      round trip of codebook values, reconstruction error bound
  double_quant      bit budget printed on the pages (0.37 / ~0.4 bit saved,
                    ~0.5 -> ~0.13 bit overhead), exact mean via math.fsum,
                    error bound of the linear 8-bit code
  dequant           round trip, bound, bf16 rounding checked against torch
  forward/backward  exact directional derivatives, special cases (B=0, A=0,
                    X=I, one-hot dY), fp64 torch autograd
  silu glue         fp64 torch autograd
  merge             B = 0 reduces to the dequantised base; constant
                    adapters give the closed form W + alpha a b; hand-worked
                    bf16 rounding ties; bf16 rounding against torch
  philox            the published Philox4x32-10 known-answer vectors; the
                    same round function at 64-bit width against numpy's
                    Philox bit generator
  dropout           keep rate within binomial bounds, p = 0 is the identity,
                    counter-based (row subsets equal slices), scale exact;
                    forward/backward with the mask fixed: all-kept reduces to
                    the plain layer, exact directional derivatives
  int4 codebook     even spacing, round trip, error bound; NF4 beats it on
                    Gaussian blocks in error and in code entropy, as the
                    pages argue
  float8 DQ table  its values against torch's own float8_e4m3fn decoding of
                    all 256 bit patterns; count, range, symmetry, exact zero;
                    round trip of the levels; nearest-level bound; fewer
                    absmax reconstruction errors than the linear code on a
                    heavy-tailed group
No function is "parity unpinned".
"""
from .nf4 import (  # noqa: F401
    NF4_DELTA, nf4_codebook, dq_codebook, int4_codebook, fp8_e4m3_values, dq_float8_codebook,
    nearest_index, absmax_blocks,
    quantize_nf4, quantize_blocks, pack_nibbles, unpack_nibbles, double_quant, dequant_absmax,
    dequant_nf4, dequant_codes, f32_to_bf16_bits, bf16_bits_to_f64, bits_per_param,
)
from .qlora import (  # noqa: F401
    lora_scale, forward, backward, silu_mul_forward, silu_mul_backward,
    mlp_forward, mlp_backward, merge, f64_to_bf16_bits,
)
from .dropout import (  # noqa: F401
    philox, philox4x32_words, dropout_threshold, dropout_scale, dropout_mask, dropout_apply,
    pack_mask, forward_dropout, backward_dropout,
)
