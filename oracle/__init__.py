"""CPU oracle for the weight-only quantized decode linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports or calls it, and it
imports nothing from the product: the two share only the seeded input
generators in ``wqd_inputs``.

It computes, plainly and slowly, what the decode linear layer computes:

* ``formats``: bfloat16 / float16 / FP8-E4M3 rounding and decoding, in float64;
* ``quant``:   the three weight formats (bf16, FP8-E4M3 + per-row fp32 scale,
  W4A16 = uint4 codes in groups of 128 with an fp16 scale and a uint4 zero
  point) and their exact dequantisation;
* ``gemm``:    y = x . dequant(W)^T in float64, rounded once to bf16; the
  SwiGLU of a gate/up pair, silu(x . gate^T) * (x . up^T);
* ``spec``:    the speculative-sampling accept / reject step over the verify
  pass's target and draft distributions;
* ``w8a8``:    the W8A8-FP8 variant: one dynamic E4M3 scale for the whole
  activation tensor, activation codes, and the product of the two code
  matrices (exact in float64) times both scales;
* ``attention``: decode attention over a KV cache with grouped-query heads
  (one query per sequence, softmax over its first len positions), from a bf16
  cache or from an FP8-E4M3 one (one scale per tensor for K and for V);
* ``bytes``:   the bytes a call or a step moves (codes, scales, zero points,
  activations; KV cache per sequence) and the step's lower bound, as the
  pages define them.

Pins (tests marked ``not gpu``): exhaustive E4M3 decode against its closed
form and against the printed maximum 448; a brute-force nearest-value encoder;
bf16/fp16 rounding against torch's and numpy's conversions and hand-built
boundary cases; W4A16 codes against a brute-force argmin over the 16 grid
points; the products against exact rational arithmetic on tiny shapes and
against special cases (integer matmul, identity, zero); the accept / reject
step against the pages' worked three-token example, the theorem that its output
is distributed as the target (integrated over a grid of the uniforms), a
pure-Python inverse-CDF walk and its special cases; the byte model against the
byte counts and bounds the pages print (70e9 parameters in three formats, the
KV cache of a 2,048-token sequence, the batch-1 and batch-32 floors, the CS336
4096 x 4096 INT4 count); the FP8 dequantisation against the round-to-nearest
error bound on the original weights; the W8A8 product against exact rationals,
activation codes against a brute-force nearest E4M3 value, activations on the
E4M3 grid reducing to the weight-only product, and the activation rounding
bound; decode attention against closed forms (one position, equal keys, a
dominant key, a 3:1 split), invariances, per-group values and torch's float64
scaled-dot-product attention; the FP8 cache's codes against a brute-force
nearest E4M3 value and its saturation, and attention over an FP8 cache with
power-of-two scales (every value exact in bf16) against the bf16 attention on
the same values.  No function here is
"parity unpinned".
"""
from .formats import (  # noqa: F401
    BF16_MAX,
    E4M3_MAX,
    bf16_bits_from_value,
    bf16_bits_to_f64,
    bf16_round,
    bf16_to_bits,
    e4m3_decode,
    e4m3_encode,
    fp16_round_f32,
)
from .gemm import qgemm_exact, qgemm_ref, silu, swiglu_exact  # noqa: F401
from .quant import (  # noqa: F401
    FMTS,
    GROUP,
    dequant_exact,
    dequant_f32,
    fp8_row_scales,
    quantize,
    quantize_bf16,
    quantize_fp8,
    quantize_w4a16,
    w4a16_group_params,
)
from .attention import (  # noqa: F401
    decode_attention_exact,
    decode_attention_fp8kv_exact,
    decode_attention_fp8kv_ref,
    decode_attention_ref,
    quantize_kv_fp8,
)
from .w8a8 import act_scale, qgemm_w8a8_exact, qgemm_w8a8_ref, quantize_act  # noqa: F401
from .spec import accept, draw_units, inverse_cdf_draw, residual, spec_accept, spec_accept_one  # noqa: F401
