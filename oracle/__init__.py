"""CPU oracle for group-wise round-to-nearest weight quantization and the
fused-dequantization matrix-vector product.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library; the two agree only through the byte layout and
arithmetic that the docstrings below define.

The oracle is plain and slow on purpose: numpy, scalar formulas per group, an
explicit nearest-value search over each format's code table, and an fp64
matrix-vector product.  Sources for what it computes:

* RTN as the quantizer, data-free and one-shot -- Kogan, "Is (Selective)
  Round-To-Nearest Quantization All You Need?", abstract.
* INT8 as the up-precision format for selected layers -- same page, abstract
  and method section ("from INT4 to INT8").
* FP4 in sign-magnitude form with a redundant negative zero, and RaZeR's
  remapping of that code to a special value chosen per group -- Chen et al.,
  "The Power of Negative Zero: Datatype Customization for Quantized Large
  Language Models", abstract and method section.
* Separate scales for positive and negative values, with no more storage than
  asymmetric INT -- Zhang et al., "AFPQ: Asymmetric Floating Point
  Quantization for LLMs", abstract.
* Block formats that share a scale across packed numbers, and the 6-bit width
  implied by the stated 5x memory density over float32 -- Zhang et al.,
  "Revisiting Block-based Quantisation: What is Important for Sub-8-bit LLM
  Inference?", abstract.

Where the pages leave a step open (rounding ties, scale formulas, code layout)
the oracle takes one reading; each is stated at the function that uses it.
Parity unpinned by the pages (fixed by our reading and checked for internal
consistency only): the INT4 range [min(w,0), max(w,0)], RaZeR's per-candidate
scale absmax/max(6,|v|) and its fp64 SSE tie order, the canonical +0 code,
AFPQ's scale formulas, the BFP exponent/mantissa alignment, INT8 symmetry,
and the clipping search's ratio grid (20 - c) / 20 and tie order (the pages
name clipping without a procedure; the search itself is pinned by brute force
in exact rational arithmetic and by its invariants).
"""

from .formats import (  # noqa: F401
    FORMATS,
    E2M1_MAGNITUDES,
    RAZER_SPECIALS,
    Quantized,
    quantize,
    dequantize,
    quantize_clipped,
    clip_bound,
    CLIP_MAX_CANDIDATES,
)
from .layout import pack, unpack, packed_nbytes, buffer_nbytes, device_bytes  # noqa: F401
from .gemv import gemv_f64  # noqa: F401
from .attn import attn_decode_f64, kv_rows  # noqa: F401
from .w8a8 import quantize_activations, integer_product, gemm_w8a8  # noqa: F401
