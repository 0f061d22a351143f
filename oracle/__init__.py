"""CPU oracle for the exact-attention forward pass and its FP8 variant.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here. The product
path (the HIP library and its Python binding) never imports, calls or links it,
and shares no code with it.

Everything is plain NumPy in float64 unless a function states that it mirrors
a float32 decision (the FP8 quantizer takes its rounding decisions in float32,
the precision the quantize kernel uses).

Sources, cited by page title and section:

* [NL]  "FlashAttention-3 (NL)" (systems-analysis.info), and its Greek mirror
  "FlashAttention-3 (EL)".
* [GN]  "FlashAttention-3: Schnellere und präzisere Attention durch
  Asynchronität und geringe Präzision" (GeekNews, de.news.hada.io).

Parity pins for every function are in ``tests/test_oracle.py``; the one
function without an external pin is listed as "parity unpinned" in its own
docstring (``fp8_attention_sim``: only the ratio of its two error figures is
pinned by the pages).
"""

from .attention import (  # noqa: F401
    attention,
    attention_rows,
    attention_tiled,
    attention_partial,
    merge_partials,
    allowed_mask,
)
from .varlen import attention_varlen  # noqa: F401
from .backward import attention_backward  # noqa: F401
from .hadamard import sylvester, fwht, random_sign_hadamard  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize_blocks,
    quantize_per_tensor,
    hadamard_quantize,
    dequantize_blocks,
)
from .fp8_pipeline import (  # noqa: F401
    fp8_attention_sim, fp8_attention_rows, p_rounding_bound, p_rounding_lse_bound, round_p, rmse, P_EXP_RANGE)
from .rope import rope_angles, rotary, rotary_f32, rope_hadamard_quantize  # noqa: F401
