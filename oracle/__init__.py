"""CPU oracle for the fused exact-attention forward pass — TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports it, calls it or falls back to it.

The oracle is plain numpy in float64.  It materialises the full score matrix
for each (batch, head) -- exactly what the fused method avoids -- applies the
score modifiers and the mask, then takes the softmax and the product with V.

Sources (pages, cited by title and section):
  * "FlashAttention 4: Γρηγορότερη και Αποδοτική σε Μνήμη Προσοχή για LLMs"
    (el.linux-konsole.com) -- section "Εισαγωγή" (introduction): attention
    multiplies queries by keys, normalises with a softmax, then multiplies by
    the values; section "Γιατί οι πυρήνες προσοχής..." (why attention kernels
    dominate cost): only the per-row maximum and sum are kept per query row.
  * "PyTorchs FlexAttention mit FlashAttention-4 ist ein Game-Changer"
    (liora.io) -- opening section: the score/mask variants ALiBi, sliding
    window, document masking and soft-capping; section "Aktuelle
    Einschränkungen": block sparsity (skipping fully masked blocks).
  * "FlashAttention-3: Rekordverdächtige Geschwindigkeit und Präzision bei
    AI-Modellen" (ctol-digital.de) -- section "Analyse": FP8 with block
    quantisation, and the processing against outlier features read as
    incoherent processing (quant.py).

Every function is pinned by the CPU tests (brute force, library special cases,
closed forms and invariants); see tests/test_oracle_*.py.
"""

from .decode import decode_bf16, decode_e4m3, dequant_blocks, decode_problem  # noqa: F401
from .attention import (  # noqa: F401
    default_alibi_slopes,
    visible,
    scores_ref,
    attention_ref,
    attention_problem,
    attention_varlen_ref,
    varlen_doc_ids_ref,
)
from .blockmap import blockmap_ref, row_intervals_ref, visible_pairs_ref  # noqa: F401
from .quant import e4m3_encode, hadamard, quantize_blocks_ref, rotation, signs_from_bits  # noqa: F401
from .attention_bwd import attention_bwd_ref, attention_bwd_problem  # noqa: F401
from . import fp4  # noqa: F401
