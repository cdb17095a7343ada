"""CPU fp64 oracle for sliding-window attention (SWA) — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``sliding_window_attention_amd``) never imports, calls or links anything here,
and this package imports nothing from the product: the two share no code.

Everything is float64 NumPy.  Each function follows one passage of the source
pages, cited by page title and section.  Short tags used in citations:

  [KB]  "Sliding Window Attention", LLM architecture knowledge base
        (lizeman.github.io/llm-arch-kb/attention/sliding-window/)
  [MB]  "How Sliding Window Attention Works" (mbrenndoerfer.com)
  [G3]  "Sliding Window Attention — Gemma 3" study note
        (ai-engineer-exhaustive.pages.dev/research/gemma3/gemma3-sliding-window)
  [PP]  "Sliding Window Attention: From Local Windows to Global Context"
        (prathamp.com/blog/attention-sliding-window)
  [ST]  "Sliding Window Attention (SWA)" glossary entry (superteams.ai)

Modules
  index_sets  connectivity sets S_t (causal, symmetric/dilated/global, ring decode)
  attention   masked softmax attention over those sets (+ the dense-mask form)
  ring        the rolling-buffer KV cache write rule (one token or a chunk)
  tiles       brute-force band-tile classification for a (BM, BN) tiling
  rope        rotary position embedding (rotate-half form) for the fused-RoPE variant

Pins: every function here is pinned in ``tests/test_oracle_pins.py`` against the
pages' printed tables and examples, closed forms, textbook special cases
(``torch.nn.functional.scaled_dot_product_attention`` in float64) and brute force.
Output values at the large synthetic workloads have no printed values on the
pages; there the fp64 definition itself is the reference ("parity unpinned"
beyond the special cases and invariants listed in the tests).
"""

from .index_sets import (
    causal_index_set,
    causal_dilated_index_set,
    causal_sink_index_set,
    symmetric_index_set,
    longformer_index_set,
    decode_index_set,
    causal_mask,
    longformer_mask,
)
from .attention import (
    attend,
    swa_prefill,
    swa_decode,
    swa_prefill_cached,
    swa_longformer,
    dense_masked_attention,
)
from .ring import ring_write, ring_slot, ring_append, ring_from_sequence
from .tiles import band_tiles_bruteforce
from .rope import rope_rotate_half

__all__ = [
    "causal_index_set",
    "causal_dilated_index_set",
    "rope_rotate_half",
    "symmetric_index_set",
    "longformer_index_set",
    "decode_index_set",
    "causal_mask",
    "longformer_mask",
    "attend",
    "swa_prefill",
    "swa_decode",
    "swa_longformer",
    "dense_masked_attention",
    "ring_write",
    "ring_from_sequence",
    "band_tiles_bruteforce",
]
