"""CPU fp64 oracle for per-rank ring attention under the head-tail (zigzag) layout.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``context_ring_attention_zigzag_amd``) and imports nothing from it.

Pages this oracle follows (cited by title and section):

* "Context Parallelism" (Ultralytics glossary), sections "How context
  parallelism works" and "Practical use and trade-offs".
* "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)"
  (orangingq.tistory.com), sections "Context Parallelism (CP)" and
  "Implementation quirk: symmetric chunk assignment".
* the Megatron page's "Implementation quirk" also fixes that rotary position
  embeddings take global positions (``oracle/rope.py``);
* "Sequence Parallelism and Ring Attention" (aiunderstanding.org), sections
  "Deep dive", "Technical insight", "The future of sequence parallelism and
  ring attention" (striped layout) and the FAQ.

Every function here is pinned by ``tests/test_oracle.py`` to something other
than itself (brute force, a library routine, closed forms, the pages' cp=4
table; the rotary frequencies theta_j by hand-computed angles for every pair
j, checked with scalar math.cos / math.sin). No function is "parity unpinned".
"""

from .rope import HALF, INTERLEAVED, rope, rope_pairs, rope_theta  # noqa: F401
from .ring_attention import (  # noqa: F401
    CONTIGUOUS,
    STRIPED,
    ZIGZAG,
    allowed_mask,
    attention_backward,
    causal_pairs_striped,
    causal_pairs_zigzag,
    count_pairs,
    finalize,
    fold_block,
    full_attention,
    init_state,
    kv_head,
    layout,
    merge,
    padded_len,
    rank_reference,
    ring_backward,
    rows_backward,
    ring_emulation,
    ring_source,
)
