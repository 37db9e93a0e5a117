"""Float64 CPU oracle for exact attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library under
``paged_kv_flashattention_amd/``; the two meet only through the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

Every function here states the passage of the source pages it follows.  The
pages are cited by title and section:

* "8. Kernels and Attention Backends" (igniting.github.io inference guide),
  sections "Attention is an I/O problem", "Counting attention's traffic",
  "Test the kernel at three levels".
* "The Stack Below the Stack (Part 2): Below Python" (desigeek), sections
  2.1 "Kernel fusion" (online softmax), 2.2 "Flash-Decoding", 5 (the
  FlexAttention causal mask ``q_idx >= kv_idx``).
* "Inside Ion: Custom Attention Kernels for NVIDIA Grace" (cumuluslabs.io),
  "IonAttention in One Paragraph" (paged KV, eager KV writeback).

``oracle/fp8.py`` adds the FP8 (E4M3) page format: decode, a nearest-value
encoder, the pool quantiser and the quantising page write.

Parity status: every function below is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_fp8.py`` (brute force, a library routine, closed forms and
invariants).  No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    gather_sequence_kv,
    attend_rows,
    attention_ref,
    attention_rows_ref,
    block_map_mask,
    softmax_probs_ref,
    tiled_attend_rows,
    split_partials_ref,
    merge_ref,
    kv_write_ref,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize_ref,
    dequantize_pool,
    kv_write_fp8_ref,
    page_scales,
)
