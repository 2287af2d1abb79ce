"""Plain, slow CPU oracle for paged decode attention and its cache kernels.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (``paged_kv_cache_433_amd``) never imports it and
shares no code with it: the two meet only at the seeded input arrays.

Every result is computed from its plain definition in float64 (attention) or
as an exact bit copy (slot scatter, copy-on-write, swapping), citing the page
passage it follows:

* "vLLM: Anatomy and Mechanisms of High-Throughput LLM Inference", section
  "PagedAttention: The vLLM Innovation" / "Block-Level Management" (block
  tables map logical blocks to physical blocks; 16-token default block) and
  "Memory Sharing via Copy-on-Write (CoW)" (only the diverging block is
  copied) and "Preemption and Recovery" (evicted KV blocks move to CPU RAM);
* "Inside vLLM: Anatomy of a High-Throughput LLM Inference System", section
  "Scheduler" (a decode step runs over the most recent token with every
  earlier K/V vector already cached) and section "LLM Engine constructor"
  (per-block size 2 * block_size * num_kv_heads * head_size * dtype bytes);
* "vLLM Internals", section "The Block Manager" (per-request block tables;
  a preempted request's blocks are swapped to CPU and back);
* "vLLM: Anatomy and Mechanisms", section "Prefix Caching" (prompts with a
  common beginning reuse the cached blocks), read with the CoW section for
  ``decode_shared``, and for trees of shared prefixes in ``decode_shared_tree``.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against facts the pages or mathematics fix (a library routine on the dense
special case, closed forms, invariants, the pages' worked example). No
function is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    bf16_bits_to_f64,
    copy_blocks,
    decode,
    decode_multi,
    decode_shared,
    decode_shared_tree,
    decode_sequence,
    reshape_and_cache,
    swap_blocks,
)
