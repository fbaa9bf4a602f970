"""CPU oracle for paged decode attention and the paged KV cache operations.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in this package.  The library under
``paged_kv_cache_116_amd/`` never imports it, and this package imports nothing
from the library: the two share no code, tables or helpers.

Everything here is plain, slow and written to be checked by eye against the
pages that define the method.  Floating point work is done in float64
(widening float32 / bfloat16 / float16 inputs to float64 is exact).  Integer
and byte work (block-table resolution, cache append, block copy, the block
manager) is exact by construction.

Sources, cited in the modules by tag and section:

  [pofe]    "PagedAttention: paging the KV cache" (pofe.ai)
  [lesson]  "PagedAttention" lesson in "How Text Is Generated"
            (learn.pranaymahendrakar.com)
  [note]    "PagedAttention: Manage the Cache Without Moving the Sequence"
            (neelmishra.github.io)
  [claims]  "Paged Attention" (firehose-demo claims page)
  [arch]    "PagedAttention: Virtual-Memory KV Cache Management, Continuous
            Batching, and PyTorch Architecture" (ailinkdeeptech.com)

Modules:
  paging        block-table resolution, explicit gather, slot accounting
  attention     decode attention by explicit gather + two-pass softmax,
                the block-wise online-softmax recurrence, the
                log-sum-exp merge of partition states, and causal
                chunked prefill over the paged history
  cache_ops     cache append (one or several tokens per sequence) and
                block copy on pool copies
  fp8           E4M3FN codes for FP8 cache blocks: encode, decode, append
  block_manager free list, reference counts, fork, copy-on-write and
                preemption by swapping
  prefix_cache  automatic prefix caching: block-aligned prefixes of token
                ids looked up and shared, evictable cached blocks
  allocator_toy contiguous-reservation vs paged accounting of a toy workload

Every function in this package is pinned by a ``-m "not gpu"`` test against
values printed on the pages, closed forms, brute force or an independent
library routine.  The FP8 scale convention (a code stands for
decode(code) * scale) is a reading, not a page's statement; it is pinned by
the round trip that any scale convention must satisfy (a stored code gives
back the value it was written for, within half an E4M3 step, at scales other
than 1), which an inverted scale fails.  Planted mistakes in each function
(wrong index, sign, term, operand, rounding, order or threshold) were checked
to fail at least one pin.
"""

from . import paging, attention, cache_ops, block_manager, allocator_toy, fp8  # noqa: F401
