"""CPU oracle for paged single-query attention and the two paging helpers.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call
or execute anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
constants or helpers with the HIP path.

Everything is plain numpy in float64 (inputs are fp16 and are widened
exactly).  Where the pages fix a result with a plain definition the oracle is
that definition written out:

* attention for one query token over a sequence's keys and values
  ("PagedAttention", e-fortepiano.pl, section "Formulació matemàtica");
* the paged cache is that same attention after mapping logical blocks to
  physical blocks through a block table (same page, section "Descripció");
* appending a token writes it into the slot its block table names, and a
  copy-on-write duplicates a whole physical page ("Atención paginada en
  modelos de lenguaje grandes (LLM)", 7minutos.es, the PagePool /
  PagedRequest part and the prefix-sharing part).

Pins (tests/test_oracle.py) tie every function to something other than
itself: closed forms, torch's float64 scaled-dot-product attention on the
CPU, a pure-Python brute force, and the invariants the pages state.
"""

from .paged_attention import (  # noqa: F401
    BLOCK_TOKENS,
    attention_ref,
    blockwise_attention_ref,
    gather_ref,
    pool_element_index,
    paged_decode_ref,
)
from .cache_ops import append_ref, cow_ref  # noqa: F401
from .grouped import grouped_decode_ref, grouped_tables_ref  # noqa: F401
from .prefill import paged_prefill_ref  # noqa: F401
from .contiguous import contiguous_decode_ref  # noqa: F401
