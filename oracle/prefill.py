"""Float64 reference for paged prefill: several query tokens per sequence
attending causally over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Sources, by page and section:

* "PagedAttention" (e-fortepiano.pl), section "Formulació matemàtica": the
  attention is that of causal self-attention, computed block by block over
  the paged cache; for a query token the keys it sees are those of the
  tokens up to and including its own position.
* same page, section "Descripció": the cache of a sequence is reached
  through its block table, whatever the physical placement of its blocks.
* "Atención paginada en modelos de lenguaje grandes (LLM)" (7minutos.es),
  PagePool / PagedRequest part: a request's tokens are appended slot by slot
  as they are processed, so a prompt is written into its pages before (or
  while) it is attended to.

Readings where the pages are silent:

* a prefill call processes, for every sequence b, its last
  ``n_b = query_start[b+1] - query_start[b]`` cached tokens as queries (the
  prompt, or one chunk of it, already appended); query row i of sequence b
  sits at position ``p = context_lens[b] - n_b + i`` and attends to
  positions 0 .. p of the same sequence (its own token included, as in the
  decode);
* rows whose position would be negative (more queries than cached tokens)
  are zero rows, like a sequence with no context in the decode;
* the scale is the caller's, as in the decode.
"""

import numpy as np

from .paged_attention import attention_ref, gather_ref


def paged_prefill_ref(q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                      seqs=None):
    """q: [Tq][H][D] fp16 (rows of sequence b: query_start[b] ..
    query_start[b+1]-1); pools and tables as for ``paged_decode_ref``.
    Returns float64 [Tq][H][D]; with ``seqs`` only those sequences' rows are
    computed (the others are NaN)."""
    q = np.asarray(q)
    Tq, H, D = q.shape
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.full((Tq, H, D), np.nan, dtype=np.float64)
    B = len(qs) - 1
    for b in (range(B) if seqs is None else seqs):
        ctx = int(context_lens[b])
        n = int(qs[b + 1] - qs[b])
        K = gather_ref(k_pool, block_tables[b], ctx, H, D)
        V = gather_ref(v_pool, block_tables[b], ctx, H, D)
        for i in range(n):
            p = ctx - n + i
            out[qs[b] + i] = attention_ref(q[qs[b] + i], K[:p + 1], V[:p + 1], scale) \
                if p >= 0 else 0.0
    return out
