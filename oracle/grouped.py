"""Float64 reference for decoding groups of sequences that share leading blocks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Sources, by page and section:

* "PagedAttention" (e-fortepiano.pl), section "Descripció": physical blocks
  are reference counted and shared between requests or between the decoding
  branches of one request (parallel sampling, beam search); every branch
  still attends to its own sequence, so sharing changes where the keys and
  values live, not what is computed.
* "Atención paginada en modelos de lenguaje grandes (LLM)" (7minutos.es),
  prefix-sharing part: a fork shares every page of its owner, and a page is
  copied before a holder writes into it, so the pages two branches still
  share are whole (full) pages at the front of their tables.

What a grouped call computes is therefore the plain per-sequence decode of
``paged_attention.paged_decode_ref``; this module only spells out how the
call's grouping arguments are read (a contract of this library, not of the
pages):

* group g holds the consecutive sequences
  ``[group_offsets[g], group_offsets[g+1])`` (offsets clamped into [0, B];
  a group with a negative size is empty); only its first ``max_group_size``
  members are decoded, the others and sequences in no group get zero rows;
* the group's first ``shared_blocks[g]`` logical blocks are read through the
  table row of its first member, for every member, after clamping that count
  into [0, min over the decoded members of full blocks (context // 16)].
  With tables that really share those blocks (the block manager's output),
  this is exactly each member's own table.
"""

import numpy as np

from .paged_attention import BLOCK_TOKENS, paged_decode_ref


def grouped_tables_ref(block_tables, context_lens, group_offsets, shared_blocks,
                       max_group_size, ctx_limit=None):
    """The block table and context length each sequence is decoded with under
    the grouping contract above (zero length for sequences not decoded)."""
    tables = np.array(block_tables, dtype=np.int64, copy=True)
    lens = np.asarray(context_lens, dtype=np.int64)
    if ctx_limit is not None:
        lens = np.clip(lens, 0, ctx_limit)
    lens = np.maximum(lens, 0)
    B = lens.shape[0]
    out_lens = np.zeros(B, dtype=np.int64)
    offs = np.clip(np.asarray(group_offsets, dtype=np.int64), 0, B)
    for g in range(len(offs) - 1):
        lo = int(offs[g])
        n = min(max(int(offs[g + 1]) - lo, 0), max_group_size)
        if n == 0:
            continue
        members = range(lo, lo + n)
        full = min(int(lens[b]) // BLOCK_TOKENS for b in members)
        s = min(max(int(shared_blocks[g]), 0), full)
        for b in members:
            tables[b, :s] = tables[lo, :s]
            out_lens[b] = lens[b]
    return tables, out_lens


def grouped_decode_ref(q, k_pool, v_pool, block_tables, context_lens, group_offsets,
                       shared_blocks, scale, max_group_size=16, ctx_limit=None):
    """Decode every sequence of the batch under the grouping contract; float64
    [B][H][D], zero rows for sequences that are not decoded."""
    tables, lens = grouped_tables_ref(block_tables, context_lens, group_offsets, shared_blocks,
                                      max_group_size, ctx_limit)
    return paged_decode_ref(q, k_pool, v_pool, tables, lens, scale)
