"""Float64 reference for decode over a contiguous KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Source: "PagedAttention" (e-fortepiano.pl), sections "Limitacions i
alternatives" and "Atenció": vAttention keeps each request's keys and values
contiguous in (virtual) memory, one [context][heads][dim] tensor per layer
for the request, and keeps the standard attention computation unchanged.
Here the batch's caches are one array of rows: sequence b's token t is row
b * row_tokens + t.  The output is the plain single-query attention of
``paged_attention.attention_ref`` over the sequence's first context_lens[b]
rows.
"""

import numpy as np

from .paged_attention import attention_ref


def contiguous_decode_ref(q, k_rows, v_rows, row_tokens, context_lens, scale):
    """q: [B][H][D] fp16; k_rows, v_rows: [rows][H][D] fp16 with sequence b at
    rows b*row_tokens ..; returns float64 [B][H][D]."""
    q = np.asarray(q)
    B, H, D = q.shape
    out = np.empty((B, H, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        lo = b * row_tokens
        out[b] = attention_ref(q[b], k_rows[lo:lo + n], v_rows[lo:lo + n], scale)
    return out
