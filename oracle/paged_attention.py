"""Float64 reference for single-query attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Sources, by page and section:

* "PagedAttention" (e-fortepiano.pl, Catalan encyclopedia article),
  section "Formulació matemàtica": for one query token of causal
  self-attention the output is the softmax over ``q.k_t / sqrt(d)`` of the
  keys seen so far, used to weight the values; with the cache cut into
  blocks of B tokens the same result is computed block by block, one score
  vector per block, which the article says preserves the attention result.
* same page, section "Descripció": a sequence's cache is a run of logical
  blocks, and a block table maps each logical block to a physical block
  anywhere in GPU memory.
* "Atención paginada en modelos de lenguaje grandes (LLM)" (7minutos.es),
  PagePool part: pages of 16 tokens each.

Readings where the pages are silent:

* the scale is supplied by the caller (the workloads pass 1/sqrt(D) as a
  float32); the oracle widens it to float64;
* the query attends to every cached token of its sequence, its own
  included (the caller appends the new token before decoding);
* a sequence with no cached tokens produces a zero output row;
* the physical layout of one pool (K or V) is
  ``[num_blocks][H][D/8][16][8]``: inside the tile of one (block, head)
  the head dimension is cut into groups of eight consecutive values, and
  each group stores its eight values for token 0, then token 1, ... up to
  token 15.  ``pool_element_index`` spells this out element by element.
"""

import numpy as np

# Tokens per page ("Atención paginada ...", 7minutos.es, PagePool part:
# "each with 16 tokens").
BLOCK_TOKENS = 16
# Values of one head dimension stored together for one token in a tile.
_GROUP = 8


def pool_element_index(block, head, token, dim, num_heads, head_dim):
    """Flat fp16 element index of value ``dim`` of ``token`` (0..15 inside its
    block) for ``head`` in physical ``block`` of a pool laid out as
    ``[num_blocks][H][D/8][16][8]``."""
    group, within = divmod(dim, _GROUP)
    tile = block * num_heads + head
    return ((tile * (head_dim // _GROUP) + group) * BLOCK_TOKENS + token) * _GROUP + within


def _tiles(pool, num_heads, head_dim):
    """View a pool (any shape, fp16) as [num_blocks][H][D/8][16][8]."""
    flat = np.asarray(pool).reshape(-1)
    per_block = num_heads * head_dim * BLOCK_TOKENS
    if flat.size % per_block:
        raise ValueError("pool size is not a whole number of blocks")
    return flat.reshape(flat.size // per_block, num_heads, head_dim // _GROUP,
                        BLOCK_TOKENS, _GROUP)


def gather_ref(pool, table, n, num_heads, head_dim):
    """Logical tokens 0..n-1 of one sequence as a contiguous float64
    ``[n][H][D]`` array: token t lives in physical block ``table[t // 16]`` at
    position ``t % 16`` ("PagedAttention", e-fortepiano.pl, "Descripció")."""
    tiles = _tiles(pool, num_heads, head_dim)
    out = np.empty((n, num_heads, head_dim), dtype=np.float64)
    for t in range(n):
        blk = int(table[t // BLOCK_TOKENS])
        if not 0 <= blk < tiles.shape[0]:
            raise IndexError(f"token {t}: physical block {blk} outside the pool")
        # tiles[blk, h, g, pos, w] is dim g*8+w of head h
        out[t] = tiles[blk, :, :, t % BLOCK_TOKENS, :].reshape(num_heads, head_dim)
    return out


def attention_ref(q, K, V, scale):
    """Single-query attention, plain definition ("PagedAttention",
    e-fortepiano.pl, "Formulació matemàtica").

    q: [H][D]; K, V: [n][H][D]; returns float64 [H][D] with
    ``out[h] = sum_t softmax_t(scale * q[h].K[t,h]) * V[t,h]``.
    An empty context gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    if n == 0:
        return np.zeros(q.shape, dtype=np.float64)
    scores = float(scale) * np.einsum("hd,nhd->hn", q, K)       # [H][n]
    top = scores.max(axis=1, keepdims=True)                     # for exp range only
    weights = np.exp(scores - top)
    norm = weights.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", weights, V) / norm


def blockwise_attention_ref(q, K, V, scale, block=BLOCK_TOKENS):
    """The block-by-block form of the same attention, in the order the
    "Formulació matemàtica" section of "PagedAttention" (e-fortepiano.pl)
    gives it: cut keys and values into blocks of ``block`` tokens, form one
    score vector per block (exponentials of the scaled dot products divided
    by the sum of exponentials over *all* keys), and add up each value block
    weighted by its score vector.  No maximum is subtracted, as in the
    formulation; the inputs used with it keep exp() in range."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    H, D = q.shape
    if n == 0:
        return np.zeros((H, D), dtype=np.float64)
    nblk = -(-n // block)
    key_blocks = [K[j * block:(j + 1) * block] for j in range(nblk)]
    val_blocks = [V[j * block:(j + 1) * block] for j in range(nblk)]
    exp_blocks = [np.exp(float(scale) * np.einsum("hd,nhd->hn", q, Kj))
                  for Kj in key_blocks]
    denom = sum(e.sum(axis=1) for e in exp_blocks)               # [H]
    out = np.zeros((H, D), dtype=np.float64)
    for Vj, Ej in zip(val_blocks, exp_blocks):
        a_j = Ej / denom[:, None]                                # score vector of block j
        out += np.einsum("hn,nhd->hd", a_j, Vj)
    return out


def paged_decode_ref(q, k_pool, v_pool, block_tables, context_lens, scale, seqs=None):
    """Decode for a batch: for each sequence b, gather its ``context_lens[b]``
    tokens through ``block_tables[b]`` and apply ``attention_ref``.

    q: [B][H][D] fp16; pools: [num_blocks][H][D/8][16][8] fp16 (any shape
    with that many elements); block_tables: [B][max_blocks] int; context_lens:
    [B] int.  ``seqs`` restricts the work to some sequences (rows of the
    result for the others are NaN).  Returns float64 [B][H][D]."""
    q = np.asarray(q)
    B, H, D = q.shape
    out = np.full((B, H, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        K = gather_ref(k_pool, block_tables[b], n, H, D)
        V = gather_ref(v_pool, block_tables[b], n, H, D)
        out[b] = attention_ref(q[b], K, V, scale)
    return out
