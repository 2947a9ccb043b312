"""Float-free references for the two paging helpers: slot-mapped append and
block copy-on-write.  Both are exact fp16 bit copies.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:

* "Atención paginada en modelos de lenguaje grandes (LLM)" (7minutos.es),
  PagePool / PagedRequest part: each generated token lands in the page its
  block table names; a new page is claimed when the token count crosses a
  page boundary.
* same page, prefix-sharing part, and "PagedAttention" (e-fortepiano.pl),
  "Descripció": a shared page that must change is first copied whole into a
  newly allocated page (copy-on-write at block granularity); the other
  sharers keep pointing at the original, which is left unchanged.

Readings where the pages are silent: a slot is ``physical_block * 16 + position``;
a negative slot means "skip this row"; slots and copy pairs are free of
conflicts (no slot twice, no destination that is also a source or a repeated
destination), so the order in which the copies happen does not matter.
"""

import numpy as np

from .paged_attention import BLOCK_TOKENS, _GROUP


def append_ref(k_new, v_new, slot_mapping, k_pool, v_pool):
    """Return copies of (k_pool, v_pool) with row t of ``k_new``/``v_new``
    ([T][H][D] fp16) written at ``slot_mapping[t]``.

    Pools are ``[num_blocks][H][D/8][16][8]`` fp16; the write for slot s puts
    dim d of head h at block s//16, position s%16, group d//8, lane d%8."""
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    T, H, D = k_new.shape
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    kt = k_out.reshape(-1, H, D // _GROUP, BLOCK_TOKENS, _GROUP)
    vt = v_out.reshape(-1, H, D // _GROUP, BLOCK_TOKENS, _GROUP)
    seen = set()
    for t in range(T):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        blk, pos = divmod(s, BLOCK_TOKENS)
        if blk >= kt.shape[0]:
            raise IndexError(f"slot {s} outside the pool")
        kt[blk, :, :, pos, :] = k_new[t].reshape(H, D // _GROUP, _GROUP)
        vt[blk, :, :, pos, :] = v_new[t].reshape(H, D // _GROUP, _GROUP)
    return k_out, v_out


def cow_ref(pools, pairs):
    """Return copies of every pool in ``pools`` (a list of per-layer pools,
    each ``[num_blocks][...]``) where, for each (src, dst) in ``pairs``, the
    whole physical block dst is replaced by block src as it was before any
    copy."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    srcs = set(int(s) for s in pairs[:, 0])
    dsts = [int(d) for d in pairs[:, 1]]
    if len(set(dsts)) != len(dsts) or srcs.intersection(dsts):
        raise ValueError("conflicting copy pairs")
    out = []
    for pool in pools:
        before = np.asarray(pool)
        after = np.array(before, copy=True)
        for s, d in pairs:
            after[d] = before[s]
        out.append(after)
    return out
