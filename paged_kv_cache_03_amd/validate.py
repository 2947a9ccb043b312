"""Host-side checks of the caller contracts that the kernels do not verify.

The kernels trust their index arguments: duplicate slots, copy pairs that
overlap, or a block written by one sequence while another reads it leave
the pools dependent on the order in which the GPU happens to run the
writes.  These checks find such inputs on the host.  They copy the index
tensors to host memory (a synchronising read), so the wrappers in ``ops``
run them only in debug mode: ``set_debug(True)``, or the environment
variable ``PAGEDKV_DEBUG=1`` when the package is imported.

Contracts, by source:

* copy-on-write ("Atención paginada en modelos de lenguaje grandes (LLM)",
  7minutos.es, prefix-sharing part; "PagedAttention", e-fortepiano.pl,
  "Descripció"): a shared page is copied whole into a fresh page and the
  other holders keep the original unchanged, so a copy's destination is
  never a source of the same batch of copies and no destination is written
  twice;
* append (same tutorial, PagePool / PagedRequest part): each token has one
  slot, so no slot is written twice;
* fused appends: a block that receives new tokens in a call is not read by
  another sequence of the same call.

Every function raises ``ContractError`` (a ``ValueError``) naming the first
offending entry, and returns None when the input is valid.
"""

import os

import numpy as np

BLOCK_TOKENS = 16

_debug = os.environ.get("PAGEDKV_DEBUG", "") not in ("", "0")


class ContractError(ValueError):
    pass


def set_debug(flag):
    """Turn the host checks in ``ops`` on or off; returns the old setting."""
    global _debug
    old = _debug
    _debug = bool(flag)
    return old


def debug_enabled():
    return _debug


def _host(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def check_cow_pairs(pairs, num_blocks=None):
    """(src, dst) rows: no destination twice, no destination that is also a
    source, and (with ``num_blocks``) every id inside the pool."""
    p = _host(pairs).reshape(-1, 2).astype(np.int64)
    if num_blocks is not None:
        bad = np.nonzero((p < 0).any(axis=1) | (p >= num_blocks).any(axis=1))[0]
        if bad.size:
            i = int(bad[0])
            raise ContractError(f"copy pair {i} ({p[i, 0]}, {p[i, 1]}) lies outside the pool of "
                                f"{num_blocks} blocks")
    dst = p[:, 1]
    uniq, first, counts = np.unique(dst, return_index=True, return_counts=True)
    if (counts > 1).any():
        d = int(uniq[counts > 1][0])
        raise ContractError(f"block {d} is the destination of more than one copy pair")
    both = np.intersect1d(p[:, 0], dst)
    if both.size:
        raise ContractError(f"block {int(both[0])} is both a source and a destination")


def check_slots(slot_mapping, num_blocks=None):
    """Slots (``block * 16 + position``; negative = skip): none written twice,
    and (with ``num_blocks``) none past the pool."""
    s = _host(slot_mapping).reshape(-1).astype(np.int64)
    live = s[s >= 0]
    if num_blocks is not None and live.size and int(live.max()) >= num_blocks * BLOCK_TOKENS:
        t = int(np.nonzero(s >= num_blocks * BLOCK_TOKENS)[0][0])
        raise ContractError(f"slot {int(s[t])} of row {t} lies past the pool of {num_blocks} "
                            "blocks")
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        raise ContractError(f"slot {int(uniq[counts > 1][0])} is written twice")


def _used_blocks(tables, lens):
    """(sequence, block id) of every table entry a sequence reads."""
    out = []
    for b, n in enumerate(lens):
        nb = -(-max(int(n), 0) // BLOCK_TOKENS)
        out.extend((b, int(x)) for x in tables[b, :nb])
    return out


def _written_not_read_by_others(written, tables, lens, what):
    readers = {}
    for b, blk in _used_blocks(tables, lens):
        readers.setdefault(blk, set()).add(b)
    for b, blk in written:
        others = readers.get(blk, set()) - {b}
        if others:
            raise ContractError(f"block {blk} receives {what} of sequence {b} but is also read "
                                f"by sequence {min(others)} in the same call")


def check_decode_append(block_tables, context_lens):
    """Fused decode append: the last block of each non-empty sequence (where
    its new token goes) belongs to that sequence alone."""
    tables = _host(block_tables)
    lens = _host(context_lens).reshape(-1)
    written = [(b, int(tables[b, (int(n) - 1) // BLOCK_TOKENS])) for b, n in enumerate(lens)
               if int(n) > 0]
    _written_not_read_by_others(written, tables, lens, "the new token")


def check_prefill_append(block_tables, context_lens, query_start):
    """Fused prefill append: no block that receives new tokens of one
    sequence appears in another sequence's table (the part it reads)."""
    tables = _host(block_tables)
    lens = _host(context_lens).reshape(-1)
    qs = _host(query_start).reshape(-1)
    written = []
    for b, n in enumerate(lens):
        n = int(n)
        rows = int(qs[b + 1]) - int(qs[b])
        first = max(n - rows, 0)
        if first >= n:
            continue
        for j in range(first // BLOCK_TOKENS, -(-n // BLOCK_TOKENS)):
            written.append((b, int(tables[b, j])))
    _written_not_read_by_others(written, tables, lens, "new tokens")
