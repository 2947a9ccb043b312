"""Seeded synthetic inputs for paged decode, shared by the tests and the bench.

This module draws random numbers and hands out physical block ids; it holds
none of the attention arithmetic and imports neither the oracle nor the
product package.  Its workloads are shaped like the pages' own: a GPT-style
model of 32 layers x 32 heads x 128 dims in fp16 ("Atención paginada en
modelos de lenguaje grandes (LLM)", 7minutos.es, bytes-per-token part), pages
of 16 tokens, a maximum sequence of 2048 tokens, responses averaging about
500 tokens, 10 to 200 concurrent requests, and a shared system prompt (same
page, prefix-sharing part).

Pools are ``[num_blocks][H][D/8][16][8]`` fp16 arrays filled with N(0,1)
(float32 draws rounded to fp16).  Block tables are int32
``[B][max_blocks]`` with -1 past each sequence's blocks.  A slot is
``physical_block * 16 + position``.

Draw order for every case: lengths, then the free-list permutation, then q,
then the pools, then any new tokens.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 16
MAX_SEQ = 2048
GROUP = 8
_CHUNK = 1 << 24  # elements per draw when filling large pools


@dataclass
class Case:
    name: str
    num_heads: int
    head_dim: int
    num_blocks: int
    context_lens: np.ndarray            # int32 [B] tokens attended, after any append
    block_tables: np.ndarray            # int32 [B][max_blocks]
    q: np.ndarray                       # fp16 [B][H][D]
    scale: float                        # float32 value
    k_pool: Optional[np.ndarray] = None  # fp16 [NB][H][D/8][16][8]
    v_pool: Optional[np.ndarray] = None
    k_new: Optional[np.ndarray] = None   # fp16 [T][H][D]
    v_new: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # int32 [T]
    cow_pairs: Optional[np.ndarray] = None     # int32 [n][2] (src, dst)
    shared_tables: Optional[np.ndarray] = None  # tables before copy-on-write
    query_start: Optional[np.ndarray] = None    # int32 [B+1], prefill: rows of q per sequence
    num_layers: int = 1
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def max_context(self):
        return int(self.context_lens.max()) if self.context_lens.size else 0

    def kv_tokens(self):
        return int(self.context_lens.astype(np.int64).sum())


def _scale(head_dim):
    return float(np.float32(1.0 / np.sqrt(np.float64(head_dim))))


def normal_fp16(rng, shape):
    """N(0,1) float32 draws rounded to fp16, drawn in fixed-size chunks."""
    out = np.empty(int(np.prod(shape)), dtype=np.float16)
    for lo in range(0, out.size, _CHUNK):
        hi = min(out.size, lo + _CHUNK)
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    return out.reshape(shape)


def pool_shape(num_blocks, num_heads, head_dim):
    return (num_blocks, num_heads, head_dim // GROUP, BLOCK, GROUP)


def _tables(lens_blocks, free, width):
    """Hand out ids from the front of ``free`` in sequence order."""
    tables = np.full((len(lens_blocks), width), -1, dtype=np.int32)
    ptr = 0
    for b, nb in enumerate(lens_blocks):
        tables[b, :nb] = free[ptr:ptr + nb]
        ptr += nb
    return tables, ptr


def _blocks(n):
    return -(-int(n) // BLOCK)


def _slot(table_row, pos):
    return int(table_row[pos // BLOCK]) * BLOCK + pos % BLOCK


def tiny(seed=0):
    """4 sequences of 1, 15, 16 and 37 tokens; 4 heads x 64; a 16-block pool;
    the tables take the blocks of a random permutation in order."""
    rng = np.random.default_rng(seed)
    H, D, NB = 4, 64, 16
    lens = np.array([1, 15, 16, 37], dtype=np.int32)
    free = rng.permutation(NB).astype(np.int32)
    nblk = [_blocks(n) for n in lens]
    tables, _ = _tables(nblk, free, max(nblk))
    q = normal_fp16(rng, (len(lens), H, D))
    k_pool = normal_fp16(rng, pool_shape(NB, H, D))
    v_pool = normal_fp16(rng, pool_shape(NB, H, D))
    case = Case("tiny", H, D, NB, lens, tables, q, _scale(D), k_pool, v_pool)
    case.meta["seed"] = seed
    return case


def draw_lengths(rng, batch):
    """Prompt U[32, 256] plus response geometric(mean 500), capped at 2048."""
    prompt = rng.integers(32, 256, size=batch, endpoint=True)
    response = rng.geometric(1.0 / 500.0, size=batch)
    return np.minimum(prompt + response, MAX_SEQ).astype(np.int32)


def gpt_batch(batch, seed, num_blocks=None, append=False, heads=32, head_dim=128,
              fill=True):
    """One layer of a GPT-style batch.

    Without ``append``: ``num_blocks`` (default 4096) blocks, tables from a
    shuffled free list.  With ``append``: each sequence of final length L
    holds L-1 cached tokens and appends one new token (a new block when
    (L-1) % 16 == 0); the pool is the blocks needed after the append plus 10%
    free, rounded up."""
    rng = np.random.default_rng(seed)
    lens = draw_lengths(rng, batch)
    nblk = [_blocks(n) for n in lens]
    need = int(sum(nblk))
    if num_blocks is None:
        num_blocks = -(-need * 11 // 10) if append else 4096
    if need > num_blocks:
        raise ValueError("pool too small for the drawn lengths")
    free = rng.permutation(num_blocks).astype(np.int32)
    tables, _ = _tables(nblk, free, max(nblk))
    q = normal_fp16(rng, (batch, heads, head_dim))
    case = Case(f"gpt_b{batch}" + ("_append" if append else ""), heads, head_dim,
                num_blocks, lens, tables, q, _scale(head_dim))
    case.meta["seed"] = seed
    if fill:
        case.k_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
        case.v_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
    if append:
        if not fill:  # keep the draw order fixed whether or not pools are drawn
            rng = np.random.default_rng([seed, 1])
        case.k_new = normal_fp16(rng, (batch, heads, head_dim))
        case.v_new = normal_fp16(rng, (batch, heads, head_dim))
        case.slot_mapping = np.array(
            [_slot(tables[b], int(lens[b]) - 1) for b in range(batch)], dtype=np.int32)
    return case


def shared_prefix(batch=100, seed=3, prefix_tokens=1024, suffix_max=500, heads=32,
                  head_dim=128, fill=True):
    """A system prompt of ``prefix_tokens`` stored once and shared by every
    table, then a private suffix of U[0, suffix_max] tokens per sequence.

    The prefix's last block is copied per sequence (copy-on-write); the copy
    pairs are ``cow_pairs`` and ``shared_tables`` are the tables before the
    copy.  With a prefix that ends inside a block the suffix starts in that
    private copy, so the suffix tokens are supplied as ``k_new``/``v_new``
    with their ``slot_mapping``; with a whole-block prefix the suffix blocks
    are drawn into the pool like everything else."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(0, suffix_max, size=batch, endpoint=True).astype(np.int32)
    lens = (prefix_tokens + suffix).astype(np.int32)
    pblocks = _blocks(prefix_tokens)
    partial = prefix_tokens % BLOCK != 0
    nblk = [_blocks(n) for n in lens]
    private = [nb - pblocks for nb in nblk]   # blocks after the prefix
    need = pblocks + batch + int(sum(private))
    num_blocks = -(-need * 11 // 10)
    free = rng.permutation(num_blocks).astype(np.int32)
    prefix_ids = free[:pblocks]
    ptr = pblocks
    width = max(nblk)
    tables = np.full((batch, width), -1, dtype=np.int32)
    shared = np.full((batch, width), -1, dtype=np.int32)
    pairs = np.empty((batch, 2), dtype=np.int32)
    for b in range(batch):
        copy_id = free[ptr]
        ptr += 1
        own = free[ptr:ptr + private[b]]
        ptr += private[b]
        shared[b, :pblocks] = prefix_ids
        shared[b, pblocks:nblk[b]] = own
        tables[b] = shared[b]
        tables[b, pblocks - 1] = copy_id
        pairs[b] = (prefix_ids[-1], copy_id)
    q = normal_fp16(rng, (batch, heads, head_dim))
    case = Case(f"shared_prefix_{prefix_tokens}", heads, head_dim, num_blocks, lens,
                tables, q, _scale(head_dim), cow_pairs=pairs, shared_tables=shared)
    case.meta.update(seed=seed, prefix_tokens=prefix_tokens, prefix_blocks=pblocks,
                     prefix_ids=prefix_ids.copy(), suffix=suffix)
    if fill:
        case.k_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
        case.v_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
    if partial:
        # the suffix is written after the copy: into the copy's free tail,
        # then into the sequence's own blocks
        if not fill:
            rng = np.random.default_rng([seed, 1])
        T = int(suffix.sum())
        case.k_new = normal_fp16(rng, (T, heads, head_dim))
        case.v_new = normal_fp16(rng, (T, heads, head_dim))
        slots = np.empty(T, dtype=np.int32)
        t = 0
        for b in range(batch):
            for pos in range(prefix_tokens, int(lens[b])):
                slots[t] = _slot(tables[b], pos)
                t += 1
        case.slot_mapping = slots
    return case


def full_step(batch=200, layers=32, context=MAX_SEQ, seed=4, heads=32, head_dim=128,
              beams=1):
    """The full decode step: ``layers`` layers, every sequence at ``context``
    tokens after appending one token per sequence per layer.

    ``beams == 1``: independent sequences, ``batch * context / 16`` blocks per
    layer.  ``beams > 1``: ``batch / beams`` groups; the beams of a group
    share every block but the last; beam 0 keeps the group's last block and
    beams 1.. get copies of it (``cow_pairs``), then each beam appends its own
    token into its own last block.  Block ids are the same in every layer.
    Pools are not drawn here (they are filled on the device); see
    ``device_pool``."""
    rng = np.random.default_rng(seed)
    nb_seq = _blocks(context)
    lens = np.full(batch, context, dtype=np.int32)
    if beams == 1:
        num_blocks = batch * nb_seq
        free = rng.permutation(num_blocks).astype(np.int32)
        tables, _ = _tables([nb_seq] * batch, free, nb_seq)
        pairs = None
        shared = None
    else:
        if batch % beams:
            raise ValueError("batch must be a multiple of beams")
        groups = batch // beams
        num_blocks = groups * (nb_seq + beams - 1)
        free = rng.permutation(num_blocks).astype(np.int32)
        tables = np.empty((batch, nb_seq), dtype=np.int32)
        shared = np.empty((batch, nb_seq), dtype=np.int32)
        pairs = np.empty((groups * (beams - 1), 2), dtype=np.int32)
        ptr = 0
        for g in range(groups):
            base = free[ptr:ptr + nb_seq]
            ptr += nb_seq
            for j in range(beams):
                b = g * beams + j
                shared[b] = base
                tables[b] = base
                if j:
                    tables[b, -1] = free[ptr]
                    pairs[g * (beams - 1) + j - 1] = (base[-1], free[ptr])
                    ptr += 1
    q = normal_fp16(rng, (layers, batch, heads, head_dim))
    k_new = normal_fp16(rng, (layers, batch, heads, head_dim))
    v_new = normal_fp16(rng, (layers, batch, heads, head_dim))
    slots = np.array([_slot(tables[b], context - 1) for b in range(batch)], dtype=np.int32)
    case = Case(f"full_step_l{layers}_b{batch}" + (f"_beam{beams}" if beams > 1 else ""),
                heads, head_dim, num_blocks, lens, tables, q, _scale(head_dim),
                k_new=k_new, v_new=v_new, slot_mapping=slots, cow_pairs=pairs,
                shared_tables=shared, num_layers=layers)
    case.meta.update(seed=seed, beams=beams)
    return case


def prefill(batch=200, seed=6, cached=0, chunk=None, heads=32, head_dim=128, fill=True):
    """Prefill of one layer: every sequence processes ``n_b`` new tokens as
    queries (a prompt: U[32, 256] tokens, or a fixed ``chunk``) after
    ``cached`` tokens already in its pages, so its context is cached + n_b.

    ``q`` is [sum n_b][H][D] with sequence b's rows at
    query_start[b] .. query_start[b+1]-1; ``k_new``/``v_new`` hold the new
    tokens' keys and values with their ``slot_mapping`` (appended before the
    attention); the pools (blocks needed plus 10%, shuffled) hold the cached
    tokens."""
    rng = np.random.default_rng(seed)
    if chunk is None:
        n = rng.integers(32, 256, size=batch, endpoint=True).astype(np.int32)
    else:
        n = np.full(batch, chunk, dtype=np.int32)
    lens = (cached + n).astype(np.int32)
    nblk = [_blocks(x) for x in lens]
    need = int(sum(nblk))
    num_blocks = -(-need * 11 // 10)
    free = rng.permutation(num_blocks).astype(np.int32)
    tables, _ = _tables(nblk, free, max(nblk))
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(qs[-1])
    q = normal_fp16(rng, (T, heads, head_dim))
    name = f"prefill_b{batch}" + (f"_c{cached}+{chunk}" if chunk is not None else "_prompt")
    case = Case(name, heads, head_dim, num_blocks, lens, tables, q, _scale(head_dim),
                query_start=qs)
    case.meta.update(seed=seed, cached=cached, chunk=chunk)
    if fill:
        case.k_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
        case.v_pool = normal_fp16(rng, pool_shape(num_blocks, heads, head_dim))
    else:
        rng = np.random.default_rng([seed, 1])
    case.k_new = normal_fp16(rng, (T, heads, head_dim))
    case.v_new = normal_fp16(rng, (T, heads, head_dim))
    case.slot_mapping = np.array([_slot(tables[b], p) for b in range(batch)
                                  for p in range(cached, int(lens[b]))], dtype=np.int32)
    return case


def table_groups(tables, lens, max_group=16):
    """Grouping arguments for a batch whose tables are given as arrays:
    consecutive sequences whose first block is the same physical block form
    a group (cut at ``max_group`` members); a group's shared count is the
    number of leading blocks all its members map alike, limited to blocks
    full for every member.  Returns (group_offsets [G+1], shared_blocks [G])
    as int32 arrays."""
    tables = np.asarray(tables)
    lens = np.asarray(lens)
    B = len(lens)
    offs, shared = [0], []
    b = 0
    while b < B:
        e = b + 1
        while (e < B and e - b < max_group and lens[b] > 0 and lens[e] > 0
               and tables[e, 0] == tables[b, 0]):
            e += 1
        s = int(min(lens[b:e]) // BLOCK)
        for r in range(b + 1, e):
            k = 0
            while k < s and tables[r, k] == tables[b, k]:
                k += 1
            s = k
        offs.append(e)
        shared.append(s)
        b = e
    return np.array(offs, dtype=np.int32), np.array(shared, dtype=np.int32)


def device_pool(torch, case, layer, which, device):
    """Fill one layer's K (which=0) or V (which=1) pool on ``device`` with
    N(0,1) fp16 from a generator seeded by (seed, layer, which)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * (case.meta.get("seed", 0) + 1) + 2 * layer + which)
    shape = pool_shape(case.num_blocks, case.num_heads, case.head_dim)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float16)


def poison_unused(case, value=np.nan):
    """Write ``value`` into every pool slot no query may read: the positions
    past each sequence's context in its last block, and every block no table
    names.  Tables after any copy-on-write are the ones used."""
    valid = np.zeros(case.num_blocks, dtype=np.int64)   # readable positions per block
    table_sets = [case.block_tables]
    if case.shared_tables is not None:
        table_sets.append(case.shared_tables)
    for tables in table_sets:
        for b in range(case.batch):
            n = int(case.context_lens[b])
            nb = _blocks(n)
            ids = tables[b, :nb]
            valid[ids[:-1]] = BLOCK
            if nb:
                tail = n - (nb - 1) * BLOCK
                valid[ids[-1]] = max(valid[ids[-1]], tail)
    for pool in (case.k_pool, case.v_pool):
        for blk in np.nonzero(valid < BLOCK)[0]:
            pool[blk, :, :, valid[blk]:, :] = value
    return case
