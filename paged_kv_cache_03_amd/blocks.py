"""Host-side block manager: the bookkeeping that produces the block tables,
slot mappings and copy-on-write pairs the kernels consume.

Sources:

* "Atención paginada en modelos de lenguaje grandes (LLM)" (7minutos.es),
  PagePool / PagedRequest part: a flat pool of equal pages of 16 tokens with
  a free list and a reference count per page; a page whose count drops to
  zero goes straight back to the free list; a request keeps a block table
  from logical page index to physical page id and claims a new page each
  time its token count crosses a page boundary.
* same page, prefix-sharing part: ``share`` raises a page's count without
  allocating; ``cow_copy`` allocates a new page and lowers the original's
  count; a request that must write into a shared page first gets a private
  copy of it, the other sharers are unaffected.
* "PagedAttention" (e-fortepiano.pl), "Descripció": logical blocks map to
  physical blocks through the table and need not be contiguous; physical
  blocks are reference counted and shared between requests or decoding
  branches, with block-granular copy-on-write.

Readings where the pages are silent: the owner of a shared prefix holds one
reference; a copy happens only when a shared page is about to be written
(a page held once is written in place); pool exhaustion raises
``PoolExhausted`` (no eviction); the free list hands pages out in ascending
order unless a seed shuffles it.
"""

from collections import deque

import numpy as np

PAGE_TOKENS = 16


class PoolExhausted(RuntimeError):
    pass


def kv_bytes_per_token(layers, heads, head_dim, dtype_bytes=2):
    """K and V for one token across all layers (the factor 2 is K and V;
    queries are not cached)."""
    return 2 * layers * heads * head_dim * dtype_bytes


class PagePool:
    """Physical pages, a free list and a reference count per page."""

    def __init__(self, num_pages, page_tokens=PAGE_TOKENS, seed=None):
        if num_pages <= 0:
            raise ValueError("num_pages must be positive")
        self.num_pages = int(num_pages)
        self.page_tokens = int(page_tokens)
        order = np.arange(self.num_pages)
        if seed is not None:
            order = np.random.default_rng(seed).permutation(self.num_pages)
        self._free = deque(int(i) for i in order)
        self.refcount = [0] * self.num_pages
        self._copies = []          # (src, dst) pairs not yet handed to the device

    # -- allocation -------------------------------------------------------
    def alloc(self):
        if not self._free:
            raise PoolExhausted(f"all {self.num_pages} pages are in use")
        page = self._free.popleft()
        assert self.refcount[page] == 0
        self.refcount[page] = 1
        return page

    def share(self, page):
        """One more holder of ``page``; nothing is allocated."""
        if self.refcount[page] <= 0:
            raise ValueError(f"page {page} is not allocated")
        self.refcount[page] += 1

    def release(self, page):
        """One holder fewer; at zero the page is free again at once."""
        if self.refcount[page] <= 0:
            raise ValueError(f"page {page} released more often than held")
        self.refcount[page] -= 1
        if self.refcount[page] == 0:
            self._free.append(page)

    def cow_copy(self, page):
        """Private copy of a shared page for one holder: a new page whose
        contents must become those of ``page`` (recorded as a (src, dst) pair
        for ``cow_copy_blocks``), and one reference fewer on the original."""
        if self.refcount[page] <= 1:
            raise ValueError(f"page {page} is not shared")
        new = self.alloc()
        self.refcount[page] -= 1
        self._copies.append((page, new))
        return new

    def take_copy_pairs(self):
        """The pending (src, dst) pairs as an int32 [n][2] array; clears them.
        A page copied and then released before the copy ran still appears:
        the device copy is harmless."""
        pairs = np.array(self._copies, dtype=np.int32).reshape(-1, 2)
        self._copies = []
        return pairs

    # -- accounting -------------------------------------------------------
    @property
    def num_free(self):
        return len(self._free)

    @property
    def num_used(self):
        return self.num_pages - len(self._free)

    def used_fraction(self):
        return self.num_used / self.num_pages

    def check(self):
        """Invariants: every page is either free (count 0, listed once) or
        in use (count > 0, not listed)."""
        free = list(self._free)
        assert len(free) == len(set(free)), "page listed twice on the free list"
        fs = set(free)
        for p in range(self.num_pages):
            if p in fs:
                assert self.refcount[p] == 0, f"free page {p} has references"
            else:
                assert self.refcount[p] > 0, f"page {p} is neither free nor held"


class PagedRequest:
    """One sequence: its block table and token count."""

    def __init__(self, pool, name=None):
        self.pool = pool
        self.name = name
        self.block_table = []
        self.num_tokens = 0

    @classmethod
    def sharing(cls, pool, owner, name=None):
        """A request that starts with ``owner``'s tokens (a shared system
        prompt, or a fork for parallel sampling / beam search): every page of
        the owner is shared, nothing is allocated."""
        req = cls(pool, name)
        for page in owner.block_table:
            pool.share(page)
        req.block_table = list(owner.block_table)
        req.num_tokens = owner.num_tokens
        return req

    def fork(self, name=None):
        return PagedRequest.sharing(self.pool, self, name)

    def append_token(self):
        """Make room for the next token and return its slot
        (physical page * 16 + position).  A page boundary claims a new page;
        writing into a page that other requests share first gives this request
        a private copy of it."""
        pos = self.num_tokens % self.pool.page_tokens
        if pos == 0:
            self.block_table.append(self.pool.alloc())
        else:
            last = self.block_table[-1]
            if self.pool.refcount[last] > 1:
                self.block_table[-1] = self.pool.cow_copy(last)
        self.num_tokens += 1
        return self.block_table[-1] * self.pool.page_tokens + pos

    generate_token = append_token

    def append_tokens(self, n):
        return [self.append_token() for _ in range(n)]

    def free(self):
        for page in self.block_table:
            self.pool.release(page)
        self.block_table = []
        self.num_tokens = 0

    @property
    def num_pages(self):
        return len(self.block_table)

    def last_page_waste(self):
        """Unfilled slots of the last page."""
        return self.num_pages * self.pool.page_tokens - self.num_tokens


def tables_share_blocks(requests):
    """Whether any physical page appears more than once across the batch's
    block tables (a shared prompt, forked branches): then the decode should
    keep K/V in the caches rather than stream it."""
    seen = set()
    for r in requests:
        for page in r.block_table:
            if page in seen:
                return True
            seen.add(page)
    return False


def decode_groups(requests, max_group=16):
    """Arrange a batch for the grouped decode: requests whose tables start
    with the same physical page (forks of one prompt, beams of one request)
    are put next to each other, in first-seen order, and cut into groups of
    at most ``max_group``.

    Returns (order, group_offsets, shared_blocks): ``order`` lists request
    indices in their new batch order; group g is order[group_offsets[g] :
    group_offsets[g+1]]; ``shared_blocks[g]`` is the number of leading pages
    every member of g maps to the same physical pages, counting only pages
    that are full for every member (a page still being written belongs to
    one holder after its copy-on-write)."""
    if max_group <= 0:
        raise ValueError("max_group must be positive")
    buckets, keys = {}, []
    for i, r in enumerate(requests):
        key = r.block_table[0] if r.block_table else ("private", i)
        if key not in buckets:
            buckets[key] = []
            keys.append(key)
        buckets[key].append(i)
    order, offsets, shared = [], [0], []
    for key in keys:
        members = buckets[key]
        for c in range(0, len(members), max_group):
            chunk = [requests[i] for i in members[c:c + max_group]]
            s = min(r.num_tokens // r.pool.page_tokens for r in chunk)
            first = chunk[0].block_table
            for r in chunk[1:]:
                k = 0
                while k < s and r.block_table[k] == first[k]:
                    k += 1
                s = k
            order.extend(members[c:c + max_group])
            offsets.append(len(order))
            shared.append(s)
    return (np.array(order, dtype=np.int64), np.array(offsets, dtype=np.int32),
            np.array(shared, dtype=np.int32))


def device_arrays(requests, width=None):
    """Block tables ([B][width] int32, -1 padded) and context lengths ([B]
    int32) for a batch of requests."""
    width = width or max((r.num_pages for r in requests), default=1) or 1
    tables = np.full((len(requests), width), -1, dtype=np.int32)
    lens = np.zeros(len(requests), dtype=np.int32)
    for i, r in enumerate(requests):
        if r.num_pages > width:
            raise ValueError("table wider than width")
        tables[i, :r.num_pages] = r.block_table
        lens[i] = r.num_tokens
    return tables, lens
