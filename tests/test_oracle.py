"""Pins for the CPU oracle: every function is checked against something other
than itself (closed forms, torch's float64 attention, brute force, and the
invariants the pages state)."""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import (BLOCK_TOKENS, append_ref, attention_ref, blockwise_attention_ref,
                    cow_ref, gather_ref, paged_decode_ref, pool_element_index)


def _rand_case(rng, B, H, D, lens, NB=None, shuffle=True):
    """Random pools plus tables handing out distinct ids."""
    nblk = [-(-int(n) // 16) for n in lens]
    NB = NB or max(sum(nblk), 1) + 3
    ids = rng.permutation(NB) if shuffle else np.arange(NB)
    width = max(max(nblk), 1)
    tables = np.full((B, width), -1, dtype=np.int32)
    p = 0
    for b, nb in enumerate(nblk):
        tables[b, :nb] = ids[p:p + nb]
        p += nb
    q = rng.standard_normal((B, H, D)).astype(np.float16)
    kp = rng.standard_normal(wl.pool_shape(NB, H, D)).astype(np.float16)
    vp = rng.standard_normal(wl.pool_shape(NB, H, D)).astype(np.float16)
    return q, kp, vp, tables, np.asarray(lens, dtype=np.int32)


def _write_contiguous(K, table, H, D, NB):
    """Place a contiguous [n][H][D] sequence into a fresh flat pool, element by
    element, at the positions the documented layout gives."""
    pool = np.zeros(NB * H * D * BLOCK_TOKENS, dtype=np.float16)
    n = K.shape[0]
    for t in range(n):
        blk = int(table[t // BLOCK_TOKENS])
        for h in range(H):
            for d in range(D):
                pool[pool_element_index(blk, h, t % BLOCK_TOKENS, d, H, D)] = K[t, h, d]
    return pool.reshape(wl.pool_shape(NB, H, D))


# ---------------------------------------------------------------- closed forms

def test_single_token_returns_its_value():
    """ctx = 1: the only weight is 1, so the output is that token's value."""
    rng = np.random.default_rng(1)
    q, kp, vp, tables, lens = _rand_case(rng, 3, 4, 64, [1, 1, 1])
    out = paged_decode_ref(q, kp, vp, tables, lens, 0.125)
    for b in range(3):
        v0 = gather_ref(vp, tables[b], 1, 4, 64)[0]
        assert np.array_equal(out[b], v0)


def test_zero_query_is_mean_of_values():
    """q = 0 gives equal scores, so the output is the plain mean of V."""
    rng = np.random.default_rng(2)
    q, kp, vp, tables, lens = _rand_case(rng, 2, 2, 64, [37, 16])
    q[:] = 0
    out = paged_decode_ref(q, kp, vp, tables, lens, 0.125)
    for b in range(2):
        V = gather_ref(vp, tables[b], int(lens[b]), 2, 64)
        np.testing.assert_allclose(out[b], V.mean(axis=0), rtol=0, atol=1e-14)


def test_two_token_closed_form():
    """Two keys with known scores a, b: out = (e^a v0 + e^b v1) / (e^a + e^b)."""
    H, D = 1, 64
    q = np.zeros((H, D)); q[0, 3] = 2.0
    K = np.zeros((2, H, D)); K[0, 0, 3] = 1.5; K[1, 0, 3] = -0.5
    V = np.zeros((2, H, D)); V[0, 0, :] = 1.0; V[1, 0, :] = -3.0
    scale = 0.25
    a, b = scale * 2.0 * 1.5, scale * 2.0 * -0.5
    expect = (math.exp(a) * 1.0 + math.exp(b) * -3.0) / (math.exp(a) + math.exp(b))
    out = attention_ref(q, K, V, scale)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-14)
    # the larger score must carry the larger weight (a sign slip flips this)
    assert out[0, 0] > -1.0


def test_empty_context_is_zero():
    rng = np.random.default_rng(3)
    q, kp, vp, tables, lens = _rand_case(rng, 2, 2, 64, [0, 5])
    out = paged_decode_ref(q, kp, vp, tables, lens, 0.125)
    assert np.array_equal(out[0], np.zeros((2, 64)))


# ------------------------------------------------------------ library routine

@pytest.mark.parametrize("D,lens", [(64, [1, 15, 16, 37]), (128, [300, 17, 2048])])
def test_matches_torch_sdpa_float64(D, lens):
    """Gathered K/V through torch's float64 scaled_dot_product_attention."""
    rng = np.random.default_rng(4)
    H = 4
    q, kp, vp, tables, lens = _rand_case(rng, len(lens), H, D, lens)
    scale = float(np.float32(1 / math.sqrt(D)))
    out = paged_decode_ref(q, kp, vp, tables, lens, scale)
    for b in range(len(lens)):
        n = int(lens[b])
        K = torch.from_numpy(gather_ref(kp, tables[b], n, H, D)).permute(1, 0, 2)
        V = torch.from_numpy(gather_ref(vp, tables[b], n, H, D)).permute(1, 0, 2)
        Q = torch.from_numpy(q[b].astype(np.float64)).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        np.testing.assert_allclose(out[b], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

def test_brute_force_tiny():
    """The tiny workload by pure-Python loops with math.exp and math.fsum,
    reading the pool element by element at the documented positions."""
    c = wl.tiny()
    out = paged_decode_ref(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    H, D = c.num_heads, c.head_dim
    kf = c.k_pool.reshape(-1)
    vf = c.v_pool.reshape(-1)
    for b in range(c.batch):
        n = int(c.context_lens[b])
        for h in range(H):
            scores = []
            for t in range(n):
                blk = int(c.block_tables[b][t // 16])
                scores.append(c.scale * math.fsum(
                    float(c.q[b, h, d]) * float(kf[pool_element_index(blk, h, t % 16, d, H, D)])
                    for d in range(D)))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            den = math.fsum(w)
            for d in range(D):
                num = math.fsum(
                    w[t] * float(vf[pool_element_index(int(c.block_tables[b][t // 16]), h,
                                                       t % 16, d, H, D)])
                    for t in range(n))
                assert abs(out[b, h, d] - num / den) <= 1e-12


# ----------------------------------------------------------------- invariants

def test_paged_equals_contiguous():
    """A sequence stored through a block table, in any blocks, gives the same
    output as plain attention over the contiguous sequence."""
    rng = np.random.default_rng(5)
    H, D, n, NB = 2, 64, 41, 9
    K = rng.standard_normal((n, H, D)).astype(np.float16)
    V = rng.standard_normal((n, H, D)).astype(np.float16)
    q = rng.standard_normal((1, H, D)).astype(np.float16)
    for table in (np.arange(3), rng.permutation(NB)[:3], np.array([8, 0, 5])):
        kp = _write_contiguous(K, table, H, D, NB)
        vp = _write_contiguous(V, table, H, D, NB)
        assert np.array_equal(gather_ref(kp, table, n, H, D), K.astype(np.float64))
        out = paged_decode_ref(q, kp, vp, table[None, :], np.array([n]), 0.125)
        np.testing.assert_array_equal(out[0], attention_ref(q[0], K, V, 0.125))


def test_physical_relabelling_is_bitwise_invariant():
    """Moving blocks to other physical ids and rewriting the tables to match
    leaves every output bit unchanged."""
    rng = np.random.default_rng(6)
    q, kp, vp, tables, lens = _rand_case(rng, 4, 4, 64, [1, 15, 16, 37])
    NB = kp.shape[0]
    perm = rng.permutation(NB)
    kp2 = np.empty_like(kp); kp2[perm] = kp
    vp2 = np.empty_like(vp); vp2[perm] = vp
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    a = paged_decode_ref(q, kp, vp, tables, lens, 0.125)
    b = paged_decode_ref(q, kp2, vp2, t2, lens, 0.125)
    assert np.array_equal(a, b)


def test_shared_blocks_equal_private_copies():
    """Sequences pointing at the same physical prefix give the same outputs as
    sequences holding private copies of it."""
    c = wl.shared_prefix(batch=6, seed=11, prefix_tokens=64, suffix_max=40, heads=2,
                         head_dim=64)
    shared = paged_decode_ref(c.q, c.k_pool, c.v_pool, c.shared_tables, c.context_lens,
                              c.scale)
    kp, vp = cow_ref([c.k_pool, c.v_pool], c.cow_pairs)
    private = paged_decode_ref(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
    assert np.array_equal(shared, private)


def test_blockwise_form_equals_plain():
    """The per-block score-vector form of the attention equals the plain form."""
    rng = np.random.default_rng(7)
    for n in (1, 16, 17, 300):
        q = rng.standard_normal((3, 64))
        K = rng.standard_normal((n, 3, 64))
        V = rng.standard_normal((n, 3, 64))
        np.testing.assert_allclose(blockwise_attention_ref(q, K, V, 0.125),
                                   attention_ref(q, K, V, 0.125), rtol=0, atol=1e-12)


def _partitioned(q, K, V, scale, part):
    """Split-context rearrangement: each partition keeps (max, sum, weighted
    sum) of its own scores; the partials are merged with exp(m_p - M)."""
    n = K.shape[0]
    parts = []
    for lo in range(0, n, part):
        s = scale * np.einsum("hd,nhd->hn", q, K[lo:lo + part])
        m = s.max(axis=1)
        w = np.exp(s - m[:, None])
        parts.append((m, w.sum(axis=1), np.einsum("hn,nhd->hd", w, V[lo:lo + part])))
    M = np.max([p[0] for p in parts], axis=0)
    num = sum(np.exp(m - M)[:, None] * acc for m, _, acc in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den[:, None]


@pytest.mark.parametrize("part", [16, 64, 256])
def test_partitioned_merge_equals_plain(part):
    """The split-context merge the GPU path uses is an exact rearrangement."""
    rng = np.random.default_rng(8)
    for n in (1, 255, 256, 257, 2048):
        q = rng.standard_normal((2, 128))
        K = rng.standard_normal((n, 2, 128)) * 3
        V = rng.standard_normal((n, 2, 128))
        np.testing.assert_allclose(_partitioned(q, K, V, 0.088, part),
                                   attention_ref(q, K, V, 0.088), rtol=0, atol=1e-12)


# ------------------------------------------------------------ append and copy

def test_append_then_gather_round_trips():
    """Appending a sequence token by token into the slots its table names and
    reading it back through the table returns the sequence."""
    rng = np.random.default_rng(9)
    H, D, n, NB = 3, 64, 35, 7
    K = rng.standard_normal((n, H, D)).astype(np.float16)
    V = rng.standard_normal((n, H, D)).astype(np.float16)
    table = rng.permutation(NB)[:3]
    slots = np.array([table[t // 16] * 16 + t % 16 for t in range(n)], dtype=np.int32)
    kp = np.zeros(wl.pool_shape(NB, H, D), dtype=np.float16)
    vp = np.zeros_like(kp)
    kp2, vp2 = append_ref(K, V, slots, kp, vp)
    assert np.array_equal(gather_ref(kp2, table, n, H, D), K.astype(np.float64))
    assert np.array_equal(gather_ref(vp2, table, n, H, D), V.astype(np.float64))
    # nothing outside the written slots changed
    written = np.zeros(kp.shape, dtype=bool)
    for t in range(n):
        written[table[t // 16], :, :, t % 16, :] = True
    assert not kp2[~written].any() and not vp2[~written].any()
    assert not kp.any()  # input untouched


def test_append_skips_negative_slots_and_rejects_duplicates():
    rng = np.random.default_rng(10)
    k = rng.standard_normal((3, 1, 64)).astype(np.float16)
    kp = np.zeros(wl.pool_shape(2, 1, 64), dtype=np.float16)
    k2, _ = append_ref(k, k, np.array([-1, 5, -7]), kp, kp)
    assert np.array_equal(gather_ref(k2, [0], 6, 1, 64)[5], k[1].astype(np.float64))
    assert np.count_nonzero(k2) == np.count_nonzero(k[1])
    with pytest.raises(ValueError):
        append_ref(k, k, np.array([4, 4, 1]), kp, kp)


def test_cow_copies_whole_blocks_and_rejects_conflicts():
    rng = np.random.default_rng(12)
    pools = [rng.standard_normal((6, 2, 8, 16, 8)).astype(np.float16) for _ in range(3)]
    out = cow_ref(pools, [[1, 4], [2, 5]])
    for before, after in zip(pools, out):
        assert np.array_equal(after[4], before[1]) and np.array_equal(after[5], before[2])
        keep = [0, 1, 2, 3]
        assert np.array_equal(after[keep], before[keep])
    # chained pairs read the state before any copy
    out = cow_ref(pools, [[1, 4], [0, 3]])
    assert np.array_equal(out[0][3], pools[0][0])
    with pytest.raises(ValueError):
        cow_ref(pools, [[1, 4], [4, 5]])   # a destination is also a source
    with pytest.raises(ValueError):
        cow_ref(pools, [[1, 4], [2, 4]])   # a destination repeated


# ------------------------------------------------------- grouped (shared) decode

def _forked_case(rng, H=2, D=64, prompt=45, branches=(3, 0, 17, 16), extra=5, copies=False):
    """One prompt forked into len(branches) branches that each write their own
    tokens (copy-on-write of the partial last page), plus ``extra`` tokens in
    an unrelated request; tables from the block manager.  With ``copies`` the
    branches hold private copies (same data, other page ids) of the prompt's
    full pages instead of sharing them."""
    from paged_kv_cache_03_amd.blocks import PagedRequest, PagePool
    pool = PagePool(64, seed=7)
    owner = PagedRequest(pool)
    owner.append_tokens(prompt)
    reqs = [owner.fork() for _ in branches]
    for r, n in zip(reqs, branches):
        r.append_tokens(n)
    other = PagedRequest(pool)
    other.append_tokens(extra)
    batch = [owner] + reqs + [other]
    NB = pool.num_pages
    kp = rng.standard_normal(wl.pool_shape(NB, H, D)).astype(np.float16)
    vp = rng.standard_normal(wl.pool_shape(NB, H, D)).astype(np.float16)
    if copies:
        full = prompt // BLOCK_TOKENS
        for r in reqs:
            for j in range(full):
                new = pool.alloc()
                kp[new] = kp[r.block_table[j]]
                vp[new] = vp[r.block_table[j]]
                r.block_table[j] = new
    from paged_kv_cache_03_amd.blocks import device_arrays
    tables, lens = device_arrays(batch)
    q = rng.standard_normal((len(batch), H, D)).astype(np.float16)
    return batch, q, kp, vp, tables, lens


def test_grouped_decode_is_plain_decode_on_shared_tables():
    """Sharing changes where K/V live, not what is computed ("Descripció"):
    with the block manager's grouping the grouped oracle gives exactly the
    per-sequence decode."""
    from oracle import grouped_decode_ref
    from paged_kv_cache_03_amd.blocks import decode_groups
    rng = np.random.default_rng(21)
    batch, q, kp, vp, tables, lens = _forked_case(rng)
    order, offs, shared = decode_groups(batch, max_group=3)
    assert shared.max() == 2            # 45 tokens: two full prompt pages shared
    q, tables, lens = q[order], tables[order], lens[order]
    scale = 0.125
    got = grouped_decode_ref(q, kp, vp, tables, lens, offs, shared, scale, max_group_size=3)
    assert np.array_equal(got, paged_decode_ref(q, kp, vp, tables, lens, scale))


def test_grouped_leader_rule_equals_private_copies():
    """Branches that hold private copies of the prompt pages (same data, other
    ids) give the same result when the call says the pages are shared: the
    grouped call reads them through the first member's table."""
    from oracle import grouped_decode_ref, grouped_tables_ref
    rng = np.random.default_rng(22)
    batch, q, kp, vp, tables, lens = _forked_case(rng, copies=True)
    B = len(batch)
    offs = np.array([0, B - 1, B], dtype=np.int32)      # prompt owner + branches, then the other
    shared = np.array([2, 0], dtype=np.int32)
    eff, _ = grouped_tables_ref(tables, lens, offs, shared, 16)
    assert not np.array_equal(eff, tables)               # other ids really are substituted
    scale = 0.125
    got = grouped_decode_ref(q, kp, vp, tables, lens, offs, shared, scale)
    assert np.array_equal(got, paged_decode_ref(q, kp, vp, tables, lens, scale))


def test_grouped_contract_edges():
    """Shared counts past any member's full pages are clamped; members past
    the group size limit, sequences in no group and groups of negative size
    get zero rows."""
    from oracle import grouped_decode_ref
    rng = np.random.default_rng(23)
    batch, q, kp, vp, tables, lens = _forked_case(rng)
    B = len(batch)
    scale = 0.125
    plain = paged_decode_ref(q, kp, vp, tables, lens, scale)
    # one group over the forks with a huge shared count: clamped to 2
    offs = np.array([0, 1, B - 1, B], dtype=np.int32)
    got = grouped_decode_ref(q, kp, vp, tables, lens, offs, [0, 99, 0], scale)
    assert np.array_equal(got, plain)
    # group size limit 2: the third and fourth forks are not decoded
    got = grouped_decode_ref(q, kp, vp, tables, lens, offs, [0, 2, 0], scale, max_group_size=2)
    assert np.array_equal(got[:3], plain[:3]) and np.array_equal(got[B - 1], plain[B - 1])
    assert not got[3:B - 1].any()
    # the last sequence in no group; a group of negative size
    offs = np.array([0, 3, 2, B - 1], dtype=np.int32)
    got = grouped_decode_ref(q, kp, vp, tables, lens, offs, [2, 2, 2], scale)
    assert np.array_equal(got[:3], plain[:3]) and not got[B - 1].any()


# ------------------------------------------------------------------- prefill

def _prefill_case(rng, H, D, lens, nq):
    q_, kp, vp, tables, lens = _rand_case(rng, len(lens), H, D, lens)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), H, D)).astype(np.float16)
    return q, kp, vp, tables, lens, qs


def test_prefill_matches_torch_sdpa_causal_float64():
    """Every sequence's query rows against torch's float64 attention with an
    explicit mask: row i (position ctx - n + i) sees keys 0 .. that position."""
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(31)
    H, D = 3, 64
    lens, nq = [37, 16, 70, 5], [37, 3, 20, 5]
    q, kp, vp, tables, lens, qs = _prefill_case(rng, H, D, lens, nq)
    scale = 0.125
    out = paged_prefill_ref(q, kp, vp, tables, lens, qs, scale)
    for b in range(len(lens)):
        n, ctx = nq[b], int(lens[b])
        K = torch.from_numpy(gather_ref(kp, tables[b], ctx, H, D)).permute(1, 0, 2)
        V = torch.from_numpy(gather_ref(vp, tables[b], ctx, H, D)).permute(1, 0, 2)
        Q = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).permute(1, 0, 2)
        pos = torch.arange(ctx - n, ctx)[:, None]
        mask = torch.arange(ctx)[None, :] <= pos                  # [n][ctx]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=scale)
        np.testing.assert_allclose(out[qs[b]:qs[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_prefill_brute_force_tiny():
    """Pure-Python loops over the pool at the documented element positions."""
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(32)
    H, D = 2, 16
    lens, nq = [19, 7], [4, 7]
    q, kp, vp, tables, lens, qs = _prefill_case(rng, H, D, lens, nq)
    scale = 0.25
    out = paged_prefill_ref(q, kp, vp, tables, lens, qs, scale)
    kf, vf = kp.reshape(-1), vp.reshape(-1)
    for b in range(2):
        ctx, n = int(lens[b]), nq[b]
        for i in range(n):
            p = ctx - n + i
            for h in range(H):
                at = lambda t, d: pool_element_index(int(tables[b][t // 16]), h, t % 16, d, H, D)
                s = [scale * math.fsum(float(q[qs[b] + i, h, d]) * float(kf[at(t, d)])
                                       for d in range(D)) for t in range(p + 1)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                den = math.fsum(w)
                for d in range(D):
                    num = math.fsum(w[t] * float(vf[at(t, d)]) for t in range(p + 1))
                    assert abs(out[qs[b] + i, h, d] - num / den) <= 1e-12


def test_prefill_position_zero_and_too_many_queries():
    """The query at position 0 sees only its own token: the output is that
    token's value exactly.  Rows past the context's start are zero."""
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(33)
    H, D = 2, 64
    q, kp, vp, tables, lens, qs = _prefill_case(rng, H, D, [9], [12])
    out = paged_prefill_ref(q, kp, vp, tables, lens, qs, 0.125)
    assert not out[:3].any()                                   # positions -3, -2, -1
    v0 = gather_ref(vp, tables[0], 1, H, D)[0]
    assert np.array_equal(out[3], v0.astype(np.float64))


def test_prefill_chunks_agree_with_one_pass():
    """Causal attention of a token depends on its prefix only: a prompt
    processed in one call or in two chunks (the second over a longer cached
    context) gives the same rows bit for bit; and the last row of each chunk
    is the decode of the sequence at that length."""
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(34)
    H, D = 2, 64
    q, kp, vp, tables, lens, qs = _prefill_case(rng, H, D, [53], [53])
    whole = paged_prefill_ref(q, kp, vp, tables, lens, qs, 0.125)
    first = paged_prefill_ref(q[:20], kp, vp, tables, np.array([20]), [0, 20], 0.125)
    second = paged_prefill_ref(q[20:], kp, vp, tables, lens, [0, 33], 0.125)
    assert np.array_equal(whole, np.concatenate([first, second]))
    dec = paged_decode_ref(q[19:20], kp, vp, tables, np.array([20]), 0.125)
    assert np.array_equal(first[19], dec[0])


# ------------------------------------------------------------ contiguous cache

def test_contiguous_decode_equals_paged_decode():
    """The same tokens in a contiguous row array and scattered over a block
    pool through tables give the same decode ("Atenció": the standard
    attention is kept), bit for bit in float64; rows past a context are
    never read (NaN there changes nothing)."""
    from oracle import contiguous_decode_ref
    rng = np.random.default_rng(35)
    H, D, L = 3, 64, 96
    lens = np.array([1, 17, 96, 40, 0], dtype=np.int32)
    B = len(lens)
    k_rows = np.full((B * L, H, D), np.nan, dtype=np.float16)
    v_rows = np.full((B * L, H, D), np.nan, dtype=np.float16)
    for b, n in enumerate(lens):
        k_rows[b * L:b * L + n] = rng.standard_normal((n, H, D))
        v_rows[b * L:b * L + n] = rng.standard_normal((n, H, D))
    q = rng.standard_normal((B, H, D)).astype(np.float16)
    out = contiguous_decode_ref(q, k_rows, v_rows, L, lens, 0.125)
    assert np.isfinite(out).all()
    # scatter into a pool through shuffled tables, element by element
    nblk = [-(-int(n) // 16) for n in lens]
    NB = sum(nblk) + 2
    ids = rng.permutation(NB)
    tables = np.full((B, max(nblk)), -1, dtype=np.int32)
    kp = np.zeros(NB * H * D * 16, dtype=np.float16)
    vp = np.zeros_like(kp)
    p = 0
    for b, n in enumerate(lens):
        tables[b, :nblk[b]] = ids[p:p + nblk[b]]
        p += nblk[b]
        for t in range(int(n)):
            for h in range(H):
                for d in range(D):
                    i = pool_element_index(int(tables[b, t // 16]), h, t % 16, d, H, D)
                    kp[i] = k_rows[b * L + t, h, d]
                    vp[i] = v_rows[b * L + t, h, d]
    shape = wl.pool_shape(NB, H, D)
    assert np.array_equal(out, paged_decode_ref(q, kp.reshape(shape), vp.reshape(shape), tables,
                                                lens, 0.125))
