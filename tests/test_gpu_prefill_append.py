"""The prefill with its append fused in (``pa_prefill_append``) on the GPU,
through the C ABI: pools equal the oracle's append bit for bit, outputs
match the float64 oracle within max-abs 2e-3 and relative L2 1e-3, and both
equal ``kv_append`` followed by ``pa_prefill`` bit for bit.

The cases cover new tokens that start on a block boundary (prompts, aligned
chunks: every block with a new token is read from the caller's rows), that
start inside a block (the block shared with cached tokens is written first
by the small boundary kernel), more new rows than positions (rows at a
negative position write nothing), empty sequences, and sequences long
enough that several 128-row query groups own blocks."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import append_ref, paged_prefill_ref
from paged_kv_cache_03_amd import kv_append, pa_prefill, pa_prefill_append
from tests._gpu import assert_close, device_pools, to_dev, to_host

pytestmark = pytest.mark.gpu


def natural_slots(tables, lens, qs):
    """Slot of every new row: row i of sequence b is position
    lens[b] - n_b + i, through the table; rows at a negative position -1."""
    slots = []
    for b in range(len(lens)):
        n = int(qs[b + 1] - qs[b])
        for i in range(n):
            p = int(lens[b]) - n + i
            slots.append(int(tables[b][p // 16]) * 16 + p % 16 if p >= 0 else -1)
    return np.array(slots, dtype=np.int32)


def _case(seed, H, D, lens, nq):
    rng = np.random.default_rng(seed)
    nblk = [-(-n // 16) for n in lens]
    NB = sum(nblk) + 5
    ids = rng.permutation(NB).astype(np.int32)
    tables = np.full((len(lens), max(max(nblk), 1)), -1, dtype=np.int32)
    p = 0
    for b, nb in enumerate(nblk):
        tables[b, :nb] = ids[p:p + nb]
        p += nb
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(qs[-1])
    q = wl.normal_fp16(rng, (T, H, D))
    k_new = wl.normal_fp16(rng, (T, H, D))
    v_new = wl.normal_fp16(rng, (T, H, D))
    kp = wl.normal_fp16(rng, wl.pool_shape(NB, H, D))
    vp = wl.normal_fp16(rng, wl.pool_shape(NB, H, D))
    for row, n in zip(tables, lens):           # slots past the context hold NaN
        if n % 16:
            kp[row[n // 16], :, :, n % 16:, :] = np.nan
            vp[row[n // 16], :, :, n % 16:, :] = np.nan
    return q, k_new, v_new, kp, vp, tables, np.array(lens, dtype=np.int32), qs


def _both(q, k_new, v_new, kp, vp, tables, lens, qs, scale, max_ctx):
    """The fused call and the two separate calls on copies of the same pools."""
    print(f"prefill_append: rows={len(q)} B={len(lens)} max_ctx={max_ctx}", flush=True)
    kf, vf = to_dev(kp), to_dev(vp)
    ks, vs = kf.clone(), vf.clone()
    args = (to_dev(tables), to_dev(lens), to_dev(qs), scale)
    out_f = pa_prefill_append(to_dev(q), to_dev(k_new), to_dev(v_new), kf, vf, *args,
                              max_context_len=max_ctx)
    slots = natural_slots(tables, lens, qs)
    kv_append(to_dev(k_new), to_dev(v_new), to_dev(slots), ks, vs)
    out_s = pa_prefill(to_dev(q), ks, vs, *args, max_context_len=max_ctx)
    torch.cuda.synchronize()
    return out_f, kf, vf, out_s, ks, vs, slots


def _check(q, k_new, v_new, kp, vp, tables, lens, qs, scale, what, seqs=None):
    out_f, kf, vf, out_s, ks, vs, slots = _both(q, k_new, v_new, kp, vp, tables, lens, qs,
                                                scale, int(lens.max()))
    k_ref, v_ref = append_ref(k_new, v_new, slots, kp, vp)
    for got, ref, name in ((kf, k_ref, "k_pool"), (vf, v_ref, "v_pool")):
        assert np.array_equal(to_host(got).view(np.uint16), ref.view(np.uint16)), f"{what}: {name}"
    assert torch.equal(kf.view(torch.int16), ks.view(torch.int16))
    assert torch.equal(vf.view(torch.int16), vs.view(torch.int16))
    assert torch.equal(out_f, out_s), f"{what}: fused and separate outputs differ"
    ref = paged_prefill_ref(q, k_ref, v_ref, tables, lens, qs, scale, seqs=seqs)
    assert_close(out_f, ref, what)


@pytest.mark.parametrize("H,D", [(4, 64), (6, 128), (32, 128)])
def test_ragged_boundaries(H, D):
    """Prompts (start 0), aligned chunks (start 32, 48), chunks starting
    inside a block (50, 150, 391, 8), one query, more rows than positions,
    an empty sequence, last blocks cut at several offsets."""
    lens = [37, 70, 48, 5, 9, 0, 40, 200, 400, 399, 16]
    nq = [37, 20, 16, 12, 12, 0, 1, 200, 250, 8, 8]
    q, k_new, v_new, kp, vp, tables, lens, qs = _case(90 + H, H, D, lens, nq)
    _check(q, k_new, v_new, kp, vp, tables, lens, qs, float(np.float32(D ** -0.5)),
           f"ragged fused prefill H={H} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_heads_per_item_same_bits(D):
    """Items of 1, 2, 4 and 8 heads (H = 6: items of 4 and 8 end on a short
    head group), new tokens on and off block boundaries, one pair of blocks
    per head, several query groups owning blocks: pools and outputs equal bit
    for bit for every choice, and the oracle's append and attention."""
    H = 6
    lens = [37, 70, 48, 5, 9, 0, 40, 200, 400, 399, 16, 30, 0]
    nq = [37, 20, 16, 12, 12, 0, 1, 200, 250, 8, 8, 30, 4]   # the last: rows, no position
    q, k_new, v_new, kp, vp, tables, lens, qs = _case(70 + D, H, D, lens, nq)
    scale = float(np.float32(D ** -0.5))
    res = {}
    for k in (1, 2, 4, 8):
        print(f"prefill_append heads_per_item={k} D={D}", flush=True)
        kf, vf = to_dev(kp), to_dev(vp)
        out = pa_prefill_append(to_dev(q), to_dev(k_new), to_dev(v_new), kf, vf, to_dev(tables),
                                to_dev(lens), to_dev(qs), scale, max_context_len=int(lens.max()),
                                heads_per_item=k)
        torch.cuda.synchronize()
        res[k] = (out, kf, vf)
    for k in (2, 4, 8):
        for a, b in zip(res[k], res[1]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), k
    k_ref, v_ref = append_ref(k_new, v_new, natural_slots(tables, lens, qs), kp, vp)
    assert np.array_equal(to_host(res[8][1]).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(to_host(res[8][2]).view(np.uint16), v_ref.view(np.uint16))
    ref = paged_prefill_ref(q, k_ref, v_ref, tables, lens, qs, scale)
    assert_close(res[8][0], ref, f"fused prefill, 8 heads per item, D={D}")


def test_long_sequences_many_owners():
    """Contexts of thousands of tokens: a 700-token chunk starting inside a
    block (several query groups each own the blocks their rows start), a
    whole 1,000-token prompt, and one query at the end of 3,001."""
    lens = [4000, 1000, 3001]
    nq = [700, 1000, 1]
    q, k_new, v_new, kp, vp, tables, lens, qs = _case(97, 4, 64, lens, nq)
    _check(q, k_new, v_new, kp, vp, tables, lens, qs, float(np.float32(64 ** -0.5)),
           "long fused prefill")


def test_prompt_workload():
    """200 prompts of U[32, 256] tokens, 32 heads x 128: pools bit exact
    over the whole pools, 24 sequences in full against the oracle, and the
    fused call equal to append + prefill bit for bit."""
    c = wl.prefill()
    assert np.array_equal(c.slot_mapping,
                          natural_slots(c.block_tables, c.context_lens, c.query_start))
    seqs = list(range(0, 200, 9)) + [199]
    _check(c.q, c.k_new, c.v_new, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
           c.query_start, c.scale, "prompt workload, fused", seqs=seqs)


@pytest.mark.parametrize("cached", [1536, 1000])
def test_chunked_workload(cached):
    """512 new tokens over 1,536 cached (block aligned) or 1,000 cached (the
    new tokens start inside block 62), 32 sequences x 32 heads x 128: pools
    bit exact, three sequences in full against the oracle, and the fused
    call equal to append + prefill bit for bit."""
    c = wl.prefill(32, seed=7, cached=cached, chunk=512)
    assert np.array_equal(c.slot_mapping,
                          natural_slots(c.block_tables, c.context_lens, c.query_start))
    _check(c.q, c.k_new, c.v_new, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
           c.query_start, c.scale, f"chunked workload over {cached}, fused", seqs=[0, 13, 31])


@pytest.mark.parametrize("D", [64, 128])
def test_new_token_blocks_outside_the_pool_are_not_written(D):
    """Table entries of blocks holding new tokens set to -1 or past the
    pool: the block shared with cached tokens (written by the boundary
    kernel) and all-new blocks (written while staged).  Nothing is written
    for them, as kv_append skips those slots, so the pools equal kv_append's
    and the oracle's append of the remaining rows bit for bit; the other
    sequences' outputs equal the separate calls' and the oracle's.  Reads of
    such entries are clamped into the pool, so the test stays in bounds."""
    H = 4
    lens = [70, 150, 48, 200, 37, 400]
    nq = [20, 100, 16, 200, 37, 250]
    q, k_new, v_new, kp, vp, tables, lens, qs = _case(83 + D, H, D, lens, nq)
    NB = kp.shape[0]
    # sequence 0: new tokens start at 50, inside block 3 (boundary kernel)
    # sequence 1: new tokens 50..149; block 5 is all new, past the pool
    # sequence 3: a prompt; blocks 0 and 7 all new, -1 and past the pool
    # sequence 5: new tokens 150..399; block 9 (boundary, -1), block 20 (-1)
    bad = {(0, 3): -1, (1, 5): NB + 3, (3, 0): -1, (3, 7): NB, (5, 9): -1, (5, 20): -1}
    for (b, j), ent in bad.items():
        tables[b, j] = ent
    affected = sorted({b for b, _ in bad})
    scale = float(np.float32(D ** -0.5))
    out_f, kf, vf, out_s, ks, vs, slots = _both(q, k_new, v_new, kp, vp, tables, lens, qs,
                                                scale, int(lens.max()))
    assert torch.equal(kf.view(torch.int16), ks.view(torch.int16))
    assert torch.equal(vf.view(torch.int16), vs.view(torch.int16))
    inside = (slots >= 0) & (slots < NB * 16)
    # new positions that fall in the bad blocks: 14 + 16 + 16 + 16 + 10 + 16
    assert (~inside).sum() == 88
    k_ref, v_ref = append_ref(k_new[inside], v_new[inside], slots[inside], kp, vp)
    assert np.array_equal(to_host(kf).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(to_host(vf).view(np.uint16), v_ref.view(np.uint16))
    good = [b for b in range(len(lens)) if b not in affected]
    rows = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in good])
    assert torch.equal(out_f[rows], out_s[rows])
    ref = paged_prefill_ref(q, k_ref, v_ref, tables, lens, qs, scale, seqs=good)
    assert_close(out_f, ref, f"fused prefill, entries outside the pool, D={D}")


def test_staging_at_the_lds_limit():
    """The fused call with its LDS staging within a few entries of the
    limit: 7,100 sequences and one 16,000-token context (1,000 block ids)
    whose last 300 tokens are new (some of them in a block shared with
    cached tokens), besides thousands of short prompts and chunks."""
    rng = np.random.default_rng(95)
    B = 7100
    lens = rng.integers(0, 17, size=B)
    nq = np.minimum(lens, rng.integers(0, 3, size=B))
    lens[3500], nq[3500] = 16000, 300
    lens[0], nq[0] = 16, 16
    lens[-1], nq[-1] = 9, 9
    assert ((((B + 2) & ~1) + 1000 + 1) * 4) <= 32 * 1024
    q, k_new, v_new, kp, vp, tables, lens, qs = _case(95, 2, 64, list(lens), list(nq))
    _check(q, k_new, v_new, kp, vp, tables, lens, qs, float(np.float32(64 ** -0.5)),
           "fused prefill at the LDS staging limit")

