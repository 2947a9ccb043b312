"""Parity of the grouped decode (sequences sharing leading blocks, one MFMA
column per member) with the CPU oracle on the GPU, through the C ABI.

Outputs are compared element by element with the float64 oracle within
max-abs 2e-3 and relative L2 1e-3, at small sizes in full and at the
beam-search full-step size on sampled sequences plus, for every row, against
the single-query decode (which the other tests tie to the oracle)."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import append_ref, cow_ref, grouped_decode_ref, paged_decode_ref
from paged_kv_cache_03_amd import (PagedRequest, PagePool, cow_copy_blocks, decode_groups,
                                   device_arrays, kv_append, pa_decode, pa_decode_grouped)
from tests._gpu import MAX_ABS, assert_close, dev, device_pools, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_grouped(q, kp, vp, tables, lens, offs, shared, scale, max_ctx, group_size=16,
                keep_cached=False):
    print(f"grouped decode: B={len(lens)} G={len(shared)} group_size={group_size} "
          f"max_ctx={max_ctx}", flush=True)
    out = pa_decode_grouped(to_dev(q), kp, vp, to_dev(tables), to_dev(lens), to_dev(offs),
                            to_dev(shared), scale, max_context_len=max_ctx,
                            group_size=group_size, keep_cached=keep_cached)
    torch.cuda.synchronize()
    return out


def _poison_tails(kp, vp, tables, lens):
    """NaN into every slot past a sequence's context in its last block (the
    only unused slots a table reaches)."""
    for row, n in zip(tables, lens):
        n = int(n)
        if n % 16:
            blk = int(row[n // 16])
            kp[blk, :, :, n % 16:, :] = np.nan
            vp[blk, :, :, n % 16:, :] = np.nan


def _forked_batch(seed, H, D, prompts=(45, 64, 3, 200, 32), max_branches=6):
    """Prompts forked into branches that each write 0..40 tokens of their
    own (copy-on-write of a shared partial page, as the block manager does),
    shuffled; pools drawn for every page, unused slots NaN."""
    rng = np.random.default_rng(seed)
    pool = PagePool(600, seed=seed)
    batch = []
    for n in prompts:
        owner = PagedRequest(pool)
        owner.append_tokens(n)
        batch.append(owner)
        for _ in range(int(rng.integers(0, max_branches + 1))):
            f = owner.fork()
            f.append_tokens(int(rng.integers(0, 41)))
            batch.append(f)
    rng.shuffle(batch)
    tables, lens = device_arrays(batch)
    NB = pool.num_pages
    kp = wl.normal_fp16(rng, wl.pool_shape(NB, H, D))
    vp = wl.normal_fp16(rng, wl.pool_shape(NB, H, D))
    _poison_tails(kp, vp, tables, lens)
    q = wl.normal_fp16(rng, (len(batch), H, D))
    return batch, q, kp, vp, tables, lens


@pytest.mark.parametrize("H,D", [(4, 64), (32, 128), (6, 128)])
@pytest.mark.parametrize("group_size", [16, 3])
def test_forked_batches(H, D, group_size):
    batch, q, kp, vp, tables, lens = _forked_batch(11 + H + group_size, H, D)
    order, offs, shared = decode_groups(batch, max_group=group_size)
    q, tables, lens = q[order], tables[order], lens[order]
    scale = float(np.float32(D ** -0.5))
    max_ctx = int(lens.max())
    out = run_grouped(q, to_dev(kp), to_dev(vp), tables, lens, offs, shared, scale, max_ctx,
                      group_size=group_size)
    ref = grouped_decode_ref(q, kp, vp, tables, lens, offs, shared, scale, group_size)
    assert np.array_equal(ref, paged_decode_ref(q, kp, vp, tables, lens, scale))
    assert_close(out, ref, f"forked H={H} D={D} group_size={group_size}")


def test_contract_edges():
    """Contexts of 0, a shared count past the members' full blocks, members
    past group_size, and a last group of negative size that leaves the
    sequences after it in no group."""
    H, D = 4, 64
    batch, q, kp, vp, tables, lens = _forked_batch(5, H, D, prompts=(40, 40, 17, 33),
                                                   max_branches=3)
    order, offs, shared = decode_groups(batch, max_group=16)
    q, tables, lens = q[order], tables[order], lens[order].copy()
    assert len(shared) >= 4
    lens[offs[1] - 1] = 0                        # one member of the first group is empty
    m = len(shared) - 2                          # groups 0..m-1 kept, group m negative
    offs = np.concatenate([offs[:m + 1], [offs[m] - 2]]).astype(np.int32)
    shared = (shared[:m + 1] + 5).astype(np.int32)   # clamped by the kernel
    scale = 0.125
    for gs in (16, 2):
        out = run_grouped(q, to_dev(kp), to_dev(vp), tables, lens, offs, shared, scale,
                          int(lens.max()), group_size=gs)
        ref = grouped_decode_ref(q, kp, vp, tables, lens, offs, shared, scale, gs)
        assert_close(out, ref, f"contract edges group_size={gs}")
        zero = ~ref.any(axis=(1, 2))
        assert zero.any() and not to_host(out)[zero].any(), "rows not decoded must be zero"


def test_singletons_match_oracle():
    """Every sequence its own group: the grouped kernel is then a plain
    decode on the matrix cores."""
    c = wl.gpt_batch(10, seed=1)
    kp, vp = device_pools(c)
    offs = np.arange(c.batch + 1, dtype=np.int32)
    shared = np.zeros(c.batch, dtype=np.int32)
    out = run_grouped(c.q, kp, vp, c.block_tables, c.context_lens, offs, shared, c.scale,
                      c.max_context)
    assert_close(out, paged_decode_ref(c.q, c.k_pool, c.v_pool, c.block_tables,
                                       c.context_lens, c.scale), "singletons batch10")


def test_shared_prefix_groups():
    """100 sequences on a 1024-token shared prefix, in groups of 16: through
    the shared tables (64 shared blocks) and after the copy-on-write of the
    prefix's last block (63 shared); every row against the oracle; the cache
    policy changes no bit; repeated calls agree bit for bit."""
    c = wl.shared_prefix()
    kp, vp = device_pools(c)
    offs, shared = wl.table_groups(c.shared_tables, c.context_lens)
    assert set(shared.tolist()) == {64}
    out = run_grouped(c.q, kp, vp, c.shared_tables, c.context_lens, offs, shared, c.scale,
                      c.max_context)
    ref = paged_decode_ref(c.q, c.k_pool, c.v_pool, c.shared_tables, c.context_lens, c.scale)
    assert_close(out, ref, "shared prefix, 64 shared blocks")
    cow_copy_blocks(to_dev(c.cow_pairs), [kp], [vp])
    k_ref, v_ref = cow_ref([c.k_pool, c.v_pool], c.cow_pairs)
    offs, shared = wl.table_groups(c.block_tables, c.context_lens)
    assert set(shared.tolist()) == {63}
    out = run_grouped(c.q, kp, vp, c.block_tables, c.context_lens, offs, shared, c.scale,
                      c.max_context)
    assert_close(out, paged_decode_ref(c.q, k_ref, v_ref, c.block_tables, c.context_lens,
                                       c.scale), "shared prefix after copy-on-write")
    again = run_grouped(c.q, kp, vp, c.block_tables, c.context_lens, offs, shared, c.scale,
                        c.max_context, keep_cached=True)
    assert torch.equal(again, out)


def test_beam_step_full_size():
    """The 4-beam full step at full size (200 sequences x 2048 tokens x 32
    heads x 128, 127 shared blocks per group of 4): copy-on-write of each
    group's last block, append of each beam's token, grouped decode.
    Sampled sequences against the oracle (pools read back before any kernel),
    every row against the single-query decode."""
    c = wl.full_step(layers=1, beams=4)
    torch.cuda.empty_cache()
    kp, vp = device_pools(c, 0)
    seqs = [0, 1, 2, 3, 57, 99, 150, 199]
    ids = np.unique(np.concatenate([c.block_tables[seqs].ravel(), c.cow_pairs[:, 0]]))
    idx = torch.from_numpy(ids.astype(np.int64)).to(dev())
    k_s, v_s = to_host(kp.index_select(0, idx)), to_host(vp.index_select(0, idx))
    remap = {int(b): i for i, b in enumerate(ids)}
    cow_copy_blocks(to_dev(c.cow_pairs), [kp], [vp])
    kv_append(to_dev(c.k_new[0]), to_dev(c.v_new[0]), to_dev(c.slot_mapping), kp, vp)
    offs, shared = wl.table_groups(c.block_tables, c.context_lens)
    assert len(shared) == 50 and set(shared.tolist()) == {127}
    out = run_grouped(c.q[0], kp, vp, c.block_tables, c.context_lens, offs, shared, c.scale, 2048)
    flat = pa_decode(to_dev(c.q[0]), kp, vp, to_dev(c.block_tables), to_dev(c.context_lens),
                     c.scale, max_context_len=2048)
    torch.cuda.synchronize()
    # oracle on the sampled sequences: copy, append, decode
    pairs = np.array([[remap.get(int(s), -1), remap.get(int(d), -1)] for s, d in c.cow_pairs])
    pairs = pairs[(pairs >= 0).all(axis=1)]
    k_s, v_s = cow_ref([k_s, v_s], pairs)
    slots = np.array([remap[int(x) // 16] * 16 + int(x) % 16 for x in c.slot_mapping[seqs]])
    k_s, v_s = append_ref(c.k_new[0][seqs], c.v_new[0][seqs], slots, k_s, v_s)
    tables = np.vectorize(lambda x: remap.get(int(x), -1))(c.block_tables[seqs]).astype(np.int32)
    ref = np.full((c.batch, c.num_heads, c.head_dim), np.nan)
    ref[seqs] = paged_decode_ref(c.q[0][seqs], k_s, v_s, tables, c.context_lens[seqs], c.scale)
    assert_close(out, ref, "beam step, sampled sequences")
    diff = (out.float() - flat.float()).abs().max().item()
    print(f"[beam step] grouped vs single-query decode, all rows: max |diff| = {diff:.3e}",
          flush=True)
    assert diff <= 2 * MAX_ABS
    del kp, vp
    torch.cuda.empty_cache()
