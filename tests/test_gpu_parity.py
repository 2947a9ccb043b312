"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Append and copy-on-write are compared bit for bit over whole pools; decode is
compared element by element within max-abs 2e-3 and relative L2 1e-3 of the
float64 oracle.  Full-size workloads use the default launch configuration
(the one the bench times); the full-step workload is checked on sampled
sequences."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import append_ref, attention_ref, cow_ref, paged_decode_ref
from paged_kv_cache_03_amd import (PagedRequest, PagePool, _lib, cow_copy_blocks, device_arrays,
                                   kv_append, pa_decode, pool_shape)
from tests._gpu import assert_close, dev, device_pools, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_decode(case, kp, vp, tables=None, partition=0, keep_cached=False):
    tables = case.block_tables if tables is None else tables
    q = to_dev(case.q)
    out = pa_decode(q, kp, vp, to_dev(tables), to_dev(case.context_lens), case.scale,
                    max_context_len=case.max_context, partition_tokens=partition,
                    keep_cached=keep_cached)
    torch.cuda.synchronize()
    return out


def oracle(case, kp, vp, tables=None, seqs=None):
    tables = case.block_tables if tables is None else tables
    return paged_decode_ref(case.q, kp, vp, tables, case.context_lens, case.scale, seqs=seqs)


def test_native_library_is_loaded():
    lib = _lib.load_library()
    assert lib._name == _lib.LIB_PATH
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


@pytest.mark.parametrize("partition", [0, 16, 32, 512])
def test_tiny(partition):
    c = wl.tiny()
    kp, vp = device_pools(c)
    out = run_decode(c, kp, vp, partition=partition)
    assert_close(out, oracle(c, c.k_pool, c.v_pool), f"tiny part={partition}")
    # context 1: the output is that token's value exactly
    blk = int(c.block_tables[0, 0])
    v0 = c.v_pool[blk, :, :, 0, :].reshape(c.num_heads, c.head_dim)
    assert np.array_equal(to_host(out)[0].view(np.uint16), v0.view(np.uint16))


@pytest.mark.parametrize("partition", [0, 16])
def test_tiny_with_unused_slots_poisoned(partition):
    c = wl.poison_unused(wl.tiny())
    kp, vp = device_pools(c)
    out = run_decode(c, kp, vp, partition=partition)
    assert_close(out, oracle(c, c.k_pool, c.v_pool), f"tiny NaN-poisoned part={partition}")


def _edge_case(H, D, lens, seed):
    rng = np.random.default_rng(seed)
    nblk = [-(-n // 16) for n in lens]
    NB = sum(nblk) + 5
    ids = rng.permutation(NB).astype(np.int32)
    width = max(max(nblk), 1)
    tables = np.full((len(lens), width), -1, dtype=np.int32)
    p = 0
    for b, nb in enumerate(nblk):
        tables[b, :nb] = ids[p:p + nb]
        p += nb
    c = wl.Case("edge", H, D, NB, np.array(lens, dtype=np.int32), tables,
                wl.normal_fp16(rng, (len(lens), H, D)), float(np.float32(D ** -0.5)),
                wl.normal_fp16(rng, wl.pool_shape(NB, H, D)),
                wl.normal_fp16(rng, wl.pool_shape(NB, H, D)))
    return wl.poison_unused(c)


@pytest.mark.parametrize("H,D", [(32, 128), (4, 64), (6, 128), (3, 64)])
@pytest.mark.parametrize("partition", [0, 16, 256, 512])
def test_edge_contexts(H, D, partition):
    """Empty, single-token, block-boundary and maximum contexts, odd head
    counts (2- and 1-wave workgroups), NaN in every unread slot."""
    c = _edge_case(H, D, [0, 1, 15, 16, 17, 255, 256, 257, 2048, 33], seed=H + D + partition)
    kp, vp = device_pools(c)
    out = run_decode(c, kp, vp, partition=partition, keep_cached=(H % 2 == 1))
    ref = oracle(c, c.k_pool, c.v_pool)
    assert_close(out, ref, f"edge H={H} D={D} part={partition}")
    assert not to_host(out)[0].any()          # empty context -> zero row


@pytest.mark.parametrize("partition", [0, 512])
def test_long_contexts(partition):
    """Contexts far past the 2,048-token workloads (65,543 and 40,000
    tokens: thousands of blocks per sequence, ranges and partitions that
    stage hundreds of block ids) next to tiny and empty ones."""
    c = _edge_case(4, 64, [65543, 3, 40000, 0], seed=91 + partition)
    kp, vp = device_pools(c)
    out = run_decode(c, kp, vp, partition=partition)
    assert_close(out, oracle(c, c.k_pool, c.v_pool), f"long contexts part={partition}")
    assert not to_host(out)[3].any()


def test_batch10():
    c = wl.gpt_batch(10, seed=1)
    kp, vp = device_pools(c)
    for part in (0, 64, 256):
        out = run_decode(c, kp, vp, partition=part)
        assert_close(out, oracle(c, c.k_pool, c.v_pool), f"batch10 part={part}")


def test_batch200_append_then_decode():
    """The headline workload: one new token per sequence appended through its
    slot, then decode over every context, in the default launch
    configuration."""
    c = wl.gpt_batch(200, seed=2, append=True, fill=False)
    kp, vp = device_pools(c)
    k_host, v_host = to_host(kp), to_host(vp)
    kv_append(to_dev(c.k_new), to_dev(c.v_new), to_dev(c.slot_mapping), kp, vp)
    torch.cuda.synchronize()
    k_ref, v_ref = append_ref(c.k_new, c.v_new, c.slot_mapping, k_host, v_host)
    assert np.array_equal(to_host(kp).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(to_host(vp).view(np.uint16), v_ref.view(np.uint16))
    out = run_decode(c, kp, vp)
    assert_close(out, oracle(c, k_ref, v_ref), "batch200 append+decode")


def test_batch200_other_partitions():
    c = wl.gpt_batch(200, seed=2, append=True, fill=False)
    kp, vp = device_pools(c)
    ref = oracle(c, to_host(kp), to_host(vp), seqs=range(0, 200, 7))
    for part in (128, 512):
        assert_close(run_decode(c, kp, vp, partition=part), ref, f"batch200 part={part}")


def test_shared_prefix_copy_on_write():
    """1024-token prefix shared by 100 tables; its last block copied per
    sequence.  The copy is bit exact over whole pools, and decode through the
    private copies equals decode through the shared block bit for bit."""
    c = wl.shared_prefix(fill=False)
    kp, vp = device_pools(c)
    k_host, v_host = to_host(kp), to_host(vp)
    shared_out = run_decode(c, kp, vp, tables=c.shared_tables)
    cow_copy_blocks(to_dev(c.cow_pairs), [kp], [vp])
    torch.cuda.synchronize()
    k_ref, v_ref = cow_ref([k_host, v_host], c.cow_pairs)
    assert np.array_equal(to_host(kp).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(to_host(vp).view(np.uint16), v_ref.view(np.uint16))
    out = run_decode(c, kp, vp)
    assert torch.equal(out, shared_out)
    assert_close(out, oracle(c, k_ref, v_ref), "shared prefix")
    # the cache policy changes no bit, with either strategy
    assert torch.equal(run_decode(c, kp, vp, keep_cached=True), out)
    p256 = run_decode(c, kp, vp, partition=256)
    assert torch.equal(run_decode(c, kp, vp, partition=256, keep_cached=True), p256)


def test_shared_prefix_ending_inside_a_block():
    """A 1000-token prefix (62 full blocks + 8 tokens): the partially filled
    block is copied per sequence, the suffix is appended into the copy and
    beyond, and unread slots hold NaN."""
    c = wl.poison_unused(wl.shared_prefix(batch=40, seed=5, prefix_tokens=1000, suffix_max=300))
    kp, vp = device_pools(c)
    cow_copy_blocks(to_dev(c.cow_pairs), [kp], [vp])
    kv_append(to_dev(c.k_new), to_dev(c.v_new), to_dev(c.slot_mapping), kp, vp)
    torch.cuda.synchronize()
    k_ref, v_ref = cow_ref([c.k_pool, c.v_pool], c.cow_pairs)
    k_ref, v_ref = append_ref(c.k_new, c.v_new, c.slot_mapping, k_ref, v_ref)
    assert np.array_equal(to_host(kp).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(to_host(vp).view(np.uint16), v_ref.view(np.uint16))
    out = run_decode(c, kp, vp)
    assert_close(out, oracle(c, k_ref, v_ref), "prefix 1000 cow+append")


class _Sample:
    """Host copies of the blocks a few sequences read, taken from the
    device pools before any kernel touches them, renumbered compactly."""

    def __init__(self, case, kp, vp, seqs):
        self.seqs = list(seqs)
        sets = [case.block_tables[self.seqs]]
        if case.shared_tables is not None:
            sets.append(case.shared_tables[self.seqs])
        ids = np.unique(np.concatenate([t.reshape(-1) for t in sets]))
        ids = ids[ids >= 0]
        self.remap = {int(b): i for i, b in enumerate(ids)}
        idx = torch.from_numpy(ids.astype(np.int64)).to(kp.device)
        self.k = to_host(kp.index_select(0, idx))
        self.v = to_host(vp.index_select(0, idx))
        self.case = case

    def _ids(self, a):
        return np.array([self.remap.get(int(x), -1) for x in np.ravel(a)],
                        dtype=np.int32).reshape(np.shape(a))

    def reference(self, q, k_new, v_new):
        """cow_ref, then append_ref of the sampled rows, then the oracle."""
        c = self.case
        k, v = self.k, self.v
        if c.cow_pairs is not None:
            pairs = self._ids(c.cow_pairs)
            keep = (pairs >= 0).all(axis=1)
            k, v = cow_ref([k, v], pairs[keep])
        slots = self._ids(c.slot_mapping[self.seqs] // 16) * 16 + c.slot_mapping[self.seqs] % 16
        k, v = append_ref(k_new[self.seqs], v_new[self.seqs], slots, k, v)
        out = np.full((c.batch, c.num_heads, c.head_dim), np.nan)
        tables = self._ids(c.block_tables[self.seqs])
        out[self.seqs] = paged_decode_ref(q[self.seqs], k, v, tables,
                                          c.context_lens[self.seqs], c.scale)
        return out


@pytest.mark.parametrize("beams", [1, 4])
def test_full_step_sampled(beams):
    """Full-step shapes (200 sequences x 2048 tokens x 32 heads x 128) on two
    layers: copy-on-write for the beam groups, then per layer append and
    decode; sampled sequences checked against the oracle (fed from the pools
    as drawn), copies and appends bit exact."""
    c = wl.full_step(layers=2, beams=beams)
    torch.cuda.empty_cache()
    seqs = [0, 1, 2, 3, 57, 99, 150, 199]
    pools = [device_pools(c, layer) for layer in range(c.num_layers)]
    samples = [_Sample(c, kp, vp, seqs) for kp, vp in pools]
    if c.cow_pairs is not None:
        src = torch.from_numpy(c.cow_pairs[:, 0].astype(np.int64)).to(dev())
        dst = torch.from_numpy(c.cow_pairs[:, 1].astype(np.int64)).to(dev())
        before = [(kp.index_select(0, src), vp.index_select(0, src)) for kp, vp in pools]
        cow_copy_blocks(to_dev(c.cow_pairs), [p[0] for p in pools], [p[1] for p in pools])
        for (kp, vp), (ks, vs) in zip(pools, before):
            assert torch.equal(kp.index_select(0, dst), ks)
            assert torch.equal(vp.index_select(0, dst), vs)
    slots = to_dev(c.slot_mapping)
    tables = to_dev(c.block_tables)
    lens = to_dev(c.context_lens)
    blk = torch.from_numpy((c.slot_mapping // 16).astype(np.int64)).to(dev())
    rows = torch.arange(c.batch, device=dev())
    for layer, (kp, vp) in enumerate(pools):
        kn, vn = to_dev(c.k_new[layer]), to_dev(c.v_new[layer])
        kv_append(kn, vn, slots, kp, vp)
        out = pa_decode(to_dev(c.q[layer]), kp, vp, tables, lens, c.scale, max_context_len=2048)
        torch.cuda.synchronize()
        # every appended token sits at position 15 of the block its slot names
        got = kp.index_select(0, blk)[rows, :, :, 15, :]
        assert torch.equal(got.reshape(c.batch, c.num_heads, c.head_dim), kn)
        ref = samples[layer].reference(c.q[layer], c.k_new[layer], c.v_new[layer])
        assert_close(out, ref, f"full step beams={beams} layer={layer}")
    del pools
    torch.cuda.empty_cache()


def test_physical_relabelling_is_bitwise_invariant():
    c = wl.gpt_batch(10, seed=1)
    kp, vp = device_pools(c)
    out = run_decode(c, kp, vp)
    perm = np.random.default_rng(0).permutation(c.num_blocks)
    inv = torch.from_numpy(np.argsort(perm).astype(np.int64)).to(dev())
    kp2, vp2 = kp.index_select(0, inv), vp.index_select(0, inv)   # block i moves to perm[i]
    t2 = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    out2 = run_decode(c, kp2, vp2, tables=t2)
    assert torch.equal(out, out2)


def test_repeatable():
    c = wl.gpt_batch(200, seed=2, append=True, fill=False)
    kp, vp = device_pools(c)
    a = run_decode(c, kp, vp)
    b = run_decode(c, kp, vp)
    assert torch.equal(a, b)


def test_block_manager_end_to_end():
    """Requests grow token by token through the host block manager (shuffled
    pool, forks with copy-on-write); every few steps the decode over the
    paged cache is compared with plain attention over each request's
    contiguous history kept by the test."""
    rng = np.random.default_rng(42)
    H, D = 8, 128
    pool = PagePool(400, seed=1)
    kp = torch.full(pool_shape(400, H, D), float("nan"), dtype=torch.float16, device=dev())
    vp = torch.full_like(kp, float("nan"))
    reqs, hist = [], []
    for i in range(6):
        r = PagedRequest(pool, f"r{i}")
        reqs.append(r)
        hist.append(([], []))
    scale = float(np.float32(D ** -0.5))
    checked = 0
    for step in range(140):
        if step in (30, 75):            # fork two requests (parallel sampling)
            for src in (0, 3):
                reqs.append(reqs[src].fork())
                hist.append((list(hist[src][0]), list(hist[src][1])))
        slots = np.array([r.append_token() for r in reqs], dtype=np.int32)
        pairs = pool.take_copy_pairs()
        if pairs.size:
            cow_copy_blocks(to_dev(pairs), [kp], [vp])
        k_new = wl.normal_fp16(rng, (len(reqs), H, D))
        v_new = wl.normal_fp16(rng, (len(reqs), H, D))
        for i in range(len(reqs)):
            hist[i][0].append(k_new[i])
            hist[i][1].append(v_new[i])
        kv_append(to_dev(k_new), to_dev(v_new), to_dev(slots), kp, vp)
        if step % 9 == 0 or step == 139:
            q = wl.normal_fp16(rng, (len(reqs), H, D))
            tables, lens = device_arrays(reqs)
            out = pa_decode(to_dev(q), kp, vp, to_dev(tables), to_dev(lens), scale,
                            max_context_len=int(lens.max()), partition_tokens=32)
            torch.cuda.synchronize()
            ref = np.stack([attention_ref(q[i], np.stack(hist[i][0]), np.stack(hist[i][1]), scale)
                            for i in range(len(reqs))])
            assert_close(out, ref, f"block manager step {step}")
            checked += 1
    assert checked >= 15
    pool.check()


def test_plain_entry_point_at_the_headline_shape():
    """``pkv_pa_decode`` itself, called through ctypes with its own
    signature (no binding in between) on the batch-200 workload (32 heads x
    128, contexts up to 2048): its output equals ``pkv_pa_decode_ex`` with
    the default partition and no flags bit for bit, and all 200 sequences
    match the float64 oracle within max-abs 2e-3 and relative L2 1e-3."""
    import ctypes

    lib = _lib.load_library()
    c = wl.gpt_batch(200, seed=2, append=True)   # the headline batch; decoded as it stands
    kp, vp = device_pools(c)
    q, tables, lens = to_dev(c.q), to_dev(c.block_tables), to_dev(c.context_lens)
    B, H, D = c.q.shape
    NB = kp.shape[0]
    ws_bytes = lib.pkv_pa_decode_workspace_size(B, H, D, c.max_context)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    i32p = lambda t: ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    outs = []
    for ex in (False, True):
        out = torch.full((B, H, D), float("nan"), dtype=torch.float16, device=dev())
        common = (p(q), p(kp), p(vp), i32p(tables), tables.shape[1], i32p(lens), c.max_context,
                  B, H, D, 16, NB, ctypes.c_float(c.scale), p(out), p(ws), ws_bytes)
        print(f"pkv_pa_decode{'_ex' if ex else ''}: B={B} H={H} D={D} NB={NB}", flush=True)
        code = lib.pkv_pa_decode_ex(*common, 0, 0, stream) if ex else \
            lib.pkv_pa_decode(*common, stream)
        assert code == 0, lib.pkv_status_string(code)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert_close(outs[0], oracle(c, c.k_pool, c.v_pool), "pkv_pa_decode, batch 200")
