"""Limits of the decode on the GPU through the C ABI: a batch too large for
the flat plan's LDS staging (the call falls back to fixed partitions), and
calls issued on other streams than the default one, alone and two at once.

Outputs are compared with the float64 oracle within max-abs 2e-3 and
relative L2 1e-3, and across streams bit for bit."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import paged_decode_ref
from paged_kv_cache_03_amd import PagedKVError, pa_decode, pa_decode_append, pa_decode_workspace_size
from tests._gpu import assert_close, dev, device_pools, to_dev

pytestmark = pytest.mark.gpu


def _many_short(B, H, D, max_len, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len, size=B, endpoint=True).astype(np.int32)
    nblk = [-(-int(n) // 16) for n in lens]
    NB = sum(nblk) + 7
    ids = rng.permutation(NB).astype(np.int32)
    tables = np.full((B, max(max(nblk), 1)), -1, dtype=np.int32)
    p = 0
    for b, nb in enumerate(nblk):
        tables[b, :nb] = ids[p:p + nb]
        p += nb
    return wl.Case("many_short", H, D, NB, lens, tables, wl.normal_fp16(rng, (B, H, D)),
                   float(np.float32(D ** -0.5)), wl.normal_fp16(rng, wl.pool_shape(NB, H, D)),
                   wl.normal_fp16(rng, wl.pool_shape(NB, H, D)))


def test_batch_beyond_flat_staging_uses_partitions():
    """5,000 sequences of 0-64 tokens: the flat plan would stage 2B + 1 + the
    longest range of int32 in LDS (> 32 KiB), so the default plan is the
    partitioned one; every sequence against the oracle.  The fused append,
    which needs the flat plan, declines the shape."""
    B, H, D = 5000, 4, 64
    c = _many_short(B, H, D, 64, seed=77)
    flat_lds = (2 * B + 1 + -(-B * 4 // 512)) * 4
    assert flat_lds > 32 * 1024
    kp, vp = device_pools(c)
    print(f"large batch: B={B} workspace={pa_decode_workspace_size(B, H, D, c.max_context)}",
          flush=True)
    out = pa_decode(to_dev(c.q), kp, vp, to_dev(c.block_tables), to_dev(c.context_lens), c.scale,
                    max_context_len=c.max_context)
    torch.cuda.synchronize()
    assert_close(out, paged_decode_ref(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.scale), "batch 5000, partitioned fallback")
    assert not out[torch.from_numpy(c.context_lens == 0).to(dev())].any()
    with pytest.raises(PagedKVError) as err:
        pa_decode_append(to_dev(c.q), to_dev(c.q), to_dev(c.q), kp, vp, to_dev(c.block_tables),
                         to_dev(c.context_lens), c.scale, max_context_len=c.max_context)
    assert "unsupported" in str(err.value).lower() or err.value.code == 4


def test_other_streams_alone_and_concurrent():
    """The binding passes torch's current stream: decodes issued on two
    side streams at once, each with its own workspace, give the default
    stream's outputs bit for bit."""
    ca = wl.gpt_batch(64, seed=11)
    cb = _many_short(300, 8, 128, 700, seed=12)
    pools = [device_pools(ca), device_pools(cb)]
    args = []
    for c, (kp, vp) in zip((ca, cb), pools):
        args.append((to_dev(c.q), kp, vp, to_dev(c.block_tables), to_dev(c.context_lens), c.scale,
                     c.max_context))
    ref = [pa_decode(*a[:6], max_context_len=a[6]) for a in args]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for i, (s, a) in enumerate(zip(streams, args)):
            with torch.cuda.stream(s):
                ws = torch.empty(max(1, pa_decode_workspace_size(a[0].shape[0], a[0].shape[1],
                                                                 a[0].shape[2], a[6])),
                                 dtype=torch.uint8, device=dev())
                outs[i] = pa_decode(*a[:6], max_context_len=a[6], workspace=ws)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), f"stream {i}, repetition {rep}"
    assert_close(ref[0], paged_decode_ref(ca.q, ca.k_pool, ca.v_pool, ca.block_tables,
                                          ca.context_lens, ca.scale), "batch 64 default stream")


def test_debug_mode_rejects_contract_violations_before_launch():
    """With the host checks on, conflicting copy pairs, a slot written twice
    and a fused append into a block another sequence reads raise
    ContractError before anything is enqueued: the pools stay as they were.
    With the checks off the same calls are not inspected."""
    from paged_kv_cache_03_amd import ContractError, cow_copy_blocks, kv_append, set_debug

    H, D, NB = 2, 64, 8
    kp = torch.randn(wl.pool_shape(NB, H, D), device=dev()).half()
    vp = torch.randn(wl.pool_shape(NB, H, D), device=dev()).half()
    k0, v0 = kp.clone(), vp.clone()
    rows = torch.randn(3, H, D, device=dev()).half()
    old = set_debug(True)
    try:
        with pytest.raises(ContractError):
            cow_copy_blocks(to_dev(np.array([[1, 5], [2, 5]], dtype=np.int32)), [kp], [vp])
        with pytest.raises(ContractError):
            kv_append(rows, rows, to_dev(np.array([3, 4, 3], dtype=np.int32)), kp, vp)
        tables = to_dev(np.array([[4, 5], [4, 6]], dtype=np.int32))
        with pytest.raises(ContractError):
            pa_decode_append(rows[:2].contiguous(), rows[:2].contiguous(), rows[:2].contiguous(),
                             kp, vp, tables, to_dev(np.array([16, 30], dtype=np.int32)), 0.125)
        torch.cuda.synchronize()
        assert torch.equal(kp, k0) and torch.equal(vp, v0)
    finally:
        set_debug(old)


def test_copy_probe_copies_every_byte():
    """The copy probe (the read + write reference rate of the bench) copies
    its source whole, the tail past the last full grid stride included, and
    writes nothing past the end of its destination."""
    from paged_kv_cache_03_amd.ops import hbm_copy_probe
    n = (1 << 20) + 48
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(dev())
    dst = torch.zeros(n + 64, dtype=torch.uint8, device=dev())
    print("copy probe", n, flush=True)
    hbm_copy_probe(src, dst[:n], 64)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert not dst[n:].any()


def test_lds_probe_reads_what_it_wrote():
    """The LDS probe's 16-byte reads return the pattern it wrote (each
    wave's fold equals the one computed here), its transpose reads give
    the same fold on two runs, and every wave reports a positive cycle
    count."""
    from paged_kv_cache_03_amd.ops import lds_read_probe
    G, W, R = 8, 4, 3
    cycles = torch.zeros(G * W, dtype=torch.int64, device=dev())
    sink = torch.zeros(G * W, dtype=torch.int32, device=dev())
    print("lds probe, form 0", flush=True)
    lds_read_probe(cycles, sink, G, W, R, 0)
    torch.cuda.synchronize()
    assert (cycles > 0).all()
    # lane l of wave w reads unit i = ((r*16 + k + w) % 64) * 64 + l, which
    # holds {i, 3i, i ^ 0x5555, i + 7}, and adds x ^ w = i ^ (i + 7); the
    # wave's fold is lane 0's sum plus lane 1's (mod 2^32)
    want = []
    for w in range(W):
        tot = 0
        for lane in (0, 1):
            for r in range(R):
                for k in range(16):
                    i = ((r * 16 + k + w) % 64) * 64 + lane
                    tot += i ^ (i + 7)
        want.append(tot % (1 << 32))
    got = sink.cpu().numpy().astype(np.int64) % (1 << 32)
    assert [int(x) for x in got.reshape(G, W)[0]] == want
    assert (got.reshape(G, W) == got.reshape(G, W)[0]).all()
    print("lds probe, form 1", flush=True)
    lds_read_probe(cycles, sink, G, W, R, 1)
    torch.cuda.synchronize()
    first = sink.clone()
    lds_read_probe(cycles, sink, G, W, R, 1)
    torch.cuda.synchronize()
    assert torch.equal(first, sink) and (cycles > 0).all()

