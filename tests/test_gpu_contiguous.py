"""The contiguous virtual-memory KV cache (physical chunks mapped on demand)
and the decode over it, on the GPU through the C ABI.

Decode outputs are compared with the float64 oracle within max-abs 2e-3 and
relative L2 1e-3, and with the paged decode of the same tokens bit for bit
(same kernel, same positions); mapping accounting is checked exactly."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import contiguous_decode_ref
from paged_kv_cache_03_amd import VirtualKV, contig_decode, pa_decode
from tests._gpu import assert_close, dev, device_pools, to_dev, to_host

pytestmark = pytest.mark.gpu


def _round_up(x, a):
    return -(-x // a) * a


def _expected_mapped(lens, row_bytes, chunk, buffers):
    return sum(_round_up(_round_up(int(n), 16) * row_bytes, chunk) for n in lens) * buffers


def _append_all(vkv, layer, k_rows, v_rows, lens, L):
    """Write every token of every sequence (host rows [B*L][H][D]) through
    pkv_vkv_append."""
    seq = np.concatenate([np.full(int(n), b, dtype=np.int32) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(int(n), dtype=np.int32) for n in lens])
    rows = seq.astype(np.int64) * L + pos
    vkv.append(layer, to_dev(k_rows[rows]), to_dev(v_rows[rows]), to_dev(seq), to_dev(pos))


def test_lifecycle_small():
    """Grow, append, decode; a context above a request's mapped tokens is
    clamped to them; release and grow again reuse the pooled chunks."""
    rng = np.random.default_rng(60)
    H, D, L, B = 4, 64, 512, 6
    row = H * D * 2
    chunk = 64 << 10
    lens = np.array([1, 15, 16, 100, 512, 0], dtype=np.int32)
    vkv = VirtualKV(B, L, 1, H, D, chunk_bytes=chunk)
    try:
        for b, n in enumerate(lens):
            vkv.grow(b, int(n))
        st = vkv.stats()
        assert st["mapped_bytes"] == _expected_mapped(lens, row, chunk, 2)
        assert st["chunk_bytes"] == chunk and st["granularity"] > 0 and chunk % st["granularity"] == 0
        k_rows = np.full((B * L, H, D), np.nan, dtype=np.float16)
        v_rows = np.full((B * L, H, D), np.nan, dtype=np.float16)
        for b, n in enumerate(lens):
            k_rows[b * L:b * L + n] = wl.normal_fp16(rng, (int(n), H, D))
            v_rows[b * L:b * L + n] = wl.normal_fp16(rng, (int(n), H, D))
        _append_all(vkv, 0, k_rows, v_rows, lens, L)
        # rows past a request's mapped tokens are skipped, not written
        vkv.append(0, to_dev(wl.normal_fp16(rng, (2, H, D))), to_dev(wl.normal_fp16(rng, (2, H, D))),
                   to_dev(np.array([5, 0], dtype=np.int32)), to_dev(np.array([0, 128], dtype=np.int32)))
        # (request 0 maps one 64 KiB chunk = 128 rows; request 5 maps none)
        q = wl.normal_fp16(rng, (B, H, D))
        asked = lens.copy()
        asked[5] = 64                              # nothing mapped: clamped to 0, a zero row
        out = contig_decode(to_dev(q), vkv, 0, to_dev(asked), 0.125, max_context_len=L)
        torch.cuda.synchronize()
        ref = contiguous_decode_ref(q, k_rows, v_rows, L, lens, 0.125)
        assert_close(out, ref, "virtual contiguous cache, small")
        assert not to_host(out)[5].any()
        # release one request and grow another: the pool serves it
        created = vkv.stats()["chunks_created"]
        vkv.release(4)
        assert vkv.stats()["pooled_bytes"] == _round_up(512 * row, chunk) * 2
        vkv.grow(3, 300)
        assert vkv.stats()["chunks_created"] == created
        lens2 = lens.copy()
        lens2[4], lens2[3] = 0, 300
        k_rows[3 * L + 100:3 * L + 300] = wl.normal_fp16(rng, (200, H, D))
        v_rows[3 * L + 100:3 * L + 300] = wl.normal_fp16(rng, (200, H, D))
        _append_all(vkv, 0, k_rows, v_rows, lens2, L)
        out = contig_decode(to_dev(q), vkv, 0, to_dev(lens2), 0.125, max_context_len=L)
        torch.cuda.synchronize()
        assert_close(out, contiguous_decode_ref(q, k_rows, v_rows, L, lens2, 0.125),
                     "virtual contiguous cache after release and regrow")
        assert vkv.stats()["mapped_bytes"] == _expected_mapped(lens2, row, chunk, 2)
    finally:
        vkv.close()


def test_batch200_contiguous_equals_paged_bitwise():
    """The headline batch (200 sequences, 32 heads x 128, contexts up to
    2048) copied token by token from the block pool into a 2 MiB-chunk
    virtual cache: the contiguous decode gives the paged decode's output bit
    for bit, and maps exactly the rounded-up chunks."""
    c = wl.gpt_batch(200, seed=2, append=True, fill=False)
    kp, vp = device_pools(c)
    H, D, L = c.num_heads, c.head_dim, 2048
    chunk = 2 << 20
    q = to_dev(c.q)
    lens = to_dev(c.context_lens)
    paged = pa_decode(q, kp, vp, to_dev(c.block_tables), lens, c.scale, max_context_len=c.max_context)
    vkv = VirtualKV(c.batch, L, 1, H, D, chunk_bytes=chunk)
    try:
        for b, n in enumerate(c.context_lens):
            vkv.grow(b, int(n))
        assert vkv.stats()["mapped_bytes"] == _expected_mapped(c.context_lens, H * D * 2, chunk, 2)
        # token rows of every sequence, gathered from the tile layout on the device
        NB = c.num_blocks
        tok = lambda pool: pool.view(NB, H, D // 8, 16, 8).permute(0, 3, 1, 2, 4).reshape(NB, 16, H, D)
        seq = np.concatenate([np.full(int(n), b, dtype=np.int32) for b, n in enumerate(c.context_lens)])
        pos = np.concatenate([np.arange(int(n), dtype=np.int32) for n in c.context_lens])
        blk = torch.from_numpy(c.block_tables[seq, pos // 16].astype(np.int64)).to(dev())
        slot = torch.from_numpy((pos % 16).astype(np.int64)).to(dev())
        k_tok = tok(kp)[blk, slot].contiguous()
        v_tok = tok(vp)[blk, slot].contiguous()
        vkv.append(0, k_tok, v_tok, to_dev(seq), to_dev(pos))
        del k_tok, v_tok
        out = contig_decode(q, vkv, 0, lens, c.scale, max_context_len=c.max_context)
        torch.cuda.synchronize()
        assert torch.equal(out, paged)
    finally:
        vkv.close()
