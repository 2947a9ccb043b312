"""torch-facing wrappers over the C ABI: argument marshalling only.

Tensors must be on one HIP device and contiguous; every call is enqueued on
that device's current torch stream and returns without synchronising.  All
arithmetic happens in the HIP kernels of libpagedkv.so.

Pool layout (both K and V, per layer): ``[num_blocks][H][D/8][16][8]``
fp16; ``pool_shape`` gives it.
"""

import ctypes

import torch

from . import _lib, validate

BLOCK_TOKENS = 16


def pool_shape(num_blocks, num_heads, head_dim):
    return (num_blocks, num_heads, head_dim // 8, BLOCK_TOKENS, 8)


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _pool_blocks(pool, name, H, D, device):
    _need(pool, name, torch.float16, device)
    per_block = H * BLOCK_TOKENS * D
    if pool.numel() % per_block:
        raise ValueError(f"{name} is not a whole number of [H][D/8][16][8] blocks")
    return pool.numel() // per_block


def pa_decode_workspace_size(batch, num_heads, head_dim, max_context_len, partition_tokens=0):
    lib = _lib.load_library()
    return int(lib.pkv_pa_decode_workspace_size_ex(batch, num_heads, head_dim,
                                                   max_context_len, partition_tokens))


def default_partition(batch, num_heads, head_dim, max_context_len):
    return int(_lib.load_library().pkv_pa_decode_default_partition(
        batch, num_heads, head_dim, max_context_len))


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None, *,
              max_context_len=None, workspace=None, partition_tokens=0, keep_cached=False):
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the first
    context_lens[b] tokens of sequence b, read through block_tables[b].

    q: [B][H][D] fp16; pools: [NB][H][D/8][16][8] fp16; block_tables:
    [B][max_blocks] int32; context_lens: [B] int32.  ``max_context_len`` must
    be >= every context length; when omitted it is read back from the device
    (one synchronisation).  ``workspace``: a uint8 device tensor of at least
    ``pa_decode_workspace_size(...)`` bytes, allocated here when omitted.
    ``keep_cached``: load K/V with the normal cache policy instead of
    streaming it, for batches whose tables share blocks (see
    ``blocks.tables_share_blocks``); the result is the same either way."""
    lib = _lib.load_library()
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    B, H, D = q.shape
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, ndim=2)
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens do not match the batch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, dev, ndim=3)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B][H][D]")
    need = pa_decode_workspace_size(B, H, D, max_context_len, partition_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        ws_bytes = workspace.numel()
    with torch.cuda.device(dev):
        code = lib.pkv_pa_decode_ex(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), max_context_len, B, H, D, BLOCK_TOKENS, NB, float(scale),
            _ptr(out), _ptr(workspace), ws_bytes, partition_tokens,
            _lib.DECODE_KEEP_KV_CACHED if keep_cached else 0, _stream_handle(dev))
    _lib.check("pkv_pa_decode", code)
    return out


def pa_decode_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                     out=None, *, max_context_len=None, workspace=None, keep_cached=False):
    """One decode step with its append fused in (one launch): the new token
    of every non-empty sequence b (k_new[b], v_new[b]: [B][H][D] fp16) is
    written to its last position context_lens[b] - 1 in the pools, then
    ``pa_decode`` runs over the context, the new token included.  Same pools
    and output, bit for bit, as ``kv_append`` with those slots followed by
    ``pa_decode``.  The other arguments are those of ``pa_decode``."""
    lib = _lib.load_library()
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    B, H, D = q.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, torch.float16, dev, ndim=3)
        if tuple(t.shape) != (B, H, D):
            raise ValueError(f"{name} must be [B][H][D] like q")
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, ndim=2)
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens do not match the batch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, dev, ndim=3)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B][H][D]")
    need = pa_decode_workspace_size(B, H, D, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        ws_bytes = workspace.numel()
    if validate.debug_enabled():
        validate.check_decode_append(block_tables, context_lens)
    with torch.cuda.device(dev):
        code = lib.pkv_pa_decode_append(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), max_context_len, B, H, D, BLOCK_TOKENS, NB,
            float(scale), _ptr(out), _ptr(workspace), ws_bytes,
            _lib.DECODE_KEEP_KV_CACHED if keep_cached else 0, _stream_handle(dev))
    _lib.check("pkv_pa_decode_append", code)
    return out


def pa_decode_grouped_workspace_size(batch, num_heads, head_dim, max_context_len, num_groups,
                                     group_size=16):
    return int(_lib.load_library().pkv_pa_decode_grouped_workspace_size(
        batch, num_heads, head_dim, max_context_len, num_groups, group_size))


def pa_decode_grouped(q, k_pool, v_pool, block_tables, context_lens, group_offsets,
                      shared_blocks, scale, out=None, *, max_context_len=None, group_size=16,
                      workspace=None, keep_cached=False):
    """``pa_decode`` for a batch arranged in groups of sequences that share
    leading blocks (see ``blocks.decode_groups``): group g is sequences
    [group_offsets[g], group_offsets[g+1]) and its first shared_blocks[g]
    logical blocks are read once for all its members.  ``group_offsets``
    ([G+1]) and ``shared_blocks`` ([G]) are int32 device tensors; the other
    arguments are as for ``pa_decode``."""
    lib = _lib.load_library()
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    B, H, D = q.shape
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, ndim=2)
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    _need(group_offsets, "group_offsets", torch.int32, dev, ndim=1)
    _need(shared_blocks, "shared_blocks", torch.int32, dev, ndim=1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens do not match the batch")
    G = shared_blocks.shape[0]
    if group_offsets.shape[0] != G + 1:
        raise ValueError("group_offsets must have one entry more than shared_blocks")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, dev, ndim=3)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B][H][D]")
    need = pa_decode_grouped_workspace_size(B, H, D, max_context_len, G, group_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        ws_bytes = workspace.numel()
    with torch.cuda.device(dev):
        code = lib.pkv_pa_decode_grouped(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), max_context_len, _ptr(group_offsets), _ptr(shared_blocks), G,
            group_size, B, H, D, BLOCK_TOKENS, NB, float(scale), _ptr(out), _ptr(workspace),
            ws_bytes, _lib.DECODE_KEEP_KV_CACHED if keep_cached else 0, _stream_handle(dev))
    _lib.check("pkv_pa_decode_grouped", code)
    return out


def pa_decode_append_noalloc(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                             out, *, max_context_len, keep_cached=False):
    """``pa_decode_append`` through ``pkv_pa_decode_append_noalloc``: no
    workspace, nothing allocated (the caller passes ``out`` and
    ``max_context_len``); the partial results live in the library's fixed
    per-GPU scratch array, so calls that overlap on one GPU race."""
    lib = _lib.load_library()
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    B, H, D = q.shape
    for name, t in (("k_new", k_new), ("v_new", v_new), ("out", out)):
        _need(t, name, torch.float16, dev, ndim=3)
        if tuple(t.shape) != (B, H, D):
            raise ValueError(f"{name} must be [B][H][D] like q")
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, ndim=2)
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens do not match the batch")
    if validate.debug_enabled():
        validate.check_decode_append(block_tables, context_lens)
    with torch.cuda.device(dev):
        code = lib.pkv_pa_decode_append_noalloc(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), int(max_context_len), B, H, D,
            BLOCK_TOKENS, NB, float(scale), _ptr(out),
            _lib.DECODE_KEEP_KV_CACHED if keep_cached else 0, _stream_handle(dev))
    _lib.check("pkv_pa_decode_append_noalloc", code)
    return out


def pa_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, out=None, *,
               max_context_len=None, heads_per_item=None):
    """Causal attention of each sequence's last n_b cached tokens (its rows
    query_start[b] .. query_start[b+1]-1 of q, [T][H][D] fp16) over its paged
    cache: row i of sequence b sits at position context_lens[b] - n_b + i.
    ``query_start`` is an int32 device tensor of B+1 entries; the other
    arguments are as for ``pa_decode``.  ``heads_per_item`` (1, 2, 4 or 8;
    None: chosen from the sizes) sets how many heads of one 128-row query
    group a workgroup takes at a time; the output does not depend on it."""
    return _prefill(q, None, None, k_pool, v_pool, block_tables, context_lens, query_start,
                    scale, out, max_context_len, heads_per_item)


def pa_prefill_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, query_start,
                      scale, out=None, *, max_context_len=None, heads_per_item=None):
    """``pa_prefill`` with the append of the new tokens fused in: row r of
    k_new / v_new ([T][H][D] fp16, like q) is written to the slot of its
    position (through the block table) in both pools, and the queries attend
    as for ``pa_prefill``; ``context_lens`` counts the new tokens.  Pools and
    output equal ``kv_append`` followed by ``pa_prefill`` bit for bit."""
    return _prefill(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, query_start,
                    scale, out, max_context_len, heads_per_item)


_HEADS_CODE = {None: 0, 1: 1, 2: 2, 4: 3, 8: 4}


def _prefill(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, query_start, scale,
             out, max_context_len, heads_per_item):
    if heads_per_item not in _HEADS_CODE:
        raise ValueError("heads_per_item must be None, 1, 2, 4 or 8")
    flags = _HEADS_CODE[heads_per_item] << 8
    lib = _lib.load_library()
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    T, H, D = q.shape
    append = k_new is not None
    if append:
        _need(k_new, "k_new", torch.float16, dev, ndim=3)
        _need(v_new, "v_new", torch.float16, dev, ndim=3)
        if tuple(k_new.shape) != (T, H, D) or tuple(v_new.shape) != (T, H, D):
            raise ValueError("k_new and v_new must have the shape of q")
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, ndim=2)
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    _need(query_start, "query_start", torch.int32, dev, ndim=1)
    B = context_lens.shape[0]
    if block_tables.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("block_tables / query_start do not match context_lens")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, dev, ndim=3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must have the shape of q")
    if append and validate.debug_enabled():
        validate.check_prefill_append(block_tables, context_lens, query_start)
    tail = (_ptr(block_tables), block_tables.shape[1], _ptr(context_lens), max_context_len,
            _ptr(query_start), T, B, H, D, BLOCK_TOKENS, NB, float(scale), _ptr(out), flags,
            _stream_handle(dev))
    with torch.cuda.device(dev):
        if append:
            name = "pkv_pa_prefill_append"
            code = lib.pkv_pa_prefill_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                             _ptr(v_pool), *tail)
        else:
            name = "pkv_pa_prefill"
            code = lib.pkv_pa_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), *tail)
    _lib.check(name, code)
    return out


class VirtualKV:
    """A contiguous KV cache in virtual memory with physical chunks mapped
    on demand (pkv_vkv_* of the C ABI): per layer one K and one V buffer of
    [max_batch][max_context][H][D] fp16.  Create it with the target device
    current; ``close()`` (or garbage collection) frees it."""

    def __init__(self, max_batch, max_context, num_layers, num_heads, head_dim,
                 chunk_bytes=2 << 20):
        self._lib = _lib.load_library()
        handle = ctypes.c_void_p()
        _lib.check("pkv_vkv_create", self._lib.pkv_vkv_create(
            max_batch, max_context, num_layers, num_heads, head_dim, chunk_bytes,
            ctypes.byref(handle)))
        self.handle = handle
        self.max_batch, self.max_context = max_batch, max_context
        self.num_layers, self.num_heads, self.head_dim = num_layers, num_heads, head_dim

    def grow(self, seq, tokens):
        _lib.check("pkv_vkv_grow", self._lib.pkv_vkv_grow(self.handle, seq, tokens))

    def release(self, seq):
        _lib.check("pkv_vkv_release", self._lib.pkv_vkv_release(self.handle, seq))

    def buffers(self, layer):
        """(K, V) device addresses of ``layer``'s buffers."""
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _lib.check("pkv_vkv_buffers", self._lib.pkv_vkv_buffers(self.handle, layer,
                                                                ctypes.byref(k), ctypes.byref(v)))
        return k.value, v.value

    def capacity_ptr(self):
        return self._lib.pkv_vkv_capacity(self.handle)

    def stats(self):
        info = _lib.VkvInfo()
        _lib.check("pkv_vkv_stats", self._lib.pkv_vkv_stats(self.handle, ctypes.byref(info)))
        return {name: getattr(info, name) for name, _ in info._fields_}

    def append(self, layer, k, v, seq_ids, positions):
        """Write row t of k / v ([T][H][D] fp16) as token positions[t] of
        request seq_ids[t] (int32 device tensors), on the current stream."""
        _need(k, "k", torch.float16, ndim=3)
        dev = k.device
        _need(v, "v", torch.float16, dev, ndim=3)
        _need(seq_ids, "seq_ids", torch.int32, dev, ndim=1)
        _need(positions, "positions", torch.int32, dev, ndim=1)
        T = k.shape[0]
        if tuple(k.shape) != (T, self.num_heads, self.head_dim) or v.shape != k.shape or \
                seq_ids.shape[0] != T or positions.shape[0] != T:
            raise ValueError("k, v, seq_ids, positions do not match")
        with torch.cuda.device(dev):
            code = self._lib.pkv_vkv_append(self.handle, layer, _ptr(k), _ptr(v), _ptr(seq_ids),
                                            _ptr(positions), T, _stream_handle(dev))
        _lib.check("pkv_vkv_append", code)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self._lib.pkv_vkv_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def contig_decode_workspace_size(batch, num_heads, head_dim, max_context_len):
    return int(_lib.load_library().pkv_contig_decode_workspace_size(
        batch, num_heads, head_dim, max_context_len))


def _contig_call(q, k_addr, v_addr, row_tokens, context_lens, capacity_addr, scale, out,
                 max_context_len, workspace):
    lib = _lib.load_library()
    dev = q.device
    B, H, D = q.shape
    _need(context_lens, "context_lens", torch.int32, dev, ndim=1)
    if context_lens.shape[0] != B:
        raise ValueError("context_lens does not match the batch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, dev, ndim=3)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B][H][D]")
    need = contig_decode_workspace_size(B, H, D, max_context_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    with torch.cuda.device(dev):
        code = lib.pkv_contig_decode(
            _ptr(q), ctypes.c_void_p(k_addr), ctypes.c_void_p(v_addr), row_tokens,
            _ptr(context_lens), ctypes.c_void_p(capacity_addr), max_context_len, B, H, D,
            float(scale), _ptr(out), _ptr(workspace), workspace.numel(), 0, _stream_handle(dev))
    _lib.check("pkv_contig_decode", code)
    return out


def contig_decode(q, vkv, layer, context_lens, scale, out=None, *, max_context_len=None,
                  workspace=None):
    """``pa_decode`` over the contiguous virtual-memory cache ``vkv``
    (a VirtualKV): sequence b reads rows b*max_context .. of ``layer``'s
    buffers, clamped to its mapped tokens."""
    _need(q, "q", torch.float16, ndim=3)
    B, H, D = q.shape
    if B > vkv.max_batch or H != vkv.num_heads or D != vkv.head_dim:
        raise ValueError("q does not match the virtual cache")
    kb, vb = vkv.buffers(layer)
    return _contig_call(q, kb, vb, vkv.max_context, context_lens, vkv.capacity_ptr(), scale, out,
                        max_context_len, workspace)


def contig_decode_rows(q, k_rows, v_rows, row_tokens, context_lens, scale, out=None, *,
                       capacity=None, max_context_len=None, workspace=None):
    """``pa_decode`` over contiguous K/V rows in ordinary tensors
    ([B*row_tokens][H][D] fp16): sequence b's token t is row
    b*row_tokens + t; ``capacity`` (int32 [B], optional) clamps the
    contexts."""
    _need(q, "q", torch.float16, ndim=3)
    dev = q.device
    B, H, D = q.shape
    for name, t in (("k_rows", k_rows), ("v_rows", v_rows)):
        _need(t, name, torch.float16, dev, ndim=3)
        if tuple(t.shape[1:]) != (H, D) or t.shape[0] < B * row_tokens:
            raise ValueError(f"{name} must hold B*row_tokens rows of [H][D]")
    cap = 0
    if capacity is not None:
        _need(capacity, "capacity", torch.int32, dev, ndim=1)
        cap = capacity.data_ptr()
    return _contig_call(q, k_rows.data_ptr(), v_rows.data_ptr(), row_tokens, context_lens, cap,
                        scale, out, max_context_len, workspace)


def kv_append(k, v, slot_mapping, k_pool, v_pool):
    """Write row t of k / v ([T][H][D] fp16) into slot slot_mapping[t]
    (block slot//16, position slot%16) of one layer's pools; negative slots
    are skipped."""
    lib = _lib.load_library()
    _need(k, "k", torch.float16, ndim=3)
    dev = k.device
    _need(v, "v", torch.float16, dev, ndim=3)
    if v.shape != k.shape:
        raise ValueError("k and v differ in shape")
    T, H, D = k.shape
    _need(slot_mapping, "slot_mapping", torch.int32, dev, ndim=1)
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per row")
    NB = _pool_blocks(k_pool, "k_pool", H, D, dev)
    if _pool_blocks(v_pool, "v_pool", H, D, dev) != NB:
        raise ValueError("k_pool and v_pool differ in size")
    if validate.debug_enabled():
        validate.check_slots(slot_mapping, NB)
    with torch.cuda.device(dev):
        code = lib.pkv_kv_append(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_pool),
                                 _ptr(v_pool), NB, H, D, BLOCK_TOKENS, _stream_handle(dev))
    _lib.check("pkv_kv_append", code)


def cow_copy_blocks(src_dst_pairs, k_pools, v_pools):
    """For every (src, dst) row of ``src_dst_pairs`` ([n][2] int32, device)
    copy physical block src over block dst in every layer's K and V pool
    (lists of equally shaped fp16 pools)."""
    lib = _lib.load_library()
    k_pools = list(k_pools)
    v_pools = list(v_pools)
    if not k_pools or len(k_pools) != len(v_pools):
        raise ValueError("need one K and one V pool per layer")
    dev = k_pools[0].device
    _need(src_dst_pairs, "src_dst_pairs", torch.int32, dev, ndim=2)
    if src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [n][2]")
    first = k_pools[0]
    for i, p in enumerate(k_pools + v_pools):
        _need(p, f"pool {i}", torch.float16, dev)
        if p.shape != first.shape:
            raise ValueError("all pools must have the same shape")
    NB = first.shape[0]
    block_bytes = first[0].numel() * first.element_size()
    if validate.debug_enabled():
        validate.check_cow_pairs(src_dst_pairs, NB)
    L = len(k_pools)
    karr = (ctypes.c_void_p * L)(*[p.data_ptr() for p in k_pools])
    varr = (ctypes.c_void_p * L)(*[p.data_ptr() for p in v_pools])
    with torch.cuda.device(dev):
        code = lib.pkv_cow_copy_blocks(karr, varr, L, _ptr(src_dst_pairs),
                                       src_dst_pairs.shape[0], NB, block_bytes,
                                       _stream_handle(dev))
    _lib.check("pkv_cow_copy_blocks", code)


def hbm_read_probe(buf, sink, workgroups=2048):
    """Read the whole of ``buf`` (a device tensor of a multiple of 16 bytes)
    once, linearly, with non-temporal loads (measurement aid; see
    pkv_hbm_read_probe).  ``sink``: a 4-byte-or-larger device tensor."""
    lib = _lib.load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    with torch.cuda.device(buf.device):
        code = lib.pkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                      workgroups, _stream_handle(buf.device))
    _lib.check("pkv_hbm_read_probe", code)


def hbm_copy_probe(src, dst, workgroups=4096):
    """Copy ``src`` to ``dst`` (contiguous device tensors of the same
    multiple of 16 bytes), each workgroup over a contiguous slice
    (measurement aid: the read + write rate; see pkv_hbm_copy_probe)."""
    lib = _lib.load_library()
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or dst.device != src.device:
        raise ValueError("src and dst must have the same size, on one device")
    with torch.cuda.device(src.device):
        code = lib.pkv_hbm_copy_probe(_ptr(src), _ptr(dst), nbytes, workgroups,
                                      _stream_handle(src.device))
    _lib.check("pkv_hbm_copy_probe", code)


def lds_read_probe(cycles, sink, workgroups, waves, rounds, form):
    """Time LDS reads on every CU (measurement aid, see pkv_lds_read_probe):
    ``cycles`` (int64) and ``sink`` (int32) are contiguous device tensors of
    ``workgroups * waves`` entries; form 0 is 16-byte row reads, form 1 the
    prefill's transpose reads."""
    lib = _lib.load_library()
    n = workgroups * waves
    _need(cycles, "cycles", torch.int64, ndim=1)
    _need(sink, "sink", torch.int32, cycles.device, ndim=1)
    if cycles.numel() != n or sink.numel() != n:
        raise ValueError("cycles and sink need workgroups * waves entries")
    with torch.cuda.device(cycles.device):
        code = lib.pkv_lds_read_probe(_ptr(cycles), _ptr(sink), workgroups, waves, rounds, form,
                                      _stream_handle(cycles.device))
    _lib.check("pkv_lds_read_probe", code)


def hbm_gather_probe(buf, order, chunk_bytes, sink, workgroups=512):
    """Read ``buf`` as chunks of ``chunk_bytes`` in the order of ``order``
    (int32 device tensor, one entry per chunk); measurement aid, see
    pkv_hbm_gather_probe."""
    lib = _lib.load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _need(order, "order", torch.int32, buf.device, ndim=1)
    if chunk_bytes <= 0 or nbytes % chunk_bytes or order.numel() != nbytes // chunk_bytes:
        raise ValueError("order must have one entry per chunk of buf")
    with torch.cuda.device(buf.device):
        code = lib.pkv_hbm_gather_probe(_ptr(buf), nbytes, _ptr(order), chunk_bytes, _ptr(sink),
                                        workgroups, _stream_handle(buf.device))
    _lib.check("pkv_hbm_gather_probe", code)
