"""PagedAttention decode on MI355X (gfx950).

Single-query attention over a KV cache cut into 16-token blocks scattered
across a physical block pool and reached through per-sequence block tables,
plus the two paging helpers: slot-mapped append and block copy-on-write.
The compute runs in hand-written HIP kernels behind the C ABI of
``libpagedkv.so`` (include/pagedkv.h); ``ops`` marshals torch tensors to it,
``blocks`` is the host-side block manager that produces tables, slots and
copy pairs.
"""

from ._lib import LIB_PATH, LibraryMissing, PagedKVError, load_library  # noqa: F401
from .blocks import (PAGE_TOKENS, PagedRequest, PagePool, PoolExhausted,  # noqa: F401
                     decode_groups, device_arrays, kv_bytes_per_token, tables_share_blocks)
from .ops import (VirtualKV, contig_decode, contig_decode_rows,  # noqa: F401
                  contig_decode_workspace_size,
                  cow_copy_blocks, default_partition,
                  kv_append, pa_decode, pa_decode_append, pa_decode_append_noalloc,
                  pa_decode_grouped, pa_decode_grouped_workspace_size, pa_decode_workspace_size,
                  pa_prefill, pa_prefill_append, pool_shape)
from .validate import ContractError, debug_enabled, set_debug  # noqa: F401
