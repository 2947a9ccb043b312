/*
 * pagedkv — single-query attention over a block-paged KV cache on MI355X
 * (gfx950), plus the two paging helpers it needs: slot-mapped append of new
 * tokens and block-granular copy-on-write.
 *
 * C ABI: plain pointers and sizes.  Every pointer named "device" must point
 * to memory on the current HIP device; "host" pointers are read before the
 * call returns.  Every entry point is asynchronous on the given stream
 * (a hipStream_t passed as void*, NULL for the null stream): it performs no
 * device allocation and no host/device synchronisation, and the caller owns
 * every buffer and keeps it alive until the stream has passed the call.
 *
 * All argument checks run on the host before any HIP call, so a bad call
 * returns its status code and touches neither the device nor the stream.
 * Device-side contract violations (a block id outside [0, num_blocks), a
 * context_lens entry above max_context_len) are not reported: the kernels
 * clamp or skip them so that no access leaves the buffers (a context is
 * clamped to max_context_len), and the results for the affected rows are
 * unspecified.  A block id outside the pool is clamped for reading only:
 * every call that writes the pools (the appends, fused or not, and the
 * copy-on-write) writes nothing for it, so no other sequence's block is
 * touched.
 *
 * Sources: "PagedAttention" (e-fortepiano.pl, Catalan encyclopedia
 * article), sections "Descripció" and "Formulació matemàtica"; "Atención
 * paginada en modelos de lenguaje grandes (LLM)" (7minutos.es), the
 * PagePool / PagedRequest part and the prefix-sharing (copy-on-write) part.
 *
 * Layouts (all row-major, fp16 = IEEE binary16):
 *   q, out          [B][H][D]
 *   k_pool, v_pool  [num_blocks][H][D/8][16][8]: one physical block holds
 *                   16 tokens for every head; inside the tile of one
 *                   (block, head) the head dimension is split into D/8
 *                   groups of 8 consecutive values and each group stores its
 *                   8 values for token 0, token 1, ..., token 15 in turn.
 *                   Value d of head h for the token at position p of block n
 *                   is element ((n*H + h)*(D/8) + d/8)*128 + p*8 + d%8.
 *   block_tables    [B][max_blocks_per_seq] int32: logical block j of
 *                   sequence b lives in physical block block_tables[b][j];
 *                   entries past the sequence's last block are ignored.
 *   context_lens    [B] int32: tokens of sequence b that its query attends
 *                   to (positions 0 .. context_lens[b]-1, the query's own
 *                   token included once it has been appended).
 *   slot_mapping    [T] int32: slot = physical_block*16 + position; a
 *                   negative slot skips that row.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL_PTR = 1,            /* a required pointer is NULL */
  PKV_ERR_BAD_SHAPE = 2,           /* negative or zero size where one is needed,
                                      D not 64/128, table narrower than the context */
  PKV_ERR_MISALIGNED = 3,          /* a data pointer is not 16-byte aligned
                                      (int32 arrays: 4-byte) */
  PKV_ERR_UNSUPPORTED = 4,         /* block_size other than 16 */
  PKV_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below the required size */
  PKV_ERR_HIP = 6,                 /* the HIP runtime reported a launch error */
  PKV_ERR_SCRATCH_TOO_SMALL = 7    /* the shape needs more than the library's fixed
                                      scratch buffer (PKV_NOALLOC_SCRATCH_BYTES) */
};

/* Tokens per physical block ("Atención paginada ...", 7minutos.es,
 * PagePool part: pages of 16 tokens). */
#define PKV_BLOCK_TOKENS 16

/*
 * Bytes of device workspace pkv_pa_decode needs for this shape.  Pure host
 * function; max_context_len is the largest entry of context_lens the caller
 * will pass.  Returns 0 for invalid sizes (and for the partitioned strategy
 * when every sequence fits in one partition).  The workspace holds
 * intermediate results only: its contents need no initialisation and are
 * not meaningful after the call.
 */
size_t pkv_pa_decode_workspace_size(int32_t B, int32_t H, int32_t D,
                                    int32_t max_context_len);

/*
 * PagedAttention decode ("PagedAttention", e-fortepiano.pl, "Formulació
 * matemàtica" and "Descripció"): for every sequence b and head h,
 *
 *   out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) * V_t,
 *
 * over t = 0 .. context_lens[b]-1, where K_t / V_t are read from physical
 * block block_tables[b][t/16] at position t%16 of k_pool / v_pool.  The
 * result is computed block by block in fp32 with an online softmax and
 * rounded to fp16 (round to nearest even); a sequence with context 0 gets a
 * zero row.  By default the blocks of all sequences are lined up and cut
 * into equal ranges, one per resident workgroup; a sequence cut by a range
 * boundary leaves partial results that are merged in ascending position
 * order (with pkv_pa_decode_ex and a partition length, each sequence is cut
 * into fixed partitions instead).  The arithmetic order depends only on the
 * logical positions and the context lengths of the batch, so moving blocks
 * to other physical ids or sharing them between sequences does not change
 * any output bit.  K/V tiles are streamed with a non-temporal cache policy
 * (see PKV_DECODE_KEEP_KV_CACHED).
 *
 * device: q, k_pool, v_pool, out (16-byte aligned), block_tables,
 *         context_lens, workspace (256-byte aligned, may be NULL when the
 *         required size is 0).
 * host:   sizes, scale; max_context_len >= every context_lens[b] chooses the
 *         partitioning; block_size must be 16; max_blocks_per_seq*16 must be
 *         >= max_context_len.
 */
int pkv_pa_decode(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t max_context_len,
                  int32_t B, int32_t H, int32_t D, int32_t block_size,
                  int32_t num_blocks, float scale, void* out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Flags of pkv_pa_decode_ex. */
#define PKV_DECODE_KEEP_KV_CACHED 1u  /* load K/V tiles with the normal cache
                                         policy instead of streaming them
                                         (non-temporal): for batches whose
                                         tables share physical blocks (a
                                         shared prompt, forks), so that
                                         repeated blocks are found in L2.
                                         Results are identical either way. */

/*
 * pkv_pa_decode with an explicit partition length in tokens (a positive
 * multiple of 16, at most 512), or 0 for the default choice, and flags
 * (0 or PKV_DECODE_KEEP_KV_CACHED; other bits are rejected with
 * PKV_ERR_BAD_SHAPE).  The workspace size for it is
 * pkv_pa_decode_workspace_size_ex with the same partition value.
 */
int pkv_pa_decode_ex(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len,
                     int32_t B, int32_t H, int32_t D, int32_t block_size,
                     int32_t num_blocks, float scale, void* out,
                     void* workspace, size_t workspace_bytes,
                     int32_t partition_tokens, uint32_t flags, void* stream);

/*
 * One decode step with its append fused in: for every sequence b with
 * context_lens[b] >= 1, the keys and values of its new token, k_new[b] and
 * v_new[b] ([B][H][D] fp16), are written to its last position,
 * t = context_lens[b] - 1 (block block_tables[b][t/16], slot t%16 of
 * k_pool / v_pool), and the decode of pkv_pa_decode over positions
 * 0 .. t follows, the new token included ("PagedAttention",
 * e-fortepiano.pl, "Descripció": the key and value of each generated token
 * go to the sequence's last block before the next attention step).  The
 * pools and the output are those of pkv_kv_append with slot
 * block_tables[b][t/16] * 16 + t%16 for each b, then pkv_pa_decode, bit for
 * bit.  The decode kernel takes the new token into the tile it holds in
 * registers where the sequence's last block is read, and the merge kernel
 * of the same call writes it to the pools, so the append costs no launch of
 * its own and no wait inside the decode's load stream.
 *
 * device: q, k_new, v_new, k_pool, v_pool (written), out (16-byte aligned),
 *         block_tables, context_lens, workspace (as for pkv_pa_decode, size
 *         pkv_pa_decode_workspace_size).  The last block of each sequence
 *         must not be shared with another sequence of the batch (a shared
 *         block is copied before it is written, see pkv_cow_copy_blocks).
 * host:   as for pkv_pa_decode; flags 0 or PKV_DECODE_KEEP_KV_CACHED.
 *         Always the flat strategy: a shape it cannot stage returns
 *         PKV_ERR_UNSUPPORTED (use pkv_kv_append + pkv_pa_decode_ex then).
 */
int pkv_pa_decode_append(const void* q, const void* k_new, const void* v_new,
                         void* k_pool, void* v_pool, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t max_context_len, int32_t B, int32_t H, int32_t D,
                         int32_t block_size, int32_t num_blocks, float scale,
                         void* out, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream);

/*
 * pkv_pa_decode_append for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels, pools and
 * output as pkv_pa_decode_append (bit for bit), minus the workspace: the
 * partial results live in a fixed device array of the library,
 * PKV_NOALLOC_SCRATCH_BYTES bytes on every GPU it runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a device looks up that device's copy of
 * the array, with the device current.
 *
 * Limit: shapes whose pkv_pa_decode_workspace_size exceeds
 * PKV_NOALLOC_SCRATCH_BYTES return PKV_ERR_SCRATCH_TOO_SMALL before any HIP
 * call (4 MiB holds every shape the fused call accepts up to H = 2048: the
 * flat plan needs about 2 MiB of partials at D = 128 plus 4 (B + 1) bytes).
 * The array's contents are left from the previous call and need no
 * clearing (every partial is written before it is read).  All calls on one
 * GPU share the one array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give unspecified results; calls ordered on one stream are safe.
 *
 * Errors as for pkv_pa_decode_append, plus PKV_ERR_SCRATCH_TOO_SMALL, and
 * PKV_ERR_HIP when the array's device address cannot be looked up.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int pkv_pa_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t B, int32_t H, int32_t D,
                                 int32_t block_size, int32_t num_blocks, float scale,
                                 void* out, uint32_t flags, void* stream);

size_t pkv_pa_decode_workspace_size_ex(int32_t B, int32_t H, int32_t D,
                                       int32_t max_context_len,
                                       int32_t partition_tokens);

/* Partition length in tokens that pkv_pa_decode uses for this shape, or 0
 * when it uses the default range strategy (every batch whose sequence
 * offsets and range block ids fit the workgroup's LDS budget). */
int32_t pkv_pa_decode_default_partition(int32_t B, int32_t H, int32_t D,
                                        int32_t max_context_len);

/*
 * Slot-mapped append of new tokens into one layer's pools ("Atención
 * paginada ...", 7minutos.es, PagePool / PagedRequest part: each generated
 * token is stored in the page its block table names).  For every row t
 * with slot_mapping[t] >= 0, k[t] and v[t] ([H][D] fp16 each) are copied
 * bit for bit into position slot%16 of block slot/16.  Rows with a
 * negative slot or a block >= num_blocks are skipped.  Two rows with the
 * same slot are a caller error (which one lands is unspecified).
 *
 * device: k, v ([T][H][D], 16-byte aligned), slot_mapping, k_pool, v_pool.
 */
int pkv_kv_append(const void* k, const void* v, const int32_t* slot_mapping,
                  int32_t T, void* k_pool, void* v_pool, int32_t num_blocks,
                  int32_t H, int32_t D, int32_t block_size, void* stream);

/*
 * Block-granular copy-on-write ("Atención paginada ...", 7minutos.es,
 * prefix-sharing part; "PagedAttention", e-fortepiano.pl, "Descripció"):
 * for every pair (src, dst) in src_dst_pairs and every layer l, the whole
 * physical block dst of k_pools[l] and of v_pools[l] becomes a bit copy of
 * block src.  Reference counts live with the caller.  Pairs must be
 * conflict-free (no dst repeated, no dst that is also a src); pairs with an
 * id outside [0, num_blocks) are skipped.
 *
 * host:   k_pools, v_pools: arrays of num_layers device pointers (16-byte
 *         aligned), read before the call returns.
 * device: src_dst_pairs [n_pairs][2] int32.
 * block_bytes: bytes of one block of one pool (H*16*D*2 for fp16), a
 *         positive multiple of 16.
 */
int pkv_cow_copy_blocks(void* const* k_pools, void* const* v_pools,
                        int32_t num_layers, const int32_t* src_dst_pairs,
                        int32_t n_pairs, int32_t num_blocks, int64_t block_bytes,
                        void* stream);

/*
 * Decode for groups of sequences that share leading blocks: the branches of
 * parallel sampling or beam search, requests forked from one prompt
 * ("PagedAttention", e-fortepiano.pl, "Descripció": physical blocks shared
 * between requests and decoding branches through the block tables; "Atención
 * paginada ...", 7minutos.es, prefix-sharing part: a fork shares its owner's
 * pages, and a page is copied before a holder writes into it, so the pages
 * still shared are full pages at the front of the tables).
 *
 * Every output row is the single-query decode of pkv_pa_decode for that
 * sequence (same formula, fp32 arithmetic, fp16 output); a shared block is
 * read once for all members of its group, and the score and value products
 * of a tile run on the matrix cores for all members at once (probabilities
 * enter the value product rounded to fp16, so results match pkv_pa_decode
 * to rounding, not bit for bit).
 *
 * Grouping (device int32 arrays, read as follows):
 *   group g, 0 <= g < num_groups, holds the consecutive sequences
 *   [group_offsets[g], group_offsets[g+1]) (offsets clamped into [0, B],
 *   non-decreasing; a group with a negative size is empty); only its first
 *   group_size members are decoded;
 *   the group's first group_shared_blocks[g] logical blocks, clamped into
 *   [0, min over its decoded members of context_lens/16], are read through
 *   the table row of its first member for every member (so they must be the
 *   same physical blocks, or blocks holding the same data, in every
 *   member's table).
 * Sequences in no group, members past group_size and sequences with
 * context 0 get zero rows.  Overlapping groups are a caller error (rows
 * unspecified, no access out of bounds).
 *
 * device: q, k_pool, v_pool, out (16-byte aligned), block_tables,
 *         context_lens, group_offsets (num_groups + 1 entries),
 *         group_shared_blocks (num_groups entries), workspace (256-byte
 *         aligned, at least pkv_pa_decode_grouped_workspace_size bytes).
 * host:   num_groups >= 0, with B + num_groups at most 11259 (the context
 *         lengths and group offsets are staged in on-chip memory);
 *         1 <= group_size <= 16; the
 *         other sizes, block_size, max_context_len and flags as for
 *         pkv_pa_decode_ex (PKV_DECODE_KEEP_KV_CACHED is accepted; shared
 *         blocks are read once either way).
 * The workspace holds intermediate results only (no initialisation needed).
 */
int pkv_pa_decode_grouped(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len,
                          const int32_t* group_offsets, const int32_t* group_shared_blocks,
                          int32_t num_groups, int32_t group_size,
                          int32_t B, int32_t H, int32_t D, int32_t block_size,
                          int32_t num_blocks, float scale, void* out,
                          void* workspace, size_t workspace_bytes, uint32_t flags,
                          void* stream);

/* Workspace bytes for pkv_pa_decode_grouped (0 for invalid sizes or B = 0). */
size_t pkv_pa_decode_grouped_workspace_size(int32_t B, int32_t H, int32_t D,
                                            int32_t max_context_len, int32_t num_groups,
                                            int32_t group_size);

/*
 * Paged prefill ("PagedAttention", e-fortepiano.pl, "Formulació
 * matemàtica": causal self-attention over the paged cache, block by block):
 * the last n_b = query_start[b+1] - query_start[b] tokens of every sequence
 * b (its prompt, or a chunk of it, already written to its pages, e.g. with
 * pkv_kv_append) are queries.  Query row r = query_start[b] + i sits at
 * position p = context_lens[b] - n_b + i and
 *
 *   out[r][h] = sum_{t <= p} softmax_t(scale * q[r][h] . K_t) * V_t,
 *
 * with K_t / V_t read through block_tables[b] as for pkv_pa_decode (fp32
 * arithmetic on the matrix cores; online softmax whose reference maximum is
 * raised only when a score exceeds it by more than 8 (log2 units), so the
 * fp16 weights stay below 256; the running sum adds the rounded weights;
 * fp16 output with round to nearest even).  Rows at a negative position
 * (n_b > context_lens[b]) are zero rows.  Any finite scale, of either sign.
 *
 * device: q and out [num_query_rows][H][D] fp16 (16-byte aligned), k_pool,
 *         v_pool, block_tables, context_lens, query_start (B + 1 entries,
 *         non-decreasing, query_start[B] <= num_query_rows; rows outside
 *         [0, num_query_rows) are skipped).
 * host:   sizes, scale, max_context_len (>= every context_lens[b]; contexts
 *         are clamped to it), block_size 16, flags 0 or
 *         PKV_PREFILL_HEADS_PER_ITEM(k).  The block ids of one sequence are
 *         staged in LDS after a table of B + 1 entries, from an even entry
 *         and with one spare: (E + ceil(max_context_len / 16) + 1) * 4 bytes,
 *         E = B + 1 rounded up to even, must not exceed 32 KiB.  No
 *         workspace.
 *
 * Work decomposition: a workgroup takes 128 query rows of one sequence for
 * k heads at a time (k = 1, 2, 4 or 8), and streams the sequence's blocks
 * once per head, straight from one head into the next.  By default k is
 * chosen from the sizes (the largest that keeps about four such items per
 * resident workgroup); PKV_PREFILL_HEADS_PER_ITEM(k) fixes it.  The outputs
 * are the same bit for bit for every k.
 */
#define PKV_PREFILL_HEADS_PER_ITEM(k)                                            \
  ((k) == 1 ? 1u << 8 : (k) == 2 ? 2u << 8 : (k) == 4 ? 3u << 8 : (k) == 8 ? 4u << 8 : 0xffu << 8)

int pkv_pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t max_context_len,
                   const int32_t* query_start, int32_t num_query_rows,
                   int32_t B, int32_t H, int32_t D, int32_t block_size,
                   int32_t num_blocks, float scale, void* out, uint32_t flags,
                   void* stream);

/*
 * Prefill with its append fused in ("Atención paginada en modelos de
 * lenguaje grandes (LLM)", 7minutos.es, PagePool / PagedRequest part: a
 * request's tokens are written into its pages slot by slot as they are
 * processed; "PagedAttention", e-fortepiano.pl, "Formulació matemàtica"):
 * the same result as pkv_kv_append of the new rows followed by
 * pkv_pa_prefill, in one call.  Row r = query_start[b] + i of k_new / v_new
 * is the key / value of position p = context_lens[b] - n_b + i of sequence b
 * (context_lens counts the new tokens); it is written to slot
 * block_tables[b][p / 16] * 16 + p % 16 of both pools (rows at a negative
 * position are not written), and the queries attend as for pkv_pa_prefill.
 * Blocks whose tokens are all new are read from k_new / v_new rather than
 * from the pools; the new tokens of a block that also holds cached tokens
 * are written by a first, small kernel, so any split of a sequence into
 * chunks is allowed.  Pools and out equal those of the two separate calls
 * bit for bit, provided no block that receives new tokens of one sequence
 * appears in another sequence's table in the same call: the other sequence
 * would read that block from the pools while it is being written (a
 * prompt prefix shared by several sequences is written by one call and
 * shared afterwards, or copied first, see pkv_cow_copy_blocks).
 *
 * device: k_new, v_new [num_query_rows][H][D] fp16 (16-byte aligned), the
 *         rest as for pkv_pa_prefill; k_pool and v_pool are written.
 * host:   as for pkv_pa_prefill.  query_start must stay within
 *         [0, num_query_rows]; otherwise the new tokens' slots and the
 *         outputs are unspecified (no memory outside the buffers passed is
 *         touched).  Errors as for pkv_pa_prefill, and PKV_ERR_NULL_PTR /
 *         PKV_ERR_MISALIGNED for k_new and v_new.
 */
int pkv_pa_prefill_append(const void* q, const void* k_new, const void* v_new,
                          void* k_pool, void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, const int32_t* query_start,
                          int32_t num_query_rows, int32_t B, int32_t H, int32_t D,
                          int32_t block_size, int32_t num_blocks, float scale, void* out,
                          uint32_t flags, void* stream);

/*
 * Contiguous KV cache in virtual memory, physical memory on demand: the
 * alternative to paging that "PagedAttention" (e-fortepiano.pl) describes in
 * "Limitacions i alternatives" and "Atenció" (vAttention).  Each layer's K
 * and V cache is one contiguous virtual buffer [max_batch][max_context][H][D]
 * fp16 (request b owns rows b*max_context .. +max_context-1), reserved up
 * front; physical memory is mapped into a request's part of every buffer,
 * chunk_bytes at a time, as it grows.  Built on the HIP virtual memory API
 * of the current device.  Calls are synchronous on the host and not
 * thread-safe.
 *
 * pkv_vkv_create: max_context a multiple of 16; D 64 or 128; chunk_bytes a
 *   multiple of the device's mapping granularity that divides
 *   max_context*H*D*2.  Reserves 2*num_layers buffers; maps nothing.
 * pkv_vkv_grow: maps chunks until request `seq` can hold `tokens` tokens
 *   (rounded up to 16) in every layer.  Chunks of released requests are
 *   reused before new physical memory is created.  Never shrinks.
 * pkv_vkv_release: waits for the device, then unmaps all of `seq`'s chunks
 *   (kept for reuse) and sets its readable tokens to 0.
 * pkv_vkv_destroy: waits for the device, unmaps and frees everything.
 * pkv_vkv_buffers: the K and V virtual buffers of `layer` (device
 *   pointers; only rows below a request's readable tokens are mapped).
 * pkv_vkv_capacity: device int32 [max_batch], each request's readable
 *   tokens (its mapped rows, a multiple of 16, at most max_context); pass it
 *   to pkv_contig_decode so that no unmapped row is ever read.
 * pkv_vkv_append: asynchronously on `stream`, writes row t of k / v
 *   ([T][H][D] fp16, device) as token positions[t] of request seq_ids[t]
 *   in `layer` (device int32 arrays); rows outside a request's readable
 *   tokens or with an invalid request are skipped.
 * pkv_vkv_stats: physical bytes mapped (all buffers), bytes pooled for
 *   reuse, bytes reserved, the chunk size, the granularity, map calls,
 *   chunks created and host seconds spent mapping.
 */
typedef struct pkv_vkv pkv_vkv;

typedef struct pkv_vkv_info {
  uint64_t mapped_bytes;
  uint64_t pooled_bytes;
  uint64_t reserved_bytes;
  uint64_t chunk_bytes;
  uint64_t granularity;
  uint64_t map_calls;
  uint64_t chunks_created;
  double map_seconds;
} pkv_vkv_info;

int pkv_vkv_create(int32_t max_batch, int32_t max_context, int32_t num_layers, int32_t H,
                   int32_t D, size_t chunk_bytes, pkv_vkv** out);
int pkv_vkv_destroy(pkv_vkv* vkv);
int pkv_vkv_grow(pkv_vkv* vkv, int32_t seq, int32_t tokens);
int pkv_vkv_release(pkv_vkv* vkv, int32_t seq);
int pkv_vkv_buffers(const pkv_vkv* vkv, int32_t layer, void** k_buf, void** v_buf);
const int32_t* pkv_vkv_capacity(const pkv_vkv* vkv);
int pkv_vkv_append(const pkv_vkv* vkv, int32_t layer, const void* k, const void* v,
                   const int32_t* seq_ids, const int32_t* positions, int32_t T, void* stream);
int pkv_vkv_stats(const pkv_vkv* vkv, pkv_vkv_info* info);

/*
 * Decode over a contiguous KV cache ("PagedAttention", e-fortepiano.pl,
 * "Atenció": the standard attention, unchanged, on contiguous K and V):
 * out[b][h] as for pkv_pa_decode, with token t of sequence b read from row
 * b*row_tokens + t of k_buf / v_buf ([rows][H][D] fp16, device).  The same
 * flat-strategy kernel as pkv_pa_decode, addressing rows instead of table
 * entries.  `capacity` (device int32 [B], may be NULL): tokens each
 * sequence may read; contexts are clamped to it (pkv_vkv_capacity).
 * row_tokens: a multiple of 16, >= max_context_len.  flags must be 0.  The
 * workspace (256-byte aligned) is pkv_contig_decode_workspace_size bytes.
 * Returns PKV_ERR_UNSUPPORTED for batches too large for the flat strategy.
 */
int pkv_contig_decode(const void* q, const void* k_buf, const void* v_buf, int32_t row_tokens,
                      const int32_t* context_lens, const int32_t* capacity,
                      int32_t max_context_len, int32_t B, int32_t H, int32_t D, float scale,
                      void* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                      void* stream);
size_t pkv_contig_decode_workspace_size(int32_t B, int32_t H, int32_t D,
                                        int32_t max_context_len);

/*
 * Measurement aids, not part of the decode path.  Each reads `bytes` (a
 * multiple of 16) of device memory `buf` with 16-byte non-temporal loads
 * from `workgroups` workgroups of 256 threads, asynchronously on `stream`,
 * and stores nothing in practice (`sink`, 4 device bytes, is written only
 * for a data pattern that does not occur).  Their timings are the HBM read
 * rates plain reads reach on this GPU, the references for the decode
 * kernel's block reads.
 *
 * pkv_hbm_read_probe: one linear pass over the buffer.
 *
 * pkv_hbm_gather_probe: the buffer as `bytes / chunk_bytes` chunks
 * (`chunk_bytes` a power of two from 1 KiB to 1 MiB dividing `bytes`), read
 * whole in the order of `chunk_order` (device int32, one entry per chunk;
 * entries are clamped into range), 16 KiB in flight per wave.  A random
 * permutation of 4 KiB chunks is the access pattern of 16-token blocks of
 * one 128-dim head scattered over a pool.
 *
 * pkv_hbm_copy_probe: copies `bytes` (a multiple of 16) from `src` to `dst`
 * (device, 16-byte aligned, not overlapping), each of the `workgroups`
 * workgroups over a contiguous slice, 16-byte non-temporal loads: as many
 * bytes written as read, the read/write mix of a step that reads its inputs
 * once and writes as much back (the prefill with its append fused in).
 */
int pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, int32_t workgroups,
                       void* stream);
int pkv_hbm_gather_probe(const void* buf, size_t bytes, const int32_t* chunk_order,
                         int32_t chunk_bytes, void* sink, int32_t workgroups, void* stream);
int pkv_hbm_copy_probe(const void* src, void* dst, size_t bytes, int32_t workgroups,
                       void* stream);

/*
 * pkv_lds_read_probe: the rate at which a CU reads its LDS, with the read
 * forms of the prefill's pair loop ("PagedAttention", e-fortepiano.pl,
 * "Formulació matemàtica": the block-by-block products read every K and V
 * tile from LDS once per 32 query rows).  `workgroups` workgroups of `waves`
 * waves (1..16), one per CU (each holds 96 KiB of LDS), fill 64 KiB of LDS
 * and then read it `rounds` times per wave, conflict-free: form 0 as 16-byte
 * reads of whole 1 KiB rows (16 KiB per wave and round), form 1 as the
 * 8-byte transpose reads of the value products (ds_read_b64_tr_b16 at the
 * prefill's swizzled offsets, 8 KiB per wave and round).  Each wave w writes
 * its shader-clock cycles over the reads to cycles[w] (device, 8-byte
 * aligned, workgroups * waves entries) and a fold of the data it read to
 * sink[w] (device, 4-byte aligned, as many entries).  Asynchronous on
 * `stream`.  Errors: PKV_ERR_BAD_SHAPE (sizes or form out of range),
 * PKV_ERR_NULL_PTR, PKV_ERR_MISALIGNED, PKV_ERR_HIP.
 */
int pkv_lds_read_probe(uint64_t* cycles, uint32_t* sink, int32_t workgroups, int32_t waves,
                       int32_t rounds, int32_t form, void* stream);

/* Static description of a status code. */
const char* pkv_status_string(int code);

/* Library ABI version (increments when a signature changes). */
int32_t pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
