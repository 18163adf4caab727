/*
 * pa.h - paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels and a host-side block manager.
 * Every argument is a plain pointer or integer; no C++ or framework type
 * crosses this boundary.
 *
 * Pages cited (by title and section):
 *   [OS]  "PagedAttention: How vLLM Serves AI Like an Operating System"
 *   [VIZ] "vLLM Architecture and PagedAttention - Interactive Visualization"
 *
 * ------------------------------------------------------------------------
 * Memory model
 * ------------------------------------------------------------------------
 * The KV cache is cut into fixed blocks of 16 tokens that can sit anywhere
 * in one pool; a per-sequence block table maps logical block i to a
 * physical block ([OS] "PagedAttention: Virtual Memory for KV Cache", How It
 * Works and the memory-layout example).  block_size is 16, the pages'
 * size; 32 and 64 are supported as variants (every entry point takes
 * block_size, the same for all calls on one pool), anything else is
 * PA_EUNSUPPORTED.  Below, bs = block_size.
 *
 * Pools.  k_cache and v_cache are separate device arrays
 *     [num_blocks][num_kv_heads][bs * head_dim]      (elements of `dtype`)
 * and one (block, kv head) run is bs * head_dim contiguous elements: bs / 16
 * tiles of 16 tokens one after another (tokens 0-15 of the block in the
 * first, 16-31 in the second, ...).  Inside a tile (t = token offset
 * 0..15, d = dim):
 *     K(t, d) at  ((d / 8) * 16 + t) * 8 + d % 8
 *                 i.e. [head_dim/8][16 tokens][8 dims]
 *     V(t, d) at  (((d / 32) * 4 + t / 4) * 16 + d % 16) * 8
 *                   + ((d / 16) % 2) * 4 + t % 4
 *                 i.e. [head_dim/32][4 token quads][16 dims][2 halves][4 tokens]
 * This order lets a 64-lane wave read a tile as whole 1 KiB runs of 16-byte
 * loads that land directly in matrix-core operand registers.  head_dim must
 * be a multiple of 32; the kernels support 64 and 128.
 *
 * Slots.  Token position p of a sequence lives in logical block p / bs at
 * offset p % bs; its slot is  physical_block * bs + p % bs  (int64).  A
 * negative slot means "skip this token".
 *
 * Block tables.  int32 [num_seqs][max_blocks_per_seq], row-major; only the
 * first ceil(context_len / bs) entries of a row are read.  context_lens is
 * int32 [num_seqs] and counts every cached token including the one(s) the
 * step just wrote.
 *
 * Query heads.  q head h reads kv head h / (num_q_heads / num_kv_heads);
 * num_q_heads must be a multiple of num_kv_heads (1 <= group <= 16).
 *
 * ------------------------------------------------------------------------
 * Conventions
 * ------------------------------------------------------------------------
 * Ownership:  every device pointer is allocated and owned by the caller; no
 *   entry point allocates device memory.  Split-context scratch is a
 *   caller-provided workspace sized by pa_decode_workspace_bytes().
 * Streams:    `stream` is a hipStream_t (NULL = the default stream).  Every
 *   device entry point only enqueues work on it and returns; results are
 *   valid once the stream reaches that point.  The host never reads device
 *   memory and never synchronises.
 * Errors:     every entry point validates its scalar arguments before any
 *   launch and returns a status; pa_last_error() gives a message (per
 *   thread).  No C++ exception crosses the ABI.
 * Device-side guards: a table entry outside [0, num_blocks), a context_len
 *   above max_context_len or beyond the table width, or a slot beyond the
 *   pool never causes an out-of-bounds access: the affected output row is
 *   written as NaN (attention) or the token is skipped (cache write).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,       /* argument outside the contract                  */
  PA_EUNSUPPORTED = 2, /* dtype, head_dim, group or block_size not built */
  PA_EWORKSPACE = 3,   /* workspace missing or smaller than required     */
  PA_EHIP = 4,         /* the HIP runtime reported an error              */
  PA_ENOSPC = 5,       /* block manager: not enough free blocks          */
  PA_ENOENT = 6        /* block manager: unknown sequence                */
} pa_status_t;

/* Element types.  The two sentinels give the type the range of int32_t, so
 * any 32-bit value a caller passes is a value of the type and is refused
 * with PA_EUNSUPPORTED rather than being undefined in the C++ library. */
typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PA_DTYPE_RANGE_MAX_ = 2147483647
} pa_dtype_t;

/* Version string of the library build. */
const char* pa_version(void);

/* Message describing the last non-OK status returned on this thread. */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------
 * Cache write.  Stores each new token's K and V rows into its slot, bit for
 * bit, for every kv head: blocks are filled as tokens arrive ([OS] "The
 * Magic: No Pre-allocation"; "PagedAttention: Virtual Memory for KV Cache",
 * How It Works).
 *   key, value      device [num_tokens][num_kv_heads][head_dim] of dtype
 *   k_cache,v_cache device pools (layout above), modified in place
 *   slot_mapping    device int64 [num_tokens]; < 0 skips the token.  Slots in
 *                   one call must be distinct.
 * num_tokens == 0 is a no-op.
 * ---------------------------------------------------------------------- */
pa_status_t pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * One step's appends with the block tables and context lengths resident on
 * the device: the cache write above, plus, for each token,
 *     block_tables[row][pos / bs] = slot / bs
 * (the block the slot lies in: a block opened on demand when pos % bs == 0,
 * the fresh copy after a copy-on-write, the unchanged block otherwise --
 * [OS] "The Magic: No Pre-allocation", "Copy-on-Write: Sharing KV Cache"),
 * and context_lens[r] = new_context_lens[r] for every row r.  A serving step
 * then ships only its tokens' slots, rows and positions and the new lengths
 * (about 1 KB for 64 sequences) instead of whole tables, and the decode that
 * follows reads tables and lengths where this call left them.
 *   key, value        device [num_tokens][num_kv_heads][head_dim] of dtype
 *   slot_mapping      int64 [num_tokens]   (< 0: skip the token)
 *   token_rows        int32 [num_tokens]   row of the token's sequence in
 *                                          block_tables / context_lens
 *   token_positions   int32 [num_tokens]   the token's position in its sequence
 *   new_context_lens  int32 [num_seqs]
 * These four may be device memory or pinned host memory (each value is read
 * once).  block_tables (device int32 [num_seqs][max_blocks_per_seq]) and
 * context_lens (device int32 [num_seqs]) are updated in place.  A token whose
 * row or position falls outside the table is stored but does not touch the
 * table.  Slots in one call must be distinct.
 * ---------------------------------------------------------------------- */
pa_status_t pa_append_step(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, const int32_t* token_rows,
                           const int32_t* token_positions, int32_t num_tokens,
                           int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t* context_lens, const int32_t* new_context_lens, int32_t num_seqs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_append_step with the step's metadata in host memory: slot_mapping,
 * token_rows, token_positions and new_context_lens are ordinary (pageable
 * or pinned) host arrays whose values are copied into the launch's kernel
 * arguments before the call returns, so the caller may overwrite them at
 * once and the kernel reads nothing across the host link.  Every other
 * argument, the result and the error behaviour are those of pa_append_step.
 * One launch carries up to 128 tokens and 256 lengths (about 3 KB of
 * arguments); a larger step is split into several launches on the stream.
 * ---------------------------------------------------------------------- */
pa_status_t pa_append_step_host(const void* key, const void* value, void* k_cache, void* v_cache,
                                const int64_t* slot_mapping, const int32_t* token_rows,
                                const int32_t* token_positions, int32_t num_tokens,
                                int32_t* block_tables, int32_t max_blocks_per_seq,
                                int32_t* context_lens, const int32_t* new_context_lens, int32_t num_seqs,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int64_t num_blocks, pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Copy whole physical blocks (K and V, all kv heads) src -> dst: the copy a
 * shared block gets before a sequence writes into it ([OS] "Copy-on-Write:
 * Sharing KV Cache").
 *   pairs   device int64 [num_pairs][2] = (src, dst); destinations distinct
 *           and never a source of the same call.
 * ---------------------------------------------------------------------- */
pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Move whole blocks (K and V, all kv heads) between two pools of the same
 * geometry: the copy behind preempting a request by moving its blocks to CPU
 * memory and bringing them back ([OS] "vLLM Architecture", the scheduler's
 * third duty).  Block pairs[i][0] of the source pools goes to block
 * pairs[i][1] of the destination pools.  Either side may be pinned host
 * memory (swap out: device -> host; swap in: host -> device); the two sides
 * must be different pools.
 *   pairs   int64 [num_pairs][2] = (src, dst), device or pinned host memory;
 *           destinations distinct.  A pair outside [0, src_blocks) x
 *           [0, dst_blocks) is skipped.
 * ---------------------------------------------------------------------- */
pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k,
                           const void* src_v, int64_t src_blocks, const int64_t* pairs,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Set block_tables[row][idx] = block for each patch (row, idx, block): how a
 * device-resident table follows a request that comes back from CPU memory
 * into new blocks.  patches: int32 [num_patches][3], device or pinned host
 * memory; a patch outside the table is skipped.
 * ---------------------------------------------------------------------- */
pa_status_t pa_patch_tables(int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                            const int32_t* patches, int32_t num_patches, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention over the paged cache: for every sequence s and q head h,
 *     out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 * over the context_lens[s] tokens of s, reading K_s / V_s through the block
 * table ([OS] "PagedAttention: Virtual Memory for KV Cache"; the result is
 * that of contiguous attention, [OS] "Throughput Impact: The Numbers").
 *
 *   out             device [num_seqs][num_q_heads][head_dim] of out_dtype
 *                   (PA_F32, or the input dtype)
 *   q               device [num_seqs][num_q_heads][head_dim] of dtype
 *   max_context_len host upper bound of context_lens (sizes the grid)
 *   partition_size  tokens per context partition, a multiple of 16, or 0
 *                   to let the library choose (pa_decode_partition_size
 *                   reports the choice).  Sequences longer than one
 *                   partition are split; the pieces are merged exactly by
 *                   a log-sum-exp reduction.  At most 65535 partitions
 *                   (ceil(max_context_len / partition)); more give
 *                   PA_EUNSUPPORTED.
 *   workspace       device scratch of at least
 *                   pa_decode_workspace_bytes(...) bytes (may be NULL when
 *                   that is 0); its contents are private to the call.
 * A sequence with context_len 0 gets a zero row.  dtype PA_F32 runs on the
 * vector ALUs; PA_F16 / PA_BF16 use the matrix cores with fp32
 * accumulation and an fp32 softmax.
 * ---------------------------------------------------------------------- */
/* Effective partition size for these sizes (partition_size 0 = the
 * library's choice: 512 tokens where the longest context spans more than 8
 * partitions of 512 and the (sequence, kv head) pairs are fewer than 4096,
 * which runs the persistent grid; otherwise 512 to 4096 tokens, as large as
 * keeps >= 1024 workgroups, small enough that the longest context spans >= 4
 * partitions once the pairs alone reach 1024, and 4096 once they reach
 * 4096); -1 for invalid arguments.  pa_decode_noalloc takes the second rule
 * where the first one's partials would not fit its array. */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t partition_size);

/* How decode's partition launch is shaped for these sizes on the current
 * device, and its workgroup count (*workgroups, may be NULL):
 *   PA_DECODE_GRID_VECTOR      fp32: one workgroup per (query head,
 *                              partition), vector ALUs
 *   PA_DECODE_GRID_PARTITIONS  fp16 / bf16 whose longest context spans at
 *                              most 8 partitions: one workgroup per (kv head,
 *                              sequence, partition); with 16 or more kv heads
 *                              and enough of them, dealt unevenly over the
 *                              XCDs, plus up to ~5% that exit at once
 *   PA_DECODE_GRID_PERSISTENT  fp16 / bf16 beyond: as many workgroups as are
 *                              resident at once (occupancy x CUs, at most one
 *                              per partition); each takes a share of the
 *                              batch's tiles (each pair weighed by its tiles
 *                              plus a fixed start-up cost; with one query per
 *                              sequence the odd XCDs' workgroups take 23/25
 *                              of an even one's), whole partitions only, a
 *                              boundary that would split off only a few tiles
 *                              of a pair moved to the pair's edge, and folds
 *                              the partitions of one (sequence, kv head) it
 *                              holds in registers, so the merge reads about
 *                              one partial per workgroup instead of one per
 *                              partition.
 * -1 for invalid arguments.  Results are the same whichever shape runs
 * (within the stated tolerances; each shape is deterministic). */
enum { PA_DECODE_GRID_VECTOR = 0, PA_DECODE_GRID_PARTITIONS = 1, PA_DECODE_GRID_PERSISTENT = 2 };
int32_t pa_decode_launch_shape(pa_dtype_t dtype, int32_t head_dim, pa_dtype_t out_dtype, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                               int32_t partition_size, int64_t* workgroups);

/* Workspace bytes pa_decode needs for these sizes (0: none). */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size);

pa_status_t pa_decode(void* out, pa_dtype_t out_dtype, const void* q,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                      float scale, int32_t max_context_len, int32_t partition_size,
                      void* workspace, size_t workspace_bytes,
                      pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, contract and results as pa_decode, without the workspace: the
 * split-context partials go to a device array of
 * pa_decode_noalloc_scratch_bytes() (64 MiB) that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine); sizes whose
 * workspace (pa_decode_workspace_bytes) exceeds the array give
 * PA_EWORKSPACE.  All calls on one GPU share that GPU's array: calls that
 * overlap on one GPU (on different streams) race and must not be issued.
 * The first call on a device also looks the array's address up
 * (hipGetSymbolAddress); a failure there gives PA_EHIP.
 * ---------------------------------------------------------------------- */
size_t pa_decode_noalloc_scratch_bytes(void);

pa_status_t pa_decode_noalloc(void* out, pa_dtype_t out_dtype, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              float scale, int32_t max_context_len, int32_t partition_size,
                              pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Several queries per sequence: the last q_len positions of each context
 * (ctx - q_len .. ctx - 1, their K/V already written), each attending
 * causally to keys 0 .. its own position -- e.g. verifying q_len drafted
 * tokens in one step.  This is the chunked-prefill computation
 * (pa_prefill_chunk) for a chunk small enough that all q_len x group
 * (query, head) pairs of a kv head fit the 16 matrix-core columns decode
 * already pads to, so it runs at decode's bandwidth:
 *   q    device [num_seqs][q_len][num_q_heads][head_dim] of dtype
 *   out  device [num_seqs][q_len][num_q_heads][head_dim] of out_dtype
 * Requires q_len * (num_q_heads / num_kv_heads) <= 16 and fp16 / bf16
 * (PA_EUNSUPPORTED otherwise), context_lens[s] >= q_len (else NaN rows).
 * q_len 1 is pa_decode.  Other arguments as pa_decode; the workspace is
 * sized by pa_decode_multi_workspace_bytes.
 * ---------------------------------------------------------------------- */
size_t pa_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                       int32_t partition_size);

pa_status_t pa_decode_multi(void* out, pa_dtype_t out_dtype, const void* q, int32_t q_len,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int64_t num_blocks,
                            float scale, int32_t max_context_len, int32_t partition_size,
                            void* workspace, size_t workspace_bytes,
                            pa_dtype_t dtype, void* stream);

/* The two launches pa_decode makes, for callers that time or schedule them
 * separately.  pa_decode_partitions writes finished rows of single-partition
 * sequences to `out` and partial results of the others to `workspace`;
 * pa_decode_reduce then merges those partials into `out`.  Same arguments
 * and contract as pa_decode. */
pa_status_t pa_decode_partitions(void* out, pa_dtype_t out_dtype, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, int32_t max_context_len, int32_t partition_size,
                                 void* workspace, size_t workspace_bytes,
                                 pa_dtype_t dtype, void* stream);

pa_status_t pa_decode_reduce(void* out, pa_dtype_t out_dtype, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                             const void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill: causal attention of a chunk of chunk_len new queries per
 * sequence over the paged cache ([OS] "PagedAttention: Virtual Memory for
 * KV Cache": a request's tokens live in fixed-size blocks that its block
 * table maps from logical to physical position; a chunk of new tokens is
 * stored into such blocks and attends through the same table).  The chunk
 * occupies the last chunk_len
 * positions of the context (its K/V already written by
 * pa_reshape_and_cache); query i of sequence s sits at position
 * context_lens[s] - chunk_len + i and attends keys 0 .. that position.
 *   out  device [num_seqs][chunk_len][num_q_heads][head_dim] of out_dtype
 *   q    device [num_seqs][chunk_len][num_q_heads][head_dim] of dtype
 * Requires context_lens[s] >= chunk_len (else that sequence's rows are NaN).
 * dtype PA_F16 / PA_BF16 only (matrix cores, fp32 accumulation).  A chunk
 * whose rows (chunk_len x query group) or workgroup count would exceed the
 * device's int counters gives PA_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
pa_status_t pa_prefill_chunk(void* out, pa_dtype_t out_dtype, const void* q, int32_t chunk_len,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float scale, int32_t max_context_len,
                             pa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Measurement probe: reads `bytes` of device memory once with the load
 * style decode uses (16-byte non-temporal buffer loads) and discards the
 * data (a 4-byte write to *sink happens only for one improbable XOR of the
 * input).  Timing it gives the HBM read ceiling against which decode's
 * achieved bandwidth is set.  buf must be 16-byte aligned; `workgroups`
 * sizes the grid (each reads 16 KiB per round).
 * ---------------------------------------------------------------------- */
pa_status_t pa_probe_read_bandwidth(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Measurement probe for the access pattern of paged decode: reads the
 * tiles tiles[0 .. num_tiles) of tile_bytes bytes each (tile i is
 * buf + i * tile_bytes; a multiple of 1024 up to 64 KiB) with the same
 * 16-byte non-temporal loads, wave by wave with two tiles in flight, and
 * discards the data like pa_probe_read_bandwidth.  A random permutation of
 * the tiles of a large buffer gives the ceiling of a gather of scattered
 * blocks.  tiles: int32, device memory; an index outside
 * [0, buf_bytes / tile_bytes) is skipped without a memory access.  buf must
 * be 16-byte aligned; `workgroups` (4 waves each) sizes the grid.
 * ---------------------------------------------------------------------- */
pa_status_t pa_probe_gather_bandwidth(const void* buf, int64_t buf_bytes, const int32_t* tiles, int64_t num_tiles,
                                      int32_t tile_bytes, uint32_t* sink, int32_t workgroups, void* stream);

/* ------------------------------------------------------------------------
 * Host block manager.  One pool of num_blocks blocks of block_size (16, 32
 * or 64) tokens; per sequence a list of physical blocks; a free list;
 * reference counts for shared blocks.
 *   - allocation on demand: a token at offset 0 of a fresh block takes a
 *     new block, so n tokens hold ceil(n/bs) blocks and waste at most bs - 1
 *     slots ([OS] "The Magic: No Pre-allocation");
 *   - release on finish ([VIZ] "Page Table Visualization");
 *   - sharing by fork (parallel sampling) and by a common prefix (system
 *     prompt), with copy-on-write before a write into a shared block
 *     ([OS] "Copy-on-Write: Sharing KV Cache").
 * The free list is a queue: allocation takes its head, a block whose count
 * drops to zero joins its tail.  Its initial order is `free_order` (a
 * permutation of 0..num_blocks-1), or ascending when NULL.
 * Every update is all-or-nothing: PA_ENOSPC leaves the state unchanged,
 * which is the point where a scheduler would preempt.  All pointers here
 * are host pointers.  A pa_bm_t is not thread-safe.
 * ---------------------------------------------------------------------- */
typedef struct pa_bm pa_bm_t;

pa_bm_t* pa_bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order);
void pa_bm_destroy(pa_bm_t* bm);

/* New sequence holding num_tokens (>= 0) tokens in fresh blocks. */
pa_status_t pa_bm_add_seq(pa_bm_t* bm, int64_t seq, int32_t num_tokens);

/* New sequence sharing the first prefix_tokens (a multiple of bs, within the
 * prefix sequence) of prefix_seq, plus tail_tokens in fresh blocks. */
pa_status_t pa_bm_add_seq_with_prefix(pa_bm_t* bm, int64_t seq, int64_t prefix_seq,
                                      int32_t prefix_tokens, int32_t tail_tokens);

/* child shares every block of parent (reference counts + 1). */
pa_status_t pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t child);

/* Drop the sequence; blocks whose count reaches 0 return to the free list
 * in logical order. */
pa_status_t pa_bm_free_seq(pa_bm_t* bm, int64_t seq);

/* Append one token to each of seqs[0..n) in order (a sequence may repeat).
 * slots[i] receives the slot of token i.  When a token lands in a shared
 * block, the writer first moves to a fresh copy: the pair (old, new) is
 * appended to cow_pairs ([n][2], may be NULL only if no copy occurs) and
 * *num_cow counts them; the device copy (pa_copy_blocks) must run before
 * the cache write. */
pa_status_t pa_bm_append_tokens(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                                int64_t* cow_pairs, int32_t* num_cow);

/* Fill table [n][max_blocks] (padding with pad_id) and context_lens [n]. */
pa_status_t pa_bm_block_table(const pa_bm_t* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                              int32_t pad_id, int32_t* table, int32_t* context_lens);

int64_t pa_bm_num_free(const pa_bm_t* bm);
int32_t pa_bm_refcount(const pa_bm_t* bm, int64_t block);          /* -1: out of range  */
double pa_bm_usage(const pa_bm_t* bm);                              /* used / num_blocks */
int32_t pa_bm_num_tokens(const pa_bm_t* bm, int64_t seq);           /* -1: unknown       */
/* Copy the free list, head first, into out[0..cap); returns its length. */
int64_t pa_bm_free_list(const pa_bm_t* bm, int32_t* out, int64_t cap);

/* ------------------------------------------------------------------------
 * Automatic prefix caching ([OS] "Copy-on-Write: Sharing KV Cache", Prefix
 * Caching; [NL] item 5, Prefix Caching): requests that start with the same
 * tokens share the blocks of that prefix without naming each other.
 * Turn it on once, before the first sequence.  pa_bm_add_seq_tokens adds a
 * sequence from its token ids: each full block is identified by its whole
 * prefix (a hash of the previous block's identity and its own bs ids,
 * confirmed against the stored ids); the leading run of blocks that are
 * already cached is shared (count + 1), the rest are fresh, and fresh full
 * blocks become cached.  *cached_tokens (a multiple of bs) tells the caller
 * how many leading tokens are already in the cache: only tokens from there
 * on need their K/V computed and written.  A cached block whose count drops
 * to zero is not freed but kept, least recently released first in line for
 * eviction; it can still be claimed by a later match, and allocation takes
 * it (dropping its identity) only when the free queue is empty.
 * pa_bm_num_free counts free plus evictable blocks; pa_bm_num_cached_free
 * the evictable ones.  With caching on, pa_bm_free_seq releases a sequence's
 * blocks deepest first, so a prefix is evicted from its end.  A new block
 * whose prefix identity is already held by an evictable block takes the
 * identity over; the old block goes to the free queue.
 * ---------------------------------------------------------------------- */
pa_status_t pa_bm_enable_prefix_cache(pa_bm_t* bm);
pa_status_t pa_bm_add_seq_tokens(pa_bm_t* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                                 int32_t* cached_tokens);
int64_t pa_bm_num_cached_free(const pa_bm_t* bm);

/* ------------------------------------------------------------------------
 * Swap pool.  A second pool of num_host_blocks blocks in CPU memory, with its
 * own ids, free queue (ascending at first) and reference counts, to which a
 * preempted request's blocks move ([OS] "vLLM Architecture").  Set once.
 *
 * pa_bm_swap_out moves every block of seqs[0..n) to the host pool: one host
 * block per distinct device block of the list (a block shared inside the
 * list moves once and stays shared; a block also held by a sequence outside
 * the list stays on the device for it, and the listed ones get a copy).
 * pairs ([Σ blocks][2], (device, host)) receives the copies the device must
 * make, in order; *num_pairs counts them.  Device blocks whose count drops to
 * zero join the free queue.  A swapped-out sequence keeps its length; it
 * cannot be appended to, forked, shared as a prefix or put in a block table
 * until pa_bm_swap_in brings it back, into fresh device blocks (pairs =
 * (host, device)).  Both are all-or-nothing (PA_ENOSPC when the target pool
 * is short).  pa_bm_free_seq works in either residence.
 * ---------------------------------------------------------------------- */
pa_status_t pa_bm_set_host_pool(pa_bm_t* bm, int64_t num_host_blocks);
pa_status_t pa_bm_swap_out(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t* num_pairs);
pa_status_t pa_bm_swap_in(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t* num_pairs);
int32_t pa_bm_is_swapped(const pa_bm_t* bm, int64_t seq);       /* 1 / 0; -1: unknown  */
int64_t pa_bm_num_free_host(const pa_bm_t* bm);
int32_t pa_bm_host_refcount(const pa_bm_t* bm, int64_t block);  /* -1: out of range   */

/* ------------------------------------------------------------------------
 * Continuous-batching step scheduler over a block manager ([OS] "Continuous
 * Batching: The Other Half" and "vLLM Architecture"; [VIZ] "Continuous
 * Batching").  Requests arrive with a prompt length and a final length; each
 * step decides which requests run in which of max_rows batch rows and emits
 * the host-side half of the step:
 *   1. requests that reached their final length are freed (their rows and
 *      blocks come back at once);
 *   2. the blocks every running request's next token needs are reserved;
 *      while they do not fit, the latest-arrived running request is
 *      preempted: swapped out to the host pool, or, when the host pool
 *      cannot hold it, freed and requeued with prompt = its tokens so far;
 *   3. swapped-out requests come back, earliest arrival first, while a row
 *      and their blocks (plus the reserve) are free; not one preempted in
 *      this step;
 *   4. only when nothing is swapped out, waiting requests are admitted,
 *      earliest arrival first, while a row and their prompt's blocks are
 *      free and the step's token count stays within max_batched_tokens (the
 *      first admission of a step is always allowed; the count includes
 *      prompt tokens found in the prefix cache); an admitted request's
 *      prompt tokens are written this step;
 *   5. every request running before the admissions appends one token.
 * Priority is arrival (submit) order; a request keeps its row while it runs;
 * a new or returning one takes the lowest free row.  The scheduler owns the
 * sequences it creates (ids are the request ids); do not change them through
 * the block manager while it runs.
 *
 * The device half of a step, in this order on one stream: swap out
 * (pa_swap_blocks device -> host), swap in (host -> device), copy-on-write
 * (pa_copy_blocks), table patches (pa_patch_tables), then pa_append_step with
 * slots / token_rows / token_positions / context_lens, then decode over the
 * max_rows rows (an empty row has length 0 and gives a zero row).  The swap
 * out may instead run on another stream as soon as the previous step's
 * pa_append_step is done, provided the rest of the step waits for it.
 * The arrays in pa_sched_out_t belong to the scheduler and stay valid until
 * its next step or destruction.
 * pa_sched_step returns PA_ENOENT, changing nothing, when a request it runs
 * or holds swapped out is no longer in the block manager; after any other
 * error status the scheduler's state is unspecified (destroy it).
 * ---------------------------------------------------------------------- */
typedef struct pa_sched pa_sched_t;

typedef struct {
  int32_t num_tokens;             /* K/V rows to write this step               */
  const int64_t* slots;           /* [num_tokens]                              */
  const int32_t* token_rows;      /* [num_tokens]                              */
  const int32_t* token_positions; /* [num_tokens]                              */
  int32_t num_rows;               /* = max_rows                                */
  const int32_t* context_lens;    /* [num_rows], 0 for an empty row            */
  const int64_t* row_seq;         /* [num_rows], request id or -1              */
  int32_t num_swap_out;
  const int64_t* swap_out_pairs;  /* [num_swap_out][2] (device, host)          */
  int32_t num_swap_in;
  const int64_t* swap_in_pairs;   /* [num_swap_in][2] (host, device)           */
  int32_t num_cow;
  const int64_t* cow_pairs;       /* [num_cow][2] (src, dst) device blocks     */
  int32_t num_patches;
  const int32_t* table_patches;   /* [num_patches][3] (row, logical, physical): swapped-in
                                     requests, and cached prefix blocks of admitted ones */
  int32_t num_finished;
  const int64_t* finished;        /* requests retired at the start of the step */
  int32_t num_admitted, num_swapped_in, num_preempted_swap, num_preempted_recompute;
  int32_t num_running, num_waiting, num_swapped;
  int32_t num_cached_tokens;      /* admitted prompt tokens found in the prefix cache (not written) */
} pa_sched_out_t;

pa_sched_t* pa_sched_create(pa_bm_t* bm, int32_t max_rows, int32_t max_blocks_per_seq,
                            int32_t max_batched_tokens);
void pa_sched_destroy(pa_sched_t* s);
/* seq >= 0; 1 <= prompt_tokens <= total_tokens; the request must fit the
 * pool and the table width on its own. */
pa_status_t pa_sched_submit(pa_sched_t* s, int64_t seq, int32_t prompt_tokens, int32_t total_tokens);
/* The same with the prompt's token ids (prompt_ids[prompt_tokens], copied),
 * for a block manager with prefix caching on: admission then shares the
 * cached blocks of the prompt's longest cached prefix (pa_bm_add_seq_tokens),
 * counts only the blocks it takes (fresh, or claimed back from the evictable
 * list), lists only the prompt tokens after the cached ones for writing, and
 * lists the cached blocks' table entries as patches (no token write sets
 * them).
 * A request preempted for recompute comes back by count, without its ids. */
pa_status_t pa_sched_submit_tokens(pa_sched_t* s, int64_t seq, const int32_t* prompt_ids,
                                   int32_t prompt_tokens, int32_t total_tokens);
pa_status_t pa_sched_step(pa_sched_t* s, pa_sched_out_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
