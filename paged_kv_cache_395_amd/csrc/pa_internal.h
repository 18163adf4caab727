// Host-side declarations shared by the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Record a message for pa_last_error() and return `st`.
pa_status_t fail(pa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

struct DecodeArgs {
  void* out;
  bool out_f32;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int64_t num_blocks;
  float scale_log2;  // scale * log2(e): scores live in the exp2 domain
  int32_t max_context_len;
  int32_t partition;
  int32_t num_partitions;  // ceil(max_context_len / partition)
  int32_t q_len;           // queries per sequence (1: plain decode)
  int32_t tile_shift;      // log2(block_size / 16)
  // workspace (all null when num_partitions <= 1): the call's geometry for
  // the merge's check, the partial-slot count of every (sequence, kv head),
  // and the partial slots
  int32_t* ws_hdr;         // [8]
  int32_t* ws_nseg;        // [S][Hkv]
  float* ws_acc;           // [S][q_len][Hq][num_partitions][D]
  float* ws_m;             // [S][q_len][Hq][num_partitions]
  float* ws_l;             // [S][q_len][Hq][num_partitions]
  pa_dtype_t dtype;
  hipStream_t stream;
};

// fp16 / bf16 decode runs one workgroup per partition while the longest
// context spans at most kPartitionGridMax partitions, and on the persistent
// grid beyond: there, one partial per partition would cost more than the
// per-partition grid's better balance gains.  Measured on one MI355X:
// 16 x 32,768 tokens at 512-token partitions (64 per context): 380 us per
// partition, 333 us persistent; the same at 4096 (8): 329 vs 334; 256
// lognormal GQA contexts at 512 (16): 271 vs 254; 64 MHA contexts
// U[128, 2048] at 512 (4 to 5): 176 vs 182.
constexpr int32_t kPartitionGridMax = 8;
inline bool decode_uses_persistent_grid(int32_t num_partitions) { return num_partitions > kPartitionGridMax; }

// The per-partition grid's items ((kv head, sequence, partition), kv head
// fastest) go to workgroup i = item i, which runs on XCD i % 8: kv head g on
// XCD g % 8, so K/V blocks that several sequences share stay in one XCD's
// L2.  With 16 or more kv heads (from 8 rounds of 192 items on) they are
// dealt in rounds of 192 instead, each XCD 23 of them and the even XCDs 2
// more, since the odd XCDs finish equal work about 8% later (7B MHA decode
// -2.7%); with 8 kv heads that cost the shared-prefix batch 1.6% and the
// serving loops' decode 2.5-5% through the blocks it moved off their XCD,
// so there workgroup i stays item i.  Workgroups whose item is past the
// last exit.
constexpr int64_t kWeightedItemsMin = 8 * 192;
constexpr int32_t kWeightedKvHeadsMin = 16;
constexpr bool partition_grid_weighted(int64_t items, int32_t kv_heads) {
  return items >= kWeightedItemsMin && items < (int64_t(1) << 31) && kv_heads >= kWeightedKvHeadsMin;
}
constexpr int64_t partition_grid_workgroups(int64_t items, int32_t kv_heads) {
  return partition_grid_weighted(items, kv_heads) ? 8 * (25 * ((items - 1) / 192) + 25) : items;
}

// pa_decode with `scratch` (scratch_bytes) as its workspace; PA_EWORKSPACE
// when the sizes need more.
pa_status_t decode_in_scratch(void* scratch, size_t scratch_bytes, void* out, pa_dtype_t out_dtype, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              int32_t max_blocks, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t bs, int64_t NB, float scale, int32_t max_ctx, int32_t partition,
                              pa_dtype_t dtype, void* stream);

hipError_t launch_decode_partitions(const DecodeArgs& a);
hipError_t launch_decode_reduce(const DecodeArgs& a);
// Workgroups of the fp16 / bf16 decode kernel resident at once on the current device.
int64_t decode_resident_workgroups(pa_dtype_t dtype, int32_t head_dim, bool out_f32);

struct PrefillArgs {
  void* out;
  bool out_f32;
  const void* q;
  int32_t chunk;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int64_t num_blocks;
  float scale_log2;
  int32_t max_context_len;
  int32_t tile_shift;  // log2(block_size / 16)
  pa_dtype_t dtype;
  hipStream_t stream;
};

hipError_t launch_prefill_chunk(const PrefillArgs& a);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int64_t num_blocks, int32_t tile_shift, int elem_bytes,
                                    hipStream_t stream);

struct AppendStepArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;
  const int32_t* rows;
  const int32_t* positions;
  int32_t num_tokens;
  int32_t* tables;
  int32_t max_blocks;
  int32_t* ctx;
  const int32_t* new_ctx;
  int32_t num_rows;
  int32_t num_kv_heads, head_dim;
  int64_t num_blocks;
  int32_t tile_shift;  // log2(block_size / 16)
  int elem_bytes;
  hipStream_t stream;
};

hipError_t launch_append_step(const AppendStepArgs& a);

// One launch's share of a step whose metadata travels in the kernel
// arguments (pa_append_step_host): at most kArgTokens tokens and kArgRows
// lengths, about 3 KB of arguments.
constexpr int kArgTokens = 128;
constexpr int kArgRows = 256;
struct AppendArgsMeta {
  int64_t slots[kArgTokens];
  int32_t rows[kArgTokens];
  int32_t positions[kArgTokens];
  int32_t new_ctx[kArgRows];
  int32_t num_tokens;  // tokens of this launch (key / value point at the first)
  int32_t row0;        // first row whose length this launch sets
  int32_t num_rows;    // lengths this launch sets
};
hipError_t launch_append_step_args(const AppendStepArgs& a, const AppendArgsMeta& meta);

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int64_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks,
                              hipStream_t stream);
hipError_t launch_patch_tables(int32_t* tables, int32_t max_blocks, int32_t num_rows, const int32_t* patches,
                               int32_t num_patches, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups, hipStream_t stream);
hipError_t launch_gather_probe(const void* buf, int64_t buf_tiles, const int32_t* tiles, int64_t num_tiles,
                               int32_t tile_bytes, uint32_t* sink, int32_t workgroups, hipStream_t stream);

}  // namespace pa
