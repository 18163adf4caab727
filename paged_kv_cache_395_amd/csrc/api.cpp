// C ABI of the paged-attention library: argument validation, workspace
// sizing and kernel dispatch.  Nothing here touches device memory contents or
// synchronises; every device entry point only enqueues work on `stream`.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cstring>
#include <string>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;

int elem_bytes(pa_dtype_t t) { return t == PA_F32 ? 4 : 2; }
bool known_dtype(pa_dtype_t t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr float kLog2e = 1.4426950408889634f;

pa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// log2 of 16-token tiles per block for the supported block sizes, else -1.
int32_t tile_shift_of(int32_t block_size) {
  return block_size == 16 ? 0 : block_size == 32 ? 1 : block_size == 64 ? 2 : -1;
}

pa_status_t check_pool(int32_t kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype_t dtype) {
  if (!known_dtype(dtype)) return fail(PA_EUNSUPPORTED, "unknown dtype %d", int(dtype));
  if (tile_shift_of(block_size) < 0)
    return fail(PA_EUNSUPPORTED, "block_size must be 16, 32 or 64 (got %d)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (kv_heads <= 0) return fail(PA_EINVAL, "num_kv_heads must be positive (got %d)", kv_heads);
  if (num_blocks <= 0) return fail(PA_EINVAL, "num_blocks must be positive");
  return PA_OK;
}

// Tokens per context partition when the caller passes 0.  A partition is
// the work of one workgroup; sequences longer than one partition leave fp32
// partials (accumulator, max, sum) that a second kernel merges.  Writing
// those partials costs far more decode time than their share of the bytes
// (HBM writes interleaved with the read stream), so partitions are made as
// large as the grid allows: starting from 512 tokens they double, up to
// 4096, while the grid still holds >= kMinWorkgroups workgroups (4 per CU)
// and, once the (sequence, kv head) pairs alone fill the GPU, while the
// longest context still spans at least 4 partitions (larger ones only
// unbalance ragged batches).  With >= kManyPairs pairs (16 per CU) the
// pairs balance the GPU on their own and partitions go straight to 4096:
// on 1,024 sequences x 8 kv heads of up to ~1,200 tokens that drops the
// split and the merge launch (+10% per step), while at 2,048 pairs the
// 4-partition rule stays the better choice.
constexpr int32_t kMinPartition = 512;
constexpr int32_t kMaxDefaultPartition = 4096;
constexpr int64_t kMinWorkgroups = 1024;
constexpr int64_t kManyPairs = 4096;

// The rule above, for the per-partition grid.
int32_t spread_partition(int64_t S, int64_t Hkv, int64_t max_ctx) {
  const int64_t pairs = S * Hkv;
  int32_t p = kMinPartition;
  while (p < kMaxDefaultPartition) {
    const int64_t next = 2 * int64_t(p);
    if (pairs * ceil_div(max_ctx, next) < kMinWorkgroups) break;
    if (pairs >= kMinWorkgroups && pairs < kManyPairs && ceil_div(max_ctx, next) < 4) break;
    p = int32_t(next);
  }
  return p;
}

// Where the longest context spans more than kPartitionGridMax partitions of
// kMinPartition tokens (and the pairs do not balance the GPU alone), decode
// runs on the persistent grid, whose shares balance better the finer the
// partitions they are cut at, while its partials stay about one per
// workgroup whatever the partition size; there the partition stays at
// kMinPartition (the fewest tokens that keep the partition count within
// 65535).  Measured on one MI355X against the rule above: 256 lognormal GQA
// contexts 74.4% vs 73.3% of 8 TB/s (P 512 persistent vs 2048 per
// partition), 16 x 32,768 tokens 81.1% vs 80.5% (512 vs 4096, both
// persistent); 1,024 shared-prefix contexts of up to 4,096 tokens stay on
// the rule above (4096 per partition: 80.4%, 512 per partition: 75.1%).
int32_t choose_partition(int64_t S, int64_t Hkv, int64_t max_ctx, int32_t requested) {
  if (requested != 0) return requested;
  if (S * Hkv < kManyPairs && ceil_div(max_ctx, kMinPartition) > kPartitionGridMax) {
    const int64_t least = (ceil_div(max_ctx, 65535) + 15) / 16 * 16;
    return int32_t(least > kMinPartition ? least : kMinPartition);
  }
  return spread_partition(S, Hkv, max_ctx);
}

struct DecodeCheck {
  int32_t partition;
  int32_t nparts;
};

pa_status_t check_decode(const void* out, pa_dtype_t out_dtype, const void* q, int32_t q_len, const void* k,
                         const void* v, const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t S,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int64_t NB, float scale, int32_t max_ctx,
                         int32_t partition, pa_dtype_t dtype, DecodeCheck* dc) {
  pa_status_t st = check_pool(Hkv, D, bs, NB, dtype);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_EINVAL, "num_seqs must be >= 0");
  if (Hq <= 0 || Hq % Hkv != 0) return fail(PA_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(PA_EUNSUPPORTED, "query group %d > 16", Hq / Hkv);
  if (q_len < 1) return fail(PA_EINVAL, "q_len must be >= 1");
  if (q_len > 1 && dtype == PA_F32) return fail(PA_EUNSUPPORTED, "several queries per sequence need fp16 or bf16");
  if (q_len > 1 && (Hq / Hkv) * q_len > 16)
    return fail(PA_EUNSUPPORTED, "q_len %d x query group %d > 16: use pa_prefill_chunk", q_len, Hq / Hkv);
  if (int64_t(S) * q_len > 65535) return fail(PA_EUNSUPPORTED, "num_seqs x q_len must be <= 65535");
  if (!(out_dtype == PA_F32 || out_dtype == dtype))
    return fail(PA_EUNSUPPORTED, "out_dtype must be PA_F32 or the input dtype");
  if (max_ctx < 0) return fail(PA_EINVAL, "max_context_len must be >= 0");
  if (max_blocks < 0 || int64_t(max_blocks) * bs < max_ctx)
    return fail(PA_EINVAL, "max_blocks_per_seq (%d) cannot hold max_context_len (%d)", max_blocks, max_ctx);
  if (!isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (partition < 0 || partition % 16 != 0) return fail(PA_EINVAL, "partition_size must be 0 or a positive multiple of 16");
  partition = choose_partition(S, Hkv, max_ctx, partition);
  if (S > 0 && (!out || !q || !k || !v || !tables || !ctx)) return fail(PA_EINVAL, "null pointer argument");
  const int64_t nparts = max_ctx == 0 ? 1 : ceil_div(max_ctx, partition);
  // partitions index the third grid dimension of the mfma path (at most 65535)
  if (nparts > 65535) return fail(PA_EUNSUPPORTED, "%lld partitions > 65535: use a larger partition_size", (long long)nparts);
  if (S > 65535 || Hq > 65535) return fail(PA_EUNSUPPORTED, "num_seqs and num_q_heads must be <= 65535");
  dc->partition = partition;
  dc->nparts = int32_t(nparts);
  return PA_OK;
}

// Workspace of a split decode (none without a split): a 256-byte header (the
// call's geometry, checked by the merge), the partial-slot count of every
// (sequence, kv head), then the partials acc [rows][D], m [rows], l [rows]
// with rows = S * q_len * Hq * nparts; 256-byte aligned pieces.
int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

size_t ws_size(int64_t S, int64_t q_len, int64_t Hq, int64_t Hkv, int64_t D, int64_t nparts) {
  if (nparts <= 1) return 0;
  const int64_t rows = S * q_len * Hq * nparts;
  return size_t(256 + align256(S * Hkv * 4) + align256(rows * D * 4) + 2 * align256(rows * 4));
}

void split_workspace(void* ws, int64_t S, int64_t q_len, int64_t Hq, int64_t Hkv, int64_t D, int64_t nparts,
                     DecodeArgs* a) {
  const int64_t rows = S * q_len * Hq * nparts;
  char* p = static_cast<char*>(ws);
  a->ws_hdr = reinterpret_cast<int32_t*>(p);
  p += 256;
  a->ws_nseg = reinterpret_cast<int32_t*>(p);
  p += align256(S * Hkv * 4);
  a->ws_acc = reinterpret_cast<float*>(p);
  p += align256(rows * D * 4);
  a->ws_m = reinterpret_cast<float*>(p);
  p += align256(rows * 4);
  a->ws_l = reinterpret_cast<float*>(p);
}

enum class DecodePhase { kBoth, kPartitions, kReduce };

pa_status_t run_decode(DecodePhase phase, void* out, pa_dtype_t out_dtype, const void* q, int32_t q_len,
                       const void* k_cache, const void* v_cache, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                       int64_t NB, float scale, int32_t max_ctx, int32_t partition, void* workspace,
                       size_t workspace_bytes_given, pa_dtype_t dtype, void* stream) {
  DecodeCheck dc{};
  pa_status_t st = check_decode(out, out_dtype, q, q_len, k_cache, v_cache, block_tables, max_blocks, context_lens,
                                S, Hq, Hkv, D, bs, NB, scale, max_ctx, partition, dtype, &dc);
  if (st != PA_OK) return st;
  const size_t need = ws_size(S, q_len, Hq, Hkv, D, dc.nparts);
  if (need > 0 && (workspace == nullptr || workspace_bytes_given < need))
    return fail(PA_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes_given);
  if (S == 0) return PA_OK;
  DecodeArgs a{};
  a.out = out;
  a.out_f32 = out_dtype == PA_F32;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.context_lens = context_lens;
  a.num_seqs = S;
  a.num_q_heads = Hq;
  a.num_kv_heads = Hkv;
  a.head_dim = D;
  a.num_blocks = NB;
  a.scale_log2 = scale * kLog2e;
  a.max_context_len = max_ctx;
  a.partition = dc.partition;
  a.num_partitions = dc.nparts;
  a.q_len = q_len;
  a.tile_shift = tile_shift_of(bs);
  if (need > 0) split_workspace(workspace, S, q_len, Hq, Hkv, D, dc.nparts, &a);
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  if (phase != DecodePhase::kReduce) {
    st = hip_status(launch_decode_partitions(a), "decode partition launch");
    if (st != PA_OK) return st;
  }
  if (phase != DecodePhase::kPartitions) st = hip_status(launch_decode_reduce(a), "decode reduce launch");
  return st;
}

}  // namespace

pa_status_t decode_in_scratch(void* scratch, size_t scratch_bytes, void* out, pa_dtype_t out_dtype, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              int32_t max_blocks, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t bs, int64_t NB, float scale, int32_t max_ctx, int32_t partition,
                              pa_dtype_t dtype, void* stream) {
  DecodeCheck dc{};
  pa_status_t st = check_decode(out, out_dtype, q, 1, k_cache, v_cache, block_tables, max_blocks, context_lens, S, Hq,
                                Hkv, D, bs, NB, scale, max_ctx, partition, dtype, &dc);
  if (st != PA_OK) return st;
  size_t need = ws_size(S, 1, Hq, Hkv, D, dc.nparts);
  if (need > scratch_bytes && partition == 0) {
    // the library's choice does not fit the array: take the per-partition
    // grid's larger partitions (fewer partial slots), as pa_decode chose
    // before the persistent grid's finer default
    partition = spread_partition(S, Hkv, max_ctx);
    need = ws_size(S, 1, Hq, Hkv, D, max_ctx == 0 ? 1 : ceil_div(max_ctx, partition));
  }
  if (need > scratch_bytes)
    return fail(PA_EWORKSPACE,
                "these sizes need %zu bytes of split-context scratch; the allocation-free decode holds %zu "
                "(use pa_decode with a workspace, or a larger partition_size)",
                need, scratch_bytes);
  return run_decode(DecodePhase::kBoth, out, out_dtype, q, 1, k_cache, v_cache, block_tables, max_blocks,
                    context_lens, S, Hq, Hkv, D, bs, NB, scale, max_ctx, partition, scratch, scratch_bytes, dtype,
                    stream);
}

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_version(void) { return "pa 0.1 gfx950"; }

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status_t pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype_t dtype,
                                 void* stream) {
  pa_status_t st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_EINVAL, "num_tokens must be >= 0");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return fail(PA_EINVAL, "null pointer argument");
  return hip_status(launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                             head_dim, num_blocks, tile_shift_of(block_size), elem_bytes(dtype),
                                             static_cast<hipStream_t>(stream)),
                    "reshape_and_cache launch");
}

namespace {

// Checks the arguments of a step's appends and fills the launch arguments
// (shared by the device-metadata and kernel-argument variants).
pa_status_t prepare_append(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, const int32_t* token_rows, const int32_t* token_positions,
                           int32_t num_tokens, int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t* context_lens, const int32_t* new_context_lens, int32_t num_seqs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           pa_dtype_t dtype, void* stream, AppendStepArgs* a) {
  pa_status_t st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_seqs < 0) return fail(PA_EINVAL, "num_tokens and num_seqs must be >= 0");
  if (max_blocks_per_seq <= 0) return fail(PA_EINVAL, "max_blocks_per_seq must be positive");
  if (num_tokens > 0 && (!key || !value || !k_cache || !v_cache || !slot_mapping || !token_rows || !token_positions ||
                         !block_tables))
    return fail(PA_EINVAL, "null pointer argument");
  if (num_seqs > 0 && (!context_lens || !new_context_lens)) return fail(PA_EINVAL, "null pointer argument");
  // grid: one column of workgroups per token, then one workgroup per 128 lengths
  if (int64_t(num_tokens) + (int64_t(num_seqs) + 127) / 128 > INT32_MAX) return fail(PA_EUNSUPPORTED, "grid too large");
  a->key = key;
  a->value = value;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->slots = slot_mapping;
  a->rows = token_rows;
  a->positions = token_positions;
  a->num_tokens = num_tokens;
  a->tables = block_tables;
  a->max_blocks = max_blocks_per_seq;
  a->ctx = context_lens;
  a->new_ctx = new_context_lens;
  a->num_rows = num_seqs;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->num_blocks = num_blocks;
  a->tile_shift = tile_shift_of(block_size);
  a->elem_bytes = elem_bytes(dtype);
  a->stream = static_cast<hipStream_t>(stream);
  return PA_OK;
}

}  // namespace

pa_status_t pa_append_step(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, const int32_t* token_rows, const int32_t* token_positions,
                           int32_t num_tokens, int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t* context_lens, const int32_t* new_context_lens, int32_t num_seqs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           pa_dtype_t dtype, void* stream) {
  AppendStepArgs a{};
  const pa_status_t st = prepare_append(key, value, k_cache, v_cache, slot_mapping, token_rows, token_positions,
                                        num_tokens, block_tables, max_blocks_per_seq, context_lens, new_context_lens,
                                        num_seqs, num_kv_heads, head_dim, block_size, num_blocks, dtype, stream, &a);
  if (st != PA_OK) return st;
  return hip_status(launch_append_step(a), "append_step launch");
}

pa_status_t pa_append_step_host(const void* key, const void* value, void* k_cache, void* v_cache,
                                const int64_t* slot_mapping, const int32_t* token_rows,
                                const int32_t* token_positions, int32_t num_tokens, int32_t* block_tables,
                                int32_t max_blocks_per_seq, int32_t* context_lens,
                                const int32_t* new_context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype_t dtype,
                                void* stream) {
  AppendStepArgs a{};
  const pa_status_t st = prepare_append(key, value, k_cache, v_cache, slot_mapping, token_rows, token_positions,
                                        num_tokens, block_tables, max_blocks_per_seq, context_lens, new_context_lens,
                                        num_seqs, num_kv_heads, head_dim, block_size, num_blocks, dtype, stream, &a);
  if (st != PA_OK) return st;
  // launch i carries tokens [i * kArgTokens, ...) and lengths [i * kArgRows, ...)
  const int64_t launches = std::max(ceil_div(num_tokens, kArgTokens), ceil_div(num_seqs, kArgRows));
  const int64_t token_bytes = int64_t(num_kv_heads) * head_dim * a.elem_bytes;
  for (int64_t i = 0; i < launches; ++i) {
    AppendArgsMeta m{};
    const int64_t t0 = i * kArgTokens, r0 = i * kArgRows;
    m.num_tokens = int32_t(std::min<int64_t>(std::max<int64_t>(num_tokens - t0, 0), kArgTokens));
    m.num_rows = int32_t(std::min<int64_t>(std::max<int64_t>(num_seqs - r0, 0), kArgRows));
    m.row0 = m.num_rows > 0 ? int32_t(r0) : 0;
    if (m.num_tokens > 0) {
      std::memcpy(m.slots, slot_mapping + t0, sizeof(int64_t) * m.num_tokens);
      std::memcpy(m.rows, token_rows + t0, sizeof(int32_t) * m.num_tokens);
      std::memcpy(m.positions, token_positions + t0, sizeof(int32_t) * m.num_tokens);
    }
    if (m.num_rows > 0) std::memcpy(m.new_ctx, new_context_lens + r0, sizeof(int32_t) * m.num_rows);
    AppendStepArgs ai = a;
    ai.key = static_cast<const char*>(key) + (m.num_tokens > 0 ? t0 * token_bytes : 0);
    ai.value = static_cast<const char*>(value) + (m.num_tokens > 0 ? t0 * token_bytes : 0);
    const pa_status_t sl = hip_status(launch_append_step_args(ai, m), "append_step_host launch");
    if (sl != PA_OK) return sl;
  }
  return PA_OK;
}

pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           pa_dtype_t dtype, void* stream) {
  pa_status_t st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_EINVAL, "num_pairs must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return fail(PA_EINVAL, "null pointer argument");
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return hip_status(launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, pairs, num_pairs, block_bytes, num_blocks,
                                       num_blocks, static_cast<hipStream_t>(stream)),
                    "copy_blocks launch");
}

pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k, const void* src_v,
                           int64_t src_blocks, const int64_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, pa_dtype_t dtype, void* stream) {
  pa_status_t st = check_pool(num_kv_heads, head_dim, block_size, dst_blocks, dtype);
  if (st != PA_OK) return st;
  if (src_blocks <= 0) return fail(PA_EINVAL, "src_blocks must be positive");
  if (num_pairs < 0) return fail(PA_EINVAL, "num_pairs must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return fail(PA_EINVAL, "null pointer argument");
  if (src_k == dst_k || src_v == dst_v) return fail(PA_EINVAL, "source and destination pools must differ");
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return hip_status(launch_copy_blocks(dst_k, dst_v, src_k, src_v, pairs, num_pairs, block_bytes, src_blocks,
                                       dst_blocks, static_cast<hipStream_t>(stream)),
                    "swap_blocks launch");
}

pa_status_t pa_patch_tables(int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                            const int32_t* patches, int32_t num_patches, void* stream) {
  if (num_patches < 0 || num_seqs < 0 || max_blocks_per_seq <= 0) return fail(PA_EINVAL, "bad sizes");
  if (num_patches == 0) return PA_OK;
  if (!block_tables || !patches) return fail(PA_EINVAL, "null pointer argument");
  return hip_status(launch_patch_tables(block_tables, max_blocks_per_seq, num_seqs, patches, num_patches,
                                        static_cast<hipStream_t>(stream)),
                    "patch_tables launch");
}

int32_t pa_decode_launch_shape(pa_dtype_t dtype, int32_t head_dim, pa_dtype_t out_dtype, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                               int32_t partition_size, int64_t* workgroups) {
  if (!known_dtype(dtype) || (head_dim != 64 && head_dim != 128) || num_seqs < 0 || num_kv_heads <= 0 ||
      num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_context_len < 0 || partition_size < 0 ||
      partition_size % 16 != 0)
    return -1;
  if (!(out_dtype == PA_F32 || out_dtype == dtype)) return -1;
  const int32_t p = choose_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  const int64_t nparts = max_context_len == 0 ? 1 : ceil_div(max_context_len, p);
  int64_t n = 0;
  int32_t shape = PA_DECODE_GRID_PARTITIONS;
  if (dtype == PA_F32) {
    shape = PA_DECODE_GRID_VECTOR;
    n = int64_t(num_seqs) * num_q_heads * nparts;  // one workgroup per (query head, partition)
  } else if (decode_uses_persistent_grid(int32_t(nparts))) {
    shape = PA_DECODE_GRID_PERSISTENT;
    n = std::max<int64_t>(1, std::min(decode_resident_workgroups(dtype, head_dim, out_dtype == PA_F32),
                                      int64_t(num_seqs) * num_kv_heads * nparts));
  } else {
    n = partition_grid_workgroups(int64_t(num_seqs) * num_kv_heads * nparts, num_kv_heads);
  }
  if (workgroups) *workgroups = n;
  return shape;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t partition_size) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 || partition_size < 0 || partition_size % 16 != 0)
    return -1;
  return choose_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  if (partition_size < 0 || partition_size % 16 != 0) return 0;
  const int32_t p = choose_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  return ws_size(num_seqs, 1, num_q_heads, num_kv_heads, head_dim, ceil_div(max_context_len, p));
}

size_t pa_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 0)
    return 0;
  if (partition_size < 0 || partition_size % 16 != 0) return 0;
  const int32_t p = choose_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  return ws_size(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, ceil_div(max_context_len, p));
}

pa_status_t pa_decode_multi(void* out, pa_dtype_t out_dtype, const void* q, int32_t q_len, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                            int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
                            pa_dtype_t dtype, void* stream) {
  return run_decode(DecodePhase::kBoth, out, out_dtype, q, q_len, k_cache, v_cache, block_tables, max_blocks_per_seq,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                    max_context_len, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status_t pa_decode(void* out, pa_dtype_t out_dtype, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, float scale, int32_t max_context_len,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype_t dtype,
                      void* stream) {
  return run_decode(DecodePhase::kBoth, out, out_dtype, q, 1, k_cache, v_cache, block_tables, max_blocks_per_seq,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                    max_context_len, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status_t pa_decode_partitions(void* out, pa_dtype_t out_dtype, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, int32_t max_context_len, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, pa_dtype_t dtype, void* stream) {
  return run_decode(DecodePhase::kPartitions, out, out_dtype, q, 1, k_cache, v_cache, block_tables, max_blocks_per_seq,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                    max_context_len, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status_t pa_decode_reduce(void* out, pa_dtype_t out_dtype, const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                             int32_t partition_size, const void* workspace, size_t workspace_bytes, void* stream) {
  if (head_dim != 64 && head_dim != 128) return fail(PA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (!(out_dtype == PA_F32 || out_dtype == PA_F16 || out_dtype == PA_BF16))
    return fail(PA_EUNSUPPORTED, "unknown out_dtype");
  if (num_seqs < 0 || max_context_len < 0) return fail(PA_EINVAL, "bad sizes");
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads,
                num_kv_heads);
  if (partition_size < 0 || partition_size % 16 != 0)
    return fail(PA_EINVAL, "partition_size must be 0 or a positive multiple of 16");
  const int32_t p = choose_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  const int64_t nparts = max_context_len == 0 ? 1 : ceil_div(max_context_len, p);
  const size_t need = ws_size(num_seqs, 1, num_q_heads, num_kv_heads, head_dim, nparts);
  if (need == 0 || num_seqs == 0) return PA_OK;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PA_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if (!out || !context_lens) return fail(PA_EINVAL, "null pointer argument");
  DecodeArgs a{};
  a.out = out;
  a.out_f32 = out_dtype == PA_F32;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_context_len = max_context_len;
  a.max_blocks = int32_t(ceil_div(max_context_len, 16));
  a.partition = p;
  a.num_partitions = int32_t(nparts);
  a.q_len = 1;
  split_workspace(const_cast<void*>(workspace), num_seqs, 1, num_q_heads, num_kv_heads, head_dim, nparts, &a);
  a.dtype = out_dtype == PA_F32 ? PA_F16 : out_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_decode_reduce(a), "decode reduce launch");
}

pa_status_t pa_prefill_chunk(void* out, pa_dtype_t out_dtype, const void* q, int32_t chunk_len, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float scale, int32_t max_context_len, pa_dtype_t dtype, void* stream) {
  pa_status_t st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (dtype == PA_F32) return fail(PA_EUNSUPPORTED, "prefill runs on the matrix cores: fp16 or bf16 only");
  if (num_seqs < 0 || chunk_len < 0) return fail(PA_EINVAL, "num_seqs and chunk_len must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16) return fail(PA_EUNSUPPORTED, "query group %d > 16", num_q_heads / num_kv_heads);
  if (!(out_dtype == PA_F32 || out_dtype == dtype)) return fail(PA_EUNSUPPORTED, "out_dtype must be PA_F32 or the input dtype");
  if (max_context_len < chunk_len) return fail(PA_EINVAL, "max_context_len must be >= chunk_len");
  if (max_blocks_per_seq < 0 || int64_t(max_blocks_per_seq) * block_size < max_context_len)
    return fail(PA_EINVAL, "max_blocks_per_seq cannot hold max_context_len");
  if (!isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (num_seqs == 0 || chunk_len == 0) return PA_OK;
  // rows (query, head of the group) and workgroups are counted in int on the device
  const int64_t rows = int64_t(chunk_len) * (num_q_heads / num_kv_heads);
  if (rows > INT32_MAX / 2 || (rows / 16 + 1) * num_seqs * num_kv_heads > INT32_MAX)
    return fail(PA_EUNSUPPORTED, "grid too large");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return fail(PA_EINVAL, "null pointer argument");
  PrefillArgs a{};
  a.out = out;
  a.out_f32 = out_dtype == PA_F32;
  a.q = q;
  a.chunk = chunk_len;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * kLog2e;
  a.max_context_len = max_context_len;
  a.tile_shift = tile_shift_of(block_size);
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_prefill_chunk(a), "prefill launch");
}

pa_status_t pa_probe_read_bandwidth(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                    void* stream) {
  if (bytes < 0 || workgroups <= 0) return fail(PA_EINVAL, "bytes must be >= 0 and workgroups > 0");
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return fail(PA_EINVAL, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(PA_EINVAL, "buf must be 16-byte aligned");
  return hip_status(launch_read_probe(buf, bytes, sink, workgroups, static_cast<hipStream_t>(stream)),
                    "read probe launch");
}

pa_status_t pa_probe_gather_bandwidth(const void* buf, int64_t buf_bytes, const int32_t* tiles, int64_t num_tiles,
                                      int32_t tile_bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (buf_bytes < 0 || num_tiles < 0 || workgroups <= 0) return fail(PA_EINVAL, "sizes must be >= 0 and workgroups > 0");
  if (tile_bytes <= 0 || tile_bytes % 1024 != 0 || tile_bytes > (64 << 10))
    return fail(PA_EINVAL, "tile_bytes must be a multiple of 1024 up to 64 KiB (got %d)", tile_bytes);
  if (num_tiles == 0) return PA_OK;
  if (!buf || !tiles || !sink) return fail(PA_EINVAL, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(PA_EINVAL, "buf must be 16-byte aligned");
  if (buf_bytes / tile_bytes > INT32_MAX) return fail(PA_EUNSUPPORTED, "more than 2^31 tiles in buf");
  return hip_status(launch_gather_probe(buf, buf_bytes / tile_bytes, tiles, num_tiles, tile_bytes, sink, workgroups,
                                        static_cast<hipStream_t>(stream)),
                    "gather probe launch");
}

}  // extern "C"
