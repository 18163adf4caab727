// Cache write (each new token's K/V rows into its slot) and whole-block copy
// for copy-on-write.  Both are bit copies; neither interprets the values.
//
// Pages: "PagedAttention: How vLLM Serves AI Like an Operating System" --
// blocks are filled on demand as tokens are stored (section "PagedAttention:
// Virtual Memory for KV Cache", How It Works; "The Magic: No
// Pre-allocation"), and a shared block is copied before a sequence may
// modify it (section "Copy-on-Write: Sharing KV Cache").

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Element offset of the 16-token tile that holds `slot`, for kv head h: a
// (block, kv head) run is 2^sh consecutive tiles of 16 * D elements.
__device__ inline int64_t slot_tile(int64_t slot, int h, int kv_heads, int head_dim, int sh) {
  const int64_t blk = slot >> (4 + sh);
  const int64_t sub = (slot >> 4) & ((1 << sh) - 1);
  return (((blk * kv_heads + h) << sh) + sub) * int64_t(kBlockTokens * head_dim);
}

// One thread moves one 8-element run (dims 8j..8j+7 of one kv head) of one
// token.  K: the run is contiguous in the tile ([D/8][16][8]), one vector
// store.  V: the 8 dims scatter to 8 positions of the [D/32][4][16][2][4]
// tile, one element each.
template <typename E>
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ kc,
                         E* __restrict__ vc, const int64_t* __restrict__ slots, int32_t num_tokens,
                         int32_t kv_heads, int32_t head_dim, int64_t num_blocks, int32_t sh) {
  typedef E vec8 __attribute__((ext_vector_type(8)));
  const int runs_per_head = head_dim / 8;
  const int runs_per_token = kv_heads * runs_per_head;
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= int64_t(num_tokens) * runs_per_token) return;
  const int t = int(c / runs_per_token);
  const int rem = int(c - int64_t(t) * runs_per_token);
  const int h = rem / runs_per_head;
  const int j = rem - h * runs_per_head;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (num_blocks << (4 + sh))) return;  // skipped token, or outside the pool
  const int o = int(slot & 15);
  const int64_t src = (int64_t(t) * kv_heads + h) * head_dim + 8 * j;
  const int64_t tile = slot_tile(slot, h, kv_heads, head_dim, sh);

  const vec8 kv = *reinterpret_cast<const vec8*>(key + src);
  *reinterpret_cast<vec8*>(kc + tile + (j * kBlockTokens + o) * 8) = kv;

  const vec8 vv = *reinterpret_cast<const vec8*>(value + src);
  E* vt = vc + tile;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * j + e;
    const int off = (((d >> 5) * 4 + (o >> 2)) * 16 + (d & 15)) * 8 + ((d >> 4) & 1) * 4 + (o & 3);
    vt[off] = vv[e];
  }
}

template <typename E>
using Vec8 = E __attribute__((ext_vector_type(8)));

// A step's token t is spread over gridDim.y workgroups: thread i of
// workgroup (t, y) moves run c = y * blockDim.x + i (dims 8j..8j+7 of kv
// head c / (D / 8)), so the scattered single-element V stores of one token
// run on several CUs.
__device__ inline int step_run() { return int(blockIdx.y * blockDim.x + threadIdx.x); }

// This thread's K/V run of token t (zeros past the token's runs), loaded
// before the slot is known.
template <typename E>
__device__ inline void load_step_run(const E* __restrict__ key, const E* __restrict__ value, int t, int32_t kv_heads,
                                     int32_t head_dim, Vec8<E>& kv, Vec8<E>& vv) {
  const int runs_per_head = head_dim / 8;
  const int c = step_run();
  kv = Vec8<E>{};
  vv = Vec8<E>{};
  if (c < kv_heads * runs_per_head) {
    const int h = c / runs_per_head, j = c - h * runs_per_head;
    const int64_t src = (int64_t(t) * kv_heads + h) * head_dim + 8 * j;
    kv = *reinterpret_cast<const Vec8<E>*>(key + src);
    vv = *reinterpret_cast<const Vec8<E>*>(value + src);
  }
}

// Stores this thread's run of token t into `slot`; the first thread of the
// token sets table[row][pos / 16] = slot / 16: the block the slot lies in (a
// new block when pos % 16 == 0, the fresh copy after a copy-on-write, the
// same block otherwise).
template <typename E>
__device__ inline void store_step_run(E* __restrict__ kc, E* __restrict__ vc, int64_t slot, int row, int pos,
                                      int32_t* tables, int32_t max_blocks, int32_t num_rows, int32_t kv_heads,
                                      int32_t head_dim, int64_t num_blocks, int32_t sh, Vec8<E> kv, Vec8<E> vv) {
  if (slot < 0 || slot >= (num_blocks << (4 + sh))) return;  // skipped token, or outside the pool
  const int c = step_run();
  if (c == 0 && row >= 0 && row < num_rows && pos >= 0 && (pos >> (4 + sh)) < max_blocks)
    tables[int64_t(row) * max_blocks + (pos >> (4 + sh))] = int32_t(slot >> (4 + sh));
  const int runs_per_head = head_dim / 8;
  if (c >= kv_heads * runs_per_head) return;
  const int h = c / runs_per_head, j = c - h * runs_per_head;
  const int o = int(slot & 15);
  const int64_t tile = slot_tile(slot, h, kv_heads, head_dim, sh);
  *reinterpret_cast<Vec8<E>*>(kc + tile + (j * kBlockTokens + o) * 8) = kv;
  E* vt = vc + tile;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * j + e;
    vt[(((d >> 5) * 4 + (o >> 2)) * 16 + (d & 15)) * 8 + ((d >> 4) & 1) * 4 + (o & 3)] = vv[e];
  }
}

// One step's appends with the block tables and context lengths kept on the
// device: workgroups (t < T, y) store token t; the workgroups (t >= T, 0)
// after those copy new_ctx into ctx.  The token's (slot, row, pos) are read
// once per workgroup, by thread 0, into LDS: they may live in pinned host
// memory, where every read crosses the host link.
constexpr int kAppendThreads = 128;
template <typename E>
__global__ void __launch_bounds__(kAppendThreads)
append_step_kernel(const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ kc, E* __restrict__ vc,
                   const int64_t* slots, const int32_t* rows, const int32_t* positions, int32_t num_tokens,
                   int32_t* tables, int32_t max_blocks, int32_t* ctx, const int32_t* new_ctx, int32_t num_rows,
                   int32_t kv_heads, int32_t head_dim, int64_t num_blocks, int32_t sh) {
  const int t = blockIdx.x;
  if (t >= num_tokens) {
    const int i = (t - num_tokens) * blockDim.x + threadIdx.x;
    if (blockIdx.y == 0 && i < num_rows) ctx[i] = new_ctx[i];
    return;
  }
  __shared__ int64_t s_slot;
  __shared__ int32_t s_row, s_pos;
  // the thread's K/V run is read before the metadata wait, so the device
  // reads overlap the (slower) read of the slot from host memory
  Vec8<E> kv, vv;
  load_step_run(key, value, t, kv_heads, head_dim, kv, vv);
  if (threadIdx.x == 0) {
    s_slot = slots[t];
    s_row = rows[t];
    s_pos = positions[t];
  }
  __syncthreads();
  store_step_run(kc, vc, s_slot, s_row, s_pos, tables, max_blocks, num_rows, kv_heads, head_dim, num_blocks, sh, kv,
                 vv);
}

// The same step with its metadata in the kernel arguments (one launch's
// share of the tokens and rows, copied from host memory at launch): every
// thread reads its token's (slot, row, pos) through the scalar cache from
// the argument segment in device memory, and nothing crosses the host link.
// key / value point at the launch's first token.
template <typename E>
__global__ void __launch_bounds__(kAppendThreads)
append_args_kernel(const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ kc, E* __restrict__ vc,
                   const AppendArgsMeta meta, int32_t* tables, int32_t max_blocks, int32_t* ctx, int32_t num_rows,
                   int32_t kv_heads, int32_t head_dim, int64_t num_blocks, int32_t sh) {
  const int t = blockIdx.x;
  if (t >= meta.num_tokens) {
    const int i = (t - meta.num_tokens) * blockDim.x + threadIdx.x;
    if (blockIdx.y == 0 && i < meta.num_rows) ctx[meta.row0 + i] = meta.new_ctx[i];
    return;
  }
  Vec8<E> kv, vv;
  load_step_run(key, value, t, kv_heads, head_dim, kv, vv);
  store_step_run(kc, vc, meta.slots[t], meta.rows[t], meta.positions[t], tables, max_blocks, num_rows, kv_heads,
                 head_dim, num_blocks, sh, kv, vv);
}

// Grid (chunks of one block, pairs, 2): z = 0 copies K, z = 1 copies V; each
// thread moves 16 bytes of block pairs[i][0] of the source pools into block
// pairs[i][1] of the destination pools.  Copy-on-write passes one pool as
// both; a swap passes the device pools and pinned host pools (either way).
__global__ void __launch_bounds__(256)
copy_blocks_kernel(char* __restrict__ dk, char* __restrict__ dv, const char* __restrict__ sk,
                   const char* __restrict__ sv, const int64_t* __restrict__ pairs, int64_t block_bytes,
                   int64_t src_blocks, int64_t dst_blocks) {
  char* dst_base = blockIdx.z ? dv : dk;
  const char* src_base = blockIdx.z ? sv : sk;
  const int64_t src = pairs[2 * int64_t(blockIdx.y)];
  const int64_t dst = pairs[2 * int64_t(blockIdx.y) + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t off = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 16;
  if (off >= block_bytes) return;
  *reinterpret_cast<u32x4_t*>(dst_base + dst * block_bytes + off) =
      *reinterpret_cast<const u32x4_t*>(src_base + src * block_bytes + off);
}

// One thread per patch (row, logical block, physical block).
__global__ void __launch_bounds__(256)
patch_tables_kernel(int32_t* __restrict__ tables, int32_t max_blocks, int32_t num_rows,
                    const int32_t* __restrict__ patches, int32_t num_patches) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_patches) return;
  const int32_t row = patches[3 * i], idx = patches[3 * i + 1], blk = patches[3 * i + 2];
  if (row < 0 || row >= num_rows || idx < 0 || idx >= max_blocks) return;
  tables[int64_t(row) * max_blocks + idx] = blk;
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int64_t num_blocks, int32_t tile_shift, int elem_bytes,
                                    hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t runs = int64_t(num_tokens) * num_kv_heads * (head_dim / 8);
  const dim3 grid(unsigned((runs + 255) / 256));
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), slots, num_tokens,
                       num_kv_heads, head_dim, num_blocks, tile_shift);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint32_t*>(key), static_cast<const uint32_t*>(value),
                       static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache), slots, num_tokens,
                       num_kv_heads, head_dim, num_blocks, tile_shift);
  }
  return hipGetLastError();
}

// workgroups per token: one 8-element run per thread
int64_t step_run_groups(const AppendStepArgs& a) {
  return (int64_t(a.num_kv_heads) * (a.head_dim / 8) + kAppendThreads - 1) / kAppendThreads;
}

hipError_t launch_append_step(const AppendStepArgs& a) {
  const int64_t ctx_groups = (int64_t(a.num_rows) + kAppendThreads - 1) / kAppendThreads;
  const int64_t grid_x = int64_t(a.num_tokens) + ctx_groups;
  if (grid_x == 0) return hipSuccess;
  const dim3 grid(unsigned(grid_x), unsigned(step_run_groups(a)));
  if (a.elem_bytes == 2) {
    hipLaunchKernelGGL(append_step_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, a.stream,
                       static_cast<const uint16_t*>(a.key), static_cast<const uint16_t*>(a.value),
                       static_cast<uint16_t*>(a.k_cache), static_cast<uint16_t*>(a.v_cache), a.slots, a.rows,
                       a.positions, a.num_tokens, a.tables, a.max_blocks, a.ctx, a.new_ctx, a.num_rows,
                       a.num_kv_heads, a.head_dim, a.num_blocks, a.tile_shift);
  } else {
    hipLaunchKernelGGL(append_step_kernel<uint32_t>, grid, dim3(kAppendThreads), 0, a.stream,
                       static_cast<const uint32_t*>(a.key), static_cast<const uint32_t*>(a.value),
                       static_cast<uint32_t*>(a.k_cache), static_cast<uint32_t*>(a.v_cache), a.slots, a.rows,
                       a.positions, a.num_tokens, a.tables, a.max_blocks, a.ctx, a.new_ctx, a.num_rows,
                       a.num_kv_heads, a.head_dim, a.num_blocks, a.tile_shift);
  }
  return hipGetLastError();
}

hipError_t launch_append_step_args(const AppendStepArgs& a, const AppendArgsMeta& meta) {
  const int64_t grid_x = int64_t(meta.num_tokens) + (int64_t(meta.num_rows) + kAppendThreads - 1) / kAppendThreads;
  if (grid_x == 0) return hipSuccess;
  const dim3 grid(unsigned(grid_x), unsigned(step_run_groups(a)));
  if (a.elem_bytes == 2) {
    hipLaunchKernelGGL(append_args_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, a.stream,
                       static_cast<const uint16_t*>(a.key), static_cast<const uint16_t*>(a.value),
                       static_cast<uint16_t*>(a.k_cache), static_cast<uint16_t*>(a.v_cache), meta, a.tables,
                       a.max_blocks, a.ctx, a.num_rows, a.num_kv_heads, a.head_dim, a.num_blocks, a.tile_shift);
  } else {
    hipLaunchKernelGGL(append_args_kernel<uint32_t>, grid, dim3(kAppendThreads), 0, a.stream,
                       static_cast<const uint32_t*>(a.key), static_cast<const uint32_t*>(a.value),
                       static_cast<uint32_t*>(a.k_cache), static_cast<uint32_t*>(a.v_cache), meta, a.tables,
                       a.max_blocks, a.ctx, a.num_rows, a.num_kv_heads, a.head_dim, a.num_blocks, a.tile_shift);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int64_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks,
                              hipStream_t stream) {
  const unsigned chunks = unsigned((block_bytes / 16 + 255) / 256);
  for (int32_t first = 0; first < num_pairs; first += 65535) {
    const int32_t n = num_pairs - first < 65535 ? num_pairs - first : 65535;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(chunks, unsigned(n), 2), dim3(256), 0, stream,
                       static_cast<char*>(dst_k), static_cast<char*>(dst_v), static_cast<const char*>(src_k),
                       static_cast<const char*>(src_v), pairs + 2 * int64_t(first), block_bytes, src_blocks,
                       dst_blocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_patch_tables(int32_t* tables, int32_t max_blocks, int32_t num_rows, const int32_t* patches,
                               int32_t num_patches, hipStream_t stream) {
  if (num_patches == 0) return hipSuccess;
  hipLaunchKernelGGL(patch_tables_kernel, dim3(unsigned((num_patches + 255) / 256)), dim3(256), 0, stream, tables,
                     max_blocks, num_rows, patches, num_patches);
  return hipGetLastError();
}

}  // namespace pa
