// Decode without a caller workspace and without any allocation, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The split-context partials and the merge's bookkeeping go to `scratch`, a
// file-scope device array of kNoAllocScratchBytes that every GPU the library
// runs on holds from the library's load until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is a host-side
// stand-in, not a device address): the first call on each device looks up
// that device's address with hipGetSymbolAddress, with the device current,
// and every call uses the address kept for its device.  All calls on one GPU
// share its array; calls that overlap on one GPU (different streams) race
// for it.  Nothing in it has to start at zero: each call's partition launch
// writes the header, the slot counts and every partial its merge reads.

#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // scratch's address on each device, once looked up

pa_status_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_EUNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

pa_status_t pa_decode_noalloc(void* out, pa_dtype_t out_dtype, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              float scale, int32_t max_context_len, int32_t partition_size, pa_dtype_t dtype,
                              void* stream) {
  void* ptr = nullptr;
  const pa_status_t st = scratch_on_current_device(&ptr);
  if (st != PA_OK) return st;
  return decode_in_scratch(ptr, kNoAllocScratchBytes, out, out_dtype, q, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, scale, max_context_len, partition_size, dtype, stream);
}

}  // extern "C"
