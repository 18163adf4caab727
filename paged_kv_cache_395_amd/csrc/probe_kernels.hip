// Measurement probe: the HBM read ceiling of this GPU for the load style the
// decode kernel uses (16-byte non-temporal buffer loads, 4 in flight per
// lane), so decode's achieved bandwidth can be set against what a plain
// stream of reads reaches on the same part.

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr int64_t kChunkBytes = int64_t(kProbeThreads) * kProbeUnroll * 16;  // per workgroup per round

// Each workgroup reads chunks blockIdx.x, blockIdx.x + gridDim.x, ... of
// kChunkBytes; a resource per chunk bounds the loads (the tail past `bytes`
// reads as zeros).  The XOR of everything read goes to `sink` only if it
// equals a value no input produces in practice, so the loads cannot be
// removed.
__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const char* buf, int64_t bytes, uint32_t* sink) {
  uint32_t acc = 0;
  const int off = threadIdx.x * 16;
  for (int64_t c = blockIdx.x; c * kChunkBytes < bytes; c += gridDim.x) {
    const int64_t base = c * kChunkBytes;
    const int64_t left = bytes - base;
    const int range = int(left < kChunkBytes ? left : kChunkBytes);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(buf + base), 0, range, kBufferRsrcWord3);
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + u * kProbeThreads * 16, 0,
                                                                                kCachePolicyNT));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(workgroups)), dim3(kProbeThreads), 0, stream,
                     static_cast<const char*>(buf), bytes, sink);
  return hipGetLastError();
}

}  // namespace pa
