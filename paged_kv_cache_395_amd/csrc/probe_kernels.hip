// Measurement probes: the HBM read ceiling of this GPU for the load style the
// decode kernel uses (16-byte non-temporal buffer loads), once for a plain
// stream of reads and once for a gather of whole tiles in random order (the
// access pattern of paged decode), so decode's achieved bandwidth can be set
// against what each reaches on the same part.

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

constexpr int kGatherWaves = 4;

// Wave v of the grid (v = blockIdx.x * 4 + wave) reads tiles[v], tiles[v +
// waves], ... each as tile_bytes / 1024 wave loads of 16 bytes per lane
// through a resource bounded to the tile, two tiles in flight, the way a
// decode wave walks its blocks.  Same sink rule as the stream probe.
__global__ void __launch_bounds__(kGatherWaves * kWave)
gather_probe_kernel(const char* buf, int64_t buf_tiles, const int32_t* tiles, int64_t num_tiles, int32_t tile_bytes,
                    uint32_t* sink) {
  const int lane = lane_id();
  const int64_t wave = int64_t(blockIdx.x) * kGatherWaves + (threadIdx.x >> 6);
  const int64_t waves = int64_t(gridDim.x) * kGatherWaves;
  const int runs = tile_bytes / 1024;
  uint32_t acc = 0;
  for (int64_t t = wave; t < num_tiles; t += 2 * waves) {
    // a tile index outside buf gets an empty range: zeros, no access
    const int64_t i0 = tiles[t];
    const int64_t i1 = t + waves < num_tiles ? tiles[t + waves] : -1;
    const bool ok0 = i0 >= 0 && i0 < buf_tiles, ok1 = i1 >= 0 && i1 < buf_tiles;
    const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(buf + (ok0 ? i0 : 0) * tile_bytes), 0, ok0 ? tile_bytes : 0, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(buf + (ok1 ? i1 : 0) * tile_bytes), 0, ok1 ? tile_bytes : 0, kBufferRsrcWord3);
    for (int part = 0; part < runs; part += 4) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int off = lane * 16 + (part + u) * 1024;  // past the tile (runs % 4 != 0): zeros, no access
        v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, kCachePolicyNT));
        v[4 + u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, kCachePolicyNT));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_gather_probe(const void* buf, int64_t buf_tiles, const int32_t* tiles, int64_t num_tiles,
                               int32_t tile_bytes, uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(gather_probe_kernel, dim3(unsigned(workgroups)), dim3(kGatherWaves * kWave), 0, stream,
                     static_cast<const char*>(buf), buf_tiles, tiles, num_tiles, tile_bytes, sink);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(workgroups)), dim3(kProbeThreads), 0, stream,
                     static_cast<const char*>(buf), bytes, sink);
  return hipGetLastError();
}

}  // namespace pa
