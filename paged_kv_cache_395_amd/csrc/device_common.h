// Device helpers shared by the gfx950 kernels: element types, 16-byte
// vector loads, wave-level reductions and the matrix-core instructions used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;  // tokens per KV block
constexpr int kWave = 64;         // CDNA wavefront width

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// Element-type tags of the 16-bit storage formats.  Storage is always the raw
// 16-bit pattern; the tags pick conversions and matrix-core instructions.
struct Bf16 {
  __device__ static inline float to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
  // round to nearest even (hardware conversion)
  __device__ static inline uint16_t from_float(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
  }
};
struct F16 {
  __device__ static inline float to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  __device__ static inline uint16_t from_float(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
  }
};

// 16-byte global load of 8 consecutive 16-bit elements as raw bits.
__device__ inline u32x4_t load16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Buffer resources (base, range) for raw buffer loads.  Word 3 of a CDNA3/4
// resource: 32-bit data format, no swizzle, no index striding.  A load whose
// offset falls outside the range returns zeros and issues no memory access.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache-policy operand of buffer loads: the non-temporal hint (streamed data
// that is read once).
constexpr int kCachePolicyNT = 2;

// ---------------------------------------------------------------------------
// Matrix-core products, 16x16 output tiles, fp32 accumulate.
//
// For every 16x16xK instruction used here the operand lane layout is: lane l
// supplies row (l % 16) of A and column (l % 16) of B, each with the k-slice
// owned by lane group l / 16; the accumulator lane l holds column (l % 16),
// rows 4 * (l / 16) + 0..3.  A and B assign k-values to (lane, element) the
// same way, so any consistent assignment of a contraction index to k is valid.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<Bf16> {
  // K = 32: 8 elements per lane (one 16-byte chunk)
  __device__ static inline f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // K = 16: 4 elements per lane (two dwords)
  __device__ static inline f32x4_t k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
    u32x2_t a = {a0, a1}, b = {b0, b1};
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
};

template <> struct Mfma<F16> {
  __device__ static inline f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4_t k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
    u32x2_t a = {a0, a1}, b = {b0, b1};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};

// Pack two 16-bit patterns into one dword (lo first).
__device__ inline uint32_t pack2(uint16_t lo, uint16_t hi) { return uint32_t(lo) | (uint32_t(hi) << 16); }

// Cross-lane exchange within the wave.
__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ inline float shfl(float v, int src) { return __shfl(v, src, kWave); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the 4 lane groups of 16 (lanes n, n + 16, n + 32, n + 48), on
// the permute network (no LDS round trip): swapping rows 1 <-> 0 and 3 <-> 2,
// then the two wave halves, leaves every lane with the max of its column.
__device__ inline float quad_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Lane group of 16 (0..3) and lane within it.
__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace pa
