// Chunked prefill over the paged cache for gfx950 (matrix cores).
//
// A chunk of C new queries per sequence sits at the last C positions of its
// context; query i attends keys 0 .. ctx - C + i (causal).  K/V are reached
// through the block table exactly as in decode ("PagedAttention: How vLLM
// Serves AI Like an Operating System", section "PagedAttention: Virtual
// Memory for KV Cache").
//
// Work split: rows are (query i, head n of the kv group), row = i * G + n.
// One workgroup of WAVES waves owns WAVES * RT * 16 consecutive rows of one
// (kv head, sequence) and walks the key blocks in order.  Each 16-token K/V
// tile is fetched from HBM once per workgroup into double-buffered LDS and
// read by every wave.  Products are written transposed as in decode:
//   S^T[token][row] = K . Q^T   (16x16x32),   O^T[dim][row] += V^T . P^T (16x16x16)
// with P split hi + lo in the input type.

#include <math.h>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct PParams {
  void* out;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* tables;
  const int32_t* ctxs;
  int64_t num_blocks;
  float scale_log2;
  int32_t max_blocks;
  int32_t chunk, hq, hkv, max_ctx;
};

template <typename T, bool OUT_F32>
__device__ inline void store_row4(void* out, int64_t idx, f32x4_t v) {
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + idx) = v;
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + idx;
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
    u32x2_t p = {pack2(T::from_float(v[0]), T::from_float(v[1])), pack2(T::from_float(v[2]), T::from_float(v[3]))};
    *reinterpret_cast<u32x2_t*>(o) = p;
  }
}

template <typename T, int D, int WAVES, int RT, bool OUT_F32>
__global__ void __launch_bounds__(WAVES * 64)
prefill_mfma_kernel(PParams P) {
  constexpr int DC = D / 32;
  constexpr int NT = D / 16;
  constexpr int kThreads = WAVES * 64;
  constexpr int kTileElems = kBlockTokens * D;
  constexpr int kTileChunks = kTileElems / 8;  // 16-byte chunks per tile
  constexpr int kRowsPerWave = RT * 16;
  constexpr int kRowsPerWG = WAVES * kRowsPerWave;
  constexpr int kStage = (kTileChunks + kThreads - 1) / kThreads;

  __shared__ u32x4_t s_k[2][kTileChunks];
  __shared__ u32x4_t s_v[2][kTileChunks];

  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, quad = lane >> 4;
  const int G = P.hq / P.hkv;
  const int C = P.chunk;
  const int R = C * G;
  const int ctx = P.ctxs[s];
  const int row_wg0 = tile * kRowsPerWG;
  if (row_wg0 >= R) return;

  if (ctx < C || ctx > P.max_ctx || ctx > P.max_blocks * kBlockTokens) {
    // contract violation: NaN rows for this workgroup's share
    const float nan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < kRowsPerWG * D; idx += kThreads) {
      const int row = row_wg0 + idx / D, d = idx % D;
      if (row >= R) break;
      const int i = row / G, hh = row - i * G;
      const int64_t o = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D + d;
      if constexpr (OUT_F32) static_cast<float*>(P.out)[o] = nan;
      else static_cast<uint16_t*>(P.out)[o] = T::from_float(nan);
    }
    return;
  }

  // rows of this lane, one per row tile
  int last[RT];
  bool live[RT];
  u32x4_t qb[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row_wg0 + w * kRowsPerWave + rt * 16 + n;
    live[rt] = row < R;
    const int i = live[rt] ? row / G : 0;
    const int hh = live[rt] ? row - i * G : 0;
    last[rt] = ctx - C + i;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qb[rt][c] = live[rt] ? load16(P.q + ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D + 8 * (4 * c + quad))
                           : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const int row_wg_last = min(R, row_wg0 + kRowsPerWG) - 1;
  const int nkb = (ctx - C + row_wg_last / G) / kBlockTokens + 1;  // key blocks any row of the WG needs
  const int32_t* trow = P.tables + int64_t(s) * P.max_blocks;
  const int64_t blk_stride = int64_t(P.hkv) * kTileElems;
  const uint16_t* kg = P.k + int64_t(g) * kTileElems;
  const uint16_t* vg = P.v + int64_t(g) * kTileElems;

  float m[RT], lsum[RT];
  f32x4_t o[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = false;

  u32x4_t stk[kStage], stv[kStage];
  auto fetch = [&](int kb) {
    int phys = trow[kb];
    if (phys < 0 || int64_t(phys) >= P.num_blocks) {
      bad = true;
      phys = 0;
    }
    const uint16_t* kt = kg + int64_t(phys) * blk_stride;
    const uint16_t* vt = vg + int64_t(phys) * blk_stride;
#pragma unroll
    for (int e = 0; e < kStage; ++e) {
      const int c = threadIdx.x + e * kThreads;
      if (c < kTileChunks) {
        stk[e] = load16(kt + c * 8);
        stv[e] = load16(vt + c * 8);
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int e = 0; e < kStage; ++e) {
      const int c = threadIdx.x + e * kThreads;
      if (c < kTileChunks) {
        s_k[buf][c] = stk[e];
        s_v[buf][c] = stv[e];
      }
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) fetch(kb + 1);

    u32x4_t kc[DC], vc[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      kc[c] = s_k[buf][c * 64 + lane];
      vc[c] = s_v[buf][c * 64 + lane];
    }
    const int tok_base = kb * kBlockTokens + 4 * quad;
    if (kb * kBlockTokens + kBlockTokens > ctx) {
      const int valid = ctx - kb * kBlockTokens;
      const int t0 = 4 * quad;
      const uint32_t m01 = (t0 + 0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        vc[c][0] &= m01;
        vc[c][1] &= m23;
        vc[c][2] &= m01;
        vc[c][3] &= m23;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) sc = Mfma<T>::k32(kc[c], qb[rt][c], sc);
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = (tok_base + r <= last[rt]) ? sc[r] * P.scale_log2 : -INFINITY;
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = fmaxf(bm, shfl_xor(bm, 16));
      bm = fmaxf(bm, shfl_xor(bm, 32));
      const float mn = fmaxf(m[rt], bm);
      const float alpha = fast_exp2(m[rt] - mn);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - mn);
      lsum[rt] = lsum[rt] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m[rt] = mn;
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = T::from_float(pr[r]);
        lo[r] = T::from_float(pr[r] - T::to_float(hi[r]));
      }
      const uint32_t bh0 = pack2(hi[0], hi[1]), bh1 = pack2(hi[2], hi[3]);
      const uint32_t bl0 = pack2(lo[0], lo[1]), bl1 = pack2(lo[2], lo[3]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t a0 = vc[t / 2][2 * (t % 2)];
        const uint32_t a1 = vc[t / 2][2 * (t % 2) + 1];
        f32x4_t acc = o[rt][t] * alpha;
        acc = Mfma<T>::k16(a0, a1, bh0, bh1, acc);
        o[rt][t] = Mfma<T>::k16(a0, a1, bl0, bl1, acc);
      }
    }
    if (kb + 1 < nkb) stage(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lsum[rt];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (!live[rt]) continue;
    const int row = row_wg0 + w * kRowsPerWave + rt * 16 + n;
    const int i = row / G, hh = row - i * G;
    const int64_t obase = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D;
    const float inv = bad ? __builtin_nanf("") : 1.f / l;
#pragma unroll
    for (int t = 0; t < NT; ++t) store_row4<T, OUT_F32>(P.out, obase + 16 * t + 4 * quad, o[rt][t] * inv);
  }
}

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRT = 2;

template <typename T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, const PParams& p) {
  constexpr int rows_per_wg = kPrefillWaves * kPrefillRT * 16;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t R = int64_t(a.chunk) * G;
  const dim3 grid(unsigned((R + rows_per_wg - 1) / rows_per_wg), unsigned(a.num_kv_heads), unsigned(a.num_seqs));
  if (a.out_f32) {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, kPrefillWaves, kPrefillRT, true>), grid, dim3(kPrefillWaves * 64), 0,
                       a.stream, p);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, kPrefillWaves, kPrefillRT, false>), grid, dim3(kPrefillWaves * 64), 0,
                       a.stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillArgs& a) {
  if (a.num_seqs == 0 || a.chunk == 0) return hipSuccess;
  PParams p{};
  p.out = a.out;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k_cache);
  p.v = static_cast<const uint16_t*>(a.v_cache);
  p.tables = a.block_tables;
  p.ctxs = a.context_lens;
  p.num_blocks = a.num_blocks;
  p.scale_log2 = a.scale_log2;
  p.max_blocks = a.max_blocks;
  p.chunk = a.chunk;
  p.hq = a.num_q_heads;
  p.hkv = a.num_kv_heads;
  p.max_ctx = a.max_context_len;
  if (a.dtype == PA_BF16) return a.head_dim == 64 ? launch_prefill_t<Bf16, 64>(a, p) : launch_prefill_t<Bf16, 128>(a, p);
  return a.head_dim == 64 ? launch_prefill_t<F16, 64>(a, p) : launch_prefill_t<F16, 128>(a, p);
}

}  // namespace pa
