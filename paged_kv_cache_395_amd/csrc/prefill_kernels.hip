// Chunked prefill over the paged cache for gfx950 (matrix cores).
//
// A chunk of C new queries per sequence sits at the last C positions of its
// context; query i attends keys 0 .. ctx - C + i (causal).  K/V are reached
// through the block table exactly as in decode ("PagedAttention: How vLLM
// Serves AI Like an Operating System", section "PagedAttention: Virtual
// Memory for KV Cache").
//
// Work split: rows are (query i, head n of the kv group), row = i * G + n.
// One workgroup of 4 waves owns 128 consecutive rows (2 tiles of 16 per
// wave) of one (kv head, sequence) and walks the keys in stages of 64 (4
// blocks); wave w fetches block w of each stage for the whole workgroup.
// K tiles go from HBM straight into LDS (16-byte direct-to-LDS loads).  V
// tiles go through registers: the loading wave converts its tile to fp16
// and stores it in LDS already in the A-operand layout of the PV product
// (the two blocks of a pair side by side in each lane's 16 bytes), so each
// operand is one 16-byte LDS read.  Both are double-buffered so the next
// stage loads while this one computes.
// Products are written transposed as in decode, all on the 16x16x32
// matrix instructions (the 16x16x16 forms run at half their rate):
//   S^T[token][row] = K . Q^T                      (per 16-token block)
//   O^T[dim][row]  += V^T . P^T                    (per pair of blocks, K = 32)
//   l[row]         += 1 . P^T                      (the row sums, same P)
// P is carried in fp16 (11 significant bits); the row sums are taken from
// the same rounded P, so a weight's rounding changes numerator and
// denominator together.  bf16 V is exact in fp16 below 2^16 in magnitude
// (values under 2^-17 lose low bits, an absolute error below 2^-24); a
// block holding anything larger, or a NaN, keeps its bf16 bits, and the
// pair it belongs to runs with P split hi + lo in bf16 instead.  The grid
// is one-dimensional and XCD-aware: all row tiles of one (sequence, kv
// head) run on one XCD, so their shared K / V stream is fetched from HBM
// once into that XCD's L2.

#include <math.h>

#include <type_traits>

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
  int32_t tile_shift;  // log2 of 16-token tiles per block (one table entry per block)
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

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kStageBlocks = 4;                        // 16-token blocks per stage
constexpr int kTabWindow = 2048;                       // block-table entries held in LDS
constexpr int kXcds = 8;
constexpr int kPrefillRowTiles = 2;      // 16-row tiles per wave
constexpr int kPrefillWavesPerSimd = 2;  // register budget: two waves per SIMD

typedef __attribute__((address_space(3))) void lds_void;

// Wait for this wave's outstanding memory loads (LDS-bound ones included).
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// NaN-propagating max (one v_maximum3_f32 per two inputs, no operand
// canonicalisation, which fmaxf needs for its NaN-ignoring semantics)
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the 4 lane groups of 16 (lanes n, n + 16, n + 32, n + 48) on the
// permute network; NaN-propagating
__device__ inline float quad_vmax(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// bf16 pair -> fp16 pair (exact below 2^16 in magnitude); big collects the
// largest magnitude seen (NaN once any value is NaN) so a wave can tell
// whether its tile converted exactly
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t x, float& big) {
  const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xFFFF0000u);
  big = vmax(big, vmax(__builtin_fabsf(lo), __builtin_fabsf(hi)));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
// fp16 pair holding bf16-representable values -> the same values in bf16 (exact)
__device__ inline uint32_t f16x2_to_bf16x2(uint32_t x) {
  const float lo = F16::to_float(uint16_t(x)), hi = F16::to_float(uint16_t(x >> 16));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}
// two floats -> fp16 pair, round to nearest even
__device__ inline uint32_t f16x2_rne(float a, float b) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// P is formed as 2^(c s - m + kPOffset): at most 2^(8 + 7) under the 2^8
// margin of the reference max, inside fp16's range, with the smallest
// weights 2^7 further above fp16's subnormals.  The offset cancels in O / l.
constexpr float kPOffset = 7.f;
// bf16 magnitudes from here up do not fit fp16; a tile holding one (or a
// NaN) keeps its bf16 bits
constexpr float kF16Limit = 65536.f;

// RT 16-row tiles per wave; WPE waves per SIMD the register budget is cut for
template <typename T, int D, bool OUT_F32, int RT, int WPE>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
prefill_mfma_kernel(PParams P, int tiles_per_pair, int num_pairs) {
  constexpr bool kBf16 = std::is_same<T, Bf16>::value;
  constexpr int kPfRT = RT;
  constexpr int kPfRows = kPfWaves * kPfRT * 16;  // rows per workgroup
  constexpr int DC = D / 32;                         // 16-byte chunks per lane per tile
  constexpr int NT = D / 16;                         // 16-dim output tiles
  constexpr int kTileElems = kBlockTokens * D;
  constexpr int kTileBytes = kTileElems * 2;
  constexpr int kRunsPerTile = kTileBytes / 1024;    // 1 KiB wave loads per tile
  static_assert(kRunsPerTile == DC, "one 16-byte chunk per lane per 1 KiB run");
  static_assert(kStageBlocks == kPfWaves, "each wave loads one block of a stage");
  constexpr int kStageU4 = kStageBlocks * kTileElems / 8;  // u32x4 per stage buffer (K or V)

  __shared__ u32x4_t s_k0[kStageU4];
  __shared__ u32x4_t s_k1[kStageU4];
  // V operands of a stage: [pair][output tile t][lane] 16 bytes = the lane's
  // 4 tokens of dim 16 t + (lane % 16) in the pair's first block, then the
  // same in its second block
  __shared__ u32x4_t s_v0[kStageU4];
  __shared__ u32x4_t s_v1[kStageU4];
  __shared__ int32_t s_tab[kTabWindow];
  __shared__ int s_vkeep[2][kStageBlocks];  // per V buffer: block kept in bf16
  __shared__ int s_bad;

  // XCD-aware work order: workgroup id % 8 picks the XCD; groups of 8
  // (sequence, kv head) pairs are dealt one per XCD, each with all its tiles
  const int id = blockIdx.x;
  const int full = (num_pairs / kXcds) * kXcds;
  int pair, tile;
  if (id < full * tiles_per_pair) {
    const int k = id / kXcds;
    pair = (k / tiles_per_pair) * kXcds + id % kXcds;
    tile = k % tiles_per_pair;
  } else {
    const int r = id - full * tiles_per_pair;
    pair = full + r / tiles_per_pair;
    tile = r % tiles_per_pair;
  }
  const int s = pair / P.hkv, g = pair - (pair / P.hkv) * P.hkv;

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, quad = lane >> 4;
  const int G = P.hq / P.hkv;
  const int C = P.chunk;
  const int R = C * G;
  const int ctx = P.ctxs[s];
  const int row_wg0 = tile * kPfRows;
  if (row_wg0 >= R) return;

  if (ctx < C || ctx > P.max_ctx || int64_t(ctx) > (int64_t(P.max_blocks) * kBlockTokens << P.tile_shift)) {
    // contract violation: NaN rows for this workgroup's share
    const float nan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < kPfRows * D; idx += kPfThreads) {
      const int row = row_wg0 + idx / D, d = idx % D;
      if (row >= R) break;
      const int i = row / G, hh = row - i * G;
      const int64_t o = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D + d;
      if constexpr (OUT_F32) static_cast<float*>(P.out)[o] = nan;
      else static_cast<uint16_t*>(P.out)[o] = T::from_float(nan);
    }
    return;
  }

  // rows of this lane (one per row tile), their last attended key, Q^T operands
  int last[kPfRT];
  bool live[kPfRT];
  u32x4_t qb[kPfRT][DC];
#pragma unroll
  for (int rt = 0; rt < kPfRT; ++rt) {
    const int row = row_wg0 + (w * kPfRT + rt) * 16 + n;
    live[rt] = row < R;
    const int i = live[rt] ? row / G : 0;
    const int hh = live[rt] ? row - i * G : 0;
    last[rt] = live[rt] ? ctx - C + i : -1;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qb[rt][c] = live[rt] ? load16(P.q + ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D + 8 * (4 * c + quad))
                           : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // Wait for the Q operands here, on every path.  Left to the compiler, the
  // wait lands at their first use inside the key loop, where a path that
  // skips the first stage's load makes it count the next stage's tile
  // loads too: every other stage then waited for its successor's tiles
  // before its first product (a third of the kernel's time).
  wait_loads();
  const int row_wg_last = min(R, row_wg0 + kPfRows) - 1;
  const int first_masked = ctx - C + row_wg0 / G;          // smallest last-key of the workgroup's rows
  const int nkb = (ctx - C + row_wg_last / G) / kBlockTokens + 1;  // key blocks any row needs
  const int nst = (nkb + kStageBlocks - 1) / kStageBlocks;
  const int32_t* trow = P.tables + int64_t(s) * P.max_blocks;
  const int sh = P.tile_shift;
  const int64_t blk_stride = (int64_t(P.hkv) << sh) * kTileElems;
  const char* kg = reinterpret_cast<const char*>(P.k + (int64_t(g) << sh) * kTileElems);
  const char* vg = reinterpret_cast<const char*>(P.v + (int64_t(g) << sh) * kTileElems);

  float m[kPfRT];
  f32x4_t lacc[kPfRT];  // row sums, every element of a lane holds its row's
  f32x4_t o[kPfRT][NT];
#pragma unroll
  for (int rt = 0; rt < kPfRT; ++rt) {
    m[rt] = -INFINITY;
    lacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) o[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  int bad = 0;

  int tab_base = 0;
  auto fill_table = [&](int base) {  // all threads; caller synchronises
    // one entry per 16-token tile (a block of 2^sh tiles repeats its entry)
    for (int j = threadIdx.x; j < kTabWindow && base + j < nkb; j += kPfThreads) s_tab[j] = trow[(base + j) >> sh];
  };

  // Loads of the stage's tiles: each lane moves 16 bytes per 1 KiB run.
  // Wave w fetches block w of the stage: its K tile into LDS directly, its
  // V tile into vreg.
  // One lookup and one buffer resource per tile (base in scalar registers,
  // range = the tile), so each load needs only the lane's 16-byte offset
  // and the run's scalar offset; a block past the key window or outside the
  // pool gets an empty range and reads as zeros without touching memory.
  const int lane_off = lane * 16;
  u32x4_t vreg[DC];
  auto issue_stage = [&](int st, u32x4_t* kbuf) {
    const int blk = st * kStageBlocks + w;
    const int phys = blk < nkb ? __builtin_amdgcn_readfirstlane(s_tab[blk - tab_base]) : 0;
    const bool in_pool = phys >= 0 && int64_t(phys) < P.num_blocks;
    bad |= blk < nkb && !in_pool;
    const bool ok = blk < nkb && in_pool;
    const int64_t off = ok ? (int64_t(phys) * blk_stride + int64_t(blk & ((1 << sh) - 1)) * kTileElems) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg + off), 0,
                                                                        ok ? kTileBytes : 0, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg + off), 0,
                                                                        ok ? kTileBytes : 0, kBufferRsrcWord3);
#pragma unroll
    for (int part = 0; part < kRunsPerTile; ++part) {
      lds_void* dst = (lds_void*)(kbuf + w * (kTileElems / 8) + part * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst, 16, lane_off, part * 1024, 0, 0);
    }
#pragma unroll
    for (int part = 0; part < kRunsPerTile; ++part)
      vreg[part] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, part * 1024, 0));
  };

  // The wave's V tile (block w of the stage) to LDS in the operand layout,
  // as fp16 when every value converts exactly.  Chunk cc of a V tile holds,
  // for lane (quad, n), tokens 4 quad + 0..3 of dim 32 cc + n (first 8
  // bytes) and of dim 32 cc + 16 + n (last 8 bytes): the lane's part of
  // output tiles 2 cc and 2 cc + 1.
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
  auto commit_v = [&](u32x4_t* vbuf, int slot) {
    u32x2_t* dst = reinterpret_cast<u32x2_t*>(vbuf) + ((w >> 1) * NT * 64 + lane) * 2 + (w & 1);
    bool keep = false;
    u32x4_t y[DC];
    if constexpr (kBf16) {
      float big = 0.f;
#pragma unroll
      for (int cc = 0; cc < DC; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) y[cc][j] = bf16x2_to_f16x2(vreg[cc][j], big);
      keep = __builtin_amdgcn_ballot_w64(!(big < kF16Limit)) != 0;
    }
    if (!kBf16 || keep) {
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) y[cc] = vreg[cc];
    }
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) {
      dst[(2 * cc) * 64 * 2] = u32x2_t{y[cc][0], y[cc][1]};
      dst[(2 * cc + 1) * 64 * 2] = u32x2_t{y[cc][2], y[cc][3]};
    }
    if (lane == 0) s_vkeep[slot][w] = keep;
  };

  // Scores are kept raw (q . k) and the scale is folded into the exponent:
  // p = 2^(c s - m) with c = scale * log2(e) > 0 (a negative scale flips the
  // sign bits of q, which is exact; a zero scale becomes a tiny positive one
  // so masked keys stay at -inf), so the row max is taken over raw scores.
  float c = P.scale_log2;
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int rt = 0; rt < kPfRT; ++rt)
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) qb[rt][cc] ^= u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, 1e-30f);

  const u32x4_t ones_f16 = u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  const u32x4_t ones_bf16 = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  // MASKED: the stage holds keys past some row's causal limit, past the
  // context or past the key window; every other stage skips all mask work
  auto compute_stage = [&](auto masked_tag, int st, const u32x4_t* kbuf, const u32x4_t* vbuf, int slot) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = st * kStageBlocks * kBlockTokens;
    const int nvalid = min(kStageBlocks, nkb - st * kStageBlocks);  // blocks of this stage in the key window
    // ---- raw scores of the stage's 4 blocks for both row tiles
    f32x4_t sc[kPfRT][kStageBlocks];
    auto scores = [&]() {
#pragma unroll
      for (int b = 0; b < kStageBlocks; ++b) {
        u32x4_t kf[DC];
#pragma unroll
        for (int cc = 0; cc < DC; ++cc) kf[cc] = kbuf[b * (kTileElems / 8) + cc * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < kPfRT; ++rt) {
          f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int cc = 0; cc < DC; ++cc) acc = Mfma<T>::k32(kf[cc], qb[rt][cc], acc);
          if constexpr (MASKED) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = k0 + b * kBlockTokens + 4 * quad + r;
              acc[r] = (key <= last[rt] && b < nvalid) ? acc[r] : -INFINITY;
            }
          }
          sc[rt][b] = acc;
        }
      }
    };
    // ---- P of pair pr: 8 values per lane and row tile = tokens 4 quad +
    // 0..3 of the pair's first block, then of its second (the k order of
    // the V operands)
    auto probabilities = [&](int pr, float (&pv)[kPfRT][8]) {
#pragma unroll
      for (int rt = 0; rt < kPfRT; ++rt) {
        const float neg_m = kPOffset - m[rt];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[rt][e] = fast_exp2(fmaf(sc[rt][2 * pr + e / 4][e % 4], c, neg_m));
      }
    };
    scores();
    // ---- one reference-max check per stage: the max moves only past a 2^8
    // margin (rare after the first stage), so the accumulator rescale is
    // mostly skipped and the rest of the stage is straight-line code
    float bm[kPfRT];
    bool grow_any = false;
#pragma unroll
    for (int rt = 0; rt < kPfRT; ++rt) {
      float v = -INFINITY;
#pragma unroll
      for (int b = 0; b < kStageBlocks; ++b)
        v = vmax(v, vmax(vmax(sc[rt][b][0], sc[rt][b][1]), vmax(sc[rt][b][2], sc[rt][b][3])));
      bm[rt] = quad_vmax(v) * c;
      grow_any |= bm[rt] > m[rt] + 8.f;
    }
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
      for (int rt = 0; rt < kPfRT; ++rt) {
        const float mn = bm[rt] > m[rt] + 8.f ? bm[rt] : m[rt];
        const float alpha = fast_exp2(m[rt] - mn);
        lacc[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] *= alpha;
        m[rt] = mn;
      }
    }
    // ---- O^T += V^T P^T and l += 1 P^T over each pair of blocks (K = 32)
    auto pair_masks = [&](int pr, uint32_t (&mk)[4]) {
      mk[0] = mk[1] = mk[2] = mk[3] = ~0u;
      if constexpr (MASKED) {
        // blocks outside the window and slots past the context may hold
        // anything (NaN included): zero them so 0 * garbage never reaches o
        const int t0 = k0 + 4 * quad;
        const int b0 = 2 * pr, b1 = 2 * pr + 1;
        const int e0 = b0 < nvalid ? ctx - (t0 + b0 * kBlockTokens) : 0;  // valid tokens of the quad
        const int e1 = b1 < nvalid ? ctx - (t0 + b1 * kBlockTokens) : 0;
        mk[0] = (e0 > 0 ? 0x0000FFFFu : 0u) | (e0 > 1 ? 0xFFFF0000u : 0u);
        mk[1] = (e0 > 2 ? 0x0000FFFFu : 0u) | (e0 > 3 ? 0xFFFF0000u : 0u);
        mk[2] = (e1 > 0 ? 0x0000FFFFu : 0u) | (e1 > 1 ? 0xFFFF0000u : 0u);
        mk[3] = (e1 > 2 ? 0x0000FFFFu : 0u) | (e1 > 3 ? 0xFFFF0000u : 0u);
      }
    };
#pragma unroll
    for (int pr = 0; pr < kStageBlocks / 2; ++pr) {
      float pv[kPfRT][8];
      probabilities(pr, pv);
      uint32_t mk[4];
      pair_masks(pr, mk);
      const u32x4_t* vop = vbuf + pr * NT * 64 + lane;
      bool keep0 = false, keep1 = false;
      if constexpr (kBf16) {
        keep0 = __builtin_amdgcn_readfirstlane(s_vkeep[slot][2 * pr]) != 0;
        keep1 = __builtin_amdgcn_readfirstlane(s_vkeep[slot][2 * pr + 1]) != 0;
      }
      if (!keep0 && !keep1) {
        // P in fp16, one product per operand
        u32x4_t ph[kPfRT];
#pragma unroll
        for (int rt = 0; rt < kPfRT; ++rt) {
          ph[rt] = u32x4_t{f16x2_rne(pv[rt][0], pv[rt][1]), f16x2_rne(pv[rt][2], pv[rt][3]),
                           f16x2_rne(pv[rt][4], pv[rt][5]), f16x2_rne(pv[rt][6], pv[rt][7])};
          lacc[rt] = Mfma<F16>::k32(ones_f16, ph[rt], lacc[rt]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x4_t av = vop[t * 64];
          if constexpr (MASKED) av = av & u32x4_t{mk[0], mk[1], mk[2], mk[3]};
#pragma unroll
          for (int rt = 0; rt < kPfRT; ++rt) o[rt][t] = Mfma<F16>::k32(av, ph[rt], o[rt][t]);
        }
      } else if constexpr (kBf16) {
        // a block of the pair holds V beyond fp16: the pair runs in bf16
        // with P split hi + lo (fp16 halves go back to bf16, exactly)
        u32x4_t ph[kPfRT], pl[kPfRT];
#pragma unroll
        for (int rt = 0; rt < kPfRT; ++rt) {
          uint16_t hi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hi[e] = Bf16::from_float(pv[rt][e]);
            lo[e] = Bf16::from_float(pv[rt][e] - Bf16::to_float(hi[e]));
          }
          ph[rt] = u32x4_t{pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(hi[4], hi[5]), pack2(hi[6], hi[7])};
          pl[rt] = u32x4_t{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]), pack2(lo[6], lo[7])};
          lacc[rt] = Mfma<Bf16>::k32(ones_bf16, ph[rt], lacc[rt]);
          lacc[rt] = Mfma<Bf16>::k32(ones_bf16, pl[rt], lacc[rt]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x4_t av = vop[t * 64];
          if (!keep0) {
            av[0] = f16x2_to_bf16x2(av[0]);
            av[1] = f16x2_to_bf16x2(av[1]);
          }
          if (!keep1) {
            av[2] = f16x2_to_bf16x2(av[2]);
            av[3] = f16x2_to_bf16x2(av[3]);
          }
          if constexpr (MASKED) av = av & u32x4_t{mk[0], mk[1], mk[2], mk[3]};
#pragma unroll
          for (int rt = 0; rt < kPfRT; ++rt) {
            o[rt][t] = Mfma<Bf16>::k32(av, ph[rt], o[rt][t]);
            o[rt][t] = Mfma<Bf16>::k32(av, pl[rt], o[rt][t]);
          }
        }
      }
    }
  };
  // Stages wholly below every row's causal limit and inside the key window
  // (all but the last few) need no masks: they run double-buffered, the next
  // stage loading while this one computes.  The masked tail runs one stage at
  // a time.
  const int nst_plain = min(nst, (first_masked + 1) / (kStageBlocks * kBlockTokens));
  auto refill_table_for = [&](int st) {
    // keep the table window over the blocks of stage st (it only moves
    // forward; the check both ways keeps a stale window from being read)
    if (st * kStageBlocks < tab_base || (st + 1) * kStageBlocks - tab_base > kTabWindow) {
      __syncthreads();
      tab_base = st * kStageBlocks;
      fill_table(tab_base);
      __syncthreads();
    }
  };
  if (threadIdx.x == 0) s_bad = 0;
  fill_table(0);
  __syncthreads();
  if (nst_plain > 0) {
    issue_stage(0, s_k0);
    wait_loads();
    commit_v(s_v0, 0);
    __syncthreads();
  }
  // two stages per iteration so each buffer has a fixed name (the compiler
  // then knows the loads into one never alias reads of the other)
  for (int st = 0; st < nst_plain; st += 2) {
    const bool next1 = st + 1 < nst_plain;
    if (next1) {
      refill_table_for(st + 1);
      issue_stage(st + 1, s_k1);
    }
    compute_stage(std::false_type{}, st, s_k0, s_v0, 0);
    wait_loads();
    if (next1) commit_v(s_v1, 1);
    __syncthreads();
    if (!next1) break;
    const bool next2 = st + 2 < nst_plain;
    if (next2) {
      refill_table_for(st + 2);
      issue_stage(st + 2, s_k0);
    }
    compute_stage(std::false_type{}, st + 1, s_k1, s_v1, 1);
    wait_loads();
    if (next2) commit_v(s_v0, 0);
    __syncthreads();
  }
  for (int st = nst_plain; st < nst; ++st) {
    refill_table_for(st);
    issue_stage(st, s_k0);
    wait_loads();
    commit_v(s_v0, 0);
    __syncthreads();
    compute_stage(std::true_type{}, st, s_k0, s_v0, 0);
    __syncthreads();
  }

  // an out-of-pool table entry seen by any wave poisons every row
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;
#pragma unroll
  for (int rt = 0; rt < kPfRT; ++rt) {
    if (!live[rt]) continue;
    const int row = row_wg0 + (w * kPfRT + rt) * 16 + n;
    const int i = row / G, hh = row - i * G;
    const int64_t obase = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D;
    const float inv = any_bad ? __builtin_nanf("") : 1.f / lacc[rt][0];
#pragma unroll
    for (int t = 0; t < NT; ++t) store_row4<T, OUT_F32>(P.out, obase + 16 * t + 4 * quad, o[rt][t] * inv);
  }
}

template <typename T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, const PParams& p) {
  constexpr int RT = kPrefillRowTiles, WPE = kPrefillWavesPerSimd;
  constexpr int rows = kPfWaves * RT * 16;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t R = int64_t(a.chunk) * G;
  const int tiles = int((R + rows - 1) / rows);
  const int pairs = a.num_seqs * a.num_kv_heads;  // the caller bounds tiles x pairs by INT32_MAX
  const dim3 grid(unsigned(int64_t(tiles) * pairs));
  if (a.out_f32) {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, true, RT, WPE>), grid, dim3(kPfThreads), 0, a.stream, p, tiles, pairs);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, false, RT, WPE>), grid, dim3(kPfThreads), 0, a.stream, p, tiles,
                       pairs);
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
  p.tile_shift = a.tile_shift;
  if (a.dtype == PA_BF16) return a.head_dim == 64 ? launch_prefill_t<Bf16, 64>(a, p) : launch_prefill_t<Bf16, 128>(a, p);
  return a.head_dim == 64 ? launch_prefill_t<F16, 64>(a, p) : launch_prefill_t<F16, 128>(a, p);
}

}  // namespace pa
