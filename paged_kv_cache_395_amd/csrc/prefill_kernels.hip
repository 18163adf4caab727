// Chunked prefill over the paged cache for gfx950 (matrix cores).
//
// A chunk of C new queries per sequence sits at the last C positions of its
// context; query i attends keys 0 .. ctx - C + i (causal).  K/V are reached
// through the block table exactly as in decode ("PagedAttention: How vLLM
// Serves AI Like an Operating System", section "PagedAttention: Virtual
// Memory for KV Cache").
//
// Work split: rows are (query i, head n of the kv group), row = i * G + n.
// One workgroup of 8 waves per CU owns 256 consecutive rows (2 tiles of 16
// per wave) of one (kv head, sequence) and walks the keys in stages of 64
// (4 blocks).  Waves 0-3 fetch the stage: K straight into LDS, V raw into
// LDS (16-byte direct-to-LDS loads), one block per wave, double-buffered so
// the next stage loads while this one computes.  The V tiles are then
// converted to fp16 and stored in LDS in the A-operand layout of the PV
// product (the two blocks of a pair side by side in each lane's 16 bytes),
// so each operand is one 16-byte LDS read and each value is converted once
// per 256 rows.
// Products are written transposed as in decode, all on the 16x16x32
// matrix instructions (the 16x16x16 forms run at half their rate):
//   S^T[token][row] = K . Q^T                      (per 16-token block)
//   O^T[dim][row]  += V^T . P^T                    (per pair of blocks, K = 32)
//   l[row]         += 1 . P^T                      (the row sums, same P)
// P is carried in fp16 (11 significant bits); the row sums are taken from
// the same rounded P, so a weight's rounding changes numerator and
// denominator together.  bf16 V is exact in fp16 below 2^16 in magnitude
// (values under 2^-17 lose low bits, an absolute error below 2^-24).  A
// workgroup's key loop first runs with every V run in fp16; if a run held
// anything larger, or a NaN, inside the context, the loop runs again on the
// exact path, where such a run keeps its bf16 bits and the pair of blocks it
// belongs to runs in bf16 with each weight split exactly into hi + lo bf16
// halves instead.  The grid is one-dimensional and XCD-aware:
// all row tiles of one (sequence, kv head) run on one XCD, so their shared
// K / V stream is fetched from HBM once into that XCD's L2.

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

constexpr int kStageBlocks = 4;                        // 16-token blocks per stage
constexpr int kXcds = 8;

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
// (only the halves `valid` keeps count toward big: slots past the context
// are never read, whatever they hold)
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t x, uint32_t valid, float& big) {
  const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xFFFF0000u);
  const uint32_t xv = x & valid;
  big = vmax(big, vmax(__builtin_fabsf(__uint_as_float(xv << 16)), __builtin_fabsf(__uint_as_float(xv & 0xFFFF0000u))));
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
// a weight from here up means the reference fell more than 8 below a score
constexpr float kPOverflow = 32768.f;
// The reference before any key: below every finite score, yet finite, so a
// masked key's weight 2^(-inf - m) is exactly 0 (with m = -inf it would be
// NaN and hide the first stage's overflow) and every other weight is +inf.
constexpr float kMStart = -3.40282347e38f;

// Whether any of the 2 x 8 fp16 values reaches `limit` (a NaN among them
// hides the others: the max propagates it)
__device__ inline bool f16_words_reach(const u32x4_t (&w)[2], float limit) {
  typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h8_t a = __builtin_elementwise_maximum(__builtin_bit_cast(h8_t, w[0]), __builtin_bit_cast(h8_t, w[1]));
  const h4_t b = __builtin_elementwise_maximum(__builtin_shufflevector(a, a, 0, 1, 2, 3),
                                               __builtin_shufflevector(a, a, 4, 5, 6, 7));
  const h2_t d = __builtin_elementwise_maximum(__builtin_shufflevector(b, b, 0, 1), __builtin_shufflevector(b, b, 2, 3));
  return float(__builtin_elementwise_maximum(d.x, d.y)) >= limit;
}
// bf16 magnitudes from here up do not fit fp16; a tile holding one (or a
// NaN) keeps its bf16 bits
constexpr float kF16Limit = 65536.f;

// ---------------------------------------------------------------------------
// Ping-pong form: one workgroup of 8 waves per CU owns 256 rows; waves 0-3
// (group 0) and 4-7 (group 1) own 128 of them each.  Every wave runs the same
// sequence per stage k, a matrix phase M(k) = PV(k-1) + QK(k) and a VALU
// phase S(k) (row max, reference check and rescale, P in fp16, and the
// conversion of a share of V), separated by workgroup barriers; group 1 runs
// one phase behind group 0 (it passes one barrier first, group 0 one last),
// so each SIMD always has one wave in its products and one in its vector
// work (the hardware overlaps the two across waves, not within one wave's
// instruction stream).  Group 0 fetches stage k+1 (K straight into LDS, V raw
// into LDS) at the start of M(k) and waits for it at the end of S(k); S(j) of
// group h converts its half of V(j + h) into the operand buffer.  K, raw V
// and V operands are double-buffered.  The masked tail runs afterwards, both
// groups in step.
// ---------------------------------------------------------------------------
constexpr int kPpWaves = 8;
constexpr int kPpThreads = kPpWaves * kWave;
constexpr int kPpRowTiles = 2;  // 16-row tiles per wave

template <typename T, int D, bool OUT_F32>
__global__ void __launch_bounds__(kPpThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_mfma_kernel(PParams P, int tiles_per_pair, int num_pairs) {
  constexpr bool kBf16 = std::is_same<T, Bf16>::value;
  constexpr int RT = kPpRowTiles;
  constexpr int kRows = kPpWaves * RT * 16;  // rows per workgroup
  constexpr int DC = D / 32;                  // 16-byte chunks per lane per tile
  constexpr int NT = D / 16;                  // 16-dim output tiles
  constexpr int kTileElems = kBlockTokens * D;
  constexpr int kTileBytes = kTileElems * 2;
  constexpr int kRuns = kTileBytes / 1024;    // 1 KiB wave loads per tile
  constexpr int kRunsPerWave = kRuns / 2;     // each group converts half of a block's runs
  static_assert(kRuns == DC && kRunsPerWave >= 1, "one 16-byte chunk per lane per run, two waves per block");
  static_assert(2 * kStageBlocks == kPpWaves, "a block per wave of a group");
  constexpr int kStageU4 = kStageBlocks * kTileElems / 8;  // u32x4 per stage buffer

  __shared__ u32x4_t s_k0[kStageU4];
  __shared__ u32x4_t s_k1[kStageU4];
  __shared__ u32x4_t s_r0[kStageU4];  // raw V tiles
  __shared__ u32x4_t s_r1[kStageU4];
  // V operands: [pair][output tile t][lane] 16 bytes = the lane's 4 tokens
  // of dim 16 t + (lane % 16) in the pair's first block, then in its second
  __shared__ u32x4_t s_o0[kStageU4];
  __shared__ u32x4_t s_o1[kStageU4];
  // per operand buffer, byte 2 b + h set = the runs of block b converted by
  // group h kept their bf16 bits (word pr covers the blocks of pair pr)
  __shared__ uint32_t s_keep[2][2];
  __shared__ int s_bad;
  __shared__ int s_fallback;  // some V value of the workgroup's keys needs its bf16 bits

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
  const int grp = w >> 2;
  const int n = lane & 15, quad = lane >> 4;
  const int G = P.hq / P.hkv;
  const int C = P.chunk;
  const int R = C * G;
  const int ctx = P.ctxs[s];
  const int row_wg0 = tile * kRows;
  if (row_wg0 >= R) return;

  if (ctx < C || ctx > P.max_ctx || int64_t(ctx) > (int64_t(P.max_blocks) * kBlockTokens << P.tile_shift)) {
    const float nan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < kRows * D; idx += kPpThreads) {
      const int row = row_wg0 + idx / D, d = idx % D;
      if (row >= R) break;
      const int i = row / G, hh = row - i * G;
      const int64_t o = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D + d;
      if constexpr (OUT_F32) static_cast<float*>(P.out)[o] = nan;
      else static_cast<uint16_t*>(P.out)[o] = T::from_float(nan);
    }
    return;
  }

  int last[RT];
  bool live[RT];
  u32x4_t qb[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row_wg0 + (w * RT + rt) * 16 + n;
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
  // wait lands at their first use inside the key loop, where it counts the
  // next stage's tile loads too and every stage then waits for its
  // successor's tiles before its first product.
  wait_loads();
  const int row_wg_last = min(R, row_wg0 + kRows) - 1;
  const int first_masked = ctx - C + row_wg0 / G;
  const int nkb = (ctx - C + row_wg_last / G) / kBlockTokens + 1;
  const int nst = (nkb + kStageBlocks - 1) / kStageBlocks;
  const int32_t* trow = P.tables + int64_t(s) * P.max_blocks;
  const int sh = P.tile_shift;
  const int64_t blk_stride = (int64_t(P.hkv) << sh) * kTileElems;
  const char* kg = reinterpret_cast<const char*>(P.k + (int64_t(g) << sh) * kTileElems);
  const char* vg = reinterpret_cast<const char*>(P.v + (int64_t(g) << sh) * kTileElems);

  float m[RT];
  f32x4_t lacc[RT];
  f32x4_t o[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kMStart;
    lacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) o[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  int bad = 0;

  // Table entry (physical block) of this wave's block of stage st (a block
  // of 2^sh tiles repeats its entry); -1 past the key window.  It is a
  // vector load: the main loop loads it a stage ahead and reads it into a
  // scalar only when it issues that stage, so its wait never covers the
  // tile loads issued just before it.
  const int my_blk = w & 3;
  auto load_entry = [&](int st) __attribute__((always_inline)) {
    const int blk = st * kStageBlocks + my_blk;
    return blk < nkb ? trow[blk >> sh] : -1;
  };
  auto lookup = [&](int st) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(load_entry(st)); };
  // Fetch runs [r0, r0 + nr) of block my_blk of stage st, K and raw V,
  // straight into LDS (one buffer resource per tile; a block past the key
  // window or outside the pool gets an empty range and reads as zeros).
  const int lane_off = lane * 16;
  auto issue_runs = [&](int st, int phys, u32x4_t* kbuf, u32x4_t* rbuf, int r0, auto nr_tag)
      __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_tag)::value;
    const int blk = st * kStageBlocks + my_blk;
    const bool in_pool = phys >= 0 && int64_t(phys) < P.num_blocks;
    bad |= blk < nkb && !in_pool;
    const bool ok = blk < nkb && in_pool;
    const int64_t off = ok ? (int64_t(phys) * blk_stride + int64_t(blk & ((1 << sh) - 1)) * kTileElems) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg + off), 0,
                                                                        ok ? kTileBytes : 0, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg + off), 0,
                                                                        ok ? kTileBytes : 0, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int part = r0 + i;
      lds_void* dk = (lds_void*)(kbuf + my_blk * (kTileElems / 8) + part * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dk, 16, lane_off, part * 1024, 0, 0);
      lds_void* dv = (lds_void*)(rbuf + my_blk * (kTileElems / 8) + part * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dv, 16, lane_off, part * 1024, 0, 0);
    }
  };

  // Group grp's runs of block my_blk, raw V to the operand buffer, as fp16
  // when every value converts exactly.  Run cc of a V tile holds, for lane
  // (quad, n), tokens 4 quad + 0..3 of dim 32 cc + n (first 8 bytes) and of
  // dim 32 cc + 16 + n (last 8 bytes): the lane's part of output tiles 2 cc
  // and 2 cc + 1, stored beside the paired block's part.
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
  const int run0 = grp * kRunsPerWave;
  // On the fast pass the conversion is stored as it is and only reported
  // (the pass is redone if any run needed its bf16 bits); the exact pass
  // keeps such runs raw and records them per operand buffer for PV.
  // In the masked tail `ntok` is the number of block my_blk's tokens inside
  // the context: lane (quad, n)'s word j holds tokens 4 quad + 2 (j % 2) and
  // the next one.
  auto convert_own = [&](const u32x4_t* rbuf, u32x4_t* obuf, int slot, auto slow_tag, auto masked_tag, int ntok)
      __attribute__((always_inline)) {
    constexpr bool SLOW = decltype(slow_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    uint32_t valid[2] = {~0u, ~0u};
    if constexpr (MASKED) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 4 * quad + 2 * h;
        valid[h] = (t < ntok ? 0x0000FFFFu : 0u) | (t + 1 < ntok ? 0xFFFF0000u : 0u);
      }
    }
    u32x2_t* dst = reinterpret_cast<u32x2_t*>(obuf) + ((my_blk >> 1) * NT * 64 + lane) * 2 + (my_blk & 1);
    u32x4_t x[kRunsPerWave], y[kRunsPerWave];
#pragma unroll
    for (int i = 0; i < kRunsPerWave; ++i) x[i] = rbuf[my_blk * (kTileElems / 8) + (run0 + i) * 64 + lane];
    bool keep = false;
    if constexpr (kBf16) {
      float big = 0.f;
#pragma unroll
      for (int i = 0; i < kRunsPerWave; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) y[i][j] = bf16x2_to_f16x2(x[i][j], valid[j % 2], big);
      keep = __builtin_amdgcn_ballot_w64(!(big < kF16Limit)) != 0;
      if constexpr (SLOW) {
        if (keep) {
#pragma unroll
          for (int i = 0; i < kRunsPerWave; ++i) y[i] = x[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRunsPerWave; ++i) y[i] = x[i];
    }
#pragma unroll
    for (int i = 0; i < kRunsPerWave; ++i) {
      const int cc = run0 + i;
      dst[(2 * cc) * 64 * 2] = u32x2_t{y[i][0], y[i][1]};
      dst[(2 * cc + 1) * 64 * 2] = u32x2_t{y[i][2], y[i][3]};
    }
    if constexpr (SLOW) {
      if (lane == 0) reinterpret_cast<uint8_t*>(s_keep[slot])[my_blk * 2 + grp] = keep;
    }
    return keep;
  };

  float c = P.scale_log2;
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) qb[rt][cc] ^= u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, 1e-30f);
  const u32x4_t ones_f16 = u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};

  // ---- QK of stage st: raw scores, -inf outside the causal / context window
  auto qk = [&](auto masked_tag, int st, const u32x4_t* kbuf, f32x4_t (&sc)[RT][kStageBlocks])
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = st * kStageBlocks * kBlockTokens;
    const int nvalid = min(kStageBlocks, nkb - st * kStageBlocks);
#pragma unroll
    for (int b = 0; b < kStageBlocks; ++b) {
      u32x4_t kf[DC];
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) kf[cc] = kbuf[b * (kTileElems / 8) + cc * 64 + lane];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
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
  // ---- S: row max, reference check and rescale, P in fp16 (8 values per
  // lane, row tile and pair: tokens 4 quad + 0..3 of the pair's first block,
  // then of its second)
  // The weights are formed first at the current reference; only when one of
  // them reaches 2^15 (a score more than ~8 above the reference, or any key
  // at the starting reference) is the row max taken, the reference moved and
  // P formed again.  Without such a weight every P < 2^15 fits fp16, and
  // with one the same rule as an up-front max check applies, so the result
  // is that of checking the max first.  Only a NaN score (from NaN or
  // infinite inputs) makes a NaN weight, and it hides only its own row's
  // weights from the check (that row's output is NaN either way).
  auto softmax = [&](const f32x4_t (&sc)[RT][kStageBlocks], u32x4_t (&ph)[RT][kStageBlocks / 2])
      __attribute__((always_inline)) {
    auto weights = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float neg_m = kPOffset - m[rt];
#pragma unroll
        for (int pr = 0; pr < kStageBlocks / 2; ++pr) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(sc[rt][2 * pr + j / 4][j % 4], c, neg_m));
          ph[rt][pr] = u32x4_t{f16x2_rne(e[0], e[1]), f16x2_rne(e[2], e[3]), f16x2_rne(e[4], e[5]), f16x2_rne(e[6], e[7])};
        }
      }
    };
    weights();
    bool over = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) over |= f16_words_reach(ph[rt], kPOverflow);
    if (__builtin_amdgcn_ballot_w64(over)) {
      float bm[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float v = -INFINITY;
#pragma unroll
        for (int b = 0; b < kStageBlocks; ++b)
          v = vmax(v, vmax(vmax(sc[rt][b][0], sc[rt][b][1]), vmax(sc[rt][b][2], sc[rt][b][3])));
        bm[rt] = quad_vmax(v) * c;
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mn = bm[rt] > m[rt] + 8.f ? bm[rt] : m[rt];
        const float alpha = fast_exp2(m[rt] - mn);
        lacc[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] *= alpha;
        m[rt] = mn;
      }
      weights();
    }
  };
  // ---- PV of stage st: O^T += V^T P^T and l += 1 P^T per pair (K = 32)
  auto pv = [&](auto masked_tag, int st, const u32x4_t* obuf, int slot, const u32x4_t (&ph)[RT][kStageBlocks / 2],
                auto slow_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool SLOW = decltype(slow_tag)::value;  // the pass that honours kept bf16 runs
#pragma unroll
    for (int pr = 0; pr < kStageBlocks / 2; ++pr) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) lacc[rt] = Mfma<F16>::k32(ones_f16, ph[rt][pr], lacc[rt]);
      uint32_t mk[4] = {~0u, ~0u, ~0u, ~0u};
      if constexpr (MASKED) {
        const int k0 = st * kStageBlocks * kBlockTokens;
        const int nvalid = min(kStageBlocks, nkb - st * kStageBlocks);
        const int t0 = k0 + 4 * quad;
        const int b0 = 2 * pr, b1 = 2 * pr + 1;
        const int e0 = b0 < nvalid ? ctx - (t0 + b0 * kBlockTokens) : 0;
        const int e1 = b1 < nvalid ? ctx - (t0 + b1 * kBlockTokens) : 0;
        mk[0] = (e0 > 0 ? 0x0000FFFFu : 0u) | (e0 > 1 ? 0xFFFF0000u : 0u);
        mk[1] = (e0 > 2 ? 0x0000FFFFu : 0u) | (e0 > 3 ? 0xFFFF0000u : 0u);
        mk[2] = (e1 > 0 ? 0x0000FFFFu : 0u) | (e1 > 1 ? 0xFFFF0000u : 0u);
        mk[3] = (e1 > 2 ? 0x0000FFFFu : 0u) | (e1 > 3 ? 0xFFFF0000u : 0u);
      }
      const u32x4_t* vop = obuf + pr * NT * 64 + lane;
      uint32_t keep = 0;
      if constexpr (kBf16 && SLOW) keep = __builtin_amdgcn_readfirstlane(s_keep[slot][pr]);
      if (keep == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x4_t av = vop[t * 64];
          if constexpr (MASKED) av = av & u32x4_t{mk[0], mk[1], mk[2], mk[3]};
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) o[rt][t] = Mfma<F16>::k32(av, ph[rt][pr], o[rt][t]);
        }
      } else if constexpr (kBf16 && SLOW) {
        // V of the pair partly kept in bf16: the pair runs in bf16 with each
        // fp16 weight split exactly into hi + lo bf16 halves (one row tile at
        // a time: this rare path must not hold more registers than the
        // common one)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          u32x4_t phi, plo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t x = ph[rt][pr][j];
            const float a = F16::to_float(uint16_t(x)), b = F16::to_float(uint16_t(x >> 16));
            const uint16_t ha = Bf16::from_float(a), hb = Bf16::from_float(b);
            phi[j] = pack2(ha, hb);
            plo[j] = pack2(Bf16::from_float(a - Bf16::to_float(ha)), Bf16::from_float(b - Bf16::to_float(hb)));
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t av = vop[t * 64];
            const int h = (t / 2) / kRunsPerWave;  // group that converted run t / 2
            if (!((keep >> (8 * h)) & 0xFFu)) {
              av[0] = f16x2_to_bf16x2(av[0]);
              av[1] = f16x2_to_bf16x2(av[1]);
            }
            if (!((keep >> (8 * (2 + h))) & 0xFFu)) {
              av[2] = f16x2_to_bf16x2(av[2]);
              av[3] = f16x2_to_bf16x2(av[3]);
            }
            if constexpr (MASKED) av = av & u32x4_t{mk[0], mk[1], mk[2], mk[3]};
            o[rt][t] = Mfma<Bf16>::k32(av, phi, o[rt][t]);
            o[rt][t] = Mfma<Bf16>::k32(av, plo, o[rt][t]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };

  if (threadIdx.x == 0) {
    s_bad = 0;
    s_fallback = 0;
  }
  // The key loop.  The fast pass takes every V run as fp16 (no per-pair
  // branch in the matrix phase, so both pairs' products share one block);
  // a run whose values need their bf16 bits (beyond fp16's range, or a NaN)
  // flags the workgroup, which then runs the loop again on the exact path.
  auto run = [&](auto slow_tag) __attribute__((always_inline)) {
    bool fb = false;  // this wave converted a run that needs its bf16 bits
    const int K = min(nst, (first_masked + 1) / (kStageBlocks * kBlockTokens));  // plain stages
    f32x4_t sc[RT][kStageBlocks];
    u32x4_t ph[RT][kStageBlocks / 2];
    int entry_next = 0;  // group 0: table entry of the stage it fetches next
    if (K > 0) {
      if (grp == 0) {
        issue_runs(0, lookup(0), s_k0, s_r0, 0, std::integral_constant<int, kRuns>{});
        if (K > 1) entry_next = load_entry(1);
        wait_loads();
      }
      __syncthreads();
      if (grp == 1) {
        fb |= convert_own(s_r0, s_o0, 0, slow_tag, std::false_type{}, 0);  // group 1's share of V(0), in the phase group 0 spends on M(0)
        __syncthreads();
      }
    }
    // One stage: M(k), barrier, S(k), barrier.  Stage k uses buffers k % 2
    // (fixed names per half of the loop body, so the compiler sees the loads
    // into one never alias reads of the other).
    auto stage = [&](int k, const u32x4_t* kb, const u32x4_t* ob_prev, int slot_prev, u32x4_t* kb_next,
                     u32x4_t* rb_next, const u32x4_t* rb, u32x4_t* ob, int slot, u32x4_t* ob_next, int slot_next)
        __attribute__((always_inline)) {
      if (grp == 0 && k + 1 < K) {
        issue_runs(k + 1, __builtin_amdgcn_readfirstlane(entry_next), kb_next, rb_next, 0,
                   std::integral_constant<int, kRuns>{});
        if (k + 2 < K) entry_next = load_entry(k + 2);
      }
      if (k > 0) pv(std::false_type{}, k - 1, ob_prev, slot_prev, ph, slow_tag);
      qk(std::false_type{}, k, kb, sc);
      __syncthreads();
      softmax(sc, ph);
      if (grp == 0) {
        fb |= convert_own(rb, ob, slot, slow_tag, std::false_type{}, 0);  // V(k)
        wait_loads();               // stage k + 1
      } else if (k + 1 < K) {
        fb |= convert_own(rb_next, ob_next, slot_next, slow_tag, std::false_type{}, 0);  // V(k + 1)
      }
      __syncthreads();
    };
    for (int k = 0; k < K; k += 2) {
      stage(k, s_k0, s_o1, 1, s_k1, s_r1, s_r0, s_o0, 0, s_o1, 1);
      if (k + 1 >= K) break;
      stage(k + 1, s_k1, s_o0, 0, s_k0, s_r0, s_r1, s_o1, 1, s_o0, 0);
    }
    if (K > 0) {
      // M(K): PV of the last plain stage; then the two groups meet again
      if ((K - 1) % 2 == 0) pv(std::false_type{}, K - 1, s_o0, 0, ph, slow_tag);
      else pv(std::false_type{}, K - 1, s_o1, 1, ph, slow_tag);
      if (grp == 0) __syncthreads();
      __syncthreads();
    }
    // masked tail: both groups in step, each wave fetching half a block
    for (int st = K; st < nst; ++st) {
      issue_runs(st, lookup(st), s_k0, s_r0, run0, std::integral_constant<int, kRunsPerWave>{});
      wait_loads();
      __syncthreads();
      fb |= convert_own(s_r0, s_o0, 0, slow_tag, std::true_type{}, ctx - (st * kStageBlocks + my_blk) * kBlockTokens);
      __syncthreads();
      f32x4_t scm[RT][kStageBlocks];
      u32x4_t phm[RT][kStageBlocks / 2];
      qk(std::true_type{}, st, s_k0, scm);
      softmax(scm, phm);
      pv(std::true_type{}, st, s_o0, 0, phm, slow_tag);
      __syncthreads();
    }
    if (fb && lane == 0) s_fallback = 1;
  };
  run(std::false_type{});
  if constexpr (kBf16) {
    __syncthreads();  // every wave has reported: the flag is final
    if (s_fallback) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        m[rt] = kMStart;
        lacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      run(std::true_type{});
    }
  }

  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (!live[rt]) continue;
    const int row = row_wg0 + (w * RT + rt) * 16 + n;
    const int i = row / G, hh = row - i * G;
    const int64_t obase = ((int64_t(s) * C + i) * P.hq + int64_t(g) * G + hh) * D;
    const float inv = any_bad ? __builtin_nanf("") : 1.f / lacc[rt][0];
#pragma unroll
    for (int t = 0; t < NT; ++t) store_row4<T, OUT_F32>(P.out, obase + 16 * t + 4 * quad, o[rt][t] * inv);
  }
}

template <typename T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, const PParams& p) {
  constexpr int rows = kPpWaves * kPpRowTiles * 16;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t R = int64_t(a.chunk) * G;
  const int tiles = int((R + rows - 1) / rows);
  const int pairs = a.num_seqs * a.num_kv_heads;  // the caller bounds tiles x pairs by INT32_MAX
  const dim3 grid(unsigned(int64_t(tiles) * pairs));
  if (a.out_f32) {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, true>), grid, dim3(kPpThreads), 0, a.stream, p, tiles, pairs);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, D, false>), grid, dim3(kPpThreads), 0, a.stream, p, tiles, pairs);
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
