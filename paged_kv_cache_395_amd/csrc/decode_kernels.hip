// Paged decode attention for gfx950.
//
// out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s, where K_s / V_s are the
// context's K and V rows reached through the sequence's block table: logical
// block i of a sequence is physical block table[s][i], and blocks sit
// anywhere in the pool ("PagedAttention: How vLLM Serves AI Like an
// Operating System", section "PagedAttention: Virtual Memory for KV Cache").
// Paging moves data, not results ("Throughput Impact: The Numbers"): the
// output equals contiguous attention up to floating-point order.
//
// Work split: one workgroup (4 waves) per (kv head, sequence, context
// partition).  Each wave walks every 4th 16-token block of the partition,
// keeps an online softmax (reference max in the exp2 domain, running sum,
// accumulator), and the 4 waves merge in LDS.  A sequence that fits one
// partition writes its output row directly; longer ones leave (accumulator,
// max, sum) partials that the reduce kernel merges by log-sum-exp in a fixed
// order, so results are deterministic.
//
// fp16 / bf16 run on the matrix cores.  All G = Hq / Hkv query heads of a kv
// head share each K/V tile, so every tile is read from HBM once:
//   S^T[token][head] = K[token][:] . Q[head][:]     (16x16x32, K tile = A)
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]   (16x16x16)
// Writing both products transposed puts the 16 (padded) query heads on the
// accumulator column, so a lane holds one head's scores and one head's
// output dims: the softmax rescale needs no data movement.  P is split into
// hi + lo halves of the input type before the PV product so it keeps ~16
// (bf16) / ~22 (fp16) mantissa bits; K, Q and V products are exact in fp32.
// fp32 inputs use the vector ALUs (one workgroup per query head).
//
// Several queries per sequence (verifying C drafted tokens at positions
// ctx - C .. ctx - 1) share each tile the same way: the accumulator columns
// are the G * C (query, head) pairs of the kv group, and column (i, n) sees
// keys up to position ctx - C + i, so G * C <= 16 runs at decode's
// bandwidth with the causal limit applied per column.

#include <math.h>

#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;  // the merges below name the 4 waves' slots explicitly
constexpr int kThreads = kWaves * kWave;
// "no max yet": finite so that 2^(s - m) of a masked score is 0, not NaN
constexpr float kNoMax = -1e30f;
// first word of the workspace header the partition kernels write
constexpr int32_t kWorkspaceMagic = 0x50413031;

struct KParams {
  void* out;
  const uint16_t* q16;
  const float* q32;
  const uint16_t* k16;
  const uint16_t* v16;
  const float* k32;
  const float* v32;
  const int32_t* tables;
  const int32_t* ctxs;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  int64_t num_blocks;
  float scale_log2;
  int32_t max_blocks;
  int32_t hq, hkv, max_ctx, partition, nparts_max;
  int32_t qlen;  // queries per sequence (1: plain decode)
  int32_t num_seqs, head_dim;
  // the merge's bookkeeping in the workspace (null without one): the call's
  // geometry, and per (sequence, kv head) the number of partial slots
  int32_t* ws_hdr;
  int32_t* ws_nseg;
  // log2 of 16-token tiles per block: a (block, kv head) run of the pool is
  // 2^tile_shift consecutive tiles; the table has one entry per block
  int32_t tile_shift;
};

template <typename T, bool OUT_F32>
__device__ inline void store_out(void* out, int64_t idx, float v) {
  if constexpr (OUT_F32) {
    static_cast<float*>(out)[idx] = v;
  } else {
    static_cast<uint16_t*>(out)[idx] = T::from_float(v);
  }
}

// Four consecutive output elements (idx a multiple of 4), stored
// non-temporally: nothing in the kernel reads them back.
template <typename T, bool OUT_F32>
__device__ inline void store_out4(void* out, int64_t idx, f32x4_t v) {
  if constexpr (OUT_F32) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + idx));
  } else {
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
    const u32x2_t p = {pack2(T::from_float(v[0]), T::from_float(v[1])), pack2(T::from_float(v[2]), T::from_float(v[3]))};
    __builtin_nontemporal_store(p, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + idx));
  }
}

// A context length the grid / table cannot cover is a caller error: report it
// as NaN rows instead of reading out of bounds.
__device__ inline bool context_out_of_contract(int ctx, const KParams& P) {
  return ctx < 0 || ctx > P.max_ctx || int64_t(ctx) > (int64_t(P.max_blocks) * kBlockTokens << P.tile_shift);
}

// ------------------------------------------------------------------------
// Matrix-core decode (fp16 / bf16) on a persistent grid.
//
// The batch's work is one stream of 16-token tiles in (sequence, kv head,
// tile) order; each (sequence, kv head) pair's tiles are cut into
// partitions of P.partition tokens.  The grid holds as many workgroups as
// fit on the GPU at once, and workgroup b takes the partitions that start
// in the b-th equal share of the stream, so every workgroup reads the same
// number of tiles to within one partition whatever the mix of context
// lengths.  The partitions of one pair that fall to one workgroup form a
// segment, folded by the online softmax in registers.  A pair split over
// several workgroups leaves one fp32 partial (accumulator, max, sum) per
// segment for the log-sum-exp merge, i.e. about one per workgroup instead
// of one per partition: partials written to HBM in the middle of the read
// stream cost far more than their bytes (with one partial per 512-token
// partition, 16 x 32,768 tokens took 380 us; with the same stores kept in
// one cache-resident region, 321 us).
//
// Inside a segment wave w takes tiles w, w + 4, ...  Its physical block ids
// are read once per window of 64 tiles into one VGPR (lane i = tile i) and
// picked with readlane.  K and V tiles are fetched with buffer loads
// through a per-tile resource whose range is the tile: an index past the
// window gets an empty range, which returns zeros without touching memory,
// so every loop iteration issues the same loads in the same order and the
// compiler's wait counts stay exact (a load under a branch makes it wait
// for all outstanding loads).  The loads are non-temporal: each tile is
// read exactly once.
// ------------------------------------------------------------------------
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, kBufferRsrcWord3);
}

__device__ inline u32x4_t load16_nt(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT));
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// 16-token tiles of one (sequence, kv head) pair that decode reads; 0 for a
// sequence whose rows are written without reading (an empty context, or a
// length outside the contract).
__device__ inline int pair_tiles(int ctx, const KParams& P) {
  if (ctx <= 0 || ctx < P.qlen || context_out_of_contract(ctx, P)) return 0;
  return (ctx + kBlockTokens - 1) / kBlockTokens;
}

// What a segment costs beyond its tiles, in tiles: its start (query and
// table loads, then the first tiles) and its merge are latency nothing else
// in the workgroup hides.  The persistent split weighs every pair by its
// tiles plus this, so a share of many short contexts holds fewer tiles
// (measured on 256 lognormal GQA contexts: 267 us with 0, 254 us with 8, 255
// with 16; 64 x U[128, 2048] MHA contexts: 196, 182, 182; since a segment's
// merge overlaps the next one's start, GQA 254 / 250.5 / 249.3 / 250.6 us
// with 8 / 10 / 12 / 14, four queries per sequence and 16 x 32,768 equal).
constexpr int kSegmentCost = 12;

// Share weights of the persistent split's even and odd workgroups (XCDs).
constexpr int64_t kEvenShareWeight = 25;
constexpr int64_t kOddShareWeight = 23;


// Boundary x of the weighted stream, inside the pair whose weighted range
// starts at a (tiles, nu partitions of ut tiles, the first starting at
// pb = a + kSegmentCost): unchanged, or moved to pb (all of the pair after
// it) or to just past the last partition's start (all of it before).
__device__ inline int64_t snap_boundary(int64_t x, int64_t a, int tiles, int nu, int ut, int snap) {
  const int64_t pb = a + kSegmentCost;
  if (x <= pb) return x;
  const int64_t k = (x - pb + ut - 1) / ut;  // partitions starting before x
  if (k >= nu) return x;
  const int64_t left = k * ut, right = tiles - left;
  if (right <= snap && right <= left) return pb + int64_t(nu - 1) * ut + 1;
  if (left <= snap) return pb;
  return x;
}

// The call's geometry, recorded by the partition kernel for the merge.
__device__ inline void write_header(const KParams& P) {
  int32_t* h = P.ws_hdr;
  h[0] = kWorkspaceMagic;
  h[1] = P.partition;
  h[2] = P.nparts_max;
  h[3] = P.num_seqs * P.qlen;
  h[4] = P.hq;
  h[5] = P.hkv;
  h[6] = P.head_dim;
  h[7] = P.max_ctx;
}

// LDS of one segment's 4-wave merge.
template <int D>
struct DecodeShared {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][16][D + 4];  // rows stay 16-byte aligned
  int bad[kWaves];             // per wave: a table entry outside the pool was seen
};

// LDS of the persistent grid's split: per-thread tile sums, then their
// exclusive prefix; the batch's total; the first sequence of the share.
struct SplitShared {
  int64_t scan[kThreads];
  int64_t total, base0;
  int64_t lo, hi;  // the share's boundaries after snapping
  int s0;
};

// One segment: tokens [tok0, tok0 + ntok) of kv head g of sequence s, the
// partitions of that pair that fall to this workgroup.  segment_run folds
// the tiles and leaves each wave's (max, sum, accumulator) in LDS;
// segment_combine (below) merges the four waves into the pair's rows.
// `mid` runs once per wave as soon as the segment's first tiles are in
// flight: the persistent grid combines the previous segment there, so that
// work and the new segment's first round trip to memory overlap.
template <typename T, int D, typename Mid>
__device__ __forceinline__ void segment_run(const KParams& P, DecodeShared<D>& sh, int s, int g, int ctx,
                                            int tok0, int ntok, bool first, Mid&& mid) {
  constexpr int DC = D / 32;  // 16-byte chunks per lane per tile
  constexpr int NT = D / 16;  // 16-dim output tiles
  constexpr int kTileElems = kBlockTokens * D;

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // head column of this lane
  const int quad = lane >> 4;  // token quad / k-slice of this lane
  const int G = P.hq / P.hkv;
  const int C = P.qlen;
  const int ncol = G * C;  // accumulator columns in use: (query i, head n) = column i * G + n
  // output / partial row of column c: query i = c / G, head g * G + c % G
  auto col_row = [&](int c) {
    return (int64_t(s) * C + c / G) * P.hq + int64_t(g) * G + c % G;
  };

  const int nblk = (ntok + kBlockTokens - 1) / kBlockTokens;
  const int tsh = P.tile_shift;
  const int tile0 = tok0 / kBlockTokens;  // the segment's first tile in the sequence
  const int32_t* trow = P.tables + int64_t(s) * P.max_blocks;

  // Q^T as the B operand: lane supplies column n, dims 8 * (4 i + quad) + 0..7.
  u32x4_t qb[DC];
#pragma unroll
  for (int i = 0; i < DC; ++i) {
    if (n < ncol) {
      qb[i] = load16(P.q16 + col_row(n) * D + 8 * (4 * i + quad));
    } else {
      qb[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // last key column n may attend (its query's position)
  const int last_n = ctx - C + (n < ncol ? n / G : 0);

  const uint16_t* kg = P.k16 + (int64_t(g) << tsh) * kTileElems;
  const uint16_t* vg = P.v16 + (int64_t(g) << tsh) * kTileElems;
  const int64_t blk_stride = (int64_t(P.hkv) << tsh) * kTileElems;
  const int voff = lane * 16;

  // Online softmax in the exp2 domain.  The reference max m of head n is
  // moved only when a score exceeds it by more than 2^8: until then
  // p = 2^(s - m) <= 256, which fp32 sums and the hi + lo split of P hold
  // exactly as well as p <= 1, and the accumulator rescale (a multiply of
  // all of o) is skipped on most tiles.
  // -1e30 rather than -inf: a column whose keys of a tile are all masked
  // (only with C > 1) then gets p = 0, not 2^(-inf + inf)
  float m = kNoMax;     // reference max of column n, same in every quad
  float lsum = 0.f;     // this lane's share of the sum of head n
  f32x4_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  const int ntw_all = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;  // tiles of this wave
  if (ntw_all == 0) mid();
  for (int wb = 0; wb < ntw_all; wb += kWave) {
    const int ntw = min(kWave, ntw_all - wb);
    const int tbl = lane < ntw ? trow[(tile0 + kWaves * (wb + lane) + w) >> tsh] : 0;

    auto rsrc = [&](int i, const uint16_t* base) {
      const int phys = __builtin_amdgcn_readlane(tbl, i < ntw ? i : 0);
      const int sub = (tile0 + kWaves * (wb + i) + w) & ((1 << tsh) - 1);  // tile inside the block
      const bool ok = i < ntw && phys >= 0 && int64_t(phys) < P.num_blocks;
      bad |= i < ntw && !ok;  // an entry outside the pool: NaN result, nothing read
      return tile_rsrc(base + int64_t(ok ? phys : 0) * blk_stride + (ok ? sub : 0) * kTileElems,
                       ok ? kTileElems * 2 : 0);
    };
    auto load = [&](int i, u32x4_t* kd, u32x4_t* vd) {
      const auto rk = rsrc(i, kg);
      const auto rv = rsrc(i, vg);
      // fixed issue order of the load groups: the wait counts at the loop
      // head are exact only when every path issues them in one order
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < DC; ++c) kd[c] = load16_nt(rk, voff + c * 1024);
#pragma unroll
      for (int c = 0; c < DC; ++c) vd[c] = load16_nt(rv, voff + c * 1024);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto step = [&](u32x4_t* kt, u32x4_t* vt, int i) {
      // scores: lane holds S^T[token 4 * quad + r][head n]
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) sc = Mfma<T>::k32(kt[c], qb[c], sc);
      const int jb = kWaves * (wb + i) + w;
      const int valid = min(kBlockTokens, ntok - jb * kBlockTokens);  // slots inside the context
      const int lim = last_n - (tok0 + jb * kBlockTokens);             // last attended slot of column n
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = (4 * quad + r <= lim) ? sc[r] * P.scale_log2 : -INFINITY;
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = fmaxf(bm, shfl_xor(bm, 16));
      bm = fmaxf(bm, shfl_xor(bm, 32));
      const bool grow = bm > m + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? bm : m;
        const float alpha = fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t] *= alpha;
        m = mn;
      }
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m);
      lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);

      // P^T as the B operand, split hi + lo in the input type
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = T::from_float(pr[r]);
        lo[r] = T::from_float(pr[r] - T::to_float(hi[r]));
      }
      const uint32_t bh0 = pack2(hi[0], hi[1]), bh1 = pack2(hi[2], hi[3]);
      const uint32_t bl0 = pack2(lo[0], lo[1]), bl1 = pack2(lo[2], lo[3]);
      if (valid < kBlockTokens) {
        // slots past the context may hold anything (NaN included): zero them
        // so 0 * garbage never reaches the accumulator
        const int t0 = 4 * quad;
        const uint32_t m01 = (t0 + 0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
        const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          vt[c][0] &= m01;
          vt[c][1] &= m23;
          vt[c][2] &= m01;
          vt[c][3] &= m23;
        }
      }
      // V^T as the A operand: output tile t = dims 16 t .. 16 t + 15 is half
      // (t % 2) of chunk t / 2 -- tokens 4 * quad + 0..3 of dim 16 t + n.
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t a0 = vt[t / 2][2 * (t % 2)];
        const uint32_t a1 = vt[t / 2][2 * (t % 2) + 1];
        o[t] = Mfma<T>::k16(a0, a1, bh0, bh1, o[t]);
        o[t] = Mfma<T>::k16(a0, a1, bl0, bl1, o[t]);
      }
    };

    // two tiles in flight: while one is computed the other is loading
    u32x4_t ka[DC], va[DC], kb[DC], vb[DC];
    load(0, ka, va);
    if (wb == 0) mid();
    load(1, kb, vb);
    for (int i = 0; i < ntw; i += 2) {
      step(ka, va, i);
      load(i + 2, ka, va);
      if (i + 1 < ntw) step(kb, vb, i + 1);
      load(i + 3, kb, vb);
    }
  }
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);

  // ---- each wave leaves its (max, sum) per column and its accumulator in
  // LDS for segment_combine.
  if (!first) __syncthreads();  // every reader of the previous segment's merge is done
  if (lane == 0) sh.bad[w] = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (quad == 0) {
    sh.m[w][n] = m;
    sh.l[w][n] = lsum;
  }
  if (n < ncol) {
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4_t*>(&sh.o[w][n][16 * t + 4 * quad]) = o[t];
  }
  __syncthreads();
}

// Merge of the four waves' results in LDS into the rows of (s, g): each
// half-wave combines one whole column (32 lanes x 4 dims): wave w takes
// columns w, w + 4, ..., its lower half the even ones of those.  Each lane
// reads the four waves' values of its four dims with 16-byte LDS reads and
// the column's four weights once, and a column's output row leaves as one
// contiguous run.  With nseg == 1 the segment was the whole context and the
// rows are final; otherwise they go to partial slot `seg` of the pair's nseg.
template <typename T, int D, bool OUT_F32>
__device__ __forceinline__ void segment_combine(const KParams& P, DecodeShared<D>& sh, int s, int g, int nseg,
                                                int seg) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = P.hq / P.hkv;
  const int C = P.qlen;
  const int ncol = G * C;
  auto col_row = [&](int c) {
    return (int64_t(s) * C + c / G) * P.hq + int64_t(g) * G + c % G;
  };
  static_assert(kWaves == 4, "one flag per wave");
  static_assert(D == 4 * 32 || D == 2 * 32, "a half-wave covers a row in whole 4-dim pieces");
  const bool any_bad = (sh.bad[0] | sh.bad[1] | sh.bad[2] | sh.bad[3]) != 0;
  constexpr int kLanesPerRow = D / 4;  // lanes of one column's row
  const int half = lane / 32;
  for (int c = w + kWaves * half; c < ncol; c += 2 * kWaves) {
    for (int part = lane % 32; part < kLanesPerRow; part += 32) {
      const int d0 = 4 * part;
      float mw[kWaves], M = kNoMax;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        mw[ww] = sh.m[ww][c];
        M = fmaxf(M, mw[ww]);
      }
      float L = 0.f;
      f32x4_t O = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = fast_exp2(mw[ww] - M);
        L += f * sh.l[ww][c];
        O += f * *reinterpret_cast<const f32x4_t*>(&sh.o[ww][c][d0]);
      }
      if (any_bad) O = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      const int64_t row = col_row(c);
      if (nseg == 1) {
        store_out4<T, OUT_F32>(P.out, row * D + d0, O * (1.f / L));
      } else {
        const int64_t prow = row * P.nparts_max + seg;
        __builtin_nontemporal_store(O, reinterpret_cast<f32x4_t*>(P.ws_acc + prow * D + d0));
        if (d0 == 0) {
          P.ws_m[prow] = M;
          P.ws_l[prow] = L;
        }
      }
    }
  }
}

// A whole segment, run and merged.
template <typename T, int D, bool OUT_F32>
__device__ __forceinline__ void decode_segment(const KParams& P, DecodeShared<D>& sh, int s, int g, int ctx,
                                               int tok0, int ntok, int nseg, int seg) {
  segment_run<T, D>(P, sh, s, g, ctx, tok0, ntok, true, [] {});
  segment_combine<T, D, OUT_F32>(P, sh, s, g, nseg, seg);
}

// Rows of sequence s's kv head g that are written without reading: zeros
// for an empty context, NaN for a length outside the contract.
template <typename T, int D, bool OUT_F32>
__device__ void write_unread_rows(const KParams& P, int s, int g, int ctx) {
  const int G = P.hq / P.hkv, C = P.qlen, ncol = G * C;
  const float v = ctx == 0 ? 0.f : __builtin_nanf("");
  for (int idx = threadIdx.x; idx < ncol * D; idx += kThreads) {
    const int c = idx / D, d = idx % D;
    const int64_t row = (int64_t(s) * C + c / G) * P.hq + int64_t(g) * G + c % G;
    store_out<T, OUT_F32>(P.out, row * D + d, v);
  }
}

// One workgroup per (kv head, sequence, partition), grid (Hkv, S,
// partitions): for batches whose longest context spans few partitions.  The
// hardware deals workgroups to the 8 XCDs round-robin by linear id, so the
// kv head runs fastest and every XCD gets an even share of the partitions
// that hold work (with the partition index fastest, the XCDs serving late
// partitions, which are empty for short contexts, sat idle).
template <typename T, int D, bool OUT_F32>
__global__ void __launch_bounds__(kThreads)
decode_partition_kernel(KParams P) {
  __shared__ DecodeShared<D> sh;
  // this workgroup's item (see partition_grid_workgroups): grid (Hkv, S,
  // partitions), or one dimension dealt over the XCDs
  int g = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int64_t items = int64_t(P.hkv) * P.num_seqs * P.nparts_max;
  if (partition_grid_weighted(items, P.hkv)) {  // items < 2^31 (checked at launch)
    const uint32_t x = blockIdx.x % 8, r = blockIdx.x / 8;
    uint32_t j;
    if (x % 2 == 0) {
      const uint32_t R = r / 25, rr = r % 25;
      j = rr < 23 ? 192 * R + 8 * rr + x : 192 * R + 184 + 4 * (rr - 23) + x / 2;
    } else {
      j = 192 * (r / 23) + 8 * (r % 23) + x;
    }
    if (j >= uint32_t(items)) return;
    const uint32_t hkv = uint32_t(P.hkv), js = j / hkv;
    g = int(j - js * hkv);
    s = int(js % uint32_t(P.num_seqs));
    part = int(js / uint32_t(P.num_seqs));
  }
  if (g == 0 && s == 0 && part == 0 && threadIdx.x == 0 && P.ws_hdr != nullptr) write_header(P);
  const int ctx = P.ctxs[s];
  const bool read = pair_tiles(ctx, P) > 0;
  const int nparts = read ? (ctx + P.partition - 1) / P.partition : 0;
  if (part == 0 && threadIdx.x == 0 && P.ws_nseg != nullptr) P.ws_nseg[int64_t(s) * P.hkv + g] = nparts;
  if (!read) {
    if (part == 0) write_unread_rows<T, D, OUT_F32>(P, s, g, ctx);
    return;
  }
  const int tok0 = part * P.partition;
  if (tok0 >= ctx) return;
  decode_segment<T, D, OUT_F32>(P, sh, s, g, ctx, tok0, min(P.partition, ctx - tok0), nparts, part);
}

// The persistent grid.  Three waves per SIMD: two tiles in flight per wave
// then keep enough reads outstanding per CU for the HBM stream (two waves per
// SIMD do not).
template <typename T, int D, bool OUT_F32>
__global__ void __launch_bounds__(kThreads, 3)
decode_persistent_kernel(KParams P) {
  __shared__ DecodeShared<D> sh;
  __shared__ SplitShared sp;
  const int S = P.num_seqs;
  const int tid = threadIdx.x;

  if (blockIdx.x == 0 && tid == 0 && P.ws_hdr != nullptr) write_header(P);

  // ---- the batch's tiles (kv heads included) and this workgroup's share.
  // Thread i sums the tiles of sequences [i * chunk, (i + 1) * chunk); wave 0
  // turns the 256 sums into an exclusive prefix.
  const int chunk = (S + kThreads - 1) / kThreads;
  const int sa = min(S, tid * chunk), sb = min(S, sa + chunk);
  auto weight = [&](int ctx) {
    const int t = pair_tiles(ctx, P);
    return t > 0 ? t + kSegmentCost : 0;
  };
  int64_t mine = 0;
  for (int s = sa; s < sb; ++s) mine += weight(P.ctxs[s]);
  mine *= P.hkv;
  sp.scan[tid] = mine;
  __syncthreads();
  if (tid < kWave) {
    int64_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = sp.scan[4 * tid + i];
    const int64_t tot = (a[0] + a[1]) + (a[2] + a[3]);
    int64_t inc = tot;
#pragma unroll
    for (int k = 1; k < kWave; k <<= 1) {
      const int64_t y = __shfl_up(inc, k, kWave);
      if (tid >= k) inc += y;
    }
    int64_t e = inc - tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sp.scan[4 * tid + i] = e;
      e += a[i];
    }
    if (tid == kWave - 1) sp.total = inc;
  }
  __syncthreads();
  const int64_t T_all = uniform64(sp.total);
  const int ut = P.partition / kBlockTokens;  // tiles per partition
  // Every share holds at least one partition's worth of tiles, so each
  // workgroup between the first and the last owner of a pair's partitions
  // owns at least one of them: a pair's segments are numbered without gaps.
  const int64_t nw = max<int64_t>(1, min<int64_t>(gridDim.x, T_all / ut));
  const int64_t b = blockIdx.x;
  // Workgroup b runs on XCD b % 8, and the odd XCDs finish equal shares
  // about 8% later than the even ones; with one query per sequence the odd
  // workgroups get 23/25 of an even one's share (measured on three MI355X:
  // GQA lognormal -1.6 / -1.1 / -2.2%, 16 x 32,768 -1.0 / -1.1 / -0.9%, the
  // reverse weighting +2 to 3.5% on every shape; four queries per sequence
  // +0.7 / +0.5%, so those stay unweighted).  Only while every share stays at
  // least two partitions long.  Boundary j sits at T_all C(j) / C(nw) with
  // C(j) = ceil(j / 2) we + floor(j / 2) wo.
  const bool weigh = P.qlen == 1 && T_all / nw >= 2 * ut;
  const int64_t we = weigh ? kEvenShareWeight : 1, wo = weigh ? kOddShareWeight : 1;
  auto cum = [&](int64_t j) { return (j + 1) / 2 * we + j / 2 * wo; };
  const int64_t ctot = cum(nw);
  auto boundary = [&](int64_t j) { return T_all * cum(j) / ctot; };
  const int64_t lo0 = boundary(b);
  const int64_t hi0 = b < nw ? boundary(b + 1) : lo0;
  // A share boundary that would leave at most `snap` tiles of a pair on one
  // side moves to that side's edge, so the pair is not split: the partials
  // of a split pair cost decode time in proportion to its rows, the move's
  // imbalance does not (on 256 lognormal contexts with 4 queries per
  // sequence, 16 rows per pair: 293.6 us unmoved, 287 us with up to 16 or
  // 32 tiles moved; with a fixed 16 tiles, 1-row pairs slowed by 1.3% and
  // with 32 by 6%).  Boundaries move only inside the pair they fall in, at
  // most one each way per pair, and never past another boundary while every
  // share is longer than the move plus a partition.
  const int rows = P.hq / P.hkv * P.qlen;
  const int snap = T_all * min(we, wo) / ctot > min(rows, ut) + ut ? min(rows, ut) : 0;
  auto snap_at = [&](int64_t x, int s, int64_t base) {
    const int ctx = P.ctxs[s];
    const int t = weight(ctx);
    const int64_t a = base + (x - base) / t * t;
    return snap_boundary(x, a, pair_tiles(ctx, P), (ctx + P.partition - 1) / P.partition, ut, snap);
  };
  if (lo0 < hi0) {
    // the threads whose sequences hold tiles lo0 and hi0 find them (the
    // first also the sequence the share starts in)
    const int64_t e = sp.scan[tid];
    if (e <= lo0 && lo0 < e + mine) {
      int64_t base = e;
      int s = sa;
      for (; s < sb; ++s) {
        const int64_t ts = int64_t(weight(P.ctxs[s])) * P.hkv;
        if (base + ts > lo0) break;
        base += ts;
      }
      sp.s0 = s;
      sp.base0 = base;
      sp.lo = snap_at(lo0, s, base);
    }
    if (e <= hi0 && hi0 < e + mine) {
      int64_t base = e;
      int s = sa;
      for (; s < sb; ++s) {
        const int64_t ts = int64_t(weight(P.ctxs[s])) * P.hkv;
        if (base + ts > hi0) break;
        base += ts;
      }
      sp.hi = snap_at(hi0, s, base);
    }
  }
  __syncthreads();
  if (lo0 < hi0) {
    const int64_t lo = uniform64(sp.lo);
    const int64_t hi = hi0 < T_all ? uniform64(sp.hi) : hi0;
    // pair (s, g) spans t = its tiles + kSegmentCost of the weighted stream;
    // its partition k starts at pb + k * ut and belongs to the workgroup
    // whose share holds that position once the boundaries have moved
    // the last boundary at or before x: the largest j with C(j) <= y
    auto owner = [&](int64_t x) {
      const int64_t y = ((x + 1) * ctot - 1) / T_all;
      const int64_t k = y / (we + wo);
      return 2 * k + (y - k * (we + wo) >= we ? 1 : 0);
    };
    int s = uniform(sp.s0);
    int64_t base = uniform64(sp.base0);
    bool first = true;  // no earlier segment's merge to wait for
    // the previous segment, merged while the next one's first tiles load
    bool pending = false;
    int ps = 0, pg = 0, pnseg = 0, pseg = 0;
    auto combine_previous = [&] {
      if (pending) segment_combine<T, D, OUT_F32>(P, sh, ps, pg, pnseg, pseg);
    };
    while (s < S && base < hi) {
      const int ctx = uniform(P.ctxs[s]);
      const int t = weight(ctx);
      if (t > 0) {
        const int nu = (ctx + P.partition - 1) / P.partition;
        const int tiles = t - kSegmentCost;
        for (int g = 0; g < P.hkv; ++g) {
          const int64_t a = base + int64_t(g) * t;
          const int64_t pb = a + kSegmentCost;
          if (pb >= hi) break;
          const int64_t last = pb + int64_t(nu - 1) * ut;  // the pair's last partition
          if (last < lo) continue;
          const int k0 = lo <= pb ? 0 : int((lo - pb + ut - 1) / ut);
          const int k1 = min(nu - 1, int((hi - pb + ut - 1) / ut) - 1);
          if (k0 > k1) continue;
          // the first boundary past pb may have moved to pb, the last one
          // before `last` past it
          int64_t first_owner = owner(pb);
          int64_t last_owner = owner(last);
          if (first_owner < last_owner) {
            const int64_t jf = first_owner + 1, jl = last_owner;
            if (snap_boundary(boundary(jf), a, tiles, nu, ut, snap) == pb) ++first_owner;
            if (snap_boundary(boundary(jl), a, tiles, nu, ut, snap) == last + 1) --last_owner;
          }
          const int nseg = int(last_owner - first_owner + 1);
          const int tok0 = k0 * P.partition;
          const int ntok = min((k1 + 1) * P.partition, ctx) - tok0;
          segment_run<T, D>(P, sh, s, g, ctx, tok0, ntok, first, combine_previous);
          first = false;
          pending = true;
          ps = s;
          pg = g;
          pnseg = nseg;
          pseg = int(b - first_owner);
          if (k0 == 0 && P.ws_nseg != nullptr && tid == 0) P.ws_nseg[int64_t(s) * P.hkv + g] = nseg;
        }
      }
      base += int64_t(t) * P.hkv;
      ++s;
    }
    combine_previous();  // the last segment
  }

  // rows outside the stream: an empty context gives zeros, a length outside
  // the contract NaN (reported, nothing read)
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const int ctx = P.ctxs[s];
    if (pair_tiles(ctx, P) > 0) continue;
    for (int gg = 0; gg < P.hkv; ++gg) write_unread_rows<T, D, OUT_F32>(P, s, gg, ctx);
    if (P.ws_nseg != nullptr)
      for (int gg = tid; gg < P.hkv; gg += kThreads) P.ws_nseg[int64_t(s) * P.hkv + gg] = 0;
  }
}

// ------------------------------------------------------------------------
// Vector-ALU partition kernel (fp32).  Grid (partitions, Hq, S); one
// workgroup per query head.  Lane (quad, c): K tile token c, V dims
// 32 i + 16 h + c for tokens 4 quad + 0..3.
// ------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads)
decode_f32_kernel(KParams P) {
  constexpr int DC = D / 32;
  constexpr int64_t kTile = int64_t(kBlockTokens) * D;
  typedef float f32x8_t __attribute__((ext_vector_type(8)));

  __shared__ float s_m[kWaves], s_l[kWaves];
  __shared__ float s_o[kWaves][D];
  __shared__ int s_bad;

  const int part = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, quad = lane >> 4;
  const int G = P.hq / P.hkv;
  const int g = h / G;
  const int ctx = P.ctxs[s];
  const int64_t row = int64_t(s) * P.hq + h;
  const bool no_read = context_out_of_contract(ctx, P) || ctx == 0;
  // every partition is its own partial slot; the merge reads how many
  if (part == 0 && h % G == 0 && threadIdx.x == 0 && P.ws_nseg != nullptr)
    P.ws_nseg[int64_t(s) * P.hkv + g] = no_read ? 0 : (ctx + P.partition - 1) / P.partition;
  if (part == 0 && h == 0 && s == 0 && threadIdx.x == 0 && P.ws_hdr != nullptr) write_header(P);

  if (no_read) {
    if (part == 0) {
      const float v = ctx == 0 ? 0.f : __builtin_nanf("");
      for (int d = threadIdx.x; d < D; d += kThreads) static_cast<float*>(P.out)[row * D + d] = v;
    }
    return;
  }
  const int tok0 = part * P.partition;
  if (tok0 >= ctx) return;
  const int ntok = min(P.partition, ctx - tok0);
  const int nblk = (ntok + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (ctx + P.partition - 1) / P.partition;
  const int sh = P.tile_shift;
  const int tile0 = tok0 / kBlockTokens;
  const int32_t* trow = P.tables + int64_t(s) * P.max_blocks;

  f32x8_t qv[DC];
#pragma unroll
  for (int i = 0; i < DC; ++i) qv[i] = *reinterpret_cast<const f32x8_t*>(P.q32 + row * D + 8 * (4 * i + quad));

  const int64_t blk_stride = (int64_t(P.hkv) << sh) * kTile;
  float m = -INFINITY, lsum = 0.f;
  float acc[DC][2];
#pragma unroll
  for (int i = 0; i < DC; ++i) acc[i][0] = acc[i][1] = 0.f;
  bool bad = false;

  for (int jb = w; jb < nblk; jb += kWaves) {
    int phys = trow[(tile0 + jb) >> sh];
    if (phys < 0 || int64_t(phys) >= P.num_blocks) {
      bad = true;
      phys = 0;
    }
    const int64_t tile = ((int64_t(g) << sh) + ((tile0 + jb) & ((1 << sh) - 1))) * kTile;
    const float* kt = P.k32 + int64_t(phys) * blk_stride + tile + lane * 8;
    const float* vt = P.v32 + int64_t(phys) * blk_stride + tile + lane * 8;
    f32x8_t kk[DC], vv[DC];
#pragma unroll
    for (int i = 0; i < DC; ++i) kk[i] = *reinterpret_cast<const f32x8_t*>(kt + i * 512);
#pragma unroll
    for (int i = 0; i < DC; ++i) vv[i] = *reinterpret_cast<const f32x8_t*>(vt + i * 512);

    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qv[i][e], kk[i][e], dot);
    dot += shfl_xor(dot, 16);
    dot += shfl_xor(dot, 32);
    const int valid = min(kBlockTokens, ntok - jb * kBlockTokens);
    const float sv = c < valid ? dot * P.scale_log2 : -INFINITY;
    float bm = sv;
    bm = fmaxf(bm, shfl_xor(bm, 1));
    bm = fmaxf(bm, shfl_xor(bm, 2));
    bm = fmaxf(bm, shfl_xor(bm, 4));
    bm = fmaxf(bm, shfl_xor(bm, 8));
    const float mn = fmaxf(m, bm);
    const float alpha = fast_exp2(m - mn);
    const float pc = fast_exp2(sv - mn);
    lsum = lsum * alpha + pc;
    m = mn;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = shfl(pc, (lane & 48) | (4 * quad + r));
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float a = acc[i][hh] * alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float term = pr[r] * vv[i][hh * 4 + r];
          a += (4 * quad + r < valid) ? term : 0.f;
        }
        acc[i][hh] = a;
      }
  }
  // every quad holds the same per-token sums; fold the 16 tokens of a quad
  lsum += shfl_xor(lsum, 1);
  lsum += shfl_xor(lsum, 2);
  lsum += shfl_xor(lsum, 4);
  lsum += shfl_xor(lsum, 8);
#pragma unroll
  for (int i = 0; i < DC; ++i)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      acc[i][hh] += shfl_xor(acc[i][hh], 16);
      acc[i][hh] += shfl_xor(acc[i][hh], 32);
    }

  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  if (lane == 0) {
    s_m[w] = m;
    s_l[w] = lsum;
  }
  if (quad == 0) {
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) s_o[w][32 * i + 16 * hh + c] = acc[i][hh];
  }
  __syncthreads();
  const bool any_bad = s_bad != 0;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float M = s_m[0];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(s_m[ww] - M);
      L += f * s_l[ww];
      O += f * s_o[ww][d];
    }
    if (any_bad) O = __builtin_nanf("");
    if (nparts == 1) {
      static_cast<float*>(P.out)[row * D + d] = O / L;
    } else {
      const int64_t prow = row * P.nparts_max + part;
      P.ws_acc[prow * D + d] = O;
      if (d == 0) {
        P.ws_m[prow] = M;
        P.ws_l[prow] = L;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Log-sum-exp merge of the partials.  One workgroup per (sequence, kv head)
// pair, grid (Hkv, S):
//   M = max_j m_j,  w_j = 2^(m_j - M),  out = sum_j w_j acc_j / sum_j w_j l_j
// over the pair's partial slots j, whose count the partition kernel
// recorded (at most 1: the pair's rows are already final, and the
// workgroup leaves after that one read -- most pairs of a batch of short
// contexts).  Thread t merges dims 8 (t % (D / 8)) .. + 7 of the pair's row
// t / (D / 8), so all rows of a pair merge at once (with one wave per row,
// the 16 rows of four queries per sequence took four round trips to memory
// in series).  A row of up to kReduceFew slots loads all its partials at
// once; longer rows run over their slots in order.  Sums run in slot order,
// so the result is deterministic.  A workspace whose header does not match
// this call's geometry (not filled by the partition launch of the same
// sizes) gives NaN rows instead of a merge at the wrong stride.
// ------------------------------------------------------------------------
constexpr int kReduceFew = 8;  // rows with at most this many slots load them all at once
constexpr int kMergeDims = 8;  // dims per thread

template <typename T, int D, bool OUT_F32>
__global__ void __launch_bounds__(kThreads)
decode_reduce_kernel(KParams P) {
  constexpr int kRowThreads = D / kMergeDims;
  const int g = blockIdx.x, s = blockIdx.y;
  const int G = P.hq / P.hkv, C = P.qlen;
  const int c = threadIdx.x / kRowThreads, d0 = threadIdx.x % kRowThreads * kMergeDims;
  if (c >= G * C) return;
  // output row of column c: query c / G of head g * G + c % G
  const int64_t orow = (int64_t(s) * C + c / G) * P.hq + int64_t(g) * G + c % G;
  auto store8 = [&](f32x4_t lo, f32x4_t hi) {
    store_out4<T, OUT_F32>(P.out, orow * D + d0, lo);
    store_out4<T, OUT_F32>(P.out, orow * D + d0 + 4, hi);
  };
  const int32_t* hd = P.ws_hdr;
  if (hd[0] != kWorkspaceMagic || hd[1] != P.partition || hd[2] != P.nparts_max || hd[3] != P.num_seqs * P.qlen ||
      hd[4] != P.hq || hd[5] != P.hkv || hd[6] != D || hd[7] != P.max_ctx) {
    const float nan = __builtin_nanf("");
    store8(f32x4_t{nan, nan, nan, nan}, f32x4_t{nan, nan, nan, nan});
    return;
  }
  // partial slots of the pair, at most the partitions the workspace holds
  const int nparts = min(P.ws_nseg[int64_t(s) * P.hkv + g], P.nparts_max);
  if (nparts <= 1) return;  // written by the partition kernel

  const int64_t prow0 = orow * P.nparts_max;
  const float* acc = P.ws_acc + prow0 * D + d0;
  f32x4_t O0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, O1 = O0;
  float L = 0.f;
  // every partial of the row at once: one round trip to memory (entries
  // past the row's last slot reload that one and weigh 0)
  auto few = [&](auto nj_tag) __attribute__((always_inline)) {
    constexpr int NJ = decltype(nj_tag)::value;
    float mj[NJ], lj[NJ];
    f32x4_t a0[NJ], a1[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int jj = min(j, nparts - 1);
      mj[j] = P.ws_m[prow0 + jj];
      lj[j] = P.ws_l[prow0 + jj];
      a0[j] = *reinterpret_cast<const f32x4_t*>(acc + int64_t(jj) * D);
      a1[j] = *reinterpret_cast<const f32x4_t*>(acc + int64_t(jj) * D + 4);
    }
    float M = mj[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) M = fmaxf(M, mj[j]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float wj = j < nparts ? fast_exp2(mj[j] - M) : 0.f;
      L += wj * lj[j];
      O0 += wj * a0[j];
      O1 += wj * a1[j];
    }
  };
  if (nparts <= 2) {
    few(std::integral_constant<int, 2>{});
  } else if (nparts <= 4) {
    few(std::integral_constant<int, 4>{});
  } else if (nparts <= kReduceFew) {
    few(std::integral_constant<int, kReduceFew>{});
  } else {
    float M = -INFINITY;
#pragma unroll 8
    for (int j = 0; j < nparts; ++j) M = fmaxf(M, P.ws_m[prow0 + j]);
#pragma unroll 4
    for (int j = 0; j < nparts; ++j) {
      const float wj = fast_exp2(P.ws_m[prow0 + j] - M);
      L += wj * P.ws_l[prow0 + j];
      O0 += wj * *reinterpret_cast<const f32x4_t*>(acc + int64_t(j) * D);
      O1 += wj * *reinterpret_cast<const f32x4_t*>(acc + int64_t(j) * D + 4);
    }
  }
  store8(O0 / L, O1 / L);
}

KParams make_params(const DecodeArgs& a) {
  KParams p{};
  p.out = a.out;
  p.q16 = static_cast<const uint16_t*>(a.q);
  p.q32 = static_cast<const float*>(a.q);
  p.k16 = static_cast<const uint16_t*>(a.k_cache);
  p.v16 = static_cast<const uint16_t*>(a.v_cache);
  p.k32 = static_cast<const float*>(a.k_cache);
  p.v32 = static_cast<const float*>(a.v_cache);
  p.tables = a.block_tables;
  p.ctxs = a.context_lens;
  p.ws_acc = a.ws_acc;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.num_blocks = a.num_blocks;
  p.scale_log2 = a.scale_log2;
  p.max_blocks = a.max_blocks;
  p.hq = a.num_q_heads;
  p.hkv = a.num_kv_heads;
  p.max_ctx = a.max_context_len;
  p.partition = a.partition;
  p.nparts_max = a.num_partitions;
  p.qlen = a.q_len;
  p.tile_shift = a.tile_shift;
  p.num_seqs = a.num_seqs;
  p.head_dim = a.head_dim;
  p.ws_hdr = a.ws_hdr;
  p.ws_nseg = a.ws_nseg;
  return p;
}

// Workgroups of `kernel` (kThreads threads) that fit on the current device
// at once: its occupancy per CU times the CU count, looked up once per device.
template <typename K>
int64_t resident_workgroups(K kernel) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int64_t> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || cus <= 0)
    cus = 1;
  const int64_t n = int64_t(per_cu) * cus;
  if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// One resident grid: as many workgroups as fit at once, never more than
// there are partitions in the batch's upper bound.
template <typename T, int D, bool OUT_F32>
hipError_t launch_mfma_grid(const DecodeArgs& a, const KParams& p) {
  const auto kernel = decode_persistent_kernel<T, D, OUT_F32>;
  const int64_t units = int64_t(a.num_seqs) * a.num_kv_heads * std::max(1, a.num_partitions);
  const int64_t n = std::max<int64_t>(1, std::min(resident_workgroups(kernel), units));
  hipLaunchKernelGGL(kernel, dim3(unsigned(n)), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

template <typename T, int D, bool OUT_F32>
hipError_t launch_partition_grid(const DecodeArgs& a, const KParams& p) {
  const int64_t items = int64_t(a.num_kv_heads) * a.num_seqs * a.num_partitions;
  const dim3 grid = partition_grid_weighted(items, a.num_kv_heads)
                        ? dim3(unsigned(partition_grid_workgroups(items, a.num_kv_heads)))
                        : dim3(unsigned(a.num_kv_heads), unsigned(a.num_seqs), unsigned(a.num_partitions));
  hipLaunchKernelGGL((decode_partition_kernel<T, D, OUT_F32>), grid, dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mfma(const DecodeArgs& a, const KParams& p) {
  if (decode_uses_persistent_grid(a.num_partitions))
    return a.out_f32 ? launch_mfma_grid<T, D, true>(a, p) : launch_mfma_grid<T, D, false>(a, p);
  return a.out_f32 ? launch_partition_grid<T, D, true>(a, p) : launch_partition_grid<T, D, false>(a, p);
}

template <typename T, int D>
hipError_t launch_reduce(const DecodeArgs& a, const KParams& p) {
  // one workgroup per (sequence, kv head) pair, 8 dims of one row per thread
  const int threads = a.num_q_heads / a.num_kv_heads * a.q_len * (D / kMergeDims);
  const dim3 grid(unsigned(a.num_kv_heads), unsigned(a.num_seqs));
  const dim3 block(unsigned((threads + kWave - 1) / kWave * kWave));
  if (a.out_f32) {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, true>), grid, block, 0, a.stream, p);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, false>), grid, block, 0, a.stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a) {
  const KParams p = make_params(a);
  if (a.dtype == PA_F32) {
    const dim3 grid(unsigned(a.num_partitions), unsigned(a.num_q_heads), unsigned(a.num_seqs));
    if (a.head_dim == 64) {
      hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(kThreads), 0, a.stream, p);
    } else {
      hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(kThreads), 0, a.stream, p);
    }
    return hipGetLastError();
  }
  if (a.dtype == PA_BF16) return a.head_dim == 64 ? launch_mfma<Bf16, 64>(a, p) : launch_mfma<Bf16, 128>(a, p);
  return a.head_dim == 64 ? launch_mfma<F16, 64>(a, p) : launch_mfma<F16, 128>(a, p);
}

int64_t decode_resident_workgroups(pa_dtype_t dtype, int32_t head_dim, bool out_f32) {
  if (dtype == PA_BF16) {
    if (head_dim == 64)
      return out_f32 ? resident_workgroups(decode_persistent_kernel<Bf16, 64, true>)
                     : resident_workgroups(decode_persistent_kernel<Bf16, 64, false>);
    return out_f32 ? resident_workgroups(decode_persistent_kernel<Bf16, 128, true>)
                   : resident_workgroups(decode_persistent_kernel<Bf16, 128, false>);
  }
  if (head_dim == 64)
    return out_f32 ? resident_workgroups(decode_persistent_kernel<F16, 64, true>)
                   : resident_workgroups(decode_persistent_kernel<F16, 64, false>);
  return out_f32 ? resident_workgroups(decode_persistent_kernel<F16, 128, true>)
                 : resident_workgroups(decode_persistent_kernel<F16, 128, false>);
}

hipError_t launch_decode_reduce(const DecodeArgs& a) {
  if (a.num_partitions <= 1) return hipSuccess;
  const KParams p = make_params(a);
  // the output conversion is the only type-dependent step
  if (a.dtype == PA_BF16) return a.head_dim == 64 ? launch_reduce<Bf16, 64>(a, p) : launch_reduce<Bf16, 128>(a, p);
  return a.head_dim == 64 ? launch_reduce<F16, 64>(a, p) : launch_reduce<F16, 128>(a, p);
}

}  // namespace pa
