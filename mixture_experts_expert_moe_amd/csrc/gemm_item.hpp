// One work item of the small-tile grouped GEMMs (gate/up + SwiGLU, down):
// the device code shared by the grouped GEMM launches (gemm.hip) and the
// fused decode layer (decode.hip), so both compute every output element with
// the same instructions in the same order.
//
// Work item = (tile of <= 64 rows of one group) x (16 or 32 gate/up pairs, or
// 64 down columns); the item's waves split K.  Within an item:
//   MFMA A operand = 16 weight rows (lane l: row l % 16, K-group l / 16),
//   MFMA B operand = 16 token rows  (lane l: row l % 16, same K-group),
//   D[i][j] lands in lane j + 16 * (i / 4), register i % 4, so a lane owns four
//   consecutive output columns of one row.
// The weights go straight from HBM to registers (each weight element of a
// tile is read by exactly one lane); K is walked in one fixed order for every
// tile, so a row's result does not depend on the tile it falls in.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace item {

template <int WF>
struct FmtTraits;
// KS: K elements one stage covers (4 lane groups x one 16-byte load per lane).
template <>
struct FmtTraits<kBF16> { static constexpr int KS = 32; };
template <>
struct FmtTraits<kF32> { static constexpr int KS = 16; };
template <>
struct FmtTraits<kI8> { static constexpr int KS = 64; };
template <>
struct FmtTraits<kQ4> { static constexpr int KS = 128; };
template <>
struct FmtTraits<kMX4> { static constexpr int KS = 128; };  // one 16x16x128 scaled MFMA per stage

// Stages per batch: a batch is what one wave keeps in flight while it computes
// the previous one.  Fewer stages for tall tiles keeps the B registers bounded.
#ifndef MOE_STAGES_SMALL
#define MOE_STAGES_SMALL 4
#endif
#ifndef MOE_STAGES_LARGE
#define MOE_STAGES_LARGE 2
#endif
template <int WF, int NSUB>
constexpr int stages() {
  return WF == kQ4 || WF == kMX4 ? 1 : (NSUB <= 2 ? MOE_STAGES_SMALL : MOE_STAGES_LARGE);
}

struct Kp {  // kernel parameters
  const void* act;
  const int8_t* act_q;
  const float* act_scale;
  const int32_t* row_token;
  const int32_t* sched;
  const void* w;
  const void* w_scale;
  const void* w_min;
  void* out;
  int K, N, T, R;
  int tiles_ub;     // upper bound on small tiles (the grid's size), <= the schedule's capacity
  int act_row0;     // down: row r of the activations (and of act_scale) is stored at r - act_row0
};

// Stores that other workgroups of the same launch read after a grid barrier
// (the fused decode layer) use agent-scope relaxed atomic stores: the sc1
// cache policy writes them through to memory instead of leaving them dirty in
// the XCD's L2, where another XCD's loads would not see them.
__device__ __forceinline__ void st_coh64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh64(const void* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Weight operand of one stage for one 16-row block (A operand).
struct AStage {
  u32x4 v;               // raw 16 bytes
  Q4Block blk;           // 4-bit block parameters
  uint32_t sc;           // MXFP4: the lane's E8M0 block scale byte
};

template <int WF>
__device__ __forceinline__ void load_a(AStage& s, const Kp& p, size_t wrow, int k0, int q) {
  if constexpr (WF == kBF16) {
    s.v = ld16((const uint16_t*)p.w + wrow * p.K + k0 + 8 * q);
  } else if constexpr (WF == kF32) {
    s.v = ld16((const float*)p.w + wrow * p.K + k0 + 4 * q);
  } else if constexpr (WF == kI8) {
    s.v = ld16((const int8_t*)p.w + wrow * p.K + k0 + 16 * q);
  } else if constexpr (WF == kMX4) {
    // lane group q holds the whole 32-element block k0/32 + q and its scale
    s.v = ld16((const uint8_t*)p.w + wrow * (size_t)(p.K / 2) + k0 / 2 + 16 * q);
    s.sc = ((const uint8_t*)p.w_scale)[wrow * (size_t)(p.K / 32) + k0 / 32 + q];
  } else {
    // lane group q holds the whole 32-code block k0/32 + q
    s.v = ld16((const uint8_t*)p.w + wrow * (size_t)(p.K / 2) + k0 / 2 + 16 * q);
    const size_t b = wrow * (size_t)(p.K / 32) + k0 / 32 + q;
    s.blk = q4_block(((const uint16_t*)p.w_scale)[b], ((const uint16_t*)p.w_min)[b]);
  }
}

// Activation operand of one stage for one 16-row block (B operand).
template <int WF>
struct BStage {
  u32x4 v[WF == kQ4 ? 4 : WF == kMX4 ? 2 : 1];
  uint32_t sc;  // MXFP8 activations: the lane's E8M0 block scale byte
};

template <int WF>
__device__ __forceinline__ void load_b(BStage<WF>& s, const Kp& p, size_t arow, int k0, int q) {
  if constexpr (WF == kBF16) {
    s.v[0] = ld16((const uint16_t*)p.act + arow * p.K + k0 + 8 * q);
  } else if constexpr (WF == kF32) {
    s.v[0] = ld16((const float*)p.act + arow * p.K + k0 + 4 * q);
  } else if constexpr (WF == kI8) {
    s.v[0] = ld16(p.act_q + arow * p.K + k0 + 16 * q);
  } else if constexpr (WF == kMX4) {
    // The FP8 operand of the 16x16x128 scaled MFMA: lane group q holds K
    // k0+16q .. +15 in its first four registers and k0+64+16q .. +15 in the
    // last four; its scale byte is that of block k0/32 + q, as for the FP4
    // operand (whose lane group q holds the whole block).
    s.v[0] = ld16(p.act_q + arow * p.K + k0 + 16 * q);
    s.v[1] = ld16(p.act_q + arow * p.K + k0 + 64 + 16 * q);
    s.sc = reinterpret_cast<const uint8_t*>(p.act_scale)[arow * (size_t)(p.K / 32) + k0 / 32 + q];
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) s.v[m] = ld16((const uint16_t*)p.act + arow * p.K + k0 + 32 * q + 8 * m);
  }
}

template <int WF>
using Acc = typename std::conditional<WF == kI8, i32x4, f32x4>::type;

// One stage: NA weight blocks x NSUB token blocks.
template <int WF, int NA, int NSUB>
__device__ __forceinline__ void mma_stage(Acc<WF> (&acc)[NA][NSUB], const AStage (&a)[NA],
                                          const BStage<WF> (&b)[NSUB]) {
#pragma unroll
  for (int n = 0; n < NA; ++n) {
    if constexpr (WF == kQ4) {
      u32x4 w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) w[m] = q4_decode8(a[n].v[m], a[n].blk);
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[n][s] = mfma_bf16_16x16x32(w[m], b[s].v[m], acc[n][s]);
    } else {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if constexpr (WF == kBF16) {
          acc[n][s] = mfma_bf16_16x16x32(a[n].v, b[s].v[0], acc[n][s]);
        } else if constexpr (WF == kF32) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[n][s] = mfma_f32_16x16x4(__uint_as_float(a[n].v[j]), __uint_as_float(b[s].v[0][j]), acc[n][s]);
        } else if constexpr (WF == kMX4) {
          acc[n][s] = mfma_mx4_mx8_16x16x128(a[n].v, a[n].sc, b[s].v[0], b[s].v[1], b[s].sc, acc[n][s]);
        } else {
          acc[n][s] = mfma_i8_16x16x64(a[n].v, b[s].v[0], acc[n][s]);
        }
      }
    }
  }
}

__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }

// SiLU of the int8 path with each fp32 operation rounded once and exp taken
// in fp64 then rounded to fp32.  The device fp64 exp is accurate to about one
// fp64 ulp, so fp32(exp(-g)) agrees with the host's (also fp64 exp, rounded)
// except when exp(-g) falls within a few fp64 ulps of an fp32 rounding
// boundary (probability about 2^-29 per value).
__device__ __forceinline__ float silu_exact(float g) {
  const float e = (float)exp(-(double)g);
  return __fdiv_rn(g, __fadd_rn(1.0f, e));
}

template <bool kCoh>
__device__ __forceinline__ void store4(const Kp& p, bool f32, int r, int col, const float v[4]) {
  if (f32) {
    float* o = (float*)p.out + (size_t)r * p.N + col;
    if constexpr (kCoh) {
      st_coh64(o, ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]));
      st_coh64(o + 2, ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]));
    } else {
      *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
    }
  } else {
    uint16_t* o = (uint16_t*)p.out + (size_t)r * p.N + col;
    const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
    if constexpr (kCoh) st_coh64(o, ((uint64_t)hi << 32) | lo);
    else *reinterpret_cast<u32x2*>(o) = u32x2{lo, hi};
  }
}

// Gate/up epilogue: SwiGLU of the pair (gate block, up block); lane owns
// output columns col .. col+3 of row r.
template <int WF, bool kCoh>
__device__ __forceinline__ void store_gu(const Kp& p, int r, int col, const Acc<WF>& g, const Acc<WF>& u, int group,
                                         int tok) {
  float v[4];
  if constexpr (WF == kI8) {
    const float xs = p.act_scale[tok];
    const float* ws = (const float*)p.w_scale + (size_t)group * 2 * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ag = __fmul_rn(__fmul_rn((float)g[i], xs), ws[col + i]);
      const float au = __fmul_rn(__fmul_rn((float)u[i], xs), ws[p.N + col + i]);
      v[i] = __fmul_rn(silu_exact(ag), au);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = silu_fast(g[i]) * u[i];
  }
  store4<kCoh>(p, WF == kF32 || WF == kI8 || WF == kMX4, r, col, v);
}

template <int WF, bool kCoh>
__device__ __forceinline__ void store_down(const Kp& p, int r, int col, const Acc<WF>& y, int group) {
  float v[4];
  if constexpr (WF == kI8) {
    const float hs = p.act_scale[r - p.act_row0];
    const float* ws = (const float*)p.w_scale + (size_t)group * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(__fmul_rn((float)y[i], hs), ws[col + i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = y[i];
  }
  store4<kCoh>(p, WF == kF32 || WF == kI8 || WF == kMX4, r, col, v);
}

// 16-row weight blocks per work item: 4 (gate/up: 32 gate/up pairs; down: 64
// columns), or 2 for the gate/up GEMM of decode steps (16 pairs, twice the
// items, so that the few touched experts' weights spread over all CUs).
constexpr int kItemBlocks = 4;

#ifndef MOE_SPLIT_GU
#define MOE_SPLIT_GU 4
#endif
#ifndef MOE_SPLIT_DN
#define MOE_SPLIT_DN 2
#endif
// Waves per workgroup; they split an item's K range.
template <bool kGU>
constexpr int split() { return kGU ? MOE_SPLIT_GU : MOE_SPLIT_DN; }

// One work item: rows [row0, row0 + rows) of one group against four 16-row
// weight blocks: gate rows n0.., n0+16.. and up rows n0.., n0+16.. of the
// group for gate/up (32 output columns), or output columns n0 .. n0+63 for
// down.  Each activation fragment feeds all four blocks.  The four waves of the workgroup take
// consecutive quarters of the K batches; each walks its quarter in batches of
// U stages with the next batch's loads in flight while the current one
// computes.  Partial sums meet in LDS and are added in wave order
// ((w0 + w1) + w2) + w3, so the result does not depend on scheduling.
// `wave` is the wave's index among the item's waves; every thread of the
// workgroup must call this (it holds one workgroup barrier), with
// active = false for waves that have no item this round (no loads, no
// stores).  kCoh: outputs are stored for other workgroups of the launch.
template <int WF, bool kGU, int NSUB, int NA, bool kCoh = false>
__device__ __forceinline__ void gemm_item(const Kp& p, int group, int row0, int rows, int n0, Acc<WF>* red, int wave,
                                          bool active = true) {
  constexpr int KS = FmtTraits<WF>::KS;
  constexpr int U = stages<WF, NSUB>();
  constexpr int KB = KS * U;
  static_assert(NA == 4 || (NA == 2 && kGU), "item shapes");
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, q = lane / 16;
  size_t wrow[NA];
  if constexpr (kGU && NA == 2) {
    wrow[0] = (size_t)group * 2 * p.N + n0 + lr;  // gate rows
    wrow[1] = wrow[0] + p.N;                      // up rows
  } else if constexpr (kGU) {
    wrow[0] = (size_t)group * 2 * p.N + n0 + lr;  // gate rows
    wrow[1] = wrow[0] + 16;
    wrow[2] = wrow[0] + p.N;                      // up rows
    wrow[3] = wrow[1] + p.N;
  } else {
#pragma unroll
    for (int n = 0; n < NA; ++n) wrow[n] = (size_t)group * p.N + n0 + 16 * n + lr;
  }
  size_t arow[NSUB];
  int tok[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int rr = (16 * s + lr < rows) ? row0 + 16 * s + lr : row0;
    if constexpr (kGU) {
      tok[s] = active ? min(max(p.row_token[rr], 0), p.T - 1) : 0;
      arow[s] = (size_t)tok[s];
    } else {
      tok[s] = rr;
      arow[s] = (size_t)(rr - p.act_row0);
    }
  }
  Acc<WF> acc[NA][NSUB];
#pragma unroll
  for (int n = 0; n < NA; ++n)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[n][s] = Acc<WF>{0, 0, 0, 0};

  AStage a0[U][NA], a1[U][NA];
  BStage<WF> b0[U][NSUB], b1[U][NSUB];
  // Weight loads need only the tile; token loads (gate/up) also need the
  // rows' tokens, so every batch issues its weights first.
  auto load_w = [&](AStage (&a)[U][NA], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NA; ++n) load_a<WF>(a[u][n], p, wrow[n], kb + u * KS, q);
  };
  auto load_t = [&](BStage<WF> (&b)[U][NSUB], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) load_b<WF>(b[u][s], p, arow[s], kb + u * KS, q);
  };
  auto compute = [&](const AStage (&a)[U][NA], const BStage<WF> (&b)[U][NSUB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) mma_stage<WF, NA, NSUB>(acc, a[u], b[u]);
  };
  // The waves' K ranges are cut in units of the largest batch (a one-block
  // tile's), the same for every tile height, so a row's partial sums never
  // depend on the tile it falls in; a wave walks its range in batches of KB.
  constexpr int KP = KS * stages<WF, 1>();
  static_assert(KP % KB == 0, "batch must divide the partition unit");
  constexpr int kSplit = split<kGU>();
  const int units = p.K / KP;
  const int ubeg = wave * units / kSplit, uend = (wave + 1) * units / kSplit;
  const int nb = active ? (uend - ubeg) * (KP / KB) : 0;
  const int kbase = ubeg * KP;
  // The first two batches.  Gate/up: both batches' weights go out before
  // the token loads, which wait for the rows' tokens; down (rows index h
  // directly): batch by batch, so the first batch does not wait for the
  // second (loads retire in order).
  if constexpr (kGU) {
    if (nb > 0) load_w(a0, kbase);
    if (nb > 1) load_w(a1, kbase + KB);
    if (nb > 0) load_t(b0, kbase);
    if (nb > 1) load_t(b1, kbase + KB);
  } else {
    if (nb > 0) {
      load_w(a0, kbase);
      load_t(b0, kbase);
    }
    if (nb > 1) {
      load_w(a1, kbase + KB);
      load_t(b1, kbase + KB);
    }
  }
  for (int i = 0; i < nb; i += 2) {
    compute(a0, b0);
    if (i + 2 < nb) {
      load_w(a0, kbase + (i + 2) * KB);
      load_t(b0, kbase + (i + 2) * KB);
    }
    if (i + 1 < nb) compute(a1, b1);
    if (i + 3 < nb) {
      load_w(a1, kbase + (i + 3) * KB);
      load_t(b1, kbase + (i + 3) * KB);
    }
  }
  // Cross-wave reduction: waves 1..3 park their partials, wave 0 adds them in order.
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) red[(((wave - 1) * NA + n) * NSUB + s) * kWave + lane] = acc[n][s];
  }
  __syncthreads();
  if (wave != 0 || !active) return;
#pragma unroll
  for (int w = 1; w < kSplit; ++w)
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[n][s] += red[(((w - 1) * NA + n) * NSUB + s) * kWave + lane];
  // D[i][j] of block (n, s) is in lane j + 16 * (i / 4), register i % 4:
  // this lane holds columns 4q .. 4q+3 of the block for row 16 s + lr.
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if (16 * s + lr < rows) {
      const int r = row0 + 16 * s + lr;
      if constexpr (kGU && NA == 2) {
        store_gu<WF, kCoh>(p, r, n0 + 4 * q, acc[0][s], acc[1][s], group, tok[s]);
      } else if constexpr (kGU) {
        store_gu<WF, kCoh>(p, r, n0 + 4 * q, acc[0][s], acc[2][s], group, tok[s]);
        store_gu<WF, kCoh>(p, r, n0 + 16 + 4 * q, acc[1][s], acc[3][s], group, tok[s]);
      } else {
#pragma unroll
        for (int n = 0; n < NA; ++n) store_down<WF, kCoh>(p, r, n0 + 16 * n + 4 * q, acc[n][s], group);
      }
    }
  }
}

// The down item of gemm_item<WF, false, 1, 4> in two halves, so that its
// weight loads can be sent before the activations exist (before a grid
// barrier): issue() loads the wave's weights, finish() loads the token rows,
// runs the MFMAs, reduces across the waves and stores -- the same loads into
// the same batches and the same MFMA order as gemm_item, so the same bits.  A
// wave's share of K must fit in kBatches of gemm_item's register batches
// (two: K <= 512 for bf16 and 4-bit weights, K <= 1024 for int8; one: half
// that); issue() sends the first kPre of them, finish() the rest.
template <int WF, int kBatches, int kPre = kBatches>
struct DownItem {
  static_assert(kBatches == 1 || kBatches == 2, "one or two batches");
  static_assert(kPre >= 1 && kPre <= kBatches, "batches sent early");
  static constexpr int NA = 4, NSUB = 1;
  static constexpr int KS = FmtTraits<WF>::KS, U = stages<WF, NSUB>(), KB = KS * U;
  AStage a0[U][NA], a1[kBatches == 2 ? U : 1][NA];
  size_t wrow[NA];
  int nb, kbase;

  __device__ __forceinline__ void issue(const Kp& p, int group, int n0, int wave, bool active) {
    constexpr int KP = KS * stages<WF, 1>();
    constexpr int kSplit = split<false>();
    const int lr = (threadIdx.x % kWave) % 16, q = (threadIdx.x % kWave) / 16;
#pragma unroll
    for (int n = 0; n < NA; ++n) wrow[n] = (size_t)group * p.N + n0 + 16 * n + lr;
    const int units = p.K / KP;
    const int ubeg = wave * units / kSplit, uend = (wave + 1) * units / kSplit;
    nb = active ? min(kBatches, (uend - ubeg) * (KP / KB)) : 0;
    kbase = ubeg * KP;
    if (nb > 0)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int n = 0; n < NA; ++n) load_a<WF>(a0[u][n], p, wrow[n], kbase + u * KS, q);
    if constexpr (kPre == 2) load_second(p);
  }
  __device__ __forceinline__ void load_second(const Kp& p) {
    if constexpr (kBatches == 2) {
      const int q = (threadIdx.x % kWave) / 16;
      if (nb > 1)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int n = 0; n < NA; ++n) load_a<WF>(a1[u][n], p, wrow[n], kbase + KB + u * KS, q);
    }
  }

  template <bool kCoh>
  __device__ __forceinline__ void finish(const Kp& p, int group, int row0, int rows, int n0, Acc<WF>* red, int wave,
                                         bool active) {
    const int lane = threadIdx.x % kWave, lr = lane % 16, q = lane / 16;
    const int rr = lr < rows ? row0 + lr : row0;
    const size_t arow = (size_t)(rr - p.act_row0);
    if constexpr (kPre == 1) load_second(p);
    Acc<WF> acc[NA][NSUB];
#pragma unroll
    for (int n = 0; n < NA; ++n) acc[n][0] = Acc<WF>{0, 0, 0, 0};
    BStage<WF> b0[U][NSUB];
    if (nb > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_b<WF>(b0[u][0], p, arow, kbase + u * KS, q);
#pragma unroll
      for (int u = 0; u < U; ++u) mma_stage<WF, NA, NSUB>(acc, a0[u], b0[u]);
    }
    if constexpr (kBatches == 2) {
      if (nb > 1) {
        BStage<WF> b1[U][NSUB];
#pragma unroll
        for (int u = 0; u < U; ++u) load_b<WF>(b1[u][0], p, arow, kbase + KB + u * KS, q);
#pragma unroll
        for (int u = 0; u < U; ++u) mma_stage<WF, NA, NSUB>(acc, a1[u], b1[u]);
      }
    }
    constexpr int kSplit = split<false>();
    if (wave > 0) {
#pragma unroll
      for (int n = 0; n < NA; ++n) red[((wave - 1) * NA + n) * kWave + lane] = acc[n][0];
    }
    __syncthreads();
    if (wave != 0 || !active) return;
#pragma unroll
    for (int w = 1; w < kSplit; ++w)
#pragma unroll
      for (int n = 0; n < NA; ++n) acc[n][0] += red[((w - 1) * NA + n) * kWave + lane];
    if (lr < rows) {
#pragma unroll
      for (int n = 0; n < NA; ++n) store_down<WF, kCoh>(p, row0 + lr, n0 + 16 * n + 4 * q, acc[n][0], group);
    }
  }
};

// Output columns one work item covers: 8 NA gate/up pairs, or 16 NA down columns.
template <bool kGU, int NA>
constexpr int item_cols() { return kGU ? 8 * NA : 16 * NA; }


}  // namespace item
}  // namespace moe
