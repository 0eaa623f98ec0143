// Grouped expert GEMMs: gate/up + SwiGLU (moe_grouped_gemm_gu) and down
// (moe_grouped_gemm_down), each one launch over the device-resident tile
// schedule, every expert (and the shared expert) included.  The grid is sized
// on the host from an upper bound on the work items (one workgroup per item;
// workgroups past the schedule's item count exit at once), so no host-device
// round trip is needed to size it.
//
// Why one launch: dispatching experts one at a time serialises the layer
// ("~2.7s fixed per-request TTFT = ~4,900 serialized per-expert NPU execs",
// section "Evidence"); the fix is one run per operator per layer over all the
// experts' rows (same page, section "The fix"), and a chunk of rows routed
// per token instead of grouped was the slow path in Atlas issue #145 (the
// 2026-10-27 trace comment).  The shared expert is one more group of the same
// launch, as the fused "gate_up_shared" / "silu_down_shared" kernels there do.
//
// Work item = (tile of <= 64 rows of one group) x (32 gate/up pairs -- 16 for
// decode steps of at most 16 tokens, where the few touched experts would
// otherwise occupy too few CUs -- or 64 down columns); one workgroup per item,
// its waves splitting K.  Every output element goes through the same
// instructions whatever the item shape, so results do not depend on it.
// Within an item:
//   MFMA A operand = 16 weight rows (lane l: row l % 16, K-group l / 16),
//   MFMA B operand = 16 token rows  (lane l: row l % 16, same K-group),
//   D[i][j] lands in lane j + 16 * (i / 4), register i % 4, so a lane owns four
//   consecutive output columns of one row.
// The weights go straight from HBM to registers (each weight element of a
// tile is read by exactly one lane); K is walked in one fixed order for every
// tile, so a row's result does not depend on the tile it falls in.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

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
  return WF == kQ4 ? 1 : (NSUB <= 2 ? MOE_STAGES_SMALL : MOE_STAGES_LARGE);
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
};

// Weight operand of one stage for one 16-row block (A operand).
struct AStage {
  u32x4 v;               // raw 16 bytes
  Q4Block blk;           // 4-bit block parameters
};

template <int WF>
__device__ __forceinline__ void load_a(AStage& s, const Kp& p, size_t wrow, int k0, int q) {
  if constexpr (WF == kBF16) {
    s.v = ld16((const uint16_t*)p.w + wrow * p.K + k0 + 8 * q);
  } else if constexpr (WF == kF32) {
    s.v = ld16((const float*)p.w + wrow * p.K + k0 + 4 * q);
  } else if constexpr (WF == kI8) {
    s.v = ld16((const int8_t*)p.w + wrow * p.K + k0 + 16 * q);
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
  u32x4 v[WF == kQ4 ? 4 : 1];
};

template <int WF>
__device__ __forceinline__ void load_b(BStage<WF>& s, const Kp& p, size_t arow, int k0, int q) {
  if constexpr (WF == kBF16) {
    s.v[0] = ld16((const uint16_t*)p.act + arow * p.K + k0 + 8 * q);
  } else if constexpr (WF == kF32) {
    s.v[0] = ld16((const float*)p.act + arow * p.K + k0 + 4 * q);
  } else if constexpr (WF == kI8) {
    s.v[0] = ld16(p.act_q + arow * p.K + k0 + 16 * q);
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

__device__ __forceinline__ void store4(const Kp& p, bool f32, int r, int col, const float v[4]) {
  if (f32) {
    f32x4 o = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>((float*)p.out + (size_t)r * p.N + col) = o;
  } else {
    u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
  }
}

// Gate/up epilogue: SwiGLU of the pair (gate block, up block); lane owns
// output columns col .. col+3 of row r.
template <int WF>
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
  store4(p, WF == kF32 || WF == kI8, r, col, v);
}

template <int WF>
__device__ __forceinline__ void store_down(const Kp& p, int r, int col, const Acc<WF>& y, int group) {
  float v[4];
  if constexpr (WF == kI8) {
    const float hs = p.act_scale[r];
    const float* ws = (const float*)p.w_scale + (size_t)group * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(__fmul_rn((float)y[i], hs), ws[col + i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = y[i];
  }
  store4(p, WF == kF32 || WF == kI8, r, col, v);
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
template <int WF, bool kGU, int NSUB, int NA>
__device__ __forceinline__ void gemm_item(const Kp& p, int group, int row0, int rows, int n0, Acc<WF>* red) {
  constexpr int KS = FmtTraits<WF>::KS;
  constexpr int U = stages<WF, NSUB>();
  constexpr int KB = KS * U;
  static_assert(NA == 4 || (NA == 2 && kGU), "item shapes");
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
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
      tok[s] = min(max(p.row_token[rr], 0), p.T - 1);
      arow[s] = (size_t)tok[s];
    } else {
      tok[s] = rr;
      arow[s] = (size_t)rr;
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
  const int nb = (uend - ubeg) * (KP / KB);
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
  if (wave != 0) return;
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
        store_gu<WF>(p, r, n0 + 4 * q, acc[0][s], acc[1][s], group, tok[s]);
      } else if constexpr (kGU) {
        store_gu<WF>(p, r, n0 + 4 * q, acc[0][s], acc[2][s], group, tok[s]);
        store_gu<WF>(p, r, n0 + 16 + 4 * q, acc[1][s], acc[3][s], group, tok[s]);
      } else {
#pragma unroll
        for (int n = 0; n < NA; ++n) store_down<WF>(p, r, n0 + 16 * n + 4 * q, acc[n][s], group);
      }
    }
  }
}

// Output columns one work item covers: 8 NA gate/up pairs, or 16 NA down columns.
template <bool kGU, int NA>
constexpr int item_cols() { return kGU ? 8 * NA : 16 * NA; }

// One launch over (tile x column block) items; the grid is sized on the host
// from an upper bound and each workgroup takes one item, in schedule order
// (heaviest tiles first).  Workgroup b runs on XCD b % 8, so the column blocks
// of every tile are spread evenly over the eight XCDs.
#ifndef MOE_GEMM_WAVES_PER_SIMD
#define MOE_GEMM_WAVES_PER_SIMD 2
#endif
// Occupancy target: two waves per SIMD keeps enough loads in flight; the
// 4-bit path needs more registers for its dequantised operands, unless an
// item holds at most 32 rows (kSub = 2).
template <int WF, int kSub>
constexpr int waves_per_simd() { return WF == kQ4 && kSub > 2 ? 1 : MOE_GEMM_WAVES_PER_SIMD; }

// Items cover at most kSub 16-row blocks of a tile: a 64-row tile is cut
// into 64 / (16 kSub) row chunks, each its own item (an empty chunk exits).
// kSub = 4: one item per tile.  The 4-bit down GEMM of calls with enough
// tokens uses kSub = 2: half the registers, so twice the waves per SIMD and
// twice the loads in flight, for a second read of a tall tile's weights
// (the shared expert's); a few-token call (tiles of one block) keeps kSub = 4,
// where the extra, empty chunks only cost dispatch time.
template <int WF, bool kGU, int kSub, int NA>
__global__ __launch_bounds__(kWave* split<kGU>()) __attribute__((amdgpu_waves_per_eu(waves_per_simd<WF, kSub>())))
void grouped_gemm_kernel(Kp p) {
  __shared__ Acc<WF> red[(split<kGU>() > 1 ? split<kGU>() - 1 : 1) * NA * kSub * kWave];
  constexpr int kChunks = 4 / kSub, kChunkRows = 16 * kSub;
  static_assert(kChunks * kChunkRows == kTileRows, "chunks cover a tile");
  const int per_tile = p.N / item_cols<kGU, NA>();
  const int w = blockIdx.x;
  const int mt = w / (per_tile * kChunks), rem = w % (per_tile * kChunks);
  const int chunk = rem / per_tile, nt = rem % per_tile;
  // The tile entry is read together with the tile count (one round trip):
  // the clamped index stays inside the schedule, and an entry past the count
  // is never used.
  const i32x4 tile = *reinterpret_cast<const i32x4*>(p.sched + kSchedHeader + (size_t)min(mt, p.tiles_ub - 1) * kTileInts);
  const int n_tiles = p.sched[0];
  // both loads complete here, before the exit test (one round trip, not two)
  asm volatile("" ::"s"(tile[0]), "s"(tile[1]), "s"(tile[2]), "s"(n_tiles));
  if (mt >= n_tiles) return;
  const int group = tile[0], row0 = tile[1] + chunk * kChunkRows;
  const int rows = min(kChunkRows, tile[2] - chunk * kChunkRows);
  if (rows <= 0) return;
  const int n0 = nt * item_cols<kGU, NA>();
  switch ((rows + 15) / 16) {
    case 1: gemm_item<WF, kGU, 1, NA>(p, group, row0, rows, n0, red); break;
    case 2: gemm_item<WF, kGU, kSub >= 2 ? 2 : 1, NA>(p, group, row0, rows, n0, red); break;
    case 3: gemm_item<WF, kGU, kSub >= 3 ? 3 : 1, NA>(p, group, row0, rows, n0, red); break;
    default: gemm_item<WF, kGU, kSub >= 4 ? 4 : 1, NA>(p, group, row0, rows, n0, red); break;
  }
}

Kp kernel_params(const GemmArgs& a, int64_t tiles) {
  return Kp{a.act, a.act_q, a.act_scale, a.row_token, a.sched, a.w, a.w_scale, a.w_min, a.out, a.K, a.N, a.T, a.R, (int)tiles};
}

// Upper bound on small tiles: every non-empty group adds at most one partial tile.
int64_t tiles_upper_bound(const GemmArgs& a) {
  return (a.R + kTileRows - 1) / kTileRows + std::min<int64_t>(a.G, a.R);
}

template <int WF, bool kGU, int kSub, int NA = kItemBlocks>
hipError_t launch_fmt(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = tiles_upper_bound(a);
  const int64_t items = tiles * (a.N / item_cols<kGU, NA>()) * (4 / kSub);
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0 || grid > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_gemm_kernel<WF, kGU, kSub, NA>), dim3(grid), dim3(kWave * split<kGU>()), 0, stream,
                     kernel_params(a, tiles));
  return hipGetLastError();
}

// 4-bit down GEMMs of calls with at least this many tokens cut tiles into 32-row items.
constexpr int kQ4DownChunkMinT = 32;

#ifndef MOE_GU_HALF_ITEMS_MAX_T
#define MOE_GU_HALF_ITEMS_MAX_T 16
#endif
// Gate/up GEMMs of calls with at most this many tokens use 16-pair items.
constexpr int kGuHalfItemsMaxT = MOE_GU_HALF_ITEMS_MAX_T;

template <bool kGU>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  if constexpr (kGU) {
    if (a.T <= kGuHalfItemsMaxT && a.N % item_cols<true, 2>() == 0) {
      switch (a.wfmt) {
        case kF32: return launch_fmt<kF32, true, 4, 2>(a, stream);
        case kBF16: return launch_fmt<kBF16, true, 4, 2>(a, stream);
        case kI8: return launch_fmt<kI8, true, 4, 2>(a, stream);
        case kQ4: return launch_fmt<kQ4, true, 4, 2>(a, stream);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (a.wfmt) {
    case kF32: return launch_fmt<kF32, kGU, 4>(a, stream);
    case kBF16: return launch_fmt<kBF16, kGU, 4>(a, stream);
    case kI8: return launch_fmt<kI8, kGU, 4>(a, stream);
    case kQ4:
      if constexpr (!kGU) {
        if (a.T >= kQ4DownChunkMinT) return launch_fmt<kQ4, kGU, 2>(a, stream);
      }
      return launch_fmt<kQ4, kGU, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_up(const GemmArgs& a, hipStream_t stream) { return launch<true>(a, stream); }
hipError_t launch_down(const GemmArgs& a, hipStream_t stream) { return launch<false>(a, stream); }

}  // namespace moe
