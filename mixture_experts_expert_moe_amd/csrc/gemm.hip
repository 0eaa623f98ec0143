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
#include "gemm_item.hpp"

namespace moe {
namespace {

using namespace item;

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
    case 1: gemm_item<WF, kGU, 1, NA>(p, group, row0, rows, n0, red, threadIdx.x / kWave); break;
    case 2: gemm_item<WF, kGU, kSub >= 2 ? 2 : 1, NA>(p, group, row0, rows, n0, red, threadIdx.x / kWave); break;
    case 3: gemm_item<WF, kGU, kSub >= 3 ? 3 : 1, NA>(p, group, row0, rows, n0, red, threadIdx.x / kWave); break;
    default: gemm_item<WF, kGU, kSub >= 4 ? 4 : 1, NA>(p, group, row0, rows, n0, red, threadIdx.x / kWave); break;
  }
}

Kp kernel_params(const GemmArgs& a, int64_t tiles) {
  return Kp{a.act, a.act_q, a.act_scale, a.row_token, a.sched, a.w, a.w_scale, a.w_min, a.out, a.K, a.N, a.T, a.R, (int)tiles, 0};
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
        case kMX4: return launch_fmt<kMX4, true, 4, 2>(a, stream);
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
    case kMX4: return launch_fmt<kMX4, kGU, 2>(a, stream);  // 32-row items: no spills at two waves per SIMD
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_up(const GemmArgs& a, hipStream_t stream) { return launch<true>(a, stream); }
hipError_t launch_down(const GemmArgs& a, hipStream_t stream) { return launch<false>(a, stream); }

}  // namespace moe
