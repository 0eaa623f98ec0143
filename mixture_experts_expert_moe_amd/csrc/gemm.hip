// Grouped expert GEMMs: gate/up + SwiGLU (moe_grouped_gemm_gu) and down
// (moe_grouped_gemm_down), each ONE persistent launch over the device-resident
// tile schedule, every expert (and the shared expert) included.
//
// Why one launch: dispatching experts one at a time serialises the layer
// ("~2.7s fixed per-request TTFT = ~4,900 serialized per-expert NPU execs",
// section "Evidence"); the fix is one run per operator per layer over all the
// experts' rows (same page, section "The fix"), and a chunk of rows routed
// per token instead of grouped was the slow path in Atlas issue #145 (the
// 2026-10-27 trace comment).  The shared expert is one more group of the same
// launch, as the fused "gate_up_shared" / "silu_down_shared" kernels there do.
//
// Work item = (tile of <= 64 rows of one group) x (16 output columns).  A
// workgroup is one wave; it takes items from a per-XCD counter (items of one
// XCD are a contiguous range, so the rows of a tile stay in that XCD's L2),
// then steals from the other XCDs.  Within an item:
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
// KS: K elements one stage covers; U: stages per batch of loads.
template <>
struct FmtTraits<kBF16> { static constexpr int KS = 32, U = 8; };
template <>
struct FmtTraits<kF32> { static constexpr int KS = 16, U = 8; };
template <>
struct FmtTraits<kI8> { static constexpr int KS = 64, U = 4; };
template <>
struct FmtTraits<kQ4> { static constexpr int KS = 128, U = 2; };

struct Kp {  // kernel parameters
  const void* act;
  const int8_t* act_q;
  const float* act_scale;
  const int32_t* row_token;
  int32_t* sched;
  const void* w;
  const void* w_scale;
  const void* w_min;
  void* out;
  int K, N, T, R;
};

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Eight 4-bit codes (one 32-bit word, code n at bits 4n) -> 8 bf16 of scale * q + min.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float sc, float mn) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  u32x4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float v0 = fmaf(sc, (float)((lo >> (8 * b)) & 0xffu), mn);
    const float v1 = fmaf(sc, (float)((hi >> (8 * b)) & 0xffu), mn);
    r[b] = pack_bf16x2(v0, v1);
  }
  return r;
}

// Weight operand of one stage for one weight row (A operand).
template <int WF>
struct AStage {
  u32x4 v;            // raw 16 bytes
  float sc = 0, mn = 0;  // 4-bit block parameters
};

template <int WF>
__device__ __forceinline__ void load_a(AStage<WF>& s, const Kp& p, size_t wrow, int k0, int q) {
  if constexpr (WF == kBF16) {
    s.v = ld16((const uint16_t*)p.w + wrow * p.K + k0 + 8 * q);
  } else if constexpr (WF == kF32) {
    s.v = ld16((const float*)p.w + wrow * p.K + k0 + 4 * q);
  } else if constexpr (WF == kI8) {
    s.v = ld16((const int8_t*)p.w + wrow * p.K + k0 + 16 * q);
  } else {
    s.v = ld16((const uint8_t*)p.w + wrow * (size_t)(p.K / 2) + k0 / 2 + 16 * q);
    const size_t b = wrow * (size_t)(p.K / 32) + k0 / 32 + q;
    s.sc = half_bits_to_f32(((const uint16_t*)p.w_scale)[b]);
    s.mn = half_bits_to_f32(((const uint16_t*)p.w_min)[b]);
  }
}

// Activation operand of one stage for one token row (B operand).
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

template <int WF>
__device__ __forceinline__ void mma(Acc<WF>& c, const AStage<WF>& a, const BStage<WF>& b) {
  if constexpr (WF == kBF16) {
    c = mfma_bf16_16x16x32(a.v, b.v[0], c);
  } else if constexpr (WF == kF32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = mfma_f32_16x16x4(__uint_as_float(a.v[j]), __uint_as_float(b.v[0][j]), c);
  } else if constexpr (WF == kI8) {
    c = mfma_i8_16x16x64(a.v, b.v[0], c);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = mfma_bf16_16x16x32(dequant8(a.v[m], a.sc, a.mn), b.v[m], c);
  }
}

__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }

// SiLU of the int8 path with each fp32 operation rounded once and exp taken
// in fp64 then rounded, i.e. fp32(exp(-g)) is the correctly rounded value.
__device__ __forceinline__ float silu_exact(float g) {
  const float e = (float)exp(-(double)g);
  return __fdiv_rn(g, __fadd_rn(1.0f, e));
}

template <int WF, bool kGU>
__device__ __forceinline__ void store_out(const Kp& p, int r, int col, const Acc<WF>& g_acc, const Acc<WF>& u_acc,
                                          int group, int tok) {
  float v[4];
  if constexpr (WF == kI8) {
    if constexpr (kGU) {
      const float xs = p.act_scale[tok];
      const float* ws = (const float*)p.w_scale + (size_t)group * 2 * p.N;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ag = __fmul_rn(__fmul_rn((float)g_acc[i], xs), ws[col + i]);
        const float au = __fmul_rn(__fmul_rn((float)u_acc[i], xs), ws[p.N + col + i]);
        v[i] = __fmul_rn(silu_exact(ag), au);
      }
    } else {
      const float hs = p.act_scale[r];
      const float* ws = (const float*)p.w_scale + (size_t)group * p.N;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(__fmul_rn((float)g_acc[i], hs), ws[col + i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = kGU ? silu_fast(g_acc[i]) * u_acc[i] : g_acc[i];
  }
  if constexpr (WF == kF32 || WF == kI8) {
    f32x4 o = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>((float*)p.out + (size_t)r * p.N + col) = o;
  } else {
    u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
  }
}

template <int WF, bool kGU, int NSUB>
__device__ __forceinline__ void gemm_item(const Kp& p, int group, int row0, int rows, int n0) {
  using Tr = FmtTraits<WF>;
  const int lane = threadIdx.x;
  const int lr = lane % 16, q = lane / 16;
  // Weight rows: gate/up -> W[g][n0 + lr] and W[g][N + n0 + lr] of [G][2N][K]; down -> W[g][n0 + lr] of [G][N][K].
  const size_t wrow_g = kGU ? (size_t)group * 2 * p.N + n0 + lr : (size_t)group * p.N + n0 + lr;
  const size_t wrow_u = wrow_g + p.N;
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
  Acc<WF> acc_g[NSUB], acc_u[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    acc_g[s] = Acc<WF>{0, 0, 0, 0};
    acc_u[s] = Acc<WF>{0, 0, 0, 0};
  }
  for (int kb = 0; kb < p.K; kb += Tr::KS * Tr::U) {
    AStage<WF> ag[Tr::U], au[Tr::U];
    BStage<WF> b[Tr::U][NSUB];
#pragma unroll
    for (int u = 0; u < Tr::U; ++u) {
      const int k0 = kb + u * Tr::KS;
      load_a<WF>(ag[u], p, wrow_g, k0, q);
      if constexpr (kGU) load_a<WF>(au[u], p, wrow_u, k0, q);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) load_b<WF>(b[u][s], p, arow[s], k0, q);
    }
#pragma unroll
    for (int u = 0; u < Tr::U; ++u) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        mma<WF>(acc_g[s], ag[u], b[u][s]);
        if constexpr (kGU) mma<WF>(acc_u[s], au[u], b[u][s]);
      }
    }
  }
  // Lane owns output columns n0 + 4q .. n0 + 4q + 3 of row row0 + 16 s + lr.
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if (16 * s + lr < rows) store_out<WF, kGU>(p, row0 + 16 * s + lr, n0 + 4 * q, acc_g[s], acc_u[s], group, tok[s]);
  }
}

template <int WF, bool kGU>
__global__ __launch_bounds__(kWave) void grouped_gemm_kernel(Kp p) {
  const int n_tiles = p.sched[0];
  const int nt_per_tile = p.N / 16;
  const int total = n_tiles * nt_per_tile;
  int* next = p.sched + (kGU ? kSchedGuNext : kSchedDnNext);
  int* done = p.sched + (kGU ? kSchedGuDone : kSchedDnDone);
  const int per = (total + kXcds - 1) / kXcds;
  const int home = blockIdx.x % kXcds;
  const int lane = threadIdx.x;
  for (int xi = 0; xi < kXcds; ++xi) {
    const int x = (home + xi) % kXcds;
    const int beg = x * per, end = min(total, beg + per);
    while (true) {
      int w = 0;
      if (lane == 0) w = atomicAdd(next + x, 1);
      w = __shfl(w, 0, kWave) + beg;
      if (w >= end) break;
      const int mt = w / nt_per_tile, nt = w % nt_per_tile;
      const int32_t* tile = p.sched + kSchedHeader + (size_t)mt * kTileInts;
      const int group = tile[0], row0 = tile[1], rows = tile[2];
      const int n0 = nt * 16;
      switch ((rows + 15) / 16) {
        case 1: gemm_item<WF, kGU, 1>(p, group, row0, rows, n0); break;
        case 2: gemm_item<WF, kGU, 2>(p, group, row0, rows, n0); break;
        case 3: gemm_item<WF, kGU, 3>(p, group, row0, rows, n0); break;
        default: gemm_item<WF, kGU, 4>(p, group, row0, rows, n0); break;
      }
    }
  }
  // The last workgroup out resets the counters for the next launch.
  __threadfence();
  if (lane == 0) {
    const int d = atomicAdd(done, 1);
    if (d == (int)gridDim.x - 1) {
      for (int x = 0; x < kXcds; ++x) atomicExch(next + x, 0);
      atomicExch(done, 0);
    }
  }
}

int grid_for(const GemmArgs& a, int items_bound) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  int grid = std::min(items_bound, cus * 8);
  grid = std::max(kXcds, (grid + kXcds - 1) / kXcds * kXcds);
  return grid;
}

template <bool kGU>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  Kp p{a.act, a.act_q, a.act_scale, a.row_token, const_cast<int32_t*>(a.sched), a.w, a.w_scale, a.w_min,
       a.out, a.K, a.N, a.T, a.R};
  // Upper bound on tiles: every non-empty group adds at most one partial tile.
  const int64_t tiles = (a.R + 63) / 64 + std::min<int64_t>(a.G, a.R);
  const int grid = grid_for(a, (int)std::min<int64_t>(tiles * (a.N / 16), 1 << 30));
  switch (a.wfmt) {
    case kF32: hipLaunchKernelGGL((grouped_gemm_kernel<kF32, kGU>), dim3(grid), dim3(kWave), 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((grouped_gemm_kernel<kBF16, kGU>), dim3(grid), dim3(kWave), 0, stream, p); break;
    case kI8: hipLaunchKernelGGL((grouped_gemm_kernel<kI8, kGU>), dim3(grid), dim3(kWave), 0, stream, p); break;
    case kQ4: hipLaunchKernelGGL((grouped_gemm_kernel<kQ4, kGU>), dim3(grid), dim3(kWave), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmArgs& a, hipStream_t stream) { return launch<true>(a, stream); }
hipError_t launch_down(const GemmArgs& a, hipStream_t stream) { return launch<false>(a, stream); }

}  // namespace moe
