// Big-tile grouped GEMMs for groups with many rows (compute-bound prefill):
// gate/up + SwiGLU and down over the big tiles of the schedule, bf16 or 4-bit
// block weights.
//
// Where a group has hundreds of rows the layer is bound by the matrix cores,
// not by weight bytes, and the weight operand must be reused over many tokens
// from on-chip memory.  A block owns 128 weight rows x 256 token rows; both
// operands of each 64-wide K stage are staged in LDS (double-buffered: the
// next stage's global loads are in flight while the current one computes);
// 4-bit codes are dequantised to bf16 once per block by the thread that loads
// them, before they reach LDS, so each weight is decoded once per 256 tokens.
// Four waves each compute a 64 x 128 tile with v_mfma_f32_16x16x32_bf16.
//
// The shared expert and every routed expert go through the same launch; the
// grouping itself is the point of the pages' "concatenated-expert" fix
// ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM", section "The
// fix") and of "the lever is M>1" ("MoE Decode Partition and Submit Floor",
// M2 update).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBN = 128;                 // weight rows per block
constexpr int kBM = kBigTileRows;        // token rows per block
constexpr int kBK = 64;                  // K per stage
constexpr int kRow = kBK * 2 + 16;       // LDS bytes per staged row (bf16 + 16 B pad)
constexpr int kStageBytes = (kBN + kBM) * kRow;
constexpr int kThreads = 256;
constexpr int kDepth = 4;              // stages of global loads in flight

struct Bp {
  const void* act;          // x [T][K] (gate/up, gathered by row_token) or h [R][K] (down), bf16
  const int32_t* row_token;
  const int32_t* sched;
  const void* w;
  const void* w_scale;
  const void* w_min;
  void* out;                // h [R][N] or y [R][N], bf16
  int K, N, T;
};

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint32_t deq2(uint32_t lo_byte, uint32_t hi_byte, float sc, float mn) {
  return pack_bf16x2(fmaf(sc, (float)lo_byte, mn), fmaf(sc, (float)hi_byte, mn));
}

// Weight row (index into [G][rows][K]) of staged A row j of a block.
template <bool kGU>
__device__ __forceinline__ size_t a_row(const Bp& p, int group, int n0, int j) {
  if constexpr (kGU) {
    // 64 gate/up pairs: wave half wn = j / 64 holds gate rows n0+32wn .. +31, then the matching up rows.
    const int wn = j / 64, jj = j % 64;
    const int i = n0 + 32 * wn + (jj % 32);
    return (size_t)group * 2 * p.N + (jj < 32 ? i : p.N + i);
  } else {
    return (size_t)group * p.N + n0 + j;
  }
}

template <int WF>
struct AReg {
  u32x4 v[WF == kQ4 ? 1 : 4];
  uint32_t sc, mn;  // fp16 bits (zero-extended), converted when the stage is stored
};

// The prefetch loads are issued as opaque vector loads so the compiler cannot
// sink them next to their use (which would expose the full memory latency at
// every stage); completion is awaited explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ u32x4 gload16(const void* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}
__device__ __forceinline__ uint32_t gload_u16(const void* p) {
  uint32_t r;
  asm volatile("global_load_ushort %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}
// Vector-memory loads each thread issues per stage.
template <int WF>
constexpr int loads_per_stage() { return WF == kQ4 ? 1 + 2 + 8 : 4 + 8; }

// Wait until this thread's loads of all but the newest n stages have landed.
template <int WF, int n>
__device__ __forceinline__ void wait_stages() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n * loads_per_stage<WF>()) : "memory");
}
// Make later uses of a stage's registers depend on the wait above.
template <int WF>
__device__ __forceinline__ void tie(AReg<WF>& a, u32x4 (&b)[8]) {
#pragma unroll
  for (int i = 0; i < (WF == kQ4 ? 1 : 4); ++i) asm volatile("" : "+v"(a.v[i]));
  if constexpr (WF == kQ4) asm volatile("" : "+v"(a.sc), "+v"(a.mn));
#pragma unroll
  for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(b[c]));
}

// Global -> registers for one stage.  A: thread t covers row t / 2, half t % 2
// of the stage (32 K); B: thread t covers token row t (64 K).
template <int WF, bool kGU>
__device__ __forceinline__ void load_stage(const Bp& p, AReg<WF>& a, u32x4 (&b)[8], size_t arow, size_t brow,
                                           int k0) {
  const int half = threadIdx.x % 2;
  if constexpr (WF == kQ4) {
    const int kb = k0 + 32 * half;  // one 32-code block
    a.v[0] = gload16((const uint8_t*)p.w + arow * (size_t)(p.K / 2) + kb / 2);
    const size_t blk = arow * (size_t)(p.K / 32) + kb / 32;
    a.sc = gload_u16((const uint16_t*)p.w_scale + blk);
    a.mn = gload_u16((const uint16_t*)p.w_min + blk);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) a.v[c] = gload16((const uint16_t*)p.w + arow * p.K + k0 + 32 * half + 8 * c);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) b[c] = gload16((const uint16_t*)p.act + brow * p.K + k0 + 8 * c);
}

// Registers -> LDS for one stage (4-bit codes decoded here, once per block).
template <int WF>
__device__ __forceinline__ void store_stage(uint8_t* st, const AReg<WF>& a, const u32x4 (&b)[8]) {
  const int t = threadIdx.x;
  uint8_t* arow = st + (t / 2) * kRow + 64 * (t % 2);
  if constexpr (WF == kQ4) {
    const float sc = half_bits_to_f32((uint16_t)a.sc), mn = half_bits_to_f32((uint16_t)a.mn);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w = a.v[0][m];  // codes 8m .. 8m+7 of the block
      const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
      u32x4 d;
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = deq2((lo >> (8 * q)) & 0xffu, (hi >> (8 * q)) & 0xffu, sc, mn);
      *reinterpret_cast<u32x4*>(arow + 16 * m) = d;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(arow + 16 * c) = a.v[c];
  }
  uint8_t* brow = st + (kBN + t) * kRow;
#pragma unroll
  for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(brow + 16 * c) = b[c];
}

__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }

template <int WF, bool kGU>
__global__ __launch_bounds__(kThreads) void big_gemm_kernel(Bp p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
  const int n_big = p.sched[kSchedBig];
  const int cols = kGU ? kBN / 2 : kBN;  // output columns per block
  const int per_tile = p.N / cols;
  const int w = blockIdx.x;
  if (w >= n_big * per_tile) return;
  const int mt = w / per_tile, nt = w % per_tile;
  const int32_t* tile = p.sched + p.sched[kSchedBigStart] + (size_t)mt * kTileInts;
  const int group = tile[0], row0 = tile[1], rows = tile[2];
  const int n0 = nt * cols;

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int lr = lane % 16, q = lane / 16;
  const int wn = wave & 1, wm = wave >> 1;
  // loader rows
  const size_t arow = a_row<kGU>(p, group, n0, t / 2);
  const int rr = t < rows ? row0 + t : row0;
  const size_t brow = kGU ? (size_t)min(max(p.row_token[rr], 0), p.T - 1) : (size_t)rr;

  f32x4 acc[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Register ring of kDepth stages: the global loads of stage s + kDepth are
  // issued while stage s computes, so kDepth stages of loads are in flight.
  AReg<WF> areg[kDepth];
  u32x4 breg[kDepth][8];
  // K is a multiple of 256, so the stage count is a multiple of the ring depth.
  // Every iteration refills one slot (near the end with the last stage again,
  // an L2 hit), which keeps the number of loads in flight the same everywhere
  // and lets each wait be a constant.
  const int nk = p.K / kBK;
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_stage<WF, kGU>(p, areg[d], breg[d], arow, brow, d * kBK);
  wait_stages<WF, kDepth - 1>();
  tie<WF>(areg[0], breg[0]);
  store_stage<WF>(lds, areg[0], breg[0]);
  __syncthreads();
  for (int s0 = 0; s0 < nk; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = s0 + d;
      // slot d held stage s, already in LDS: refill it
      load_stage<WF, kGU>(p, areg[d], breg[d], arow, brow, min(s + kDepth, nk - 1) * kBK);
      const uint8_t* st = lds + (s & 1) * kStageBytes;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 af[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
          af[b] = *reinterpret_cast<const u32x4*>(st + (wn * 64 + 16 * b + lr) * kRow + kk * 64 + 16 * q);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 bf =
              *reinterpret_cast<const u32x4*>(st + (kBN + wm * 128 + 16 * c + lr) * kRow + kk * 64 + 16 * q);
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[b][c] = mfma_bf16_16x16x32(af[b], bf, acc[b][c]);
        }
      }
      // stage s + 1 sits in slot dn; the kDepth - 1 stages issued after it stay in flight
      const int dn = (d + 1) % kDepth;
      wait_stages<WF, kDepth - 1>();
      tie<WF>(areg[dn], breg[dn]);
      if (s + 1 < nk) store_stage<WF>(lds + ((s + 1) & 1) * kStageBytes, areg[dn], breg[dn]);
      __syncthreads();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the ring's last refills, before its registers are reused
  // Epilogue: block b's D[i][j] is in lane j + 16 * (i / 4), register i % 4.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int tr = wm * 128 + 16 * c + lr;
    if (tr >= rows) continue;
    const int r = row0 + tr;
    if constexpr (kGU) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = n0 + 32 * wn + 16 * b + 4 * q;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu_fast(acc[b][c][i]) * acc[b + 2][c][i];
        u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = n0 + 64 * wn + 16 * b + 4 * q;
        u32x2 o = {pack_bf16x2(acc[b][c][0], acc[b][c][1]), pack_bf16x2(acc[b][c][2], acc[b][c][3])};
        *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
      }
    }
  }
}

template <bool kGU>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  if (a.wfmt != kBF16 && a.wfmt != kQ4) return hipErrorInvalidValue;
  Bp p{a.act, a.row_token, a.sched, a.w, a.w_scale, a.w_min, a.out, a.K, a.N, a.T};
  const int cols = kGU ? kBN / 2 : kBN;
  const int64_t items = ((int64_t)a.R / kBigTileMin + 1) * (a.N / cols);  // each big tile has >= 128 rows
  if (items > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  if (a.wfmt == kQ4)
    hipLaunchKernelGGL((big_gemm_kernel<kQ4, kGU>), dim3(items), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((big_gemm_kernel<kBF16, kGU>), dim3(items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_big_gate_up(const GemmArgs& a, hipStream_t stream) { return launch<true>(a, stream); }
hipError_t launch_big_down(const GemmArgs& a, hipStream_t stream) { return launch<false>(a, stream); }

}  // namespace moe
