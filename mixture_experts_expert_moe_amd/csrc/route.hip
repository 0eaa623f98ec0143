// Router: logits, top-k selection and gates (moe_route_topk).
//
// The routed layer sends each token to its k highest-scoring experts and
// weights their outputs by a softmax over those k scores ("top-8+shared" in
// "~2.7s fixed per-request TTFT ... concatenated-expert GEMM", section "The
// fix"; softmax placement and tie order are readings, see the header).
//
// Logits are accumulated in fp64 on the matrix cores (v_mfma_f64_16x16x4f64)
// and rounded once to fp32.  Every bf16 x bf16 (or fp32 x fp32) product is
// exact in fp64, so fp64 sums in different orders differ only in their last
// fp64 bits, and they round to the same fp32 logit except when the exact sum
// lies within those few fp64 ulps of an fp32 rounding boundary (probability
// about 2^-29 per logit).  Outside those rare cases the top-k decision does
// not depend on how the sum is blocked.
#include "common.hpp"
#include "kernels.hpp"
#include "route_permute.hpp"

namespace moe {
namespace {

// Waves per block, each taking an equal share of H: eight for partial sums
// over a slice of H (few blocks), four for whole logits (many blocks, but
// fewer than one 32 x 32 tile per CU, where route_logits32_kernel takes over).
template <bool kPartial> constexpr int route_waves() { return kPartial ? 8 : 4; }

// One block computes logits for 16 tokens x 16 experts.  Lane l of a wave
// holds token/expert (l % 16) and loads 8 consecutive h (one 16-byte load for
// bf16, two for fp32) at h = base + 8 * (l / 16); MFMA step s of the 8 uses
// element s, so A (x) and B (w_router) see the same permutation of K.
// kPartial: block (x, y, z) takes slice x of H (gridDim.x slices) for tokens
// 16 z .. 16 z + 15 and writes its fp64 partial sums, partials[slice][t][e],
// instead of logits.
template <bool kF32, bool kPartial>
__global__ __launch_bounds__(kWave* route_waves<kPartial>()) void route_logits_kernel(const void* __restrict__ x,
                                                                        const void* __restrict__ wr,
                                                                        const float* __restrict__ bias,
                                                                        float* __restrict__ logits,
                                                                        double* __restrict__ partials, int T, int H,
                                                                        int E) {
  constexpr int kRouteWaves = route_waves<kPartial>();
  __shared__ double part[kRouteWaves][16][17];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t0 = (kPartial ? blockIdx.z : blockIdx.x) * 16, e0 = blockIdx.y * 16;
  const int r = lane % 16, q = lane / 16;
  const int t = min(t0 + r, T - 1), e = min(e0 + r, E - 1);
  const int hs = kPartial ? H / gridDim.x : H;  // this block's share of H
  const int hq = hs / kRouteWaves;
  const int hbeg = (kPartial ? blockIdx.x * hs : 0) + wave * hq;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};  // two independent MFMA chains
  // Batches of kNb steps of 32 h: all loads of a batch are issued before its MFMAs.
  constexpr int kNb = kPartial ? 8 : 4;
  for (int h0 = hbeg; h0 < hbeg + hq; h0 += 32 * kNb) {
    u32x4 xv[kNb][kF32 ? 2 : 1], wv[kNb][kF32 ? 2 : 1];
#pragma unroll
    for (int u = 0; u < kNb; ++u) {
      const int hh = h0 + 32 * u + 8 * q;
      if (h0 + 32 * u < hbeg + hq) {
        if constexpr (kF32) {
          const float* xp = (const float*)x + (size_t)t * H + hh;
          const float* wp = (const float*)wr + (size_t)e * H + hh;
          xv[u][0] = ld16(xp);
          xv[u][1] = ld16(xp + 4);
          wv[u][0] = ld16(wp);
          wv[u][1] = ld16(wp + 4);
        } else {
          xv[u][0] = ld16((const uint16_t*)x + (size_t)t * H + hh);
          wv[u][0] = ld16((const uint16_t*)wr + (size_t)e * H + hh);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kNb; ++u) {
      if (h0 + 32 * u < hbeg + hq) {
        float xa[8], wb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kF32) {
            xa[i] = __uint_as_float(xv[u][0][i]);
            xa[4 + i] = __uint_as_float(xv[u][1][i]);
            wb[i] = __uint_as_float(wv[u][0][i]);
            wb[4 + i] = __uint_as_float(wv[u][1][i]);
          } else {
            xa[2 * i] = __uint_as_float(xv[u][0][i] << 16);
            xa[2 * i + 1] = __uint_as_float(xv[u][0][i] & 0xffff0000u);
            wb[2 * i] = __uint_as_float(wv[u][0][i] << 16);
            wb[2 * i + 1] = __uint_as_float(wv[u][0][i] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int s = 0; s < 8; s += 2) {
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[s], (double)wb[s], acc, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[s + 1], (double)wb[s + 1], acc2, 0, 0, 0);
        }
      }
    }
  }
  // D layout of the f64 16x16x4 MFMA: lane l, register i holds D[4 * i + l / 16][l % 16]
  // (row = token, column = expert) -- unlike the f32-output MFMAs, whose register i
  // holds row 4 * (l / 16) + i.
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][4 * i + q][r] = acc[i] + acc2[i];
  __syncthreads();
  if (wave == 0) {
    for (int idx = lane; idx < 256; idx += kWave) {
      const int tt = idx / 16, ee = idx % 16;
      if (t0 + tt < T && e0 + ee < E) {
        double s = part[0][tt][ee];
#pragma unroll
        for (int w = 1; w < kRouteWaves; ++w) s += part[w][tt][ee];
        if constexpr (kPartial) {
          partials[((size_t)blockIdx.x * T + t0 + tt) * E + e0 + ee] = s;
        } else {
          float v = (float)s;
          if (bias) v = __fadd_rn(v, bias[e0 + ee]);
          logits[(size_t)(t0 + tt) * E + e0 + ee] = v;
        }
      }
    }
  }
}

// Whole logits of 32 tokens x 32 experts per block, for calls with at least
// one such tile per CU.  Each of the kRoute32Waves waves takes an equal share
// of H and keeps four 16 x 16 accumulators (token half x expert half), so each
// x or router element it converts to fp64 feeds two MFMAs instead of one (the
// 16 x 16 blocks above convert both operands of every MFMA); lanes load and
// order K as above.  The waves' fp64 sums are added in wave order in LDS and
// rounded once.  (T = 2048, H = 2048, E = 128: 27.5 -> 21.8 us; below one tile
// per CU the 16 x 16 blocks are faster, as each block here keeps its CU's
// matrix cores busy for about 20 us.)
constexpr int kRoute32Waves = 8;
constexpr int kRoute32Batch = 2;  // 32-h steps whose loads are issued together
constexpr int kRoute32HMult = 32 * kRoute32Batch * kRoute32Waves;  // H must be a multiple

template <bool kF32>
__global__ __launch_bounds__(kWave* kRoute32Waves) void route_logits32_kernel(const void* __restrict__ x,
                                                                             const void* __restrict__ wr,
                                                                             const float* __restrict__ bias,
                                                                             float* __restrict__ logits, int T,
                                                                             int H, int E) {
  constexpr int V = kF32 ? 2 : 1;  // 16-byte loads per 8 elements
  __shared__ double part[kRoute32Waves][32][33];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int r = lane % 16, q = lane / 16;
  const int row[4] = {min(t0 + r, T - 1), min(t0 + 16 + r, T - 1), min(e0 + r, E - 1), min(e0 + 16 + r, E - 1)};
  const int hq = H / kRoute32Waves, hbeg = wave * hq;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int h0 = hbeg; h0 < hbeg + hq; h0 += 32 * kRoute32Batch) {
    u32x4 v[kRoute32Batch][4][V];  // [step][x lo, x hi, w lo, w hi][load]
#pragma unroll
    for (int u = 0; u < kRoute32Batch; ++u) {
      const int hh = h0 + 32 * u + 8 * q;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const void* base = o < 2 ? x : wr;
        if constexpr (kF32) {
          const float* p = (const float*)base + (size_t)row[o] * H + hh;
          v[u][o][0] = ld16(p);
          v[u][o][V - 1] = ld16(p + 4);
        } else {
          v[u][o][0] = ld16((const uint16_t*)base + (size_t)row[o] * H + hh);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRoute32Batch; ++u) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        double d[4];
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          if constexpr (kF32) {
            d[o] = (double)__uint_as_float(v[u][o][s / 4][s % 4]);
          } else {
            const uint32_t w2 = v[u][o][0][s / 2];
            d[o] = (double)__uint_as_float(s % 2 ? (w2 & 0xffff0000u) : (w2 << 16));
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(d[i], d[2 + j], acc[i][j], 0, 0, 0);
      }
    }
  }
  // D layout as above: register k of lane l holds row 4 k + l / 16, column l % 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) part[wave][16 * i + 4 * k + q][16 * j + r] = acc[i][j][k];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += kWave * kRoute32Waves) {
    const int tt = idx / 32, ee = idx % 32;
    if (t0 + tt < T && e0 + ee < E) {
      double sum = part[0][tt][ee];
#pragma unroll
      for (int w = 1; w < kRoute32Waves; ++w) sum += part[w][tt][ee];
      float lv = (float)sum;
      if (bias) lv = __fadd_rn(lv, bias[e0 + ee]);
      logits[(size_t)(t0 + tt) * E + e0 + ee] = lv;
    }
  }
}

// One wave per token: the top-k by rounds of wave-wide maxima and the gates
// of route_permute.hpp.
// kSlices > 0: the token's logits are first summed from kSlices fp64
// partials in slice order, rounded once (+ bias), and written out.
template <int kSlices>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits_in,
                                                        const double* __restrict__ partials,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out,
                                                        int32_t* __restrict__ topk_ids,
                                                        float* __restrict__ topk_w, int T, int E, int k) {
  __shared__ float s_sel[4][16];
  __shared__ float s_row[kSlices > 0 ? 4 : 1][256];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* row = logits_in + (size_t)t * E;
  if constexpr (kSlices > 0) {
    for (int e = lane; e < E; e += kWave) {
      double s = partials[(size_t)t * E + e];
#pragma unroll
      for (int sl = 1; sl < kSlices; ++sl) s += partials[((size_t)sl * T + t) * E + e];
      float v = (float)s;
      if (bias) v = __fadd_rn(v, bias[e]);
      logits_out[(size_t)t * E + e] = v;
      s_row[wave][e] = v;
    }
    wave_lds_sync();
    row = s_row[wave];
  }
  topk_wave_max_any(row, E, k, topk_ids + (size_t)t * k, topk_w + (size_t)t * k, nullptr, s_sel[wave]);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int tb = (a.T + 15) / 16, eb = (a.E + 15) / 16;
  // too few 16 x 16 blocks to fill the CUs: split H, sum the partials in the top-k
  const bool split = a.partials && a.T > kSmallRouteT && tb * eb < 256 && a.H % (256 * kRouteSplit) == 0;
  if (split) {
    dim3 grid(kRouteSplit, eb, tb);
    if (a.act_f32)
      hipLaunchKernelGGL((route_logits_kernel<true, true>), grid, dim3(kWave * route_waves<true>()), 0, stream, a.x,
                         a.w_router, nullptr, nullptr, a.partials, a.T, a.H, a.E);
    else
      hipLaunchKernelGGL((route_logits_kernel<false, true>), grid, dim3(kWave * route_waves<true>()), 0, stream, a.x,
                         a.w_router, nullptr, nullptr, a.partials, a.T, a.H, a.E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_topk_kernel<kRouteSplit>, dim3((a.T + 3) / 4), dim3(256), 0, stream, a.logits,
                       a.partials, a.bias, a.logits, a.topk_ids, a.topk_w, a.T, a.E, a.k);
    return hipGetLastError();
  }
  const int tb32 = (a.T + 31) / 32, eb32 = (a.E + 31) / 32;
  if (tb32 * eb32 >= 256 && a.H % kRoute32HMult == 0) {
    dim3 grid(tb32, eb32);
    if (a.act_f32)
      hipLaunchKernelGGL(route_logits32_kernel<true>, grid, dim3(kWave * kRoute32Waves), 0, stream, a.x, a.w_router,
                         a.bias, a.logits, a.T, a.H, a.E);
    else
      hipLaunchKernelGGL(route_logits32_kernel<false>, grid, dim3(kWave * kRoute32Waves), 0, stream, a.x, a.w_router,
                         a.bias, a.logits, a.T, a.H, a.E);
  } else {
    dim3 grid(tb, eb);
    if (a.act_f32)
      hipLaunchKernelGGL((route_logits_kernel<true, false>), grid, dim3(kWave * route_waves<false>()), 0, stream, a.x,
                         a.w_router, a.bias, a.logits, nullptr, a.T, a.H, a.E);
    else
      hipLaunchKernelGGL((route_logits_kernel<false, false>), grid, dim3(kWave * route_waves<false>()), 0, stream, a.x,
                         a.w_router, a.bias, a.logits, nullptr, a.T, a.H, a.E);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk_kernel<0>, dim3((a.T + 3) / 4), dim3(256), 0, stream, a.logits, nullptr, nullptr,
                     nullptr, a.topk_ids, a.topk_w, a.T, a.E, a.k);
  return hipGetLastError();
}

hipError_t launch_route_partials(const RouteArgs& a, double* partials, int slices, hipStream_t stream) {
  dim3 grid(slices, (a.E + 15) / 16);
  if (a.act_f32)
    hipLaunchKernelGGL((route_logits_kernel<true, true>), grid, dim3(kWave * route_waves<true>()), 0, stream, a.x,
                       a.w_router, nullptr, nullptr, partials, a.T, a.H, a.E);
  else
    hipLaunchKernelGGL((route_logits_kernel<false, true>), grid, dim3(kWave * route_waves<true>()), 0, stream, a.x,
                       a.w_router, nullptr, nullptr, partials, a.T, a.H, a.E);
  return hipGetLastError();
}

}  // namespace moe
