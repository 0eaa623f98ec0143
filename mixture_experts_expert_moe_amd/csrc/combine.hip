// Gate-weighted combine (moe_combine) and RMSNorm (moe_rmsnorm).
//
// Combine: each token sums its k routed rows weighted by its gates, then its
// shared-expert row with weight 1 (the shared expert is always on, "top-8+shared"
// in "~2.7s fixed per-request TTFT ... concatenated-expert GEMM", section "The
// fix"), then the residual if given.  One block per token, each thread owns 8
// consecutive output elements: a segmented reduction with no atomics, summed
// in fp32 in a fixed order (slots 0..k-1, shared, residual).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <bool kYF32>
__device__ __forceinline__ void load8(const void* y, size_t off, float v[8]) {
  if constexpr (kYF32) {
    const u32x4 a = ld16((const float*)y + off), b = ld16((const float*)y + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 a = ld16((const uint16_t*)y + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
}

template <bool kYF32, bool kOutF32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ residual, void* __restrict__ out,
                                                      int H, int k, int S) {
  const int t = blockIdx.x;
  const int kS = k + S;
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < kS; ++j) {
      const int r = token_row[(size_t)t * kS + j];
      if (r < 0) continue;
      const float g = (j < k) ? topk_w[(size_t)t * k + j] : 1.0f;
      float v[8];
      load8<kYF32>(y, (size_t)r * H + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    if (residual) {
      float v[8];
      load8<true>(residual, (size_t)t * H + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if constexpr (kOutF32) {
      float* o = (float*)out + (size_t)t * H + c0;
      *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                 pack_bf16x2(acc[6], acc[7])};
      *reinterpret_cast<u32x4*>((uint16_t*)out + (size_t)t * H + c0) = o;
    }
  }
}

// RMSNorm with unit gain, fp32: xn = bf16(x * (1 / sqrt(mean(x^2) + eps))).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, uint16_t* __restrict__ xn, int H,
                                                      float eps) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float ss = 0.f;
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 2048) {
    float v[8];
    load8<true>(x, (size_t)t * H + c0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(tot, (float)H), eps)));
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 2048) {
    float v[8];
    load8<true>(x, (size_t)t * H + c0, v);
    u32x4 o = {pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv),
               pack_bf16x2(v[4] * inv, v[5] * inv), pack_bf16x2(v[6] * inv, v[7] * inv)};
    *reinterpret_cast<u32x4*>(xn + (size_t)t * H + c0) = o;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(a.T), dim3(256), 0, stream, a.y, a.token_row, a.topk_w, a.residual, a.out, a.H,
                       a.k, a.S);
  };
  if (a.y_f32) {
    if (a.out_f32) go(combine_kernel<true, true>);
    else go(combine_kernel<true, false>);
  } else {
    if (a.out_f32) go(combine_kernel<false, true>);
    else go(combine_kernel<false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, uint16_t* xn, int T, int H, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, x, xn, H, eps);
  return hipGetLastError();
}

}  // namespace moe
