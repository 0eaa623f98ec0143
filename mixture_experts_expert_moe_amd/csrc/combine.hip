// Gate-weighted combine (moe_combine), RMSNorm (moe_rmsnorm), and the two
// fused for stacked layers (moe_combine_rmsnorm: layer l's output and layer
// l + 1's normalised input in one launch).
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

// RMSNorm reduction shared by the stand-alone kernel and the fused combine:
// the thread's fp32 sum of squares (its chunks in order, fmaf in element
// order), an xor-shuffle tree over the wave, the four wave sums as
// (w0 + w1) + (w2 + w3), then 1 / sqrt(mean + eps) with each operation
// rounded once.  Both kernels run it in 256-thread blocks, so for the same
// fp32 row they produce the same bits.
__device__ __forceinline__ float rms_inv(float ss, int H, float eps, float* s_part) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  return __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(tot, (float)H), eps)));
}

__device__ __forceinline__ u32x4 scale_bf16x8(const float v[8], float inv) {
  return u32x4{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv),
               pack_bf16x2(v[4] * inv, v[5] * inv), pack_bf16x2(v[6] * inv, v[7] * inv)};
}

// Chunks of 8 elements a thread owns in the fused combine + RMSNorm (H <= 8192).
constexpr int kNormChunks = 4;

// kNorm: the output (fp32) is also normalised into xn (bf16), the input of
// the next stacked layer, from the values held in registers.
template <bool kYF32, bool kOutF32, bool kNorm>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ residual, void* __restrict__ out,
                                                      uint16_t* __restrict__ xn, float eps, int H, int k, int S) {
  static_assert(!kNorm || kOutF32, "the normalised stream is fp32");
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  const int kS = k + S;
  // out[t][c0 .. c0+8) into acc.  The rows' loads go out kBatch at a time,
  // unconditionally (a missing row, r < 0, reads row 0 and is not added), so
  // that they are in flight together; the sum keeps the slot order.
  constexpr int kBatch = 9;
  auto chunk = [&](int c0, float (&acc)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < kS; j0 += kBatch) {
      int r[kBatch];
      float g[kBatch], v[kBatch][8];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + u;
        r[u] = j < kS ? token_row[(size_t)t * kS + j] : -1;
        g[u] = j < k ? topk_w[(size_t)t * k + j] : 1.0f;
        load8<kYF32>(y, (size_t)max(r[u], 0) * H + c0, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (r[u] < 0) continue;  // uniform over the block
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[u], v[u][i], acc[i]);
      }
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
  };
  if constexpr (!kNorm) {
    for (int c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
      float acc[8];
      chunk(c0, acc);
    }
  } else {
    float keep[kNormChunks][8];
    float ss = 0.f;
#pragma unroll
    for (int ch = 0; ch < kNormChunks; ++ch) {
      const int c0 = threadIdx.x * 8 + ch * 256 * 8;
      if (c0 < H) {
        chunk(c0, keep[ch]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(keep[ch][i], keep[ch][i], ss);
      }
    }
    const float inv = rms_inv(ss, H, eps, s_part);
#pragma unroll
    for (int ch = 0; ch < kNormChunks; ++ch) {
      const int c0 = threadIdx.x * 8 + ch * 256 * 8;
      if (c0 < H) *reinterpret_cast<u32x4*>(xn + (size_t)t * H + c0) = scale_bf16x8(keep[ch], inv);
    }
  }
}

// RMSNorm with unit gain, fp32: xn = bf16(x * (1 / sqrt(mean(x^2) + eps))).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, uint16_t* __restrict__ xn, int H,
                                                      float eps) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  float ss = 0.f;
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 2048) {
    float v[8];
    load8<true>(x, (size_t)t * H + c0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
  const float inv = rms_inv(ss, H, eps, s_part);
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 2048) {
    float v[8];
    load8<true>(x, (size_t)t * H + c0, v);
    *reinterpret_cast<u32x4*>(xn + (size_t)t * H + c0) = scale_bf16x8(v, inv);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(a.T), dim3(256), 0, stream, a.y, a.token_row, a.topk_w, a.residual, a.out, a.xn,
                       a.eps, a.H, a.k, a.S);
  };
  if (a.xn) {
    if (!a.out_f32 || a.H > 256 * 8 * kNormChunks) return hipErrorInvalidValue;
    if (a.y_f32) go(combine_kernel<true, true, true>);
    else go(combine_kernel<false, true, true>);
  } else if (a.y_f32) {
    if (a.out_f32) go(combine_kernel<true, true, false>);
    else go(combine_kernel<true, false, false>);
  } else {
    if (a.out_f32) go(combine_kernel<false, true, false>);
    else go(combine_kernel<false, false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, uint16_t* xn, int T, int H, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, x, xn, H, eps);
  return hipGetLastError();
}

}  // namespace moe
