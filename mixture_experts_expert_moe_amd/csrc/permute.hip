// Token -> expert permutation (moe_permute), per-row int8 quantisation and
// MXFP8 block quantisation.
//
// Grouping every token of an expert into one contiguous block of rows is what
// lets the expert GEMMs run as one grouped launch rather than one launch per
// expert ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM",
// sections "Evidence" and "The fix"; "eight tokens through each expert in one
// go", OpenFlowLM-Next issue #74).
//
// One workgroup of 16 waves, all in LDS:
//  1. per-expert token bitmap: bit t of bits[e] is set when token t chose e
//     (each (token, slot) pair ORs one bit, so the bitmap is order-independent;
//     rows at an odd stride where it fits, so that lanes with different
//     experts hit different banks);
//  2. per expert, an exclusive prefix of the popcounts of its 32-token words
//     (one wave per expert, a wave-wide scan over the words);
//  3. group offsets by a wave-wide scan over the groups, and the tile list:
//     full 64-row tiles first, then partial tiles by descending height, so a
//     launch that deals tiles in order starts the heaviest work first;
//  4. row of (t, e) = offset[e] + prefix[e][t / 32] + popcount of the bits of
//     bits[e][t / 32] below t.
// Rows of an expert come out in ascending token order; the result is unique.
#include "common.hpp"
#include "kernels.hpp"
#include "route_permute.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ topk_ids,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ token_row,
                                                               int32_t* __restrict__ sched, int T, int E, int k,
                                                               int S, int big_on, int big_start, int Ws) {
  extern __shared__ uint32_t lds[];
  permute_block(topk_ids, offsets, row_token, token_row, sched, T, E, k, S, big_on, big_start, Ws, lds);
}

// One block per row.
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, bool src_f32,
                                                        int8_t* __restrict__ q, float* __restrict__ scale,
                                                        int cols) {
  quant_row_block<256>(src, src_f32, q, scale, blockIdx.x, cols);
}

// MXFP8: each lane quantises 8 consecutive values; the 4 lanes of a 32-value
// block (consecutive lanes) share its max |v| through two lane swaps, and the
// first of them writes the block's scale byte.  n = rows * cols is a multiple
// of 256, so lanes past the end come in whole blocks of four.
template <bool kF32>
__global__ __launch_bounds__(256) void quant_mx8_kernel(const void* __restrict__ src, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, size_t n) {
  const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  float v[8];
  if constexpr (kF32) {
    const u32x4 a = ld16((const float*)src + i0), b = ld16((const float*)src + i0 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __uint_as_float(a[j]);
      v[4 + j] = __uint_as_float(b[j]);
    }
  } else {
    const u32x4 a = ld16((const uint16_t*)src + i0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(a[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32(a[j] >> 16);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  const uint32_t s = mx8_scale_byte(m);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= e4m3_code(v[j], s) << (8 * j);
    hi |= e4m3_code(v[4 + j], s) << (8 * j);
  }
  *reinterpret_cast<u32x2*>(codes + i0) = u32x2{lo, hi};
  if ((threadIdx.x & 3) == 0) scales[i0 / 32] = (uint8_t)s;
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const size_t lds = permute_lds_bytes(a.T, a.E);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, stream, a.topk_ids, a.offsets, a.row_token,
                     a.token_row, a.sched, a.T, a.E, a.k, a.S, a.big_on ? 1 : 0, a.big_start,
                     permute_word_stride(a.T, a.E));
  return hipGetLastError();
}

hipError_t launch_quant_mx8_rows(const void* src, bool src_f32, uint8_t* codes, uint8_t* scales, int64_t rows,
                                 int cols, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols % 256) return hipErrorInvalidValue;
  const size_t n = (size_t)rows * cols;
  const int64_t blocks = (int64_t)((n + 2047) / 2048);  // 2048 values per block
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (src_f32)
    hipLaunchKernelGGL(quant_mx8_kernel<true>, dim3(blocks), dim3(256), 0, stream, src, codes, scales, n);
  else
    hipLaunchKernelGGL(quant_mx8_kernel<false>, dim3(blocks), dim3(256), 0, stream, src, codes, scales, n);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(a.rows), dim3(256), 0, stream, a.src, a.src_f32, a.q, a.scale,
                     a.cols);
  return hipGetLastError();
}

}  // namespace moe
