// Token -> expert permutation (moe_permute) and per-row int8 quantisation.
//
// Grouping every token of an expert into one contiguous block of rows is what
// lets the expert GEMMs run as one grouped launch rather than one launch per
// expert ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM",
// sections "Evidence" and "The fix"; "eight tokens through each expert in one
// go", OpenFlowLM-Next issue #74).
//
// One workgroup of 16 waves, all in LDS:
//  1. per-expert token bitmap: bit t of bits[e] is set when token t chose e
//     (each (token, slot) pair ORs one bit, so the bitmap is order-independent);
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
                                                               int S, int big_on, int big_start) {
  extern __shared__ uint32_t lds[];
  permute_block(topk_ids, offsets, row_token, token_row, sched, T, E, k, S, big_on, big_start, lds);
}

// One block per row.
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, bool src_f32,
                                                        int8_t* __restrict__ q, float* __restrict__ scale,
                                                        int cols) {
  quant_row_block<256>(src, src_f32, q, scale, blockIdx.x, cols);
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const size_t lds = permute_lds_bytes(a.T, a.E);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, stream, a.topk_ids, a.offsets, a.row_token,
                     a.token_row, a.sched, a.T, a.E, a.k, a.S, a.big_on ? 1 : 0, a.big_start);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(a.rows), dim3(256), 0, stream, a.src, a.src_f32, a.q, a.scale,
                     a.cols);
  return hipGetLastError();
}

}  // namespace moe
