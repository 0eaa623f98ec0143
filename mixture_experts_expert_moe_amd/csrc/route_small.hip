// Routing and permutation of a few tokens (T <= kSmallRouteT) in two
// launches instead of four (logits, top-k, permutation, int8 quantisation of
// x): the router logits are first summed over slices of H by many blocks
// (route_logits_kernel, fp64 partials), then one block finishes everything --
// the sum of the partials in slice order rounded once to fp32 (+ bias), the
// top-k and gates of every token, the permutation with its tile schedule,
// and, for int8 weights, the per-token quantisation of x.  It calls the same
// device code as the stand-alone kernels.  Few-token calls are decode steps,
// where the pages find the launch count, not the arithmetic, to be the cost
// ("MoE Decode Partition and Submit Floor", section 3; "~2.7s fixed
// per-request TTFT ... concatenated-expert GEMM", section "Evidence").
#include "common.hpp"
#include "kernels.hpp"
#include "route_permute.hpp"

namespace moe {
namespace {

static_assert(kSmallRouteT <= kPermWaves, "one wave per token in the top-k step");

template <bool kF32>
__global__ __launch_bounds__(kPermThreads) void route_finish_kernel(RoutePermuteArgs a) {
  __shared__ float s_logit[kSmallRouteT * 256];           // T x E logits
  __shared__ int32_t s_ids[kSmallRouteT * 16];            // T x k ids
  __shared__ long long s_key[kSmallRouteT][kTopkKeys];    // top-k scratch, one row per wave
  __shared__ float s_sel[kSmallRouteT][16];
  __shared__ uint32_t s_perm[(kSmallRouteT + 31) / 32 * 256 * 3 / 2];  // permute_lds_bytes(T <= 32, E <= 256)
  const int T = a.r.T, E = a.r.E, k = a.r.k;
  const int wave = threadIdx.x / kWave;
  // int8: the token's row of x is loaded now and quantised after the top-k
  const bool quant = a.x_q && wave < T;
  const bool preload = quant && a.r.H <= QuantRow<kF32>::kMaxCols;
  QuantRow<kF32> xrow;
  if (preload) xrow.load(a.r.x, wave, a.r.H);
  // 1. logits: partial sums in slice order, rounded once, + bias
  for (int i = threadIdx.x; i < T * E; i += kPermThreads) {
    double s = a.partials[i];
    for (int sl = 1; sl < a.slices; ++sl) s += a.partials[(size_t)sl * T * E + i];
    float v = (float)s;
    if (a.r.bias) v = __fadd_rn(v, a.r.bias[i % E]);
    a.r.logits[i] = v;
    s_logit[i] = v;
  }
  __syncthreads();
  // 2. top-k and gates, one wave per token; int8: the token's quantisation of x
  if (wave < T) {
    topk_wave(s_logit + wave * E, E, k, a.r.topk_ids + wave * k, a.r.topk_w + wave * k, s_ids + wave * k,
              s_key[wave], s_sel[wave]);
    if (quant) xrow.quantise(a.r.x, a.x_q, a.x_scale, wave, a.r.H, preload);
  }
  __syncthreads();
  // 3. permutation and tile schedule
  permute_block(s_ids, a.p.offsets, a.p.row_token, a.p.token_row, a.p.sched, T, E, k, a.p.S, 0, a.p.big_start,
                s_perm);
}

}  // namespace

hipError_t launch_route_permute_small(const RoutePermuteArgs& a, hipStream_t stream) {
  if (a.r.T > kSmallRouteT || a.r.E > 256 || a.r.k > 16 || a.slices < 1 || a.slices > kRouteSlices ||
      permute_lds_bytes(a.r.T, a.r.E) > (size_t)(kSmallRouteT + 31) / 32 * 256 * 6)
    return hipErrorInvalidValue;
  hipError_t e = launch_route_partials(a.r, a.partials, a.slices, stream);
  if (e != hipSuccess) return e;
  if (a.r.act_f32)
    hipLaunchKernelGGL(route_finish_kernel<true>, dim3(1), dim3(kPermThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(route_finish_kernel<false>, dim3(1), dim3(kPermThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
