// Routing and permutation of a few tokens (T <= kSmallRouteT) in two
// launches instead of four (logits, top-k, permutation, int8 quantisation of
// x): the router logits are first summed over slices of H by many blocks
// (route_logits_kernel, fp64 partials), then one block finishes everything --
// the sum of the partials in slice order rounded once to fp32 (+ bias), the
// top-k and gates of every token, the permutation with its tile schedule,
// and, for int8 weights, the per-token quantisation of x.  The top-k keys,
// the selection and gates, the int8 code and the permutation are the same
// device functions the stand-alone kernels call, and the ranks are the same
// whether counted or taken by rounds of maxima, so the results agree bit for
// bit.  Few-token calls are decode steps, where the pages find
// the launch count, not the arithmetic, to be the cost ("MoE Decode
// Partition and Submit Floor", section 3; "~2.7s fixed per-request TTFT ...
// concatenated-expert GEMM", section "Evidence").
#include "common.hpp"
#include "kernels.hpp"
#include "route_permute.hpp"

namespace moe {
namespace {

static_assert(kSmallRouteT == kPermWaves, "at least one wave per token");
static_assert(kSmallRouteT <= kFewTokens, "few-token permutation");

// Each token gets P = 16 / (the power of two >= T) of the block's 16 waves:
// they split the key range of its top-k ranks (partial counts summed with
// LDS atomics, exact in any order) and the columns of its int8 quantisation
// (slice maxima combined after a barrier).  Wave part 0 then selects the k
// experts and their gates.  With one wave per token (from 9 tokens on) that
// wave takes the ranks by rounds of maxima (topk_wave_max) instead.
template <bool kF32>
__global__ __launch_bounds__(kPermThreads) void route_finish_kernel(RoutePermuteArgs a) {
  __shared__ float s_logit[kSmallRouteT * 256];             // T x E logits
  __shared__ long long s_key[kSmallRouteT * kTopkKeys];     // T rows of E keys (+ pad)
  __shared__ int32_t s_above[kSmallRouteT * 256];           // T x E ranks
  __shared__ int32_t s_ids[kSmallRouteT * 16];              // T x k ids
  __shared__ float s_sel[kSmallRouteT][16];
  __shared__ float s_amax[kPermWaves];
  const int T = a.r.T, E = a.r.E, k = a.r.k, H = a.r.H;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int P = T <= 1 ? 16 : T <= 2 ? 8 : T <= 4 ? 4 : T <= 8 ? 2 : 1;
  const int t = wave / P, part = wave % P;
  const bool tok = t < T;
  // int8: this wave's columns of the token's row of x, loaded now
  const bool quant = a.x_q && tok;
  const int c0 = part * (H / P), c1 = c0 + H / P;
  const void* xrow = (const uint8_t*)a.r.x + (size_t)t * H * (kF32 ? 4 : 2);
  QuantSlice<kF32> xs;
  if (quant) xs.load(xrow, c0, c1);
  // 1. logits: partial sums in slice order, rounded once, + bias; their keys
  for (int i = threadIdx.x; i < T * E; i += kPermThreads) {
    double s = a.partials[i];
    for (int sl = 1; sl < a.slices; ++sl) s += a.partials[(size_t)sl * T * E + i];
    float v = (float)s;
    if (a.r.bias) v = __fadd_rn(v, a.r.bias[i % E]);
    a.r.logits[i] = v;
    s_logit[i] = v;
    s_key[(i / E) * kTopkKeys + i % E] = topk_key(v, i % E);
    s_above[i] = 0;
  }
  if ((E & 1) && threadIdx.x < T) s_key[threadIdx.x * kTopkKeys + E] = kNoKey;
  __syncthreads();
  // 2a. partial ranks over this wave's part of the keys; slice max of x
  if (tok) {
    const int chunk = ((E + P - 1) / P + 1) & ~1;
    const int lo = part * chunk, hi = min(E, lo + chunk);
    if (lo < hi && P > 1) {  // a token with one wave: ranked by topk_wave_max below
      const long long* keys = s_key + t * kTopkKeys;
      if (E <= kWave) rank_part<1>(keys, E, lo, hi, s_above + t * E);
      else if (E <= 2 * kWave) rank_part<2>(keys, E, lo, hi, s_above + t * E);
      else rank_part<4>(keys, E, lo, hi, s_above + t * E);
    }
    if (quant) {
      const float m = xs.absmax(xrow, c0, c1);
      if (lane == 0) s_amax[wave] = m;
    }
  }
  __syncthreads();
  // 2b. top-k and gates (part 0); int8: every part quantises its columns
  if (tok) {
    if (part == 0) {
      const float* lg = s_logit + t * E;
      const int32_t* ab = s_above + t * E;
      int32_t* ids = a.r.topk_ids + t * k;
      float* w = a.r.topk_w + t * k;
      if (P == 1) topk_wave_max_any(lg, E, k, ids, w, s_ids + t * k, s_sel[t]);
      else if (E <= kWave) select_token<1>(lg, ab, E, k, ids, w, s_ids + t * k, s_sel[t]);
      else if (E <= 2 * kWave) select_token<2>(lg, ab, E, k, ids, w, s_ids + t * k, s_sel[t]);
      else select_token<4>(lg, ab, E, k, ids, w, s_ids + t * k, s_sel[t]);
    }
    if (quant) {
      const float amax = wave_max_dpp(lane < P ? s_amax[t * P + lane] : 0.f);
      const float s = __fdiv_rn(amax, 127.0f);
      if (part == 0 && lane == 0) a.x_scale[t] = s;
      xs.quantise(xrow, c0, c1, s, a.x_q + (size_t)t * H);
    }
  }
  __syncthreads();
  // 3. permutation and tile schedule
  permute_few_block(s_ids, a.p.offsets, a.p.row_token, a.p.token_row, a.p.sched, T, E, k, a.p.S, a.p.big_start);
}

}  // namespace

hipError_t launch_route_permute_small(const RoutePermuteArgs& a, hipStream_t stream) {
  if (a.r.T > kSmallRouteT || a.r.E > 256 || a.r.k > 16 || a.slices < 1 || a.slices > kRouteSlices)
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
