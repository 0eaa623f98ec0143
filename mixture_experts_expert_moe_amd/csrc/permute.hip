// Token -> expert permutation (moe_permute) and per-row int8 quantisation.
//
// Grouping every token of an expert into one contiguous block of rows is what
// lets the expert GEMMs run as one grouped launch rather than one launch per
// expert ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM",
// sections "Evidence" and "The fix"; "eight tokens through each expert in one
// go", OpenFlowLM-Next issue #74).
//
// One workgroup of 16 waves.  Tokens are taken in chunks of 64 (lane = token).
// Pass 1: each wave finds, for every expert present in its chunk, the ballot
// of lanes that chose it; a lane's rank inside the chunk is the popcount of
// that ballot below its lane, the chunk's count its full popcount.  Pass 2:
// per-expert exclusive prefix over chunks, then offsets over experts and the
// tile schedule.  Pass 3: row = offset[e] + chunk base + rank.  Rows of an
// expert come out in ascending token order; the result is unique.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxK = 16;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ topk_ids,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ token_row,
                                                               int32_t* __restrict__ sched, int T, int E, int k,
                                                               int S) {
  extern __shared__ uint16_t cnt[];  // [chunks][E]: count, then exclusive base
  __shared__ int32_t s_off[257 + 1];
  __shared__ int32_t s_tile[257 + 1];
  const int G = E + S;
  const int chunks = (T + 63) / 64;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int kS = k + S;
  for (int i = threadIdx.x; i < chunks * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();

  // Pass 1: ballot ranks within each chunk.
  for (int c = wave; c < chunks; c += kPermWaves) {
    const int t = c * 64 + lane;
    const bool valid = t < T;
    int ids[kMaxK];
    unsigned pending = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      int id = (valid && j < k) ? topk_ids[(size_t)t * k + j] : -1;
      if ((unsigned)id < (unsigned)E) pending |= 1u << j;
      else id = -1;
      ids[j] = id;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    while (true) {
      const uint64_t act = __ballot(pending != 0);
      if (act == 0) break;
      const int leader = __ffsll((unsigned long long)act) - 1;
      int cand = -1;
#pragma unroll
      for (int j = kMaxK - 1; j >= 0; --j)
        if ((pending >> j) & 1u) cand = ids[j];
      const int e = __shfl(cand, leader, kWave);
      int slot = -1;
#pragma unroll
      for (int j = kMaxK - 1; j >= 0; --j)
        if (((pending >> j) & 1u) && ids[j] == e) slot = j;
      const uint64_t m = __ballot(slot >= 0);
      // A repeated expert id (not produced by the router) gets further ranks.
      const int prev = cnt[c * E + e];
      if (slot >= 0) {
        token_row[(size_t)t * kS + slot] = prev + __popcll(m & below);  // rank, finalised in pass 3
        pending &= ~(1u << slot);
      }
      if (lane == leader) cnt[c * E + e] = (uint16_t)(prev + __popcll(m));
    }
  }
  __syncthreads();

  // Pass 2a: per-expert exclusive prefix over chunks.
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int run = 0;
    for (int c = 0; c < chunks; ++c) {
      const int v = cnt[c * E + e];
      cnt[c * E + e] = (uint16_t)run;
      run += v;
    }
    s_tile[e] = run;  // total rows of expert e (temporarily)
  }
  __syncthreads();
  // Pass 2b: offsets over groups and the tile schedule (one thread; G <= 257).
  if (threadIdx.x == 0) {
    int off = 0, tiles = 0;
    for (int g = 0; g < G; ++g) {
      const int n = (g < E) ? s_tile[g] : T;
      s_off[g] = off;
      s_tile[g] = tiles;
      off += n;
      tiles += (n + kTileRows - 1) / kTileRows;
    }
    s_off[G] = off;
    s_tile[G] = tiles;
    sched[0] = tiles;
    sched[1] = G;
    sched[2] = off;
  }
  for (int i = threadIdx.x; i < kSchedHeader; i += kPermThreads)
    if (i >= 3) sched[i] = 0;
  __syncthreads();
  for (int g = threadIdx.x; g <= G; g += kPermThreads) offsets[g] = s_off[g];
  for (int g = threadIdx.x; g < G; g += kPermThreads) {
    const int n = s_off[g + 1] - s_off[g];
    int32_t* dst = sched + kSchedHeader + (size_t)s_tile[g] * kTileInts;
    for (int i = 0; i * kTileRows < n; ++i) {
      dst[i * kTileInts + 0] = g;
      dst[i * kTileInts + 1] = s_off[g] + i * kTileRows;
      dst[i * kTileInts + 2] = min(kTileRows, n - i * kTileRows);
      dst[i * kTileInts + 3] = 0;
    }
  }

  // Pass 3: final rows.
  for (int c = wave; c < chunks; c += kPermWaves) {
    const int t = c * 64 + lane;
    if (t >= T) continue;
    for (int j = 0; j < k; ++j) {
      const int e = topk_ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) {  // not produced by the router: no row
        token_row[(size_t)t * kS + j] = -1;
        continue;
      }
      const int row = s_off[e] + cnt[c * E + e] + token_row[(size_t)t * kS + j];
      token_row[(size_t)t * kS + j] = row;
      row_token[row] = t;
    }
    if (S) {
      const int row = s_off[E] + t;
      token_row[(size_t)t * kS + k] = row;
      row_token[row] = t;
    }
  }
}

// One block per row: s = max|v| / 127, q = clamp(rne(v / s), -127, 127).
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, bool src_f32,
                                                        int8_t* __restrict__ q, float* __restrict__ scale,
                                                        int cols) {
  __shared__ float s_max[4];
  const int row = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto load = [&](int c) -> float {
    return src_f32 ? ((const float*)src)[(size_t)row * cols + c]
                   : bf16_bits_to_f32(((const uint16_t*)src)[(size_t)row * cols + c]);
  };
  float amax = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) amax = fmaxf(amax, fabsf(load(c)));
  amax = wave_max(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) scale[row] = s;
  for (int c = threadIdx.x; c < cols; c += 256) {
    float r = 0.f;
    if (s != 0.f) r = fminf(127.f, fmaxf(-127.f, rintf(__fdiv_rn(load(c), s))));
    q[(size_t)row * cols + c] = (int8_t)r;
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)((a.T + 63) / 64) * a.E * sizeof(uint16_t);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, stream, a.topk_ids, a.offsets, a.row_token,
                     a.token_row, a.sched, a.T, a.E, a.k, a.S);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(a.rows), dim3(256), 0, stream, a.src, a.src_f32, a.q, a.scale,
                     a.cols);
  return hipGetLastError();
}

}  // namespace moe
