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

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxGroups = 257;

// Exclusive wave-wide prefix sum (64 lanes), returns the lane's exclusive sum; *total = sum of all lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int lane = threadIdx.x % kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  *total = __shfl(inc, kWave - 1, kWave);
  return inc - v;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ topk_ids,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ token_row,
                                                               int32_t* __restrict__ sched, int T, int E, int k,
                                                               int S, int big_on, int big_start) {
  extern __shared__ uint32_t lds[];
  const int W = (T + 31) / 32;                       // 32-token words per expert
  uint32_t* bits = lds;                              // [E][W]
  uint16_t* pre = (uint16_t*)(lds + (size_t)E * W);  // [E][W] exclusive popcount prefix
  __shared__ int32_t s_off[kMaxGroups + 1];
  __shared__ int32_t s_tile[kMaxGroups + 1];
  __shared__ int32_t s_cnt[kMaxGroups];
  const int G = E + S;
  const int kS = k + S;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int pairs = T * k;

  for (int i = threadIdx.x; i < E * W; i += kPermThreads) bits[i] = 0u;
  __syncthreads();
  // 1. bitmap
  for (int i = threadIdx.x; i < pairs; i += kPermThreads) {
    const int e = topk_ids[i], t = i / k;
    if ((unsigned)e < (unsigned)E) atomicOr(&bits[e * W + t / 32], 1u << (t % 32));
  }
  __syncthreads();
  // 2. per-expert prefix over words
  for (int e = wave; e < E; e += kPermWaves) {
    int base = 0;
    for (int w0 = 0; w0 < W; w0 += kWave) {
      const int w = w0 + lane;
      const int c = w < W ? __popc(bits[e * W + w]) : 0;
      int tot;
      const int ex = wave_excl_scan(c, &tot);
      if (w < W) pre[e * W + w] = (uint16_t)(base + ex);
      base += tot;
    }
    if (lane == 0) s_cnt[e] = base;
  }
  if (S && threadIdx.x == 0) s_cnt[E] = T;
  __syncthreads();
  // 3. offsets over groups, then the two tile lists (wave 0 scans; each lane
  //    takes 5 consecutive groups).  With big tiles on, a group of >= 128 rows
  //    is cut into tiles of 128 rows (a remainder of >= 64 rows is one more,
  //    partial, big tile; a smaller remainder goes to small tiles).  Small
  //    tiles hold <= 64 rows: all full ones first (by group), then the partial
  //    ones by descending height (ties by group) -- heavy tiles first.
  __shared__ int32_t s_hist[kTileRows];  // partial small tiles per height, then start slot per height
  __shared__ int32_t s_small[kMaxGroups];      // rows of g handled by small tiles (the last rows of g)
  __shared__ int32_t s_big[kMaxGroups + 1];    // first big tile of g
  if (threadIdx.x < kTileRows) s_hist[threadIdx.x] = 0;
  __syncthreads();
  if (wave == 0) {
    constexpr int kPer = (kMaxGroups + kWave - 1) / kWave;
    int rows_sum = 0, full_sum = 0, big_sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int g = lane * kPer + i;
      const int n = g < G ? s_cnt[g] : 0;
      int nbig = 0, nsmall = n;
      if (big_on && n >= kBigTileMin) {
        nbig = n / kBigTileRows + (n % kBigTileRows >= kBigPartMin ? 1 : 0);
        nsmall = n % kBigTileRows >= kBigPartMin ? 0 : n % kBigTileRows;
      }
      rows_sum += n;
      full_sum += nsmall / kTileRows;
      big_sum += nbig;
    }
    int rows_tot, full_tot, big_tot;
    int r = wave_excl_scan(rows_sum, &rows_tot);
    int f = wave_excl_scan(full_sum, &full_tot);
    int b = wave_excl_scan(big_sum, &big_tot);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int g = lane * kPer + i;
      if (g < G) {
        const int n = s_cnt[g];
        int nbig = 0, nsmall = n;
        if (big_on && n >= kBigTileMin) {
          nbig = n / kBigTileRows + (n % kBigTileRows >= kBigPartMin ? 1 : 0);
          nsmall = n % kBigTileRows >= kBigPartMin ? 0 : n % kBigTileRows;
        }
        s_off[g] = r;
        s_tile[g] = f;  // first full small tile of g
        s_big[g] = b;
        s_small[g] = nsmall;
        r += n;
        f += nsmall / kTileRows;
        b += nbig;
        if (nsmall % kTileRows) atomicAdd(&s_hist[nsmall % kTileRows], 1);
      }
    }
    if (lane == 0) {
      s_off[G] = rows_tot;
      s_tile[G] = full_tot;
      s_big[G] = big_tot;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // start slot of each partial height, tallest first
    int slot = s_tile[G];
    for (int h = kTileRows - 1; h >= 1; --h) {
      const int c = s_hist[h];
      s_hist[h] = slot;
      slot += c;
    }
    s_hist[0] = slot;  // total small tiles
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kSchedHeader; i += kPermThreads)
    sched[i] = i == kSchedSmall ? s_hist[0] : i == kSchedGroups ? G : i == kSchedRows ? s_off[G]
             : i == kSchedBig ? s_big[G] : i == kSchedBigStart ? big_start : 0;
  for (int g = threadIdx.x; g <= G; g += kPermThreads) offsets[g] = s_off[g];
  for (int g = threadIdx.x; g < G; g += kPermThreads) {
    const int n = s_off[g + 1] - s_off[g];
    const int nsmall = s_small[g];
    const int big_rows = n - nsmall;
    // big tiles of g: rows [s_off[g], s_off[g] + big_rows) in pieces of 128 (last one partial)
    int32_t* bdst = sched + big_start + (size_t)s_big[g] * kTileInts;
    for (int i = 0; i * kBigTileRows < big_rows; ++i) {
      bdst[i * kTileInts + 0] = g;
      bdst[i * kTileInts + 1] = s_off[g] + i * kBigTileRows;
      bdst[i * kTileInts + 2] = min(kBigTileRows, big_rows - i * kBigTileRows);
      bdst[i * kTileInts + 3] = 0;
    }
    // small tiles of g: the remaining rows
    const int row_base = s_off[g] + big_rows;
    const int full = nsmall / kTileRows, rem = nsmall % kTileRows;
    int32_t* dst = sched + kSchedHeader + (size_t)s_tile[g] * kTileInts;
    for (int i = 0; i < full; ++i) {
      dst[i * kTileInts + 0] = g;
      dst[i * kTileInts + 1] = row_base + i * kTileRows;
      dst[i * kTileInts + 2] = kTileRows;
      dst[i * kTileInts + 3] = 0;
    }
    if (rem) {
      // rank among partial tiles of the same height: groups below g with that height
      int before = 0;
      for (int h = 0; h < g; ++h) before += (s_small[h] % kTileRows) == rem;
      int32_t* t = sched + kSchedHeader + (size_t)(s_hist[rem] + before) * kTileInts;
      t[0] = g;
      t[1] = row_base + full * kTileRows;
      t[2] = rem;
      t[3] = 0;
    }
  }
  // 4. rows
  for (int i = threadIdx.x; i < pairs; i += kPermThreads) {
    const int e = topk_ids[i], t = i / k, j = i % k;
    int row = -1;
    if ((unsigned)e < (unsigned)E) {
      const int w = e * W + t / 32;
      row = s_off[e] + pre[w] + __popc(bits[w] & ((1u << (t % 32)) - 1u));
      row_token[row] = t;
    }
    token_row[(size_t)t * kS + j] = row;
  }
  if (S) {
    for (int t = threadIdx.x; t < T; t += kPermThreads) {
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
