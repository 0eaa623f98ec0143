// Device functions shared by the routing and permutation kernels: the top-k
// of one token by one wave, the permutation by one block and the int8
// quantisation of one row by one block.  The stand-alone kernels and the
// fused small-T routing kernel call the same code, so their results agree
// bit for bit.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxGroups = 257;

// Wave-wide (64-lane) scans and reductions with DPP lane moves, which stay in
// the VALU instead of a round trip through the LDS crossbar per step: row
// shifts by 1, 2, 4, 8 within each 16-lane row, then the row broadcasts of
// lanes 15 and 31 (the gfx9 wave-scan pattern).  Every lane of the wave must
// be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, kCtrl, kRowMask, 0xf, false);
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Inclusive prefix sum over the wave (lanes that read past the start of a
// row or of the wave add 0).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i32<kDppShr1, 0xf>(0, v);
  v += dpp_i32<kDppShr2, 0xf>(0, v);
  v += dpp_i32<kDppShr4, 0xf>(0, v);
  v += dpp_i32<kDppShr8, 0xf>(0, v);
  v += dpp_i32<kDppBcast15, 0xa>(0, v);
  v += dpp_i32<kDppBcast31, 0xc>(0, v);
  return v;
}

// Exclusive wave-wide prefix sum, returns the lane's exclusive sum; *total = sum of all lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int inc = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(inc, kWave - 1);
  return inc - v;
}

// Maximum over the wave (max is exact, so the combining order does not
// matter).  Lanes that read past the start of a row keep their own value.
__device__ __forceinline__ float wave_max_dpp(float v) {
  int b = __float_as_int(v);
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppShr1, 0xf>(b, b))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppShr2, 0xf>(b, b))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppShr4, 0xf>(b, b))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppShr8, 0xf>(b, b))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppBcast15, 0xa>(b, b))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_i32<kDppBcast31, 0xc>(b, b))));
  return __int_as_float(__builtin_amdgcn_readlane(b, kWave - 1));
}

// Orders LDS writes of this wave before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Top-k by ranks.  Every (logit, id) pair gets a 64-bit key that orders
// larger logits first and, among equal logits, the lower expert id first (+0
// and -0 are equal; logits are finite), so all keys differ and the slot of a
// selected expert is its rank: the number of keys above its own.  The gates
// are the softmax of the k selected logits in fp64, summed in slot order,
// rounded once.  Lane l of a wave owns the candidates e = l + 64 j, j < kPer.
constexpr int kTopkKeys = 258;  // E <= 256, plus one pad key for odd E
__device__ __forceinline__ long long topk_key(float v, int e) {
  const int b = __float_as_int(v) == (int)0x80000000 ? 0 : __float_as_int(v);
  const int o = b >= 0 ? b : b ^ 0x7fffffff;  // order-preserving for finite floats
  return (long long)o * 256 + (255 - e);
}
constexpr long long kNoKey = (long long)INT64_MIN;

// Adds to above[j] the number of keys in s_key[lo, hi) (lo even; s_key[hi]
// readable when hi is odd) larger than key[j].
template <int kPer>
__device__ __forceinline__ void topk_count(const long long* s_key, int lo, int hi, const long long (&key)[kPer],
                                           int (&above)[kPer]) {
#pragma unroll 4
  for (int e = lo; e < hi; e += 2) {
    const long long k0 = s_key[e], k1 = s_key[e + 1];
#pragma unroll
    for (int j = 0; j < kPer; ++j) above[j] += (int)(k0 > key[j]) + (int)(k1 > key[j]);
  }
}

// Given every candidate's full rank: ids / w (and ids_copy, if non-null)
// receive the k selected experts in slot order; s_sel: k floats of LDS
// scratch for this wave.
template <int kPer>
__device__ __forceinline__ void topk_select(const float (&val)[kPer], const int (&above)[kPer], int E, int k,
                                            int32_t* ids, float* w, int32_t* ids_copy, float* s_sel) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    if (e < E && above[j] < k) {
      ids[above[j]] = e;
      s_sel[above[j]] = val[j];
      if (ids_copy) ids_copy[above[j]] = e;
    }
  }
  wave_lds_sync();
  const double top = (double)s_sel[0];
  const double ex = lane < k ? exp((double)s_sel[lane] - top) : 0.0;
  double den = 0.0;
  for (int s = 0; s < k; ++s) den += readlane_f64(ex, s);
  if (lane < k) w[lane] = (float)(ex / den);
}

// Ranks of token t's candidates against the keys of one part of its E.
template <int kPer>
__device__ __forceinline__ void rank_part(const long long* keys, int E, int lo, int hi, int32_t* above_sum) {
  const int lane = threadIdx.x % kWave;
  long long key[kPer];
  int above[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < E ? keys[e] : kNoKey;
    above[j] = 0;
  }
  topk_count<kPer>(keys, lo, hi, key, above);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (lane + kWave * j < E) atomicAdd(&above_sum[lane + kWave * j], above[j]);
}
template <int kPer>
__device__ __forceinline__ void select_token(const float* logit, const int32_t* above_sum, int E, int k, int32_t* ids,
                                             float* w, int32_t* ids_copy, float* s_sel) {
  const int lane = threadIdx.x % kWave;
  float val[kPer];
  int above[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    val[j] = e < E ? logit[e] : 0.f;
    above[j] = e < E ? above_sum[e] : k;
  }
  topk_select<kPer>(val, above, E, k, ids, w, ids_copy, s_sel);
}

// Maximum of a 64-bit value over the wave (the pattern of wave_max_dpp on
// both 32-bit halves); every lane of the wave must be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ long long dpp_max_i64(long long v) {
  const int lo = (int)(v & 0xffffffffll), hi = (int)(v >> 32);
  const int nlo = dpp_i32<kCtrl, kRowMask>(lo, lo), nhi = dpp_i32<kCtrl, kRowMask>(hi, hi);
  const long long n = ((long long)nhi << 32) | (unsigned)nlo;
  return n > v ? n : v;
}
__device__ __forceinline__ long long wave_max_i64(long long v) {
  v = dpp_max_i64<kDppShr1, 0xf>(v);
  v = dpp_max_i64<kDppShr2, 0xf>(v);
  v = dpp_max_i64<kDppShr4, 0xf>(v);
  v = dpp_max_i64<kDppShr8, 0xf>(v);
  v = dpp_max_i64<kDppBcast15, 0xa>(v);
  v = dpp_max_i64<kDppBcast31, 0xc>(v);
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffffll), kWave - 1);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), kWave - 1);
  return ((long long)hi << 32) | (unsigned)lo;
}

// Top-k of one token by one wave in k rounds of a wave-wide maximum over the
// keys (all distinct), each taking out the largest key left: the candidate
// taken in round r has rank r, so topk_select gets the same ranks as from
// counting keys.  Used where a token has a wave to itself: counting ranks
// then costs each lane E / 64 x E key comparisons, the rounds k reductions.
// logit: the token's E logits (global or shared memory).
template <int kPer>
__device__ __forceinline__ void topk_wave_max(const float* logit, int E, int k, int32_t* ids, float* w,
                                              int32_t* ids_copy, float* s_sel) {
  const int lane = threadIdx.x % kWave;
  long long key[kPer];
  float val[kPer];
  int above[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    val[j] = e < E ? logit[e] : 0.f;
    key[j] = e < E ? topk_key(val[j], e) : kNoKey;
    above[j] = k;
  }
  for (int r = 0; r < k; ++r) {
    long long m = key[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j) m = key[j] > m ? key[j] : m;
    m = wave_max_i64(m);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (key[j] == m) {
        above[j] = r;
        key[j] = kNoKey;
      }
    }
  }
  topk_select<kPer>(val, above, E, k, ids, w, ids_copy, s_sel);
}
__device__ __forceinline__ void topk_wave_max_any(const float* logit, int E, int k, int32_t* ids, float* w,
                                                  int32_t* ids_copy, float* s_sel) {
  if (E <= kWave) topk_wave_max<1>(logit, E, k, ids, w, ids_copy, s_sel);
  else if (E <= 2 * kWave) topk_wave_max<2>(logit, E, k, ids, w, ids_copy, s_sel);
  else topk_wave_max<4>(logit, E, k, ids, w, ids_copy, s_sel);
}

// Row `row` of src by one block of NT threads: s = max|v| / 127 (IEEE
// division), q = clamp(rne(v / s), -127, 127); s = 0 gives q = 0.  The block
// may call this for several rows in turn.
template <int NT>
__device__ __forceinline__ void quant_row_block(const void* __restrict__ src, bool src_f32, int8_t* __restrict__ q,
                                                float* __restrict__ scale, int row, int cols) {
  __shared__ float s_max[NT / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto load = [&](int c) -> float {
    return src_f32 ? ((const float*)src)[(size_t)row * cols + c]
                   : bf16_bits_to_f32(((const uint16_t*)src)[(size_t)row * cols + c]);
  };
  float amax = 0.f;
  for (int c = threadIdx.x; c < cols; c += NT) amax = fmaxf(amax, fabsf(load(c)));
  amax = wave_max_dpp(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = s_max[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) amax = fmaxf(amax, s_max[w]);
  const float s = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) scale[row] = s;
  for (int c = threadIdx.x; c < cols; c += NT) {
    q[(size_t)row * cols + c] = (int8_t)quant_i8(load(c), s);
  }
  __syncthreads();  // s_max is reused by the next row
}

// Columns [c0, c1) of one row by one wave, for a row quantised by several
// waves: 16-byte loads of 8 (bf16) or 4 (fp32) values per lane, kept in
// registers (load() can be issued early so its latency overlaps other work;
// a slice longer than the registers hold is streamed).  absmax() gives the
// slice's max |v|; quantise() writes its codes at the row's scale, the same
// clamp(rne(v / s), -127, 127) as quant_row_block.
template <bool kF32>
struct QuantSlice {
  static constexpr int V = kF32 ? 4 : 8;  // values per 16-byte load
  static constexpr int kRegs = 8;         // loads per lane kept in registers
  u32x4 keep[kRegs];

  __device__ static float val(const u32x4& u, int i) {
    return kF32 ? __uint_as_float(u[i]) : bf16_bits_to_f32(i % 2 ? (u[i / 2] >> 16) : (u[i / 2] & 0xffffu));
  }
  __device__ static bool in_regs(int c0, int c1) { return c1 - c0 <= kRegs * kWave * V; }
  __device__ static u32x4 ld(const void* row, int c) { return ld16((const uint8_t*)row + (size_t)c * (kF32 ? 4 : 2)); }

  __device__ void load(const void* row, int c0, int c1) {
    if (!in_regs(c0, c1)) return;
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
      const int c = c0 + (j * kWave + lane) * V;
      if (c < c1) keep[j] = ld(row, c);
    }
  }
  __device__ float absmax(const void* row, int c0, int c1) const {
    const int lane = threadIdx.x % kWave;
    float amax = 0.f;
    if (in_regs(c0, c1)) {
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const int c = c0 + (j * kWave + lane) * V;
        if (c < c1)
#pragma unroll
          for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(val(keep[j], i)));
      }
    } else {
      for (int c = c0 + lane * V; c < c1; c += kWave * V) {
        const u32x4 u = ld(row, c);
#pragma unroll
        for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(val(u, i)));
      }
    }
    return wave_max_dpp(amax);
  }
  __device__ static void put(const u32x4& u, float s, int8_t* __restrict__ q) {
    uint32_t packed[V / 4];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t b = (uint32_t)(uint8_t)(int8_t)quant_i8(val(u, i), s);
      if (i % 4 == 0) packed[i / 4] = b; else packed[i / 4] |= b << (8 * (i % 4));
    }
    if constexpr (V == 8) *reinterpret_cast<u32x2*>(q) = u32x2{packed[0], packed[1]};
    else *reinterpret_cast<uint32_t*>(q) = packed[0];
  }
  // q: the row's codes (column 0)
  __device__ void quantise(const void* row, int c0, int c1, float s, int8_t* __restrict__ q) const {
    const int lane = threadIdx.x % kWave;
    if (in_regs(c0, c1)) {
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const int c = c0 + (j * kWave + lane) * V;
        if (c < c1) put(keep[j], s, q + c);
      }
    } else {
      for (int c = c0 + lane * V; c < c1; c += kWave * V) put(ld(row, c), s, q + c);
    }
  }
};

// Inclusive prefix sum within aligned segments of kSeg lanes (kSeg a power of
// two <= 64): row shifts masked at segment starts, then the row broadcasts
// for 32- and 64-lane segments.  Every lane of the wave must be active.
template <int kSeg>
__device__ __forceinline__ int seg_incl_scan(int v) {
  const int l = (threadIdx.x % kWave) % kSeg;
  int t;
  if constexpr (kSeg >= 2) { t = dpp_i32<kDppShr1, 0xf>(0, v); v += l >= 1 ? t : 0; }
  if constexpr (kSeg >= 4) { t = dpp_i32<kDppShr2, 0xf>(0, v); v += l >= 2 ? t : 0; }
  if constexpr (kSeg >= 8) { t = dpp_i32<kDppShr4, 0xf>(0, v); v += l >= 4 ? t : 0; }
  if constexpr (kSeg >= 16) { t = dpp_i32<kDppShr8, 0xf>(0, v); v += l >= 8 ? t : 0; }
  if constexpr (kSeg >= 32) v += dpp_i32<kDppBcast15, 0xa>(0, v);
  if constexpr (kSeg >= 64) v += dpp_i32<kDppBcast31, 0xc>(0, v);
  return v;
}

// Per-expert exclusive prefix of the popcounts of its W <= kSeg words, and
// its total: each wave pass takes 64 / kSeg experts, one lane per word.
template <int kSeg>
__device__ __forceinline__ void prefix_words(const uint32_t* bits, uint16_t* pre, int32_t* s_cnt, int E, int W,
                                             int Ws) {
  constexpr int kPer = kWave / kSeg;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int e0 = wave * kPer; e0 < E; e0 += kPermWaves * kPer) {
    const int e = e0 + lane / kSeg, w = lane % kSeg;
    const bool in = e < E && w < W;
    const int c = in ? __popc(bits[e * Ws + w]) : 0;
    const int inc = seg_incl_scan<kSeg>(c);
    if (in) pre[e * Ws + w] = (uint16_t)(inc - c);
    if (e < E && w == kSeg - 1) s_cnt[e] = inc;
  }
}

// The permutation by one block of kPermThreads threads (all in LDS; `lds` is
// permute_lds_bytes(T, E) bytes of shared memory, Ws = permute_word_stride(T,
// E) the row stride of the bitmap).  topk_ids may point to global or shared
// memory.
constexpr int kIdBatch = 16;  // ids per thread in flight at once (T * k <= 16384 in one batch)

__device__ __forceinline__ void permute_block(const int32_t* topk_ids, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ row_token, int32_t* __restrict__ token_row,
                                              int32_t* __restrict__ sched, int T, int E, int k, int S, int big_on,
                                              int big_start, int Ws, uint32_t* lds) {
  const int W = (T + 31) / 32;                        // 32-token words per expert
  uint32_t* bits = lds;                               // [E][Ws]
  uint16_t* pre = (uint16_t*)(lds + (size_t)E * Ws);  // [E][Ws] exclusive popcount prefix
  __shared__ int32_t s_off[kMaxGroups + 1];
  __shared__ int32_t s_tile[kMaxGroups + 1];
  __shared__ int32_t s_cnt[kMaxGroups];
  const int G = E + S;
  const int kS = k + S;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int pairs = T * k;

  for (int i = threadIdx.x; i < E * Ws; i += kPermThreads) bits[i] = 0u;
  __syncthreads();
  // 1. bitmap.  Each thread issues kIdBatch loads of ids before the first
  //    atomic that needs one, so their latencies overlap.
  for (int i0 = threadIdx.x; i0 < pairs; i0 += kPermThreads * kIdBatch) {
    int ids[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int i = i0 + u * kPermThreads;
      ids[u] = i < pairs ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int e = ids[u], t = (i0 + u * kPermThreads) / k;
      if ((unsigned)e < (unsigned)E) atomicOr(&bits[e * Ws + t / 32], 1u << (t % 32));
    }
  }
  __syncthreads();
  // 2. per-expert prefix over words (a single word: prefix 0, count = popcount)
  if (W == 1) {
    for (int e = threadIdx.x; e < E; e += kPermThreads) {
      pre[e] = 0;
      s_cnt[e] = __popc(bits[e]);
    }
  } else if (W <= kWave) {
    // 64 / seg experts per wave pass, one lane per word (seg = the power of two >= W)
    if (W <= 2) prefix_words<2>(bits, pre, s_cnt, E, W, Ws);
    else if (W <= 4) prefix_words<4>(bits, pre, s_cnt, E, W, Ws);
    else if (W <= 8) prefix_words<8>(bits, pre, s_cnt, E, W, Ws);
    else if (W <= 16) prefix_words<16>(bits, pre, s_cnt, E, W, Ws);
    else if (W <= 32) prefix_words<32>(bits, pre, s_cnt, E, W, Ws);
    else prefix_words<64>(bits, pre, s_cnt, E, W, Ws);
  } else for (int e = wave; e < E; e += kPermWaves) {
    int base = 0;
    for (int w0 = 0; w0 < W; w0 += kWave) {
      const int w = w0 + lane;
      const int c = w < W ? __popc(bits[e * Ws + w]) : 0;
      int tot;
      const int ex = wave_excl_scan(c, &tot);
      if (w < W) pre[e * Ws + w] = (uint16_t)(base + ex);
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
  __shared__ int32_t s_rank[kMaxGroups];  // rank of g's partial tile among the partial tiles of its height
  if (wave == 0) {
    // start slot of each partial height, tallest first: lane l takes height 63 - l
    static_assert(kTileRows == kWave, "one lane per tile height");
    const int h = kTileRows - 1 - lane;
    const int c = h >= 1 ? s_hist[h] : 0;
    int total;
    const int ex = wave_excl_scan(c, &total);
    if (h >= 1) s_hist[h] = s_tile[G] + ex;
    if (lane == 0) s_hist[0] = s_tile[G] + total;  // total small tiles (lane 0 read height 63 already)
  } else if (wave == 1) {
    // ranks: groups in chunks of 64 (one per lane).  Lanes holding the same
    // height are found with one ballot per height bit; rank = lower such
    // lanes + the chunks before (a running count per height).
    __shared__ int32_t s_run[kTileRows];
    s_run[lane] = 0;
    for (int c0 = 0; c0 < G; c0 += kWave) {
      const int g = c0 + lane;
      const int rem = g < G ? s_small[g] % kTileRows : 0;
      uint64_t same = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 6; ++bit) {
        const uint64_t m = __ballot((rem >> bit) & 1);
        same &= ((rem >> bit) & 1) ? m : ~m;
      }
      const int r = __popcll(same & ((1ull << lane) - 1ull));
      const int base = rem ? s_run[rem] : 0;
      __builtin_amdgcn_wave_barrier();
      // the highest lane of each height adds the chunk's count
      if (rem && (same >> lane) == 1ull) s_run[rem] = base + r + 1;
      __builtin_amdgcn_wave_barrier();
      if (g < G) s_rank[g] = base + r;
    }
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
      // partial tiles of one height in group order
      int32_t* t = sched + kSchedHeader + (size_t)(s_hist[rem] + s_rank[g]) * kTileInts;
      t[0] = g;
      t[1] = row_base + full * kTileRows;
      t[2] = rem;
      t[3] = 0;
    }
  }
  // 4. rows (ids loaded in batches as in 1)
  for (int i0 = threadIdx.x; i0 < pairs; i0 += kPermThreads * kIdBatch) {
    int ids[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int i = i0 + u * kPermThreads;
      ids[u] = i < pairs ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int i = i0 + u * kPermThreads;
      if (i >= pairs) break;
      const int e = ids[u], t = i / k, j = i % k;
      int row = -1;
      if ((unsigned)e < (unsigned)E) {
        const int w = e * Ws + t / 32;
        row = s_off[e] + pre[w] + __popc(bits[w] & ((1u << (t % 32)) - 1u));
        row_token[row] = t;
      }
      token_row[(size_t)t * kS + j] = row;
    }
  }
  if (S) {
    for (int t = threadIdx.x; t < T; t += kPermThreads) {
      const int row = s_off[E] + t;
      token_row[(size_t)t * kS + k] = row;
      row_token[row] = t;
    }
  }
}

// The permutation of a few tokens (T <= 16, so every group holds <= 16 rows
// and is one partial tile) by one block of NT threads, with the same results
// as permute_block.  Every (token, expert) pair has a distinct key
// e * 256 + t, and everything is a count over the keys:
//   row of (t, e)   = number of keys below its own (rows are grouped by
//                     expert, token-ascending inside a group);
//   offsets[g]      = number of keys with expert < g (g <= E), then the
//                     shared group's T rows;
//   slot of g's tile = groups with more rows + groups of the same height and
//                     lower index (per-height counts and group bitmaps).
// topk_ids and every output may point to global or shared memory.
constexpr int kFewTokens = 16;
template <int NT>
__device__ __forceinline__ void permute_few_block_t(const int32_t* topk_ids, int32_t* offsets, int32_t* row_token,
                                                    int32_t* token_row, int32_t* sched, int T, int E, int k, int S,
                                                    int big_start) {
  constexpr int kMaxPairs = kFewTokens * 16;
  constexpr int kMaskWords = (kMaxGroups + 31) / 32;
  __shared__ __attribute__((aligned(16))) uint32_t s_pkey[kMaxPairs];
  __shared__ int32_t s_off[kMaxGroups + 1];
  __shared__ int32_t s_hist[kFewTokens + 1];                // groups per height (1..16)
  __shared__ uint32_t s_hmask[kFewTokens + 1][kMaskWords];  // groups of each height
  const int G = E + S, kS = k + S, pairs = T * k;
  const int tid = threadIdx.x;
  if (T == 1) {
    // One token: every touched group holds one row, so the counts below
    // reduce to ranks among the token's experts.  The row of expert e, its
    // group offset and its tile slot (all heights are 1: slots by group
    // index) are all the number of chosen experts below e; the shared group
    // comes last.  Wave 0 ranks the ids (k <= 16 lane reads each); then every
    // thread takes group offsets.
    __shared__ int32_t s_one[16];
    if (tid < kWave) {
      const int e = tid < k ? topk_ids[tid] : -1;
      const bool v = (unsigned)e < (unsigned)E;
      int row = 0;
      for (int l = 0; l < k; ++l) {
        const int el = __shfl(e, l);
        row += ((unsigned)el < (unsigned)E && el < e) ? 1 : 0;
      }
      const int nv = (int)__popcll(__ballot(v));
      if (tid < k) {
        s_one[tid] = v ? e : -1;
        token_row[tid] = v ? row : -1;
        if (v) {
          row_token[row] = 0;
          int32_t* t4 = sched + kSchedHeader + (size_t)row * kTileInts;
          t4[0] = e;
          t4[1] = row;
          t4[2] = 1;
          t4[3] = 0;
        }
      }
      if (tid == 0 && S) {
        token_row[k] = nv;
        row_token[nv] = 0;
        int32_t* t4 = sched + kSchedHeader + (size_t)nv * kTileInts;
        t4[0] = E;
        t4[1] = nv;
        t4[2] = 1;
        t4[3] = 0;
      }
      if (tid < kSchedHeader)
        sched[tid] = tid == kSchedSmall ? nv + S : tid == kSchedGroups ? G : tid == kSchedRows ? nv + S
                   : tid == kSchedBigStart ? big_start : 0;
    }
    __syncthreads();
    for (int g = tid; g <= G; g += NT) {
      int off = 0;
      for (int l = 0; l < k; ++l) off += (unsigned)s_one[l] < (unsigned)min(g, E) ? 1 : 0;
      offsets[g] = off + (g > E ? 1 : 0);
    }
    return;
  }
  // 1. keys (padded to a multiple of 4 with keys above every real key); clear the height tables
  const int pairs4 = (pairs + 3) & ~3;
  for (int i = tid; i < pairs4; i += NT) {
    const int e = i < pairs ? topk_ids[i] : -1;
    s_pkey[i] = (unsigned)e < (unsigned)E ? (uint32_t)e * 256u + (uint32_t)(i / k) : 0xffffffffu;
  }
  for (int i = tid; i < (kFewTokens + 1) * (kMaskWords + 1); i += NT) {
    if (i < kFewTokens + 1) s_hist[i] = 0;
    else (&s_hmask[0][0])[i - (kFewTokens + 1)] = 0u;
  }
  __syncthreads();
  // 2. rows of the pairs and group offsets (both count over the keys)
  for (int i = tid; i < pairs; i += NT) {
    const uint32_t key = s_pkey[i];
    const int t = i / k, j = i % k;
    int row = -1;
    if (key != 0xffffffffu) {
      row = 0;
#pragma unroll 4
      for (int m = 0; m < pairs4; m += 4) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(s_pkey + m);
        row += (q[0] < key) + (q[1] < key) + (q[2] < key) + (q[3] < key);
      }
      row_token[row] = t;
    }
    token_row[(size_t)t * kS + j] = row;
  }
  // groups go first to the threads past the pairs: g = (tid - pairs) mod NT
  for (int g = (tid + NT - pairs % NT) % NT; g <= E; g += NT) {
    int off = 0;
#pragma unroll 4
    for (int m = 0; m < pairs4; m += 4) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(s_pkey + m);
      off += ((q[0] >> 8) < (uint32_t)g) + ((q[1] >> 8) < (uint32_t)g) + ((q[2] >> 8) < (uint32_t)g) +
             ((q[3] >> 8) < (uint32_t)g);
    }
    s_off[g] = off;
    offsets[g] = off;
    if (S && g == E) {
      s_off[E + 1] = off + T;
      offsets[E + 1] = off + T;
    }
  }
  __syncthreads();
  if (S) {
    for (int t = tid; t < T; t += NT) {
      const int row = s_off[E] + t;
      token_row[(size_t)t * kS + k] = row;
      row_token[row] = t;
    }
  }
  // 3. heights
  for (int g = tid; g < G; g += NT) {
    const int n = s_off[g + 1] - s_off[g];
    if (n > 0) {
      atomicAdd(&s_hist[n], 1);
      atomicOr(&s_hmask[n][g / 32], 1u << (g % 32));
    }
  }
  __syncthreads();
  // 4. tiles: taller groups first, then lower group index
  for (int g = tid; g < G; g += NT) {
    const int n = s_off[g + 1] - s_off[g];
    if (n <= 0) continue;
    // (fixed trip counts, so the LDS reads are all in flight at once)
    int slot = 0;
#pragma unroll
    for (int h = 1; h <= kFewTokens; ++h) slot += h > n ? s_hist[h] : 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) slot += w < g / 32 ? __popc(s_hmask[n][w]) : 0;
    slot += __popc(s_hmask[n][g / 32] & ((1u << (g % 32)) - 1u));
    int32_t* t4 = sched + kSchedHeader + (size_t)slot * kTileInts;
    t4[0] = g;
    t4[1] = s_off[g];
    t4[2] = n;
    t4[3] = 0;
  }
  for (int i = tid; i < kSchedHeader; i += NT) {
    int tiles = 0;
    for (int h = 1; h <= kFewTokens; ++h) tiles += s_hist[h];
    sched[i] = i == kSchedSmall ? tiles : i == kSchedGroups ? G : i == kSchedRows ? s_off[G]
             : i == kSchedBigStart ? big_start : 0;
  }
}
__device__ __forceinline__ void permute_few_block(const int32_t* topk_ids, int32_t* offsets, int32_t* row_token,
                                                  int32_t* token_row, int32_t* sched, int T, int E, int k, int S,
                                                  int big_start) {
  permute_few_block_t<kPermThreads>(topk_ids, offsets, row_token, token_row, sched, T, E, k, S, big_start);
}

}  // namespace moe
