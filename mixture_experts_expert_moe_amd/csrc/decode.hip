// The routed MoE layer for a few tokens (decode steps) in one launch
// (moe_decode_layer): router logits, top-k and gates, the permutation, the
// grouped gate/up GEMM with SwiGLU, the grouped down GEMM and the combine;
// optionally with the RMSNorm of an fp32 residual stream in front and the
// residual added at the end (one stacked layer, x + MoE(RMSNorm(x))).
//
// At decode sizes the layer's arithmetic is tiny and the pages find the fixed
// cost per dispatched operation to be what sets the floor: per-expert
// dispatch serialised the NPU path ("~2.7s fixed per-request TTFT = ~4,900
// serialized per-expert NPU execs", sections "Evidence" and "The fix"), a
// submit floor dominated small expert GEMMs ("MoE Decode Partition and Submit
// Floor", section 3), and a per-token expert path was the slow case on an
// AMD GPU (Atlas issue #145, the 2026-10-27 trace comment).  Here the whole
// layer is one launch of one block per CU, with three grid-wide barriers:
//
//   P0  every block stages the layer input of every token in its LDS (the
//       RMSNorm of the residual stream, or a copy of x) and, for int8 or
//       MXFP4 weights, its int8 or MXFP8 codes; then fp64 partial router
//       logits of (expert, slice of H) units
//   --- barrier
//   P1  every block sums the partials, takes the top-k of every token and
//       builds the permutation and tile list in its own LDS (identical in
//       every block, so no barrier is needed before the GEMMs); block 0
//       writes them out for the caller
//   P2  gate/up + SwiGLU: (tile, 16-pair) items, two per block at a time
//   --- barrier (the first down round's weights are loaded while waiting)
//   P3  down: (tile, 64-column) items, four per block at a time; each item
//       stages its tile's h rows in LDS (int8: quantised per row there; MX:
//       to MXFP8 per 32 columns)
//   --- barrier
//   P4  combine (+ residual): (token, 256-column) units spread over blocks
//
// The GEMM work items are the same device code as the grouped GEMM launches
// (gemm_item.hpp), and the routing pieces, the RMSNorm and the combine follow
// the same arithmetic in the same order as the separate kernels, so the
// results equal those of the separate calls bit for bit.
//
// Data that one block writes and another reads after a barrier (partial
// logits, h, y) is stored with agent-scope relaxed atomic stores and read with
// buffer loads, both with the sc1 cache policy: written through to memory and
// read from the coherent level, so the XCDs' separate L2 caches never hand out
// a stale copy.  Each wave waits for its own stores to complete before its
// block arrives at a barrier.  The barrier is two-level: blocks count in
// per-XCD counters (workgroups are dealt to the eight XCDs round-robin), the
// last of each XCD counts in the top counter, and the last of those advances
// a generation word that every block polls.  Every wait is bounded in time: a
// wait that times out sets the status word of the sync buffer and ends, so the
// launch always finishes.
#include <atomic>

#include "gemm_item.hpp"
#include "route_permute.hpp"

namespace moe {
namespace {

using namespace item;

constexpr int kThreads = 512, kWaves = kThreads / kWave;
constexpr int kTopWord = 0, kXcdWord = 64, kGenWord = 64 * 9;  // XCD x counts at kXcdWord + 64 x
static_assert(kDecodeStatusWord == 64 * 10 && 64 * 11 * 4 <= kDecodeSyncBytes, "sync words, one per 256-byte line");
static_assert(kDecodeMaxT <= kFewTokens && kDecodeMaxT * 16 <= 256, "few-token permutation");

__device__ __forceinline__ uint32_t ld_rx(const uint32_t* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_rx(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rx(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid-wide barrier (see the top of the file), in two halves so that a block
// can send loads that do not depend on the other blocks (the next phase's
// weights) between its arrival and its wait.  Counters only grow; with
// per_xcd a power of two their wrap-around keeps every modulus.  `gen` is
// the generation word's value before this barrier completes: thread 0 reads
// it once at the start of the launch (it cannot advance before this block
// arrives) and counts it up after each wait, so arriving costs only the
// counter atomics (re-reading it at each arrival put one more memory round
// trip on the path of the last block to arrive).
__device__ void grid_arrive(uint32_t* sync, int per_xcd, uint32_t gen) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = add_rx(sync + kXcdWord + 64 * (blockIdx.x % kXcds), 1u);
    if (old % (uint32_t)per_xcd == (uint32_t)per_xcd - 1u) {
      const uint32_t o2 = add_rx(sync + kTopWord, 1u);
      if (o2 % kXcds == kXcds - 1) st_rx(sync + kGenWord, gen + 1u);
    }
  }
}
__device__ void grid_wait(uint32_t* sync, uint32_t& gen, long long spin_ns) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();  // 100 MHz
    const uint64_t lim = (uint64_t)spin_ns / 10u;
    while (ld_rx(sync + kGenWord) == gen) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > lim) {
        st_rx(sync + kDecodeStatusWord, 1u);
        break;
      }
    }
  }
  ++gen;
  __syncthreads();
}
__device__ void grid_barrier(uint32_t* sync, int per_xcd, uint32_t& gen, long long spin_ns) {
  grid_arrive(sync, per_xcd, gen);
  grid_wait(sync, gen, spin_ns);
}

// Loads of data another block of this launch wrote: buffer loads with the
// sc1 cache policy (read from the coherent level, never from a stale copy in
// this XCD's L2).  As ordinary loads to the compiler they are issued back to
// back, where agent-scope atomic loads would each wait for the one before.
// Word 3 of the resource is the raw-buffer format of the gfx9 family;
// offsets past num_records bytes read as zero, so a load that may not be
// needed is issued anyway at kNoOffset rather than behind a branch (a load
// in a branch gets a full wait in front of it).
constexpr uint32_t kNoOffset = 0xfffffff0u;
template <int kAux>  // cache policy bits: 16 = sc1 (coherent), 0 = plain
struct BufLd {
  __amdgpu_buffer_rsrc_t r;
  __device__ BufLd(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
  __device__ uint64_t ld64(uint32_t byte_off) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, kAux);
    return ((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0];
  }
  __device__ u32x4 ld128(uint32_t byte_off) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kAux);
    return u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
  }
};
using CohBuf = BufLd<16>;

// Sum over the wave of an fp64 value with DPP lane moves (the wave-scan
// pattern of route_permute.hpp on both 32-bit halves): row shifts by 1, 2, 4,
// 8, then the row broadcasts of lanes 15 and 31; the total lands in lane 63.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), kCtrl, kRowMask, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), kCtrl, kRowMask, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double wave_sum_f64_last(double v) {
  v += dpp_f64<kDppShr1, 0xf>(v);
  v += dpp_f64<kDppShr2, 0xf>(v);
  v += dpp_f64<kDppShr4, 0xf>(v);
  v += dpp_f64<kDppShr8, 0xf>(v);
  v += dpp_f64<kDppBcast15, 0xa>(v);
  v += dpp_f64<kDppBcast31, 0xc>(v);
  return v;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& a, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

// LDS.  The routing state (kept from P1 to P4); the layer input: bf16 rows
// for bf16 / 4-bit weights (the gate/up B operand, kept to P2), int8 codes
// for int8 weights (kept to P2; the bf16 rows then only live in P0); and one
// region reused by phase: P0 partial sums, P1 logits and top-k keys, P2
// gate/up reductions, P3 staged h rows and down reductions.
constexpr int kMaxRows = kDecodeMaxT * 17;  // T * (k + S) with k <= 16, S <= 1
constexpr int kSchedInts = kSchedHeader + 4 * kMaxGroups;
template <int WF>
struct Lds {
  static constexpr bool kI8In = WF == kI8 || WF == kMX4;  // one-byte codes as the gate/up operand
  int32_t ids[kDecodeMaxT * 16];
  float gate[kDecodeMaxT * 16];
  int32_t off[kMaxGroups + 1];
  int32_t row_token[kMaxRows];
  int32_t token_row[kMaxRows];
  int32_t sched[kSchedInts];
  float x_scale[kDecodeMaxT];
  alignas(16) uint8_t x_sc[WF == kMX4 ? kDecodeMaxTH / 32 : 16];  // MX: E8M0 bytes of the codes
  float part[8];
  alignas(16) int8_t act[kI8In ? kDecodeMaxTH : 2 * kDecodeMaxTH];  // int8 codes, or bf16 rows
  union alignas(16) {
    struct {
      double red64[kWaves * kDecodeMaxT];
      alignas(16) uint16_t xin[kI8In ? kDecodeMaxTH : 8];  // int8 weights: the bf16 rows (P0 only)
    } p0;
    struct {
      float logit[kDecodeMaxT * 256];
      long long key[kDecodeMaxT * kTopkKeys];
      int32_t above[kDecodeMaxT * 256];
      float sel[kWaves][16];
    } route;
    f32x4 red_gu[2 * 3 * 2 * kWave];  // 2 items x 3 waves x 2 blocks
    struct {
      alignas(16) uint8_t h[4][16 * kDecodeMaxI * 2];  // 4 items x 16 rows (bf16, or int8 / E4M3 codes)
      float h_scale[4][16];
      alignas(16) uint8_t h_sc[4][WF == kMX4 ? 16 * kDecodeMaxI / 32 : 16];  // MX: E8M0 bytes of the staged rows
      f32x4 red[4 * 4 * kWave];  // 4 items x 1 wave x 4 blocks
    } dn;
  } u;
  __device__ uint16_t* rows_bf16() { return kI8In ? u.p0.xin : reinterpret_cast<uint16_t*>(act); }
};

template <int WF, bool kNormIn>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(DecodeArgs a) {
  __shared__ Lds<WF> L;
  constexpr bool kF32Out = WF == kI8 || WF == kMX4;  // h and y are fp32 for int8 and MX weights, else bf16
  const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k, S = a.S, G = E + S, kS = k + S;
  const int NB = gridDim.x, per_xcd = NB / kXcds;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool lead = blockIdx.x == 0;
  uint32_t gen = tid == 0 ? ld_rx(a.sync + kGenWord) : 0u;  // barrier generation (thread 0)
  uint16_t* xin = L.rows_bf16();  // [T][H] bf16 layer input

  // ---- P0: the layer input in LDS; int8 codes; router partial sums ------------
  int ns = 1;  // slices of H per router unit (the partials buffer holds kRouteSlices)
  while (ns * 2 <= kRouteSlices && ns * 2 * E <= NB && H % (ns * 2 * 8) == 0) ns *= 2;
  const int hs = H / ns;
  // the first router weights of this block, loaded before anything waits
  const int u0 = blockIdx.x, e0 = u0 / ns, sl0 = u0 % ns;
  u32x4 w0 = u32x4{0, 0, 0, 0};
  if (u0 < E * ns && 8 * tid < hs) w0 = ld16((const uint16_t*)a.w_router + (size_t)e0 * H + sl0 * hs + 8 * tid);
  if constexpr (kNormIn) {
    // xin = bf16(x * (1 / sqrt(mean(x^2) + eps))), x fp32: the arithmetic of
    // the RMSNorm kernel -- thread i of a 256-thread half owns the 8-value
    // chunks at 8 i + 2048 c, its squares summed with fmaf in element order,
    // an xor tree over the wave, then (w0 + w1) + (w2 + w3)
    const int half = tid / 256, i = tid % 256;
    for (int t0 = 0; t0 < T; t0 += 2) {
      const int t = t0 + half;
      float v[4][8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int c0 = i * 8 + c * 2048;
        if (t < T && c0 < H) {
          const float* src = (const float*)a.x + (size_t)t * H + c0;
          const u32x4 p = ld16(src), q = ld16(src + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[c][j] = __uint_as_float(p[j]);
            v[c][4 + j] = __uint_as_float(q[j]);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf(v[c][j], v[c][j], ss);
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
      if (lane == 0) L.part[wave] = ss;
      __syncthreads();
      const float* pp = L.part + 4 * half;
      const float tot = (pp[0] + pp[1]) + (pp[2] + pp[3]);
      const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(tot, (float)H), a.eps)));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int c0 = i * 8 + c * 2048;
        if (t < T && c0 < H)
          *reinterpret_cast<u32x4*>(xin + (size_t)t * H + c0) =
              u32x4{pack_bf16x2(v[c][0] * inv, v[c][1] * inv), pack_bf16x2(v[c][2] * inv, v[c][3] * inv),
                    pack_bf16x2(v[c][4] * inv, v[c][5] * inv), pack_bf16x2(v[c][6] * inv, v[c][7] * inv)};
      }
      __syncthreads();  // L.part is reused by the next pair of tokens
    }
  } else {
    constexpr int kChunks = kDecodeMaxTH / (8 * kThreads);  // 16-byte chunks per thread, all loaded first
    const BufLd<0> xbuf(a.x, (uint32_t)(T * H * 2));
    u32x4 v[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j) v[j] = xbuf.ld128((uint32_t)(tid + j * kThreads) * 16);
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      if (8 * (tid + j * kThreads) < T * H) *reinterpret_cast<u32x4*>(xin + 8 * (tid + j * kThreads)) = v[j];
    __syncthreads();
  }
  // router: unit u = (expert u / ns, slice u % ns of H), 8-value chunks per thread
  for (int u = blockIdx.x; u < E * ns; u += NB) {
    const int e = u / ns, sl = u % ns;
    double acc[kDecodeMaxT];
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.0;
    for (int h = sl * hs + 8 * tid; h < (sl + 1) * hs; h += 8 * kThreads) {
      float w[8];
      const bool first = u == u0 && h == sl * hs + 8 * tid;
      bf16x8_to_f32(first ? w0 : ld16((const uint16_t*)a.w_router + (size_t)e * H + h), w);
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t < T) {
          float xv[8];
          bf16x8_to_f32(*reinterpret_cast<const u32x4*>(xin + (size_t)t * H + h), xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t] += (double)xv[i] * (double)w[i];  // exact products
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) {
      if (t < T) {
        const double v = wave_sum_f64_last(acc[t]);
        if (lane == kWave - 1) L.u.p0.red64[wave * kDecodeMaxT + t] = v;
      }
    }
    __syncthreads();
    if (tid < T) {
      double v = L.u.p0.red64[tid];
      for (int w = 1; w < kWaves; ++w) v += L.u.p0.red64[w * kDecodeMaxT + tid];
      st_coh64(a.partials + ((size_t)sl * T + tid) * E + e, (uint64_t)__double_as_longlong(v));
    }
    __syncthreads();
  }
  {
    // the int8 codes are only needed from P2 on: they are made while this
    // block waits at the barrier
    grid_arrive(a.sync, per_xcd, gen);
    if constexpr (WF == kI8) {
      // per-token codes of the int8 path: token t gets P = 8 / (the power of
      // two >= T) waves (one wave per token from 8 tokens on), which split its
      // columns; their maxima meet in LDS (max is exact in any order)
      const int P = T <= 1 ? 8 : T <= 2 ? 4 : T <= 4 ? 2 : 1;
      float* s_max = reinterpret_cast<float*>(L.u.p0.red64);  // [waves] (red64 is not in use yet)
      for (int t0 = 0; t0 < T; t0 += kWaves / P) {
        const int t = t0 + wave / P, part = wave % P, cw = H / P;
        const uint16_t* row = xin + (size_t)t * H + part * cw;
        float amax = 0.f;
        if (t < T)
          for (int c = 8 * lane; c < cw; c += 8 * kWave) {
            float v[8];
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(row + c), v);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
          }
        amax = wave_max_dpp(amax);
        if (lane == 0) s_max[wave] = amax;
        __syncthreads();
        if (t < T) {
          float m = 0.f;
          for (int w = 0; w < P; ++w) m = fmaxf(m, s_max[(wave / P) * P + w]);
          const float s = __fdiv_rn(m, 127.0f);
          for (int c = 8 * lane; c < cw; c += 8 * kWave) {
            float v[8];
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(row + c), v);
            uint32_t pk[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) pk[j / 4] |= (uint32_t)(uint8_t)(int8_t)quant_i8(v[j], s) << (8 * (j % 4));
            *reinterpret_cast<u32x2*>(L.act + (size_t)t * H + part * cw + c) = u32x2{pk[0], pk[1]};
          }
          if (lane == 0 && part == 0) L.x_scale[t] = s;
        }
        __syncthreads();  // s_max is reused by the next tokens
      }
    }
    if constexpr (WF == kMX4) {
      // MXFP8 of every token (the conversion of moe_quant_mx8): a thread
      // takes 8 consecutive values, the 4 threads of a 32-value block
      // exchange their maxima (T * H / 8 is a multiple of the block size)
      for (int i0 = 0; i0 < T * H / 8; i0 += kThreads) {
        const int i = i0 + tid;
        float v[8];
        if (i < T * H / 8) bf16x8_to_f32(*reinterpret_cast<const u32x4*>(xin + 8 * i), v);
        else
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.f;
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        const uint32_t sb = mx8_scale_byte(m);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo |= e4m3_code(v[j], sb) << (8 * j);
          hi |= e4m3_code(v[4 + j], sb) << (8 * j);
        }
        if (i < T * H / 8) {
          *reinterpret_cast<u32x2*>(L.act + 8 * i) = u32x2{lo, hi};
          if ((i & 3) == 0) L.x_sc[i / 4] = (uint8_t)sb;
        }
      }
      __syncthreads();
    }
    if constexpr (WF == kI8 || WF == kMX4) {
      if (lead) {
        for (int i = tid; i < T * H / 8; i += kThreads)
          reinterpret_cast<u32x2*>(a.x_q)[i] = reinterpret_cast<const u32x2*>(L.act)[i];
        if constexpr (WF == kI8) {
          if (tid < T) a.x_scale[tid] = L.x_scale[tid];
        } else {
          for (int i = tid; i < T * H / 32; i += kThreads) reinterpret_cast<uint8_t*>(a.x_scale)[i] = L.x_sc[i];
        }
      }
    }
    grid_wait(a.sync, gen, a.spin_ns);
  }

  // ---- P1: logits, top-k, permutation (every block, in LDS) ---------------------
  const CohBuf pbuf(a.partials, (uint32_t)(ns * T * E * 8));
  for (int i = tid; i < T * E; i += kThreads) {
    uint64_t part[kRouteSlices];
#pragma unroll
    for (int sl = 0; sl < kRouteSlices; ++sl) part[sl] = pbuf.ld64(sl < ns ? (uint32_t)(sl * T * E + i) * 8 : kNoOffset);
    double s = __longlong_as_double((long long)part[0]);
    for (int sl = 1; sl < ns; ++sl) s += __longlong_as_double((long long)part[sl]);
    float v = (float)s;
    if (a.bias) v = __fadd_rn(v, a.bias[i % E]);
    L.u.route.logit[i] = v;
    L.u.route.key[(i / E) * kTopkKeys + i % E] = topk_key(v, i % E);
    L.u.route.above[i] = 0;
    if (lead) a.logits[i] = v;
  }
  if ((E & 1) && tid < T) L.u.route.key[tid * kTopkKeys + E] = kNoKey;
  __syncthreads();
  // top-k: up to 4 tokens by rank counts, token t getting P = 8 / (the power
  // of two >= T) waves, which split its keys; the counts meet in LDS
  // (integer atomics: exact in any order), then one wave selects.  From 5
  // tokens on a token has one wave: rounds of maxima (topk_wave_max).
  if (T > 4) {
    for (int t = wave; t < T; t += kWaves)
      topk_wave_max_any(L.u.route.logit + t * E, E, k, L.ids + t * k, L.gate + t * k, nullptr, L.u.route.sel[wave]);
  } else {
    const int P = T <= 1 ? 8 : T <= 2 ? 4 : 2;  // T <= 4
    for (int tw = wave; tw < T * P; tw += kWaves) {
      const int t = tw / P, part = tw % P;
      const int chunk = ((E + P - 1) / P + 1) & ~1;
      const int lo = part * chunk, hi = min(E, lo + chunk);
      if (lo < hi) {
        const long long* keys = L.u.route.key + t * kTopkKeys;
        int32_t* ab = L.u.route.above + t * E;
        if (E <= kWave) rank_part<1>(keys, E, lo, hi, ab);
        else if (E <= 2 * kWave) rank_part<2>(keys, E, lo, hi, ab);
        else rank_part<4>(keys, E, lo, hi, ab);
      }
    }
    __syncthreads();
    for (int t = wave; t < T; t += kWaves) {
      const float* lg = L.u.route.logit + t * E;
      const int32_t* ab = L.u.route.above + t * E;
      float* sel = L.u.route.sel[wave];
      if (E <= kWave) select_token<1>(lg, ab, E, k, L.ids + t * k, L.gate + t * k, nullptr, sel);
      else if (E <= 2 * kWave) select_token<2>(lg, ab, E, k, L.ids + t * k, L.gate + t * k, nullptr, sel);
      else select_token<4>(lg, ab, E, k, L.ids + t * k, L.gate + t * k, nullptr, sel);
    }
  }
  __syncthreads();
  permute_few_block_t<kThreads>(L.ids, L.off, L.row_token, L.token_row, L.sched, T, E, k, S, a.big_start);
  __syncthreads();
  const int n_tiles = L.sched[kSchedSmall];
  const int R = T * kS;
  if (lead) {
    for (int i = tid; i < T * k; i += kThreads) {
      a.topk_ids[i] = L.ids[i];
      a.topk_w[i] = L.gate[i];
    }
    for (int i = tid; i <= G; i += kThreads) a.offsets[i] = L.off[i];
    for (int i = tid; i < R; i += kThreads) {
      a.row_token[i] = L.row_token[i];
      a.token_row[i] = L.token_row[i];
    }
    for (int i = tid; i < kSchedHeader + 4 * n_tiles; i += kThreads) a.sched[i] = L.sched[i];
  }

  // ---- P2: gate/up + SwiGLU, two (tile, 16-pair) items per block at a time --------
  {
    Kp p{};
    p.act = xin;
    p.act_q = L.act;
    p.act_scale = WF == kMX4 ? reinterpret_cast<const float*>(L.x_sc) : L.x_scale;
    p.row_token = L.row_token;
    p.w = a.w_gu;
    p.w_scale = a.gu_scale;
    p.w_min = a.gu_min;
    p.out = a.h;
    p.K = H;
    p.N = I;
    p.T = T;
    p.R = R;
    const int ipt = I / 16, n_items = n_tiles * ipt;
    const int half = wave / 4;
    Acc<WF>* red = reinterpret_cast<Acc<WF>*>(L.u.red_gu) + half * 3 * 2 * kWave;
    for (int base = 0; base < n_items; base += 2 * NB) {
      __syncthreads();  // the previous round's reductions have been read
      const int it = base + half * NB + (int)blockIdx.x;
      const bool act = it < n_items;
      int g = 0, row0 = 0, rows = 1, n0 = 0;
      if (act) {
        const int32_t* tl = L.sched + kSchedHeader + (it / ipt) * kTileInts;
        g = tl[0];
        row0 = tl[1];
        rows = tl[2];
        n0 = (it % ipt) * 16;
      }
      gemm_item<WF, true, 1, 2, true>(p, g, row0, rows, n0, red, wave % 4, act);
    }
  }

  // ---- P3: down, four (tile, 64-column) items per block at a time -----------------
  // The first round's weights are loaded between this block's arrival at the
  // barrier and its wait; every later round loads its weights before it
  // stages its rows.
  {
    const int ipd = H / 64, n_items = n_tiles * ipd;
    const int quarter = wave / 2, qw = wave % 2;
    Kp p{};
    p.w = a.w_dn;
    p.w_scale = a.dn_scale;
    p.w_min = a.dn_min;
    p.out = a.y;
    p.K = I;
    p.N = H;
    p.T = T;
    p.R = R;
    p.act = L.u.dn.h[quarter];
    p.act_q = reinterpret_cast<const int8_t*>(L.u.dn.h[quarter]);
    p.act_scale = WF == kMX4 ? reinterpret_cast<const float*>(L.u.dn.h_sc[quarter]) : L.u.dn.h_scale[quarter];
    Acc<WF>* red = reinterpret_cast<Acc<WF>*>(L.u.dn.red) + quarter * 4 * kWave;
    // I <= 512: a wave's share of K is one register batch (int8) or two, all
    // of them sent early except the second of bf16's (64 registers each)
    DownItem<WF, WF == kI8 ? 1 : 2, WF == kBF16 ? 1 : (WF == kI8 ? 1 : 2)> di;
    const CohBuf hbuf(a.h, (uint32_t)(R * I * (kF32Out ? 4 : 2)));
    for (int base = 0; base < n_items; base += 4 * NB) {
      const int it = base + quarter * NB + (int)blockIdx.x;
      const bool act = it < n_items;
      int g = 0, row0 = 0, rows = 1, n0 = 0;
      if (act) {
        const int32_t* tl = L.sched + kSchedHeader + (it / ipd) * kTileInts;
        g = tl[0];
        row0 = tl[1];
        rows = tl[2];
        n0 = (it % ipd) * 64;
      }
      if (base == 0) {
        grid_arrive(a.sync, per_xcd, gen);
        di.issue(p, g, n0, qw, act);
        grid_wait(a.sync, gen, a.spin_ns);
      } else {
        __syncthreads();  // the previous round's rows and reductions have been read
        di.issue(p, g, n0, qw, act);
      }
      // stage the tile's h rows: wave qw takes rows qw, qw + 2, ...; lane
      // chunks of 4 values at columns 4 lane + 256 j (I <= 512: j < 2)
      if (act) {
        for (int r = qw; r < rows; r += 2) {
          if constexpr (WF == kI8) {
            const uint32_t src = (uint32_t)((row0 + r) * I) * 4;
            uint64_t v[2][2];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = 4 * lane + 4 * kWave * j;
              v[j][0] = hbuf.ld64(c < I ? src + 4 * c : kNoOffset);
              v[j][1] = hbuf.ld64(c < I ? src + 4 * c + 8 : kNoOffset);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if (4 * lane + 4 * kWave * j < I)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                  amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float((uint32_t)v[j][h2])),
                                           fabsf(__uint_as_float((uint32_t)(v[j][h2] >> 32)))));
            }
            const float sc = __fdiv_rn(wave_max_dpp(amax), 127.0f);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = 4 * lane + 4 * kWave * j;
              if (c < I) {
                const uint32_t b = (uint32_t)(uint8_t)(int8_t)quant_i8(__uint_as_float((uint32_t)v[j][0]), sc) |
                                   (uint32_t)(uint8_t)(int8_t)quant_i8(__uint_as_float((uint32_t)(v[j][0] >> 32)), sc) << 8 |
                                   (uint32_t)(uint8_t)(int8_t)quant_i8(__uint_as_float((uint32_t)v[j][1]), sc) << 16 |
                                   (uint32_t)(uint8_t)(int8_t)quant_i8(__uint_as_float((uint32_t)(v[j][1] >> 32)), sc) << 24;
                *reinterpret_cast<uint32_t*>(&L.u.dn.h[quarter][r * I + c]) = b;
                if (n0 == 0) *reinterpret_cast<uint32_t*>(a.h_q + (size_t)(row0 + r) * I + c) = b;
              }
            }
            if (lane == 0) {
              L.u.dn.h_scale[quarter][r] = sc;
              if (n0 == 0) a.h_scale[row0 + r] = sc;
            }
          } else if constexpr (WF == kMX4) {
            // MXFP8 per 32 columns: lane chunks of 4 values, the 8 lanes of
            // a block exchange their maxima (I <= 512: j < 2; I % 256 == 0)
            const uint32_t src = (uint32_t)((row0 + r) * I) * 4;
            uint64_t v[2][2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = 4 * lane + 4 * kWave * j;
              v[j][0] = hbuf.ld64(c < I ? src + 4 * c : kNoOffset);
              v[j][1] = hbuf.ld64(c < I ? src + 4 * c + 8 : kNoOffset);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = 4 * lane + 4 * kWave * j;
              float f[4] = {__uint_as_float((uint32_t)v[j][0]), __uint_as_float((uint32_t)(v[j][0] >> 32)),
                            __uint_as_float((uint32_t)v[j][1]), __uint_as_float((uint32_t)(v[j][1] >> 32))};
              float m = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
              m = fmaxf(m, __shfl_xor(m, 1));
              m = fmaxf(m, __shfl_xor(m, 2));
              m = fmaxf(m, __shfl_xor(m, 4));
              const uint32_t sb = mx8_scale_byte(m);
              const uint32_t b = e4m3_code(f[0], sb) | e4m3_code(f[1], sb) << 8 | e4m3_code(f[2], sb) << 16 |
                                 e4m3_code(f[3], sb) << 24;
              if (c < I) {
                *reinterpret_cast<uint32_t*>(&L.u.dn.h[quarter][r * I + c]) = b;
                if ((lane & 7) == 0) L.u.dn.h_sc[quarter][r * (I / 32) + c / 32] = (uint8_t)sb;
                if (n0 == 0) {
                  *reinterpret_cast<uint32_t*>(a.h_q + (size_t)(row0 + r) * I + c) = b;
                  if ((lane & 7) == 0)
                    reinterpret_cast<uint8_t*>(a.h_scale)[(size_t)(row0 + r) * (I / 32) + c / 32] = (uint8_t)sb;
                }
              }
            }
          } else {
            const uint32_t src = (uint32_t)((row0 + r) * I) * 2;
            for (int c = 4 * lane; c < I; c += 4 * kWave)
              *reinterpret_cast<uint64_t*>(&L.u.dn.h[quarter][(r * I + c) * 2]) = hbuf.ld64(src + 2 * c);
          }
        }
      }
      __syncthreads();
      p.act_row0 = row0;
      di.template finish<true>(p, g, row0, rows, n0, red, qw, act);
    }
  }
  grid_barrier(a.sync, per_xcd, gen, a.spin_ns);

  // ---- P4: combine (+ residual): unit (token t, 256 columns) on one wave --------
  // out[t][c] = sum_j gate[t][j] * y[row(t, j)][c] (slots in order, the shared
  // row with weight 1) + residual[t][c], fmaf in fp32 in that order: the
  // arithmetic of the combine kernel.  Lane l owns columns 4 l .. 4 l + 3.
  {
    const int upt = H / 256, n_units = T * upt;
    const CohBuf ybuf(a.y, (uint32_t)(R * H * (kF32Out ? 4 : 2)));
    const float* res = kNormIn ? (const float*)a.x : a.residual;
    for (int u = wave * NB + (int)blockIdx.x; u < n_units; u += NB * kWaves) {
      const int t = u / upt, c = (u % upt) * 256 + 4 * lane;
      constexpr int kGroup = 9;  // rows loaded together before the first is used
      float acc[4] = {0.f, 0.f, 0.f, 0.f}, rv[4];
      if (res) {
        const u32x4 q = ld16(res + (size_t)t * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = __uint_as_float(q[i]);
      }
      for (int j0 = 0; j0 < kS; j0 += kGroup) {
        float yv[kGroup][4];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const int r = j0 + j < kS ? L.token_row[t * kS + j0 + j] : -1;
          if constexpr (kF32Out) {
            const u32x4 q = ybuf.ld128(r >= 0 ? (uint32_t)(r * H + c) * 4 : kNoOffset);
#pragma unroll
            for (int i = 0; i < 4; ++i) yv[j][i] = __uint_as_float(q[i]);
          } else {
            const uint64_t q = ybuf.ld64(r >= 0 ? (uint32_t)(r * H + c) * 2 : kNoOffset);
            const uint32_t lo = (uint32_t)q, hi = (uint32_t)(q >> 32);
            yv[j][0] = __uint_as_float(lo << 16);
            yv[j][1] = __uint_as_float(lo & 0xffff0000u);
            yv[j][2] = __uint_as_float(hi << 16);
            yv[j][3] = __uint_as_float(hi & 0xffff0000u);
          }
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const int r = j0 + j < kS ? L.token_row[t * kS + j0 + j] : -1;
          if (r < 0) continue;
          const float g = j0 + j < k ? L.gate[t * k + j0 + j] : 1.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(g, yv[j][i], acc[i]);
        }
      }
      if (res) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += rv[i];
      }
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>((float*)a.out + (size_t)t * H + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      } else {
        *reinterpret_cast<u32x2*>((uint16_t*)a.out + (size_t)t * H + c) =
            u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      }
    }
  }
}

template <int WF>
void launch_fmt(const DecodeArgs& a, int nb, hipStream_t stream) {
  static_assert(sizeof(Lds<WF>) > 80 * 1024, "one block per CU");
  if (a.norm_input)
    hipLaunchKernelGGL((decode_layer_kernel<WF, true>), dim3(nb), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_layer_kernel<WF, false>), dim3(nb), dim3(kThreads), 0, stream, a);
}

}  // namespace

// Device memory of the allocation-free decode call (moe_decode_layer_static):
// the layer buffers of one call, laid out by the caller of
// decode_static_scratch.  Zero at load, so its barrier words start valid.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (the host-side name of the array is not a device address).
hipError_t decode_static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

int decode_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (cus < kXcds) return 0;
  int per = 1;
  while (per * 2 * kXcds <= cus) per *= 2;
  return per * kXcds;
}

hipError_t launch_decode_layer(const DecodeArgs& a, hipStream_t stream) {
  if (a.T < 1 || a.T > kDecodeMaxT || a.T * a.H > kDecodeMaxTH || a.I > kDecodeMaxI || a.H > 8192 ||
      a.E > 256 || a.k > 16 || (a.norm_input && !a.out_f32))
    return hipErrorInvalidValue;
  const int nb = decode_blocks();
  if (nb == 0) return hipErrorInvalidValue;
  // more than half of a CU's LDS per block: at most one block per CU, so the
  // nb <= CU count blocks are all resident together once the GPU is free
  switch (a.wfmt) {
    case kBF16: launch_fmt<kBF16>(a, nb, stream); break;
    case kI8: launch_fmt<kI8>(a, nb, stream); break;
    case kQ4: launch_fmt<kQ4>(a, nb, stream); break;
    case kMX4: launch_fmt<kMX4>(a, nb, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
