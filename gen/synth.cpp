// Seeded synthetic inputs for the routed MoE FFN layer.
//
// This module is shared by the CPU oracle's tests and by the GPU harness.  It
// only draws random numbers and stores them in the formats the layer consumes
// (fp32, bf16, int8 + per-channel scale, 4-bit blocks + fp16 scale/min).  It
// holds none of the layer's arithmetic: no routing, no GEMM, no activation,
// no activation quantisation.
//
// Random numbers: SplitMix64 (Steele, Lea & Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014) used as a counter-based
// generator: draw i of a stream with key K is mix(K + (i + 1) * golden_gamma).
// Normals: Box-Muller (1958) on pairs of draws; uniforms use the top 53 bits.
//
// Built with plain g++ into gen/libsynth.so; driven from gen/synth.py.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <thread>
#include <vector>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGamma); }

// Key of sub-stream b of stream a (also exported as synth_mix).
inline uint64_t stream_key(uint64_t a, uint64_t b) { return mix64(mix64(a) ^ (b * kGamma + 0x5EED2026ULL)); }

// Uniform in (0, 1]: top 53 bits, offset by one so log() is finite.
inline double unit_open0(uint64_t r) { return (double)((r >> 11) + 1) * (1.0 / 9007199254740992.0); }

// Element i of a standard-normal stream (pairs share one Box-Muller draw).
inline double normal_at(uint64_t key, uint64_t i) {
  const uint64_t p = i >> 1;
  const double u1 = unit_open0(draw(key, 2 * p));
  const double u2 = unit_open0(draw(key, 2 * p + 1));
  const double r = std::sqrt(-2.0 * std::log(u1));
  const double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * std::sin(a) : r * std::cos(a);
}

inline uint32_t f32_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

// fp32 -> bf16, round to nearest even (storage format of bf16 inputs).
inline uint16_t to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> IEEE binary16, round to nearest even (storage of 4-bit block params).
inline uint16_t to_f16(float f) {
  const uint32_t x = f32_bits(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                     // below 2^-14: subnormal
    float a; std::memcpy(&a, &ax, 4);
    const uint32_t q = (uint32_t)std::nearbyint(a * 16777216.0f);  // units of 2^-24, RNE
    return (uint16_t)(sign | q);
  }
  const uint32_t mant = ax & 0x7fffffu;
  const uint32_t e = (ax >> 23) - 127u + 15u;
  uint32_t h = (e << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

inline float from_f16(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  float v;
  if (e == 0) v = (float)m * (1.0f / 16777216.0f);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((float)(m | 0x400u), (int)e - 25);
  uint32_t u = f32_bits(v) | sign;
  std::memcpy(&v, &u, 4);
  return v;
}

template <class F>
void parallel_for(int64_t n, int threads, F&& f) {
  if (threads <= 1 || n < 4096) { f((int64_t)0, n); return; }
  std::vector<std::thread> pool;
  const int64_t step = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    const int64_t lo = t * step, hi = std::min<int64_t>(n, lo + step);
    if (lo >= hi) break;
    pool.emplace_back([&f, lo, hi] { f(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

// One matrix [n][k] of N(mean, std) values, computed in double and rounded to fp32.
inline float value(uint64_t key, int64_t i, float mean, float std_) {
  return (float)((double)mean + (double)std_ * normal_at(key, (uint64_t)i));
}

// Elements [i0, i0 + n) of a stream, each Box-Muller pair computed once
// (the same values as value() element by element).
inline void fill_values(uint64_t key, int64_t i0, int64_t n, float mean, float std_, float* out) {
  int64_t i = i0, end = i0 + n;
  if (i < end && (i & 1)) { *out++ = value(key, i, mean, std_); ++i; }
  for (; i + 1 < end; i += 2) {
    const uint64_t p = (uint64_t)i >> 1;
    const double u1 = unit_open0(draw(key, 2 * p));
    const double u2 = unit_open0(draw(key, 2 * p + 1));
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    *out++ = (float)((double)mean + (double)std_ * (r * std::cos(a)));
    *out++ = (float)((double)mean + (double)std_ * (r * std::sin(a)));
  }
  if (i < end) *out++ = value(key, i, mean, std_);
}

// Rows [lo, hi) of the G*n rows, each row k values of matrix g = row / n.
template <class Store>
void weight_rows(uint64_t key, int32_t n, int32_t k, float std_, int64_t lo, int64_t hi, Store store) {
  std::vector<float> w((size_t)k);
  for (int64_t r = lo; r < hi; ++r) {
    const int64_t g = r / n, row = r % n;
    fill_values(stream_key(key, (uint64_t)g), row * (int64_t)k, k, 0.f, std_, w.data());
    store(r, w.data());
  }
}

}  // namespace

extern "C" {

uint64_t synth_mix(uint64_t a, uint64_t b) { return stream_key(a, b); }

// n draws of N(mean, std), stored as fp32.
void synth_normal_f32(uint64_t key, int64_t n, float mean, float std_, float* out, int threads) {
  parallel_for(n, threads, [&](int64_t lo, int64_t hi) { fill_values(key, lo, hi - lo, mean, std_, out + lo); });
}

// n draws of N(mean, std), stored as bf16 bits (fp32 value rounded to nearest even).
void synth_normal_bf16(uint64_t key, int64_t n, float mean, float std_, uint16_t* out, int threads) {
  parallel_for(n, threads, [&](int64_t lo, int64_t hi) {
    std::vector<float> buf(4096);
    for (int64_t i = lo; i < hi; i += 4096) {
      const int64_t m = std::min<int64_t>(4096, hi - i);
      fill_values(key, i, m, mean, std_, buf.data());
      for (int64_t j = 0; j < m; ++j) out[i + j] = to_bf16(buf[j]);
    }
  });
}

// G matrices [n][k] of N(0, std) (matrix g uses key synth_mix(key, g)), stored
// as int8 with one symmetric fp32 scale per output row n:
//   scale = max|w| / 127,  q = clamp(round_half_even(w / scale), -127, 127);
//   an all-zero row gets scale 0 and q 0.
void synth_weights_i8(uint64_t key, int32_t G, int32_t n, int32_t k, float std_,
                      int8_t* q, float* scale, int threads) {
  const int64_t rows = (int64_t)G * n;
  parallel_for(rows, threads, [&](int64_t lo, int64_t hi) {
    std::vector<float> w((size_t)k);
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t g = r / n, row = r % n;
      const uint64_t kg = synth_mix(key, (uint64_t)g);
      float amax = 0.f;
      fill_values(kg, row * (int64_t)k, k, 0.f, std_, w.data());
      for (int32_t c = 0; c < k; ++c) amax = std::max(amax, std::fabs(w[c]));
      const float s = amax / 127.0f;
      scale[r] = s;
      for (int32_t c = 0; c < k; ++c) {
        float v = 0.f;
        if (s != 0.f) v = std::min(127.f, std::max(-127.f, std::nearbyint(w[c] / s)));
        q[r * k + c] = (int8_t)v;
      }
    }
  });
}

// G matrices [n][k] of N(0, std) in 4-bit blocks of 32 consecutive k:
//   mn = min(block), mx = max(block); min16 = fp16(mn), scale16 = fp16((mx - mn) / 15);
//   q = clamp(round_half_even((w - min16) / scale16), 0, 15)  (q = 0 if scale16 == 0).
// Packing: byte b of a block holds element 2b in the low nibble, 2b+1 in the high one.
// Layouts: packed [G][n][k/2] bytes, scale16/min16 [G][n][k/32] fp16 bits.
void synth_weights_q4(uint64_t key, int32_t G, int32_t n, int32_t k, float std_,
                      uint8_t* packed, uint16_t* scale16, uint16_t* min16, int threads) {
  const int64_t rows = (int64_t)G * n;
  const int32_t nb = k / 32;
  parallel_for(rows, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t g = r / n, row = r % n;
      const uint64_t kg = synth_mix(key, (uint64_t)g);
      for (int32_t b = 0; b < nb; ++b) {
        float w[32];
        float mn = INFINITY, mx = -INFINITY;
        fill_values(kg, row * (int64_t)k + b * 32, 32, 0.f, std_, w);
        for (int j = 0; j < 32; ++j) {
          mn = std::min(mn, w[j]);
          mx = std::max(mx, w[j]);
        }
        const uint16_t m16 = to_f16(mn), s16 = to_f16((mx - mn) / 15.0f);
        const float mf = from_f16(m16), sf = from_f16(s16);
        scale16[r * nb + b] = s16;
        min16[r * nb + b] = m16;
        uint8_t* dst = packed + r * (int64_t)(k / 2) + b * 16;
        for (int j = 0; j < 16; ++j) {
          uint32_t qq[2];
          for (int h = 0; h < 2; ++h) {
            float v = 0.f;
            if (sf != 0.f) v = std::min(15.f, std::max(0.f, std::nearbyint((w[2 * j + h] - mf) / sf)));
            qq[h] = (uint32_t)v;
          }
          dst[j] = (uint8_t)(qq[0] | (qq[1] << 4));
        }
      }
    }
  });
}

// G matrices [n][k] of N(0, std) in MXFP4 blocks of 32 consecutive k (the OCP
// microscaling format, Open Compute Project "OCP Microscaling Formats (MX)
// v1.0"): one E8M0 scale byte per block (value 2^(byte - 127)) and 4-bit E2M1
// elements (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Per block:
//   amax = max |w|; amax == 0 gives scale byte 0 and all codes 0; otherwise
//   byte = clamp(floor(log2(amax)) - 2 + 127, 0, 254)   (2 = the exponent of 6),
//   code = the E2M1 value nearest to w / 2^(byte - 127), ties to the even
//          mantissa, magnitudes above 6 saturated to 6.
// Packing: byte b of a block holds element 2b in the low nibble, 2b+1 in the high one.
// Layouts: packed [G][n][k/2] bytes, scales [G][n][k/32] bytes.
namespace {
uint32_t e2m1_code(float v) {
  static const float kMag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  const float a = std::fabs(v);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    const float d = std::fabs(a - kMag[c]), db = std::fabs(a - kMag[best]);
    if (d < db || (d == db && (c & 1) == 0)) best = c;  // ties to the even mantissa bit
  }
  if (a > 6.f) best = 7;
  return best == 0 ? 0u : (uint32_t)best | (v < 0.f ? 8u : 0u);
}
}  // namespace
void synth_weights_mx4(uint64_t key, int32_t G, int32_t n, int32_t k, float std_, uint8_t* packed,
                       uint8_t* scales, int threads) {
  const int64_t rows = (int64_t)G * n;
  const int32_t nb = k / 32;
  parallel_for(rows, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t g = r / n, row = r % n;
      const uint64_t kg = synth_mix(key, (uint64_t)g);
      for (int32_t b = 0; b < nb; ++b) {
        float w[32];
        fill_values(kg, row * (int64_t)k + b * 32, 32, 0.f, std_, w);
        float amax = 0.f;
        for (int j = 0; j < 32; ++j) amax = std::max(amax, std::fabs(w[j]));
        int byte = 0;
        if (amax > 0.f) {
          int ex;
          std::frexp(amax, &ex);  // amax = m 2^ex, m in [0.5, 1): floor(log2(amax)) = ex - 1
          byte = std::min(254, std::max(0, ex - 1 - 2 + 127));
        }
        scales[r * nb + b] = (uint8_t)byte;
        const float inv = (float)std::ldexp(1.0, 127 - byte);  // 1 / 2^(byte - 127), exact
        uint8_t* dst = packed + r * (int64_t)(k / 2) + b * 16;
        for (int j = 0; j < 16; ++j) {
          const uint32_t lo4 = amax > 0.f ? e2m1_code(w[2 * j] * inv) : 0u;
          const uint32_t hi4 = amax > 0.f ? e2m1_code(w[2 * j + 1] * inv) : 0u;
          dst[j] = (uint8_t)(lo4 | (hi4 << 4));
        }
      }
    }
  });
}

// G matrices [n][k] of N(0, std) as fp32 or bf16 (matrix g uses key synth_mix(key, g)).
void synth_weights_f32(uint64_t key, int32_t G, int32_t n, int32_t k, float std_, float* out, int threads) {
  parallel_for((int64_t)G * n, threads, [&](int64_t lo, int64_t hi) {
    weight_rows(key, n, k, std_, lo, hi, [&](int64_t r, const float* w) {
      std::memcpy(out + r * (int64_t)k, w, sizeof(float) * (size_t)k);
    });
  });
}

void synth_weights_bf16(uint64_t key, int32_t G, int32_t n, int32_t k, float std_, uint16_t* out, int threads) {
  parallel_for((int64_t)G * n, threads, [&](int64_t lo, int64_t hi) {
    weight_rows(key, n, k, std_, lo, hi, [&](int64_t r, const float* w) {
      for (int32_t c = 0; c < k; ++c) out[r * (int64_t)k + c] = to_bf16(w[c]);
    });
  });
}

// Seeded permutation of 0..n-1 (Fisher-Yates, Durstenfeld's form), uniform draws from the stream.
void synth_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    const uint64_t j = (uint64_t)(unit_open0(draw(key, (uint64_t)i)) * (double)(i + 1)) % (uint64_t)(i + 1);
    std::swap(out[i], out[j]);
  }
}

// Per-expert logit offset that gives a Zipf(s) popularity: expert e of rank
// r(e) in 1..n (a seeded permutation) gets -s * ln(r(e)).
void synth_zipf_bias(uint64_t key, int32_t n, double s, float* out) {
  std::vector<int32_t> perm((size_t)n);
  synth_permutation(key, n, perm.data());
  for (int32_t e = 0; e < n; ++e) out[e] = (float)(-s * std::log((double)(perm[e] + 1)));
}

}  // extern "C"
