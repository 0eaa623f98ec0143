// CPU oracle of the routed Mixture-of-Experts FFN layer.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
// benchmark's CPU-baseline leg may load or call this library.  The GPU product
// path never links, imports or falls back to it, and the two share no code.
//
// It is plain, slow and written from the layer's definition:
//
//   y_t = sum_{j<k} g_{t,j} * FFN_{e_{t,j}}(x_t)  +  [shared] FFN_shared(x_t)
//   FFN_e(x) = W_down[e] * ( silu(W_gate[e] * x) (*) (W_up[e] * x) ),  silu(a) = a / (1 + e^-a)
//   (e_{t,.}, g_{t,.}) = the k largest router logits of x_t, gates = their softmax
//
// Sources for the definition (cited by page title and section):
//  * "~2.7s fixed per-request TTFT = ~4,900 serialized per-expert NPU execs --
//    validated coarsening fix (concatenated-expert GEMM)" (FastFlowLM issue
//    #710), section "The fix": each token runs through its top-8 routed
//    experts plus a shared expert; gate and up projections are concatenated
//    (N = TOP_K x 2 x IM_EXP) and followed by a GLU on the CPU side.
//  * "MoE Decode Partition and Submit Floor" (oRKLLM/ork-driver wiki),
//    section 3, Test 1: per-expert gate/up is 2048x512 and down is 512x2048;
//    section 2: int8 dot products run on pre-quantised activations against
//    quantised weight rows.
//  * Atlas issue #145 (Strix Halo serving), the 2026-10-27 trace comment: the
//    shared expert is fused into the gate/up and the silu-down kernels.
// The pages print no formula and no worked example; every reading made where
// they are silent (softmax placement, tie order, shared-expert weight, GLU
// form, quantisation rules) is listed in the repository's design notes.
//
// Arithmetic:
//  * float paths: every dot product accumulates in fp64; activations in fp64.
//  * the router logit is the fp64 dot product rounded once to fp32 (plus an
//    optional fp32 bias, one fp32 addition); the top-k decision is taken on
//    those fp32 logits; gates are the softmax of the selected logits in fp64,
//    rounded once to fp32.
//  * int8 path: int64 accumulation asserted to fit int32, then fp32 dequant
//    ((float)acc * s_x) * s_w and fp32 SiLU, each fp32 operation rounded once.
//  * 4-bit weights: w = bf16_rne(fp32(scale * q + min)), used exactly.
//
// Build: g++ -O2 -ffp-contract=off (no fast-math); see oracle/oracle.py.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

enum Dtype { DT_F32 = 0, DT_BF16 = 1, DT_I8 = 2, DT_Q4 = 3, DT_MX4 = 4 };

// ---- number formats (the oracle's own decoders) ---------------------------

float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// IEEE binary16 -> float, exact.
float f16_value(uint16_t h) {
  const int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return (float)(sign ? -v : v);
}

// Round a float to the nearest bf16 value (ties to even), returned as float.
float round_bf16(float f) {
  if (std::isnan(f) || std::isinf(f) || f == 0.0f) return f;
  if (std::fabs(f) < 0x1p-126f)  // subnormal range: multiples of 2^-133
    return (float)std::ldexp(std::nearbyint(std::ldexp((double)f, 133)), -133);
  int e;
  const double m = std::frexp((double)f, &e);      // |m| in [0.5, 1)
  const double r = std::nearbyint(std::ldexp(m, 8));  // 8 significant bits, ties to even
  return (float)std::ldexp(r, e - 8);
}

double round_bf16_d(double d) {
  if (std::isnan(d) || std::isinf(d) || d == 0.0) return d;
  int e;
  const double m = std::frexp(d, &e);
  return std::ldexp(std::nearbyint(std::ldexp(m, 8)), e - 8);
}

// ---- OCP microscaling (MX) formats ------------------------------------------
// A block of 32 values shares one E8M0 scale byte s, worth 2^(s - 127).
double e8m0_value(uint8_t s) { return std::ldexp(1.0, (int)s - 127); }

// E2M1 element (4 bits): sign, 2 exponent bits (bias 1), 1 mantissa bit;
// exponent 0 is subnormal (mantissa x 0.5).
double e2m1_value(int code) {
  const int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double mag = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

// E4M3 element (OCP "E4M3", no infinities): sign, 4 exponent bits (bias 7),
// 3 mantissa bits; exponent 0 is subnormal (mantissa x 2^-9); largest 448.
double e4m3_value(int code) {
  const int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  const double mag = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, e - 10);
  return sign ? -mag : mag;
}

// The E4M3 value nearest to a >= 0 (ties to the even mantissa), magnitudes
// above 448 saturated to 448: a rounded to a multiple of 2^(max(E, -6) - 3),
// E = floor(log2(a)), which is the spacing of E4M3 values at a.
double e4m3_round(double a) {
  if (a == 0.0) return 0.0;
  int ex;
  std::frexp(a, &ex);  // a = m 2^ex, m in [0.5, 1)
  const int q = std::max(ex - 1, -6) - 3;
  const double r = std::ldexp(std::nearbyint(std::ldexp(a, -q)), q);
  return std::min(r, 448.0);
}
int e4m3_code(double r, bool neg) {  // r: a value e4m3_round returned
  int code;
  if (r == 0.0) return 0;
  int ex;
  std::frexp(r, &ex);
  const int E = ex - 1;
  if (E >= -6) code = ((E + 7) << 3) | (int)(std::ldexp(r, 3 - E) - 8.0);
  else code = (int)std::ldexp(r, 9);
  return code | (neg ? 0x80 : 0);
}

// MXFP8 (E4M3) quantisation of one row in blocks of 32 (the OCP MX
// conversion): amax = max |v| of the block; amax == 0 gives scale byte 0 and
// codes 0; otherwise scale byte = clamp(floor(log2(amax)) - 8 + 127, 0, 254)
// (8 = the exponent of 448), code = e4m3(v / scale).  deq receives the value
// each code stands for (code value x scale).
void quant_mx8_row(int cols, const float* v, uint8_t* codes, uint8_t* scales, double* deq) {
  for (int b = 0; b < cols / 32; ++b) {
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) amax = std::max(amax, std::fabs((double)v[b * 32 + j]));
    int s = 0;
    if (amax > 0.0) {
      int ex;
      std::frexp(amax, &ex);
      s = std::min(254, std::max(0, ex - 1 - 8 + 127));
    }
    scales[b] = (uint8_t)s;
    for (int j = 0; j < 32; ++j) {
      const double x = (double)v[b * 32 + j];
      int c = 0;
      if (amax > 0.0) c = e4m3_code(e4m3_round(std::ldexp(std::fabs(x), 127 - s)), x < 0.0);
      codes[b * 32 + j] = (uint8_t)c;
      deq[b * 32 + j] = e4m3_value(c) * e8m0_value((uint8_t)s);
    }
  }
}

double act_value(int dt, const void* x, int64_t i) {
  if (dt == DT_F32) return ((const float*)x)[i];
  return bf16_value(((const uint16_t*)x)[i]);
}

// Weight matrices of all groups: element (g, n, k) of [G][N][K], K contiguous.
struct Weights {
  int dt;
  const void* w;
  const void* scale;  // i8: float [G][N]; q4: fp16 [G][N][K/32]
  const void* mn;     // q4: fp16 [G][N][K/32]
  int N, K;

  // Exact real value of a float-format weight (4-bit: the bf16 the layer uses).
  double value(int g, int n, int k) const {
    const int64_t i = ((int64_t)g * N + n) * K + k;
    switch (dt) {
      case DT_F32: return ((const float*)w)[i];
      case DT_BF16: return bf16_value(((const uint16_t*)w)[i]);
      case DT_Q4: {
        const uint8_t byte = ((const uint8_t*)w)[i / 2];
        const int q = (k & 1) ? (byte >> 4) : (byte & 15);
        const int64_t b = ((int64_t)g * N + n) * (K / 32) + k / 32;
        const float s = f16_value(((const uint16_t*)scale)[b]);
        const float m = f16_value(((const uint16_t*)mn)[b]);
        const float v = s * (float)q + m;  // s*q is exact in fp32; one rounding in the add
        return round_bf16(v);
      }
      case DT_MX4: {
        const uint8_t byte = ((const uint8_t*)w)[i / 2];
        const int code = (k & 1) ? (byte >> 4) : (byte & 15);
        const int64_t b = ((int64_t)g * N + n) * (K / 32) + k / 32;
        return e2m1_value(code) * e8m0_value(((const uint8_t*)scale)[b]);
      }
    }
    return NAN;
  }
  int qvalue(int g, int n, int k) const { return ((const int8_t*)w)[((int64_t)g * N + n) * K + k]; }
  float row_scale(int g, int n) const { return ((const float*)scale)[(int64_t)g * N + n]; }
};

template <class F>
void parallel_for(int64_t n, int threads, F&& f) {
  if (threads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  const int use = (int)std::min<int64_t>(threads, n);
  for (int t = 0; t < use; ++t)
    pool.emplace_back([&f, t, use, n] {
      for (int64_t i = t; i < n; i += use) f(i);
    });
  for (auto& th : pool) th.join();
}

double silu(double a) { return a / (1.0 + std::exp(-a)); }

// SiLU of the int8 path, in fp32: e = fp32(exp(-g)), then 1 + e and g / (1 + e),
// each rounded once to fp32.
float silu_f32(float g) {
  const float e = (float)std::exp(-(double)g);
  const float d = 1.0f + e;
  return g / d;
}

// Symmetric per-row int8 quantisation: s = max|v| / 127, q = clamp(rne(v / s), -127, 127).
void quant_row(int n, const float* v, int8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  const float s = amax / 127.0f;
  *s_out = s;
  for (int i = 0; i < n; ++i) {
    float r = 0.0f;
    if (s != 0.0f) r = std::min(127.0f, std::max(-127.0f, std::nearbyint(v[i] / s)));
    q[i] = (int8_t)r;
  }
}

}  // namespace

extern "C" {

// Router: logits[T][E] (fp32), topk_ids[T][k] (descending logit, ties to the
// lower expert id), topk_w[T][k] (softmax over the selected logits).
// x: [T][H] in act_dt (0 fp32, 1 bf16); w_router: [E][H] in act_dt; bias: [E] or null.
int oracle_route(int T, int H, int E, int k, int act_dt, const void* x, const void* w_router,
                 const float* bias, float* logits, int32_t* topk_ids, float* topk_w) {
  if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E) return -1;
  for (int t = 0; t < T; ++t) {
    float* l = logits + (int64_t)t * E;
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += act_value(act_dt, x, (int64_t)t * H + h) * act_value(act_dt, w_router, (int64_t)e * H + h);
      float v = (float)acc;
      if (bias) v = v + bias[e];
      l[e] = v;
    }
    std::vector<int> order((size_t)E);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [l](int a, int b) { return l[a] > l[b] || (l[a] == l[b] && a < b); });
    const double top = l[order[0]];
    std::vector<double> ex((size_t)k);
    double den = 0.0;
    for (int j = 0; j < k; ++j) {
      ex[j] = std::exp((double)l[order[j]] - top);
      den += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      topk_ids[(int64_t)t * k + j] = order[j];
      topk_w[(int64_t)t * k + j] = (float)(ex[j] / den);
    }
  }
  return 0;
}

// Grouping of (token, slot) pairs by expert.  Group e < E holds the tokens that
// chose e, in ascending token order; group E (if S == 1) holds every token in
// order.  offsets[G+1], row_token[R], token_row[T][k+S], R = T*k + S*T.
int oracle_permute(int T, int E, int k, int S, const int32_t* topk_ids, int32_t* offsets,
                   int32_t* row_token, int32_t* token_row) {
  if (T < 0 || E <= 0 || k < 1 || k > E || S < 0 || S > 1) return -1;
  const int G = E + S;
  std::vector<int64_t> count((size_t)G, 0);
  for (int64_t i = 0; i < (int64_t)T * k; ++i) {
    const int e = topk_ids[i];
    if (e < 0 || e >= E) return -2;
    ++count[e];
  }
  if (S) count[E] = T;
  offsets[0] = 0;
  for (int g = 0; g < G; ++g) offsets[g + 1] = (int32_t)(offsets[g] + count[g]);
  std::vector<int64_t> cursor(offsets, offsets + G);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const int e = topk_ids[(int64_t)t * k + j];
      const int64_t r = cursor[e]++;
      row_token[r] = t;
      token_row[(int64_t)t * (k + S) + j] = (int32_t)r;
    }
    if (S) {
      const int64_t r = cursor[E]++;
      row_token[r] = t;
      token_row[(int64_t)t * (k + S) + k] = (int32_t)r;
    }
  }
  return 0;
}

// Per-row symmetric int8 quantisation (per-token activation scales).
void oracle_quant_rows_i8(int rows, int cols, const float* v, int8_t* q, float* s) {
  for (int r = 0; r < rows; ++r) quant_row(cols, v + (int64_t)r * cols, q + (int64_t)r * cols, s + r);
}

// Gate/up projection and GLU of every permuted row.
//   float formats: h[r][i] = silu(x_t . Wg[g][i]) * (x_t . Wu[g][i]), fp64, where
//   Wg[g][i] = w_gu[g][i] and Wu[g][i] = w_gu[g][I + i].
//   int8 (w_dt 2): x comes as xq [T][H] int8 + xs [T] fp32; acc is exact, then
//   a = ((float)acc * xs[t]) * w_scale[g][n] and h = silu_f32(a_g) * a_u in fp32.
// Rows of group g are offsets[g] .. offsets[g+1]-1, token row_token[r].
int oracle_gu(int T, int H, int I, int G, const int32_t* offsets, const int32_t* row_token,
              int act_dt, const void* x, const int8_t* xq, const float* xs,
              int w_dt, const void* w, const void* w_scale, const void* w_min, double* h, int threads) {
  if (T < 0 || H <= 0 || I <= 0 || G <= 0) return -1;
  const Weights W{w_dt, w, w_scale, w_min, 2 * I, H};
  std::atomic<int> bad{0};
  for (int g = 0; g < G; ++g) {
    const int r0 = offsets[g], r1 = offsets[g + 1];
    if (r1 <= r0) continue;
    if (w_dt == DT_I8) {
      parallel_for((int64_t)(r1 - r0) * I, threads, [&](int64_t idx) {
        const int r = r0 + (int)(idx / I), i = (int)(idx % I), t = row_token[r];
        int64_t ag = 0, au = 0;
        for (int c = 0; c < H; ++c) {
          const int xv = xq[(int64_t)t * H + c];
          ag += (int64_t)xv * W.qvalue(g, i, c);
          au += (int64_t)xv * W.qvalue(g, I + i, c);
        }
        if (ag > INT32_MAX || ag < INT32_MIN || au > INT32_MAX || au < INT32_MIN) bad.store(1);
        const float a_g = ((float)ag * xs[t]) * W.row_scale(g, i);
        const float a_u = ((float)au * xs[t]) * W.row_scale(g, I + i);
        h[(int64_t)r * I + i] = (double)(silu_f32(a_g) * a_u);
      });
      continue;
    }
    // Decode this group's gate/up matrix once, then plain dot products.
    std::vector<double> Wd((size_t)2 * I * H);
    parallel_for(2 * I, threads, [&](int64_t n) {
      for (int c = 0; c < H; ++c) Wd[(size_t)n * H + c] = W.value(g, (int)n, c);
    });
    parallel_for(r1 - r0, threads, [&](int64_t rr) {
      const int r = r0 + (int)rr, t = row_token[r];
      std::vector<double> xr((size_t)H);
      if (w_dt == DT_MX4) {  // the token quantised to MXFP8, as the MX path multiplies it
        std::vector<float> xf((size_t)H);
        std::vector<uint8_t> codes((size_t)H), sc((size_t)H / 32);
        for (int c = 0; c < H; ++c) xf[c] = (float)act_value(act_dt, x, (int64_t)t * H + c);
        quant_mx8_row(H, xf.data(), codes.data(), sc.data(), xr.data());
      } else {
        for (int c = 0; c < H; ++c) xr[c] = act_value(act_dt, x, (int64_t)t * H + c);
      }
      for (int i = 0; i < I; ++i) {
        double ag = 0.0, au = 0.0;
        const double* wg = &Wd[(size_t)i * H];
        const double* wu = &Wd[(size_t)(I + i) * H];
        for (int c = 0; c < H; ++c) {
          ag += xr[c] * wg[c];
          au += xr[c] * wu[c];
        }
        h[(int64_t)r * I + i] = silu(ag) * au;
      }
    });
  }
  return bad.load() ? -3 : 0;
}

// Down projection of every permuted row: y[r][n] = h[r] . Wd[g][n].
//   float formats: fp64.  int8 (w_dt 2): h[r] (fp32 values) is quantised per
//   row (s = max|h| / 127), acc exact, y = ((float)acc * s) * w_scale[g][n].
int oracle_down(int H, int I, int G, const int32_t* offsets, const double* h,
                int w_dt, const void* w, const void* w_scale, const void* w_min, double* y, int threads) {
  if (H <= 0 || I <= 0 || G <= 0) return -1;
  const Weights W{w_dt, w, w_scale, w_min, H, I};
  std::atomic<int> bad{0};
  for (int g = 0; g < G; ++g) {
    const int r0 = offsets[g], r1 = offsets[g + 1];
    if (r1 <= r0) continue;
    if (w_dt == DT_I8) {
      parallel_for(r1 - r0, threads, [&](int64_t rr) {
        const int r = r0 + (int)rr;
        std::vector<float> hv((size_t)I);
        std::vector<int8_t> hq((size_t)I);
        for (int i = 0; i < I; ++i) hv[i] = (float)h[(int64_t)r * I + i];
        float s;
        quant_row(I, hv.data(), hq.data(), &s);
        for (int n = 0; n < H; ++n) {
          int64_t acc = 0;
          for (int i = 0; i < I; ++i) acc += (int64_t)hq[i] * W.qvalue(g, n, i);
          if (acc > INT32_MAX || acc < INT32_MIN) bad.store(1);
          y[(int64_t)r * H + n] = (double)(((float)acc * s) * W.row_scale(g, n));
        }
      });
      continue;
    }
    std::vector<double> Wd((size_t)H * I);
    parallel_for(H, threads, [&](int64_t n) {
      for (int i = 0; i < I; ++i) Wd[(size_t)n * I + i] = W.value(g, (int)n, i);
    });
    parallel_for(r1 - r0, threads, [&](int64_t rr) {
      const int r = r0 + (int)rr;
      const double* hr = h + (int64_t)r * I;
      std::vector<double> hq;
      if (w_dt == DT_MX4) {  // h rounded to fp32, then quantised to MXFP8 per block of 32
        std::vector<float> hf((size_t)I);
        std::vector<uint8_t> codes((size_t)I), sc((size_t)I / 32);
        hq.resize((size_t)I);
        for (int i = 0; i < I; ++i) hf[i] = (float)hr[i];
        quant_mx8_row(I, hf.data(), codes.data(), sc.data(), hq.data());
        hr = hq.data();
      }
      for (int n = 0; n < H; ++n) {
        double acc = 0.0;
        const double* wr = &Wd[(size_t)n * I];
        for (int i = 0; i < I; ++i) acc += hr[i] * wr[i];
        y[(int64_t)r * H + n] = acc;
      }
    });
  }
  return bad.load() ? -3 : 0;
}

// Gate-weighted combine: out[t] = sum_j g[t][j] * y[token_row[t][j]] (slots in
// stored order) + y[token_row[t][k]] if S (weight 1) + residual[t] if given.  fp64.
int oracle_combine(int T, int H, int k, int S, const int32_t* token_row, const float* topk_w,
                   const double* y, const float* residual, double* out) {
  if (T < 0 || H <= 0 || k < 1 || S < 0 || S > 1) return -1;
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)topk_w[(int64_t)t * k + j] * y[(int64_t)token_row[(int64_t)t * (k + S) + j] * H + n];
      if (S) acc += y[(int64_t)token_row[(int64_t)t * (k + S) + k] * H + n];
      if (residual) acc += residual[(int64_t)t * H + n];
      out[(int64_t)t * H + n] = acc;
    }
  return 0;
}

// RMSNorm with unit gain: xn = x / sqrt(mean(x^2) + eps), fp64.
void oracle_rmsnorm(int T, int H, double eps, const float* x, double* xn) {
  for (int t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) ss += (double)x[(int64_t)t * H + h] * x[(int64_t)t * H + h];
    const double inv = 1.0 / std::sqrt(ss / H + eps);
    for (int h = 0; h < H; ++h) xn[(int64_t)t * H + h] = (double)x[(int64_t)t * H + h] * inv;
  }
}

// MXFP8 quantisation of rows [rows][cols] (cols % 32 == 0): codes [rows][cols],
// scale bytes [rows][cols/32], and the values the codes stand for (fp64).
void oracle_quant_mx8(int rows, int cols, const float* v, uint8_t* codes, uint8_t* scales, double* deq) {
  for (int r = 0; r < rows; ++r)
    quant_mx8_row(cols, v + (int64_t)r * cols, codes + (int64_t)r * cols, scales + (int64_t)r * (cols / 32),
                  deq + (int64_t)r * cols);
}

// Decoded value of every MXFP4 weight of [G][N][K] (fp64).
void oracle_mx4_values(int G, int N, int K, const uint8_t* w, const uint8_t* scales, double* out) {
  const Weights W{DT_MX4, w, scales, nullptr, N, K};
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) out[((int64_t)g * N + n) * K + k] = W.value(g, n, k);
}

// Round fp64 values to bf16 (nearest, ties to even), returned as fp64.
void oracle_round_bf16(int64_t n, const double* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16_d(in[i]);
}

// Decoded value of every 4-bit weight of [G][N][K]: bf16_rne(fp32(scale * q + min)).
void oracle_q4_values(int G, int N, int K, const uint8_t* w, const uint16_t* scale, const uint16_t* mn, float* out) {
  const Weights W{DT_Q4, w, scale, mn, N, K};
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) out[((int64_t)g * N + n) * K + k] = (float)W.value(g, n, k);
}

}  // extern "C"
