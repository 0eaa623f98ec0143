// Launch interface between the C ABI (moe_api.cpp) and the kernels.  Every
// launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum WFmt { kF32 = 0, kBF16 = 1, kI8 = 2, kQ4 = 3, kMX4 = 4 };

struct RouteArgs {
  const void* x;
  const void* w_router;
  const float* bias;
  float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int T, H, E, k;
  bool act_f32;
  double* partials;  // fp64 scratch for the logits of a call split over slices of H (or null)
};

struct PermuteArgs {
  const int32_t* topk_ids;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* token_row;
  int32_t* sched;
  int T, E, k, S;
  bool big_on;    // cut groups of >= 128 rows into 128-row big tiles
  int big_start;  // int index of the big-tile list in the schedule
};

struct QuantArgs {  // per-row symmetric int8 quantisation
  const void* src;  // [rows][cols], bf16 bits or fp32
  bool src_f32;
  int8_t* q;
  float* scale;
  const int32_t* n_rows_dev;  // if non-null, rows = *n_rows_dev (device-resident count)
  int rows, cols;
};

struct GemmArgs {
  // activations: x [T][H] (gate/up) or h [R][I] (down); int8 variants in aq/as
  const void* act;
  const int8_t* act_q;
  const float* act_scale;   // per token (gate/up) or per row (down)
  const int32_t* row_token; // gate/up: row -> token; null for down (rows index act directly)
  const int32_t* sched;
  const void* w;
  const void* w_scale;
  const void* w_min;
  void* out;                // h [R][I] (gate/up) or y [R][H] (down)
  int K;                    // reduction length (H for gate/up, I for down)
  int N;                    // output columns (I for gate/up, H for down)
  int wfmt;                 // WFmt (also fixes the activation/output formats, see moe.h)
  int T;                    // tokens (gate/up clamps row_token into [0, T))
  int R;                    // permuted rows, T * (k + S)
  int G;                    // groups
};

struct CombineArgs {
  const void* y;
  bool y_f32;
  const int32_t* token_row;
  const float* topk_w;
  const float* residual;
  void* out;
  bool out_f32;
  int T, H, k, S;
  uint16_t* xn = nullptr;  // if set: also xn = bf16 RMSNorm(out) (out fp32, H <= 8192)
  float eps = 0.f;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// Routing + permutation of T <= kSmallRouteT tokens in two launches (fused
// decode path): `slices` slices of H (H % (256 * slices) == 0), fp64 partials
// [slices][T][E] in `partials`, int8 x quantisation when x_q is non-null.
constexpr int kSmallRouteT = 16;
constexpr int kRouteSlices = 8;
struct RoutePermuteArgs {
  RouteArgs r;
  PermuteArgs p;
  double* partials;
  int slices;
  int8_t* x_q;
  float* x_scale;
};
hipError_t launch_route_partials(const RouteArgs& a, double* partials, int slices, hipStream_t stream);
hipError_t launch_route_permute_small(const RoutePermuteArgs& a, hipStream_t stream);
// A call with more tokens whose 16 x 16 logit blocks would not fill the
// GPU's CUs splits H in kRouteSplit slices (partials summed by the top-k).
constexpr int kRouteSplit = 2;
// Bytes of fp64 partials kept after the logits in the logits buffer (max_tokens tokens).
inline size_t route_partials_bytes(int64_t max_tokens, int64_t E) {
  const int64_t few = (int64_t)kRouteSlices * (max_tokens < kSmallRouteT ? max_tokens : kSmallRouteT);
  const int64_t many = (int64_t)kRouteSplit * max_tokens;
  return (size_t)(few > many ? few : many) * (size_t)E * 8;
}
inline size_t route_partials_offset(int64_t max_tokens, int64_t E) { return ((size_t)max_tokens * E * 4 + 15) / 16 * 16; }
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t stream);
// MXFP8 (E4M3 codes, one E8M0 scale byte per 32 values) of rows of bf16 or
// fp32 values; cols % 256 == 0.
hipError_t launch_quant_mx8_rows(const void* src, bool src_f32, uint8_t* codes, uint8_t* scales, int64_t rows,
                                 int cols, hipStream_t stream);
hipError_t launch_gate_up(const GemmArgs& a, hipStream_t stream);
hipError_t launch_down(const GemmArgs& a, hipStream_t stream);
// Register-A / LDS-B grouped GEMMs over the big tiles (bf16 or 4-bit) and,
// with with_small (4-bit only), the small tiles in the same launch.
hipError_t launch_big_gate_up(const GemmArgs& a, bool with_small, hipStream_t stream);
hipError_t launch_big_down(const GemmArgs& a, bool with_small, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_rmsnorm(const float* x, uint16_t* xn, int T, int H, float eps, hipStream_t stream);

// The whole layer for a few tokens in one launch (decode.hip): (RMSNorm,)
// routing, permutation, gate/up, down and combine over one block per CU with
// grid-wide barriers in between.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeSyncBytes = 4096;    // barrier words (zero before the first launch)
constexpr int kDecodeMaxTH = 32768;       // T * H: the int8 path keeps every token's codes in LDS
constexpr int kDecodeMaxI = 512;          // staged h rows of four down items in LDS
struct DecodeArgs {
  const void* x;            // [T][H] bf16 layer input, or (norm_input) the fp32 residual stream
  const void* w_router;
  const float* bias;
  const void* w_gu; const void* gu_scale; const void* gu_min;
  const void* w_dn; const void* dn_scale; const void* dn_min;
  const float* residual;    // [T][H] fp32 or null (not with norm_input: x is the residual)
  void* out;                // [T][H] out dtype
  float eps;                // RMSNorm epsilon (norm_input)
  bool norm_input;          // layer input = bf16(RMSNorm(x)), out = x + MoE(that), fp32
  // layer buffers (same meaning as for the separate calls)
  float* logits; int32_t* topk_ids; float* topk_w; int32_t* offsets; int32_t* row_token; int32_t* token_row;
  int32_t* sched; int8_t* x_q; float* x_scale; void* h; void* y; int8_t* h_q; float* h_scale;
  double* partials;         // fp64 router partial sums [slices][T][E]
  uint32_t* sync;           // kDecodeSyncBytes of barrier words
  int T, H, I, E, k, S, wfmt, big_start;
  bool out_f32;
  long long spin_ns;        // bound on one barrier wait (then the status word is set and the wait ends)
};
hipError_t launch_decode_layer(const DecodeArgs& a, hipStream_t stream);
// Blocks of the decode launch on this device (0 if the device cannot host it).
int decode_blocks();
// Device address and size of the static scratch of the allocation-free
// decode call on the current device.
hipError_t decode_static_scratch(void** ptr, size_t* bytes);
// Word of the sync buffer that a timed-out barrier wait sets to nonzero.
constexpr int kDecodeStatusWord = 64 * 10;

// The permutation kernel keeps, per expert, a row of ceil(T / 32) 32-bit
// words of token bits plus a 16-bit prefix per word in LDS.  The row stride is
// made odd where that still fits, so the rows of 64 consecutive experts start
// in 64 different LDS banks (with 64 words per row, T = 2048, every row would
// start in the same bank and a wave's 64 lanes would collide on it).
constexpr size_t kPermuteMaxLds = 60 * 1024;
inline int permute_word_stride(int64_t T, int64_t E) {
  const int64_t W = (T + 31) / 32;
  return (int)((W | 1) * E * 6 <= (int64_t)kPermuteMaxLds ? (W | 1) : W);
}
// Dynamic LDS bytes the permutation kernel needs for T tokens and E experts.
inline size_t permute_lds_bytes(int64_t T, int64_t E) { return (size_t)permute_word_stride(T, E) * (size_t)E * 6; }

// Tile schedule capacity for R_max rows over G groups: small tiles first,
// then the big-tile list (every big tile holds at least 64 rows).
inline size_t sched_small_cap(int64_t r_max, int64_t G) { return (size_t)((r_max + 63) / 64 + G); }
inline size_t sched_big_start(int64_t r_max, int64_t G) { return 32 + 4 * sched_small_cap(r_max, G); }
inline size_t sched_ints(int64_t r_max, int64_t G) { return sched_big_start(r_max, G) + 4 * (size_t)(r_max / 64 + 1); }

}  // namespace moe
