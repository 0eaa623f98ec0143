// C ABI of the routed MoE layer (include/moe.h): argument validation, buffer
// sizing and kernel launches.  Nothing here allocates, synchronises, reads the
// environment or keeps state; every check runs before the first launch, so an
// error return means nothing was enqueued.
#include "moe.h"

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace {

using moe::kBF16;
using moe::kF32;
using moe::kI8;
using moe::kQ4;

// Weights whose activations are quantised before the GEMMs (x_q, h_q).
bool quant_act(const moe_desc* d) { return d->w_dtype == MOE_I8 || d->w_dtype == MOE_MXFP4; }
bool mx(const moe_desc* d) { return d->w_dtype == MOE_MXFP4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->inter <= 0 || d->n_routed <= 0 || d->top_k <= 0 || d->max_tokens <= 0)
    return MOE_ERR_INVALID_ARG;
  if (d->top_k > d->n_routed || d->n_shared < 0 || d->n_shared > 1) return MOE_ERR_INVALID_ARG;
  if (d->hidden % 256 || d->inter % 256) return MOE_ERR_UNSUPPORTED;
  if (d->n_routed > 256 || d->top_k > 16) return MOE_ERR_UNSUPPORTED;
  if (moe::permute_lds_bytes(d->max_tokens, d->n_routed) > moe::kPermuteMaxLds) return MOE_ERR_UNSUPPORTED;
  const int a = d->act_dtype, w = d->w_dtype, o = d->out_dtype;
  if (a < MOE_F32 || a > MOE_MXFP4 || w < MOE_F32 || w > MOE_MXFP4 || o < MOE_F32 || o > MOE_MXFP4)
    return MOE_ERR_INVALID_ARG;
  if (o != MOE_F32 && o != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (a == MOE_F32) {
    if (w != MOE_F32 || o != MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else if (a == MOE_BF16) {
    if (w == MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Checks shared by every per-layer call: desc, T, the buffer struct.
moe_status check_call(const moe_desc* d, int32_t T, const moe_buffers* b) {
  const moe_status s = check_desc(d);
  if (s != MOE_OK) return s;
  if (T < 0 || !b) return MOE_ERR_INVALID_ARG;
  if (T > d->max_tokens) return MOE_ERR_BUFFER_TOO_SMALL;
  return MOE_OK;
}

bool ptr_ok(const void* p) { return p && aligned16(p); }

int groups(const moe_desc* d) { return d->n_routed + d->n_shared; }
int64_t rows(const moe_desc* d, int64_t T) { return T * (d->top_k + d->n_shared); }
bool f32_intermediates(const moe_desc* d) {
  return d->w_dtype == MOE_F32 || d->w_dtype == MOE_I8 || d->w_dtype == MOE_MXFP4;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Big tiles (128 rows, register-A / LDS-B kernel) for long prefill
// chunks with bf16 or 4-bit weights; a host-side rule on T alone.
// The 4-bit big-tile kernel addresses weights and activations with 32-bit
// byte offsets and keeps an item's scales and mins in LDS (hidden and inter
// multiples of 256 up to 2048); other layers keep the small-tile kernel.
bool q4_offsets_fit(const moe_desc* d) {
  if (d->hidden % 256 || d->inter % 256 || d->hidden > 2048 || d->inter > 2048) return false;
  const int64_t H = d->hidden, I = d->inter, G = d->n_routed + d->n_shared;
  const int64_t r_max = (int64_t)d->max_tokens * (d->top_k + d->n_shared);
  const int64_t lim = (int64_t)1 << 32;
  return G * 2 * I * (H / 2) < lim && (int64_t)d->max_tokens * H * 2 < lim && r_max * I * 2 < lim;
}

// The same for MXFP4 weights (E4M3 activations: one byte per element); the MX
// big-tile kernel also keeps an item's scale bytes in LDS, which takes
// hidden and inter multiples of 512 up to 2048.
bool mx_offsets_fit(const moe_desc* d) {
  if (d->hidden % 512 || d->inter % 512 || d->hidden > 2048 || d->inter > 2048) return false;
  const int64_t H = d->hidden, I = d->inter, G = d->n_routed + d->n_shared;
  const int64_t r_max = (int64_t)d->max_tokens * (d->top_k + d->n_shared);
  const int64_t lim = (int64_t)1 << 32;
  return G * 2 * I * (H / 2) < lim && (int64_t)d->max_tokens * H < lim && r_max * I < lim;
}

bool big_tiles(const moe_desc* d, int32_t T) {
  if (T < (d->w_dtype == MOE_Q4B32 ? moe::kBigTileMinTokensQ4 : moe::kBigTileMinTokens)) return false;
  return d->w_dtype == MOE_BF16 || (d->w_dtype == MOE_Q4B32 && q4_offsets_fit(d)) ||
         (d->w_dtype == MOE_MXFP4 && mx_offsets_fit(d));
}

// With big tiles on, the small tiles go through the big-tile kernel too, in
// the same launch as the big tiles (one launch per GEMM at every T).
bool small_in_big(const moe_desc* d, int32_t T) { return big_tiles(d, T); }

moe_status check_weights(const moe_desc* d, const moe_weights* w) {
  if (!w || !ptr_ok(w->w)) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype == MOE_I8 && !ptr_ok(w->scale)) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype == MOE_Q4B32 && (!ptr_ok(w->scale) || !ptr_ok(w->min))) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype == MOE_MXFP4 && !ptr_ok(w->scale)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case MOE_ERR_BUFFER_TOO_SMALL: return "T exceeds max_tokens";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

moe_status moe_buffer_sizes(const moe_desc* d, size_t sizes[MOE_NUM_BUFFERS]) {
  const moe_status s = check_desc(d);
  if (s != MOE_OK) return s;
  if (!sizes) return MOE_ERR_INVALID_ARG;
  const size_t M = (size_t)d->max_tokens, E = (size_t)d->n_routed, k = (size_t)d->top_k;
  const size_t S = (size_t)d->n_shared, H = (size_t)d->hidden, I = (size_t)d->inter;
  const size_t G = E + S, Rmax = M * (k + S);
  const bool i8 = d->w_dtype == MOE_I8, q = quant_act(d), m = mx(d);
  const size_t fw = f32_intermediates(d) ? 4 : 2;
  sizes[0] = moe::route_partials_offset(M, E) + moe::route_partials_bytes(M, E);  // logits + fused-route scratch
  sizes[1] = M * k * 4;                                  // topk_ids
  sizes[2] = M * k * 4;                                  // topk_w
  sizes[3] = (G + 1) * 4;                                // expert_offsets
  sizes[4] = Rmax * 4;                                   // row_token
  sizes[5] = M * (k + S) * 4;                            // token_row
  sizes[6] = moe::sched_ints((int64_t)Rmax, (int64_t)G) * 4;  // sched
  sizes[7] = q ? M * H : 0;                              // x_q
  sizes[8] = i8 ? M * 4 : m ? M * (H / 32) : 0;          // x_scale
  sizes[9] = Rmax * I * fw;                              // h
  sizes[10] = Rmax * H * fw;                             // y
  sizes[11] = q ? Rmax * I : 0;                          // h_q
  sizes[12] = i8 ? Rmax * 4 : m ? Rmax * (I / 32) : 0;   // h_scale
  sizes[13] = moe::kDecodeSyncBytes;                     // sync
  return MOE_OK;
}

// fp64 partial logits, kept after the logits in the logits buffer
double* route_scratch(const moe_desc* d, const moe_buffers* b) {
  return (double*)((char*)b->logits + moe::route_partials_offset(d->max_tokens, d->n_routed));
}

moe_status moe_route_topk(const moe_desc* d, int32_t T, const void* x, const void* w_router, const float* bias,
                          const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if (!ptr_ok(x) || !ptr_ok(w_router) || (bias && !aligned16(bias))) return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(b->logits) || !ptr_ok(b->topk_ids) || !ptr_ok(b->topk_w)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  moe::RouteArgs a{x, w_router, bias, b->logits, b->topk_ids, b->topk_w, T, d->hidden, d->n_routed, d->top_k,
                   d->act_dtype == MOE_F32, route_scratch(d, b)};
  return hip_status(moe::launch_route(a, stream));
}

moe_status moe_permute(const moe_desc* d, int32_t T, const void* x, const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if (!ptr_ok(b->topk_ids) || !ptr_ok(b->expert_offsets) || !ptr_ok(b->row_token) || !ptr_ok(b->token_row) ||
      !ptr_ok(b->sched))
    return MOE_ERR_INVALID_ARG;
  const bool i8 = d->w_dtype == MOE_I8;
  if (quant_act(d) && (!ptr_ok(x) || !ptr_ok(b->x_q) || !ptr_ok(b->x_scale))) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (i8) {
    moe::QuantArgs q{x, d->act_dtype == MOE_F32, b->x_q, b->x_scale, nullptr, T, d->hidden};
    const hipError_t e = moe::launch_quant_rows(q, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (mx(d)) {
    const hipError_t e = moe::launch_quant_mx8_rows(x, d->act_dtype == MOE_F32, (uint8_t*)b->x_q,
                                                    (uint8_t*)b->x_scale, T, d->hidden, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  const int64_t r_max = (int64_t)d->max_tokens * (d->top_k + d->n_shared);
  moe::PermuteArgs a{b->topk_ids, b->expert_offsets, b->row_token, b->token_row, b->sched, T, d->n_routed,
                     d->top_k, d->n_shared, big_tiles(d, T), (int)moe::sched_big_start(r_max, groups(d))};
  return hip_status(moe::launch_permute(a, stream));
}

moe_status moe_route_permute(const moe_desc* d, int32_t T, const void* x, const void* w_router, const float* bias,
                             const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  const bool i8 = d->w_dtype == MOE_I8;
  if (!ptr_ok(x) || !ptr_ok(w_router) || (bias && !aligned16(bias))) return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(b->logits) || !ptr_ok(b->topk_ids) || !ptr_ok(b->topk_w) || !ptr_ok(b->expert_offsets) ||
      !ptr_ok(b->row_token) || !ptr_ok(b->token_row) || !ptr_ok(b->sched))
    return MOE_ERR_INVALID_ARG;
  if (quant_act(d) && (!ptr_ok(b->x_q) || !ptr_ok(b->x_scale))) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (T > moe::kSmallRouteT) {
    if ((s = moe_route_topk(d, T, x, w_router, bias, b, stream)) != MOE_OK) return s;
    return moe_permute(d, T, x, b, stream);
  }
  int slices = moe::kRouteSlices;
  while (d->hidden % (256 * slices) != 0) slices /= 2;
  const int64_t r_max = (int64_t)d->max_tokens * (d->top_k + d->n_shared);
  moe::RoutePermuteArgs a{};
  a.r = moe::RouteArgs{x, w_router, bias, b->logits, b->topk_ids, b->topk_w, T, d->hidden, d->n_routed, d->top_k,
                       d->act_dtype == MOE_F32, route_scratch(d, b)};
  a.p = moe::PermuteArgs{b->topk_ids, b->expert_offsets, b->row_token, b->token_row, b->sched, T, d->n_routed,
                         d->top_k, d->n_shared, false, (int)moe::sched_big_start(r_max, groups(d))};
  a.partials = route_scratch(d, b);
  a.slices = slices;
  a.x_q = i8 ? b->x_q : nullptr;
  a.x_scale = i8 ? b->x_scale : nullptr;
  if (mx(d)) {
    const hipError_t e = moe::launch_quant_mx8_rows(x, d->act_dtype == MOE_F32, (uint8_t*)b->x_q,
                                                    (uint8_t*)b->x_scale, T, d->hidden, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(moe::launch_route_permute_small(a, stream));
}

moe_status moe_grouped_gemm_gu(const moe_desc* d, int32_t T, const void* x, const moe_weights* w,
                               const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if ((s = check_weights(d, w)) != MOE_OK) return s;
  const bool q = quant_act(d);
  if (q ? (!ptr_ok(b->x_q) || !ptr_ok(b->x_scale)) : !ptr_ok(x)) return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(b->row_token) || !ptr_ok(b->sched) || !ptr_ok(b->h)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  moe::GemmArgs a{};
  a.act = q ? nullptr : x;
  a.act_q = q ? b->x_q : nullptr;
  a.act_scale = q ? b->x_scale : nullptr;
  a.row_token = b->row_token;
  a.sched = b->sched;
  a.w = w->w;
  a.w_scale = w->scale;
  a.w_min = w->min;
  a.out = b->h;
  a.K = d->hidden;
  a.N = d->inter;
  a.wfmt = d->w_dtype;
  a.T = T;
  a.R = (int)rows(d, T);
  a.G = groups(d);
  if (small_in_big(d, T)) return hip_status(moe::launch_big_gate_up(a, true, stream));
  return hip_status(moe::launch_gate_up(a, stream));
}

moe_status moe_grouped_gemm_down(const moe_desc* d, int32_t T, const moe_weights* w, const moe_buffers* b,
                                 hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if ((s = check_weights(d, w)) != MOE_OK) return s;
  const bool i8 = d->w_dtype == MOE_I8, q = quant_act(d);
  if (!ptr_ok(b->h) || !ptr_ok(b->sched) || !ptr_ok(b->y)) return MOE_ERR_INVALID_ARG;
  if (q && (!ptr_ok(b->h_q) || !ptr_ok(b->h_scale))) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const int R = (int)rows(d, T);
  if (i8) {
    moe::QuantArgs qa{b->h, true, b->h_q, b->h_scale, nullptr, R, d->inter};
    const hipError_t e = moe::launch_quant_rows(qa, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (mx(d)) {
    const hipError_t e =
        moe::launch_quant_mx8_rows(b->h, true, (uint8_t*)b->h_q, (uint8_t*)b->h_scale, R, d->inter, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  moe::GemmArgs a{};
  a.act = q ? nullptr : b->h;
  a.act_q = q ? b->h_q : nullptr;
  a.act_scale = q ? b->h_scale : nullptr;
  a.row_token = nullptr;
  a.sched = b->sched;
  a.w = w->w;
  a.w_scale = w->scale;
  a.w_min = w->min;
  a.out = b->y;
  a.K = d->inter;
  a.N = d->hidden;
  a.wfmt = d->w_dtype;
  a.T = T;
  a.R = R;
  a.G = groups(d);
  if (small_in_big(d, T)) return hip_status(moe::launch_big_down(a, true, stream));
  return hip_status(moe::launch_down(a, stream));
}

moe_status moe_combine(const moe_desc* d, int32_t T, const float* residual, void* out, const moe_buffers* b,
                       hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if (!ptr_ok(out) || !ptr_ok(b->y) || !ptr_ok(b->token_row) || !ptr_ok(b->topk_w) ||
      (residual && !aligned16(residual)))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  moe::CombineArgs a{b->y, f32_intermediates(d), b->token_row, b->topk_w, residual, out,
                     d->out_dtype == MOE_F32, T, d->hidden, d->top_k, d->n_shared};
  return hip_status(moe::launch_combine(a, stream));
}

moe_status moe_combine_rmsnorm(const moe_desc* d, int32_t T, const float* residual, float eps, void* out, void* xn,
                               const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if (!ptr_ok(out) || !ptr_ok(xn) || !ptr_ok(b->y) || !ptr_ok(b->token_row) || !ptr_ok(b->topk_w) ||
      (residual && !aligned16(residual)) || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (d->out_dtype != MOE_F32 || d->hidden > 8192) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  moe::CombineArgs a{b->y, f32_intermediates(d), b->token_row, b->topk_w, residual, out, true, T, d->hidden,
                     d->top_k, d->n_shared, (uint16_t*)xn, eps};
  return hip_status(moe::launch_combine(a, stream));
}

moe_status moe_decode_layer(const moe_desc* d, int32_t T, const void* x, const void* w_router, const float* bias,
                            const moe_weights* w_gu, const moe_weights* w_down, const float* residual,
                            int32_t flags, float eps, void* out, const moe_buffers* b, hipStream_t stream) {
  moe_status s = check_call(d, T, b);
  if (s != MOE_OK) return s;
  if ((s = check_weights(d, w_gu)) != MOE_OK || (s = check_weights(d, w_down)) != MOE_OK) return s;
  const bool norm = (flags & MOE_DECODE_NORM_INPUT) != 0;
  if ((flags & ~MOE_DECODE_NORM_INPUT) != 0 || (norm && residual)) return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(x) || !ptr_ok(w_router) || (bias && !aligned16(bias)) || !ptr_ok(out) ||
      (residual && !aligned16(residual)) || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(b->logits) || !ptr_ok(b->topk_ids) || !ptr_ok(b->topk_w) || !ptr_ok(b->expert_offsets) ||
      !ptr_ok(b->row_token) || !ptr_ok(b->token_row) || !ptr_ok(b->sched) || !ptr_ok(b->h) || !ptr_ok(b->y) ||
      !ptr_ok(b->sync))
    return MOE_ERR_INVALID_ARG;
  if (quant_act(d) && (!ptr_ok(b->x_q) || !ptr_ok(b->x_scale) || !ptr_ok(b->h_q) || !ptr_ok(b->h_scale)))
    return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_BF16 || d->w_dtype == MOE_F32 || (norm && d->out_dtype != MOE_F32))
    return MOE_ERR_UNSUPPORTED;
  if (T > moe::kDecodeMaxT || (int64_t)T * d->hidden > moe::kDecodeMaxTH || d->inter > moe::kDecodeMaxI ||
      d->hidden > 8192)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (moe::decode_blocks() == 0) return MOE_ERR_UNSUPPORTED;
  const int64_t r_max = (int64_t)d->max_tokens * (d->top_k + d->n_shared);
  moe::DecodeArgs a{};
  a.x = x;
  a.w_router = w_router;
  a.bias = bias;
  a.w_gu = w_gu->w;
  a.gu_scale = w_gu->scale;
  a.gu_min = w_gu->min;
  a.w_dn = w_down->w;
  a.dn_scale = w_down->scale;
  a.dn_min = w_down->min;
  a.residual = residual;
  a.out = out;
  a.eps = eps;
  a.norm_input = norm;
  a.logits = b->logits;
  a.topk_ids = b->topk_ids;
  a.topk_w = b->topk_w;
  a.offsets = b->expert_offsets;
  a.row_token = b->row_token;
  a.token_row = b->token_row;
  a.sched = b->sched;
  a.x_q = b->x_q;
  a.x_scale = b->x_scale;
  a.h = b->h;
  a.y = b->y;
  a.h_q = b->h_q;
  a.h_scale = b->h_scale;
  a.partials = route_scratch(d, b);
  a.sync = b->sync;
  a.T = T;
  a.H = d->hidden;
  a.I = d->inter;
  a.E = d->n_routed;
  a.k = d->top_k;
  a.S = d->n_shared;
  a.wfmt = d->w_dtype;
  a.big_start = (int)moe::sched_big_start(r_max, groups(d));
  a.out_f32 = d->out_dtype == MOE_F32;
  a.spin_ns = 100000000LL;  // 0.1 s: far beyond any wait of a launch whose blocks are all resident
  return hip_status(moe::launch_decode_layer(a, stream));
}

moe_status moe_decode_layer_static(const moe_desc* d, int32_t T, const void* x, const void* w_router,
                                   const float* bias, const moe_weights* w_gu, const moe_weights* w_down,
                                   const float* residual, int32_t flags, float eps, void* out,
                                   hipStream_t stream) {
  if (!d) return MOE_ERR_INVALID_ARG;
  moe_desc ds = *d;  // the layout of the static buffers: room for kDecodeMaxT tokens
  ds.max_tokens = moe::kDecodeMaxT;
  moe_status s = check_desc(&ds);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > moe::kDecodeMaxT) return MOE_ERR_UNSUPPORTED;
  size_t sizes[MOE_NUM_BUFFERS];
  if ((s = moe_buffer_sizes(&ds, sizes)) != MOE_OK) return s;
  if (T == 0) {  // the other arguments are still checked; nothing touches the device
    void* const fake = (void*)(uintptr_t)256;
    const moe_buffers b0{(float*)fake, (int32_t*)fake, (float*)fake, (int32_t*)fake, (int32_t*)fake,
                         (int32_t*)fake, (int32_t*)fake, (int8_t*)fake, (float*)fake, fake, fake, (int8_t*)fake,
                         (float*)fake, (uint32_t*)fake};
    return moe_decode_layer(&ds, 0, x, w_router, bias, w_gu, w_down, residual, flags, eps, out, &b0, stream);
  }
  size_t total = 0;
  for (size_t z : sizes) total += (z + 255) / 256 * 256;
  void* base = nullptr;
  size_t cap = 0;
  if (moe::decode_static_scratch(&base, &cap) != hipSuccess) return MOE_ERR_HIP;
  if (total > cap) return MOE_ERR_UNSUPPORTED;
  // The grid-barrier words first, at the same place for every desc: they
  // stay valid from one call to the next only if no other layout puts its
  // data there (the rest of the layout depends on the desc's dtypes and sizes).
  static_assert(MOE_NUM_BUFFERS == 14, "sync is buffer 13");
  void* p[MOE_NUM_BUFFERS];
  size_t off = (sizes[13] + 255) / 256 * 256;
  p[13] = base;
  for (int i = 0; i < MOE_NUM_BUFFERS - 1; ++i) {
    p[i] = sizes[i] ? (void*)((char*)base + off) : nullptr;
    off += (sizes[i] + 255) / 256 * 256;
  }
  const moe_buffers b{(float*)p[0], (int32_t*)p[1], (float*)p[2], (int32_t*)p[3], (int32_t*)p[4], (int32_t*)p[5],
                      (int32_t*)p[6], (int8_t*)p[7], (float*)p[8], p[9], p[10], (int8_t*)p[11], (float*)p[12],
                      (uint32_t*)p[13]};
  return moe_decode_layer(&ds, T, x, w_router, bias, w_gu, w_down, residual, flags, eps, out, &b, stream);
}

moe_status moe_quant_mx8(int64_t rows, int32_t cols, int32_t src_dtype, const void* src, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || (src_dtype != MOE_F32 && src_dtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  if (cols % 256) return MOE_ERR_UNSUPPORTED;
  if (!ptr_ok(src) || !ptr_ok(codes) || !scales) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if ((uint64_t)rows * (uint64_t)cols / 2048 + 1 > (uint64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_quant_mx8_rows(src, src_dtype == MOE_F32, codes, scales, rows, cols, stream));
}

moe_status moe_rmsnorm(int32_t T, int32_t H, float eps, const float* x, void* xn, hipStream_t stream) {
  if (T < 0 || H <= 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (H % 256) return MOE_ERR_UNSUPPORTED;
  if (!ptr_ok(x) || !ptr_ok(xn)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_rmsnorm(x, (uint16_t*)xn, T, H, eps, stream));
}

}  // extern "C"
