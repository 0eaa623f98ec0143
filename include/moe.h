/*
 * moe.h -- C ABI of the routed Mixture-of-Experts FFN layer for AMD MI355X (gfx950).
 *
 * One MoE layer is five calls on one stream, in this order:
 *
 *   moe_route_topk        router logits, top-k experts and gates per token
 *   moe_permute           group (token, slot) pairs by expert + tile schedule
 *   moe_route_permute     the two above in one call (two launches for a few tokens)
 *   moe_grouped_gemm_gu   one launch: gate/up GEMM of every expert + SwiGLU
 *   moe_grouped_gemm_down one launch: down GEMM of every expert
 *   moe_combine           gate-weighted, atomic-free sum of each token's rows
 *   moe_combine_rmsnorm   the same, plus the RMSNorm of the result (stacked layers)
 *   (helpers: moe_rmsnorm, moe_quant_mx8)
 *
 * or, for a few tokens (decode steps), one call for all of it:
 *
 *   moe_decode_layer      the whole layer in one launch (T <= 16)
 *
 * The layer computed (the pages print no formula; this is the standard reading
 * of "top-8+shared", "GLU" and "concatenated expert GU, N = TOP_K x 2 x IM_EXP"
 * in "~2.7s fixed per-request TTFT = ~4,900 serialized per-expert NPU execs --
 * validated coarsening fix (concatenated-expert GEMM)", section "The fix"):
 *
 *   y_t = sum_{j<k} g_{t,j} FFN_{e_{t,j}}(x_t) + [n_shared] FFN_E(x_t)
 *   FFN_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),  silu(a) = a / (1 + exp(-a))
 *   e_{t,.} = the k largest router logits (ties: lower expert id first),
 *   g_{t,.} = softmax of those k logits.
 *
 * Grouping the work per expert instead of dispatching expert by expert is the
 * fix that page proposes (section "The fix"; also "eight tokens through each
 * expert in one go" in OpenFlowLM-Next issue #74, and "the lever is M>1" in
 * "MoE Decode Partition and Submit Floor", M2 update).  Expert shapes: gate/up
 * 2048x512 and down 512x2048 ("MoE Decode Partition and Submit Floor",
 * section 3, Test 1).
 *
 * Conventions (all entry points):
 *  - Every pointer except `desc`, `bufs` and `weights` (host structs) is
 *    device memory owned by the caller.  The library never allocates, frees
 *    or caches memory, keeps no state between calls, reads no environment and
 *    is safe to call from several threads.
 *  - Every call enqueues its kernels on `stream` and returns without
 *    synchronising.  No device-to-host copy happens inside a layer: expert
 *    counts and the tile schedule stay on the device.
 *  - Arguments are validated on the host first.  On any error the call returns
 *    a negative moe_status and enqueues nothing.  MOE_ERR_HIP reports a launch
 *    error; faults inside a kernel surface at the caller's next synchronisation.
 *  - T == 0 returns MOE_OK and enqueues nothing.
 *  - The calls of one layer take the same T (the GEMMs size their launches
 *    from it and read the schedule the permutation wrote for it).
 *  - The same inputs always produce the same bits (no atomics on data, fixed
 *    reduction orders, schedule-independent per-tile arithmetic).
 *  - Pointers must be 16-byte aligned; row-major layouts, last index contiguous.
 *
 * Groups: G = n_routed + n_shared.  Group e < n_routed is routed expert e; the
 * shared expert, if present, is group n_routed and receives every token.
 * Rows: R = T * (top_k + n_shared); R_max = max_tokens * (top_k + n_shared).
 */
#ifndef MOE_GFX950_H
#define MOE_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define MOE_ABI_VERSION 4

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,     /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2,     /* valid but not implemented combination (dtype, shape) */
  MOE_ERR_BUFFER_TOO_SMALL = -3,/* T > max_tokens */
  MOE_ERR_HIP = -4              /* a kernel launch failed */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,    /* IEEE binary32 */
  MOE_BF16 = 1,   /* bfloat16 bit patterns */
  MOE_I8 = 2,     /* int8 with one fp32 scale per output row (weights) or per token (activations) */
  MOE_Q4B32 = 3,  /* 4-bit unsigned codes in blocks of 32 along K, fp16 scale and fp16 min per block */
  MOE_MXFP4 = 4   /* OCP microscaling FP4: E2M1 elements in blocks of 32 along K, one E8M0 scale byte
                     per block (weights only; the activations then go through MXFP8) */
} moe_dtype;

/* Shape and formats of one layer.  Supported combinations (act, w, out):
 *   (F32, F32, F32)  fp32 throughout
 *   (BF16, BF16, BF16 or F32)
 *   (BF16, I8, BF16 or F32)    x quantised per token to int8 inside moe_permute
 *   (BF16, Q4B32, BF16 or F32) 4-bit weights dequantised to bf16 in registers
 *   (BF16, MXFP4, BF16 or F32) x and h quantised to MXFP8 (E4M3 elements, one E8M0
 *                              scale per 32) and multiplied by the scaled FP4 x FP8
 *                              MFMA (the OCP MX formats; "MoE Decode Partition and
 *                              Submit Floor", the FP4 data types it surveys)
 * Limits: hidden % 256 == 0, inter % 256 == 0, 1 <= n_routed <= 256,
 * 1 <= top_k <= min(16, n_routed), n_shared in {0, 1}, max_tokens >= 1 and
 * 6 * n_routed * ceil(max_tokens / 32) <= 61440 (the permutation keeps a token
 * bitmap and a 16-bit prefix per expert in LDS: max_tokens <= 2560 for 128
 * experts). */
typedef struct moe_desc {
  int32_t hidden;      /* H: model width (2048 in the pages' model) */
  int32_t inter;       /* I: expert intermediate width (512) */
  int32_t n_routed;    /* E: routed experts */
  int32_t top_k;       /* k: routed experts per token */
  int32_t n_shared;    /* S: always-on shared experts, 0 or 1 */
  int32_t max_tokens;  /* capacity the buffers were sized for */
  int32_t act_dtype;   /* moe_dtype of x and of the router weight: F32 or BF16 */
  int32_t w_dtype;     /* moe_dtype of the expert weights */
  int32_t out_dtype;   /* moe_dtype of the layer output: F32 or BF16 */
} moe_desc;

/* Expert weights of one projection, every group stacked: [G][N][K], K contiguous.
 * Gate/up: N = 2*inter (rows 0..I-1 gate, rows I..2I-1 up), K = hidden.
 * Down:    N = hidden, K = inter.
 *   F32/BF16: w = [G][N][K] values; scale = min = NULL.
 *   I8:       w = [G][N][K] int8; scale = float [G][N] (w_real = scale * w); min = NULL.
 *   Q4B32:    w = uint8 [G][N][K/2] (byte b of a block: code 2b low nibble, 2b+1 high nibble);
 *             scale, min = fp16 bits [G][N][K/32];
 *             w_real = bf16_rne(fp32(scale * q + min)): scale * q is exact in fp32, the add
 *             rounds once to fp32, and that fp32 value is rounded once more to bf16. */
/*   MXFP4:    w = uint8 [G][N][K/2] (byte b of a block: element 2b low nibble, 2b+1 high nibble,
 *             each an E2M1 code: sign, 2 exponent bits with bias 1, 1 mantissa bit, so the
 *             magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6); scale = uint8 E8M0 [G][N][K/32];
 *             w_real = e2m1(code) * 2^(scale - 127) (exact); min = NULL. */
typedef struct moe_weights {
  const void* w;
  const void* scale;
  const void* min;
} moe_weights;

/* Caller-owned device buffers shared by the five calls of a layer.  Sizes in
 * bytes come from moe_buffer_sizes (index = position in this struct). */
typedef struct moe_buffers {
  float* logits;            /* [max_tokens][E] fp32 router logits, then fp64 scratch of the router */
  int32_t* topk_ids;        /* [max_tokens][k] expert ids, descending logit */
  float* topk_w;            /* [max_tokens][k] gates */
  int32_t* expert_offsets;  /* [G+1] first row of each group; [G] = R */
  int32_t* row_token;       /* [R_max] token of each permuted row */
  int32_t* token_row;       /* [max_tokens][k+S] permuted row of each (token, slot); slot k = shared */
  int32_t* sched;           /* tile schedule: [0] = tile count, then {group, row0, rows, 0} per tile */
  int8_t* x_q;              /* [max_tokens][H] int8 activations (I8), E4M3 codes (MXFP4); else may be NULL */
  float* x_scale;           /* I8: [max_tokens] per-token fp32 scale; MXFP4: uint8 E8M0 [max_tokens][H/32] */
  void* h;                  /* [R_max][I] GLU output: F32 for F32/I8/MXFP4 weights, BF16 otherwise */
  void* y;                  /* [R_max][H] down output per row: F32 for F32/I8/MXFP4 weights, BF16 otherwise */
  int8_t* h_q;              /* [R_max][I] int8 (I8) or E4M3 (MXFP4) codes of h, quantised per row / block */
  float* h_scale;           /* I8: [R_max] per-row fp32 scale; MXFP4: uint8 E8M0 [R_max][I/32] */
  uint32_t* sync;           /* 4096 bytes of grid-barrier words for moe_decode_layer: zero them once after
                               allocation; every completed call leaves them valid for the next one.
                               Word 640 is the status word: nonzero after a barrier wait timed out (then
                               the call's results are undefined and the words must be zeroed again). */
} moe_buffers;

#define MOE_NUM_BUFFERS 14

/* Byte size of each moe_buffers member for `desc` (sizes[i] for member i).
 * Host only; touches no device.  Returns MOE_ERR_INVALID_ARG / UNSUPPORTED for
 * a bad or unsupported desc. */
moe_status moe_buffer_sizes(const moe_desc* desc, size_t sizes[MOE_NUM_BUFFERS]);

/* Router.  logits[t][e] = fp32(sum_h x[t][h] * w_router[e][h]) (+ bias[e], one
 * fp32 add), where the sum is accumulated in fp64 and rounded once; then the
 * k largest logits (ties -> lower id) in descending order into topk_ids, and
 * topk_w = their softmax, evaluated in fp64 and rounded once to fp32.
 *   x:        [T][H] act_dtype
 *   w_router: [E][H] act_dtype
 *   bias:     [E] fp32, or NULL for none
 * Writes bufs->logits (a call whose logits would not fill the GPU splits H in
 * two and keeps the fp64 partial sums in the scratch after the logits),
 * topk_ids, topk_w. */
moe_status moe_route_topk(const moe_desc* desc, int32_t T, const void* x, const void* w_router,
                          const float* bias, const moe_buffers* bufs, hipStream_t stream);

/* Permutation.  Groups (token, slot) pairs by expert with a wavefront-ballot
 * histogram and prefix sums: rows of group e are the tokens that chose e in
 * ascending token order; the shared group holds tokens 0..T-1.  Writes
 * expert_offsets, row_token, token_row and the tile schedule (tiles of at most
 * 64 rows of one group).  For I8 weights it also quantises x per token:
 * x_scale[t] = max_h |x[t][h]| / 127 and x_q = clamp(rne(x / x_scale), -127, 127)
 * (0 for an all-zero token).  For MXFP4 weights it quantises x to MXFP8 in
 * blocks of 32 along H (the OCP MX conversion): block max m = max |x|,
 * x_scale byte = clamp(floor(log2 m) - 8 + 127, 0, 254) (8: the exponent of
 * the largest E4M3 value, 448), x_q = the E4M3 code nearest x / 2^(byte - 127)
 * (ties to even mantissa, magnitudes above 448 saturated to 448); an all-zero
 * block has byte 0 and codes 0.
 *   x: [T][H] act_dtype (read only for I8 and MXFP4 weights; may be NULL otherwise)
 * Reads bufs->topk_ids. */
moe_status moe_permute(const moe_desc* desc, int32_t T, const void* x, const moe_buffers* bufs,
                       hipStream_t stream);

/* moe_route_topk followed by moe_permute, with the same arguments and the
 * same results bit for bit (logits, topk_ids, topk_w, expert_offsets,
 * row_token, token_row, the tile schedule, and x_q / x_scale for I8 weights).
 * For T <= 16 (decode steps) it runs in two launches instead of four: the
 * router logits are summed in fp64 over slices of H by many blocks (the
 * partial sums go to the scratch that follows the logits in bufs->logits),
 * then one block rounds them, selects the top-k, permutes and quantises.
 * (fp64 sums in a different order round to the same fp32 logit except in
 * cases that differ in the last fp64 bits exactly at an fp32 rounding
 * boundary.)  For larger T it makes the two calls. */
moe_status moe_route_permute(const moe_desc* desc, int32_t T, const void* x, const void* w_router,
                             const float* bias, const moe_buffers* bufs, hipStream_t stream);

/* Gate/up projection of every permuted row plus SwiGLU, all groups in one
 * launch over the tile schedule (for T >= 1024 with bf16 or MXFP4 weights
 * and T > 16 with Q4B32 weights, a launch of the big-tile kernel that takes
 * the 128-row tiles and the shorter ones; for those calls a token's rounding
 * may depend on the sizes of the groups it shares the call with, results
 * staying deterministic):
 *   h[r][i] = silu(x_t . Wg[g][i]) * (x_t . Wu[g][i]),  t = row_token[r], g = group of r.
 * Float weights: MFMA with fp32 accumulation, h stored in the h dtype.
 * I8 weights: exact int32 accumulation of x_q . w, then a = (fp32(acc) * x_scale[t]) * scale[g][n]
 * and h = (a_g / (1 + fp32(exp(-a_g)))) * a_u, each fp32 operation rounded once.
 * MXFP4 weights: the scaled FP4 x FP8 MFMA of the weight blocks and the MXFP8 blocks of x_q
 * (block scales applied inside the MFMA), fp32 accumulation, h in fp32.
 *   x: [T][H] act_dtype (unused for I8 weights, which read bufs->x_q / x_scale)
 * Reads expert_offsets, row_token, sched; writes bufs->h. */
moe_status moe_grouped_gemm_gu(const moe_desc* desc, int32_t T, const void* x, const moe_weights* w_gu,
                               const moe_buffers* bufs, hipStream_t stream);

/* Down projection of every permuted row, all groups in one launch (as for
 * gate/up; I8 and MXFP4 weights add one launch before it that quantises h):
 *   y[r][n] = h[r] . Wd[g][n].
 * I8 weights: each row of h is first quantised into h_q / h_scale
 * (s = max|h[r]| / 127, q = clamp(rne(h / s), -127, 127)); then
 * y = (fp32(acc) * s) * scale[g][n] with acc the exact int32 sum.
 * MXFP4 weights: each row of h (fp32) is quantised to MXFP8 in blocks of 32
 * (the conversion moe_permute applies to x) into h_q / h_scale; then the
 * scaled FP4 x FP8 MFMA with fp32 accumulation gives y in fp32.
 * Reads h, expert_offsets, sched; writes bufs->y (and h_q, h_scale for I8 and MXFP4). */
moe_status moe_grouped_gemm_down(const moe_desc* desc, int32_t T, const moe_weights* w_down,
                                 const moe_buffers* bufs, hipStream_t stream);

/* Combine.  out[t] = sum_{j<k} topk_w[t][j] * y[token_row[t][j]] (slots in
 * order) + y[token_row[t][k]] (shared, weight 1) + residual[t], in fp32, each
 * output element written by exactly one thread (no atomics).
 *   residual: [T][H] fp32 or NULL
 *   out:      [T][H] out_dtype */
moe_status moe_combine(const moe_desc* desc, int32_t T, const float* residual, void* out,
                       const moe_buffers* bufs, hipStream_t stream);

/* The whole layer for 1 <= T <= 16 tokens in one launch.  Decode steps are
 * where the cost per dispatched operation, not the arithmetic, sets the time
 * ("MoE Decode Partition and Submit Floor", section 3; "~2.7s fixed
 * per-request TTFT = ~4,900 serialized per-expert NPU execs", section
 * "Evidence").  The launch holds one block per CU and three grid-wide
 * barriers (it must not share the GPU with work that never finishes;
 * concurrent calls must not share bufs->sync).
 *   flags = 0: x is [T][H] bf16 (act_dtype BF16); out = MoE(x) (+ residual if
 *     not NULL), in out_dtype: the results of moe_route_permute,
 *     moe_grouped_gemm_gu, moe_grouped_gemm_down and moe_combine(residual).
 *   flags = MOE_DECODE_NORM_INPUT (one stacked layer): x is the [T][H] fp32
 *     residual stream; the layer input is xn = bf16(RMSNorm(x, eps)) (the bits
 *     of moe_rmsnorm) and out = x + MoE(xn) in fp32 (out_dtype must be F32,
 *     residual must be NULL); out may be x (updated in place).
 * Either way every buffer the separate calls write (logits, topk_ids,
 * topk_w, expert_offsets, row_token, token_row, sched, x_q, x_scale, h, h_q,
 * h_scale, y) holds the same bits as after those calls.
 *   w_router: [E][H] bf16;  bias: [E] fp32 or NULL
 *   w_gu, w_down: as for the GEMM calls (BF16, I8, Q4B32 or MXFP4 weights)
 *   residual: [T][H] fp32 or NULL
 * Limits (else MOE_ERR_UNSUPPORTED): T * hidden <= 32768, inter <= 512,
 * hidden <= 8192, weights BF16, I8, Q4B32 or MXFP4. */
#define MOE_DECODE_NORM_INPUT 1
moe_status moe_decode_layer(const moe_desc* desc, int32_t T, const void* x, const void* w_router, const float* bias,
                            const moe_weights* w_gu, const moe_weights* w_down, const float* residual,
                            int32_t flags, float eps, void* out, const moe_buffers* bufs, hipStream_t stream);

/* moe_decode_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and the same bits, with no buffers
 * argument.  The layer buffers of the call live in a static 8 MiB device
 * array of the library, which each GPU the library runs on holds until the
 * process ends; the call allocates nothing.  The desc's max_tokens is
 * ignored (the array is laid out for 16 tokens); T <= 16, and a desc whose
 * buffers for 16 tokens exceed 8 MiB returns MOE_ERR_UNSUPPORTED (the layer
 * shapes of the pages' model, hidden 2048, 128 experts, take about 1.8 MiB).
 * Every call on one GPU shares that GPU's array and leaves its contents there:
 * calls that overlap on one GPU (other streams, other threads) race.  The
 * grid-barrier words sit at the start of the array for every desc (zero at
 * load, valid after each completed call), the other buffers after them. */
moe_status moe_decode_layer_static(const moe_desc* desc, int32_t T, const void* x, const void* w_router,
                                   const float* bias, const moe_weights* w_gu, const moe_weights* w_down,
                                   const float* residual, int32_t flags, float eps, void* out,
                                   hipStream_t stream);

/* MXFP8 quantisation (OCP MX: E4M3 elements, one E8M0 scale byte per 32 consecutive
 * values of a row), the conversion moe_permute applies to x and moe_grouped_gemm_down
 * to h for MXFP4 weights: block maximum m = max |v|; scale byte = clamp(floor(log2 m)
 * - 8 + 127, 0, 254) (8: the exponent of 448, the largest E4M3 value), or 0 when
 * m = 0; code = the E4M3 value nearest v / 2^(byte - 127), ties to the even mantissa,
 * magnitudes above 448 saturated to 448, 0 for an all-zero block.
 *   src:    [rows][cols] fp32 (src_dtype MOE_F32) or bf16 (MOE_BF16)
 *   codes:  [rows][cols] E4M3 bytes;  scales: [rows][cols / 32] E8M0 bytes
 * cols % 256 == 0 (else MOE_ERR_UNSUPPORTED); src and codes 16-byte aligned. */
moe_status moe_quant_mx8(int64_t rows, int32_t cols, int32_t src_dtype, const void* src, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream);

/* RMSNorm with unit gain for stacked layers: xn[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps)),
 * computed in fp32.  x: [T][H] fp32; xn: [T][H] bf16.  H % 256 == 0. */
moe_status moe_rmsnorm(int32_t T, int32_t H, float eps, const float* x, void* xn, hipStream_t stream);

/* Combine fused with the RMSNorm of its result, for stacked layers
 * x_{l+1} = x_l + MoE_l(RMSNorm(x_l)): writes out exactly as moe_combine
 * (fp32 residual stream) and xn = bf16(out[t] / sqrt(mean(out[t]^2) + eps)),
 * bit for bit what moe_rmsnorm gives on that out, so the next layer's input
 * needs no launch of its own.
 *   residual: [T][H] fp32 or NULL;  out: [T][H] fp32;  xn: [T][H] bf16
 * desc->out_dtype must be MOE_F32 and hidden <= 8192 (else
 * MOE_ERR_UNSUPPORTED); eps >= 0.  xn may not alias out or residual. */
moe_status moe_combine_rmsnorm(const moe_desc* desc, int32_t T, const float* residual, float eps, void* out,
                               void* xn, const moe_buffers* bufs, hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GFX950_H */
