"""Parity of the HIP path (through the C ABI) with the CPU oracle, step by step
and end to end, on seeded inputs.  Routing ids, permutation and the int8
path are compared bit for bit; float outputs against the fp64 oracle with the
stated tolerances (max |err| / max |ref| and RMSE)."""
import sys

import numpy as np
import pytest

from gen import synth
from gen.synth import LayerSpec
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case_inputs(H, I, E, k, S, T, wt, zipf=0.0, seed=0, out=None):
    act = "f32" if wt == "f32" else "bf16"
    out = out or ("f32" if wt == "f32" else "bf16")
    spec = LayerSpec(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=S, act=act, wt=wt, out=out, zipf=zipf)
    wid = 5000 + seed
    d = synth.layer_weights(spec, wid)
    d["x"] = synth.tokens(spec, wid, T)
    d["spec"] = spec
    return d


# (name, H, I, E, k, S, T, wt, zipf): several tiles per group, ragged tails, k = 1 and k = E.
SMALL = [
    ("f32_e16k2_t37", 256, 256, 16, 2, 0, 37, "f32", 0.0),
    ("bf16_e16k4s1_t150", 256, 256, 16, 4, 1, 150, "bf16", 0.0),
    ("bf16_e8k8s1_t20", 256, 512, 8, 8, 1, 20, "bf16", 0.0),
    ("bf16_e32k1_t5", 512, 256, 32, 1, 0, 5, "bf16", 0.0),
    ("bf16_e16k4s1_t1", 256, 256, 16, 4, 1, 1, "bf16", 0.0),
    ("i8_e32k8s1_t8", 512, 256, 32, 8, 1, 8, "i8", 0.0),
    ("i8_e32k8s1_t71", 512, 256, 32, 8, 1, 71, "i8", 0.0),
    # I = 512, T at and around the few-token routing limit (16)
    ("i8_e32k8s1_t13", 512, 512, 32, 8, 1, 13, "i8", 0.0),
    ("i8_e32k8s1_t16", 512, 512, 32, 8, 1, 16, "i8", 0.0),
    ("i8_e32k4s1_t17", 512, 512, 32, 4, 1, 17, "i8", 0.0),
    ("q4_e16k4s1_t100_zipf", 256, 256, 16, 4, 1, 100, "q4", 1.1),
    ("q4_e16k2s1_t9", 512, 256, 16, 2, 1, 9, "q4", 0.0),
    # the largest expert count and top-k the library takes (256 experts, top-16)
    ("bf16_e256k16s1_t40", 256, 256, 256, 16, 1, 40, "bf16", 0.0),
    # T >= 1024: groups of >= 128 rows go through the big-tile kernels (full 128-row
    # tiles, a partial big tile when >= 64 rows remain, small tiles for the rest)
    ("bf16_e8k2s1_t1200_big", 256, 256, 8, 2, 1, 1200, "bf16", 0.0),
    # the expert shape of the pages' model (H 2048, I 512): the bf16 big-tile ring's
    # main loop runs (16 super-stages of K for gate/up, 4 for down)
    ("bf16_e8k2s1_t1100_h2048_big", 2048, 512, 8, 2, 1, 1100, "bf16", 0.0),
    ("q4_e8k2s1_t1100_big", 256, 256, 8, 2, 1, 1100, "q4", 0.0),
    ("q4_e16k4s1_t1024_zipf_big", 256, 512, 16, 4, 1, 1024, "q4", 1.1),
    ("q4_e256k16_t1100_zipf_big", 256, 256, 256, 16, 0, 1100, "q4", 1.1),
    # hidden 512: down items of two 256-column blocks (calls of >= 1024 tokens)
    ("q4_e8k2s1_t1100_h512_big", 512, 256, 8, 2, 1, 1100, "q4", 0.0),
    # a prefill chunk of the 4-bit stack (T = 256, the pages' expert shape):
    # 4-bit calls of more than 16 tokens take the big-tile kernel, here mostly
    # with 16- and 32-row items (the shared expert in two 128-row tiles); and
    # both sides of that limit
    ("q4_e128k8s1_t256_h2048_chunk", 2048, 512, 128, 8, 1, 256, "q4", 0.0),
    ("q4_e32k4s1_t17_h2048", 2048, 512, 32, 4, 1, 17, "q4", 0.0),
    ("q4_e32k4s1_t16_h2048", 2048, 512, 32, 4, 1, 16, "q4", 0.0),
    ("q4_e128k8s1_t40_h2048_last_chunk", 2048, 512, 128, 8, 1, 40, "q4", 0.0),
    # MXFP4 weights x MXFP8 activations (scaled FP4 x FP8 MFMA): 16-pair gate/up
    # items (T <= 16, few-token routing), 32-row items with ragged tails, a
    # Zipf-skewed routing, and T >= 1024 (no big tiles for this format)
    ("mx4_e32k8s1_t9", 512, 512, 32, 8, 1, 9, "mx4", 0.0),
    ("mx4_e16k4s1_t37", 256, 256, 16, 4, 1, 37, "mx4", 0.0),
    ("mx4_e16k2s1_t200_zipf", 512, 256, 16, 2, 1, 200, "mx4", 1.1),
    ("mx4_e8k2s1_t1100", 256, 256, 8, 2, 1, 1100, "mx4", 0.0),
    # MX big tiles (hidden and inter multiples of 512 up to 2048): one and two
    # 16-byte scale chunks per row in the item's LDS copy, Zipf-skewed groups
    ("mx4_e8k2s1_t1100_h512_big", 512, 512, 8, 2, 1, 1100, "mx4", 0.0),
    ("mx4_e16k4s1_t1024_h1024_zipf_big", 1024, 1024, 16, 4, 1, 1024, "mx4", 1.1),
]


def check_route(g, d, ref):
    logits, ids, w = ref
    np.testing.assert_array_equal(g.logits(), logits, err_msg="router logits (fp64-accumulated, fp32-rounded)")
    np.testing.assert_array_equal(g.ids(), ids, err_msg="top-k ids")
    gw = g.gates()
    assert np.all(np.abs(gw - w) <= np.spacing(np.maximum(np.abs(w), np.float32(1e-30)))), "gates beyond 1 ulp"


def check_permute(g, ref_perm):
    offsets, row_token, token_row = ref_perm
    np.testing.assert_array_equal(g.offsets(), offsets)
    np.testing.assert_array_equal(g.row_token(), row_token)
    np.testing.assert_array_equal(g.token_row(), token_row)
    head, small, big = g.sched()
    # The tiles cover every group's rows exactly once: small tiles of <= 64 rows,
    # big tiles of 64..128 rows (only from T = 1024 on; 4-bit weights: T = 17),
    # big tiles first within a group.
    covered = np.zeros(offsets[-1], np.int32)
    for tiles, lo, hi in ((small, 1, 64), (big, 64, 128)):
        for grp, r0, n, _ in tiles:
            assert lo <= n <= hi and offsets[grp] <= r0 and r0 + n <= offsets[grp + 1]
            covered[r0:r0 + n] += 1
    assert np.all(covered == 1)
    T = g.T
    if T < (17 if g.spec.wt == "q4" else 1024):
        assert len(big) == 0


def run_steps(name, d):
    spec = d["spec"]
    T = d["x"].shape[0]
    say("case", name, "T", T, "wt", spec.wt)
    g = gh.GpuLayer(d)
    g.route()
    ref_route = oracle.route(d["x"], d["w_router"], spec.top_k, d.get("bias"))
    check_route(g, d, ref_route)
    g.permute()
    ref_perm = oracle.permute(ref_route[1], spec.n_routed, spec.n_shared)
    check_permute(g, ref_perm)
    offsets, row_token, token_row = ref_perm
    tol = gh.tol_for(spec)
    # gate/up + SwiGLU
    g.gate_up()
    if spec.wt == "i8":
        xq, xs = oracle.quantize_x(spec, d["x"])
        np.testing.assert_array_equal(gh.buf(g.layer, "x_q", np.int8, (T, spec.hidden)), xq)
        np.testing.assert_array_equal(gh.buf(g.layer, "x_scale", np.float32, (T,)), xs)
        h_ref = oracle.gate_up(None, offsets, row_token, spec.inter, "i8", d["w_gu"], d["w_gu_scale"], xq=xq, xs=xs)
        np.testing.assert_array_equal(g.h_raw(), h_ref.astype(np.float32), err_msg="int8 gate/up (exact fp32)")
    elif spec.wt == "mx4":
        xc, xsc, _ = oracle.quant_mx8(gh.bf16_to_f64(d["x"]).astype(np.float32))
        np.testing.assert_array_equal(gh.buf(g.layer, "x_q", np.uint8, (T, spec.hidden)), xc, err_msg="x E4M3 codes")
        np.testing.assert_array_equal(gh.buf(g.layer, "x_scale", np.uint8, (T, spec.hidden // 32)), xsc,
                                      err_msg="x E8M0 scales")
        h_ref = oracle.gate_up(d["x"], offsets, row_token, spec.inter, "mx4", d["w_gu"], d["w_gu_scale"])
        gh.assert_within(g.h(), h_ref, gh.mx_gu_bound(d, offsets, row_token), what="MX gate/up h")
    else:
        h_ref = oracle.gate_up(d["x"], offsets, row_token, spec.inter, spec.wt, d["w_gu"], d["w_gu_scale"],
                               d["w_gu_min"])
        gh.assert_close(g.h(), h_ref, what="gate/up h", **tol)
    # down, fed the oracle's h in the GPU's h format
    if gh.h_dtype(spec) == np.uint16:
        h_in_bits = gh.f64_to_bf16_bits(h_ref)
        h_in = gh.bf16_to_f64(h_in_bits)
        gh.put(g.layer, "h", h_in_bits)
    else:
        h_in = h_ref.astype(np.float32).astype(np.float64)
        gh.put(g.layer, "h", h_ref.astype(np.float32))
    g.down()
    y_ref = oracle.down(h_in, offsets, spec.hidden, spec.wt, d["w_down"], d["w_down_scale"], d["w_down_min"])
    if spec.wt == "i8":
        hq_ref, hs_ref = oracle.quant_rows_i8(h_ref.astype(np.float32))
        R = h_ref.shape[0]
        np.testing.assert_array_equal(gh.buf(g.layer, "h_q", np.int8, (R, spec.inter)), hq_ref, err_msg="h_q")
        np.testing.assert_array_equal(gh.buf(g.layer, "h_scale", np.float32, (R,)), hs_ref, err_msg="h_scale")
        np.testing.assert_array_equal(g.y_raw(), y_ref.astype(np.float32), err_msg="int8 down (exact)")
    elif spec.wt == "mx4":
        hc, hsc, _ = oracle.quant_mx8(h_ref.astype(np.float32))
        R = h_ref.shape[0]
        np.testing.assert_array_equal(gh.buf(g.layer, "h_q", np.uint8, (R, spec.inter)), hc, err_msg="h E4M3 codes")
        np.testing.assert_array_equal(gh.buf(g.layer, "h_scale", np.uint8, (R, spec.inter // 32)), hsc,
                                      err_msg="h E8M0 scales")
        gh.assert_within(g.y(), y_ref, gh.mx_down_bound(d, offsets, h_in, y_ref), what="MX down y")
    else:
        gh.assert_close(g.y(), y_ref, what="down y", **tol)
    # combine, fed the oracle's y in the GPU's y format
    if gh.h_dtype(spec) == np.uint16:
        y_bits = gh.f64_to_bf16_bits(y_ref)
        y_in = gh.bf16_to_f64(y_bits)
        gh.put(g.layer, "y", y_bits)
    else:
        y_in = y_ref.astype(np.float32).astype(np.float64)
        gh.put(g.layer, "y", y_ref.astype(np.float32))
    g.combine()
    gh.torch_mod().cuda.synchronize()
    out_ref = oracle.combine(y_in, token_row, ref_route[2])
    gh.assert_close(g.output(), out_ref, what="combine", **tol)
    return g


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_steps_small(case):
    name, H, I, E, k, S, T, wt, zipf = case
    run_steps(name, case_inputs(H, I, E, k, S, T, wt, zipf))


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_small(case):
    name, H, I, E, k, S, T, wt, zipf = case
    d = case_inputs(H, I, E, k, S, T, wt, zipf, seed=1)
    say("layer", name)
    g = gh.GpuLayer(d)
    g.run()
    ref = oracle.layer(d)
    gh.assert_close(g.output(), ref, what="layer " + name, **gh.tol_for(d["spec"]))


def test_layer_fp32_full():
    d = synth.layer_inputs("fp32_e16_top2", 16)
    say("layer fp32_e16_top2 T=16")
    run_steps("fp32_e16_top2", d)
    g = gh.GpuLayer(d)
    g.run()
    mr, rm = gh.assert_close(g.output(), oracle.layer(d), what="fp32 layer", **gh.TOL_F32)
    say("fp32 full: max_rel %.3g rmse %.3g" % (mr, rm))


def test_layer_bf16_prefill_full():
    d = synth.layer_inputs("bf16_e128_top8_shared", 256)
    say("layer bf16_e128_top8_shared T=256")
    run_steps("bf16_e128_top8_shared", d)
    g = gh.GpuLayer(d)
    g.run()
    mr, rm = gh.assert_close(g.output(), oracle.layer(d), what="bf16 layer", **gh.TOL_BF16)
    say("bf16 full: max_rel %.3g rmse %.3g" % (mr, rm))


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_layer_int8_decode_full(T):
    d = synth.layer_inputs("int8_e128_top8_shared", T, stream=T)
    say("layer int8_e128_top8_shared T=%d" % T)
    g = run_steps("int8_e128_top8_shared", d)
    g2 = gh.GpuLayer(d)
    g2.run()
    ref, st = oracle.layer(d, with_steps=True)
    # the int8 path's per-row outputs are exact; the bf16 layer output within the float bar
    np.testing.assert_array_equal(g2.y_raw(), st["y"].astype(np.float32))
    mr, rm = gh.assert_close(g2.output(), ref, what="int8 layer", **gh.TOL_BF16)
    say("int8 T=%d: max_rel %.3g rmse %.3g" % (T, mr, rm))


def test_layer_q4_zipf_prefill_full():
    """T = 2048 with Zipf-skewed routing, every token: routing, permutation,
    every h row, every y row (fed the oracle's h), the combine (fed the
    oracle's y), then the whole layer end to end."""
    d = synth.layer_inputs("q4_e128_top8_shared_zipf", 2048)
    spec = d["spec"]
    say("layer q4_e128_top8_shared_zipf T=2048 (steps)")
    g = run_steps("q4_e128_top8_shared_zipf", d)
    counts = np.diff(g.offsets())
    assert counts[:spec.n_routed].max() > 64 * 8, "Zipf bias should give one expert many tiles"
    head, small, big = g.sched()
    assert len(big) > 0 and len(small) > 0
    say("layer q4_e128_top8_shared_zipf T=2048 (end to end)")
    g2 = gh.GpuLayer(d)
    g2.run()
    mr, rm = gh.assert_close(g2.output(), oracle.layer(d), what="q4 layer (all 2048 tokens)", **gh.TOL_BF16)
    say("q4 T=2048 full: max_rel %.3g rmse %.3g" % (mr, rm))


def test_zero_tokens_is_a_noop():
    d = case_inputs(256, 256, 16, 4, 1, 4, "bf16")
    g = gh.GpuLayer(d)
    g.run()
    before = g.output().copy()
    g.T = 0
    g.route()
    g.permute()
    g.gate_up()
    g.down()
    g.combine()
    gh.torch_mod().cuda.synchronize()
    g.T = 4
    np.testing.assert_array_equal(g.output(), before)


def test_deterministic_and_chunk_invariant():
    """Same bits on a re-run, and a token's output does not depend on which
    other tokens share the call (tiles differ, K order does not)."""
    d = case_inputs(256, 256, 16, 4, 1, 90, "bf16", seed=3)
    g = gh.GpuLayer(d)
    g.run()
    a = g.output().copy()
    g.run()
    np.testing.assert_array_equal(g.output(), a)
    part = dict(d)
    part["x"] = np.ascontiguousarray(d["x"][30:41])
    g2 = gh.GpuLayer(part)
    g2.run()
    np.testing.assert_array_equal(g2.output(), a[30:41])


# moe_route_permute: two launches for T <= 16 (H-sliced fp64 partial logits,
# then one block for top-k, permutation and int8 quantisation), the two
# separate calls above that.  Same results bit for bit as moe_route_topk +
# moe_permute, and the oracle's routing and permutation.
FUSED_ROUTE = [
    ("bf16_e128k8s1_t1", 2048, 512, 128, 8, 1, 1, "bf16", 0.0),
    ("bf16_e128k8s1_t2", 2048, 512, 128, 8, 1, 2, "bf16", 0.0),
    ("bf16_e128k8s1_t5", 2048, 512, 128, 8, 1, 5, "bf16", 0.0),
    ("bf16_e128k8s1_t16", 2048, 512, 128, 8, 1, 16, "bf16", 0.0),
    ("bf16_e128k8s1_t17_unfused", 2048, 512, 128, 8, 1, 17, "bf16", 0.0),
    ("i8_e128k8s1_t1", 2048, 512, 128, 8, 1, 1, "i8", 0.0),
    ("i8_e128k8s1_t8", 2048, 512, 128, 8, 1, 8, "i8", 0.0),
    ("f32_e16k2_t16", 2048, 512, 16, 2, 0, 16, "f32", 0.0),
    ("q4_e16k4s1_t4_zipf", 512, 256, 16, 4, 1, 4, "q4", 1.1),
    ("bf16_e8k8s1_t3_h256", 256, 256, 8, 8, 1, 3, "bf16", 0.0),
    ("bf16_e256k16_t16", 1024, 256, 256, 16, 0, 16, "bf16", 0.0),
    ("mx4_e128k8s1_t5", 2048, 512, 128, 8, 1, 5, "mx4", 0.0),
    # one token without a shared expert: k = 16 of 256, and k = E
    ("bf16_e256k16_t1", 1024, 256, 256, 16, 0, 1, "bf16", 0.0),
    ("bf16_e8k8_t1", 256, 256, 8, 8, 0, 1, "bf16", 0.0),
    # an expert count that is not a multiple of 64 (padding keys in the rounds
    # of maxima): one wave per token in the fused block (T = 9), and T > 16
    ("bf16_e100k6s1_t9", 256, 256, 100, 6, 1, 9, "bf16", 0.0),
    ("bf16_e100k6s1_t40", 256, 256, 100, 6, 1, 40, "bf16", 0.0),
    # 32 x 32 router blocks over 256 experts (eight expert blocks)
    ("bf16_e256k16_t1024", 512, 256, 256, 16, 0, 1024, "bf16", 0.0),
    # the largest T whose bitmap fits the permutation's LDS for 128 experts
    # (its rows keep the even word stride) and two batches of id loads
    ("bf16_e128k8s1_t2560_lds_edge", 512, 256, 128, 8, 1, 2560, "bf16", 0.0),
]

ROUTE_PERMUTE_BUFFERS = ("topk_ids", "topk_w", "expert_offsets", "row_token", "token_row", "sched", "x_q", "x_scale")


@pytest.mark.parametrize("case", FUSED_ROUTE, ids=[c[0] for c in FUSED_ROUTE])
def test_route_permute_matches_separate_calls(case):
    torch = gh.torch_mod()
    name, H, I, E, k, S, T, wt, zipf = case
    d = case_inputs(H, I, E, k, S, T, wt, zipf, seed=11)
    spec = d["spec"]
    say("case", name, "T", T)
    g = gh.GpuLayer(d)
    g.route()
    g.permute()
    torch.cuda.synchronize()
    ref = {n: g.layer.tensors[n].clone() for n in ROUTE_PERMUTE_BUFFERS if g.layer.tensors.get(n) is not None}
    for n in list(ref) + ["logits"]:
        g.layer.tensors[n].fill_(0x5a)
    g.route_permute()
    torch.cuda.synchronize()
    # routing against the oracle (logits bit for bit, ids, gates within an ulp)
    ref_route = oracle.route(d["x"], d["w_router"], spec.top_k, d.get("bias"))
    check_route(g, d, ref_route)
    check_permute(g, oracle.permute(ref_route[1], spec.n_routed, spec.n_shared))
    # every other buffer the two calls write, bit for bit (only the bytes the calls define)
    nbytes = dict(topk_ids=T * k * 4, topk_w=T * k * 4, expert_offsets=(E + S + 1) * 4, row_token=T * (k + S) * 4,
                  token_row=T * (k + S) * 4, x_q=T * H, x_scale=T * (H // 32 if wt == "mx4" else 4))
    head, small, big = g.sched()
    nbytes["sched"] = (32 + 4 * len(small)) * 4
    for n, t in ref.items():
        a = t.view(torch.uint8)[:nbytes[n]].cpu().numpy()
        b = g.layer.tensors[n].view(torch.uint8)[:nbytes[n]].cpu().numpy()
        np.testing.assert_array_equal(b, a, err_msg="%s: fused differs from moe_route_topk + moe_permute" % n)
    if wt == "i8":
        xq, xs = oracle.quantize_x(spec, d["x"])
        np.testing.assert_array_equal(gh.buf(g.layer, "x_q", np.int8, (T, H)), xq)
        np.testing.assert_array_equal(gh.buf(g.layer, "x_scale", np.float32, (T,)), xs)
    if wt == "mx4":
        xc, xsc, _ = oracle.quant_mx8(gh.bf16_to_f64(d["x"]).astype(np.float32))
        np.testing.assert_array_equal(gh.buf(g.layer, "x_q", np.uint8, (T, H)), xc)
        np.testing.assert_array_equal(gh.buf(g.layer, "x_scale", np.uint8, (T, H // 32)), xsc)


# Planted ties: router rows 5 and 9 copy row 2, so those three experts get
# equal logits for every token (the top-k must order them 2, 5, 9 wherever
# they rank), and token 0 is all zeros (every logit is +0: experts 0 .. k-1,
# equal gates).  T = 40 takes the two-block split of H (moe_route_topk), T = 12
# the few-token block (moe_route_permute).
@pytest.mark.parametrize("T, fused", [(40, False), (12, True)], ids=["split_t40", "fused_t12"])
def test_route_ties_and_zero_token(T, fused):
    d = case_inputs(512, 256, 16, 4, 1, T, "bf16", seed=9)
    wr = d["w_router"].copy()
    wr[5] = wr[2]
    wr[9] = wr[2]
    d["w_router"] = wr
    x = d["x"].copy()
    x[0] = 0
    d["x"] = x
    say("ties T", T, "fused", fused)
    g = gh.GpuLayer(d)
    if fused:
        g.route_permute()
    else:
        g.route()
    ref = oracle.route(d["x"], d["w_router"], 4, None)
    check_route(g, d, ref)
    ids = g.ids()
    np.testing.assert_array_equal(ids[0], [0, 1, 2, 3])
    for t in range(T):
        tied = [e for e in ids[t] if e in (2, 5, 9)]
        assert tied == sorted(tied), (t, ids[t])


# Whole logits in 32 x 32 blocks (calls with at least 256 such blocks and H a
# multiple of 512): fp32 activations (32 experts, T = 8200) and bf16 with a
# Zipf router bias (128 experts, T = 2047); both T leave a ragged last block.
@pytest.mark.parametrize("E, k, T, wt, zipf", [(32, 4, 8200, "f32", 0.0), (128, 8, 2047, "bf16", 1.1)],
                         ids=["f32_e32_t8200", "bf16_e128_t2047_bias"])
def test_route_whole_logits_32x32(E, k, T, wt, zipf):
    d = case_inputs(512, 256, E, k, 0, T, wt, zipf, seed=13)
    say("route 32x32 E", E, "T", T, wt)
    g = gh.GpuLayer(d)
    g.route()
    check_route(g, d, oracle.route(d["x"], d["w_router"], k, d.get("bias")))


def test_layer_mx4_zipf_prefill_full():
    """MXFP4 weights x MXFP8 activations at T = 2048 with Zipf-skewed routing,
    every token: the x and h codes bit for bit, every h and y row, then the
    whole layer end to end."""
    d = synth.layer_inputs("mx4_e128_top8_shared_zipf", 2048)
    say("layer mx4_e128_top8_shared_zipf T=2048 (steps)")
    run_steps("mx4_e128_top8_shared_zipf", d)
    say("layer mx4_e128_top8_shared_zipf T=2048 (end to end)")
    g2 = gh.GpuLayer(d)
    g2.run()
    mr, rm = gh.assert_close(g2.output(), oracle.layer(d), what="mx4 layer (all 2048 tokens)", **gh.TOL_BF16)
    say("mx4 T=2048: max_rel %.3g rmse %.3g" % (mr, rm))


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_layer_mx4_decode_full(T):
    d = synth.layer_inputs("mx4_e128_top8_shared", T, stream=T)
    say("layer mx4_e128_top8_shared T=%d" % T)
    run_steps("mx4_e128_top8_shared", d)
    g2 = gh.GpuLayer(d)
    g2.run()
    mr, rm = gh.assert_close(g2.output(), oracle.layer(d), what="mx4 layer", **gh.TOL_BF16)
    say("mx4 T=%d: max_rel %.3g rmse %.3g" % (T, mr, rm))
