"""moe_decode_layer: the whole layer for a few tokens in one launch.

It must write, bit for bit, what the separate calls write (routing,
permutation, tile schedule, int8 or MXFP8 codes, h, y and the output, also
with the RMSNorm of the residual stream in front), match the oracle (routing
exactly, outputs within the float bar, the int8 path exactly), leave the
barrier status word clear, and give the same bits when called many times in
a row and when replayed from a graph."""
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


# (name, H, I, E, k, S, T, wt)
CASES = [
    ("i8_e128k8s1_t1", 2048, 512, 128, 8, 1, 1, "i8"),
    ("i8_e128k8s1_t2", 2048, 512, 128, 8, 1, 2, "i8"),
    ("i8_e128k8s1_t4", 2048, 512, 128, 8, 1, 4, "i8"),
    ("i8_e128k8s1_t8", 2048, 512, 128, 8, 1, 8, "i8"),
    ("i8_e128k8s1_t16", 2048, 512, 128, 8, 1, 16, "i8"),
    ("q4_e128k8s1_t1", 2048, 512, 128, 8, 1, 1, "q4"),
    ("q4_e128k8s1_t5", 2048, 512, 128, 8, 1, 5, "q4"),
    ("bf16_e128k8s1_t3", 2048, 512, 128, 8, 1, 3, "bf16"),
    ("bf16_e16k4s1_t13_h512", 512, 256, 16, 4, 1, 13, "bf16"),
    ("i8_e32k8_t7_noshared", 1024, 256, 32, 8, 0, 7, "i8"),
    ("q4_e256k16s1_t16_h1024", 1024, 512, 256, 16, 1, 16, "q4"),
    ("bf16_e8k8s1_t9_h256", 256, 256, 8, 8, 1, 9, "bf16"),
    ("mx4_e128k8s1_t1", 2048, 512, 128, 8, 1, 1, "mx4"),
    ("mx4_e128k8s1_t8", 2048, 512, 128, 8, 1, 8, "mx4"),
    ("mx4_e32k8_t11_noshared_i256", 1024, 256, 32, 8, 0, 11, "mx4"),
]

BUFS = ("logits", "topk_ids", "topk_w", "expert_offsets", "row_token", "token_row", "x_q", "x_scale", "h", "y",
        "h_q", "h_scale")


def case_inputs(H, I, E, k, S, T, wt, seed):
    spec = LayerSpec(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=S, act="bf16", wt=wt, out="f32")
    d = synth.layer_weights(spec, 7000 + seed)
    d["x"] = synth.tokens(spec, 7000 + seed, T)
    d["spec"] = spec
    return d


def nbytes(spec, T):
    R = T * (spec.top_k + spec.n_shared)
    f = 4 if spec.wt in ("i8", "mx4") else 2
    mx = spec.wt == "mx4"
    return dict(logits=T * spec.n_routed * 4, topk_ids=T * spec.top_k * 4, topk_w=T * spec.top_k * 4,
                expert_offsets=(spec.groups + 1) * 4, row_token=R * 4, token_row=R * 4, x_q=T * spec.hidden,
                x_scale=T * spec.hidden // 32 if mx else T * 4, h=R * spec.inter * f, y=R * spec.hidden * f,
                h_q=R * spec.inter, h_scale=R * spec.inter // 32 if mx else R * 4)


def snapshot(g, spec, T):
    torch = gh.torch_mod()
    out = {}
    n = nbytes(spec, T)
    for name in BUFS:
        t = g.layer.tensors.get(name)
        if t is not None:
            out[name] = t.view(torch.uint8)[:n[name]].cpu().numpy().copy()
    head, small, big = g.sched()
    out["sched"] = np.concatenate([head, small.reshape(-1)])
    return out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_layer_equals_separate_calls_and_oracle(case):
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    name, H, I, E, k, S, T, wt = case
    d = case_inputs(H, I, E, k, S, T, wt, seed=hash(name) % 1000)
    spec = d["spec"]
    say("decode layer", name)
    g = gh.GpuLayer(d, max_tokens=16)
    res = torch.from_numpy(synth.tokens(spec, 77, T, stream=9, dtype="f32")).to("cuda")
    # separate calls: routing + permutation, gate/up, down, combine with the residual
    out_ref = torch.empty((T, H), dtype=torch.float32, device="cuda")
    g.route_permute()
    g.gate_up()
    g.down()
    moe.moe_combine(g.desc, T, res, out_ref, g.layer.bufs)
    torch.cuda.synchronize()
    ref = snapshot(g, spec, T)
    for n in BUFS + ("sched",):
        t = g.layer.tensors.get(n)
        if t is not None:
            t.fill_(0x5a)
    # one launch
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    g.layer.forward_decode(g.x, out, residual=res)
    torch.cuda.synchronize()
    assert moe.sync_status(g.layer.tensors) == 0, "a grid barrier timed out"
    got = snapshot(g, spec, T)
    # routing against the oracle (logits bit for bit, ids, gates within an ulp)
    ref_route = oracle.route(d["x"], d["w_router"], spec.top_k, d.get("bias"))
    np.testing.assert_array_equal(got["logits"].view(np.float32).reshape(T, E), ref_route[0])
    np.testing.assert_array_equal(got["topk_ids"].view(np.int32).reshape(T, k), ref_route[1])
    for n in BUFS + ("sched",):
        if n in ref and n != "logits":
            np.testing.assert_array_equal(got[n], ref[n], err_msg="%s: one launch differs from the separate calls" % n)
    np.testing.assert_array_equal(out.cpu().numpy(), out_ref.cpu().numpy(), err_msg="layer output")
    # the layer against the oracle
    want = oracle.layer(d, residual=synth.tokens(spec, 77, T, stream=9, dtype="f32"))
    mr, rm = gh.assert_close(out.cpu().numpy(), want, what="decode layer vs oracle", **gh.TOL_BF16)
    if wt == "i8":
        _, st = oracle.layer(d, with_steps=True)
        np.testing.assert_array_equal(got["h"].view(np.float32).reshape(-1, I), st["h"].astype(np.float32))
    say("  ok: max_rel %.3g rmse %.3g" % (mr, rm))


@pytest.mark.parametrize("wt,T", [("q4", 1), ("i8", 8), ("bf16", 3), ("q4", 16), ("mx4", 4)])
def test_decode_layer_norm_input_and_repeats(wt, T):
    """With the RMSNorm of the fp32 residual stream inside (one stacked layer):
    the same bits as moe_rmsnorm + the separate calls with the residual, in
    every buffer; 60 calls in a row (the barrier counters keep growing) give
    the same bits every time."""
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    H = 2048
    d = case_inputs(H, 512, 128, 8, 1, T, wt, seed=31)
    spec = d["spec"]
    say("decode norm-input + repeats", wt, T)
    g = gh.GpuLayer(d, max_tokens=16)
    x = torch.from_numpy(synth.tokens(spec, 78, T, stream=3, dtype="f32")).to("cuda")
    xn = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    out_ref = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_rmsnorm(T, H, 1e-6, x, xn)
    g.x = xn
    g.route_permute()
    g.gate_up()
    g.down()
    moe.moe_combine(g.desc, T, x, out_ref, g.layer.bufs)
    torch.cuda.synchronize()
    ref = snapshot(g, spec, T)
    want = out_ref.cpu().numpy()
    out = torch.empty_like(out_ref)
    for rep in range(60):
        out.fill_(float("nan"))
        g.layer.forward_decode(x, out, norm_input=True, eps=1e-6)
        if rep % 20 == 19:
            torch.cuda.synchronize()
            np.testing.assert_array_equal(out.cpu().numpy(), want, err_msg="repeat %d" % rep)
    got = snapshot(g, spec, T)
    for n in BUFS + ("sched",):
        if n in ref and n != "logits":
            np.testing.assert_array_equal(got[n], ref[n], err_msg="%s: one launch differs from the separate calls" % n)
    assert moe.sync_status(g.layer.tensors) == 0


def test_decode_stack_in_place_equals_forward():
    """MoeStack.forward_decode (one launch per layer, the residual stream
    updated in place) equals MoeStack.forward bit for bit."""
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    spec = LayerSpec(hidden=512, inter=256, n_routed=16, top_k=4, n_shared=1, wt="q4", out="f32")
    layers = [gh.dev_weights(synth.layer_weights(spec, 930, l)) for l in range(4)]
    st = moe.MoeStack(gh.desc_for(spec, 8), layers, eps=1e-6)
    for T in (1, 6):
        say("stack decode T", T)
        x = torch.from_numpy(synth.tokens(spec, 930, T, stream=4, dtype="f32")).to("cuda")
        a = x.clone()
        st.forward(a)
        b = x.clone()
        st.forward_decode(b)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(b.cpu().numpy(), a.cpu().numpy())
    assert moe.sync_status(st.tensors) == 0


def test_decode_layer_graph_replay():
    """One decode step of a 3-layer stack captured as a graph replays to the eager bits."""
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    spec = LayerSpec(hidden=2048, inter=512, n_routed=128, top_k=8, n_shared=1, wt="q4", out="f32")
    layers = [gh.dev_weights(synth.layer_weights(spec, 940, l)) for l in range(3)]
    st = moe.MoeStack(gh.desc_for(spec, 1), layers, eps=1e-6)
    inputs = [torch.from_numpy(synth.tokens(spec, 940, 1, stream=s, dtype="f32")).to("cuda") for s in range(3)]
    eager = []
    for x in inputs:
        y = x.clone()
        st.forward_decode(y)
        eager.append(y.cpu().numpy())
    buf = inputs[0].clone()
    st.forward_decode(buf)
    torch.cuda.synchronize()
    say("capture decode step")
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        st.forward_decode(buf)
    for rep in range(3):
        for i, x in enumerate(inputs):
            buf.copy_(x)
            gr.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(buf.cpu().numpy(), eager[i], err_msg="replay %d input %d" % (rep, i))
            z = x.clone()
            st.forward_decode(z)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(z.cpu().numpy(), eager[i])
    assert moe.sync_status(st.tensors) == 0
