"""moe_combine_rmsnorm: the combine of layer l fused with the RMSNorm of layer
l + 1's input.  It must write the same bits as moe_combine followed by
moe_rmsnorm, so a stack run through MoeStack.forward (fused) equals one run
layer by layer through MoeStack.layer (separate RMSNorm launches) exactly."""
import sys

import numpy as np
import pytest

from gen import synth
from gen.synth import LayerSpec
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# (weights, hidden, inter, T): hidden 2304 and 8192 give threads two and four
# chunks of the row; T spans one decode token, a ragged chunk and a full one.
CASES = [
    ("q4", 512, 256, 1),
    ("q4", 512, 256, 37),
    ("bf16", 512, 256, 256),
    ("i8", 512, 256, 9),
    ("bf16", 2304, 256, 5),
    ("bf16", 8192, 256, 3),
]


@pytest.mark.parametrize("wt,H,I,T", CASES, ids=["%s_h%d_t%d" % (c[0], c[1], c[3]) for c in CASES])
def test_forward_fused_equals_layer_by_layer(wt, H, I, T):
    import torch
    from mixture_experts_expert_moe_amd import moe
    say("fused combine+rmsnorm: wt=%s H=%d I=%d T=%d" % (wt, H, I, T))
    spec = LayerSpec(hidden=H, inter=I, n_routed=16, top_k=4, n_shared=1, wt=wt, out="f32")
    layers = [gh.dev_weights(synth.layer_weights(spec, 910, l)) for l in range(3)]
    st = moe.MoeStack(gh.desc_for(spec, 256), layers, eps=1e-6)
    x = torch.from_numpy(synth.tokens(spec, 910, T, stream=2, dtype="f32")).to("cuda")
    # layer by layer, separate RMSNorm launches
    a, b = x.clone(), torch.empty_like(x)
    xns = []
    for l in range(3):
        st.layer(l, a, b, T)
        torch.cuda.synchronize()
        xns.append(st.xn[:T].cpu().clone())
        a, b = b, a
    ref = a.cpu().numpy()
    # fused
    y = x.clone()
    st.forward(y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)
    # the fused call on its own: out as moe_combine, xn as moe_rmsnorm of that out
    d, bf = st.desc, st.bufs
    res = x.clone()
    out1, out2 = torch.empty_like(x), torch.empty_like(x)
    xn1 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    xn2 = torch.empty_like(xn1)
    moe.moe_combine_rmsnorm(d, T, res, 1e-6, out1, xn1, bf)   # buffers still hold the last layer's rows
    moe.moe_combine(d, T, res, out2, bf)
    moe.moe_rmsnorm(T, H, 1e-6, out2, xn2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out1.cpu().numpy(), out2.cpu().numpy())
    np.testing.assert_array_equal(xn1.cpu().view(torch.int16).numpy(), xn2.cpu().view(torch.int16).numpy())
    assert np.isfinite(ref).all()


# The residual branch of the combine against the oracle: y fed from the oracle
# (in the GPU's y format), residual fp32, output fp32; the fused RMSNorm output
# within one bf16 ulp of the oracle's fp64 RMSNorm of the oracle's sum.
RESIDUAL_CASES = [("bf16", 2048, 512, 128, 8, 1, 7), ("i8", 512, 256, 32, 8, 1, 3), ("q4", 512, 256, 16, 4, 1, 40),
                  ("f32", 256, 256, 16, 2, 0, 16)]


@pytest.mark.parametrize("wt,H,I,E,k,S,T", RESIDUAL_CASES, ids=["%s_t%d" % (c[0], c[6]) for c in RESIDUAL_CASES])
def test_combine_residual_matches_oracle(wt, H, I, E, k, S, T):
    import torch
    from mixture_experts_expert_moe_amd import moe
    from oracle import oracle
    say("combine + residual vs oracle: wt=%s H=%d T=%d" % (wt, H, T))
    act = "f32" if wt == "f32" else "bf16"
    spec = LayerSpec(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=S, act=act, wt=wt, out="f32")
    d = synth.layer_weights(spec, 920)
    d["x"] = synth.tokens(spec, 920, T)
    d["spec"] = spec
    res = synth.tokens(spec, 920, T, stream=3, dtype="f32")
    g = gh.GpuLayer(d)
    g.route()
    g.permute()
    g.gate_up()
    g.down()
    torch.cuda.synchronize()
    # the oracle's rows in the GPU's y format, and the routing the GPU took (checked equal to the oracle's)
    _, st = oracle.layer(d, with_steps=True)
    np.testing.assert_array_equal(g.token_row(), st["token_row"])
    np.testing.assert_array_equal(g.ids(), st["ids"])
    if gh.h_dtype(spec) == np.uint16:
        y_bits = gh.f64_to_bf16_bits(st["y"])
        y_in = gh.bf16_to_f64(y_bits)
        gh.put(g.layer, "y", y_bits)
    else:
        y_in = st["y"].astype(np.float32).astype(np.float64)
        gh.put(g.layer, "y", st["y"].astype(np.float32))
    gates = g.gates()
    ref = oracle.combine(y_in, st["token_row"], gates, residual=res)
    rd = torch.from_numpy(res).to("cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_combine(g.desc, T, rd, out, g.layer.bufs)
    out2 = torch.empty_like(out)
    xn = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_rmsnorm(g.desc, T, rd, 1e-6, out2, xn, g.layer.bufs)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gh.assert_close(got, ref, what="combine with residual", **gh.TOL_F32)
    np.testing.assert_array_equal(out2.cpu().numpy(), got)
    xn_ref = gh.f64_to_bf16_bits(oracle.rmsnorm(got, 1e-6)).astype(np.int32)
    xn_got = xn.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.int32)
    assert np.abs(xn_got - xn_ref).max() <= 1, "fused RMSNorm beyond one bf16 ulp of the oracle"
