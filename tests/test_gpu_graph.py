"""A captured HIP graph of stacked layers replays to the same bits as eager
execution, across several replays with eager work and synchronisation in
between (the library records only kernel launches, no memsets)."""
import numpy as np
import pytest

from gen import synth
from gen.synth import LayerSpec
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wt,T", [("q4", 1), ("bf16", 5), ("i8", 3)])
def test_graph_replay_matches_eager(wt, T):
    import torch
    from mixture_experts_expert_moe_amd import moe
    spec = LayerSpec(hidden=256, inter=256, n_routed=16, top_k=4, n_shared=1, wt=wt, out="f32")
    layers = [gh.dev_weights(synth.layer_weights(spec, 900, l)) for l in range(3)]
    st = moe.MoeStack(gh.desc_for(spec, 8), layers)
    inputs = [torch.from_numpy(synth.tokens(spec, 900, T, stream=s, dtype="f32")).to("cuda") for s in range(4)]
    eager = []
    for x in inputs:
        y = x.clone()
        st.forward(y)
        eager.append(y.cpu().numpy())
    torch.cuda.synchronize()
    buf = torch.empty_like(inputs[0])
    buf.copy_(inputs[0])
    st.forward(buf)                     # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.forward(buf)
    for rep in range(3):
        for i, x in enumerate(inputs):
            buf.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(buf.cpu().numpy(), eager[i], err_msg="replay %d input %d" % (rep, i))
            z = x.clone()                  # eager work between replays
            st.forward(z)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(z.cpu().numpy(), eager[i])
