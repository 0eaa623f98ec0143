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
