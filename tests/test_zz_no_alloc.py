"""moe_decode_layer_static (no allocation, layer buffers in the library's
static device array) against moe_decode_layer with caller-owned buffers:
the same output bits, on two calls in a row, the second with fewer tokens."""
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


@pytest.mark.parametrize("wt,norm", [("i8", False), ("q4", True), ("bf16", False), ("mx4", True)])
def test_static_variant_equals_buffered_call(wt, norm):
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    H = 2048
    spec = LayerSpec(hidden=H, inter=512, n_routed=128, top_k=8, n_shared=1, act="bf16", wt=wt,
                     out="f32" if norm else "bf16")
    w = gh.dev_weights(synth.layer_weights(spec, 950))
    layer = moe.MoeLayer(gh.desc_for(spec, 16), w)
    odt = torch.float32 if norm else torch.bfloat16
    for T in (12, 3):   # the second call has fewer tokens than the first
        say("static decode", wt, "norm" if norm else "plain", "T", T)
        if norm:
            x = torch.from_numpy(synth.tokens(spec, 951, T, stream=T, dtype="f32")).to("cuda")
            flags = moe.MOE_DECODE_NORM_INPUT
        else:
            x = gh.to_dev(synth.tokens(spec, 951, T, stream=T))
            flags = 0
        ref = torch.full((T, H), float("nan"), dtype=odt, device="cuda")
        got = torch.full((T, H), float("nan"), dtype=odt, device="cuda")
        moe.moe_decode_layer(layer.desc, T, x, w["w_router"], w.get("bias"), layer.gu, layer.dn, None, flags, 1e-6,
                             ref, layer.bufs)
        moe.moe_decode_layer_static(layer.desc, T, x, w["w_router"], w.get("bias"), layer.gu, layer.dn, None, flags,
                                    1e-6, got)
        torch.cuda.synchronize()
        a = ref.cpu().view(torch.int16 if odt == torch.bfloat16 else torch.int32).numpy()
        b = got.cpu().view(torch.int16 if odt == torch.bfloat16 else torch.int32).numpy()
        np.testing.assert_array_equal(b, a, err_msg="static variant differs, T=%d" % T)
        assert moe.sync_status(layer.tensors) == 0
