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


def test_static_variant_across_layouts():
    """Calls with descs of different buffer layouts in a row (int8, 4-bit,
    bf16, then int8 again) share the static array: each must still give the
    buffered call's bits (the barrier words do not move with the layout)."""
    torch = gh.torch_mod()
    from mixture_experts_expert_moe_amd import moe
    H = 2048
    layers = {}
    for wt in ("i8", "q4", "bf16"):
        spec = LayerSpec(hidden=H, inter=512, n_routed=128, top_k=8, n_shared=1, act="bf16", wt=wt, out="bf16")
        w = gh.dev_weights(synth.layer_weights(spec, 960))
        layers[wt] = (spec, w, moe.MoeLayer(gh.desc_for(spec, 16), w))
    for wt, T in (("i8", 9), ("q4", 12), ("bf16", 5), ("i8", 16)):
        spec, w, layer = layers[wt]
        say("static decode across layouts", wt, "T", T)
        x = gh.to_dev(synth.tokens(spec, 961, T, stream=T))
        ref = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_layer(layer.desc, T, x, w["w_router"], w.get("bias"), layer.gu, layer.dn, None, 0, 1e-6,
                             ref, layer.bufs)
        moe.moe_decode_layer_static(layer.desc, T, x, w["w_router"], w.get("bias"), layer.gu, layer.dn, None, 0,
                                    1e-6, got)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().view(torch.int16).numpy(), ref.cpu().view(torch.int16).numpy(),
                                      err_msg="static variant differs, %s T=%d" % (wt, T))
        assert moe.sync_status(layer.tensors) == 0
