"""MXFP8 block quantisation on the GPU (E4M3 elements, one E8M0 scale byte
per 32 values), the step in front of the scaled FP4 x FP8 MFMA: x (bf16)
inside moe_permute, h (fp32) inside moe_grouped_gemm_down, and any fp32 or
bf16 rows through moe_quant_mx8 (the same kernel).  Codes and scale
bytes must equal the oracle's bit for bit, on rows built to hit the
conversion's edge cases: all-zero blocks, ties between neighbouring E4M3
values (to the even mantissa), block maxima whose scaled value lies above 448
(saturated), values under half the smallest subnormal (zero) or exactly at it
(tie to zero), negative zero, fp32 subnormals and the clamp of the scale byte
at 0."""
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


def edge_blocks(rng, f32: bool) -> np.ndarray:
    """Blocks of 32 values (float32) covering the conversion's edge cases."""
    s8 = 2.0 ** -8  # the scale of a block whose max is in [1, 2)
    blocks = []
    blocks.append(np.zeros(32))                                        # all zero: byte 0, codes 0
    b = np.full(32, 0.25)
    b[0] = 1.0                                                         # amax 1 -> byte 119
    b[1:9] = np.array([17, 19, 21, 23, 25, 27, 29, 31]) * s8 * 0.5     # ties 8.5, 9.5, ...: to even mantissa
    b[9:13] = np.array([2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]) * s8  # at/under the subnormal tie
    b[13:17] = np.array([0.5, 1.5, 2.5, 3.5]) * 2.0 ** -9 * s8        # ties between subnormals
    b[17] = -0.0
    b[18:26] = -b[1:9]
    blocks.append(b)
    b = rng.standard_normal(32) * 0.1
    b[5] = 1.9375                                                      # scaled 496 > 448: saturates
    b[6] = -1.96875
    blocks.append(b)
    b = rng.standard_normal(32)
    b[0] = 448.0 * 2.0 ** 3                                            # exactly at the top of the grid
    blocks.append(b)
    b = rng.standard_normal(32) * 2.0 ** -30                           # small block
    blocks.append(b)
    b = rng.standard_normal(32) * 2.0 ** 40                            # large block
    blocks.append(b)
    if f32:
        b = np.zeros(32)
        b[0] = 1.5 * 2.0 ** -126                                       # byte clamps at 0 (scale 2^-127)
        b[1:8] = np.array([2.0 ** -130, 2.0 ** -135, 3 * 2.0 ** -140, 2.0 ** -149, -2.0 ** -131, 2.0 ** -127,
                           1.25 * 2.0 ** -128])                       # fp32 subnormals
        blocks.append(b)
        b = rng.standard_normal(32) * 2.0 ** -120                      # byte near the bottom
        blocks.append(b)
    return np.stack(blocks).astype(np.float32)


def rows_of(blocks: np.ndarray, cols: int, rows: int, rng) -> np.ndarray:
    """rows x cols float32: the edge blocks first, the rest N(0, 1), shuffled by block."""
    n = rows * cols // 32
    out = rng.standard_normal((n, 32)).astype(np.float32)
    idx = rng.permutation(n)[:len(blocks)]
    out[idx] = blocks
    return out.reshape(rows, cols)


def bf16_bits_rne(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits (the oracle's rounding); every edge value above is exact in bf16."""
    return gh.f64_to_bf16_bits(v.astype(np.float64))


def test_mx8_of_x_edge_cases():
    """x (bf16) quantised by moe_permute (and by the few-token moe_route_permute)."""
    rng = np.random.default_rng(2024)
    H, T = 512, 12
    spec = LayerSpec(hidden=H, inter=256, n_routed=16, top_k=4, n_shared=1, act="bf16", wt="mx4", out="f32")
    d = synth.layer_weights(spec, 8100)
    xf = rows_of(edge_blocks(rng, f32=False), H, T, rng)
    d["x"] = bf16_bits_rne(xf)
    d["spec"] = spec
    xv = gh.bf16_to_f64(d["x"]).astype(np.float32)  # the planted ties have <= 5 significant bits: exact in bf16
    want_c, want_s, _ = oracle.quant_mx8(xv)
    for fused in (False, True):
        say("x edge cases, fused route+permute", fused)
        g = gh.GpuLayer(d)
        for name in ("x_q", "x_scale"):
            g.layer.tensors[name].fill_(0x5a)
        if fused:
            g.route_permute()
        else:
            g.route()
            g.permute()
        gh.torch_mod().cuda.synchronize()
        np.testing.assert_array_equal(gh.buf(g.layer, "x_q", np.uint8, (T, H)), want_c)
        np.testing.assert_array_equal(gh.buf(g.layer, "x_scale", np.uint8, (T, H // 32)), want_s)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quant_mx8_entry_edge_cases(src):
    """moe_quant_mx8 on fp32 rows (fp32 subnormals, the byte clamped at 0) and
    bf16 rows, with a ragged row count: codes and scales bit for bit."""
    from mixture_experts_expert_moe_amd import moe
    torch = gh.torch_mod()
    rng = np.random.default_rng(91 if src == "f32" else 92)
    rows, cols = 37, 768
    v = rows_of(edge_blocks(rng, f32=(src == "f32")), cols, rows, rng)
    if src == "bf16":
        bits = bf16_bits_rne(v)
        v = gh.bf16_to_f64(bits).astype(np.float32)
        dev = torch.from_numpy(bits.view(np.int16)).to("cuda")
    else:
        dev = torch.from_numpy(v).to("cuda")
    codes = torch.full((rows * cols,), 0x5a, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows * cols // 32,), 0x5a, dtype=torch.uint8, device="cuda")
    say("moe_quant_mx8", src, rows, cols)
    moe.moe_quant_mx8(rows, cols, src, dev, codes, scales)
    torch.cuda.synchronize()
    want_c, want_s, _ = oracle.quant_mx8(v)
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(rows, cols), want_c)
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(rows, cols // 32), want_s)


def test_mx8_of_h_edge_cases():
    """h (fp32) quantised in front of the down GEMM: the GPU's codes equal the
    oracle's, and y equals the oracle's down projection of those codes."""
    rng = np.random.default_rng(77)
    H, I, T = 256, 512, 7
    spec = LayerSpec(hidden=H, inter=I, n_routed=8, top_k=2, n_shared=1, act="bf16", wt="mx4", out="f32")
    d = synth.layer_weights(spec, 8200)
    d["x"] = synth.tokens(spec, 8200, T)
    d["spec"] = spec
    g = gh.GpuLayer(d)
    g.route()
    g.permute()
    R = g.R
    h = rows_of(edge_blocks(rng, f32=True), I, R, rng)
    say("h edge cases R", R)
    gh.put(g.layer, "h", h)
    for name in ("h_q", "h_scale"):
        g.layer.tensors[name].fill_(0x5a)
    g.down()
    gh.torch_mod().cuda.synchronize()
    want_c, want_s, _ = oracle.quant_mx8(h)
    np.testing.assert_array_equal(gh.buf(g.layer, "h_q", np.uint8, (R, I)), want_c)
    np.testing.assert_array_equal(gh.buf(g.layer, "h_scale", np.uint8, (R, I // 32)), want_s)
    offsets = g.offsets()
    y_ref = oracle.down(h.astype(np.float64), offsets, H, "mx4", d["w_down"], d["w_down_scale"], None)
    gh.assert_within(g.y(), y_ref, gh.mx_down_bound(d, offsets, h, y_ref), what="down of the edge-case h")
