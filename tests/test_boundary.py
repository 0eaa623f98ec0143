"""The C-ABI library on the CPU: it loads, exports every entry point that
include/moe.h declares, sizes buffers, and rejects bad arguments before any
launch (only rejected calls are made here; nothing reaches a GPU)."""
import ctypes
import os
import re

import pytest

from mixture_experts_expert_moe_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 4


def test_status_strings():
    L = moe.lib()
    for code in (0, -1, -2, -3, -4):
        assert L.moe_status_string(code)


def bufs_all(p=FAKE):
    return moe.MoeBuffers(*([p] * len(moe.BUFFER_NAMES)))


def desc(**kw):
    base = dict(hidden=2048, inter=512, n_routed=128, top_k=8, n_shared=1, max_tokens=256, act="bf16", wt="bf16",
                out="bf16")
    base.update(kw)
    return moe.make_desc(**base)


def status(fn, *args):
    return getattr(moe.lib(), fn)(*args)


def test_buffer_sizes_match_shapes():
    s = moe.moe_buffer_sizes(desc())
    R = 256 * 9
    # fp32 logits, then 8 H-slices x min(max_tokens, 16) tokens x E of fp64 partial sums (few-token routing)
    # logits + fp64 partials: 8 slices x 16 tokens (few-token calls) or 2 slices x max_tokens
    assert s["logits"] == 256 * 128 * 4 + max(8 * 16, 2 * 256) * 128 * 8
    assert moe.moe_buffer_sizes(desc(max_tokens=3))["logits"] == 3 * 128 * 4 + max(8 * 3, 2 * 3) * 128 * 8
    assert s["topk_ids"] == s["topk_w"] == 256 * 8 * 4
    assert s["expert_offsets"] == 130 * 4
    assert s["row_token"] == R * 4 and s["token_row"] == 256 * 9 * 4
    assert s["h"] == R * 512 * 2 and s["y"] == R * 2048 * 2
    assert s["x_q"] == s["h_q"] == 0
    s8 = moe.moe_buffer_sizes(desc(wt="i8"))
    assert s8["x_q"] == 256 * 2048 and s8["h_q"] == R * 512 and s8["h"] == R * 512 * 4
    assert s["sync"] == s8["sync"] == 4096
    # MXFP4 weights: E4M3 codes of x and h, one E8M0 byte per 32 values, fp32 h and y
    sm = moe.moe_buffer_sizes(desc(wt="mx4"))
    assert sm["x_q"] == 256 * 2048 and sm["x_scale"] == 256 * 2048 // 32
    assert sm["h_q"] == R * 512 and sm["h_scale"] == R * 512 // 32
    assert sm["h"] == R * 512 * 4 and sm["y"] == R * 2048 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=2000), -2), (dict(inter=300), -2), (dict(top_k=0), -1), (dict(top_k=129), -1),
    (dict(top_k=17, n_routed=32), -2), (dict(n_shared=2), -1), (dict(max_tokens=0), -1),
    (dict(max_tokens=2600), -2), (dict(n_routed=257, top_k=8), -2), (dict(act="f32", wt="bf16"), -2),
    (dict(act="bf16", wt="f32"), -2), (dict(out="i8"), -2), (dict(act="i8"), -2),
    (dict(n_routed=256, max_tokens=1300), -2),
])
def test_bad_desc_rejected(kw, code):
    sizes = (ctypes.c_size_t * 14)()
    assert status("moe_buffer_sizes", ctypes.byref(desc(**kw)), sizes) == code


def test_calls_reject_before_launch():
    d = desc()
    b = bufs_all()
    w = moe.MoeWeights(FAKE, None, None)
    by = ctypes.byref
    # T > max_tokens
    assert status("moe_route_topk", by(d), 257, FAKE, FAKE, None, by(b), None) == -3
    assert status("moe_permute", by(d), 300, FAKE, by(b), None) == -3
    assert status("moe_route_permute", by(d), 257, FAKE, FAKE, None, by(b), None) == -3
    assert status("moe_grouped_gemm_gu", by(d), 257, FAKE, by(w), by(b), None) == -3
    assert status("moe_grouped_gemm_down", by(d), 257, by(w), by(b), None) == -3
    assert status("moe_combine", by(d), 257, None, FAKE, by(b), None) == -3
    # negative T, null pointers, misaligned pointers, missing quantisation parameters
    assert status("moe_route_topk", by(d), -1, FAKE, FAKE, None, by(b), None) == -1
    assert status("moe_route_topk", by(d), 4, None, FAKE, None, by(b), None) == -1
    assert status("moe_route_topk", by(d), 4, FAKE + 2, FAKE, None, by(b), None) == -1
    assert status("moe_route_permute", by(d), 4, None, FAKE, None, by(b), None) == -1
    assert status("moe_route_permute", by(d), 4, FAKE, FAKE, FAKE + 4, by(b), None) == -1   # misaligned bias
    assert status("moe_route_permute", by(desc(wt="i8")), 4, FAKE, FAKE, None, by(moe.MoeBuffers(
        *[None if n in ("x_q", "x_scale") else FAKE for n in moe.BUFFER_NAMES])), None) == -1  # int8 needs x_q
    assert status("moe_grouped_gemm_gu", by(d), 4, FAKE, by(moe.MoeWeights(None, None, None)), by(b), None) == -1
    d8 = desc(wt="i8")
    assert status("moe_grouped_gemm_gu", by(d8), 4, FAKE, by(w), by(b), None) == -1       # no scales
    d4 = desc(wt="q4")
    assert status("moe_grouped_gemm_down", by(d4), 4, by(moe.MoeWeights(FAKE, FAKE, None)), by(b), None) == -1
    nob = bufs_all(None)
    assert status("moe_permute", by(d), 4, FAKE, by(nob), None) == -1
    assert status("moe_combine", by(d), 4, None, FAKE, by(nob), None) == -1
    assert status("moe_rmsnorm", 4, 2000, ctypes.c_float(1e-6), FAKE, FAKE, None) == -2
    assert status("moe_rmsnorm", -1, 2048, ctypes.c_float(1e-6), FAKE, FAKE, None) == -1
    # bad desc through a compute call
    assert status("moe_combine", by(desc(hidden=100)), 4, None, FAKE, by(b), None) == -2
    # fused combine + RMSNorm: fp32 output stream only, hidden <= 8192, an xn buffer, eps >= 0
    f32 = desc(out="f32")
    eps = ctypes.c_float(1e-6)
    assert status("moe_combine_rmsnorm", by(d), 4, None, eps, FAKE, FAKE, by(b), None) == -2
    assert status("moe_combine_rmsnorm", by(desc(out="f32", hidden=8448)), 4, None, eps, FAKE, FAKE, by(b), None) == -2
    assert status("moe_combine_rmsnorm", by(f32), 4, None, eps, FAKE, None, by(b), None) == -1
    assert status("moe_combine_rmsnorm", by(f32), 4, None, eps, FAKE, FAKE + 8, by(b), None) == -1
    assert status("moe_combine_rmsnorm", by(f32), 4, None, ctypes.c_float(-1.0), FAKE, FAKE, by(b), None) == -1
    assert status("moe_combine_rmsnorm", by(f32), 257, None, eps, FAKE, FAKE, by(b), None) == -3
    assert status("moe_combine_rmsnorm", by(f32), 4, None, eps, FAKE, FAKE, by(nob), None) == -1


def test_zero_tokens_returns_ok_without_launch():
    d = desc()
    b = bufs_all()
    w = moe.MoeWeights(FAKE, None, None)
    by = ctypes.byref
    assert status("moe_route_topk", by(d), 0, FAKE, FAKE, None, by(b), None) == 0
    assert status("moe_permute", by(d), 0, FAKE, by(b), None) == 0
    assert status("moe_route_permute", by(d), 0, FAKE, FAKE, None, by(b), None) == 0
    assert status("moe_grouped_gemm_gu", by(d), 0, FAKE, by(w), by(b), None) == 0
    assert status("moe_grouped_gemm_down", by(d), 0, by(w), by(b), None) == 0
    assert status("moe_combine", by(d), 0, None, FAKE, by(b), None) == 0
    assert status("moe_rmsnorm", 0, 2048, ctypes.c_float(1e-6), FAKE, FAKE, None) == 0
    assert status("moe_combine_rmsnorm", by(desc(out="f32")), 0, None, ctypes.c_float(1e-6), FAKE, FAKE, by(b),
                  None) == 0


def test_decode_layer_rejects_before_launch():
    by = ctypes.byref
    eps = ctypes.c_float(1e-6)
    w = moe.MoeWeights(FAKE, FAKE, FAKE)
    b = bufs_all()
    NORM = moe.MOE_DECODE_NORM_INPUT

    def call(d, T, flags=0, res=None, bufs=b, wts=w, e=eps):
        return status("moe_decode_layer", by(d), T, FAKE, FAKE, None, by(wts), by(wts), res, flags, e, FAKE,
                      by(bufs), None)
    d = desc(max_tokens=32)
    f32 = desc(max_tokens=32, out="f32")
    assert call(d, 0) == 0                                   # nothing to do, nothing launched
    assert call(d, 33) == -3                                 # T > max_tokens
    assert call(d, 17) == -2                                 # more tokens than one decode launch takes
    assert call(desc(max_tokens=32, hidden=4096), 9) == -2   # T * hidden > 32768 (inputs kept in LDS)
    assert call(desc(max_tokens=32, inter=1024), 4) == -2    # staged h rows exceed LDS
    assert call(desc(max_tokens=32, act="f32", wt="f32", out="f32"), 4) == -2
    assert call(d, 4, flags=NORM) == -2                      # the residual stream is fp32
    assert call(f32, 4, flags=NORM, res=FAKE) == -1          # x is the residual in that mode
    assert call(f32, 4, flags=2) == -1                       # unknown flag
    assert call(d, 4, e=ctypes.c_float(-1.0)) == -1
    assert call(d, 4, res=FAKE + 4) == -1
    assert call(d, 4, bufs=moe.MoeBuffers(*[None if n == "sync" else FAKE for n in moe.BUFFER_NAMES])) == -1
    assert call(d, 4, wts=moe.MoeWeights(None, None, None)) == -1
    assert call(desc(max_tokens=32, wt="i8"), 4, bufs=moe.MoeBuffers(
        *[None if n == "h_q" else FAKE for n in moe.BUFFER_NAMES])) == -1


def test_decode_layer_static_rejects_before_launch():
    by = ctypes.byref
    eps = ctypes.c_float(1e-6)
    w = moe.MoeWeights(FAKE, FAKE, FAKE)

    def call(d, T, x=FAKE, flags=0):
        return status("moe_decode_layer_static", by(d) if d is not None else None, T, x, FAKE, None, by(w), by(w),
                      None, flags, eps, FAKE, None)
    d = desc(max_tokens=4)
    assert call(d, 0) == 0                      # nothing to do; the device is not touched
    assert call(d, 0, x=None) == -1             # arguments are checked even then
    assert call(None, 1) == -1
    assert call(d, -1) == -1
    assert call(d, 17) == -2                    # the static buffers are laid out for 16 tokens
    assert call(desc(hidden=2000), 1) == -2


def test_quant_mx8_rejects_before_launch():
    L = moe.lib()
    q = L.moe_quant_mx8
    assert q(0, 256, moe.MOE_F32, FAKE, FAKE, FAKE, None) == 0          # no rows: no work
    assert q(-1, 256, moe.MOE_F32, FAKE, FAKE, FAKE, None) == -1
    assert q(4, 0, moe.MOE_F32, FAKE, FAKE, FAKE, None) == -1
    assert q(4, 256, moe.MOE_I8, FAKE, FAKE, FAKE, None) == -1          # source must be fp32 or bf16
    assert q(4, 320, moe.MOE_BF16, FAKE, FAKE, FAKE, None) == -2        # cols % 256
    assert q(4, 256, moe.MOE_F32, None, FAKE, FAKE, None) == -1
    assert q(4, 256, moe.MOE_F32, FAKE, FAKE + 8, FAKE, None) == -1     # codes misaligned
    assert q(4, 256, moe.MOE_F32, FAKE, FAKE, None, None) == -1
