"""Pins of the CPU oracle against things other than itself: numpy fp64 brute
force of the dense definition, numpy int64 products, numpy's stable sort,
scipy's softmax, closed forms and hand-worked fixtures.  No GPU needed."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

from gen import synth
from gen.synth import LayerSpec
from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- independent decoders used only by these pins --------------------------

def bf16_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_round_bf16(v):
    """RNE to bf16 on the fp32 bit pattern (a different method from the oracle's)."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def q4_decode(packed, s16, m16):
    G, N, K2 = packed.shape
    q = np.empty((G, N, 2 * K2), np.float32)
    q[..., 0::2] = packed & 15
    q[..., 1::2] = packed >> 4
    s = np.repeat(s16.view(np.float16).astype(np.float32), 32, axis=-1)
    m = np.repeat(m16.view(np.float16).astype(np.float32), 32, axis=-1)
    return f32_round_bf16(s * q + m).astype(np.float64)


def weights_f64(fmt, d):
    if fmt == "f32":
        return d["w"].astype(np.float64)
    if fmt == "bf16":
        return bf16_f64(d["w"])
    if fmt == "q4":
        return q4_decode(d["w"], d["scale"], d["min"])
    raise ValueError(fmt)


def np_silu(a):
    return a / (1.0 + np.exp(-a))


def np_route(x64, wr64, k, bias=None):
    """Dense numpy routing: fp64 logits rounded to fp32, selection by (logit desc, id asc)."""
    l32 = (x64 @ wr64.T).astype(np.float32)
    if bias is not None:
        l32 = (l32 + bias.astype(np.float32)).astype(np.float32)
    T, E = l32.shape
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        ids[t] = np.lexsort((np.arange(E), -l32[t].astype(np.float64)))[:k]
    sel = np.take_along_axis(l32, ids, 1).astype(np.float64)
    gates = softmax(sel, axis=1)
    return l32, ids, gates


def np_dense_layer(x64, wr64, bias, wgu, wdn, E, k, S):
    """Brute force: every token through EVERY expert, weighted by a dense gate
    vector that is zero off the top-k; plus the shared expert with weight 1."""
    I = wgu.shape[1] // 2
    _, ids, gates = np_route(x64, wr64, k, bias)
    T = x64.shape[0]
    dense = np.zeros((T, E))
    for t in range(T):
        dense[t, ids[t]] = gates[t]
    out = np.zeros((T, wdn.shape[1]))
    for e in range(E + S):
        hh = np_silu(x64 @ wgu[e, :I].T) * (x64 @ wgu[e, I:].T)
        ye = hh @ wdn[e].T
        out += ye if e == E else dense[:, e:e + 1] * ye
    return out


def make_case(H, I, E, k, S, T, wt, act="f32", seed=0, zipf=0.0):
    spec = LayerSpec(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=S, act=act, wt=wt,
                     out="f32", zipf=zipf)
    wid = 1000 + seed
    d = synth.layer_weights(spec, wid)
    d["x"] = synth.tokens(spec, wid, T)
    d["spec"] = spec
    return d


def x_f64(d):
    x = d["x"]
    return bf16_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


SHAPES = [(64, 32, 4, 1, 0, 1), (64, 32, 8, 2, 1, 5), (128, 64, 16, 4, 1, 17), (256, 128, 128, 8, 1, 3)]


# ---- routing --------------------------------------------------------------------

@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_route_matches_numpy_bruteforce(act):
    d = make_case(256, 32, 64, 8, 1, 40, "f32", act=act, seed=1)
    logits, ids, w = oracle.route(d["x"], d["w_router"], 8)
    wr = d["w_router"]
    wr64 = bf16_f64(wr) if wr.dtype == np.uint16 else wr.astype(np.float64)
    l32, ids_np, g_np = np_route(x_f64(d), wr64, 8)
    # fp64 sums in different orders round to the same fp32 value here (1 ulp allowed).
    assert np.all(np.abs(logits - l32) <= np.spacing(np.abs(l32)))
    np.testing.assert_array_equal(ids, ids_np)
    np.testing.assert_allclose(w, g_np, rtol=2e-7, atol=0)


def test_route_invariants():
    d = make_case(256, 32, 128, 8, 1, 64, "f32", act="bf16", seed=2)
    logits, ids, w = oracle.route(d["x"], d["w_router"], 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 8 * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)                 # gates non-increasing
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == 8                # distinct experts
        sel = logits[t, ids[t]]
        rest = np.delete(logits[t], ids[t])
        assert sel.min() >= rest.max()                       # really the k largest


def test_route_k_equals_e_is_full_softmax():
    d = make_case(128, 32, 8, 8, 0, 9, "f32", seed=3)
    logits, ids, w = oracle.route(d["x"], d["w_router"], 8)
    for t in range(9):
        full = softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(w[t], full[ids[t]], rtol=2e-7)
        assert sorted(ids[t].tolist()) == list(range(8))


def test_route_top1_gate_is_exactly_one():
    d = make_case(128, 32, 16, 1, 0, 11, "f32", seed=4)
    _, _, w = oracle.route(d["x"], d["w_router"], 1)
    assert np.all(w == 1.0)


def test_route_bias_dominates():
    d = make_case(128, 32, 16, 2, 0, 13, "f32", seed=5)
    bias = np.zeros(16, np.float32)
    bias[11] = 100.0
    _, ids, w = oracle.route(d["x"], d["w_router"], 2, bias)
    assert np.all(ids[:, 0] == 11)
    assert np.all(w[:, 0] > 0.999999)


def test_route_ties_go_to_lower_id():
    d = make_case(64, 32, 8, 3, 0, 6, "f32", seed=6)
    wr = d["w_router"].copy()
    wr[5] = wr[2]          # experts 2 and 5 get identical logits
    wr[7] = wr[2]
    bias = np.zeros(8, np.float32)
    bias[[2, 5, 7]] = 50.0  # ... and the three of them are the top 3
    logits, ids, w = oracle.route(d["x"], wr, 3, bias)
    np.testing.assert_array_equal(ids, np.tile([2, 5, 7], (6, 1)))
    assert np.all(w == w[:, :1])  # equal logits, equal gates


def test_route_softmax_closed_form():
    # Two experts, logits ln 3 and 0 -> gates 3/4 and 1/4.  x = e_0, router rows
    # (ln 3, 0, ...) and 0: the fp32 logit is fp32(ln 3) and the gate is
    # e^{fp32(ln 3)} / (e^{fp32(ln 3)} + 1), within fp32 rounding of 3/4.
    x = np.zeros((1, 4), np.float32)
    x[0, 0] = 1.0
    wr = np.zeros((2, 4), np.float32)
    wr[0, 0] = math.log(3.0)
    _, ids, w = oracle.route(x, wr, 2)
    assert ids.tolist() == [[0, 1]]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-7)


# ---- permutation ---------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,S", [(1, 4, 1, 0), (37, 16, 4, 1), (256, 128, 8, 1), (5, 8, 8, 1), (0, 8, 2, 1)])
def test_permute_matches_stable_sort(T, E, k, S):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    offsets, row_token, token_row = oracle.permute(ids, E, S)
    # Independent construction: stable argsort of the flattened (token, slot) list by expert.
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    routed_tokens = order // k
    R = T * k + S * T
    assert offsets[-1] == R
    np.testing.assert_array_equal(row_token[:T * k], routed_tokens)
    counts = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(np.diff(offsets)[:E], counts)
    if S:
        np.testing.assert_array_equal(row_token[T * k:], np.arange(T))
        assert offsets[E] == T * k
    # Invariants: every token appears exactly k times among routed rows (+1 shared),
    # token_row and row_token are mutual inverses, tokens ascend inside a group.
    np.testing.assert_array_equal(np.bincount(row_token[:T * k], minlength=T), np.full(T, k))
    for t in range(T):
        for j in range(k + S):
            r = token_row[t, j]
            assert row_token[r] == t
            g = E if j == k else ids[t, j]
            assert offsets[g] <= r < offsets[g + 1]
    for g in range(E + S):
        seg = row_token[offsets[g]:offsets[g + 1]]
        assert np.all(np.diff(seg) > 0)


# ---- whole layer vs dense brute force -------------------------------------------

@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("wt", ["f32", "bf16", "q4"])
def test_layer_matches_dense_bruteforce(shape, wt):
    H, I, E, k, S, T = shape
    act = "f32" if wt == "f32" else "bf16"
    d = make_case(H, I, E, k, S, T, wt, act=act, seed=hash((shape, wt)) % 1000)
    out, st = oracle.layer(d, with_steps=True)
    wr = d["w_router"]
    wr64 = bf16_f64(wr) if wr.dtype == np.uint16 else wr.astype(np.float64)
    wgu = weights_f64(wt, {"w": d["w_gu"], "scale": d["w_gu_scale"], "min": d["w_gu_min"]})
    wdn = weights_f64(wt, {"w": d["w_down"], "scale": d["w_down_scale"], "min": d["w_down_min"]})
    ref = np_dense_layer(x_f64(d), wr64, None, wgu, wdn, E, k, S)
    # gates are fp32 in the oracle (rounded once); the brute force keeps fp64 gates.
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_layer_fp32_workload_full_size_dense():
    """The fp32 16-expert top-2 workload at full size against the brute force."""
    d = synth.layer_inputs("fp32_e16_top2", 16)
    out = oracle.layer(d)
    wgu = d["w_gu"].astype(np.float64)
    wdn = d["w_down"].astype(np.float64)
    ref = np_dense_layer(d["x"].astype(np.float64), d["w_router"].astype(np.float64), None, wgu, wdn, 16, 2, 0)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_zipf_bias_routing_dense():
    d = make_case(128, 32, 32, 4, 1, 21, "f32", seed=9, zipf=1.1)
    out = oracle.layer(d)
    wgu = d["w_gu"].astype(np.float64)
    wdn = d["w_down"].astype(np.float64)
    ref = np_dense_layer(d["x"].astype(np.float64), d["w_router"].astype(np.float64), d["bias"], wgu, wdn, 32, 4, 1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_single_expert_is_plain_swiglu_ffn():
    """E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN."""
    d = make_case(96, 48, 1, 1, 0, 7, "f32", seed=10)
    out = oracle.layer(d)
    x = d["x"].astype(np.float64)
    wg, wu = d["w_gu"][0, :48].astype(np.float64), d["w_gu"][0, 48:].astype(np.float64)
    wd = d["w_down"][0].astype(np.float64)
    a = x @ wg.T
    ref = ((a / (1 + np.exp(-a))) * (x @ wu.T)) @ wd.T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_zero_up_projection_gives_zero():
    d = make_case(64, 32, 8, 2, 1, 5, "f32", seed=11)
    d["w_gu"][:, 32:, :] = 0.0
    out = oracle.layer(d)
    assert np.all(out == 0.0)


def test_shared_expert_is_added_with_weight_one():
    """Zero every routed expert's down projection: only the shared expert remains."""
    d = make_case(64, 32, 8, 2, 1, 5, "f32", seed=12)
    d["w_down"][:8] = 0.0
    out = oracle.layer(d)
    x = d["x"].astype(np.float64)
    wg, wu = d["w_gu"][8, :32].astype(np.float64), d["w_gu"][8, 32:].astype(np.float64)
    a = x @ wg.T
    ref = (np_silu(a) * (x @ wu.T)) @ d["w_down"][8].astype(np.float64).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_token_independence():
    """Each token's output depends on that token alone (no cross-token terms)."""
    d = make_case(128, 64, 16, 4, 1, 12, "bf16", act="bf16", seed=13)
    full = oracle.layer(d)
    for lo, hi in [(0, 1), (3, 9), (11, 12)]:
        part = dict(d)
        part["x"] = np.ascontiguousarray(d["x"][lo:hi])
        np.testing.assert_array_equal(oracle.layer(part), full[lo:hi])


# ---- silu, quantisation, 4-bit, rmsnorm, bf16 rounding ---------------------------

def test_silu_closed_forms():
    # Single-expert layer with x = e_0 and hand-set rows: h = silu(a) * 1, y = h.
    for a, expect in [(1.0, 1 / (1 + math.exp(-1))), (-1.0, -1 / (1 + math.e)), (0.0, 0.0),
                      (math.log(3.0), 0.75 * math.log(3.0))]:
        x = np.zeros((1, 4), np.float32)
        x[0, 0] = 1.0
        wgu = np.zeros((1, 2, 4), np.float32)
        wgu[0, 0, 0] = a
        wgu[0, 1, 0] = 1.0
        offsets = np.array([0, 1], np.int32)
        h = oracle.gate_up(x, offsets, np.array([0], np.int32), 1, "f32", wgu)
        assert abs(h[0, 0] - expect) <= 1e-7 * max(1.0, abs(expect)), (a, h[0, 0], expect)


def test_int8_quant_closed_forms():
    v = np.array([[0.0] * 8,
                  [1.0, -1.0, 0.5, 0.25, 0.0, -0.5, 0.125, 1.0],
                  [3.0, 1.5 * 3.0 / 127, 2.5 * 3.0 / 127, -2.5 * 3.0 / 127, 0, 0, 0, -3.0]], np.float32)
    q, s = oracle.quant_rows_i8(v)
    assert s[0] == 0.0 and np.all(q[0] == 0)
    assert s[1] == np.float32(1.0) / np.float32(127.0)
    assert q[1, 0] == 127 and q[1, 1] == -127 and q[1, 7] == 127
    assert q[2, 0] == 127 and q[2, 7] == -127
    # The element that is the max maps to exactly +-127; the rest are rne(v / s).
    s2 = np.float32(3.0) / np.float32(127.0)
    for c in (1, 2, 3):
        assert q[2, c] == np.rint(np.float32(v[2, c]) / s2)


def test_int8_path_matches_int64_products():
    H, I, E, k, S, T = 256, 64, 8, 2, 1, 6
    d = make_case(H, I, E, k, S, T, "i8", act="bf16", seed=14)
    out, st = oracle.layer(d, with_steps=True)
    xq, xs = st["xq"], st["xs"]
    offsets, row_token = st["offsets"], st["row_token"]
    h = st["h"]
    wq, ws = d["w_gu"], d["w_gu_scale"]
    for g in range(E + S):
        rows = np.arange(offsets[g], offsets[g + 1])
        if rows.size == 0:
            continue
        toks = row_token[rows]
        acc = xq[toks].astype(np.int64) @ wq[g].astype(np.int64).T      # [rows][2I], exact
        assert np.abs(acc).max() < 2 ** 31
        a = (acc.astype(np.float32) * xs[toks][:, None]) * ws[g][None, :]
        ag, au = a[:, :I], a[:, I:]
        e = np.exp(-ag.astype(np.float64)).astype(np.float32)
        ref = (ag / (np.float32(1.0) + e)) * au
        np.testing.assert_array_equal(h[rows].astype(np.float32), ref)
    # down: requantise h per row, exact int products, fp32 dequant
    y = st["y"]
    hq, hs = oracle.quant_rows_i8(h.astype(np.float32))
    for g in range(E + S):
        rows = np.arange(offsets[g], offsets[g + 1])
        if rows.size == 0:
            continue
        acc = hq[rows].astype(np.int64) @ d["w_down"][g].astype(np.int64).T
        ref = (acc.astype(np.float32) * hs[rows][:, None]) * d["w_down_scale"][g][None, :]
        np.testing.assert_array_equal(y[rows].astype(np.float32), ref)


def test_q4_golden_block():
    with open(os.path.join(GOLDEN, "q4_block.json")) as f:
        gb = json.load(f)
    packed = np.array(gb["bytes"], np.uint8).reshape(1, 1, 16)
    s = np.array([[[gb["scale16"]]]], np.uint16)
    m = np.array([[[gb["min16"]]]], np.uint16)
    vals = oracle.q4_values(packed, s, m)
    np.testing.assert_array_equal(vals.reshape(-1), np.array(gb["values"], np.float32))


def test_q4_code_extremes_and_roundtrip():
    d = synth.weights(synth.key(77, 0, 4), 2, 8, 128, 0.02, "q4")
    vals = oracle.q4_values(d["w"], d["scale"], d["min"])
    ref = q4_decode(d["w"], d["scale"], d["min"])
    np.testing.assert_array_equal(vals.astype(np.float64), ref)
    s = d["scale"].view(np.float16).astype(np.float32)
    m = d["min"].view(np.float16).astype(np.float32)
    lo = f32_round_bf16(m)                     # q = 0 -> min
    hi = f32_round_bf16(np.float32(15) * s + m)  # q = 15 -> 15 * scale + min
    blocks = vals.reshape(2, 8, 4, 32)
    codes = np.empty((2, 8, 128), np.uint8)
    codes[..., 0::2] = d["w"] & 15
    codes[..., 1::2] = d["w"] >> 4
    codes = codes.reshape(2, 8, 4, 32)
    for (g, n, b, j) in zip(*np.nonzero(codes == 0)):
        assert blocks[g, n, b, j] == lo[g, n, b]
    for (g, n, b, j) in zip(*np.nonzero(codes == 15)):
        assert blocks[g, n, b, j] == hi[g, n, b]
    # Round trip of the synthetic quantiser: within half a step (plus fp16/bf16 rounding) of the draw.
    raw = synth.weights(synth.key(77, 0, 4), 2, 8, 128, 0.02, "f32")["w"].reshape(2, 8, 4, 32)
    step = np.repeat(s[..., None], 32, -1)
    err = np.abs(blocks - raw)
    assert np.all(err <= 0.5 * step + 2 ** -8 * np.abs(raw) + 1e-4 * step + 2e-5)


def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (2.0, -0.5, 1e-3):
        x = np.full((1, 64), c, np.float32)
        xn = oracle.rmsnorm(x, eps)
        expect = math.copysign(1.0, c) / math.sqrt(1.0 + eps / (float(np.float32(c)) ** 2))
        np.testing.assert_allclose(xn, expect, rtol=1e-14)
    x = np.array([[3.0, 4.0]], np.float32)
    np.testing.assert_allclose(oracle.rmsnorm(x, eps), x.astype(np.float64) / math.sqrt(12.5 + eps), rtol=1e-14)


def test_round_bf16_ties_to_even():
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8), 3.0, 0.0])
    np.testing.assert_array_equal(oracle.round_bf16(v), [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 3.0, 0.0])


# ---- residual combine and the stacked composition ----------------------------------

def bf16_rne_exact(v):
    """fp64 -> nearest bf16 value (ties to even) with exact rational arithmetic:
    the spacing of bf16 numbers in [2^e, 2^(e+1)) is 2^(e-7); v / spacing is
    rounded to the nearest integer, ties to the even one.  Normal range only."""
    from fractions import Fraction
    out = np.empty(np.shape(v))
    for i, x in enumerate(np.asarray(v, np.float64).reshape(-1)):
        if x == 0.0:
            out.flat[i] = 0.0
            continue
        f = Fraction(float(x))
        a = abs(f)
        e = math.floor(math.log2(a))
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        sp = Fraction(2) ** (e - 7)
        q = a / sp
        n = q.numerator // q.denominator
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        r = n * sp
        out.flat[i] = float(r if f > 0 else -r)
    return out


def test_bf16_rne_exact_helper():
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8), 3.0, 0.0, 255.5, 0.1])
    np.testing.assert_array_equal(bf16_rne_exact(v)[:7], [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 3.0, 0.0, 256.0])
    assert abs(bf16_rne_exact(v)[7] - 0.1) <= 2 ** -4 * 2 ** -8  # within half a spacing at 0.1
    np.testing.assert_array_equal(oracle.round_bf16(v), bf16_rne_exact(v))


@pytest.mark.parametrize("wt", ["f32", "bf16", "q4"])
def test_combine_residual_matches_dense(wt):
    """The combine's residual branch: out = dense layer + residual, element by element."""
    H, I, E, k, S, T = 128, 64, 16, 4, 1, 9
    act = "f32" if wt == "f32" else "bf16"
    d = make_case(H, I, E, k, S, T, wt, act=act, seed=31)
    res = synth.tokens(d["spec"], 1031, T, stream=5, dtype="f32")
    out = oracle.layer(d, residual=res)
    wr = d["w_router"]
    wr64 = bf16_f64(wr) if wr.dtype == np.uint16 else wr.astype(np.float64)
    wgu = weights_f64(wt, {"w": d["w_gu"], "scale": d["w_gu_scale"], "min": d["w_gu_min"]})
    wdn = weights_f64(wt, {"w": d["w_down"], "scale": d["w_down_scale"], "min": d["w_down_min"]})
    ref = np_dense_layer(x_f64(d), wr64, None, wgu, wdn, E, k, S) + res.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())
    # residual alone: zero every expert's down projection
    d0 = dict(d)
    d0["w_down"] = np.zeros_like(d["w_down"])
    if wt == "q4":  # codes 0 with min 0 decode to exactly 0
        d0["w_down_min"] = np.zeros_like(d["w_down_min"])
    np.testing.assert_array_equal(oracle.layer(d0, residual=res), res.astype(np.float64))


def test_stack_composition_matches_dense():
    """Three stacked 4-bit layers: x_{l+1} = fp32(x_l + dense_l(bf16(RMSNorm(x_l)))),
    RMSNorm in numpy fp64, bf16 rounding by exact rational arithmetic, each
    layer by the dense brute force."""
    H, I, E, k, S, T, eps = 128, 64, 16, 4, 1, 5, 1e-6
    spec = LayerSpec(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=S, act="bf16", wt="q4", out="f32")
    layers = [synth.layer_weights(spec, 1500, l) for l in range(3)]
    for dl in layers:
        dl["spec"] = spec
    x0 = synth.tokens(spec, 1500, T, stream=2, dtype="f32")
    got = oracle.stack_forward(layers, x0, eps)
    x = x0.astype(np.float32)
    for dl in layers:
        x64 = x.astype(np.float64)
        xn = bf16_rne_exact(x64 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + eps))
        wgu = weights_f64("q4", {"w": dl["w_gu"], "scale": dl["w_gu_scale"], "min": dl["w_gu_min"]})
        wdn = weights_f64("q4", {"w": dl["w_down"], "scale": dl["w_down_scale"], "min": dl["w_down_min"]})
        y = np_dense_layer(xn, bf16_f64(dl["w_router"]), None, wgu, wdn, E, k, S)
        x = (x64 + y).astype(np.float32)
    # fp32 residual stream: the brute force keeps fp64 gates, the oracle fp32 ones
    np.testing.assert_allclose(got, x, rtol=0, atol=2e-6 * np.abs(x).max())
    # one layer with steps: the bf16 input and the MoE output without the residual
    x1, st = oracle.stack_layer(layers[0], x0, eps, with_steps=True)
    np.testing.assert_array_equal(x1, oracle.stack_forward(layers[:1], x0, eps))
    x64 = x0.astype(np.float64)
    xn = bf16_rne_exact(x64 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + eps))
    np.testing.assert_array_equal(bf16_f64(st["xn"]), xn)
    np.testing.assert_allclose(st["moe"] + x64, x1.astype(np.float64), rtol=0, atol=2e-6 * np.abs(x1).max())


# ---- MX formats: MXFP4 weights, MXFP8 activations ---------------------------------

def e4m3_grid():
    """All finite E4M3 magnitudes with their codes, from the bit fields (exponent bias 7,
    exponent 0 subnormal, the all-ones pattern reserved): an enumeration independent of
    the oracle's rounding."""
    mags, codes = [], []
    for c in range(127):
        e, m = c >> 3, c & 7
        mags.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
        codes.append(c)
    return np.array(mags), np.array(codes)


def test_mx_golden_blocks():
    with open(os.path.join(GOLDEN, "mx_blocks.json")) as f:
        fx = json.load(f)
    m = fx["mxfp4"]
    w = np.array(m["bytes"] * 2, np.uint8).reshape(1, 1, 32)
    v = oracle.mx4_values(w, np.array(m["scales"], np.uint8).reshape(1, 1, 2))
    np.testing.assert_array_equal(v[0, 0, :32], m["values_scale127"])
    np.testing.assert_array_equal(v[0, 0, 32:], m["values_scale129"])
    for b in fx["mxfp8"]:
        c, s, d = oracle.quant_mx8(np.array([b["input"]], np.float32))
        assert s[0, 0] == b["scale"]
        np.testing.assert_array_equal(c[0], b["codes"])
        np.testing.assert_array_equal(d[0], b["values"])


def test_mx8_quant_is_nearest_e4m3_value():
    """On random rows spanning many binades: each block's scale puts its largest
    magnitude in [256, 512) (before saturation at 448), and every value becomes the
    E4M3 value nearest to v / scale (ties to the even code), found by brute force over
    the whole grid."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((6, 256)) * 2.0 ** rng.integers(-30, 10, (6, 1))).astype(np.float32)
    v[2, :32] = 0.0
    codes, sc, deq = oracle.quant_mx8(v)
    mags, gcodes = e4m3_grid()
    for r in range(6):
        for b in range(8):
            blk = v[r, 32 * b:32 * b + 32].astype(np.float64)
            s = int(sc[r, b])
            if not blk.any():
                assert s == 0 and not codes[r, 32 * b:32 * b + 32].any()
                continue
            X = 2.0 ** (s - 127)
            assert 256 <= np.abs(blk).max() / X < 512
            for j in range(32):
                a = abs(blk[j]) / X
                d = np.abs(mags - a)
                best = np.flatnonzero(d == d.min())
                want = gcodes[best[0]] if len(best) == 1 else [c for c in gcodes[best] if c % 2 == 0][0]
                if a > 448:
                    want = 126
                if want == 0:
                    assert codes[r, 32 * b + j] in (0, 0x80)
                else:
                    assert codes[r, 32 * b + j] == want | (0x80 if blk[j] < 0 else 0)
                assert deq[r, 32 * b + j] == np.copysign(mags[want], blk[j]) * X


def mx4_decode_np(w, s):
    """MXFP4 values by table lookup (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 the sign)."""
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1.0, -1.0], 8)
    G, N, K2 = w.shape
    c = np.empty((G, N, 2 * K2), np.int64)
    c[..., 0::2] = w & 15
    c[..., 1::2] = w >> 4
    return mag[c] * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=-1)


@pytest.mark.parametrize("shape", [(64, 32, 4, 1, 0, 3), (128, 64, 16, 4, 1, 11), (256, 128, 32, 8, 1, 5)])
def test_layer_mx4_matches_dense(shape):
    """MXFP4 weights with MXFP8 activations: every token through every expert
    (quantised token rows; h rounded to fp32 and quantised per block of 32 before
    the down projection), dense gates, shared expert with weight 1."""
    H, I, E, k, S, T = shape
    d = make_case(H, I, E, k, S, T, "mx4", act="bf16", seed=41)
    out = oracle.layer(d)
    np.testing.assert_array_equal(oracle.mx4_values(d["w_gu"], d["w_gu_scale"]), mx4_decode_np(d["w_gu"], d["w_gu_scale"]))
    wgu = mx4_decode_np(d["w_gu"], d["w_gu_scale"])
    wdn = mx4_decode_np(d["w_down"], d["w_down_scale"])
    x64 = x_f64(d)
    _, ids, gates = np_route(x64, bf16_f64(d["w_router"]), k)
    xq = oracle.quant_mx8(x64.astype(np.float32))[2]
    dense = np.zeros((T, E))
    for t in range(T):
        dense[t, ids[t]] = gates[t]
    ref = np.zeros((T, H))
    for e in range(E + S):
        hh = np_silu(xq @ wgu[e, :I].T) * (xq @ wgu[e, I:].T)
        ye = oracle.quant_mx8(hh.astype(np.float32))[2] @ wdn[e].T
        ref += ye if e == E else dense[:, e:e + 1] * ye
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())
