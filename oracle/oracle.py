"""Python driver of the CPU oracle (oracle/moe_oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.  The GPU product path never imports it.

Arrays are numpy; bf16 tensors are passed as uint16 bit patterns, 4-bit
weights as (packed uint8, fp16 scale bits, fp16 min bits), int8 weights as
(int8, fp32 per-row scale).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "i8": 2, "q4": 3, "mx4": 4}


def build(force: bool = True) -> str:
    """Compile oracle/liboracle.so with g++ -O2 (IEEE arithmetic, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i, i64, p, d = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_route.argtypes = [i, i, i, i, i, p, p, p, p, p, p]
        L.oracle_permute.argtypes = [i, i, i, i, p, p, p, p]
        L.oracle_quant_rows_i8.argtypes = [i, i, p, p, p]
        L.oracle_quant_rows_i8.restype = None
        L.oracle_gu.argtypes = [i, i, i, i, p, p, i, p, p, p, i, p, p, p, p, i]
        L.oracle_down.argtypes = [i, i, i, p, p, i, p, p, p, p, i]
        L.oracle_combine.argtypes = [i, i, i, i, p, p, p, p, p]
        L.oracle_rmsnorm.argtypes = [i, i, d, p, p]
        L.oracle_rmsnorm.restype = None
        L.oracle_round_bf16.argtypes = [i64, p, p]
        L.oracle_round_bf16.restype = None
        L.oracle_q4_values.argtypes = [i, i, i, p, p, p, p]
        L.oracle_q4_values.restype = None
        L.oracle_quant_mx8.argtypes = [i, i, p, p, p, p]
        L.oracle_quant_mx8.restype = None
        L.oracle_mx4_values.argtypes = [i, i, i, p, p, p]
        L.oracle_mx4_values.restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy"
    return a.ctypes.data


def _act_dt(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return DT["f32"]
    if x.dtype == np.uint16:
        return DT["bf16"]
    raise TypeError("activations are float32 or bf16 bits (uint16), got %s" % x.dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def route(x: np.ndarray, w_router: np.ndarray, top_k: int, bias: np.ndarray | None = None):
    """-> (logits float32 [T][E], topk_ids int32 [T][k], topk_w float32 [T][k])."""
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.dtype == x.dtype and w_router.shape[1] == H
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(lib().oracle_route(T, H, E, top_k, _act_dt(x), _p(x), _p(w_router), _p(b), _p(logits), _p(ids), _p(w)),
           "route")
    return logits, ids, w


def permute(topk_ids: np.ndarray, n_routed: int, n_shared: int):
    """-> (expert_offsets int32 [G+1], row_token int32 [R], token_row int32 [T][k+S])."""
    T, k = topk_ids.shape
    G = n_routed + n_shared
    R = T * k + n_shared * T
    offsets = np.empty(G + 1, np.int32)
    row_token = np.empty(max(R, 1), np.int32)[:R]
    token_row = np.empty((T, k + n_shared), np.int32)
    ids = np.ascontiguousarray(topk_ids, np.int32)
    _check(lib().oracle_permute(T, n_routed, k, n_shared, _p(ids), _p(offsets), _p(np.ascontiguousarray(row_token)),
                                _p(token_row)), "permute")
    return offsets, row_token, token_row


def quant_rows_i8(v: np.ndarray):
    """Per-row symmetric int8: -> (q int8, scale float32 [rows])."""
    v = np.ascontiguousarray(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().oracle_quant_rows_i8(rows, cols, _p(v), _p(q), _p(s))
    return q, s


def _wargs(fmt: str, w, scale, mn):
    arrs = [np.ascontiguousarray(a) if a is not None else None for a in (w, scale, mn)]
    return DT[fmt], arrs


def gate_up(x, offsets, row_token, inter, fmt, w, scale=None, mn=None, xq=None, xs=None, threads=None):
    """GLU output h float64 [R][I] of every permuted row (see moe_oracle.cpp, oracle_gu)."""
    G = offsets.shape[0] - 1
    R = int(offsets[-1])
    T, H = x.shape if x is not None else xq.shape
    h = np.zeros((R, inter), np.float64)
    wdt, (w, scale, mn) = _wargs(fmt, w, scale, mn)
    act = _act_dt(x) if x is not None else 0
    rc = lib().oracle_gu(T, H, inter, G, _p(offsets), _p(np.ascontiguousarray(row_token, np.int32)), act,
                         _p(x), _p(xq), _p(xs), wdt, _p(w), _p(scale), _p(mn), _p(h),
                         threads or default_threads())
    _check(rc, "gate_up")
    return h


def down(h, offsets, hidden, fmt, w, scale=None, mn=None, threads=None):
    """Down projection y float64 [R][H] of every permuted row."""
    G = offsets.shape[0] - 1
    R, inter = h.shape
    y = np.zeros((R, hidden), np.float64)
    wdt, (w, scale, mn) = _wargs(fmt, w, scale, mn)
    h = np.ascontiguousarray(h, np.float64)
    _check(lib().oracle_down(hidden, inter, G, _p(offsets), _p(h), wdt, _p(w), _p(scale), _p(mn), _p(y),
                             threads or default_threads()), "down")
    return y


def combine(y, token_row, topk_w, residual=None):
    """Gate-weighted sum over each token's rows (+ shared row, + residual), float64 [T][H]."""
    T, kS = token_row.shape
    k = topk_w.shape[1]
    S = kS - k
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    res = None if residual is None else np.ascontiguousarray(residual, np.float32)
    _check(lib().oracle_combine(T, H, k, S, _p(np.ascontiguousarray(token_row, np.int32)),
                                _p(np.ascontiguousarray(topk_w, np.float32)), _p(np.ascontiguousarray(y, np.float64)),
                                _p(res), _p(out)), "combine")
    return out


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    T, H = x.shape
    out = np.empty((T, H), np.float64)
    lib().oracle_rmsnorm(T, H, eps, _p(x), _p(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty_like(v)
    lib().oracle_round_bf16(v.size, _p(v), _p(out))
    return out


def q4_values(w, scale, mn) -> np.ndarray:
    G, N, K2 = w.shape
    out = np.empty((G, N, 2 * K2), np.float32)
    lib().oracle_q4_values(G, N, 2 * K2, _p(np.ascontiguousarray(w)), _p(np.ascontiguousarray(scale)),
                           _p(np.ascontiguousarray(mn)), _p(out))
    return out


def quant_mx8(v: np.ndarray):
    """MXFP8 (E4M3, E8M0 scale per 32) of rows: -> (codes uint8 [rows][cols], scale bytes uint8
    [rows][cols/32], values float64 [rows][cols])."""
    v = np.ascontiguousarray(v, np.float32)
    rows, cols = v.shape
    codes = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    deq = np.empty((rows, cols), np.float64)
    lib().oracle_quant_mx8(rows, cols, _p(v), _p(codes), _p(sc), _p(deq))
    return codes, sc, deq


def mx4_values(w, scales) -> np.ndarray:
    G, N, K2 = w.shape
    out = np.empty((G, N, 2 * K2), np.float64)
    lib().oracle_mx4_values(G, N, 2 * K2, _p(np.ascontiguousarray(w)), _p(np.ascontiguousarray(scales)), _p(out))
    return out


def quantize_x(spec, x):
    """int8 activations of the int8 path: x (bf16 bits or fp32) -> per-token (xq, xs)."""
    xf = bf16_to_f32(x) if x.dtype == np.uint16 else x
    return quant_rows_i8(xf)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer(d: dict, threads=None, residual=None, with_steps=False):
    """Whole layer for the inputs dict of gen.synth.layer_inputs; float64 output [T][H].

    Steps in order: route -> permute -> (int8: quantise x) -> gate/up + GLU -> down -> combine.
    """
    spec = d["spec"]
    x = d["x"]
    logits, ids, w = route(x, d["w_router"], spec.top_k, d.get("bias"))
    offsets, row_token, token_row = permute(ids, spec.n_routed, spec.n_shared)
    xq = xs = None
    if spec.wt == "i8":
        xq, xs = quantize_x(spec, x)
        h = gate_up(None, offsets, row_token, spec.inter, "i8", d["w_gu"], d["w_gu_scale"], xq=xq, xs=xs,
                    threads=threads)
    else:
        h = gate_up(x, offsets, row_token, spec.inter, spec.wt, d["w_gu"], d["w_gu_scale"], d["w_gu_min"],
                    threads=threads)
    y = down(h, offsets, spec.hidden, spec.wt, d["w_down"], d["w_down_scale"], d["w_down_min"], threads=threads)
    out = combine(y, token_row, w, residual)
    if with_steps:
        return out, dict(logits=logits, ids=ids, w=w, offsets=offsets, row_token=row_token, token_row=token_row,
                         xq=xq, xs=xs, h=h, y=y)
    return out


def stack_layer(d: dict, x: np.ndarray, eps: float, threads=None, with_steps=False):
    """One layer of the stacked workload on the fp32 residual stream x [T][H]:

        xn     = bf16_rne(x / sqrt(mean(x^2) + eps))       (RMSNorm, unit gain)
        x_next = fp32(x + MoE(xn))                          (residual added in the combine)

    d holds the layer's weights (gen.synth.layer_weights); its "x" is ignored.
    The normalised input is rounded once from fp64 to bf16 (the layer's
    activation format); the MoE output and the residual are summed in fp64
    inside the combine and rounded once to fp32, the residual stream's format.
    Returns x_next (float32), and with with_steps also a dict with the bf16
    input bits, the fp64 MoE output (without residual) and the layer's steps.
    """
    x = np.ascontiguousarray(x, np.float32)
    xn = round_bf16(rmsnorm(x, eps)).astype(np.float32)
    xn_bits = (xn.view(np.uint32) >> 16).astype(np.uint16)
    dl = dict(d)
    dl["x"] = xn_bits
    out, st = layer(dl, threads=threads, residual=x, with_steps=True)
    x_next = out.astype(np.float32)
    if with_steps:
        moe_out = combine(st["y"], st["token_row"], st["w"])
        return x_next, dict(st, xn=xn_bits, moe=moe_out)
    return x_next


def stack_forward(layers: list, x: np.ndarray, eps: float, threads=None):
    """x_{l+1} = x_l + MoE_l(RMSNorm(x_l)) over every layer of `layers` (weight dicts)."""
    for d in layers:
        x = stack_layer(d, x, eps, threads=threads)
    return x
