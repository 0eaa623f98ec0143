"""Seeded synthetic inputs for the routed MoE FFN layer (shared by the oracle
tests and the GPU harness).

Only random draws and storage formats live here; the layer's arithmetic does
not.  Every tensor comes from its own SplitMix64 stream whose key is derived
from (base seed, workload, layer, tensor, rotation), so any tensor can be
regenerated alone and two tensors never share draws.

Workloads follow the problem the pages describe: hidden 2048, expert
intermediate 512, gate/up 2048x512 and down 512x2048 per expert ("MoE Decode
Partition and Submit Floor", section 3, Test 1), top-8 routed plus one shared
expert ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM", The fix),
prompts read in 256-token chunks (OpenFlowLM-Next issue #74, Reading).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.cpp")
_LIB = os.path.join(_HERE, "libsynth.so")

BASE_SEED = 0x5EED2026

TENSOR_X, TENSOR_ROUTER, TENSOR_BIAS, TENSOR_W_GU, TENSOR_W_DOWN = 1, 2, 3, 4, 5


def build(force: bool = True) -> str:
    """Compile gen/libsynth.so with g++ (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                               "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i32, i64, f32, p = ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.synth_mix.restype = u64
        L.synth_mix.argtypes = [u64, u64]
        L.synth_normal_f32.argtypes = [u64, i64, f32, f32, p, ctypes.c_int]
        L.synth_normal_bf16.argtypes = [u64, i64, f32, f32, p, ctypes.c_int]
        L.synth_weights_f32.argtypes = [u64, i32, i32, i32, f32, p, ctypes.c_int]
        L.synth_weights_bf16.argtypes = [u64, i32, i32, i32, f32, p, ctypes.c_int]
        L.synth_weights_i8.argtypes = [u64, i32, i32, i32, f32, p, p, ctypes.c_int]
        L.synth_weights_q4.argtypes = [u64, i32, i32, i32, f32, p, p, p, ctypes.c_int]
        L.synth_weights_mx4.argtypes = [u64, i32, i32, i32, f32, p, p, ctypes.c_int]
        L.synth_permutation.argtypes = [u64, i32, p]
        L.synth_zipf_bias.argtypes = [u64, i32, ctypes.c_double, p]
        _lib = L
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(*parts: int) -> int:
    """Stream key for (workload, layer, tensor, rotation, ...)."""
    L = lib()
    k = BASE_SEED
    for p in parts:
        k = L.synth_mix(k, int(p) & 0xFFFFFFFFFFFFFFFF)
    return int(k)


def normal(k: int, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """N(0, std) draws; dtype "f32" -> float32 array, "bf16" -> uint16 bf16 bits."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, np.float32)
        lib().synth_normal_f32(k, n, 0.0, std, _ptr(out), _threads())
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        lib().synth_normal_bf16(k, n, 0.0, std, _ptr(out), _threads())
    else:
        raise ValueError(dtype)
    return out


def weights(k: int, G: int, n: int, kdim: int, std: float, fmt: str) -> dict:
    """G expert matrices [n][kdim] (K contiguous) of N(0, std) in a storage format.

    fmt "f32": {"w": float32}; "bf16": {"w": uint16 bits}; "i8": {"w": int8, "scale": float32 [G][n]};
    "q4": {"w": uint8 [G][n][kdim/2], "scale": uint16 fp16 [G][n][kdim/32], "min": same};
    "mx4": {"w": uint8 [G][n][kdim/2] E2M1 pairs, "scale": uint8 E8M0 [G][n][kdim/32]}.
    """
    L, t = lib(), _threads()
    if fmt == "f32":
        w = np.empty((G, n, kdim), np.float32)
        L.synth_weights_f32(k, G, n, kdim, std, _ptr(w), t)
        return {"w": w}
    if fmt == "bf16":
        w = np.empty((G, n, kdim), np.uint16)
        L.synth_weights_bf16(k, G, n, kdim, std, _ptr(w), t)
        return {"w": w}
    if fmt == "i8":
        w = np.empty((G, n, kdim), np.int8)
        s = np.empty((G, n), np.float32)
        L.synth_weights_i8(k, G, n, kdim, std, _ptr(w), _ptr(s), t)
        return {"w": w, "scale": s}
    if fmt == "q4":
        if kdim % 32:
            raise ValueError("4-bit blocks need K % 32 == 0")
        w = np.empty((G, n, kdim // 2), np.uint8)
        s = np.empty((G, n, kdim // 32), np.uint16)
        m = np.empty((G, n, kdim // 32), np.uint16)
        L.synth_weights_q4(k, G, n, kdim, std, _ptr(w), _ptr(s), _ptr(m), t)
        return {"w": w, "scale": s, "min": m}
    if fmt == "mx4":
        if kdim % 32:
            raise ValueError("MXFP4 blocks need K % 32 == 0")
        w = np.empty((G, n, kdim // 2), np.uint8)
        s = np.empty((G, n, kdim // 32), np.uint8)
        L.synth_weights_mx4(k, G, n, kdim, std, _ptr(w), _ptr(s), t)
        return {"w": w, "scale": s}
    raise ValueError(fmt)


def zipf_bias(k: int, n: int, s: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_zipf_bias(k, n, s, _ptr(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, n, _ptr(out))
    return out


@dataclass(frozen=True)
class LayerSpec:
    """Shape and storage formats of one routed MoE FFN layer."""
    hidden: int = 2048
    inter: int = 512
    n_routed: int = 128
    top_k: int = 8
    n_shared: int = 1
    act: str = "bf16"      # x and router weight: "f32" | "bf16"
    wt: str = "bf16"       # expert weights: "f32" | "bf16" | "i8" | "q4" | "mx4"
    out: str = "bf16"      # layer output: "f32" | "bf16"
    zipf: float = 0.0      # Zipf exponent of the per-expert router bias; 0 = no bias
    w_std: float = 0.02

    @property
    def groups(self) -> int:
        return self.n_routed + self.n_shared


@dataclass(frozen=True)
class Workload:
    name: str
    spec: LayerSpec
    tokens: tuple
    layers: int = 1
    notes: str = ""
    extra: dict = field(default_factory=dict)


# Workload ids feed the stream keys; they never change once used.
WORKLOADS = {
    "fp32_e16_top2": (1, Workload("fp32_e16_top2",
                                  LayerSpec(n_routed=16, top_k=2, n_shared=0, act="f32", wt="f32", out="f32"),
                                  tokens=(16,), notes="fp32 layer, 16 experts, top-2, no shared expert")),
    "bf16_e128_top8_shared": (2, Workload("bf16_e128_top8_shared", LayerSpec(), tokens=(256,),
                                          notes="bf16 prefill chunk of 256 tokens, uniform routing")),
    "int8_e128_top8_shared": (3, Workload("int8_e128_top8_shared", LayerSpec(wt="i8"), tokens=(1, 2, 4, 8),
                                          notes="int8 decode, per-channel weight scales, per-token activation scales")),
    "q4_e128_top8_shared_zipf": (4, Workload("q4_e128_top8_shared_zipf", LayerSpec(wt="q4", zipf=1.1), tokens=(2048,),
                                             notes="4-bit block weights, Zipf(1.1) router bias, 2048-token prefill")),
    "q4_stack40": (5, Workload("q4_stack40", LayerSpec(wt="q4", out="f32"), tokens=(256, 1), layers=40,
                               notes="40 MoE layers with RMSNorm and residual; 2600-token prompt in 256-token chunks, "
                                     "then 64 single-token decode steps",
                               extra={"prompt": 2600, "chunk": 256, "decode_steps": 64, "eps": 1e-6})),
    "mx4_e128_top8_shared_zipf": (6, Workload("mx4_e128_top8_shared_zipf", LayerSpec(wt="mx4", zipf=1.1),
                                              tokens=(2048,),
                                              notes="MXFP4 expert weights with MXFP8 activations, Zipf(1.1) router "
                                                    "bias, 2048-token prefill")),
    "mx4_e128_top8_shared": (7, Workload("mx4_e128_top8_shared", LayerSpec(wt="mx4"), tokens=(1, 2, 4, 8, 256),
                                         notes="MXFP4 expert weights with MXFP8 activations, decode rows and a "
                                               "256-token chunk")),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name][1]


def workload_id(name: str) -> int:
    return WORKLOADS[name][0]


def layer_weights(spec: LayerSpec, wid: int, layer: int = 0, rotation: int = 0) -> dict:
    """Router (+ optional bias) and expert weights of one layer."""
    H, I, E, G = spec.hidden, spec.inter, spec.n_routed, spec.groups
    out = {
        "w_router": normal(key(wid, layer, TENSOR_ROUTER, rotation), (E, H), spec.w_std, spec.act),
        "bias": zipf_bias(key(wid, layer, TENSOR_BIAS, rotation), E, spec.zipf) if spec.zipf else None,
    }
    gu = weights(key(wid, layer, TENSOR_W_GU, rotation), G, 2 * I, H, spec.w_std, spec.wt)
    dn = weights(key(wid, layer, TENSOR_W_DOWN, rotation), G, H, I, spec.w_std, spec.wt)
    for name, d in (("gu", gu), ("down", dn)):
        out["w_" + name] = d["w"]
        out["w_%s_scale" % name] = d.get("scale")
        out["w_%s_min" % name] = d.get("min")
    return out


def tokens(spec: LayerSpec, wid: int, T: int, stream: int = 0, dtype: str | None = None) -> np.ndarray:
    """T token vectors x ~ N(0, 1) in the layer's activation format (or `dtype`)."""
    return normal(key(wid, stream, TENSOR_X), (T, spec.hidden), 1.0, dtype or spec.act)


def layer_inputs(name: str, T: int, layer: int = 0, rotation: int = 0, stream: int = 0) -> dict:
    wid = workload_id(name)
    spec = workload(name).spec
    d = layer_weights(spec, wid, layer, rotation)
    d["x"] = tokens(spec, wid, T, stream)
    d["spec"] = spec
    return d
