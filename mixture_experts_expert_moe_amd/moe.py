"""ctypes binding of libmoe_gfx950.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the shared library.  PyTorch provides device memory (tensors) and the stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_gfx950.so")

MOE_F32, MOE_BF16, MOE_I8, MOE_Q4B32, MOE_MXFP4 = 0, 1, 2, 3, 4
DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16, "i8": MOE_I8, "q4": MOE_Q4B32, "mx4": MOE_MXFP4}
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_BUFFER_TOO_SMALL",
          -4: "MOE_ERR_HIP"}

# The C-ABI entry points declared in include/moe.h.
EXPORTS = ("moe_buffer_sizes", "moe_route_topk", "moe_permute", "moe_route_permute", "moe_grouped_gemm_gu",
           "moe_grouped_gemm_down", "moe_combine", "moe_combine_rmsnorm", "moe_rmsnorm", "moe_quant_mx8",
           "moe_decode_layer",
           "moe_decode_layer_static", "moe_status_string", "moe_abi_version")


class MoeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "inter", "n_routed", "top_k", "n_shared", "max_tokens",
                                              "act_dtype", "w_dtype", "out_dtype")]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("min", ctypes.c_void_p)]


BUFFER_NAMES = ("logits", "topk_ids", "topk_w", "expert_offsets", "row_token", "token_row", "sched", "x_q",
                "x_scale", "h", "y", "h_q", "h_scale", "sync")
# Word of the sync buffer that a timed-out grid barrier of moe_decode_layer sets.
SYNC_STATUS_WORD = 640


class MoeBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFER_NAMES]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s returned %s (%d)" % (fn, STATUS.get(status, "?"), status))
        self.status = status


_lib = None


def lib():
    """Load the built library (no build here: call build() first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe_gfx950.so is not built; run python -m mixture_experts_expert_moe_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
        L.moe_buffer_sizes.argtypes = [P(MoeDesc), P(ctypes.c_size_t)]
        L.moe_route_topk.argtypes = [P(MoeDesc), i32, vp, vp, vp, P(MoeBuffers), vp]
        L.moe_permute.argtypes = [P(MoeDesc), i32, vp, P(MoeBuffers), vp]
        L.moe_route_permute.argtypes = [P(MoeDesc), i32, vp, vp, vp, P(MoeBuffers), vp]
        L.moe_grouped_gemm_gu.argtypes = [P(MoeDesc), i32, vp, P(MoeWeights), P(MoeBuffers), vp]
        L.moe_grouped_gemm_down.argtypes = [P(MoeDesc), i32, P(MoeWeights), P(MoeBuffers), vp]
        L.moe_combine.argtypes = [P(MoeDesc), i32, vp, vp, P(MoeBuffers), vp]
        L.moe_combine_rmsnorm.argtypes = [P(MoeDesc), i32, vp, ctypes.c_float, vp, vp, P(MoeBuffers), vp]
        L.moe_rmsnorm.argtypes = [i32, i32, ctypes.c_float, vp, vp, vp]
        L.moe_quant_mx8.argtypes = [ctypes.c_int64, i32, i32, vp, vp, vp, vp]
        L.moe_decode_layer.argtypes = [P(MoeDesc), i32, vp, vp, vp, P(MoeWeights), P(MoeWeights), vp, i32,
                                       ctypes.c_float, vp, P(MoeBuffers), vp]
        L.moe_decode_layer_static.argtypes = [P(MoeDesc), i32, vp, vp, vp, P(MoeWeights), P(MoeWeights), vp, i32,
                                              ctypes.c_float, vp, vp]
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_abi_version.restype = i32
        for f in ("moe_buffer_sizes", "moe_route_topk", "moe_permute", "moe_route_permute", "moe_grouped_gemm_gu",
                  "moe_grouped_gemm_down", "moe_combine", "moe_combine_rmsnorm", "moe_rmsnorm", "moe_decode_layer",
                  "moe_decode_layer_static"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Tensors must live on the GPU."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor, got one on %s" % t.device)
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_desc(hidden, inter, n_routed, top_k, n_shared, max_tokens, act="bf16", wt="bf16", out="bf16") -> MoeDesc:
    return MoeDesc(hidden, inter, n_routed, top_k, n_shared, max_tokens, DTYPE_CODE[act], DTYPE_CODE[wt],
                   DTYPE_CODE[out])


def moe_buffer_sizes(desc: MoeDesc):
    sizes = (ctypes.c_size_t * len(BUFFER_NAMES))()
    _check("moe_buffer_sizes", lib().moe_buffer_sizes(ctypes.byref(desc), sizes))
    return dict(zip(BUFFER_NAMES, (int(s) for s in sizes)))


def alloc_buffers(desc: MoeDesc, device="cuda"):
    """Caller-owned device buffers (torch uint8 tensors) and their MoeBuffers struct."""
    import torch
    tensors = {}
    for name, nbytes in moe_buffer_sizes(desc).items():
        make = torch.zeros if name == "sync" else torch.empty   # the barrier words start at zero
        tensors[name] = make(max(nbytes, 16), dtype=torch.uint8, device=device) if nbytes else None
    return tensors, buffers_struct(tensors)


def buffers_struct(tensors: dict) -> MoeBuffers:
    return MoeBuffers(*[_ptr(tensors.get(n)) for n in BUFFER_NAMES])


def weights_struct(w, scale=None, mn=None) -> MoeWeights:
    return MoeWeights(_ptr(w), _ptr(scale), _ptr(mn))


def moe_route_topk(desc, T, x, w_router, bias, bufs: MoeBuffers, stream=None):
    _check("moe_route_topk", lib().moe_route_topk(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                                  ctypes.byref(bufs), _stream(stream)))


def moe_permute(desc, T, x, bufs: MoeBuffers, stream=None):
    _check("moe_permute", lib().moe_permute(ctypes.byref(desc), T, _ptr(x), ctypes.byref(bufs), _stream(stream)))


def moe_route_permute(desc, T, x, w_router, bias, bufs: MoeBuffers, stream=None):
    _check("moe_route_permute", lib().moe_route_permute(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                                        ctypes.byref(bufs), _stream(stream)))


def moe_grouped_gemm_gu(desc, T, x, w_gu: MoeWeights, bufs: MoeBuffers, stream=None):
    _check("moe_grouped_gemm_gu", lib().moe_grouped_gemm_gu(ctypes.byref(desc), T, _ptr(x), ctypes.byref(w_gu),
                                                            ctypes.byref(bufs), _stream(stream)))


def moe_grouped_gemm_down(desc, T, w_down: MoeWeights, bufs: MoeBuffers, stream=None):
    _check("moe_grouped_gemm_down", lib().moe_grouped_gemm_down(ctypes.byref(desc), T, ctypes.byref(w_down),
                                                                ctypes.byref(bufs), _stream(stream)))


def moe_combine(desc, T, residual, out, bufs: MoeBuffers, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(desc), T, _ptr(residual), _ptr(out), ctypes.byref(bufs),
                                            _stream(stream)))


def moe_combine_rmsnorm(desc, T, residual, eps, out, xn, bufs: MoeBuffers, stream=None):
    _check("moe_combine_rmsnorm", lib().moe_combine_rmsnorm(ctypes.byref(desc), T, _ptr(residual), eps, _ptr(out),
                                                            _ptr(xn), ctypes.byref(bufs), _stream(stream)))


MOE_DECODE_NORM_INPUT = 1


def moe_decode_layer(desc, T, x, w_router, bias, w_gu: MoeWeights, w_down: MoeWeights, residual, flags, eps, out,
                     bufs: MoeBuffers, stream=None):
    _check("moe_decode_layer", lib().moe_decode_layer(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                                      ctypes.byref(w_gu), ctypes.byref(w_down), _ptr(residual),
                                                      flags, eps, _ptr(out), ctypes.byref(bufs), _stream(stream)))


def moe_decode_layer_static(desc, T, x, w_router, bias, w_gu: MoeWeights, w_down: MoeWeights, residual, flags, eps,
                            out, stream=None):
    _check("moe_decode_layer_static",
           lib().moe_decode_layer_static(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(w_gu),
                                         ctypes.byref(w_down), _ptr(residual), flags, eps, _ptr(out),
                                         _stream(stream)))


def sync_status(tensors: dict) -> int:
    """Status word of a layer's sync buffer (nonzero: a grid barrier timed out)."""
    import torch
    return int(tensors["sync"].view(torch.int32)[SYNC_STATUS_WORD].item())


def moe_rmsnorm(T, H, eps, x, xn, stream=None):
    _check("moe_rmsnorm", lib().moe_rmsnorm(T, H, eps, _ptr(x), _ptr(xn), _stream(stream)))


def moe_quant_mx8(rows, cols, src_dtype, src, codes, scales, stream=None):
    """MXFP8 of rows x cols values (src_dtype "f32" or "bf16") into E4M3 codes and E8M0 scales."""
    _check("moe_quant_mx8", lib().moe_quant_mx8(rows, cols, DTYPE_CODE[src_dtype], _ptr(src), _ptr(codes),
                                                _ptr(scales), _stream(stream)))


class MoeLayer:
    """One routed MoE layer: a desc, its device buffers and its device weights.

    weights: dict with "w_router", optional "bias", and "w_gu", "w_gu_scale",
    "w_gu_min", "w_down", "w_down_scale", "w_down_min" as device tensors in the
    formats of include/moe.h (None where a format has no such part).
    """

    def __init__(self, desc: MoeDesc, weights: dict, device="cuda"):
        self.desc = desc
        self.tensors, self.bufs = alloc_buffers(desc, device)
        self.w = weights
        self.gu = weights_struct(weights["w_gu"], weights.get("w_gu_scale"), weights.get("w_gu_min"))
        self.dn = weights_struct(weights["w_down"], weights.get("w_down_scale"), weights.get("w_down_min"))

    def set_weights(self, weights: dict):
        self.w = weights
        self.gu = weights_struct(weights["w_gu"], weights.get("w_gu_scale"), weights.get("w_gu_min"))
        self.dn = weights_struct(weights["w_down"], weights.get("w_down_scale"), weights.get("w_down_min"))

    def forward(self, x, out, residual=None, stream=None):
        """The five calls of the layer on one stream; out receives [T][H]."""
        T = x.shape[0]
        d = self.desc
        moe_route_permute(d, T, x, self.w["w_router"], self.w.get("bias"), self.bufs, stream)
        moe_grouped_gemm_gu(d, T, x, self.gu, self.bufs, stream)
        moe_grouped_gemm_down(d, T, self.dn, self.bufs, stream)
        moe_combine(d, T, residual, out, self.bufs, stream)
        return out

    def forward_decode(self, x, out, residual=None, norm_input=False, eps=1e-6, stream=None):
        """The whole layer in one launch (moe_decode_layer, T <= 16); same results as forward().
        norm_input: x is the fp32 residual stream and out = x + MoE(RMSNorm(x))."""
        moe_decode_layer(self.desc, x.shape[0], x, self.w["w_router"], self.w.get("bias"), self.gu, self.dn, residual,
                         MOE_DECODE_NORM_INPUT if norm_input else 0, eps, out, self.bufs, stream)
        return out

    def view(self, name, dtype, shape):
        """Typed view of one of the layer's buffers (for inspection)."""
        import math
        t = self.tensors[name]
        n = math.prod(shape)
        return t.view(dtype)[:n].view(*shape)


class MoeStack:
    """Layers of `MoeLayer` with RMSNorm before each and an fp32 residual stream:
    x_{l+1} = x_l + MoE_l(RMSNorm(x_l)).  One shared set of buffers; per-layer
    weights.  x is [T][H] fp32 on the device and is updated in place (ping-pong
    through a second buffer)."""

    def __init__(self, desc: MoeDesc, layer_weights: list, eps: float = 1e-6, device="cuda"):
        import torch
        self.desc = desc
        self.eps = eps
        self.layers = layer_weights
        self.tensors, self.bufs = alloc_buffers(desc, device)
        self.gu = [weights_struct(w["w_gu"], w.get("w_gu_scale"), w.get("w_gu_min")) for w in layer_weights]
        self.dn = [weights_struct(w["w_down"], w.get("w_down_scale"), w.get("w_down_min")) for w in layer_weights]
        M, H = desc.max_tokens, desc.hidden
        self.xn = torch.empty((M, H), dtype=torch.bfloat16, device=device)
        self.tmp = torch.empty((M, H), dtype=torch.float32, device=device)

    def layer(self, l, x, out, T, stream=None):
        """One layer on the first T rows: out = x + MoE_l(RMSNorm(x))."""
        d, b, w = self.desc, self.bufs, self.layers[l]
        xn = self.xn[:T]
        moe_rmsnorm(T, d.hidden, self.eps, x, xn, stream)
        moe_route_permute(d, T, xn, w["w_router"], w.get("bias"), b, stream)
        moe_grouped_gemm_gu(d, T, xn, self.gu[l], b, stream)
        moe_grouped_gemm_down(d, T, self.dn[l], b, stream)
        moe_combine(d, T, x, out, b, stream)

    def forward(self, x, stream=None):
        """All layers on x ([T][H] fp32, T <= max_tokens); returns the tensor holding the result.
        The RMSNorm of every layer after the first comes out of the previous
        layer's combine (moe_combine_rmsnorm): the same bits as layer() gives,
        one launch fewer per layer."""
        T = x.shape[0]
        d, bf = self.desc, self.bufs
        xn = self.xn[:T]
        a, b = x, self.tmp[:T]
        moe_rmsnorm(T, d.hidden, self.eps, a, xn, stream)
        L = len(self.layers)
        for l in range(L):
            w = self.layers[l]
            moe_route_permute(d, T, xn, w["w_router"], w.get("bias"), bf, stream)
            moe_grouped_gemm_gu(d, T, xn, self.gu[l], bf, stream)
            moe_grouped_gemm_down(d, T, self.dn[l], bf, stream)
            if l + 1 < L:
                moe_combine_rmsnorm(d, T, a, self.eps, b, xn, bf, stream)
            else:
                moe_combine(d, T, a, b, bf, stream)
            a, b = b, a
        if a.data_ptr() != x.data_ptr():
            x.copy_(a)
        return x

    def forward_decode(self, x, stream=None):
        """As forward(), each layer in one launch (moe_decode_layer with the
        RMSNorm of the residual stream inside, x updated in place; T <= 16):
        the same bits, one launch per layer instead of four."""
        T = x.shape[0]
        d, bf = self.desc, self.bufs
        for l, w in enumerate(self.layers):
            moe_decode_layer(d, T, x, w["w_router"], w.get("bias"), self.gu[l], self.dn[l], None,
                             MOE_DECODE_NORM_INPUT, self.eps, x, bf, stream)
        return x
