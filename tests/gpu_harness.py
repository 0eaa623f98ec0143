"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
run the library's entry points step by step, read buffers back, and compare
with tolerance.  No arithmetic of the layer lives here."""
from __future__ import annotations

import numpy as np

from gen.synth import LayerSpec

TOL_BF16 = dict(max_rel=2e-2, rmse=5e-3)   # bf16 / 4-bit outputs vs the fp64 oracle
TOL_F32 = dict(max_rel=1e-4, rmse=2e-6)    # fp32 path (MFMA fp32 accumulation over K <= 2048)


def torch_mod():
    import torch
    return torch


def to_dev(a):
    """numpy -> contiguous device tensor with the same bytes (uint16 travels as int16)."""
    torch = torch_mod()
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def desc_for(spec: LayerSpec, max_tokens: int):
    from mixture_experts_expert_moe_amd import moe
    return moe.make_desc(spec.hidden, spec.inter, spec.n_routed, spec.top_k, spec.n_shared, max_tokens,
                         act=spec.act, wt=spec.wt, out=spec.out)


def dev_weights(d: dict) -> dict:
    keys = ("w_router", "bias", "w_gu", "w_gu_scale", "w_gu_min", "w_down", "w_down_scale", "w_down_min")
    return {k: to_dev(d.get(k)) for k in keys}


def buf(layer, name, dtype, shape):
    """Copy of one device buffer as numpy."""
    n = int(np.prod(shape))
    raw = layer.tensors[name].cpu().numpy()
    return raw.view(dtype)[:n].reshape(shape).copy()


def put(layer, name, arr):
    """Overwrite the start of a device buffer with the bytes of arr."""
    torch = torch_mod()
    b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
    layer.tensors[name][:b.size].copy_(torch.from_numpy(b).to("cuda"))


def bf16_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16)


def bf16_to_f64(u16) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Oracle value rounded to the bf16 the GPU stores (via the oracle's own rounding)."""
    from oracle import oracle
    r = oracle.round_bf16(np.asarray(v, np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    scale = np.abs(ref).max() if ref.size else 0.0
    max_rel = float(np.abs(diff).max() / scale) if scale > 0 else float(np.abs(diff).max() if diff.size else 0.0)
    rmse = float(np.sqrt(np.mean(diff ** 2))) if diff.size else 0.0
    return max_rel, rmse


def assert_close(got, ref, max_rel, rmse, what=""):
    mr, rm = errors(got, ref)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    assert mr <= max_rel and rm <= rmse, "%s: max_rel %.3g (bar %.3g), rmse %.3g (bar %.3g)" % (what, mr, max_rel, rm,
                                                                                               rmse)
    return mr, rm


def tol_for(spec: LayerSpec):
    return TOL_F32 if spec.wt == "f32" else TOL_BF16


def h_dtype(spec):
    return np.float32 if spec.wt in ("f32", "i8") else np.uint16


def decode(arr, dt):
    return bf16_to_f64(arr) if dt == np.uint16 else arr.astype(np.float64)


class GpuLayer:
    """A MoeLayer over seeded inputs, with step-by-step access."""

    def __init__(self, d: dict, max_tokens: int | None = None):
        from mixture_experts_expert_moe_amd import moe
        self.d = d
        self.spec = d["spec"]
        self.T = d["x"].shape[0]
        self.max_tokens = max_tokens or max(self.T, 1)
        self.desc = desc_for(self.spec, self.max_tokens)
        self.layer = moe.MoeLayer(self.desc, dev_weights(d))
        self.x = to_dev(d["x"])
        torch = torch_mod()
        odt = torch.float32 if self.spec.out == "f32" else torch.int16
        self.out = torch.zeros((max(self.T, 1), self.spec.hidden), dtype=odt, device="cuda")

    # -- steps ------------------------------------------------------------------
    def route(self, T=None):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_route_topk(self.desc, self.T if T is None else T, self.x, self.layer.w["w_router"],
                           self.layer.w.get("bias"), self.layer.bufs)

    def permute(self):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_permute(self.desc, self.T, self.x, self.layer.bufs)

    def route_permute(self):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_route_permute(self.desc, self.T, self.x, self.layer.w["w_router"], self.layer.w.get("bias"),
                              self.layer.bufs)

    def gate_up(self):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_grouped_gemm_gu(self.desc, self.T, self.x, self.layer.gu, self.layer.bufs)

    def down(self):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_grouped_gemm_down(self.desc, self.T, self.layer.dn, self.layer.bufs)

    def combine(self, residual=None):
        from mixture_experts_expert_moe_amd import moe
        moe.moe_combine(self.desc, self.T, residual, self.out, self.layer.bufs)

    def run(self, residual=None):
        self.route()
        self.permute()
        self.gate_up()
        self.down()
        self.combine(residual)
        torch_mod().cuda.synchronize()

    # -- reads ------------------------------------------------------------------
    @property
    def R(self):
        return self.T * (self.spec.top_k + self.spec.n_shared)

    def logits(self):
        return buf(self.layer, "logits", np.float32, (self.T, self.spec.n_routed))

    def ids(self):
        return buf(self.layer, "topk_ids", np.int32, (self.T, self.spec.top_k))

    def gates(self):
        return buf(self.layer, "topk_w", np.float32, (self.T, self.spec.top_k))

    def offsets(self):
        return buf(self.layer, "expert_offsets", np.int32, (self.spec.groups + 1,))

    def row_token(self):
        return buf(self.layer, "row_token", np.int32, (self.R,))

    def token_row(self):
        return buf(self.layer, "token_row", np.int32, (self.T, self.spec.top_k + self.spec.n_shared))

    def sched(self):
        """(header, small tiles [n][4], big tiles [m][4]) of the tile schedule."""
        head = buf(self.layer, "sched", np.int32, (32,))
        n_small, n_big, big_start = int(head[0]), int(head[3]), int(head[4])
        s = buf(self.layer, "sched", np.int32, (max(32 + 4 * n_small, big_start + 4 * n_big),))
        return head, s[32:32 + 4 * n_small].reshape(n_small, 4), s[big_start:big_start + 4 * n_big].reshape(n_big, 4)

    def h(self):
        dt = h_dtype(self.spec)
        return decode(buf(self.layer, "h", dt, (self.R, self.spec.inter)), dt)

    def h_raw(self):
        return buf(self.layer, "h", h_dtype(self.spec), (self.R, self.spec.inter))

    def y(self):
        dt = h_dtype(self.spec)
        return decode(buf(self.layer, "y", dt, (self.R, self.spec.hidden)), dt)

    def y_raw(self):
        return buf(self.layer, "y", h_dtype(self.spec), (self.R, self.spec.hidden))

    def output(self):
        o = self.out[:self.T].cpu().numpy()
        return bf16_to_f64(o.view(np.uint16)) if self.spec.out == "bf16" else o.astype(np.float64)
