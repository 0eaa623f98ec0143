"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
run the library's entry points step by step, read buffers back, and compare
with tolerance.  No arithmetic of the layer lives here."""
from __future__ import annotations

import numpy as np

from gen.synth import LayerSpec

TOL_BF16 = dict(max_rel=2e-2, rmse=5e-3)   # bf16 / 4-bit outputs vs the fp64 oracle
TOL_F32 = dict(max_rel=1e-4, rmse=2e-6)    # fp32 path (MFMA fp32 accumulation over K <= 2048)
# The scaled FP4 x FP8 MFMA forms exact products, adds them in groups of 8
# consecutive K aligned to the group's largest product with the bits below
# about 2^-14 of it dropped (measured on gfx950: an addend under that
# threshold next to a large product vanishes, the same addend alone is kept),
# then adds the group sums in fp32.  Seven dropped remainders per group stay
# under 2^-11 of the group's largest |product|, so a dot product is within
# MX_ACC * sum_k |a_k w_k| of the exact one.
MX_ACC = 2.0 ** -11


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


def assert_within(got, ref, bound, what=""):
    """|got - ref| <= bound element by element."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError("%s: %d of %d elements beyond the bound; worst at %s: got %.9g ref %.9g bound %.3g"
                             % (what, int(bad.sum()), bad.size, i, got[i], ref[i], bound[i]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def mx_gu_bound(d: dict, offsets, row_token) -> np.ndarray:
    """Bound on |h_gpu - h_oracle| for MXFP4 gate/up: the MFMA bound on g and u
    (MX_ACC * sum |products|) carried through h = silu(g) u (|silu'| <= 1.1),
    plus 1e-6 |h| for the fp32 rounding and the fast exp of SiLU."""
    from oracle import oracle
    I = d["spec"].inter
    xq = oracle.quant_mx8(bf16_to_f64(d["x"]).astype(np.float32))[2]
    W = oracle.mx4_values(d["w_gu"], d["w_gu_scale"])
    bound = np.zeros((int(offsets[-1]), I))
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 == r0:
            continue
        a = xq[row_token[r0:r1]]
        gu = a @ W[g].T
        s = np.abs(a) @ np.abs(W[g]).T
        gg, uu = gu[:, :I], gu[:, I:]
        dg, du = MX_ACC * s[:, :I], MX_ACC * s[:, I:]
        silu = gg / (1.0 + np.exp(-gg))
        bound[r0:r1] = 1.1 * dg * (np.abs(uu) + du) + np.abs(silu) * du + 1e-6 * np.abs(silu * uu)
    return bound


def mx_down_bound(d: dict, offsets, h_in: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Bound on |y_gpu - y_oracle| for MXFP4 down fed the fp32 rows h_in (both
    sides quantise them to the same MXFP8 codes)."""
    from oracle import oracle
    hq = oracle.quant_mx8(np.asarray(h_in, np.float32))[2]
    W = oracle.mx4_values(d["w_down"], d["w_down_scale"])
    bound = np.zeros_like(y_ref)
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            bound[r0:r1] = MX_ACC * (np.abs(hq[r0:r1]) @ np.abs(W[g]).T)
    return bound + 1e-6 * np.abs(y_ref)


def tol_for(spec: LayerSpec):
    return TOL_F32 if spec.wt == "f32" else TOL_BF16


def h_dtype(spec):
    return np.float32 if spec.wt in ("f32", "i8", "mx4") else np.uint16


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
