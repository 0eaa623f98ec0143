#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

Default workload: bf16 prefill chunk, hidden 2048, 128 routed experts
(gate/up 2048x512, down 512x2048) top-8 plus one shared expert, T = 256
tokens.  A step is one pass of the whole layer (route, permute, grouped
gate/up + SwiGLU, grouped down, combine) over one batch of fresh synthetic
tokens, inputs already resident in HBM.  Weight sets rotate every step so the
256 MB MALL cannot serve repeated weight reads.

Prints ONE JSON line: tokens/s per layer, the gate/up kernel against the HBM
roofline, the int8 T = 8 decode layer as a secondary figure, and the CPU
oracle timed on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 (the rate of the FP4 x FP8 scaled MFMA, set by its FP8 operand)
METRIC = "routed tokens/s per MoE layer (T=256 prefill, T=8 decode); % MFMA / HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(spec, n, k):
    """Bytes of one group's [n][k] weight matrix in its storage format (with scales)."""
    if spec.wt == "f32":
        return n * k * 4
    if spec.wt == "bf16":
        return n * k * 2
    if spec.wt == "i8":
        return n * k + n * 4
    if spec.wt == "mx4":
        return n * k // 2 + n * k // 32
    return n * k // 2 + 2 * (n * k // 32) * 2


def act_bytes(spec):
    return 4 if spec.act == "f32" else 2


def gu_algorithmic_bytes(spec, T, U):
    """Gate/up launch: weights of the U touched groups, tokens read once, h written once."""
    R = T * (spec.top_k + spec.n_shared)
    if spec.wt == "mx4":
        xb = T * spec.hidden + T * spec.hidden // 32  # E4M3 codes + E8M0 scales
    else:
        xb = T * spec.hidden * (1 if spec.wt == "i8" else act_bytes(spec)) + (T * 4 if spec.wt == "i8" else 0)
    hb = R * spec.inter * (4 if spec.wt in ("f32", "i8", "mx4") else 2)
    return U * weight_bytes(spec, 2 * spec.inter, spec.hidden) + xb + hb


def down_algorithmic_bytes(spec, T, U):
    R = T * (spec.top_k + spec.n_shared)
    if spec.wt == "mx4":
        ib = R * spec.inter + R * spec.inter // 32
    else:
        ib = R * spec.inter * (1 if spec.wt == "i8" else (4 if spec.wt == "f32" else 2))
    yb = R * spec.hidden * (4 if spec.wt in ("f32", "i8", "mx4") else 2)
    return U * weight_bytes(spec, spec.hidden, spec.inter) + ib + yb


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, launch_algo_bytes):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(rec.get("sources", [])):
        return None
    return rec.get("hbm_bytes_per_launch")


def synth_spec(name):
    from gen import synth
    return synth.workload(name).spec


class Runner:
    """Device-resident inputs of one workload and its MoeLayer."""

    def __init__(self, name, T, rotations, n_batches, fused=False):
        import torch
        from gen import synth
        from mixture_experts_expert_moe_amd import moe
        from tests import gpu_harness as gh

        self.torch, self.moe = torch, moe
        self.name, self.T, self.fused = name, T, fused
        wid = synth.workload_id(name)
        self.spec = spec = synth.workload(name).spec
        t0 = time.time()
        self.wsets = []
        for r in range(rotations):
            host = synth.layer_weights(spec, wid, 0, r)
            self.wsets.append(gh.dev_weights(host))
            del host
        self.x = [gh.to_dev(synth.tokens(spec, wid, T, stream=1000 + i)) for i in range(n_batches)]
        log("[bench] %s: %d weight sets + %d token batches generated and uploaded in %.1f s"
            % (name, rotations, n_batches, time.time() - t0))
        self.desc = gh.desc_for(spec, T)
        self.layer = moe.MoeLayer(self.desc, self.wsets[0])
        self.structs = [(moe.weights_struct(w["w_gu"], w["w_gu_scale"], w["w_gu_min"]),
                         moe.weights_struct(w["w_down"], w["w_down_scale"], w["w_down_min"])) for w in self.wsets]
        odt = torch.float32 if spec.out == "f32" else torch.bfloat16
        self.out = torch.empty((T, spec.hidden), dtype=odt, device="cuda")

    def step(self, i, ev=None):
        """One layer: route + permute (one call), gate/up, down, combine.  ev:
        optional list of 5 events recorded around the launches (same stream as
        the kernels)."""
        moe, d, b, T = self.moe, self.desc, self.layer.bufs, self.T
        w = self.wsets[i % len(self.wsets)]
        gu, dn = self.structs[i % len(self.wsets)]
        x = self.x[i % len(self.x)]
        if self.fused:  # the whole layer in one launch
            if ev:
                ev[0].record()
            moe.moe_decode_layer(d, T, x, w["w_router"], w.get("bias"), gu, dn, None, 0, 1e-6, self.out, b)
            if ev:
                ev[1].record()
            return
        if ev:
            ev[0].record()
        moe.moe_route_permute(d, T, x, w["w_router"], w.get("bias"), b)
        if ev:
            ev[1].record()
        moe.moe_grouped_gemm_gu(d, T, x, gu, b)
        if ev:
            ev[2].record()
        moe.moe_grouped_gemm_down(d, T, dn, b)
        if ev:
            ev[3].record()
        moe.moe_combine(d, T, None, self.out, b)
        if ev:
            ev[4].record()

    def touched_groups(self):
        offs = self.layer.tensors["expert_offsets"][:4 * (self.spec.groups + 1)].view(self.torch.int32).cpu().numpy()
        return int((np.diff(offs) > 0).sum())

    def timed(self, steps, warmup, per_kernel=True):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)] if per_kernel else None
        # whole-step wall time without events first
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        U = self.touched_groups()
        kms = None
        if per_kernel:
            for i in range(steps):
                self.step(warmup + steps + i, evs[i])
            torch.cuda.synchronize()
            names = ["decode_layer"] if self.fused else ["route_permute", "gate_up", "down", "combine"]
            kms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                   for j, n in enumerate(names)}
        return wall, U, kms

    def graph_timed(self, replays):
        """Wall time per step of the same layer steps captured in one HIP graph
        (one step per weight set, each on its own token batch) and replayed:
        the layer without the host's launch gaps."""
        torch = self.torch
        n = len(self.wsets)
        for i in range(n):
            self.step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                self.step(i)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (replays * n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, T, sample_tokens, batches=3, one_thread_tokens=16):
    """The CPU oracle (as it stands) on a bounded sample of the workload:
    `batches` distinct token batches of `sample_tokens` tokens through one
    layer on every core of this process's CPU share, and one batch of
    `one_thread_tokens` tokens on one thread."""
    from gen import synth
    from oracle import oracle
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    threads = max(1, min(16, share))  # a one-GPU machine's CPU share is 16 cores
    inputs = [synth.layer_inputs(name, sample_tokens, stream=424242 + b) for b in range(batches)]
    t0 = time.perf_counter()
    for d in inputs:
        oracle.layer(d, threads=threads)
    dt = time.perf_counter() - t0
    d1 = synth.layer_inputs(name, one_thread_tokens, stream=434343)
    t1 = time.perf_counter()
    oracle.layer(d1, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": batches * sample_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "one_thread_value": one_thread_tokens / dt1,
            "host_logical_cpus": os.cpu_count(), "affinity_cpus": share, "cpu_model": cpu_model(),
            "compile_flags": "g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -pthread",
            "sample": "%d batches of %d tokens (of the %d-token workload %s), each through one whole layer "
                      "(routing, permutation, gate/up, down, combine), fp64 C++ oracle, %.1f s wall on %d threads; "
                      "one-thread figure: %d tokens in %.1f s"
                      % (batches, sample_tokens, T, name, dt, threads, one_thread_tokens, dt1)}


def stack_figures():
    """40 stacked 4-bit layers (RMSNorm + residual): a 2600-token prompt in
    256-token chunks, then 64 single-token decode steps, eager and replayed
    from one captured HIP graph per step."""
    import torch
    from gen import synth
    from mixture_experts_expert_moe_amd import moe
    from tests import gpu_harness as gh
    name = "q4_stack40"
    wl = synth.workload(name)
    spec, L, ex = wl.spec, wl.layers, wl.extra
    wid = synth.workload_id(name)
    t0 = time.time()
    dev = [gh.dev_weights(synth.layer_weights(spec, wid, l)) for l in range(L)]
    x0 = torch.from_numpy(synth.tokens(spec, wid, ex["prompt"], stream=0, dtype="f32")).to("cuda")
    dec = torch.from_numpy(np.concatenate([synth.tokens(spec, wid, 1, stream=1 + s, dtype="f32")
                                           for s in range(ex["decode_steps"])])).to("cuda")
    log("[bench] %s: %d layers generated and uploaded in %.1f s" % (name, L, time.time() - t0))
    st = moe.MoeStack(gh.desc_for(spec, ex["chunk"]), dev, eps=ex["eps"])
    P, C = ex["prompt"], ex["chunk"]

    def prefill():
        x = x0.clone()
        for c0 in range(0, P, C):
            st.forward(x[c0:c0 + C])  # row slices are contiguous; updated in place
        return x

    prefill()
    torch.cuda.synchronize()
    t = time.perf_counter()
    prefill()
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t
    xs = dec.clone()
    for s in range(4):
        st.forward(xs[s:s + 1])
    torch.cuda.synchronize()
    t = time.perf_counter()
    for s in range(dec.shape[0]):
        st.forward(xs[s:s + 1])
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t
    # one decode step (40 layers) captured as a graph, replayed per token
    buf = torch.empty((1, spec.hidden), dtype=torch.float32, device="cuda")
    buf.copy_(dec[0:1])
    st.forward(buf)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.forward(buf)
    for s in range(4):
        g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for s in range(dec.shape[0]):
        buf.copy_(dec[s:s + 1])
        g.replay()
    torch.cuda.synchronize()
    t_graph = time.perf_counter() - t
    # the same decode steps with each layer in one launch (moe_decode_layer)
    xs = dec.clone()
    for s in range(4):
        st.forward_decode(xs[s:s + 1])
    torch.cuda.synchronize()
    t = time.perf_counter()
    for s in range(dec.shape[0]):
        st.forward_decode(xs[s:s + 1])
    torch.cuda.synchronize()
    t_dec1 = time.perf_counter() - t
    buf.copy_(dec[0:1])
    st.forward_decode(buf)
    torch.cuda.synchronize()
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        st.forward_decode(buf)
    for s in range(4):
        g1.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for s in range(dec.shape[0]):
        buf.copy_(dec[s:s + 1])
        g1.replay()
    torch.cuda.synchronize()
    t_graph1 = time.perf_counter() - t
    weights = L * spec.groups * (weight_bytes(spec, 2 * spec.inter, spec.hidden) + weight_bytes(spec, spec.hidden,
                                                                                               spec.inter))
    out = {"prefill_tokens_per_s": round(P / t_pre, 1), "prefill_ms": round(t_pre * 1e3, 3),
           "decode_tokens_per_s": round(dec.shape[0] / t_dec, 1),
           "decode_graph_tokens_per_s": round(dec.shape[0] / t_graph, 1),
           "decode_graph_ms_per_token": round(t_graph / dec.shape[0] * 1e3, 4),
           "decode_one_launch_tokens_per_s": round(dec.shape[0] / t_dec1, 1),
           "decode_one_launch_graph_tokens_per_s": round(dec.shape[0] / t_graph1, 1),
           "decode_one_launch_graph_ms_per_token": round(t_graph1 / dec.shape[0] * 1e3, 4),
           "layers": L, "weight_bytes_all_layers": weights}
    del st, dev
    return out


def mx4_figures(args, decode=True):
    """MXFP4 weights x MXFP8 activations: the T=2048 Zipf prefill (MFMA fraction
    against the fp8 peak) and decode steps T = 1, 2, 4, 8 (HBM fraction of the
    two GEMM launches, which read the touched groups' 4.25-bit weights)."""
    import torch
    out = {}
    Tq = 2048
    rq = Runner("mx4_e128_top8_shared_zipf", Tq, args.rotations, min(args.steps + args.warmup, 24))
    stq = max(3, min(args.steps, 12))
    wq, Uq, kq = rq.timed(stq, min(args.warmup, 3))
    msq = wq / stq * 1e3
    Rq = Tq * (rq.spec.top_k + rq.spec.n_shared)
    fl_gu = 2.0 * Rq * 2 * rq.spec.inter * rq.spec.hidden
    fl_dn = 2.0 * Rq * rq.spec.hidden * rq.spec.inter
    out["prefill_mx4_zipf_t2048"] = {
        "tokens_per_s": round(Tq / (msq / 1e3), 1), "ms_per_step": round(msq, 5),
        "kernel_ms": {k: round(v, 5) for k, v in kq.items()}, "touched_groups": Uq,
        "gate_up_mfma_frac_fp8": round(fl_gu / (kq["gate_up"] / 1e3) / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4),
        "down_mfma_frac_fp8": round(fl_dn / (kq["down"] / 1e3) / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4),
    }
    del rq
    torch.cuda.empty_cache()
    if not decode:
        return out
    sweep = {}
    for Td in (1, 2, 4, 8):
        rd = Runner("mx4_e128_top8_shared", Td, args.rotations, args.steps + args.warmup)
        wd, Ud, kd = rd.timed(args.steps, args.warmup)
        msd = wd / args.steps * 1e3
        b = gu_algorithmic_bytes(rd.spec, Td, Ud) + down_algorithmic_bytes(rd.spec, Td, Ud)
        rd.fused = True  # the same layer through moe_decode_layer (one launch)
        wf, Uf, kf = rd.timed(args.steps, args.warmup)
        msf = wf / args.steps * 1e3
        bl = b + 2 * rd.spec.n_routed * rd.spec.hidden  # + the router weights
        sweep[str(Td)] = {
            "tokens_per_s": round(Td / (msd / 1e3), 1), "ms_per_step": round(msd, 5),
            "kernel_ms": {k: round(v, 5) for k, v in kd.items()}, "touched_groups": Ud,
            "gemm_hbm_frac": round(b / ((kd["gate_up"] + kd["down"]) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemm_algorithmic_bytes": b,
            "one_launch": {"tokens_per_s": round(Td / (msf / 1e3), 1), "ms_per_step": round(msf, 5),
                           "launch_ms": round(kf["decode_layer"], 5),
                           "layer_hbm_frac": round(bl / (kf["decode_layer"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        }
        del rd
        torch.cuda.empty_cache()
    out["decode_mx4_sweep"] = sweep
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotations", type=int, default=8, help="distinct weight sets cycled per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the int8 T=8 decode figure")
    ap.add_argument("--no-q4", action="store_true", help="skip the 4-bit T=2048 prefill figure")
    ap.add_argument("--no-fp32", action="store_true", help="skip the fp32 16-expert figure")
    ap.add_argument("--no-stack", action="store_true", help="skip the 40-layer 4-bit stack figures")
    ap.add_argument("--cpu-sample", type=int, default=256, help="tokens of the workload the oracle runs")
    ap.add_argument("--workloads", default="headline,decode,fp32,q4,q4c,mx4,stack",
                    help="comma list of the parts to run (profiling runs pick one; mx4p: the MX prefill only); "
                         "without 'headline' the line's value is null")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a reference kernel of known "
                         "size for hardware-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    parts = set(args.workloads.split(","))
    args.no_decode = args.no_decode or "decode" not in parts
    args.no_fp32 = args.no_fp32 or "fp32" not in parts
    args.no_q4 = args.no_q4 or "q4" not in parts
    args.no_stack = args.no_stack or "stack" not in parts
    headline = "headline" in parts

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from mixture_experts_expert_moe_amd import moe
    moe.lib()
    if args.copy_calib_mb:
        n = args.copy_calib_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy of %d MiB done" % args.copy_calib_mb)
        del src, dst

    name, T = "bf16_e128_top8_shared", 256
    value = ms = roofline = None
    extra = {"weight_sets_rotated": args.rotations}
    spec = synth_spec(name)
    if headline:
        r = Runner(name, T, args.rotations, args.steps + args.warmup)
        wall, U, kms = r.timed(args.steps, args.warmup)
        ms = wall / args.steps * 1e3
        value = T / (ms / 1e3)
        gu_bytes = gu_algorithmic_bytes(spec, T, U)
        gu_ms = kms["gate_up"]
        achieved = gu_bytes / (gu_ms / 1e3) / 1e9
        dn_bytes = down_algorithmic_bytes(spec, T, U)
        R = T * (spec.top_k + spec.n_shared)
        flops = 2.0 * R * (2 * spec.inter * spec.hidden + spec.hidden * spec.inter)
        traffic = load_traffic("gate_up", name, gu_bytes)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "grouped_gemm_kernel<bf16, gate_up>", "algorithmic_bytes_per_launch": gu_bytes,
                    "avg_launch_ms": round(gu_ms, 5)}
        extra.update({
            "kernel_ms": {k: round(v, 5) for k, v in kms.items()},
            "touched_groups": U,
            "down_hbm_frac": round(dn_bytes / (kms["down"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemm_mfma_frac_bf16": round(flops / ((kms["gate_up"] + kms["down"]) / 1e3) / 1e12
                                         / MFMA_BF16_PEAK_TFLOPS, 4),
            "layer_hbm_frac": round((gu_bytes + dn_bytes) / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        })
        # the same steps replayed from a captured HIP graph (no host launch gaps)
        g_s = r.graph_timed(max(1, args.steps // len(r.wsets)))
        extra["graph_replay"] = {"tokens_per_s": round(T / g_s, 1), "ms_per_step": round(g_s * 1e3, 5)}
        del r
        torch.cuda.empty_cache()

    if not args.no_decode:
        sweep, fsweep = {}, {}
        for Td in (1, 2, 4, 8):
            rd = Runner("int8_e128_top8_shared", Td, args.rotations, args.steps + args.warmup)
            wd, Ud, kd = rd.timed(args.steps, args.warmup)
            msd = wd / args.steps * 1e3
            b = gu_algorithmic_bytes(rd.spec, Td, Ud) + down_algorithmic_bytes(rd.spec, Td, Ud)
            sweep[Td] = {
                "tokens_per_s": round(Td / (msd / 1e3), 1), "ms_per_step": round(msd, 5),
                "kernel_ms": {k: round(v, 5) for k, v in kd.items()}, "touched_groups": Ud,
                "gemm_hbm_frac": round(b / ((kd["gate_up"] + kd["down"]) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "gemm_algorithmic_bytes": b,
            }
            # the same layer through moe_decode_layer (one launch)
            rd.fused = True
            wf, Uf, kf = rd.timed(args.steps, args.warmup)
            msf = wf / args.steps * 1e3
            bl = b + 2 * rd.spec.n_routed * rd.spec.hidden  # + the router weights
            fsweep[Td] = {"tokens_per_s": round(Td / (msf / 1e3), 1), "ms_per_step": round(msf, 5),
                          "launch_ms": round(kf["decode_layer"], 5), "touched_groups": Uf,
                          "layer_hbm_frac": round(bl / (kf["decode_layer"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
            del rd
            torch.cuda.empty_cache()
        extra["decode_int8_t8"] = sweep[8]
        extra["decode_int8_sweep"] = {str(t): {k: v for k, v in r.items() if k != "kernel_ms"} for t, r in sweep.items()}
        extra["decode_int8_one_launch"] = {str(t): r for t, r in fsweep.items()}
    if not args.no_fp32:
        r1 = Runner("fp32_e16_top2", 16, args.rotations, args.steps + args.warmup)
        w1, U1, k1 = r1.timed(args.steps, args.warmup)
        ms1 = w1 / args.steps * 1e3
        b1 = gu_algorithmic_bytes(r1.spec, 16, U1) + down_algorithmic_bytes(r1.spec, 16, U1)
        extra["fp32_e16_top2_t16"] = {
            "tokens_per_s": round(16 / (ms1 / 1e3), 1), "ms_per_step": round(ms1, 5), "touched_groups": U1,
            "kernel_ms": {k: round(v, 5) for k, v in k1.items()},
            "gemm_hbm_frac": round(b1 / ((k1["gate_up"] + k1["down"]) / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        del r1
        torch.cuda.empty_cache()
    if not args.no_q4:
        Tq = 2048
        rq = Runner("q4_e128_top8_shared_zipf", Tq, args.rotations, min(args.steps + args.warmup, 24))
        stq = max(3, min(args.steps, 12))
        wq, Uq, kq = rq.timed(stq, min(args.warmup, 3))
        msq = wq / stq * 1e3
        Rq = Tq * (rq.spec.top_k + rq.spec.n_shared)
        fl_gu = 2.0 * Rq * 2 * rq.spec.inter * rq.spec.hidden
        fl_dn = 2.0 * Rq * rq.spec.hidden * rq.spec.inter
        extra["prefill_q4_zipf_t2048"] = {
            "tokens_per_s": round(Tq / (msq / 1e3), 1), "ms_per_step": round(msq, 5),
            "kernel_ms": {k: round(v, 5) for k, v in kq.items()}, "touched_groups": Uq,
            "gate_up_mfma_frac": round(fl_gu / (kq["gate_up"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "down_mfma_frac": round(fl_dn / (kq["down"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "gemm_mfma_frac": round((fl_gu + fl_dn) / ((kq["gate_up"] + kq["down"]) / 1e3) / 1e12
                                    / MFMA_BF16_PEAK_TFLOPS, 4),
        }
        del rq
        torch.cuda.empty_cache()

    if "q4c" in parts:
        # one layer of the 4-bit stack at its prefill chunk (T = 256, uniform
        # routing): HBM-bound, every group's weights read once per launch
        Tc = 256
        rc = Runner("q4_stack40", Tc, args.rotations, args.steps + args.warmup)
        wc, Uc, kc = rc.timed(args.steps, args.warmup)
        msc = wc / args.steps * 1e3
        bg, bd = gu_algorithmic_bytes(rc.spec, Tc, Uc), down_algorithmic_bytes(rc.spec, Tc, Uc)
        extra["prefill_q4_chunk_t256"] = {
            "tokens_per_s": round(Tc / (msc / 1e3), 1), "ms_per_step": round(msc, 5),
            "kernel_ms": {k: round(v, 5) for k, v in kc.items()}, "touched_groups": Uc,
            "gate_up_hbm_frac": round(bg / (kc["gate_up"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "down_hbm_frac": round(bd / (kc["down"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemm_algorithmic_bytes": bg + bd,
        }
        del rc
        torch.cuda.empty_cache()

    if "mx4" in parts or "mx4p" in parts:
        extra.update(mx4_figures(args, decode="mx4" in parts))
        torch.cuda.empty_cache()

    if not args.no_stack:
        extra["stack40_q4"] = stack_figures()
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(value, 1) if value else None, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5) if ms else None,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "tokens": T, "hidden": spec.hidden, "inter": spec.inter,
                   "routed_experts": spec.n_routed, "top_k": spec.top_k, "shared_experts": spec.n_shared,
                   "weights": spec.wt, "parallelism": "none (one GPU)"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and headline:
        line["cpu_baseline"] = cpu_baseline(name, T, min(args.cpu_sample, T))
    line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
