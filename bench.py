"""Benchmark: forward pass of one DeepSeekMoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]

A step is one pass of the whole layer (gate, dispatch, routed expert FFNs,
shared expert, combine) over one batch of synthetic tokens already resident
in HBM.  The headline workload is the V3-shaped prefill layer (T=8192, dim
7168, 256 routed experts in 8 groups keep 4, top-8, 1 shared, inter 2048,
bf16).  Beside it the same JSON line reports the other layer shapes: the
8-token fp8 decode step of the V3 layer, the V3 prefill batch in FP8 W8A8, a
V2-Lite-shaped chunk (T=512), a V2-shaped layer (T=4096), the tiny fp32 layer
(T=64) and one GPU's expert-parallel share of the V3 layer.  Random-init
weights of the layer's architecture and x ~ N(0,1), as described in synth.py.

Timing: `ms_per_step` is a region of K steps with HIP events only at its ends,
divided by K.  A second pass of K steps records events on the launch stream
between the stages of every step (gate, dispatch, gate/up GEMM, down GEMM,
combine) for the per-stage and per-step mean, median, min and p90; its
markers are kept out of the headline region.

roofline: the dominant kernel is the gate/up grouped GEMM (moe_expert_up);
its average duration over the timed steps comes from those events.  Its
algorithmic work per launch is 2*T*K*(2I)*D + 2*T*(2*S*I)*D flops and the
bytes of the touched experts' W1/W3 (plus block scales), the shared W1/W3,
x and the written h.  The bound reported is the ceiling that binds (the flops
at the dtype's MFMA peak against the bytes at 8 TB/s); both fractions are
reported.

cpu_baseline: the float64 oracle on a token sample of the headline workload,
on the host's cores; the expert weights are decoded to float64 outside the
timed region, so only the oracle's own arithmetic is timed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector)

# Measured HBM traffic per launch of the roofline kernels: rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the layer's
# launches), scaled by what the same counters read for a 1 GiB device copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  The commands and per-dispatch values
# are in profiles/.  Each figure is tied to a hash of its kernel's source and is
# reported as null once that source has changed.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
COUNTERS = {
    "prefill_up": {"sources": ("gemm_expert.hip", "common.hpp"),
                   "sha256": "cc5405a0485a7dcae974229ecbc26d0f06bd2e2c0f937aa80f8b871c8fd37b0e",
                   "fetch_kib": 12114830, "write_kib": 294927,
                   "profile": "profiles/gemm_expert_gate_up_v3_prefill_T8192_counters.md"},
    "decode_up": {"sources": ("gemm_skinny.hip", "common.hpp"),
                  "sha256": "8a86871ecd0fe49301b9a4f87bb3f4bf23a9523c288db51e2882de059ffe939c",
                  "fetch_kib": 775595, "write_kib": 3424,
                  "profile": "profiles/gemm_skinny_gate_up_v3_decode_T8_counters.md"},
    "w8a8_up": {"sources": ("gemm_fp8.hip", "common.hpp"),
                "sha256": "63849d515b9b3c98d3dfc500ddc0df40c5f38181b6a4d9f3e9df9ae0b3fc1e66",
                "fetch_kib": 5046430, "write_kib": 190350,
                "profile": "profiles/gemm_fp8_gate_up_v3_prefill_w8a8_T8192_counters.md"},
    "v2_up": {"sources": ("gemm_expert.hip", "common.hpp"),
              "sha256": "cc5405a0485a7dcae974229ecbc26d0f06bd2e2c0f937aa80f8b871c8fd37b0e",
              "fetch_kib": 3114970, "write_kib": 98512,
              "profile": "profiles/gemm_expert_gate_up_v2_T4096_counters.md"},
    "ep_up": {"sources": ("gemm_expert.hip", "common.hpp"),
              "sha256": "cc5405a0485a7dcae974229ecbc26d0f06bd2e2c0f937aa80f8b871c8fd37b0e",
              "fetch_kib": 1294826, "write_kib": 32769,
              "profile": "profiles/gemm_expert_gate_up_v3_ep_shard_T4096_E32_counters.md"},
}


def source_sha(names) -> str:
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routed_expert_moe_amd", "csrc")
    for n in names:
        with open(os.path.join(base, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch from the counter runs, or None if the kernel changed since."""
    c = COUNTERS[key]
    if c["sha256"] is None or c["sha256"] != source_sha(c["sources"]):
        return None
    return (c["fetch_kib"] * FETCH_SCALE + c["write_kib"] * WRITE_SCALE) * 1024.0


def roofline(flops: float, nbytes: float, ms: float, traffic, kernel: str,
             peak_tflops: float = PEAK_BF16_TFLOPS) -> dict:
    """The binding ceiling of a kernel: MFMA if its flops take longer at peak than its bytes, else HBM."""
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    tflops = flops / (ms / 1e3) / 1e12
    gbs = nbytes / (ms / 1e3) / 1e9
    r = {"kernel": kernel}
    if t_mfma >= t_hbm:
        r.update(bound="mfma", achieved=tflops, peak=peak_tflops, unit="TFLOP/s",
                 frac=tflops / peak_tflops)
    else:
        r.update(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=gbs / PEAK_HBM_GBS)
    r.update(traffic=traffic, traffic_unit="bytes per launch (HBM, measured)",
             avg_launch_ms=ms, algorithmic_flops=flops, algorithmic_bytes=nbytes,
             mfma_frac=tflops / peak_tflops, hbm_frac=gbs / PEAK_HBM_GBS)
    return r


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=0, help="default: 10x --steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=6144,
                    help="tokens of the headline workload the CPU oracle is timed on")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads to time (default: all); names as in the JSON")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration)")
    ap.add_argument("--library-probe", action="store_true",
                    help="only compare the gate/up GEMM with the vendor GEMM library on the same shape")
    return ap.parse_args()


STAGES = ("gate", "dispatch", "up", "down", "combine")


class Pass:
    """Device buffers for one layer and the step sequence of the hot path."""

    def __init__(self, layer):
        import torch
        from routed_expert_moe_amd import binding as B
        self.B = B
        self.layer = layer
        s = layer.shape
        self.cfg = B.config_of(s)
        B.moe_validate(self.cfg)
        self.w = B.weights_of(layer)
        T, E, K, D, I, S = s.T, s.n_routed, s.top_k, s.dim, s.inter_dim, s.n_shared
        dev, act = layer.x.device, layer.x.dtype
        self.T = T
        self.logits = torch.empty(T, E, dtype=torch.float32, device=dev)
        self.idx = torch.empty(T, K, dtype=torch.int32, device=dev)
        self.tw = torch.empty(T, K, dtype=torch.float32, device=dev)
        self.r = B.make_routing(self.cfg, T)
        R = self.r.struct.max_rows
        self.h = torch.empty(R, I, dtype=act, device=dev)
        self.y = torch.empty(R, D, dtype=act, device=dev)
        self.hs = torch.empty(T, S * I, dtype=act, device=dev) if S else None
        self.z = torch.empty(T, D, dtype=act, device=dev) if S else None
        self.out = torch.empty(T, D, dtype=act, device=dev)

    def step(self, ev=None):
        """One layer pass; ev = 6 events recorded at the stage boundaries (or None)."""
        B, L = self.B, self.layer
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        B.moe_gate(self.cfg, self.T, L.x, L.w_gate, L.bias, self.logits, self.idx, self.tw)
        rec(1)
        B.moe_permute(self.cfg, self.T, self.idx, self.r)
        if self.cfg.act_quant:
            B.moe_quant_act(self.cfg, self.T, L.x, self.r)
        rec(2)
        B.moe_expert_up(self.cfg, self.T, L.x, self.r, self.w, self.h, self.hs)
        rec(3)
        B.moe_expert_down(self.cfg, self.T, self.r, self.w, self.h, self.hs, self.y, self.z)
        rec(4)
        B.moe_combine(self.cfg, self.T, L.x, self.z, self.y, self.r, self.tw, self.out)
        rec(5)


def work_figures(layer, counts):
    """Algorithmic flops / bytes of the layer and of the gate/up kernel for the actual routing."""
    s = layer.shape
    T, E, K, D, I, S = s.T, s.n_routed, s.top_k, s.dim, s.inter_dim, s.n_shared
    P = T * K
    ab = 2 if s.act == "bf16" else 4
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[s.weight]
    touched = int((counts > 0).sum())
    w13_e = 2 * I * D * wb + (2 * I // 128) * (D // 128) * 4 * (s.weight == "fp8")
    w2_e = D * I * wb + (D // 128) * (I // 128) * 4 * (s.weight == "fp8")
    sw13 = 2 * S * I * D * wb + (2 * S * I // 128) * (D // 128) * 4 * (s.weight == "fp8") if S else 0
    sw2 = D * S * I * wb + (D // 128) * (S * I // 128) * 4 * (s.weight == "fp8") if S else 0
    flops_up = 2 * P * 2 * I * D + 2 * T * 2 * S * I * D
    # W8A8: gate/up reads x and writes h as e4m3 codes plus one fp32 scale per 128
    qb = 1 + 4 / 128 if s.act_quant else ab
    bytes_up = touched * w13_e + sw13 + T * D * qb + P * I * qb + T * S * I * qb
    flops_layer = 2 * T * E * D + 2 * P * 3 * I * D + 2 * T * 3 * S * I * D
    bytes_layer = touched * (w13_e + w2_e) + sw13 + sw2 + E * D * ab + 2 * T * D * ab
    return dict(touched=touched, flops_up=flops_up, bytes_up=bytes_up, flops_layer=flops_layer,
                bytes_layer=bytes_layer)


def progress(msg: str) -> None:
    """One line per phase on stderr (stdout carries only the JSON result)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stats(v) -> dict:
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()),
            "p90": float(np.percentile(a, 90))}


def time_pass(p: Pass, steps: int, warmup: int) -> dict:
    """Times `steps` layer passes after `warmup` untimed ones.

    The headline region is `steps` passes with events only at its two ends.  A
    second pass of `steps` steps then records events between the launches on the
    launch stream, for the per-stage and per-step times; those six markers per
    step cost about 19 us of GPU time (measured on the 0.5 ms decode step), so
    they stay out of the headline region.  Returns the headline milliseconds, its
    host wall time, and the instrumented pass's per-stage and per-step times."""
    import torch
    for _ in range(warmup):
        p.step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        p.step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for i in range(steps):
        p.step(evs[i])
    torch.cuda.synchronize()
    per = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, name in enumerate(STAGES)}
    per["step"] = [e[0].elapsed_time(e[5]) for e in evs]
    return {"total_ms": t0.elapsed_time(t1), "wall_s": wall, "per": per}


def layer_report(p: Pass, t: dict, steps: int, peak_tflops: float, traffic_key=None,
                 kernel: str = "moe_expert_up (gate/up grouped GEMM + SwiGLU)") -> dict:
    """The per-workload record: throughput, step statistics, stage medians, roofline."""
    layer, s = p.layer, p.layer.shape
    fig = work_figures(layer, p.r.counts.cpu().numpy())
    ms = t["total_ms"] / steps
    up_ms = stats(t["per"]["up"])["mean"]
    return {
        "workload": s.name, "T": s.T, "dim": s.dim, "n_routed": s.n_routed, "top_k": s.top_k,
        "n_shared": s.n_shared, "inter_dim": s.inter_dim, "score": s.score,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights (128x128 fp32 scales)"}[s.weight]
                 + (" x fp8-e4m3 activations (1x128 fp32 scales)" if s.act_quant else ""),
        "steps": steps, "ms_per_step": ms, "tokens_per_s": s.T / (ms / 1e3),
        "step_ms": stats(t["per"]["step"]),
        "stage_ms_median": {k: stats(t["per"][k])["median"] for k in STAGES},
        "experts_touched": fig["touched"],
        "layer": {"flops": fig["flops_layer"], "bytes": fig["bytes_layer"],
                  "tflops": fig["flops_layer"] / (ms / 1e3) / 1e12,
                  "mfma_frac": fig["flops_layer"] / (ms / 1e3) / 1e12 / peak_tflops,
                  "gbs": fig["bytes_layer"] / (ms / 1e3) / 1e9,
                  "hbm_frac": fig["bytes_layer"] / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                  "floor_ms": max(fig["flops_layer"] / (peak_tflops * 1e9),
                                  fig["bytes_layer"] / (PEAK_HBM_GBS * 1e6))},
        "roofline": roofline(fig["flops_up"], fig["bytes_up"], up_ms,
                             measured_traffic(traffic_key) if traffic_key else None, kernel, peak_tflops),
    }


def run_workload(shape, steps: int, warmup: int, peak_tflops: float, traffic_key=None, kernel=None,
                 keep=False):
    import torch
    from routed_expert_moe_amd import synth
    progress(f"building {shape.name}")
    dev = "cpu" if shape.T * shape.dim * shape.n_routed < 2 ** 27 else "cuda"
    layer = synth.make_layer(shape, device=dev)
    if dev == "cpu":
        for f in ("x", "w_gate", "bias", "w13", "w2", "sw13", "sw2", "w13_scale", "w2_scale",
                  "sw13_scale", "sw2_scale"):
            if getattr(layer, f) is not None:
                setattr(layer, f, getattr(layer, f).cuda())
    progress(f"timing {shape.name} ({steps} steps)")
    p = Pass(layer)
    t = time_pass(p, steps, warmup)
    kw = {} if kernel is None else {"kernel": kernel}
    rep = layer_report(p, t, steps, peak_tflops, traffic_key, **kw)
    rep["_wall_s"] = t["wall_s"]
    rep["_total_ms"] = t["total_ms"]
    if keep:
        return rep, p
    del p, layer
    torch.cuda.empty_cache()
    return rep, None


def time_bias_update(p: Pass, shape, calls: int = 200):
    """The auxiliary-loss-free bias update on the routing of the last timed batch.

    A training-time step after the gate: E counts and E biases in, E biases out,
    one tiny launch, so it is bound by launch latency, not by a roofline."""
    import torch
    B = p.B
    bias = p.layer.bias.clone()
    for _ in range(10):
        B.moe_bias_update(p.cfg, p.T, p.r, 1e-3, bias)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(calls):
        B.moe_bias_update(p.cfg, p.T, p.r, 1e-3, bias)
    b.record()
    torch.cuda.synchronize()
    return {"what": "moe_bias_update (auxiliary-loss-free balancing step) on this batch's routing",
            "us_per_call": a.elapsed_time(b) / calls * 1e3, "experts": shape.n_routed,
            "bound": "launch latency", "bytes_per_call": shape.n_routed * 12}


def time_balance_loss(p: Pass, shape, calls: int = 20):
    """The sequence-wise balance loss of the last timed batch (two sequences of T/2).

    A training-time reduction over the [T, E] logits and the routing; it reads
    T*E*4 + T*K*4 bytes, so HBM is its ceiling."""
    import torch
    B = p.B
    loss = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.moe_balance_loss_workspace_size(p.cfg, p.T, p.T // 2), 256), dtype=torch.uint8,
                     device="cuda")
    B.moe_balance_loss(p.cfg, p.T, p.T // 2, p.logits, p.idx, 1e-4, loss, workspace=ws)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(calls):
        B.moe_balance_loss(p.cfg, p.T, p.T // 2, p.logits, p.idx, 1e-4, loss, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / calls * 1e3
    nbytes = p.T * shape.n_routed * 4 + p.T * shape.top_k * 4
    return {"what": "moe_balance_loss (sequence-wise balance loss), 2 sequences of T/2 tokens",
            "us_per_call": us, "bytes_per_call": nbytes, "gbs": nbytes / us / 1e3}


def time_backward(p: Pass, shape, calls: int = 3):
    """The layer backward (moe_backward) of the last timed batch, for a seeded upstream gradient.

    Its GEMM work: the gate/up products again (a and c are recomputed, the
    forward keeps only h), dH and dX through W2 and W13, and the weight
    gradients dW2 and dW13, for the routed pairs and the shared expert, plus
    dX and dW_g of the gate: 3 x (gate/up flops) + 2 x (down flops) + 4 T E D."""
    import torch
    from routed_expert_moe_amd import synth
    B, L = p.B, p.layer
    T, E, K, D, I, S = shape.T, shape.n_routed, shape.top_k, shape.dim, shape.inter_dim, shape.n_shared
    dout = synth.make_dout(shape, device="cuda")
    grads = B.Grads.empty(p.cfg, T, L.x.dtype)
    ws = torch.empty(B.moe_backward_workspace_size(p.cfg, T), dtype=torch.uint8, device="cuda")
    p.step()

    def one():
        B.moe_backward(p.cfg, T, L.x, p.w, p.r, p.idx, p.tw, p.logits, p.y, dout, grads, workspace=ws)
    one()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in evs:
        a.record()
        one()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = sum(times) / calls
    P = T * K
    up = 2 * P * 2 * I * D + 2 * T * 2 * S * I * D
    down = 2 * P * D * I + 2 * T * D * S * I
    flops = 3 * up + 2 * down + 4 * T * E * D
    res = {"what": "moe_backward: dx, dW_gate, routed and shared dW13/dW2 for one upstream gradient",
           "ms_per_call": ms, "call_ms": stats(times), "tokens_per_s": T / (ms / 1e3), "gemm_flops": flops,
           "tflops": flops / (ms / 1e3) / 1e12, "mfma_frac": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
           "workspace_bytes": ws.numel()}

    # The training variant: the forward's gate/up GEMM also keeps a and c in fp32
    # (moe_expert_ffn_save) and the backward reads them instead of recomputing
    # (moe_backward_saved): timed as that expert FFN against moe_expert_ffn, and the
    # backward without its first GEMM (2 x gate/up + 2 x down + gate flops).
    R = p.r.struct.max_rows
    ab = torch.empty(R, 2 * I, dtype=torch.float32, device="cuda")
    abs_ = torch.empty(T, 2 * S * I, dtype=torch.float32, device="cuda") if S else None

    def ffn(save):
        if save:
            B.moe_expert_ffn_save(p.cfg, T, L.x, p.r, p.w, p.h, p.y, p.hs, p.z, ab, abs_)
        else:
            B.moe_expert_ffn(p.cfg, T, L.x, p.r, p.w, p.h, p.y, p.hs, p.z)

    def saved():
        B.moe_backward_saved(p.cfg, T, L.x, p.w, p.r, p.idx, p.tw, p.logits, p.y, dout, ab, abs_, grads,
                             workspace=ws)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]
    f_plain = timed(lambda: ffn(False), calls)
    f_save = timed(lambda: ffn(True), calls)
    b_saved = timed(saved, calls)
    ms_s = sum(b_saved) / calls
    flops_s = 2 * up + 2 * down + 4 * T * E * D
    res["saved_preacts"] = {
        "what": "moe_expert_ffn_save then moe_backward_saved (a and c kept by the forward in fp32)",
        "expert_ffn_ms": sum(f_plain) / calls, "expert_ffn_save_ms": sum(f_save) / calls,
        "backward_ms": ms_s, "backward_call_ms": stats(b_saved), "preact_bytes": (ab.numel() + (abs_.numel() if S else 0)) * 4,
        "backward_tflops": flops_s / (ms_s / 1e3) / 1e12,
        "training_step_ms_delta": (sum(f_save) - sum(f_plain)) / calls + ms_s - ms}
    del grads, ws, ab, abs_
    torch.cuda.empty_cache()
    return res


def host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cores_available": len(os.sched_getaffinity(0))}


def _oracle_time(layer, tokens=None, single_thread=False) -> dict:
    """Seconds of the float64 oracle's layer forward, weight decoding excluded.

    The oracle takes each expert's weights through a callable; the time spent
    inside it (copying the stored weights to the host and decoding them to
    float64) is measured and subtracted, so what remains is the oracle's own
    arithmetic: gate, the touched experts' SwiGLU FFNs, shared expert, combine."""
    import threadpoolctl
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
    import oracle
    from oracle import w8a8
    from oracle_bridge import bias_f64, expert_fn, shared_pair, spec_of, to_f64
    xs = layer.x if tokens is None else layer.x[:tokens]
    x = to_f64(xs)
    wg = to_f64(layer.w_gate)
    b = bias_f64(layer)
    shared = shared_pair(layer)
    fetch = expert_fn(layer, fast=True)
    spent = [0.0]

    def expert(e):
        t = time.perf_counter()
        w = fetch(e)
        spent[0] += time.perf_counter() - t
        return w
    fn = w8a8.moe_layer_w8a8 if layer.shape.act_quant else oracle.moe_layer
    limit = threadpoolctl.threadpool_limits(1) if single_thread else None
    try:
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
        t0 = time.perf_counter()
        fn(x, wg, b, expert, shared, spec_of(layer.shape))
        dt = time.perf_counter() - t0 - spent[0]
    finally:
        if limit is not None:
            limit.unregister()
    n = x.shape[0]
    return {"tokens": n, "seconds": dt, "tokens_per_s": n / dt, "threads": threads,
            "decode_seconds_excluded": spent[0]}


def cpu_baseline(layer, n_tokens: int) -> dict:
    """The float64 oracle on the first n_tokens tokens of the headline workload, on host cores."""
    r = _oracle_time(layer, tokens=n_tokens)
    out = {"value": r["tokens_per_s"], "unit": "tokens/s", "cores": r["threads"], "kind": "oracle",
           "sample": (f"first {n_tokens} tokens of the {layer.shape.name} workload, whole layer (gate on "
                      f"those tokens, {layer.shape.top_k} routed + shared SwiGLU experts, combine) in "
                      f"float64 on {r['threads']} BLAS threads; {r['seconds']:.1f} s of oracle arithmetic "
                      f"(expert weight decoding, {r['decode_seconds_excluded']:.1f} s, excluded)")}
    out.update(host_info())
    return out


def oracle_timings(extra_layers) -> dict:
    """Oracle times on the small workloads: all BLAS threads and one thread."""
    res = {}
    for name, layer, tokens in extra_layers:
        progress(f"oracle timing {name}")
        all_t = _oracle_time(layer, tokens=tokens)
        one_t = _oracle_time(layer, tokens=tokens, single_thread=True)
        res[name] = {"tokens": all_t["tokens"], "all_threads": all_t, "single_thread": one_t}
    return res


def copy_probe(mib: int):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n}))


def library_probe(reps: int = 8) -> None:
    """The routed gate/up GEMM against the vendor GEMM library (hipBLASLt through torch) on
    one shape both can run: the V3 layer's 256 experts with exactly 256 rows each (T = 8192,
    token t -> experts 8t .. 8t+7 mod 256), i.e. 256 independent 256 x 4096 x 7168 products.

    Times moe_expert_up on that routing (routed experts only), torch.bmm on the same
    products with the weights stored k-major, and one dense 65536 x 4096 x 7168 product
    (the same flops against a single weight matrix); then moe_expert_up alone with every
    expert holding 64 .. 512 rows.  Random bf16 operands; medians of `reps` calls after two
    warm-up calls.  Run it under rocprofv3 --pmc to read the clock and MFMA occupancy of
    each launch."""
    import torch
    from routed_expert_moe_amd import binding as B, configs
    sh = configs.V3_PREFILL_BF16
    cfg = B.config_of(sh)
    E, D, I, K, T = sh.n_routed, sh.dim, sh.inter_dim, sh.top_k, sh.T
    M = T * K // E
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    w13 = torch.randn(E, 2 * I, D, device=dev, dtype=torch.bfloat16, generator=g) * (D ** -0.5)
    x = torch.randn(T, D, device=dev, dtype=torch.bfloat16, generator=g)
    none = type("NoWeights", (), {k: None for k in ("w_gate", "bias", "w13_scale", "w2_scale", "sw13",
                                                   "sw13_scale", "sw2", "sw2_scale")})()
    none.w13 = w13
    none.w2 = w13        # validated as present; the gate/up half never reads it
    wts = B.weights_of(none)
    t = torch.arange(T, device=dev, dtype=torch.int32)[:, None] * K + torch.arange(K, device=dev, dtype=torch.int32)
    idx = (t % E).to(torch.int32).contiguous()
    r = B.make_routing(cfg, T)
    B.moe_permute(cfg, T, idx, r)
    h = torch.empty(r.struct.max_rows, I, device=dev, dtype=torch.bfloat16)
    a = torch.randn(E, M, D, device=dev, dtype=torch.bfloat16, generator=g)
    bk = w13.transpose(1, 2).contiguous()            # [E, D, 2I], k-major
    c = torch.empty(E, M, 2 * I, device=dev, dtype=torch.bfloat16)
    a2, b2 = a.view(E * M, D), bk[0].contiguous()
    c2 = torch.empty(E * M, 2 * I, device=dev, dtype=torch.bfloat16)
    flops = 2.0 * E * M * D * 2 * I
    out = {"shape": f"{E} experts x {M} rows, N = {2 * I}, K = {D}, bf16", "flops": flops}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for name, fn in (("moe_expert_up", lambda: B.moe_expert_up(cfg, T, x, r, wts, h)),
                     ("torch_bmm", lambda: torch.bmm(a, bk, out=c)),
                     ("torch_mm_dense", lambda: torch.mm(a2, b2, out=c2))):
        ts = []
        for i in range(reps + 2):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(ev[0].elapsed_time(ev[1]))
        st = stats(ts)
        out[name] = {"ms": st, "tflops_median": flops / (st["median"] / 1e3) / 1e12}
        progress(f"library probe {name}: {st['median']:.3f} ms")
    # the routed launch alone as the rows per expert vary (every expert the same count)
    del a, bk, c, a2, b2, c2
    sweep = {}
    for rows in (64, 128, 192, 256, 384, 512):
        Tr = rows * E // K
        xr = torch.randn(Tr, D, device=dev, dtype=torch.bfloat16, generator=g)
        tr = torch.arange(Tr, device=dev, dtype=torch.int32)[:, None] * K + torch.arange(K, device=dev, dtype=torch.int32)
        rr = B.make_routing(cfg, Tr)
        B.moe_permute(cfg, Tr, (tr % E).to(torch.int32).contiguous(), rr)
        hr = torch.empty(rr.struct.max_rows, I, device=dev, dtype=torch.bfloat16)
        ts = []
        for i in range(reps + 2):
            ev[0].record()
            B.moe_expert_up(cfg, Tr, xr, rr, wts, hr)
            ev[1].record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(ev[0].elapsed_time(ev[1]))
        med = stats(ts)["median"]
        fl = 2.0 * Tr * K * D * 2 * I
        sweep[str(rows)] = {"T": Tr, "ms_median": med, "tflops": fl / (med / 1e3) / 1e12,
                            "w13_read_once_tbs": E * 2 * I * D * 2 / (med / 1e3) / 1e12}
        progress(f"library probe rows per expert {rows}: {med:.3f} ms")
        del xr, rr, hr
    out["moe_expert_up_rows_per_expert"] = sweep
    print(json.dumps({"library_probe": out}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (the layer's single-GPU path; no multi-GPU path is built): "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.library_probe:
        library_probe()
        return
    from routed_expert_moe_amd import binding as B
    from routed_expert_moe_amd import configs, synth
    B.lib()
    only = set(filter(None, args.only.split(",")))
    want = (lambda n: not only or n in only)

    # ---- prefill: the headline workload
    shape = configs.V3_PREFILL_BF16
    res = {
        "metric": "MoE-layer tokens/s + % MFMA peak (prefill), % HBM GB/s (decode), 1 MI355X",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": shape.name, "T": shape.T, "dim": shape.dim, "n_routed": shape.n_routed,
                   "n_groups": shape.n_groups, "topk_groups": shape.topk_groups, "top_k": shape.top_k,
                   "n_shared": shape.n_shared, "inter_dim": shape.inter_dim, "score": shape.score,
                   "route_scale": shape.route_scale},
    }
    head_layer = None
    if want(shape.name):
        rep, p = run_workload(shape, args.steps, args.warmup, PEAK_BF16_TFLOPS, "prefill_up",
                              "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_expert_kernel)", keep=True)
        res["value"] = shape.T * args.steps / (rep["_total_ms"] / 1e3)
        res["ms_per_step"] = rep["_total_ms"] / args.steps
        res["wall_s"] = rep.pop("_wall_s")
        rep.pop("_total_ms")
        res["config"]["experts_touched"] = rep["experts_touched"]
        res["step_ms"] = rep["step_ms"]
        res["stage_ms_median"] = rep["stage_ms_median"]
        res["layer"] = rep["layer"]
        res["roofline"] = rep["roofline"]
        res["bias_update"] = time_bias_update(p, shape)
        res["balance_loss"] = time_balance_loss(p, shape)
        if not args.no_backward:
            progress("timing the backward")
            res["backward"] = time_backward(p, shape)
        head_layer = p.layer
        del p
        torch.cuda.empty_cache()

    def side(key, shp, steps, peak, traffic_key=None, kernel=None):
        if not want(shp.name):
            return
        rep, _ = run_workload(shp, steps, max(args.warmup, 3), peak, traffic_key, kernel)
        rep.pop("_wall_s")
        rep.pop("_total_ms")
        res[key] = rep

    side("prefill_w8a8", configs.V3_PREFILL_W8A8, args.steps, PEAK_FP8_TFLOPS, "w8a8_up",
         "moe_expert_up (fp8 x fp8 grouped GEMM + SwiGLU + h quantisation, gemm_fp8_kernel)")
    dsteps = args.decode_steps or 10 * args.steps
    side("decode", configs.V3_DECODE_FP8, dsteps, PEAK_BF16_TFLOPS, "decode_up",
         "moe_expert_up (fp8 weight-streaming gate/up + SwiGLU, gemm_skinny_kernel)")
    side("v2_T4096", configs.V2_BF16, args.steps, PEAK_BF16_TFLOPS, "v2_up",
         "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_expert_kernel)")
    side("v2lite_T512", configs.V2_LITE_BF16, 5 * args.steps, PEAK_BF16_TFLOPS, None,
         "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_expert_kernel)")
    side("tiny_f32", configs.TINY_F32, 10 * args.steps, PEAK_F32_TFLOPS, None,
         "moe_expert_up (fp32 SIMT grouped GEMM + SwiGLU, gemm_f32_kernel)")
    side("ep_shard", configs.V3_EP_SHARD_BF16, args.steps, PEAK_BF16_TFLOPS, "ep_up",
         "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_expert_kernel)")
    if "ep_shard" in res:
        res["ep_shard"]["what"] = ("one GPU's expert-parallel share of v3_prefill_bf16_T8192 (a local routing "
                                   "of the dispatched tokens stands in for the global gate; no collectives)")

    if not args.no_cpu_baseline and head_layer is not None:
        progress("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(head_layer, args.cpu_tokens)
        del head_layer
        torch.cuda.empty_cache()
        small = [("tiny_f32", synth.make_layer(configs.TINY_F32, device="cpu"), None),
                 ("v3_decode_fp8_T8", synth.make_layer(configs.V3_DECODE_FP8, device="cuda"), None)]
        res["oracle_timing"] = oracle_timings(small)
        del small
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
