"""Benchmark: forward pass of one DeepSeekMoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole layer (gate, dispatch, routed expert FFNs,
shared expert, combine) over one batch of synthetic tokens already resident
in HBM.  The headline workload is the V3-shaped prefill layer (T=8192, dim
7168, 256 routed experts in 8 groups keep 4, top-8, 1 shared, inter 2048,
bf16); the 8-token fp8 decode step of the same layer is reported beside it.
Prints one JSON line.  Random-init weights of the layer's architecture and
x ~ N(0,1), as described in synth.py.

roofline: the dominant kernel is the gate/up grouped GEMM (moe_expert_up);
its duration comes from HIP events recorded around it on the stream it runs
on, inside the timed region.  Its algorithmic work per launch is
2*T*K*(2I)*D + 2*T*(2*S*I)*D flops and the bytes of the touched experts'
W1/W3 (plus block scales), the shared W1/W3, x and the written h.  The bound
reported is the ceiling that binds: with all 256 experts touched the prefill
kernel's bytes take longer at 8 TB/s than its flops at 2.5 PFLOP/s, so it is
HBM-bound on the roofline; both fractions are reported.
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

# Measured HBM traffic per launch of the roofline kernels: rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the layer's
# launches), scaled by what the same counters read for a 1 GiB device copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  The commands and per-dispatch values
# are in profiles/.  Each figure is tied to a hash of its kernel's source and is
# reported as null once that source has changed.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
COUNTERS = {
    "prefill_up": {"sources": ("gemm_mfma2.hip", "common.hpp"),
                   "sha256": "5ea999a830e876989880a17369a4bd9983bda3dcbcad28bb01a761a5f0239d24",
                   "fetch_kib": 14221656, "write_kib": 362496,
                   "profile": "profiles/gemm_mfma2_gate_up_v3_prefill_T8192_counters.md"},
    "decode_up": {"sources": ("gemm_skinny.hip", "common.hpp"),
                  "sha256": "59dfca776df8586e4571956ac60856b9efcde10db974a41401e24df0a446861b",
                  "fetch_kib": 847312, "write_kib": 3744,
                  "profile": "profiles/gemm_skinny_gate_up_v3_decode_T8_counters.md"},
    "w8a8_up": {"sources": ("gemm_fp8.hip", "common.hpp"),
                "sha256": "c5818489c1ece2dde52e881ed7511c33516576c68d06cbbbbf1a52b4dd3c85ca",
                "fetch_kib": 9022782, "write_kib": 195868,
                "profile": "profiles/gemm_fp8_gate_up_v3_prefill_w8a8_T8192_counters.md"},
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
    ap.add_argument("--cpu-tokens", type=int, default=48)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration)")
    return ap.parse_args()


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

    def step(self, ev_up=None):
        B, L = self.B, self.layer
        B.moe_gate(self.cfg, self.T, L.x, L.w_gate, L.bias, self.logits, self.idx, self.tw)
        B.moe_permute(self.cfg, self.T, self.idx, self.r)
        if self.cfg.act_quant:
            B.moe_quant_act(self.cfg, self.T, L.x, self.r)
        if ev_up is not None:
            ev_up[0].record()
        B.moe_expert_up(self.cfg, self.T, L.x, self.r, self.w, self.h, self.hs)
        if ev_up is not None:
            ev_up[1].record()
        B.moe_expert_down(self.cfg, self.T, self.r, self.w, self.h, self.hs, self.y, self.z)
        B.moe_combine(self.cfg, self.T, L.x, self.z, self.y, self.r, self.tw, self.out)


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


def time_pass(p: Pass, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        p.step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        p.step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    up_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return total_ms, up_ms, wall


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
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        one()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / calls
    P = T * K
    up = 2 * P * 2 * I * D + 2 * T * 2 * S * I * D
    down = 2 * P * D * I + 2 * T * D * S * I
    flops = 3 * up + 2 * down + 4 * T * E * D
    res = {"what": "moe_backward: dx, dW_gate, routed and shared dW13/dW2 for one upstream gradient",
           "ms_per_call": ms, "tokens_per_s": T / (ms / 1e3), "gemm_flops": flops,
           "tflops": flops / (ms / 1e3) / 1e12, "mfma_frac": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
           "workspace_bytes": ws.numel()}
    del grads, ws
    torch.cuda.empty_cache()
    return res


def time_ep_shard(args):
    """One GPU's share of the V3 prefill layer under expert parallelism (32 local
    experts, the tokens dispatched to them, no shared expert): the same step
    sequence on that share, without the collectives that would feed it."""
    import torch
    from routed_expert_moe_amd import configs, synth
    shape = configs.V3_EP_SHARD_BF16
    layer = synth.make_layer(shape, device="cuda")
    p = Pass(layer)
    total_ms, up_ms, _ = time_pass(p, args.steps, args.warmup)
    fig = work_figures(layer, p.r.counts.cpu().numpy())
    ms = total_ms / args.steps
    res = {"workload": shape.name, "T": shape.T, "n_routed": shape.n_routed, "top_k": shape.top_k,
           "what": "one GPU's expert-parallel share of v3_prefill_bf16_T8192 (a local routing of the "
                   "dispatched tokens stands in for the global gate; no collectives)",
           "ms_per_step": ms, "pairs": shape.T * shape.top_k, "experts_touched": fig["touched"],
           "layer_tflops": fig["flops_layer"] / (ms / 1e3) / 1e12,
           "roofline": roofline(fig["flops_up"], fig["bytes_up"], up_ms, None,
                                "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_mfma2_kernel)")}
    del p, layer
    torch.cuda.empty_cache()
    return res


def cpu_baseline(layer, n_tokens: int):
    """The float64 oracle on the first n_tokens tokens of the same workload, on host cores."""
    import numpy as np
    import threadpoolctl
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
    import oracle
    from oracle_bridge import bias_f64, expert_fn, shared_pair, spec_of, to_f64
    x = to_f64(layer.x[:n_tokens])
    wg = to_f64(layer.w_gate)
    b = bias_f64(layer)
    shared = shared_pair(layer)
    t0 = time.perf_counter()
    oracle.moe_layer(x, wg, b, expert_fn(layer), shared, spec_of(layer.shape))
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"first {n_tokens} tokens of the {layer.shape.name} workload, whole layer "
                       f"(gate, {layer.shape.top_k} routed + shared SwiGLU experts, combine) in "
                       f"float64; expert weights decoded from device copies inside the timed call; "
                       f"{dt:.1f} s")}


def copy_probe(mib: int):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs the single-GPU layer forward only; --gpus {args.gpus} is not supported "
              f"(no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    from routed_expert_moe_amd import binding as B
    from routed_expert_moe_amd import configs, synth
    B.lib()

    # ---- prefill: the headline workload
    shape = configs.V3_PREFILL_BF16
    progress(f"building {shape.name}")
    layer = synth.make_layer(shape, device="cuda")
    progress(f"timing {shape.name}")
    p = Pass(layer)
    total_ms, up_ms, wall = time_pass(p, args.steps, args.warmup)
    counts = p.r.counts.cpu().numpy()
    fig = work_figures(layer, counts)
    ms = total_ms / args.steps
    tok_s = shape.T * args.steps / (total_ms / 1e3)
    res = {
        "metric": "MoE-layer tokens/s + % MFMA peak (prefill), % HBM GB/s (decode), 1 MI355X",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": shape.name, "T": shape.T, "dim": shape.dim, "n_routed": shape.n_routed,
                   "n_groups": shape.n_groups, "topk_groups": shape.topk_groups, "top_k": shape.top_k,
                   "n_shared": shape.n_shared, "inter_dim": shape.inter_dim, "score": shape.score,
                   "route_scale": shape.route_scale, "experts_touched": fig["touched"]},
        "layer": {"tflops": fig["flops_layer"] / (ms / 1e3) / 1e12,
                  "mfma_frac": fig["flops_layer"] / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                  "gbs": fig["bytes_layer"] / (ms / 1e3) / 1e9,
                  "hbm_frac": fig["bytes_layer"] / (ms / 1e3) / 1e9 / PEAK_HBM_GBS},
        "roofline": roofline(fig["flops_up"], fig["bytes_up"], up_ms, measured_traffic("prefill_up"),
                             "moe_expert_up (gate/up grouped GEMM + SwiGLU, gemm_mfma2_kernel)"),
        "wall_s": wall,
    }
    res["bias_update"] = time_bias_update(p, shape)
    res["balance_loss"] = time_balance_loss(p, shape)
    progress("timing the backward")
    res["backward"] = time_backward(p, shape)
    del p
    torch.cuda.empty_cache()

    # ---- the same prefill batch in FP8 W8A8 (fp8 weights, activations quantised 1x128)
    wshape = configs.V3_PREFILL_W8A8
    progress(f"building {wshape.name}")
    wlayer = synth.make_layer(wshape, device="cuda")
    progress(f"timing {wshape.name}")
    wp = Pass(wlayer)
    wtotal_ms, wup_ms, _ = time_pass(wp, args.steps, args.warmup)
    wfig = work_figures(wlayer, wp.r.counts.cpu().numpy())
    wms = wtotal_ms / args.steps
    res["prefill_w8a8"] = {
        "workload": wshape.name, "T": wshape.T,
        "dtype": "fp8-e4m3 weights (128x128 fp32 scales) x fp8-e4m3 activations (1x128 fp32 scales)",
        "ms_per_step": wms, "tokens_per_s": wshape.T * args.steps / (wtotal_ms / 1e3),
        "experts_touched": wfig["touched"],
        "layer_tflops": wfig["flops_layer"] / (wms / 1e3) / 1e12,
        "layer_mfma_frac_fp8": wfig["flops_layer"] / (wms / 1e3) / 1e12 / PEAK_FP8_TFLOPS,
        "roofline": roofline(wfig["flops_up"], wfig["bytes_up"], wup_ms, measured_traffic("w8a8_up"),
                             "moe_expert_up (fp8 x fp8 grouped GEMM + SwiGLU + h quantisation, gemm_fp8_kernel)",
                             PEAK_FP8_TFLOPS),
    }
    del wp, wlayer
    torch.cuda.empty_cache()

    # ---- decode: 8 tokens, fp8 expert weights
    dshape = configs.V3_DECODE_FP8
    progress(f"building {dshape.name}")
    dlayer = synth.make_layer(dshape, device="cuda")
    progress(f"timing {dshape.name}")
    dp = Pass(dlayer)
    dsteps = args.decode_steps or 10 * args.steps
    dtotal_ms, dup_ms, _ = time_pass(dp, dsteps, max(args.warmup, 3))
    dfig = work_figures(dlayer, dp.r.counts.cpu().numpy())
    dms = dtotal_ms / dsteps
    res["decode"] = {
        "workload": dshape.name, "T": dshape.T, "dtype": "fp8-e4m3 weights (128x128 fp32 scales), bf16 act",
        "steps": dsteps, "ms_per_step": dms, "tokens_per_s": dshape.T * dsteps / (dtotal_ms / 1e3),
        "experts_touched": dfig["touched"],
        "layer_gbs": dfig["bytes_layer"] / (dms / 1e3) / 1e9,
        "layer_hbm_frac": dfig["bytes_layer"] / (dms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "roofline": roofline(dfig["flops_up"], dfig["bytes_up"], dup_ms, measured_traffic("decode_up"),
                             "moe_expert_up (fp8 weight-streaming gate/up + SwiGLU, gemm_skinny_kernel)"),
    }
    del dp, dlayer
    torch.cuda.empty_cache()
    progress("timing the expert-parallel share")
    res["ep_shard"] = time_ep_shard(args)
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(layer, args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
