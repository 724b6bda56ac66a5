#!/usr/bin/env python3
"""Benchmark of the sparse MoE feed-forward layer on one MI355X.

One step = one moe_forward of the whole layer (router logits, softmax, top-k,
normalised weights, grouped SwiGLU experts, sigmoid-gated shared expert,
combine) over one batch of seeded synthetic tokens already resident in HBM.

Prints ONE JSON line.  `value` is tokens/s on the decode-shaped layer
(T=32, d_model 2560, 512 experts top-10, width 640, shared 640, bf16); the
prefill-shaped layer (T=4096) is reported inside the same line under "also".
`roofline` is for the dominant kernel of the step, timed with HIP events
recorded on the library's stream at its stage boundaries during the timed
loop.  `cpu_baseline` times the CPU oracle on the host cores.

`--config 9` (reported by default under "also") times the training backward
pass of the prefill-shaped layer: one moe_backward call (dx and every weight
gradient, plus the load-balancing loss) for the routing of its batch, with the
gate/up pre-activations its moe_forward_train saved.

`--config 7` measures the decode layer with its pre-FFN RMSNorm (one call:
moe_forward_prenorm); `--config 6` measures the same decode layer with MXFP4 expert weights
(moe_forward_mx4); its algorithmic weight bytes are 17/32 byte per element
(a 4-bit code plus one scale byte per 32 elements).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C]
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def sources_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_feed_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, stage: str):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary, if one exists for the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"counters_{stage}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"sources_sha256:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != sources_digest():
        return None
    return float(b.group(1))


def algorithmic(cfg, U: int):
    """Algorithmic HBM bytes and FLOPs of one call and of its gate/up and down
    stages: distinct routed experts touched (U), the shared expert, router,
    gate vector, x, out (fp32), topk_idx and topk_w."""
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.Fs
    b = 2                                              # bf16 activations, router
    bw = 17 / 32 if cfg.dtype == "mxfp4" else b        # bytes per expert weight
    gu_w = int(U * 2 * F * d * bw + 2 * Fs * d * bw)
    dn_w = int(U * d * F * bw + d * Fs * bw)
    call_bytes = gu_w + dn_w + E * d * b + d * b + T * d * b + T * d * 4 + T * k * 8
    flops_gu = 2 * T * k * 2 * F * d + 2 * T * 2 * Fs * d
    flops_dn = 2 * T * k * F * d + 2 * T * Fs * d
    call_flops = 2 * T * d * (E + 1) + flops_gu + flops_dn
    # the down stage's weighted per-pair rows y (T*k rows: binary32 on the
    # weight-streaming path, else 16-bit block floating point, 2d + d/8 bytes
    # a row) are traffic of this design (the combine reads them back), not of
    # the method: they are left out of its algorithmic bytes and reported as
    # down_impl_bytes
    return dict(call_bytes=call_bytes, call_flops=call_flops,
                gate_up_bytes=gu_w + T * d * b + (T * k * F + T * Fs) * b,
                gate_up_flops=flops_gu,
                down_bytes=dn_w + (T * k * F + T * Fs) * b + T * d * 4,
                down_impl_bytes=T * k * (4 * d if T * k <= 16 * E else 2 * d + d // 8),
                down_flops=flops_dn)


def algorithmic_backward(cfg, U: int):
    """Algorithmic HBM bytes and FLOPs of one backward call (the contractions
    of the gradient itself: 2x the forward's FLOPs; the recomputed gate/up
    pre-activations and router logits are not counted) and of its three
    single-kernel stages.  Bytes: each weight of a touched expert read once,
    every weight gradient written (zeros for experts no token chose), x and
    dout read, dx written."""
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.Fs
    b = 2
    rows, rows_sh = T * k, T
    w_gu, w_dn = U * 2 * F * d * b + 2 * Fs * d * b, U * d * F * b + d * Fs * b
    g_gu, g_dn = E * 2 * F * d * b + 2 * Fs * d * b, E * d * F * b + d * Fs * b
    dgu_bytes = (rows * 2 * F + rows_sh * 2 * Fs) * b
    call_bytes = (w_gu + w_dn + 2 * E * d * b + 2 * d * b + g_gu + g_dn
                  + T * d * b + T * d * 4 + T * d * 4 + T * k * 8)
    f_gu = 2 * (rows * 2 * F * d + rows_sh * 2 * Fs * d)
    f_dn = 2 * (rows * d * F + rows_sh * d * Fs)
    call_flops = 2 * (f_gu + f_dn) + 2 * 2 * T * d * (E + 1)
    return dict(call_bytes=call_bytes, call_flops=call_flops,
                dx_rows_bytes=w_gu + dgu_bytes + (rows + rows_sh) * d * b, dx_rows_flops=f_gu,
                dw_gate_up_bytes=g_gu + dgu_bytes + (rows + rows_sh) * d * b,
                dw_gate_up_flops=f_gu,
                dw_down_bytes=g_dn + (rows + rows_sh) * d * 4 + (rows * F + rows_sh * Fs) * b,
                dw_down_flops=f_dn)


def measure_backward(cfg, dev_layer, steps, warmup):
    import numpy as np
    import torch

    import sparse_moe_feed_amd as moe
    import workloads as W

    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    x = to(W.make_x(cfg.T, cfg.d, cfg.dtype, cfg.seed_x))
    dout = torch.from_numpy(W.dout_for(cfg)).cuda()
    L = dev_layer
    # the training forward of this batch: its routing and its saved gate/up
    # pre-activations are the backward pass's inputs
    _, idx, w, saved = moe.forward_train(x, L["w_router"], L["w_gate_up"], L["w_down"], cfg.k,
                                         L["w_sh_gate_up"], L["w_sh_down"], L["sh_gate"])
    shape = moe.shape_of(x, L["w_gate_up"], cfg.k, L["w_sh_gate_up"])
    ws = torch.empty(moe.backward_workspace_size(shape, cfg.T), dtype=torch.uint8, device="cuda")
    grads = moe.backward(x, L["w_router"], L["w_gate_up"], L["w_down"], idx, w, dout,
                         L["w_sh_gate_up"], L["w_sh_down"], L["sh_gate"], aux_coef=cfg.aux_coef,
                         ws=ws, saved=saved)
    aux = grads.pop("aux_loss")

    def step():
        moe.backward(x, L["w_router"], L["w_gate_up"], L["w_down"], idx, w, dout,
                     L["w_sh_gate_up"], L["w_sh_down"], L["sh_gate"], aux_coef=cfg.aux_coef,
                     ws=ws, grads=grads, aux_loss=aux, saved=saved)
    for _ in range(warmup):
        step()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    n_ev = 1 + len(moe.BACKWARD_STAGES)
    evs = [[moe.HipEvent() for _ in range(n_ev)] for _ in range(steps)]
    for i in range(steps):
        moe.stage_events(evs[i])
        step()
    torch.cuda.synchronize()
    stage_ms = {name: sum(e[j].elapsed_ms(e[j + 1]) for e in evs) / steps
                for j, name in enumerate(moe.BACKWARD_STAGES)}
    U = int(np.unique(idx.cpu().numpy()).size)
    return dict(ms=ms, stage_ms=stage_ms, U=U)


def roofline_backward(cfg, r, workload):
    a = algorithmic_backward(cfg, r["U"])
    stage = max(("dx_rows", "dw_gate_up", "dw_down"), key=lambda s: r["stage_ms"][s])
    t = r["stage_ms"][stage] * 1e-3
    by, fl = a[f"{stage}_bytes"], a[f"{stage}_flops"]
    bound = "hbm" if by / (HBM_PEAK_GBS * 1e9) >= fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=round(by / t / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(by / t / (HBM_PEAK_GBS * 1e9), 4))
    else:
        roof = dict(bound="mfma", achieved=round(fl / t / 1e12, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(fl / t / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4))
    roof.update(traffic=committed_traffic(workload, stage), kernel=stage,
                kernel_ms=round(r["stage_ms"][stage], 4), alg_bytes=by, alg_flops=fl)
    call_t = r["ms"] * 1e-3
    layer = dict(hbm_frac=round(a["call_bytes"] / call_t / (HBM_PEAK_GBS * 1e9), 4),
                 mfma_frac=round(a["call_flops"] / call_t / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                 alg_bytes=a["call_bytes"], alg_flops=a["call_flops"], unique_experts=r["U"])
    return roof, layer


def measure(cfg, dev_layer, steps, warmup):
    import numpy as np
    import torch

    import sparse_moe_feed_amd as moe
    import workloads as W

    x_np = W.make_x(cfg.T, cfg.d, cfg.dtype, cfg.seed_x)
    bias_np = W.make_bias(cfg)
    to = lambda a: None if a is None else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    x = to(x_np)
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    gamma = to(W.make_norm_weight(cfg.d, cfg.dtype, cfg.seed_w)) if cfg.prenorm else None
    L = moe.MoELayer(dev_layer["w_router"], dev_layer["w_gate_up"], dev_layer["w_down"], cfg.k,
                     dev_layer["w_sh_gate_up"], dev_layer["w_sh_down"], dev_layer["sh_gate"], bias,
                     max_tokens=cfg.T, norm_weight=gamma)
    out = torch.empty(cfg.T, cfg.d, device="cuda")
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, cfg.k, device="cuda")
    for _ in range(warmup):
        L(x, out, idx, w)
    # the timed steps: nothing but the layer calls between the two events
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        L(x, out, idx, w)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    # a second pass of the same steps with HIP events recorded by the library
    # at its stage boundaries (on its own stream) for the per-stage split
    n_ev = 1 + len(moe.STAGES)
    evs = [[moe.HipEvent() for _ in range(n_ev)] for _ in range(steps)]
    for i in range(steps):
        moe.stage_events(evs[i])
        L(x, out, idx, w)
    torch.cuda.synchronize()
    stage_ms = {name: sum(e[j].elapsed_ms(e[j + 1]) for e in evs) / steps
                for j, name in enumerate(moe.STAGES)}
    U = int(np.unique(idx.cpu().numpy()).size)
    return dict(ms=ms, wall_ms=wall * 1e3 / steps, stage_ms=stage_ms, U=U)


def roofline_of(cfg, r, workload):
    a = algorithmic(cfg, r["U"])
    stage = max(("gate_up", "down"), key=lambda s: r["stage_ms"][s])
    t = r["stage_ms"][stage] * 1e-3
    by, fl = a[f"{stage}_bytes"], a[f"{stage}_flops"]
    hbm_frac = by / t / (HBM_PEAK_GBS * 1e9)
    mfma_frac = fl / t / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if by / (HBM_PEAK_GBS * 1e9) >= fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    traffic = committed_traffic(workload, stage)
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=round(by / t / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(hbm_frac, 4))
    else:
        roof = dict(bound="mfma", achieved=round(fl / t / 1e12, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(mfma_frac, 4))
    roof.update(traffic=traffic, kernel=stage, kernel_ms=round(r["stage_ms"][stage], 4),
                alg_bytes=by, alg_flops=fl)
    call_t = r["ms"] * 1e-3
    layer = dict(hbm_frac=round(a["call_bytes"] / call_t / (HBM_PEAK_GBS * 1e9), 4),
                 mfma_frac=round(a["call_flops"] / call_t / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                 alg_bytes=a["call_bytes"], alg_flops=a["call_flops"], unique_experts=r["U"])
    return roof, layer


def measure_ceiling(nbytes=1 << 30, reps=20):
    """Practical HBM ceilings on this GPU, GB/s: a streaming read of nbytes
    by the whole chip (moe_read_probe), a device-to-device copy (bytes read +
    bytes written) and a fill (bytes written), each averaged over reps
    launches timed with events on the current stream."""
    import torch

    import sparse_moe_feed_amd as moe

    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(moe.READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")

    def rate(fn, moved):
        fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return round(moved * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)

    r = dict(read_GBs=rate(lambda: moe.read_probe(src, sink), nbytes),
             copy_GBs=rate(lambda: dst.copy_(src), 2 * nbytes),
             write_GBs=rate(lambda: dst.zero_(), nbytes), bytes=nbytes)
    del src, dst
    torch.cuda.empty_cache()
    return r


def cpu_baseline(cfg, layer_np, seconds):
    import oracle
    import workloads as W

    if cfg.backward:
        return cpu_baseline_backward(cfg, layer_np, seconds)
    # a bounded sample: the first tokens of the batch (a token's output does
    # not depend on the others), about 1-2 s of oracle work per pass
    n = min(cfg.T, 32)
    x = W.make_x(n, cfg.d, cfg.dtype, cfg.seed_x)
    bias = W.make_bias(cfg)
    if cfg.dtype == "mxfp4":
        fwd = oracle.forward_mx4
        args = (x, layer_np["w_router"], layer_np["gu"], layer_np["dn"], cfg.k, layer_np["sgu"],
                layer_np["sdn"], layer_np["sh_gate"])
    else:
        fwd = oracle.forward
        args = (x, layer_np["w_router"], layer_np["w_gate_up"], layer_np["w_down"], cfg.k,
                layer_np["w_sh_gate_up"], layer_np["w_sh_down"], layer_np["sh_gate"])
    if cfg.prenorm:
        gamma, base = W.make_norm_weight(cfg.d, cfg.dtype, cfg.seed_w), fwd
        fwd = lambda h, *a, bias=None: base(oracle.rmsnorm(h, gamma), *a, bias=bias)
    reps, t0 = 0, time.perf_counter()
    while True:
        fwd(*args, bias=bias)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    what = f"all {cfg.T} tokens" if n == cfg.T else f"the first {n} of {cfg.T} tokens"
    return dict(value=round(reps * n / el, 2), unit="tokens/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"{what} of {cfg.name}, {reps} full passes in {el:.1f} s")


def cpu_baseline_backward(cfg, layer_np, seconds):
    """The oracle's backward pass on the first 8 tokens of the batch as a
    batch of their own (routing, loss statistics and every gradient of that
    batch; routed weight gradients of the experts those tokens chose)."""
    import numpy as np

    import oracle
    import workloads as W

    n = min(cfg.T, 8)
    x = W.make_x(n, cfg.d, cfg.dtype, cfg.seed_x)
    dout = W.dout_for(cfg)[:n]
    L = layer_np
    idx, w = oracle.route(x, L["w_router"], cfg.k)
    experts = np.unique(idx)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.backward(x, L["w_router"], L["w_gate_up"], L["w_down"], idx, w, dout,
                        L["w_sh_gate_up"], L["w_sh_down"], L["sh_gate"], aux_coef=cfg.aux_coef,
                        experts=experts)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=round(reps * n / el, 2), unit="tokens/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"backward of the first {n} of {cfg.T} tokens of {cfg.name} as one batch, "
                       f"{reps} full passes in {el:.1f} s")


def device_layer(cfg, layer_np):
    """The layer's weights on the GPU: bf16 tensors, or (codes, scales) uint8
    pairs for MXFP4 expert weights."""
    import numpy as np
    import torch

    bf = lambda a: None if a is None else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if cfg.dtype == "mxfp4":
        u8 = lambda t: None if t is None else (torch.from_numpy(t[0]).cuda(),
                                               torch.from_numpy(t[1]).cuda())
        return dict(w_router=bf(layer_np["w_router"]), sh_gate=bf(layer_np["sh_gate"]),
                    w_gate_up=u8(layer_np["gu"]), w_down=u8(layer_np["dn"]),
                    w_sh_gate_up=u8(layer_np["sgu"]), w_sh_down=u8(layer_np["sdn"]))
    return {n: bf(layer_np[n]) for n in ("w_router", "w_gate_up", "w_down", "w_sh_gate_up",
                                         "w_sh_down", "sh_gate")}


def layer_key(cfg):
    return (cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.dtype, cfg.seed_w)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload of `value` (2 = decode T=32)")
    ap.add_argument("--also", default="3,4,5,9", help="extra workloads reported in the line")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the practical HBM read / copy / write ceilings (GB/s)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="leave the ceiling measurement out of the line (profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (HBM counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4}))
        return
    if args.ceiling:
        print(json.dumps({"ceiling": measure_ceiling()}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (the layer is not sharded across GPUs in this "
              f"build); got --gpus {args.gpus}, WORLD_SIZE {world}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W

    cfg = W.CONFIGS[args.config]
    layer_np = W.layer_for(cfg)
    dev_layer = device_layer(cfg, layer_np)
    run = lambda c, steps: (measure_backward if c.backward else measure)(c, dev_layer, steps,
                                                                        args.warmup)
    roof_of = lambda c, rr: (roofline_backward if c.backward else roofline_of)(c, rr, c.name)
    r = run(cfg, args.steps)
    roof, layer = roof_of(cfg, r)
    also = {}
    for c in [int(v) for v in args.also.split(",") if v]:
        c_cfg = W.CONFIGS[c]
        if layer_key(c_cfg) != layer_key(cfg):
            print(f"bench.py: --also {c} skipped ({c_cfg.name} uses another layer)",
                  file=sys.stderr)
            continue
        rc = run(c_cfg, max(3, args.steps // 2))
        rroof, rlayer = roof_of(c_cfg, rc)
        also[c_cfg.name] = dict(value=round(c_cfg.T / (rc["ms"] * 1e-3), 1), unit="tokens/s",
                                ms_per_step=round(rc["ms"], 4), roofline=rroof, layer=rlayer,
                                stage_ms={k: round(v, 4) for k, v in rc["stage_ms"].items()})
    del dev_layer
    torch.cuda.empty_cache()
    ceiling = None if args.no_ceiling else measure_ceiling()
    base = None if args.no_cpu_baseline else cpu_baseline(cfg, layer_np, args.cpu_seconds)
    line = {
        "metric": "MoE-layer tokens/s at T=32 decode and T=4096 prefill; % HBM / MFMA peak",
        "value": round(cfg.T / (r["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) tokens, N(0,0.02^2) weights (random init, no checkpoint)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "top_k": cfg.k, "d_expert": cfg.F, "d_shared": cfg.Fs, "router_bias": cfg.bias,
                   "expert_weights": "mxfp4" if cfg.dtype == "mxfp4" else "bf16",
                   "pre_norm": "rmsnorm" if cfg.prenorm else None,
                   "pass": "backward" if cfg.backward else "forward"},
        "roofline": roof,
        "layer": layer,
        "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
        "also": also,
        "ceiling": ceiling,
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
