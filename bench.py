"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1] [--no-cpu-baseline]

One step = one moe_forward call (gate, dispatch, routed + shared SwiGLU
experts, combine) over one batch of T synthetic tokens, with inputs and
weights already resident in HBM.  Prints one JSON line.

roofline: the dominant kernel is the up-projection grouped GEMM (it streams
W1 and W3 of every expert that receives a token, two thirds of the layer's
weight bytes).  Its algorithmic bytes per launch divided by its average
launch time (HIP events recorded around that launch on its own stream during
the timed steps) against the MI355X HBM peak of 8 TB/s.

measured_peaks: what the machine delivers, next to the published peaks - the
library's streaming-read kernel over 4 GiB and a dense 8192^3 bf16 GEMM.
--graph times replays of one forward captured in a HIP graph instead of eager
calls.
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

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
METRIC = "MoE-layer tokens/sec, DeepSeek-V3 shape T=4096 bf16 + T=128 decode; % MFMA/HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--also", default="c0,c2,c3,c4",
                    help="extra configs timed after the main one ('' = none)")
    ap.add_argument("--experts", default="",
                    help="b:e - time one expert-parallel rank's share: only routed experts b..e-1 "
                         "(their weights alone are uploaded); the gate still covers all experts")
    ap.add_argument("--graph", action="store_true",
                    help="capture one forward in a HIP graph and time its replays")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings (streaming read, dense bf16 GEMM)")
    ap.add_argument("--dispatch", default="",
                    help="comma-separated hand-made dispatches of the config's T*topk rows, timed on the "
                         "routed expert step alone (moe_expert_ffn): 'even' = every expert the same rows, "
                         "an integer d = experts alternately d rows below and above that")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 5 times (reference for HBM byte counters)")
    return ap.parse_args()


def up_kernel_name(cfg):
    """Name of the up-projection kernel the library launches for cfg (the
    library's rule, on R = T * topk routed rows: 256-token bf16 stream tiles
    once experts average >= 384 rows, 128-token x 512-row ones from 64 rows,
    128-token x 256-row ones from 32, 64-token ones from 8, 16-token skinny
    tiles below; fp8
    192-token stream tiles from 12 rows; bf16 tiles need widths that are
    multiples of 64)."""
    R, E = cfg.T * cfg.topk, cfg.E
    if cfg.w_dtype == "fp8":
        return "moe::stream_fp8_kernel<true>" if R >= 12 * E else "moe::up_skinny_fp8_kernel"
    if cfg.w_dtype == "bf16" and cfg.dim % 64 == 0 and cfg.inter % 64 == 0 and cfg.inter_shared % 64 == 0:
        if R >= 384 * E:
            return "moe::stream_bf16_kernel<256-token tiles, up>"
        if R >= 64 * E:
            return "moe::stream_bf16_kernel<128-token x 512-row tiles, up>"
        if R >= 32 * E:
            return "moe::stream_bf16_kernel<128-token tiles, up>"
        if R >= 8 * E:
            return "moe::stream_bf16_kernel<64-token tiles, up>"
    return "moe::up_skinny_kernel<%s>" % ("float" if cfg.w_dtype == "f32" else "unsigned short")


def workload_numbers(cfg, counts, experts=None):
    """Algorithmic FLOPs and bytes of one forward, and of the up-projection launch
    (experts=(b, e): only the routed experts of that range)."""
    if experts is not None:
        counts = counts.copy()
        counts[:experts[0]] = 0
        counts[experts[1]:] = 0
    wsz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.w_dtype]
    asz = 4 if cfg.act_dtype == "f32" else 2
    rsz = 4 if cfg.router_dtype == "f32" else 2
    T, dim, E, K, I, Is = cfg.T, cfg.dim, cfg.E, cfg.topk, cfg.inter, cfg.inter_shared
    active = int((counts > 0).sum())
    scale_b = 0
    if cfg.w_dtype == "fp8":
        scale_b = 4 * (dim // 128) * (I // 128)          # per matrix per expert
    per_expert = 3 * (I * dim * wsz + scale_b)
    shared = 3 * Is * dim * wsz + (3 * 4 * (dim // 128) * (Is // 128) if cfg.w_dtype == "fp8" else 0)
    routed_rows = int(counts.sum())                         # T * K for the full range
    flops = 2 * T * E * dim + 2 * routed_rows * 3 * dim * I + 2 * T * 3 * dim * Is
    bytes_ = active * per_expert + shared + E * dim * rsz + T * dim * asz * 2
    shared_scale_b = 4 * (dim // 128) * (Is // 128) if cfg.w_dtype == "fp8" else 0
    # up launch: W1 and W3 of the active experts and of the shared expert, x read
    # once (h is an intermediate buffer: not algorithmic)
    up_bytes = active * 2 * (I * dim * wsz + scale_b) + 2 * (Is * dim * wsz + shared_scale_b) + T * dim * asz
    up_flops = 2 * routed_rows * 2 * dim * I + 2 * T * 2 * dim * Is
    return dict(active_experts=active, flops=flops, bytes=bytes_, up_bytes=up_bytes,
                up_flops=up_flops, per_expert_up_bytes=2 * (I * dim * wsz + scale_b))


KERNEL_SOURCES = ("ffn.hip", "common.h", "kernels.h", "combine.h")   # what the expert kernels are built from


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "mixture_experts_layer_11_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM traffic from the committed rocprofv3 counter runs, if the kernel
    sources are unchanged since they were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sha = kernel_source_sha()
    ent = rec.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent["hbm_bytes_per_launch"]


def run_config(cfg, steps, warmup, torch, moe, inputs, want_layer=False, experts=None,
               graph=False):
    layer = inputs.draw_layer(cfg)
    dw = moe.upload_layer(layer, experts=experts)
    p = moe.Params.from_config(cfg)
    if experts is not None:
        p.expert_begin, p.expert_end = experts
    ws = moe.alloc_workspace(p, cfg.T)
    x = moe.to_device(layer.x, cfg.act_dtype)
    y = torch.empty((cfg.T, cfg.dim), dtype=p.act_torch, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        moe.moe_forward(p, x, dw, ws, y=y, counts=counts)
    torch.cuda.synchronize()
    step = lambda: moe.moe_forward(p, x, dw, ws, y=y, counts=counts)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            moe.moe_forward(p, x, dw, ws, y=y, counts=counts)
        torch.cuda.synchronize()
        step = g.replay
    if not graph:
        moe.moe_profile_start(steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    wall0 = time.perf_counter()
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if graph:
        # the per-kernel events are host-side records, absent from a replay:
        # time the expert kernels over the same number of eager calls
        moe.moe_profile_start(steps)
        for _ in range(steps):
            moe.moe_forward(p, x, dw, ws, y=y, counts=counts)
        torch.cuda.synchronize()
    ncalls, up_ms, dn_ms = moe.moe_profile_stop()
    ms = ev[0].elapsed_time(ev[steps]) / steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    c = counts.cpu().numpy()
    res = dict(ms=ms, ms_median=per_step[len(per_step) // 2], ms_min=per_step[0],
               wall_ms=wall * 1e3 / steps, up_ms=up_ms / max(ncalls, 1),
               down_ms=dn_ms / max(ncalls, 1), counts=c, **workload_numbers(cfg, c, experts))
    if not want_layer:
        del dw, ws, x, y
        torch.cuda.empty_cache()
        return res, None
    return res, layer


def measured_peaks(torch, moe):
    """What the machine delivers, beside the published peaks: the library's
    streaming-read kernel over a 4 GiB buffer (every byte once), and a dense
    8192^3 bf16 GEMM through torch.matmul (hipBLASLt).  Best of 5 runs each."""
    stream = torch.cuda.current_stream()

    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            out.append(a.elapsed_time(b))
        return min(out)

    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    read_ms = best_ms(lambda: moe.moe_stream_read(buf, sink))
    del buf
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    gemm_ms = best_ms(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_read_GBs": round(nbytes / (read_ms / 1e3) / 1e9, 1),
            "hbm_read_frac_of_peak": round(nbytes / (read_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_gemm_TFLOPs": round(2 * n ** 3 / (gemm_ms / 1e3) / 1e12, 1),
            "bf16_gemm_frac_of_peak": round(2 * n ** 3 / (gemm_ms / 1e3) / 1e12
                                            / MFMA_PEAK_TFLOPS["bf16"], 4),
            "how": "moe_stream_read over 4 GiB; torch.matmul 8192^3 bf16; best of 5"}


def floors(cfg, res):
    """Roofline floor of one forward: max(algorithmic FLOPs / MFMA peak,
    algorithmic bytes / HBM peak), and which one binds."""
    dt = "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype
    t_mfma = res["flops"] / (MFMA_PEAK_TFLOPS[dt] * 1e12) * 1e3
    t_hbm = res["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3
    return dict(t_floor_ms=round(max(t_mfma, t_hbm), 4), binding="mfma" if t_mfma > t_hbm else "hbm",
                roofline_frac=round(max(t_mfma, t_hbm) / res["ms"], 4),
                hbm_frac=round(res["bytes"] / (res["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                mfma_frac=round(res["flops"] / (res["ms"] / 1e3) / 1e12 / MFMA_PEAK_TFLOPS[dt], 4))


def cpu_baseline(layer, ntok):
    import oracle
    from threadpoolctl import threadpool_info
    cfg = layer.cfg
    tokens = np.arange(ntok)

    def ew(e):
        w = layer.expert(e)
        return w.w1, w.w3, w.w2, w.w1_s, w.w3_s, w.w2_s
    s = layer.shared
    sh = None if s is None else (s.w1, s.w3, s.w2, s.w1_s, s.w3_s, s.w2_s)
    t = time.perf_counter()
    oracle.moe_forward(layer.x, layer.wr, layer.bias, ew, sh, tokens=tokens,
                       act_dtype=cfg.act_dtype, w_dtype=cfg.w_dtype, router_dtype=cfg.router_dtype,
                       E=cfg.E, n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, topk=cfg.topk,
                       score_func=cfg.score_func, route_scale=cfg.route_scale)
    dt = time.perf_counter() - t
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    host = len(os.sched_getaffinity(0))
    ram = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
    # the oracle's parallel work is its BLAS calls: it runs on min(BLAS threads, cores) cores
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(min(blas, host)), "kind": "oracle",
            "host_cores": host, "blas_threads": int(blas), "host_ram_GB": round(ram / 1e9, 1),
            "sample": f"first {ntok} of the {cfg.T} tokens of {cfg.name} (gate, their routed "
                      f"experts and the shared expert), {dt:.1f} s"}


def hand_dispatch(a, torch, moe, inputs):
    """The routed expert step on hand-made dispatches (random distinct tokens per
    expert), one JSON line each: how the up and down launches respond to the
    rows per expert, with the layer's weights and T."""
    cfg = inputs.config_by_name(a.config)
    layer = inputs.draw_layer(cfg)
    dw = moe.upload_layer(layer)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    x = moe.to_device(layer.x, cfg.act_dtype)
    R = cfg.T * cfg.topk
    avg = R // cfg.E
    rng = np.random.default_rng(7)
    for spec in a.dispatch.split(","):
        d = 0 if spec == "even" else int(spec)
        counts = [avg - d if e % 2 == 0 else avg + d for e in range(cfg.E)]
        counts[-1] += R - sum(counts)
        st = np.concatenate([np.sort(rng.choice(cfg.T, size=c, replace=False)) for c in counts]).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        st_d, off_d = torch.from_numpy(st).cuda(), torch.from_numpy(off).cuda()
        out = torch.empty((R, cfg.dim), dtype=p.act_torch, device="cuda")
        for _ in range(a.warmup):
            moe.moe_expert_ffn(p, x, st_d, off_d, dw, ws, out=out)
        torch.cuda.synchronize()
        moe.moe_profile_start(a.steps)
        for _ in range(a.steps):
            moe.moe_expert_ffn(p, x, st_d, off_d, dw, ws, out=out)
        torch.cuda.synchronize()
        n, up, dn = moe.moe_profile_stop()
        print(json.dumps({"workload": cfg.name, "dispatch": spec, "rows_min": min(counts),
                          "rows_max": max(counts), "up_ms": round(up / n, 4),
                          "down_ms": round(dn / n, 4)}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path: the layer is measured on one MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 5}))
        return
    from mixture_experts_layer_11_amd import inputs, moe
    moe.lib()
    if a.dispatch:
        hand_dispatch(a, torch, moe, inputs)
        return
    peaks = None if a.no_peaks else measured_peaks(torch, moe)
    cfg = inputs.config_by_name(a.config)
    experts = tuple(int(v) for v in a.experts.split(":")) if a.experts else None
    res, layer = run_config(cfg, a.steps, a.warmup, torch, moe, inputs, want_layer=True,
                            experts=experts, graph=a.graph)
    tok_s = cfg.T / (res["ms"] / 1e3)
    up_gbs = res["up_bytes"] / (res["up_ms"] / 1e3) / 1e9
    traffic = None if experts else traffic_for("up_grouped_gemm", cfg.name)
    roof = {"bound": "hbm", "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(up_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": up_kernel_name(cfg),
            "kernel_ms": round(res["up_ms"], 4),
            "alg_bytes_per_launch": int(res["up_bytes"])}
    dt = "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt, "data": "synthetic (seeded; random-init weights of the layer shape)",
        "launch": "hip_graph" if a.graph else "eager",
        "config": {"workload": cfg.name, "T": cfg.T, "dim": cfg.dim, "n_experts": cfg.E,
                   "topk": cfg.topk, "n_groups": cfg.n_groups, "topk_groups": cfg.topk_groups,
                   "inter": cfg.inter, "shared_inter": cfg.inter_shared,
                   "active_experts": res["active_experts"],
                   **({"expert_range": list(experts)} if experts else {})},
        "roofline": roof,
        "layer": {**floors(cfg, res), "ms_median": round(res["ms_median"], 4),
                  "ms_min": round(res["ms_min"], 4), "alg_bytes": int(res["bytes"]),
                  "alg_flops": int(res["flops"]), "down_ms": round(res["down_ms"], 4)},
    }
    extra = {}
    for name in [s for s in a.also.split(",") if s]:
        c2 = inputs.config_by_name(name)
        r2, _ = run_config(c2, max(5, a.steps // 2), a.warmup, torch, moe, inputs, graph=a.graph)
        extra[c2.name] = {
            "tokens_per_s": round(c2.T / (r2["ms"] / 1e3), 1), "ms_per_step": round(r2["ms"], 4),
            "ms_median": round(r2["ms_median"], 4), "ms_min": round(r2["ms_min"], 4),
            **floors(c2, r2),
            "up_kernel_ms": round(r2["up_ms"], 4), "down_kernel_ms": round(r2["down_ms"], 4),
            "up_kernel_hbm_frac": round(r2["up_bytes"] / (r2["up_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if extra:
        out["also"] = extra
    # the CPU leg runs after every GPU timing: a GPU left idle for its ~10 s
    # has shown a first timed launch several milliseconds long
    if not a.no_cpu_baseline and not experts:
        out["cpu_baseline"] = cpu_baseline(layer, a.cpu_tokens)
    del layer
    if peaks:
        out["measured_peaks"] = peaks
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
