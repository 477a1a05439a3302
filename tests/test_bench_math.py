"""The benchmark's algorithmic work counts, recomputed matrix by matrix.

bench.py counts FLOPs and HBM bytes of one forward from the layer shape and
the run's per-expert row counts; here the same quantities are summed again
per weight matrix and per tensor, so a dropped term, a wrong factor or a
wrong byte size in bench.py shows up.  CPU only.
"""

import numpy as np
import pytest

import bench
from mixture_experts_layer_11_amd import inputs


def _per_matrix(cfg, counts):
    wsz = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.w_dtype]
    asz = 4 if cfg.act_dtype == "f32" else 2
    rsz = 4 if cfg.router_dtype == "f32" else 2
    d, i, s = cfg.dim, cfg.inter, cfg.inter_shared
    flops = 2.0 * cfg.T * d * cfg.E                       # router projection
    nbytes = cfg.E * d * rsz + cfg.T * d * asz            # router weights, x
    nbytes += cfg.T * d * asz                             # y
    for m in counts:                                      # routed experts
        for rows, cols in ((i, d), (i, d), (d, i)):       # W1, W3, W2 [out, in]
            flops += 2.0 * m * rows * cols
            if m > 0:
                nbytes += rows * cols * wsz
                if cfg.w_dtype == "fp8":
                    nbytes += 4 * (rows // 128) * (cols // 128)
    for rows, cols in ((s, d), (s, d), (d, s)):           # shared expert
        flops += 2.0 * cfg.T * rows * cols
        nbytes += rows * cols * wsz
        if cfg.w_dtype == "fp8":
            nbytes += 4 * (rows // 128) * (cols // 128)
    return flops, nbytes


@pytest.mark.parametrize("name", [c.name for c in inputs.CONFIGS])
def test_counts_match_per_matrix_sums(name):
    cfg = inputs.config_by_name(name)
    rng = np.random.default_rng(5)
    counts = rng.multinomial(cfg.T * cfg.topk, np.ones(cfg.E) / cfg.E)
    counts[:3] = 0                                        # some idle experts
    counts[3] += cfg.T * cfg.topk - counts.sum()
    r = bench.workload_numbers(cfg, counts)
    flops, nbytes = _per_matrix(cfg, counts)
    assert r["flops"] == pytest.approx(flops, rel=1e-12)
    assert r["bytes"] == pytest.approx(nbytes, rel=1e-12)
    assert r["active_experts"] == int((counts > 0).sum())


@pytest.mark.parametrize("name", [c.name for c in inputs.CONFIGS])
def test_up_launch_bytes_are_w1_w3_and_x(name):
    """The up launch's algorithmic bytes: W1 and W3 of every expert that gets
    rows, the shared W1 and W3, and x; no intermediate buffer."""
    cfg = inputs.config_by_name(name)
    counts = np.random.default_rng(2).multinomial(cfg.T * cfg.topk, np.ones(cfg.E) / cfg.E)
    counts[:2] = 0
    counts[2] += cfg.T * cfg.topk - counts.sum()
    wsz = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.w_dtype]
    asz = 4 if cfg.act_dtype == "f32" else 2
    want = cfg.T * cfg.dim * asz
    mats = [(cfg.inter, cfg.dim)] * 2 * int((counts > 0).sum()) + [(cfg.inter_shared, cfg.dim)] * 2
    for rows, cols in mats:
        want += rows * cols * wsz + (4 * (rows // 128) * (cols // 128) if cfg.w_dtype == "fp8" else 0)
    assert bench.workload_numbers(cfg, counts)["up_bytes"] == want


@pytest.mark.parametrize("name,tflop,gbytes", [
    ("c2_dsv3_prefill_T4096", 3.262, 22.76),
    ("c3_skewed_softmax_T8192", 1.136, 1.21),
    ("c4_dsv3_fp8_T8192", 6.524, 11.56),
])
def test_all_experts_active_totals(name, tflop, gbytes):
    """With every expert receiving rows the totals are fixed by the shapes alone."""
    cfg = inputs.config_by_name(name)
    counts = np.full(cfg.E, cfg.T * cfg.topk // cfg.E)
    counts[0] += cfg.T * cfg.topk - counts.sum()
    r = bench.workload_numbers(cfg, counts)
    assert r["flops"] / 1e12 == pytest.approx(tflop, abs=5e-4)
    assert r["bytes"] / 1e9 == pytest.approx(gbytes, abs=5e-3)


def test_expert_range_splits_the_routed_part():
    """Two halves of the expert range add up to the whole routed work."""
    cfg = inputs.config_by_name("c2_dsv3_prefill_T4096")
    counts = np.random.default_rng(1).multinomial(cfg.T * cfg.topk, np.ones(cfg.E) / cfg.E)
    full = bench.workload_numbers(cfg, counts)
    a = bench.workload_numbers(cfg, counts, (0, cfg.E // 2))
    b = bench.workload_numbers(cfg, counts, (cfg.E // 2, cfg.E))
    none = bench.workload_numbers(cfg, counts, (0, 0))
    routed = lambda r: r["flops"] - none["flops"]
    assert routed(a) + routed(b) == pytest.approx(routed(full), rel=1e-12)


def test_floor_takes_the_binding_roof():
    cfg = inputs.config_by_name("c2_dsv3_prefill_T4096")
    res = dict(flops=2.5e15 * 1e-3, bytes=8e12 * 2e-3, ms=4.0)   # 1 ms of MFMA, 2 ms of HBM
    f = bench.floors(cfg, res)
    assert f["binding"] == "hbm" and f["t_floor_ms"] == pytest.approx(2.0)
    assert f["roofline_frac"] == pytest.approx(0.5)


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    """The roofline object's measured HBM traffic comes from profiles/traffic.json
    and must turn null once the expert-kernel sources hash differently from the
    hash recorded with the counters."""
    import json
    import os
    path = os.path.join(bench.ROOT, "profiles", "traffic.json")
    with open(path) as f:
        rec = json.load(f)
    key = "up_grouped_gemm@c1_dsv3_decode_T128"
    assert key in rec, "the decode up launch's traffic record is missing"
    ent = rec[key]
    assert ent["hbm_bytes_per_launch"] > 0 and len(ent["source_sha"]) == 16
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: ent["source_sha"])
    assert bench.traffic_for("up_grouped_gemm", "c1_dsv3_decode_T128") == ent["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.traffic_for("up_grouped_gemm", "c1_dsv3_decode_T128") is None
    assert bench.traffic_for("up_grouped_gemm", "no_such_workload") is None


def test_kernel_source_hash_covers_every_expert_kernel_source():
    """The hash behind the traffic record covers the files the expert kernels
    are compiled from, the combine header included."""
    assert set(bench.KERNEL_SOURCES) >= {"ffn.hip", "common.h", "kernels.h", "combine.h"}
