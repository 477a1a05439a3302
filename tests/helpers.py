"""Glue between the seeded inputs and the oracle / the binding (tests only)."""

import numpy as np

import oracle
from mixture_experts_layer_11_amd import inputs


def expert_fn(layer):
    def f(e):
        ew = layer.expert(e)
        return ew.w1, ew.w3, ew.w2, ew.w1_s, ew.w3_s, ew.w2_s
    return f


def shared_tuple(layer):
    s = layer.shared
    if s is None:
        return None
    return s.w1, s.w3, s.w2, s.w1_s, s.w3_s, s.w2_s


def oracle_kwargs(cfg):
    return dict(act_dtype=cfg.act_dtype, w_dtype=cfg.w_dtype, router_dtype=cfg.router_dtype,
                E=cfg.E, n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, topk=cfg.topk,
                score_func=cfg.score_func, route_scale=cfg.route_scale)


def run_oracle(layer, tokens=None, route=None, accumulate="f32"):
    return oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer),
                              shared_tuple(layer), tokens=tokens, route=route,
                              accumulate=accumulate, **oracle_kwargs(layer.cfg))


def gate_oracle(layer, tokens=None):
    cfg = layer.cfg
    x = layer.x if tokens is None else layer.x[tokens]
    xv = oracle.moe_oracle.decode_act(x, cfg.act_dtype)
    wrv = oracle.moe_oracle.decode_act(layer.wr, cfg.router_dtype)
    return oracle.gate(xv, wrv, layer.bias, score_func=cfg.score_func, n_groups=cfg.n_groups,
                       topk_groups=cfg.topk_groups, topk=cfg.topk, route_scale=cfg.route_scale)


# Layer-output bars (max over tokens of ||dy||_inf/||r||_inf, sum|dy|/sum|r|).
# bf16 and fp32 layers: the bars the method's statement sets.  fp8 layers: the
# stated 5e-2 replaces the max bar.  The mean bar is set from what identical
# quantisation on both sides leaves: x is quantised bit-exactly, and h differs
# only where the fp32 summation order of its K-long dot products moves it
# across an e4m3 rounding boundary (one code, 1/16-1/8 of the value).  Over
# K = 7168 that is measured at mean 1.2e-3 on the full-size fp8 workload and
# 1.5e-4 - 5.3e-4 on the small ones; the three plausible quantisation mistakes
# give 2.2e-2 - 4.8e-2 (test_oracle_mutations.py).  5e-3 sits 4x above the
# first and 4.5x below the second; the stated 5e-2 as a mean bar would admit
# an unquantised h.
BF16_BAR = (2e-2, 2e-3)
FP8_BAR = (5e-2, 5e-3)


def bar(cfg):
    return FP8_BAR if cfg.w_dtype == "fp8" else BF16_BAR


def record(name, **vals):
    """Print an observed parity figure and append it as a JSON line to the file
    named by $MOE_PARITY_LOG (when set)."""
    import json
    import os
    line = json.dumps({"test": name, **{k: (float(v) if isinstance(v, (float, np.floating)) else v)
                                        for k, v in vals.items()}})
    print(line, flush=True)
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def rel_errors(y, r):
    """(max over rows of ||y_t - r_t||_inf / ||r_t||_inf, sum|y-r| / sum|r|)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    d = np.abs(y - r)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((d.max(axis=1) / den).max()), float(d.sum() / max(np.abs(r).sum(), 1e-30))


def tiny_cfg(name="t", **kw):
    base = dict(name=name, T=16, dim=128, E=8, n_groups=2, topk_groups=1, topk=2,
                score_func="sigmoid", route_scale=1.0, bias_range=0.1, inter=128,
                inter_shared=128, act_dtype="f32", w_dtype="f32", router_dtype="f32",
                seed=777)
    base.update(kw)
    return inputs.MoEConfig(**base)


# ---------------------------------------------------------------------------
# parity rule for routing (margins from the oracle's own values)
# ---------------------------------------------------------------------------

MARGIN = 1e-5
# Weights come from fp32 logits whose summation order is free; a logit
# difference dz moves a softmax weight by ~2*dz relative and a renormalised
# sigmoid weight by <= dz.  The bar admits dz up to the routing margin.
WEIGHT_RTOL = 2 * MARGIN


def _group_scores(sp_row, cfg, has_bias):
    g = sp_row.reshape(cfg.n_groups, cfg.E // cfg.n_groups).astype(np.float64)
    if has_bias:
        return np.sort(g, axis=1)[:, -2:].sum(axis=1)
    return g.max(axis=1)


def check_routing(cfg, o_w, o_idx, info, g_idx, g_w, bias):
    """Compare GPU routing with the oracle's.

    Decided tokens (oracle group and expert margins > 1e-5): the chosen sets
    must be equal and the weights per expert within WEIGHT_RTOL relative.  Other
    tokens: the GPU's choice must be admissible within the margin - every
    chosen expert's s' at least the oracle's k-th best s' minus the margin,
    at most topk_groups groups, each with a group score at least the oracle's
    topk_groups-th best minus the margin - and its weights must be the
    oracle's scores of the experts the GPU chose, formed by the gate's rule.
    Returns the boolean mask of tokens whose sets agree.
    """
    T = o_idx.shape[0]
    dec = np.minimum(info["margin_group"], info["margin_expert"]) > MARGIN
    o_sorted = np.sort(o_idx, axis=1)
    g_sorted = np.sort(g_idx, axis=1)
    same = np.all(o_sorted == g_sorted, axis=1)
    bad = np.nonzero(dec & ~same)[0]
    assert bad.size == 0, f"decided tokens routed differently: {bad[:10]}"
    # weights, matched by expert id
    oo = np.argsort(o_idx, axis=1)
    go = np.argsort(g_idx, axis=1)
    ow = np.take_along_axis(o_w, oo, 1).astype(np.float64)
    gw = np.take_along_axis(g_w, go, 1).astype(np.float64)
    rel = np.abs(gw - ow) / np.maximum(np.abs(ow), 1e-30)
    assert rel[same].max(initial=0.0) <= WEIGHT_RTOL, rel[same].max()
    if cfg.score_func == "sigmoid":
        np.testing.assert_allclose(g_w.astype(np.float64).sum(1), cfg.route_scale, rtol=1e-6)
    # distinct ids in range
    assert np.all((g_idx >= 0) & (g_idx < cfg.E))
    assert all(len(set(r)) == cfg.topk for r in g_idx.tolist())
    # admissibility of the rest
    sp = info["s_sel"].astype(np.float64)
    s = info["s"].astype(np.float64)
    gsz = cfg.E // cfg.n_groups
    for t in np.nonzero(~same)[0]:
        kth = np.sort(sp[t][o_idx[t]])[0]
        assert np.all(sp[t][g_idx[t]] >= kth - MARGIN), t
        if cfg.n_groups > 1:
            gs = _group_scores(sp[t], cfg, bias is not None)
            gk = np.sort(gs)[::-1][cfg.topk_groups - 1]
            chosen = set((g_idx[t] // gsz).tolist())
            assert len(chosen) <= cfg.topk_groups, t
            assert all(gs[g] >= gk - MARGIN for g in chosen), t
        # the GPU's weights are the gate's rule applied to the experts it chose
        ws = s[t][g_idx[t]]
        if cfg.score_func == "sigmoid":
            ws = ws / ws.sum()
        ws = ws * cfg.route_scale
        np.testing.assert_allclose(g_w[t].astype(np.float64), ws, rtol=WEIGHT_RTOL, err_msg=str(t))
    return same
