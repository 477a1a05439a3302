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


def run_oracle(layer, tokens=None, route=None):
    return oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer),
                              shared_tuple(layer), tokens=tokens, route=route,
                              **oracle_kwargs(layer.cfg))


def gate_oracle(layer, tokens=None):
    cfg = layer.cfg
    x = layer.x if tokens is None else layer.x[tokens]
    xv = oracle.moe_oracle.decode_act(x, cfg.act_dtype)
    wrv = oracle.moe_oracle.decode_act(layer.wr, cfg.router_dtype)
    return oracle.gate(xv, wrv, layer.bias, score_func=cfg.score_func, n_groups=cfg.n_groups,
                       topk_groups=cfg.topk_groups, topk=cfg.topk, route_scale=cfg.route_scale)


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
