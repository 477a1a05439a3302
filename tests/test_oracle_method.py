"""Pins of the oracle's layer arithmetic: gate, dispatch, experts, combine.

Nothing here compares the oracle with itself re-typed: each check is brute
force, a closed form, an invariant the pages state, a textbook routine, or a
hand-computed case.  The check functions are also used by
test_oracle_mutations.py, which plants plausible mistakes in the oracle and
asserts that these checks catch them.
"""

import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from mixture_experts_layer_11_amd import inputs
from tests.helpers import expert_fn, gate_oracle, oracle_kwargs, run_oracle, shared_tuple, tiny_cfg

F32 = np.float32

# tiny selection problems: (E, n_groups, topk_groups, topk, bias?, score_func)
TINY_SELECT = [
    (16, 4, 2, 4, True, "sigmoid"),      # the c0 grouping
    (16, 4, 2, 4, False, "sigmoid"),     # no bias: group score = max
    (12, 3, 2, 3, True, "softmax"),      # softmax with groups and bias
    (12, 3, 1, 2, False, "softmax"),
    (10, 1, 1, 3, True, "sigmoid"),      # no group limit
    (8, 1, 1, 8, False, "softmax"),      # topk = E
    (16, 8, 3, 5, True, "sigmoid"),      # groups of two experts
]


def _rand_scores(rng, T, E, func):
    z = rng.standard_normal((T, E)).astype(F32)
    return oracle.scores(z, func)


# ---------------------------------------------------------------------------
# check functions (shared with the mutation tests)
# ---------------------------------------------------------------------------

def check_select_vs_brute_force(seed=0, T=40):
    rng = np.random.default_rng(seed)
    for (E, G, TG, K, has_b, func) in TINY_SELECT:
        s = _rand_scores(rng, T, E, func)
        b = rng.uniform(-0.1, 0.1, E).astype(F32) if has_b else None
        idx, _ = oracle.select_experts(s, b, G, TG, K)
        bf = oracle.brute_force_select(s, b, G, TG, K)
        for t in range(T):
            assert frozenset(idx[t].tolist()) == bf[t], (E, G, TG, K, has_b, func, t)


def check_select_invariants(s, b, G, TG, K, idx):
    T, E = s.shape
    sp = (s + b).astype(F32) if b is not None else s
    gsz = E // G
    for t in range(T):
        row = sp[t].astype(np.float64)
        assert len(set(idx[t].tolist())) == K                                # K distinct
        vals = row[idx[t]]
        assert np.all(np.diff(vals) <= 0)                                     # descending s'
        if G > 1:
            grp = row.reshape(G, gsz)
            gs = np.sort(grp, 1)[:, -2:].sum(1) if b is not None else grp.max(1)
            chosen_groups = set((idx[t] // gsz).tolist())
            assert len(chosen_groups) <= TG
            # the experts come from groups that rank among the TG best
            order = np.argsort(-gs, kind="stable")
            assert chosen_groups <= set(order[:TG].tolist())
            cand = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in order[:TG]])
        else:
            cand = np.arange(E)
        other = np.setdiff1d(cand, idx[t])
        if other.size:
            assert vals.min() >= row[other].max()                             # top-k property


def check_weight_invariants(s, idx, w, func, rs):
    sel = np.take_along_axis(s, idx.astype(np.int64), 1).astype(np.float64)
    if func == "sigmoid":
        np.testing.assert_allclose(w.astype(np.float64).sum(1), rs, rtol=2e-6)
        np.testing.assert_allclose(w / rs, sel / sel.sum(1, keepdims=True), rtol=2e-6)
    else:
        np.testing.assert_allclose(w, sel * rs, rtol=1e-7)


def check_bias_selects_only(seed=1):
    """The bias moves selection; the weights come from the unbiased scores."""
    rng = np.random.default_rng(seed)
    T, E, G, TG, K = 64, 16, 4, 2, 4
    s = _rand_scores(rng, T, E, "sigmoid")
    b = rng.uniform(-0.1, 0.1, E).astype(F32)
    idx, info = oracle.select_experts(s, b, G, TG, K)
    w = oracle.routing_weights(s, idx, "sigmoid", 2.5)
    check_weight_invariants(s, idx, w, "sigmoid", 2.5)
    # a huge bias on expert 5 forces its selection; its weight is its unbiased share
    b2 = b.copy()
    b2[5] = 10.0
    idx2, _ = oracle.select_experts(s, b2, G, TG, K)
    assert np.all((idx2 == 5).any(1))
    w2 = oracle.routing_weights(s, idx2, "sigmoid", 2.5)
    sel = np.take_along_axis(s, idx2.astype(np.int64), 1).astype(np.float64)
    k5 = (idx2 == 5).argmax(1)
    np.testing.assert_allclose(w2[np.arange(T), k5], 2.5 * s[:, 5] / sel.sum(1), rtol=2e-6)
    # shifting every bias by the same constant leaves decided routing unchanged
    idx3, _ = oracle.select_experts(s, (b + F32(0.25)).astype(F32), G, TG, K)
    dec = np.minimum(info["margin_group"], info["margin_expert"]) > 1e-5
    assert dec.sum() > T // 2
    for t in np.nonzero(dec)[0]:
        assert set(idx3[t]) == set(idx[t])


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------

def test_router_logits_one_hot_and_linearity():
    rng = np.random.default_rng(0)
    wr = rng.standard_normal((8, 32)).astype(F32)
    x = np.eye(32, dtype=np.float64)[:5]
    np.testing.assert_array_equal(oracle.router_logits(x, wr), wr[:, :5].T)   # z = x W^T
    x2 = rng.standard_normal((3, 32)).astype(F32)
    z = oracle.router_logits(np.r_[x2, 2 * x2], wr)
    np.testing.assert_array_equal(z[3:], 2 * z[:3])                           # exact x2 scaling
    assert z.dtype == np.float32


def test_scores_closed_forms():
    z = np.array([[0.0, 1.0, -1.0, 20.0, -20.0]], F32)
    s = oracle.scores(z, "sigmoid")
    assert s[0, 0] == 0.5
    np.testing.assert_allclose(s, expit(z.astype(np.float64)), rtol=1e-7)
    np.testing.assert_allclose(s[0, 1] + s[0, 2], 1.0, rtol=1e-7)
    rng = np.random.default_rng(1)
    z = (rng.standard_normal((20, 64)) * 3).astype(F32)
    sm = oracle.scores(z, "softmax")
    np.testing.assert_allclose(sm.sum(1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(sm, softmax(z.astype(np.float64), axis=1), rtol=1e-6)
    np.testing.assert_allclose(oracle.scores(z + F32(5.0), "softmax"), sm, rtol=1e-5)


def test_select_matches_brute_force():
    check_select_vs_brute_force(seed=0)
    check_select_vs_brute_force(seed=1)


def test_select_invariants_dsv3_shape():
    rng = np.random.default_rng(2)
    s = _rand_scores(rng, 48, 256, "sigmoid")
    b = rng.uniform(-0.05, 0.05, 256).astype(F32)
    idx, _ = oracle.select_experts(s, b, 8, 4, 8)
    check_select_invariants(s, b, 8, 4, 8, idx)
    idx, _ = oracle.select_experts(s, None, 8, 4, 8)
    check_select_invariants(s, None, 8, 4, 8, idx)


def test_select_ties_prefer_lower_index():
    s = np.full((1, 16), 0.5, F32)
    idx, info = oracle.select_experts(s, None, 4, 2, 3)
    assert idx[0].tolist() == [0, 1, 2]
    assert info["margin_expert"][0] == 0.0 and info["margin_group"][0] == 0.0
    idx, _ = oracle.select_experts(s, np.zeros(16, F32), 1, 1, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]


def test_group_score_is_top2_sum_with_bias_and_max_without():
    # group 0: one huge score; group 1: two good scores.  Top-2 sum prefers
    # group 1, max prefers group 0.
    s = np.array([[0.9, 0.0, 0.0, 0.0, 0.6, 0.6, 0.0, 0.0]], F32)
    idx_b, _ = oracle.select_experts(s, np.zeros(8, F32), 2, 1, 2)
    idx_n, _ = oracle.select_experts(s, None, 2, 1, 2)
    assert set(idx_b[0]) == {4, 5}
    assert set(idx_n[0]) == {0, 1}


def test_weight_invariants_sigmoid_and_softmax():
    rng = np.random.default_rng(3)
    for func, rs in (("sigmoid", 2.5), ("softmax", 1.0), ("sigmoid", 1.0)):
        s = _rand_scores(rng, 30, 16, func)
        b = rng.uniform(-0.1, 0.1, 16).astype(F32)
        idx, _ = oracle.select_experts(s, b, 4, 2, 4)
        check_select_invariants(s, b, 4, 2, 4, idx)
        w = oracle.routing_weights(s, idx, func, rs)
        assert w.dtype == np.float32
        check_weight_invariants(s, idx, w, func, rs)


def test_bias_affects_selection_not_weights():
    check_bias_selects_only()


def test_c0_gate_invariants():
    layer = inputs.draw_layer(inputs.config_by_name("c0"))
    w, idx, info = gate_oracle(layer)
    c = layer.cfg
    check_select_invariants(info["s"], layer.bias, c.n_groups, c.topk_groups, c.topk, idx)
    check_weight_invariants(info["s"], idx, w, c.score_func, c.route_scale)
    bf = oracle.brute_force_select(info["s"], layer.bias, c.n_groups, c.topk_groups, c.topk)
    assert all(frozenset(idx[t].tolist()) == bf[t] for t in range(c.T))


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def check_permute(idx, E, counts, offsets, sorted_token, row_of):
    T, K = idx.shape
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * K
    np.testing.assert_array_equal(np.diff(offsets), counts)
    assert sorted(row_of.ravel().tolist()) == list(range(T * K))          # each (t,k) once
    for t in range(T):
        for k in range(K):
            p = row_of[t, k]
            e = idx[t, k]
            assert sorted_token[p] == t and offsets[e] <= p < offsets[e + 1]
    for e in range(E):
        seg = sorted_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                                   # ascending tokens


def test_permute_definition():
    rng = np.random.default_rng(4)
    for T, E, K in ((50, 16, 4), (7, 64, 6), (1, 8, 8), (33, 3, 2)):
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        out = oracle.permute(idx, E)
        check_permute(idx, E, *out)
    counts, offsets, st, ro = oracle.permute(np.zeros((0, 4), np.int32), 8)
    assert counts.sum() == 0 and offsets.tolist() == [0] * 9 and st.size == 0


# ---------------------------------------------------------------------------
# experts and combine
# ---------------------------------------------------------------------------

def test_ffn_hand_example():
    """dim 2, inter 1: FFN(x) = W2 * silu(w1.x) * (w3.x), computed by hand."""
    w1 = np.array([[0.5, -1.0]], np.float32)
    w3 = np.array([[2.0, 0.25]], np.float32)
    w2 = np.array([[1.5], [-0.75]], np.float32)
    x = np.array([[1.0, -0.5]])
    a, b = 0.5 * 1.0 + 1.0 * 0.5, 2.0 * 1.0 - 0.25 * 0.5
    h = a / (1.0 + math.exp(-a)) * b
    got = oracle.expert_ffn(x, w1, w3, w2, "f32", "f32")
    np.testing.assert_allclose(got[0], np.float32([1.5 * h, -0.75 * h]), rtol=1e-7)
    # bf16 layer: h rounded to bf16 once, output rounded to bf16
    got = oracle.expert_ffn(x, w1, w3, w2, "f32", "bf16")
    hb = float(oracle.bf16_round(h))
    np.testing.assert_array_equal(got[0], oracle.bf16_round([1.5 * hb, -0.75 * hb]))


def test_silu_textbook():
    a = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.moe_oracle.silu(a), a * expit(a), rtol=1e-14, atol=1e-300)


def _identical_experts_layer(cfg):
    layer = inputs.draw_layer(cfg)
    for e in range(cfg.E):
        layer.w1[e], layer.w3[e], layer.w2[e] = layer.w1[0], layer.w3[0], layer.w2[0]
    return layer


def test_identical_experts_closed_form():
    """All routed experts equal => y = route_scale * FFN(x) + S(x) for sigmoid (weights sum to rs)."""
    cfg = tiny_cfg(T=20, route_scale=2.0)
    layer = _identical_experts_layer(cfg)
    r = run_oracle(layer)
    xv = layer.x.astype(np.float64)
    f = oracle.expert_ffn(xv, layer.w1[0], layer.w3[0], layer.w2[0], "f32", "f32")
    sh = oracle.expert_ffn(xv, layer.shared.w1, layer.shared.w3, layer.shared.w2, "f32", "f32")
    np.testing.assert_allclose(r["y"], 2.0 * f + sh, rtol=2e-5, atol=2e-6)


def test_dense_formula_matches_sparse_loop():
    """y_routed = sum_i G_i E_i (dense gate matrix) equals the per-expert loop."""
    for cfg in (tiny_cfg(T=24), tiny_cfg(T=17, n_groups=1, topk=3, score_func="softmax",
                                          bias_range=None, act_dtype="bf16", w_dtype="bf16",
                                          router_dtype="bf16", inter_shared=0),
                inputs.config_by_name("c0")):
        layer = inputs.draw_layer(cfg)
        r = run_oracle(layer)
        d = oracle.moe_forward_dense(layer.x, layer.wr, layer.bias, expert_fn(layer),
                                     shared_tuple(layer), **oracle_kwargs(cfg))
        np.testing.assert_array_equal(r["idx"], d["idx"])
        np.testing.assert_allclose(r["y32"], d["y_exact"], rtol=1e-5, atol=1e-6)


def test_topk_equal_E_is_dense_weighted_sum():
    cfg = tiny_cfg(T=9, E=4, n_groups=1, topk_groups=1, topk=4, score_func="softmax",
                   bias_range=None, inter_shared=0)
    layer = inputs.draw_layer(cfg)
    r = run_oracle(layer)
    xv = layer.x.astype(np.float64)
    p = softmax(xv @ layer.wr.astype(np.float64).T, axis=1)
    y = sum(p[:, e:e + 1] * oracle.expert_ffn(xv, layer.w1[e], layer.w3[e], layer.w2[e],
                                               "f32", "f32") for e in range(4))
    np.testing.assert_allclose(r["y"], y, rtol=1e-5, atol=1e-6)


def test_routed_part_linear_in_route_scale_and_zero_gives_shared():
    cfg1 = tiny_cfg(T=12, route_scale=1.0)
    l1 = inputs.draw_layer(cfg1)
    r1 = run_oracle(l1)
    l1.cfg = tiny_cfg(T=12, route_scale=2.0)
    r2 = run_oracle(l1)
    l1.cfg = tiny_cfg(T=12, route_scale=0.0)
    r0 = run_oracle(l1)
    sh = oracle.expert_ffn(l1.x.astype(np.float64), l1.shared.w1, l1.shared.w3, l1.shared.w2,
                           "f32", "f32")
    np.testing.assert_array_equal(r0["y"], np.float32(sh).astype(np.float64))
    # doubling is exact in fp32: routed(rs=2) = 2 * routed(rs=1)
    routed1 = (r1["y32"] - np.float32(sh)).astype(np.float64)
    routed2 = (r2["y32"] - np.float32(sh)).astype(np.float64)
    np.testing.assert_allclose(routed2, 2 * routed1, rtol=1e-5, atol=1e-6)


def test_route_override_reproduces_own_routing():
    layer = inputs.draw_layer(inputs.SMALL_CONFIGS[1].with_T(40))
    r = run_oracle(layer)
    r2 = run_oracle(layer, route=(r["w"], r["idx"]))
    np.testing.assert_array_equal(r["y"], r2["y"])
    sub = [3, 17, 39]
    r3 = run_oracle(layer, tokens=sub)
    np.testing.assert_array_equal(r3["y"], r["y"][sub])


def test_fp8_expert_close_to_unquantised():
    """fp8 FFN (weights 128x128 blocks, activations 1x128) stays within e4m3 error of fp32."""
    rng = np.random.default_rng(7)
    dim, inter = 256, 256
    a1 = (rng.standard_normal((inter, dim)) / 16).astype(np.float32)
    a3 = (rng.standard_normal((inter, dim)) / 16).astype(np.float32)
    a2 = (rng.standard_normal((dim, inter)) / 16).astype(np.float32)
    x = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(rng.standard_normal((8, dim)).astype(np.float32)))
    q1, s1 = inputs.quantize_weight_blocks(a1)
    q3, s3 = inputs.quantize_weight_blocks(a3)
    q2, s2 = inputs.quantize_weight_blocks(a2)
    got = oracle.expert_ffn(x.astype(np.float64), q1, q3, q2, "fp8", "bf16", s1, s3, s2)
    ref = oracle.expert_ffn(x.astype(np.float64), a1, a3, a2, "f32", "f32")
    rel = np.abs(got - ref).sum() / np.abs(ref).sum()
    assert 1e-3 < rel < 0.1


# ---------------------------------------------------------------------------
# layer-dtype accumulator ([v3] MoE.forward; reading R9)
# ---------------------------------------------------------------------------

def _v3_combine_in_torch(outs, w, idx, shared, dtype):
    """The V3 class's combine (hackaday.io log, MoE.forward), written with torch
    on the CPU from its definition: an expert-contiguous permutation of the
    (token, slot) pairs (a stable sort of the expert ids), then for each
    expert in ascending id one vectorised update of its tokens' rows - the
    running sum, held in the layer dtype, plus output times weight, evaluated
    in fp32 by torch's type promotion and stored back in the layer dtype - and
    finally the shared output added with torch's own bf16 addition."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    T, K, dim = outs.shape
    o = torch.from_numpy(outs.astype(np.float32)).to(tdt)        # exact: values are layer dtype
    wt = torch.from_numpy(w.astype(np.float32))
    ids = torch.from_numpy(idx.astype(np.int64)).reshape(-1)
    perm = torch.sort(ids, stable=True).indices                  # expert-contiguous pairs
    counts = torch.bincount(ids, minlength=int(ids.max()) + 1).tolist()
    y = torch.zeros((T, dim), dtype=tdt)
    start = 0
    for c in counts:
        seg = perm[start:start + c]
        start += c
        if c == 0:
            continue
        tok, slot = seg // K, seg % K
        y[tok] = (y[tok] + o[tok, slot] * wt[tok, slot].unsqueeze(1)).to(tdt)
    z = torch.from_numpy(shared.astype(np.float32)).to(tdt)
    return torch.add(y, z).float().numpy().astype(np.float64)


def check_combine_layer_matches_torch(dtype="bf16", seed=3):
    rng = np.random.default_rng(seed)
    T, E, K, dim = 37, 24, 6, 40
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.01, 1.5, (T, K)).astype(F32)
    raw = rng.standard_normal((T, K, dim)) * 3.0
    outs = oracle.round_to(raw, dtype)
    shared = oracle.round_to(rng.standard_normal((T, dim)), dtype)
    got = oracle.combine_layer(outs, w, idx, shared, dtype)
    ref = _v3_combine_in_torch(outs, w, idx, shared, dtype)
    np.testing.assert_array_equal(got, ref)
    return got


def test_combine_layer_matches_torch_v3_statements_bf16():
    check_combine_layer_matches_torch("bf16")


def test_combine_layer_matches_torch_v3_statements_f32():
    check_combine_layer_matches_torch("f32", seed=4)


def test_combine_layer_single_expert_is_identity():
    rng = np.random.default_rng(9)
    T, dim = 11, 16
    outs = oracle.round_to(rng.standard_normal((T, 1, dim)), "bf16")
    idx = rng.integers(0, 8, (T, 1)).astype(np.int32)
    w = np.ones((T, 1), F32)
    got = oracle.combine_layer(outs, w, idx, np.zeros((T, dim)), "bf16")
    np.testing.assert_array_equal(got, outs[:, 0])


def test_combine_layer_differs_from_fp32_accumulator_within_rounding():
    # the two accumulators agree up to the extra bf16 roundings (K + 1 of them)
    rng = np.random.default_rng(12)
    T, E, K, dim = 64, 32, 8, 48
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(F32)
    outs = oracle.round_to(rng.standard_normal((T, K, dim)), "bf16")
    sh = oracle.round_to(rng.standard_normal((T, dim)), "bf16")
    a = oracle.combine_layer(outs, w, idx, sh, "bf16")
    b = oracle.round_to(oracle.combine(outs, w, idx, sh).astype(np.float64), "bf16")
    scale = np.abs(outs).sum(1).max(-1, keepdims=True) + np.abs(sh).max(-1, keepdims=True)
    assert np.all(np.abs(a - b) <= (K + 2) * 2.0 ** -8 * scale)
    assert np.any(a != b)          # and they are different methods


# ---------------------------------------------------------------------------
# expert ranges ([v3] constructor and forward: a rank's experts only)
# ---------------------------------------------------------------------------

def test_expert_ranges_partition_the_routed_sum():
    from tests.helpers import expert_fn, oracle_kwargs
    layer = inputs.draw_layer(tiny_cfg("ranges", T=40, E=16, n_groups=4, topk_groups=2, topk=4))
    kw = oracle_kwargs(layer.cfg)
    full = oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer), None, **kw)
    same = oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer), None,
                              experts=(0, 16), **kw)
    np.testing.assert_array_equal(full["y32"], same["y32"])
    parts = [oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer), None,
                                experts=(b, b + 4), **kw)["y32"].astype(np.float64)
             for b in range(0, 16, 4)]
    total = np.sum(parts, axis=0)
    # the same terms summed in another grouping: equal up to fp32 rounding
    scale = np.abs(full["y32"]).max()
    assert np.abs(total - full["y32"]).max() <= 1e-5 * scale
    # each part only holds its experts' terms
    empty = oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer), None,
                               experts=(5, 5), **kw)
    assert not np.any(empty["y32"])
