"""GPU parity of every step against the oracle, at small sizes that span
several tiles and ragged tails, through the C ABI.

Inputs come from the seeded generator or from the oracle; nothing the GPU
computes is fed back into the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_11_amd import inputs, moe
from tests.helpers import (bar, check_routing, expert_fn, gate_oracle, oracle_kwargs, record,
                           rel_errors, run_oracle, shared_tuple, tiny_cfg)

pytestmark = pytest.mark.gpu

DEV = "cuda"

BUILT = list(inputs.SMALL_CONFIGS)
ALL_SMALL = inputs.SMALL_CONFIGS


def within_bar(name, cfg, got, ref, **extra):
    """Layer-dtype outputs against the oracle's, at the bar for cfg; the
    observed errors are recorded either way."""
    mx, mean = rel_errors(got, ref)
    record(name, cfg=cfg.name, max_rel=mx, mean_rel=mean, bar=list(bar(cfg)), **extra)
    assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (name, cfg.name, mx, mean)


def _sync():
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(cfg):
        if cfg.name not in cache:
            layer = inputs.draw_layer(cfg)
            cache[cfg.name] = (layer, moe.upload_layer(layer))
        return cache[cfg.name]
    return get


def _x_dev(layer):
    return moe.to_device(layer.x, layer.cfg.act_dtype)


def shared_only(p, x, dw, ws):
    """The shared expert's output alone, through moe_combine with every routing
    weight 0 and zero expert outputs: each routed term is 0 * 0 = 0 and
    0 + S = S exactly, so y = S (the shared module's output in the layer dtype)."""
    T = x.shape[0]
    row_of = torch.arange(T * p.topk, dtype=torch.int32, device=DEV).reshape(T, p.topk)
    w = torch.zeros((T, p.topk), dtype=torch.float32, device=DEV)
    eo = torch.zeros((T * p.topk, p.dim), dtype=p.act_torch, device=DEV)
    return moe.moe_combine(p, x, eo, row_of, w, dw, ws)


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------

GATE_CFGS = ALL_SMALL + inputs.CONFIGS + [
    tiny_cfg("nobias_groups", T=300, E=64, n_groups=8, topk_groups=3, topk=6, bias_range=None,
             act_dtype="bf16", router_dtype="bf16", w_dtype="bf16", dim=256),
    tiny_cfg("softmax_groups_bias", T=257, E=32, n_groups=4, topk_groups=2, topk=5,
             score_func="softmax", act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
    tiny_cfg("E512_topk1", T=70, E=512, n_groups=8, topk_groups=1, topk=1, dim=128,
             act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
    tiny_cfg("T1", T=1, E=16, n_groups=4, topk_groups=2, topk=4),
    # two experts per lane of the selection wave, the router's K split 16 ways
    tiny_cfg("E128_split16", T=96, E=128, n_groups=4, topk_groups=2, topk=6, dim=1024,
             act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
    # an expert count that leaves the selection wave's last slots partly empty
    tiny_cfg("E200_groups", T=130, E=200, n_groups=8, topk_groups=3, topk=7, dim=512,
             act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
]


@pytest.mark.parametrize("cfg", GATE_CFGS, ids=lambda c: c.name)
def test_gate_parity(cfg):
    wr, bias, _ = inputs.draw_router(cfg)
    x = inputs.draw_x(cfg)
    xv = oracle.moe_oracle.decode_act(x, cfg.act_dtype)
    wrv = oracle.moe_oracle.decode_act(wr, cfg.router_dtype)
    o_w, o_idx, info = oracle.gate(xv, wrv, bias, score_func=cfg.score_func,
                                   n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                                   topk=cfg.topk, route_scale=cfg.route_scale)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    g_idx, g_w = moe.moe_gate(p, moe.to_device(x, cfg.act_dtype), moe.to_device(wr, cfg.router_dtype),
                              None if bias is None else torch.from_numpy(bias).to(DEV), ws)
    _sync()
    same = check_routing(cfg, o_w, o_idx, info, g_idx.cpu().numpy(), g_w.cpu().numpy(), bias)
    assert same.mean() > 0.97
    # order: descending s' on the GPU too
    sp = info["s_sel"]
    gi = g_idx.cpu().numpy()
    vals = np.take_along_axis(sp, gi.astype(np.int64), 1)
    assert np.all(np.diff(vals, axis=1) <= 1e-6)


# Exact ties: duplicated router rows (and equal bias entries) give bit-equal
# logits on both sides, so the header's rule - equal s' (and equal group
# scores) go to the lower id, the chosen ids in descending s' - decides the
# result, which must then match the oracle's bit for bit, order included.
# Checked on every token whose remaining (distinct-value) margins exceed the
# routing margin.

def _tie_layer(kind, act):
    cfg = tiny_cfg(f"ties_{kind}_{act}", T=240, E=16, n_groups=4,
                   topk_groups=1 if kind == "groups" else 2, topk=3, route_scale=2.5,
                   act_dtype=act, router_dtype=act, w_dtype=act, dim=256, seed=31)
    wr, bias, _ = inputs.draw_router(cfg)
    if kind == "pairs":          # experts 2j and 2j+1 are copies
        src = np.arange(16) // 2 * 2
    elif kind == "groups":       # group 1 copies group 0, group 3 copies group 2
        src = np.array([0, 1, 2, 3, 0, 1, 2, 3, 8, 9, 10, 11, 8, 9, 10, 11])
    else:                        # every expert the same, no bias
        src = np.zeros(16, np.int64)
    wr = wr[src].copy()
    bias = None if kind == "all" else bias[src].copy()
    return cfg, wr, bias, inputs.draw_x(cfg)


def _distinct_gaps(v, n):
    """Gaps between the n+1 largest distinct values of v (descending)."""
    u = np.unique(v.astype(np.float64))[::-1]
    return np.diff(u[: n + 1]) * -1.0 if u.size > n else np.full(n, np.inf)


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["pairs", "groups", "all"])
def test_gate_exact_ties_go_to_lower_id(kind, act):
    cfg, wr, bias, x = _tie_layer(kind, act)
    xv = oracle.moe_oracle.decode_act(x, act)
    wrv = oracle.moe_oracle.decode_act(wr, act)
    o_w, o_idx, info = oracle.gate(xv, wrv, bias, score_func=cfg.score_func,
                                   n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                                   topk=cfg.topk, route_scale=cfg.route_scale)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    g_idx, g_w = moe.moe_gate(p, moe.to_device(x, act), moe.to_device(wr, act),
                              None if bias is None else torch.from_numpy(bias).to(DEV), ws)
    _sync()
    gi, gw = g_idx.cpu().numpy(), g_w.cpu().numpy()
    sp = info["s_sel"]
    gsz = cfg.E // cfg.n_groups
    checked = []
    for t in range(cfg.T):
        gs = np.array([np.sort(sp[t, g * gsz:(g + 1) * gsz].astype(np.float64))[-2:].sum()
                       if bias is not None else sp[t, g * gsz:(g + 1) * gsz].max()
                       for g in range(cfg.n_groups)])
        ok = True
        if kind == "groups":
            ok &= bool(_distinct_gaps(gs, 1)[0] > 1e-5)        # best group pair vs the next
        else:
            ok &= bool(info["margin_group"][t] > 1e-5 or kind == "all")
        keep = np.sort(np.argsort(-gs, kind="stable")[: cfg.topk_groups])
        cand = sp[t, (keep[:, None] * gsz + np.arange(gsz)).ravel()]
        ok &= bool(np.all(_distinct_gaps(cand, 3 if kind == "groups" else 2) > 1e-5) or kind == "all")
        if ok:
            checked.append(t)
            np.testing.assert_array_equal(gi[t], o_idx[t], err_msg=f"token {t}")
    checked = np.array(checked)
    record("gate_exact_ties", kind=kind, act=act, tokens_checked=int(checked.size), T=cfg.T)
    assert checked.size >= 0.8 * cfg.T
    np.testing.assert_allclose(gw[checked], o_w[checked], rtol=2e-5)
    if kind == "all":
        assert np.all(gi == np.array([0, 1, 2], np.int32))
        np.testing.assert_allclose(gw, cfg.route_scale / 3, rtol=1e-6)


# ---------------------------------------------------------------------------
# permute (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (63, 16, 4), (64, 16, 4), (65, 32, 8),
                                   (128, 256, 8), (256, 512, 32), (257, 256, 8),
                                   (1000, 256, 8), (4096, 256, 8), (8192, 64, 6),
                                   (777, 512, 32), (300, 3, 3),
                                   (70000, 64, 6)])   # past 2^16 tokens: 274 count blocks
def test_permute_bitexact(T, E, K):
    rng = np.random.default_rng(T * 1000 + E)
    # skewed draws: half the rows favour a few experts
    pref = rng.permutation(E)[: max(K, E // 8)]
    rows = []
    for t in range(T):
        pool = pref if (t % 2 == 0 and pref.size >= K) else np.arange(E)
        rows.append(rng.choice(pool, K, replace=False))
    idx = np.stack(rows).astype(np.int32)
    p = moe.Params(dim=64, n_experts=E, n_groups=1, topk_groups=1, topk=K, inter=64,
                   shared_inter=0, score_func="sigmoid", route_scale=1.0, act_dtype="bf16",
                   router_dtype="bf16", weight_dtype="bf16")
    ws = moe.alloc_workspace(p, T)
    g = moe.moe_permute(p, torch.from_numpy(idx).to(DEV), ws)
    _sync()
    o = oracle.permute(idx, E)
    for a, b, name in zip(g, o, ("counts", "offsets", "sorted_token", "row_of")):
        np.testing.assert_array_equal(a.cpu().numpy().reshape(b.shape), b, err_msg=name)


# ---------------------------------------------------------------------------
# experts (on the oracle's own dispatch)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", BUILT, ids=lambda c: c.name)
def test_expert_ffn_parity(cfg, layers):
    layer, dw = layers(cfg)
    w, idx, info = gate_oracle(layer)
    counts, offsets, sorted_token, row_of = oracle.permute(idx, cfg.E)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    out = moe.moe_expert_ffn(p, _x_dev(layer), torch.from_numpy(sorted_token).to(DEV),
                             torch.from_numpy(offsets).to(DEV), dw, ws)
    sh = shared_only(p, _x_dev(layer), dw, ws) if cfg.inter_shared else None
    _sync()
    out = moe.to_host_values(out)
    xv = oracle.moe_oracle.decode_act(layer.x, cfg.act_dtype)
    ref = np.zeros_like(out, dtype=np.float64)
    for e in range(cfg.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        w1, w3, w2, s1, s3, s2 = expert_fn(layer)(e)
        ref[a:b] = oracle.expert_ffn(xv[sorted_token[a:b]], w1, w3, w2, cfg.w_dtype,
                                     cfg.act_dtype, s1, s3, s2)
    within_bar("expert_ffn", cfg, out, ref)
    if sh is not None:
        s = layer.shared
        sref = oracle.expert_ffn(xv, s.w1, s.w3, s.w2, cfg.w_dtype, cfg.act_dtype,
                                 s.w1_s, s.w3_s, s.w2_s)
        within_bar("expert_ffn_shared", cfg, moe.to_host_values(sh), sref)


# Hand-made dispatches whose expert sizes straddle the m-tile boundaries of
# each tile kind (the average rows per expert R / E picks the kind: 16-token
# tiles below 8, 64-token tiles below 32, 128-token tiles below 64, then
# 128-token x 512-row up tiles with 192-token down tiles below 384, 256-token
# tiles above; fp8 192-token tiles from 12, 16-token fp8 tiles below).  An
# expert of M rows runs as ceil(M / BM) m-tiles of equal size, the last
# taking the rest.  big_bf16_up straddles the 128-row up m-tiles and leaves
# the second 256-column up n-tile a quarter full (inter 320).
TILE_CASES = [
    ("mid_bf16", dict(E=8, topk=2, w_dtype="bf16"), [65, 64, 63, 29, 0, 1, 0, 0]),
    ("big_bf16", dict(E=4, topk=2, w_dtype="bf16"), [193, 0, 385, 622]),
    ("big_bf16_up", dict(E=4, topk=2, w_dtype="bf16", inter=320), [129, 256, 257, 128]),
    ("big_nt_bf16", dict(E=8, topk=2, w_dtype="bf16"), [129, 128, 1, 0, 65, 33, 27, 1]),
    ("huge_bf16", dict(E=4, topk=2, w_dtype="bf16"), [257, 513, 1, 829]),
    ("skinny_bf16", dict(E=8, topk=2, w_dtype="bf16"), [17, 0, 16, 15, 1, 1, 2, 0]),
    ("big_fp8", dict(E=4, topk=2, w_dtype="fp8"), [193, 385, 1, 21]),
    ("skinny_fp8", dict(E=8, topk=2, w_dtype="fp8"), [33, 0, 16, 17, 1, 1, 2, 0]),
]


# the shortest K loops: one to four steps per tile (32- or 64-wide bf16, 128-wide fp8)
SHORT_K_CASES = [
    ("big_bf16_k64", dict(E=4, topk=2, w_dtype="bf16", dim=64, inter=64, inter_shared=64), [193, 0, 385, 622]),
    ("big_bf16_up_k64", dict(E=4, topk=2, w_dtype="bf16", dim=64, inter=64, inter_shared=64), [129, 256, 257, 128]),
    ("huge_bf16_k128", dict(E=4, topk=2, w_dtype="bf16", dim=128, inter=64, inter_shared=128), [257, 513, 1, 829]),
    ("mid_bf16_k64", dict(E=8, topk=2, w_dtype="bf16", dim=64, inter=128, inter_shared=64), [65, 64, 63, 29, 0, 1, 0, 0]),
    ("big_fp8_k128", dict(E=4, topk=2, w_dtype="fp8", dim=128, inter=128, inter_shared=128), [193, 385, 1, 21]),
]


@pytest.mark.parametrize("name,kw,counts", TILE_CASES + SHORT_K_CASES,
                         ids=[c[0] for c in TILE_CASES + SHORT_K_CASES])
def test_expert_ffn_tile_boundaries(name, kw, counts):
    R = sum(counts)
    T = R // kw["topk"]
    kw = dict(dict(dim=256, inter=256, inter_shared=128), **kw)
    cfg = tiny_cfg(name, T=T, n_groups=1, act_dtype="bf16", router_dtype="bf16", seed=4242, **kw)
    layer = inputs.draw_layer(cfg)
    dw = moe.upload_layer(layer)
    rng = np.random.default_rng(99)
    sorted_token = np.concatenate([np.sort(rng.choice(T, size=c, replace=c > T)) for c in counts]
                                  ).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, T)
    out = moe.moe_expert_ffn(p, _x_dev(layer), torch.from_numpy(sorted_token).to(DEV),
                             torch.from_numpy(offsets).to(DEV), dw, ws)
    _sync()
    out = moe.to_host_values(out)
    xv = oracle.moe_oracle.decode_act(layer.x, cfg.act_dtype)
    for e, c in enumerate(counts):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        w1, w3, w2, s1, s3, s2 = expert_fn(layer)(e)
        ref = oracle.expert_ffn(xv[sorted_token[a:b]], w1, w3, w2, cfg.w_dtype, cfg.act_dtype,
                                s1, s3, s2)
        within_bar("expert_ffn_tiles", cfg, out[a:b], ref, expert=e, rows=int(c))


# The h quantisation fused into the fp8 up-projection epilogues (skinny tiles,
# stream tiles with ordinary and with non-temporal weight loads): with W2 the
# identity (e4m3 1.0 on the diagonal, every block scale 1.0) the expert output
# is bf16(h as quantised), element by element.  Both sides quantise per 1x128
# block of h's row; they differ only where fp32 summation order moves an h
# value across an e4m3 rounding boundary (an adjacent code) or a product across
# a bf16 one.  The same output of an oracle that skips the h quantisation is
# checked to miss the GPU's by far, so the comparison can tell the two apart.

def _bf16_ulp(v):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 7)


FUSED_H_CASES = [
    ("skinny", dict(T=40, E=16, n_groups=4, topk_groups=2, topk=4)),        # 10 rows / expert
    ("stream_nt", dict(T=200, E=8, n_groups=2, topk_groups=1, topk=2)),    # 50 rows / expert
    ("stream", dict(T=700, E=8, n_groups=2, topk_groups=1, topk=2)),       # 175 rows / expert
]


@pytest.mark.parametrize("name,kw", FUSED_H_CASES, ids=[c[0] for c in FUSED_H_CASES])
def test_fp8_fused_h_quantisation(name, kw):
    from tests.test_oracle_mutations import _fp8_ffn_with
    n = 256
    cfg = tiny_cfg(f"fp8_h_{name}", dim=n, inter=n, inter_shared=n, act_dtype="bf16",
                   router_dtype="bf16", w_dtype="fp8", seed=4343, **kw)
    layer = inputs.draw_layer(cfg)
    eye = np.zeros((n, n), np.uint8)
    eye[np.arange(n), np.arange(n)] = 0x38                       # e4m3 1.0
    layer.w2[:] = eye
    layer.w2_s[:] = 1.0
    layer.shared.w2 = eye.copy()
    layer.shared.w2_s = np.ones_like(layer.shared.w2_s)
    dw = moe.upload_layer(layer)
    w, idx, info = gate_oracle(layer)
    counts, offsets, sorted_token, row_of = oracle.permute(idx, cfg.E)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    out = moe.moe_expert_ffn(p, _x_dev(layer), torch.from_numpy(sorted_token).to(DEV),
                             torch.from_numpy(offsets).to(DEV), dw, ws)
    sh = shared_only(p, _x_dev(layer), dw, ws)
    _sync()
    xv = oracle.moe_oracle.decode_act(layer.x, cfg.act_dtype)
    no_hq = _fp8_ffn_with("h_unquantised")
    got = np.concatenate([moe.to_host_values(out), moe.to_host_values(sh)])
    refs, muts = [], []
    for e in range(cfg.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        args = (xv[sorted_token[a:b]],) + tuple(expert_fn(layer)(e)[:3]) + ("fp8", "bf16") + \
            tuple(expert_fn(layer)(e)[3:])
        refs.append((a, oracle.expert_ffn(*args)))
        muts.append((a, no_hq(*args)))
    sargs = (xv, layer.shared.w1, layer.shared.w3, layer.shared.w2, "fp8", "bf16",
             layer.shared.w1_s, layer.shared.w3_s, layer.shared.w2_s)
    ref = np.zeros_like(got, dtype=np.float64)
    mut = np.zeros_like(ref)
    for a, r in refs:
        ref[a:a + r.shape[0]] = r
    for a, r in muts:
        mut[a:a + r.shape[0]] = r
    R = out.shape[0]
    ref[R:] = oracle.expert_ffn(*sargs)
    mut[R:] = no_hq(*sargs)
    d = np.abs(got - ref)
    off = d > _bf16_ulp(ref)                       # beyond one bf16 step
    # A gross-error guard: one e4m3 step at the value's magnitude (1/8 of it)
    # plus 32 subnormal codes (2^-9 x the block scale, block max / 448), i.e.
    # 1.4e-4 of the block max.  The fp32 sums of the two projections carry an
    # absolute error of a few 1e-5 of the block max (measured: 2e-5), which
    # moves an h near zero by several of the small codes around it.
    bmax = np.abs(ref).reshape(ref.shape[0], -1, 128).max(axis=2).repeat(128, axis=1)
    sub = bmax / 448 * 2.0 ** -9
    step = np.abs(ref) / 8 + 32 * sub
    far = d > step * (1 + 2.0 ** -7) + _bf16_ulp(ref)
    off_mut = np.abs(got - mut) > _bf16_ulp(mut)
    worst = np.argsort((d / step).ravel())[-3:]
    record("fp8_fused_h", case=name, elements=int(got.size), off_by_more_than_bf16_ulp=float(off.mean()),
           beyond_one_e4m3_step=int(far.sum()), vs_unquantised_h=float(off_mut.mean()),
           worst=[[float(got.ravel()[i]), float(ref.ravel()[i]), float(sub.ravel()[i])] for i in worst])
    assert not far.any()
    assert off.mean() <= 5e-3
    assert off_mut.mean() >= 0.3


# Extreme block scales in the fp8 stream tiles: a 1x128 activation block of
# values near 1e-36 (its scale is near 2e-39, a subnormal fp32) and 128x128
# weight blocks whose scale is 0 (the block then encodes zeros whatever its
# codes).  Every block's partial product is promoted with its own
# w_scale * a_scale, so the result stays finite and matches the oracle.

@pytest.mark.parametrize("T,topk", [(700, 2), (16, 4)], ids=["stream", "skinny"])
def test_fp8_tiny_and_zero_block_scales(T, topk):
    cfg = tiny_cfg(f"fp8_extreme_T{T}", T=T, E=8, n_groups=2, topk_groups=1, topk=topk,
                   dim=256, inter=256, inter_shared=256, act_dtype="bf16", router_dtype="bf16",
                   w_dtype="fp8", seed=5151)
    layer = inputs.draw_layer(cfg)
    xv = inputs.bf16_bits_to_f32(layer.x)
    xv[5, :128] *= np.float32(1e-36)
    xv[6, 128:] *= np.float32(1e-30)
    layer.x = inputs.f32_to_bf16_bits(xv)
    for e in range(cfg.E):
        layer.w1_s[e, 0, 0] = 0.0          # W1 rows 0-127 x K block 0
        layer.w2_s[e, 1, 1] = 0.0          # W2 rows 128-255 x K block 1
    layer.shared.w3_s[1, 0] = 0.0
    dw = moe.upload_layer(layer)
    y, same = forward_and_check(cfg, layer, dw)
    assert torch.isfinite(y.float()).all()


# ---------------------------------------------------------------------------
# fp8 activation quantiser (bit-exact codes and scales)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (300, 7168)])
def test_quant_fp8_bitexact(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(3.0)
    a[0, :128] = 0.0                                     # an all-zero block
    if rows > 2:
        a[1, 128 % cols:] *= np.float32(1e-30)          # tiny values: subnormal codes
        a[2, :64] = np.float32(448.0)                   # exact saturation point
    bits = inputs.f32_to_bf16_bits(a)
    vals = inputs.bf16_bits_to_f32(bits)
    q, sc = moe.moe_quant_fp8(moe.to_device(bits, "bf16"))
    _sync()
    oq, osc, _ = oracle.quantize_act_1x128(vals)
    np.testing.assert_array_equal(sc.cpu().numpy(), osc)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)


# ---------------------------------------------------------------------------
# weight layout (a storage format: checked byte for byte against its definition)
# ---------------------------------------------------------------------------

def _tiles_reference(b):
    """[rows, row_bytes] uint8 -> the tiled byte order: tiles (row/16, byte/64)
    in row-major tile order, inside a tile the 16-byte pieces ordered by
    (byte%64)/16, then row%16."""
    rows, rb = b.shape
    return b.reshape(rows // 16, 16, rb // 64, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("rows,row_bytes", [(16, 64), (48, 128), (2048, 14336), (7168 * 2, 4096),
                                            (96, 1792)])
def test_pack_weights_bitexact(rows, row_bytes):
    rng = np.random.default_rng(rows + row_bytes)
    b = rng.integers(0, 256, (rows, row_bytes), dtype=np.uint8)
    src = torch.from_numpy(b).to(DEV)
    out = moe.moe_pack_weights(src)
    _sync()
    np.testing.assert_array_equal(out.cpu().numpy().reshape(-1), _tiles_reference(b))


# ---------------------------------------------------------------------------
# combine (synthetic expert outputs, oracle dispatch)
# ---------------------------------------------------------------------------
# The shared expert used here has an output both sides compute exactly:
# x[:, 0] = 1 and W1 = 32 on that column gives a1 = 32 for every h column,
# silu(32) = 32 (1 - 1.3e-14) rounds to 32 in fp32 and bf16; W3 picks
# x[:, 1 + j] for h column j, so h_j = 32 x[:, 1 + j] exactly; W2 picks
# h_(n mod I) for output column n.  S is therefore 32 x[:, 1 + n mod I] in
# the layer dtype, the combine's arithmetic is the only thing left to
# compare, and it must be bit-exact: same fp32 operations in the same order
# (ascending expert id, product then sum, shared output last).

def _exact_shared(act, dim, inter_s):
    w1 = np.zeros((inter_s, dim), np.float32)
    w1[:, 0] = 32.0
    w3 = np.zeros((inter_s, dim), np.float32)
    w3[np.arange(inter_s), 1 + np.arange(inter_s)] = 1.0
    w2 = np.zeros((dim, inter_s), np.float32)
    w2[np.arange(dim), np.arange(dim) % inter_s] = 1.0
    enc = (lambda a: inputs.f32_to_bf16_bits(a)) if act == "bf16" else (lambda a: a)
    mat = lambda a: moe.moe_pack_weights(moe.to_device(enc(a), act))
    dw = moe.DeviceWeights(None, None, None, None, None, ws1=mat(w1), ws3=mat(w3), ws2=mat(w2))
    return dw, (enc(w1), enc(w3), enc(w2))


def _combine_case(act, K, shared, seed, accumulate):
    rng = np.random.default_rng(seed)
    T, E, dim, inter_s = 203, 40, 320, (128 if shared else 0)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    counts, offsets, sorted_token, row_of = oracle.permute(idx, E)
    vals = (rng.standard_normal((T * K, dim)) * 2.0).astype(np.float32)
    x = rng.standard_normal((T, dim)).astype(np.float32)
    x[:, 0] = 1.0
    if act == "bf16":
        vals_s, x_s = inputs.f32_to_bf16_bits(vals), inputs.f32_to_bf16_bits(x)
        vals, x = inputs.bf16_bits_to_f32(vals_s), inputs.bf16_bits_to_f32(x_s)
    else:
        vals_s, x_s = vals, x
    p = moe.Params(dim=dim, n_experts=E, n_groups=1, topk_groups=1, topk=K, inter=64,
                   shared_inter=inter_s, score_func="sigmoid", route_scale=1.0, act_dtype=act,
                   router_dtype=act, weight_dtype=act, accumulate=accumulate)
    dw, host_w = _exact_shared(act, dim, inter_s) if shared else (None, None)
    ws = moe.alloc_workspace(p, T)
    y = moe.moe_combine(p, moe.to_device(x_s, act), moe.to_device(vals_s, act),
                        torch.from_numpy(row_of).to(DEV), torch.from_numpy(w).to(DEV), dw, ws)
    _sync()
    S = None
    if shared:
        S = 32.0 * x[:, 1 + np.arange(dim) % inter_s].astype(np.float64)
        # the oracle's own shared expert gives exactly this closed form
        so = oracle.expert_ffn(x.astype(np.float64), *host_w, act, act)
        np.testing.assert_array_equal(so, S)
    outs = vals[row_of]                                      # [T, K, dim]
    if accumulate == "layer":
        ref = oracle.combine_layer(outs, w, idx, S, act)
    else:
        ref = oracle.moe_oracle.round_to(oracle.combine(outs, w, idx, S).astype(np.float64), act)
    np.testing.assert_array_equal(moe.to_host_values(y).astype(np.float64), ref)


# K = 6 and 8: slots sorted in registers, combine fused into the shared
# expert's down tiles; K = 12 and 20: slots ranked in LDS, stand-alone combine.
@pytest.mark.parametrize("shared", [False, True], ids=["no_shared", "shared"])
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("K", [6, 12])
def test_combine_parity(act, K, shared):
    _combine_case(act, K, shared, seed=5 + K, accumulate="f32")


@pytest.mark.parametrize("shared", [False, True], ids=["no_shared", "shared"])
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("K", [8, 20])
def test_combine_layer_accumulator_bitexact(act, K, shared):
    # same arithmetic in the same order (ascending expert id, a cast after every
    # addition, the shared output last), so the result is bit-exact
    _combine_case(act, K, shared, seed=6 + K, accumulate="layer")


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def forward_and_check(cfg, layer, dw, tokens=None, accumulate="f32"):
    p = moe.Params.from_config(cfg)
    p.accumulate = accumulate
    ws = moe.alloc_workspace(p, cfg.T)
    g_idx = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=DEV)
    g_w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    y = moe.moe_forward(p, _x_dev(layer), dw, ws, topk_idx=g_idx, topk_w=g_w, counts=counts)
    _sync()
    gi, gw = g_idx.cpu().numpy(), g_w.cpu().numpy()
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=cfg.E))
    tok = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    r = run_oracle(layer, tokens=tok, accumulate=accumulate)
    same = check_routing(cfg, r["w"], r["idx"], r["info"], gi[tok], gw[tok], layer.bias)
    yv = moe.to_host_values(y)[tok]
    within_bar("forward", cfg, yv[same], r["y"][same], accumulate=accumulate,
               tokens=int(same.size), routed_alike=int(same.sum()))
    if not same.all():
        # tokens the GPU routed differently (near ties): their output is the
        # oracle's under the GPU's own routing
        sub = tok[~same]
        r2 = run_oracle(layer, tokens=sub, route=(gw[sub], gi[sub]), accumulate=accumulate)
        within_bar("forward_gpu_routing", cfg, yv[~same], r2["y"], accumulate=accumulate,
                   tokens=int(sub.size))
    return y, same


@pytest.mark.parametrize("cfg", BUILT, ids=lambda c: c.name)
def test_forward_parity(cfg, layers):
    layer, dw = layers(cfg)
    _, same = forward_and_check(cfg, layer, dw)
    assert same.mean() > 0.97


@pytest.mark.parametrize("ci", [0, 1, 3])
def test_forward_parity_layer_accumulator(ci, layers):
    # the original V3 combine (y in the layer dtype, experts in ascending id)
    cfg = inputs.SMALL_CONFIGS[ci]
    layer, dw = layers(cfg)
    _, same = forward_and_check(cfg, layer, dw, accumulate="layer")
    assert same.mean() > 0.97


@pytest.mark.parametrize("ci,rng_", [(1, (8, 24)), (0, (0, 4)), (3, (7, 16)), (9, (2, 5)),
                                     (5, (3, 11))])   # s5: 128 x 512 up tiles
def test_forward_parity_expert_range(ci, rng_):
    # one rank's share: only experts b..e-1 are uploaded and computed
    cfg = inputs.SMALL_CONFIGS[ci]
    layer = inputs.draw_layer(cfg)
    dw = moe.upload_layer(layer, experts=rng_)
    p = moe.Params.from_config(cfg)
    p.expert_begin, p.expert_end = rng_
    ws = moe.alloc_workspace(p, cfg.T)
    g_idx = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=DEV)
    g_w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=DEV)
    y = moe.moe_forward(p, _x_dev(layer), dw, ws, topk_idx=g_idx, topk_w=g_w)
    _sync()
    r = oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer), shared_tuple(layer),
                           experts=rng_, **oracle_kwargs(cfg))
    gi, gw = g_idx.cpu().numpy(), g_w.cpu().numpy()
    same = check_routing(cfg, r["w"], r["idx"], r["info"], gi, gw, layer.bias)
    yv = moe.to_host_values(y)
    within_bar("forward_expert_range", cfg, yv[same], r["y"][same], experts=list(rng_))
    if not same.all():
        sub = np.nonzero(~same)[0]
        r2 = oracle.moe_forward(layer.x, layer.wr, layer.bias, expert_fn(layer),
                                shared_tuple(layer), tokens=sub, route=(gw[sub], gi[sub]),
                                experts=rng_, **oracle_kwargs(cfg))
        within_bar("forward_expert_range_gpu_routing", cfg, yv[sub], r2["y"], experts=list(rng_))
    assert same.mean() > 0.97


def test_forward_deterministic(layers):
    cfg = inputs.SMALL_CONFIGS[1]
    layer, dw = layers(cfg)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    x = _x_dev(layer)
    y1 = moe.moe_forward(p, x, dw, ws).clone()
    ws.fill_(0x5A)
    y2 = moe.moe_forward(p, x, dw, ws)
    _sync()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


EDGE_CFGS = [
    tiny_cfg("edge_T1_bf16", T=1, act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
    tiny_cfg("edge_noshared", T=50, inter_shared=0, act_dtype="bf16", router_dtype="bf16",
             w_dtype="bf16", dim=192, inter=320),
    tiny_cfg("edge_topk1_softmax", T=77, E=8, n_groups=1, topk_groups=1, topk=1,
             score_func="softmax", bias_range=None),
    tiny_cfg("edge_nobias_groups", T=130, E=32, n_groups=4, topk_groups=2, topk=3,
             bias_range=None, act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
    tiny_cfg("edge_hot_all", T=90, E=16, n_groups=1, topk_groups=1, topk=2, score_func="softmax",
             bias_range=None, hot_experts=1, hot_scale=64.0, act_dtype="bf16",
             router_dtype="bf16", w_dtype="bf16"),
    # past 2^16 tokens: 264,000 routed rows, ~16,500 per expert (256-token
    # stream tiles, 65 m-tiles per expert), 16,500 selection workgroups
    tiny_cfg("edge_T66000_bf16", T=66000, E=16, n_groups=4, topk_groups=2, topk=4, dim=128,
             inter=128, inter_shared=128, act_dtype="bf16", router_dtype="bf16", w_dtype="bf16"),
]


@pytest.mark.parametrize("cfg", EDGE_CFGS, ids=lambda c: c.name)
def test_forward_edge_cases(cfg, layers):
    layer, dw = layers(cfg)
    forward_and_check(cfg, layer, dw)


# ---------------------------------------------------------------------------
# HIP graph capture: the whole forward enqueues no allocation, memset or host
# synchronisation, so it can be captured once and replayed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ci", [1, 3])
def test_forward_graph_replays_match_eager(ci, layers):
    cfg = inputs.SMALL_CONFIGS[ci]
    layer, dw = layers(cfg)
    p = moe.Params.from_config(cfg)
    ws = moe.alloc_workspace(p, cfg.T)
    x = _x_dev(layer)
    y = torch.empty((cfg.T, cfg.dim), dtype=p.act_torch, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        moe.moe_forward(p, x, dw, ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(p, x, dw, ws, y=y)
    for _ in range(3):
        y.fill_(0)                                     # eager work between replays
        ws.fill_(0x3C)
        _sync()
        g.replay()
        _sync()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


# ---------------------------------------------------------------------------
# measurement helper: one streaming read, nothing written for zero data
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_stream_read_leaves_sink_for_zero_data(nbytes):
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    moe.moe_stream_read(buf, sink)
    _sync()
    assert int(sink.item()) == 7
