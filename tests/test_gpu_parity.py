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
from tests.helpers import (check_routing, expert_fn, gate_oracle, oracle_kwargs, rel_errors,
                           run_oracle, shared_tuple, tiny_cfg)

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_BAR = (2e-2, 2e-3)
FP8_BAR = (5e-2, 5e-2)

BUILT = list(inputs.SMALL_CONFIGS)
ALL_SMALL = inputs.SMALL_CONFIGS


def bar(cfg):
    return FP8_BAR if cfg.w_dtype == "fp8" else BF16_BAR


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


# ---------------------------------------------------------------------------
# permute (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (63, 16, 4), (64, 16, 4), (65, 32, 8),
                                   (128, 256, 8), (256, 512, 32), (257, 256, 8),
                                   (1000, 256, 8), (4096, 256, 8), (8192, 64, 6),
                                   (777, 512, 32), (300, 3, 3)])
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
    out, sh = moe.moe_expert_ffn(p, _x_dev(layer), torch.from_numpy(sorted_token).to(DEV),
                                 torch.from_numpy(offsets).to(DEV), dw, ws)
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
    mx, mean = rel_errors(out, ref)
    assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (mx, mean)
    if sh is not None:
        s = layer.shared
        sref = oracle.expert_ffn(xv, s.w1, s.w3, s.w2, cfg.w_dtype, cfg.act_dtype,
                                 s.w1_s, s.w3_s, s.w2_s)
        mx, mean = rel_errors(moe.to_host_values(sh), sref)
        assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (mx, mean)


# Hand-made dispatches whose expert sizes straddle the m-tile boundaries of
# each tile kind (the average rows per expert R / E picks the kind: 16-token
# tiles below 8, 64-token tiles below 32, 128-token tiles below 64, 192-token
# tiles below 384, 256-token tiles above; fp8 192-token tiles from 12,
# 16-token fp8 tiles below).  An
# expert of M rows runs as ceil(M / BM) m-tiles of equal size, the last
# taking the rest.
TILE_CASES = [
    ("mid_bf16", dict(E=8, topk=2, w_dtype="bf16"), [65, 64, 63, 29, 0, 1, 0, 0]),
    ("big_bf16", dict(E=4, topk=2, w_dtype="bf16"), [193, 0, 385, 622]),
    ("big_nt_bf16", dict(E=8, topk=2, w_dtype="bf16"), [129, 128, 1, 0, 65, 33, 27, 1]),
    ("huge_bf16", dict(E=4, topk=2, w_dtype="bf16"), [257, 513, 1, 829]),
    ("skinny_bf16", dict(E=8, topk=2, w_dtype="bf16"), [17, 0, 16, 15, 1, 1, 2, 0]),
    ("big_fp8", dict(E=4, topk=2, w_dtype="fp8"), [193, 385, 1, 21]),
    ("skinny_fp8", dict(E=8, topk=2, w_dtype="fp8"), [33, 0, 16, 17, 1, 1, 2, 0]),
]


# the shortest K loops: one or two steps per tile (64-wide bf16, 128-wide fp8)
SHORT_K_CASES = [
    ("big_bf16_k64", dict(E=4, topk=2, w_dtype="bf16", dim=64, inter=64, inter_shared=64), [193, 0, 385, 622]),
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
    out, _ = moe.moe_expert_ffn(p, _x_dev(layer), torch.from_numpy(sorted_token).to(DEV),
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
        mx, mean = rel_errors(out[a:b], ref)
        assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (e, c, mx, mean)


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

@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("K", [6, 12])          # the 8-slot and the 32-slot kernels
def test_combine_parity(act, K):
    rng = np.random.default_rng(5 + K)
    T, E, dim = 203, 40, 320
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    counts, offsets, sorted_token, row_of = oracle.permute(idx, E)
    vals = rng.standard_normal((T * K, dim)).astype(np.float32)
    shv = rng.standard_normal((T, dim)).astype(np.float32)
    if act == "bf16":
        vals_s, sh_s = inputs.f32_to_bf16_bits(vals), inputs.f32_to_bf16_bits(shv)
        vals, shv = inputs.bf16_bits_to_f32(vals_s), inputs.bf16_bits_to_f32(sh_s)
    else:
        vals_s, sh_s = vals, shv
    p = moe.Params(dim=dim, n_experts=E, n_groups=1, topk_groups=1, topk=K, inter=64,
                   shared_inter=64, score_func="sigmoid", route_scale=1.0, act_dtype=act,
                   router_dtype=act, weight_dtype=act)
    y = moe.moe_combine(p, moe.to_device(vals_s, act), torch.from_numpy(row_of).to(DEV),
                        torch.from_numpy(w).to(DEV), moe.to_device(sh_s, act))
    _sync()
    outs = vals[row_of]                                      # [T, K, dim]
    ref = oracle.moe_oracle.round_to(oracle.combine(outs, w, idx, shv).astype(np.float64), act)
    # the same fp32 operations in the same order (ascending expert id, product
    # then sum, shared last), so the result is bit-exact
    np.testing.assert_array_equal(moe.to_host_values(y).astype(np.float64), ref)


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("K", [8, 20])
def test_combine_layer_accumulator_bitexact(act, K):
    # same arithmetic in the same order (ascending expert id, a cast after every
    # addition), so the result is bit-exact
    rng = np.random.default_rng(6 + K)
    T, E, dim = 157, 48, 256
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    counts, offsets, sorted_token, row_of = oracle.permute(idx, E)
    vals = (rng.standard_normal((T * K, dim)) * 2.0).astype(np.float32)
    shv = rng.standard_normal((T, dim)).astype(np.float32)
    if act == "bf16":
        vals_s, sh_s = inputs.f32_to_bf16_bits(vals), inputs.f32_to_bf16_bits(shv)
        vals, shv = inputs.bf16_bits_to_f32(vals_s), inputs.bf16_bits_to_f32(sh_s)
    else:
        vals_s, sh_s = vals, shv
    p = moe.Params(dim=dim, n_experts=E, n_groups=1, topk_groups=1, topk=K, inter=64,
                   shared_inter=64, score_func="sigmoid", route_scale=1.0, act_dtype=act,
                   router_dtype=act, weight_dtype=act, accumulate="layer")
    y = moe.moe_combine(p, moe.to_device(vals_s, act), torch.from_numpy(row_of).to(DEV),
                        torch.from_numpy(w).to(DEV), moe.to_device(sh_s, act))
    _sync()
    ref = oracle.combine_layer(vals[row_of], w, idx, shv, act)
    np.testing.assert_array_equal(moe.to_host_values(y).astype(np.float64), ref)


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
    mx, mean = rel_errors(yv[same], r["y"][same])
    assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (mx, mean)
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


@pytest.mark.parametrize("ci,rng_", [(1, (8, 24)), (0, (0, 4)), (3, (7, 16)), (9, (2, 5))])
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
    same = check_routing(cfg, r["w"], r["idx"], r["info"], g_idx.cpu().numpy(),
                         g_w.cpu().numpy(), layer.bias)
    mx, mean = rel_errors(moe.to_host_values(y)[same], r["y"][same])
    assert mx <= bar(cfg)[0] and mean <= bar(cfg)[1], (mx, mean)
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
