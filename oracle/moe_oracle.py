"""Plain, slow CPU oracle of the DeepSeek-V3-style MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or its binding and imports neither.

Sources (web pages; cited by title and section):
  [scores]  "DeepSeek-V3.2-Exp · Expert scores" - formula z = x_ffn W_r, the
            dtype note (router held in bf16, applied in fp32), the Gate
            constructor and Gate.forward code excerpts, the summary sentences.
  [combine] "DeepSeek-V3.2-Exp · Weighted expert sum" - formula
            y_routed = sum_i G_i E_i, the note that the sum is kept in fp32
            and converted to the input dtype once at the end, the MoE.forward
            code excerpt and its summary sentence.
  [v3]      hackaday.io log "Time to jump right in and swim with the big fish"
            - the original DeepSeek-V3 MoE class (constructor: Expert(dim,
            moe_inter_dim), MLP(dim, n_shared_experts*moe_inter_dim)).

Everything is computed in fp64 except where the pages fix a precision: the
router logits and everything derived from them are fp32 ([scores]: applied in
float32), and y is an fp32 accumulator cast back to the input dtype at the end
([combine]).  Where the pages are silent the readings below are used (each is
also listed in the design notes):
  R1 experts are SwiGLU MLPs: FFN(v) = W2 (silu(W1 v) * (W3 v)), no biases,
     weights [out, in]; silu(a) = a * sigmoid(a).
  R2 ties in every top-k go to the larger value first, then the lower index.
  R3 rounding points: logits z, scores s, s' = s + b, group scores and
     weights are fp32; the SwiGLU pre-activations stay unrounded; h is
     rounded once to the layer dtype (bf16; fp32 for fp32 layers; for fp8
     weights h is quantised to e4m3 per 1x128 block); each expert output and
     the shared output are rounded to the layer dtype; y is summed in fp32 in
     ascending expert order, the shared output is added last, then cast (RNE).
  R4 fp8 scheme: weights carry one fp32 scale per 128x128 block; activations
     (x for W1/W3, h for W2) are quantised per 1x128 block with
     scale = amax/448 (1.0 when amax = 0) and code = e4m3(v/scale), IEEE fp32
     division, round to nearest even, saturating to +-448 (OCP e4m3fn).
  R5 softmax weights are not renormalised (only sigmoid is).
  R6 the shared expert is one MLP of inner width n_shared * inter.
  R9 the accumulator is fp32 by default ([combine]); the original V3 class
     ([v3], its MoE.forward) is the second mode ("layer"): the running sum
     starts at zero in the layer dtype, the routed experts are visited in
     ascending id and each adds its weighted outputs to its tokens' rows, the
     update evaluated in fp32 (a bf16 tensor times fp32 weights promotes) and
     stored back in the layer dtype; the shared output is added last, with
     one more cast.
"""

from __future__ import annotations

import itertools
from typing import Callable, Optional

import numpy as np

__all__ = [
    "bf16_round", "bf16_decode", "e4m3_table", "e4m3_decode", "e4m3_encode",
    "decode_weights", "quantize_act_1x128", "router_logits", "scores",
    "select_experts", "routing_weights", "gate", "permute", "swiglu",
    "expert_ffn", "combine", "combine_layer", "round_to", "moe_forward", "moe_forward_dense",
    "brute_force_select",
]

F32 = np.float32

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def bf16_round(v) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as fp64.

    Written from the format's definition with frexp/ldexp, independently of
    any bit trick: v = m * 2^e with 0.5 <= |m| < 1, keep 8 bits of m.
    Below the smallest normal (2^-126) the spacing is fixed at 2^-133.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)          # np.round: half to even
    tiny = np.abs(v) < 2.0 ** -126
    r = np.where(tiny, np.round(v * 2.0 ** 133) * 2.0 ** -133, r)
    return r


def _bf16_value(b: np.ndarray) -> np.ndarray:
    """Value of bf16 bit patterns: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    ex = (b >> 7) & 0xFF
    fr = (b & 0x7F).astype(np.float64)
    val = np.where(ex == 0, fr * 2.0 ** -133, (1.0 + fr / 128.0) * np.exp2(ex - 127.0))
    val = np.where(ex == 0xFF, np.where(fr == 0, np.inf, np.nan), val)
    return sign * val


_BF16 = _bf16_value(np.arange(65536))


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values (lookup in the table of all 65536 codes)."""
    return _BF16[np.asarray(bits, dtype=np.uint16)]


def e4m3_table() -> np.ndarray:
    """Values of the 256 OCP e4m3fn codes (NaN for S.1111.111).

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (m * 2^-9); no infinities; largest finite magnitude 448.
    """
    c = np.arange(256)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


_E4M3 = e4m3_table()
# the 127 non-negative finite codes in increasing value order (code == position)
_E4M3_POS = _E4M3[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.int64)]


def e4m3_encode(v) -> np.ndarray:
    """Nearest e4m3fn code, ties to the even code, saturating at +-448.

    Plain definition: locate |v| between two neighbouring representable
    magnitudes and take the closer; on an exact tie take the one whose code
    (last mantissa bit) is even.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")         # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E4M3_POS[hi], hi, code)
    sign = np.where(np.signbit(v) & (code != 0), 0x80, 0)
    return (code | sign).astype(np.uint8)


def decode_weights(w: np.ndarray, dtype: str, scales: Optional[np.ndarray] = None) -> np.ndarray:
    """Storage-format weight matrix [N, K] -> fp64 values.

    "fp8": value = e4m3(code) * scale of its 128x128 block (R4).
    """
    if dtype == "f32":
        return np.asarray(w, dtype=np.float64)
    if dtype == "bf16":
        return bf16_decode(w)
    if dtype == "fp8":
        v = e4m3_decode(w)
        s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=0), 128, axis=1)
        return v * s[: v.shape[0], : v.shape[1]]
    raise ValueError(dtype)


def decode_act(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return bf16_decode(x)
    raise ValueError(dtype)


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the layer dtype (R3), returned as fp64."""
    if dtype == "f32":
        return np.asarray(v, dtype=F32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(v)
    raise ValueError(dtype)


def quantize_act_1x128(a: np.ndarray):
    """Activation quantisation (R4): rows split into 1x128 blocks.

    a: [M, K] values already held in fp32.  Returns (codes [M,K] uint8,
    scales [M, K/128] fp32, dequantised values [M,K] fp64).
    """
    a32 = np.asarray(a, dtype=F32)
    M, K = a32.shape
    blk = a32.reshape(M, K // 128, 128)
    amax = np.abs(blk).max(axis=2)
    scale = np.where(amax > 0, amax / F32(448.0), F32(1.0)).astype(F32)     # fp32 division
    q = e4m3_encode((blk / scale[:, :, None]).astype(F32))                  # fp32 division
    deq = e4m3_decode(q) * scale[:, :, None].astype(np.float64)
    return q.reshape(M, K), scale, deq.reshape(M, K)


# ---------------------------------------------------------------------------
# gate  ([scores]: formula, dtype note, Gate.forward excerpt)
# ---------------------------------------------------------------------------


def router_logits(x_vals: np.ndarray, wr_vals: np.ndarray) -> np.ndarray:
    """z = x W_r^T in fp32 (router applied in fp32): exact fp64 product, rounded once."""
    return (np.asarray(x_vals, np.float64) @ np.asarray(wr_vals, np.float64).T).astype(F32)


def scores(z: np.ndarray, score_func: str) -> np.ndarray:
    """Sigmoid elementwise, or softmax over the expert axis; fp32 results."""
    z64 = z.astype(np.float64)
    if score_func == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-z64))
    elif score_func == "softmax":
        ez = np.exp(z64 - z64.max(axis=1, keepdims=True))
        s = ez / ez.sum(axis=1, keepdims=True)
    else:
        raise ValueError(score_func)
    return s.astype(F32)


def _order_desc(vals: np.ndarray) -> np.ndarray:
    """Indices by descending value, equal values by ascending index (R2)."""
    return np.lexsort((np.arange(vals.shape[-1]), -vals.astype(np.float64)))


def select_experts(s: np.ndarray, bias: Optional[np.ndarray], n_groups: int,
                   topk_groups: int, topk: int):
    """Group-limited top-k selection for every token.

    s' = s + bias (selection only).  With n_groups > 1 the experts are viewed as
    [n_groups, E/n_groups]; a group's score is the sum of its two largest s'
    when a bias exists, else its largest s'; the topk_groups best groups stay
    and the rest are excluded; then the topk largest s' are chosen.

    Returns (idx [T, topk] int32 in descending s' order, info) where info holds
    s' and the group / expert margins used by the parity rule.
    """
    T, E = s.shape
    sp = (s + bias.astype(F32)).astype(F32) if bias is not None else s.copy()
    idx = np.empty((T, topk), dtype=np.int32)
    mg = np.full(T, np.inf)
    me = np.full(T, np.inf)
    gsz = E // n_groups
    for t in range(T):
        row = sp[t]
        if n_groups > 1:
            grp = row.reshape(n_groups, gsz)
            if bias is not None:
                top2 = np.sort(grp, axis=1)[:, -2:]
                gs = (top2[:, 0] + top2[:, 1]).astype(F32)              # fp32 sum of two
            else:
                gs = grp.max(axis=1)
            gord = _order_desc(gs)
            keep = np.sort(gord[:topk_groups])
            if topk_groups < n_groups:
                mg[t] = float(gs[gord[topk_groups - 1]]) - float(gs[gord[topk_groups]])
            cand = (keep[:, None] * gsz + np.arange(gsz)[None, :]).ravel()
        else:
            cand = np.arange(E)
        cv = row[cand]
        cord = _order_desc(cv)
        idx[t] = cand[cord[:topk]]
        if topk < cand.size:
            me[t] = float(cv[cord[topk - 1]]) - float(cv[cord[topk]])
    return idx, {"s_sel": sp, "margin_group": mg, "margin_expert": me}


def routing_weights(s: np.ndarray, idx: np.ndarray, score_func: str, route_scale: float) -> np.ndarray:
    """w = s[idx] from the unbiased scores; sigmoid weights divided by their sum;
    then multiplied by route_scale.  fp32 result (sum taken exactly, then rounded)."""
    w = np.take_along_axis(s, idx.astype(np.int64), axis=1).astype(F32)
    if score_func == "sigmoid":
        tot = w.astype(np.float64).sum(axis=1, keepdims=True).astype(F32)
        w = (w / tot).astype(F32)
    return (w * F32(route_scale)).astype(F32)


def gate(x_vals, wr_vals, bias, *, score_func, n_groups, topk_groups, topk, route_scale):
    """Gate.forward: returns (weights fp32 [T,topk], indices int32 [T,topk], info)."""
    z = router_logits(x_vals, wr_vals)
    s = scores(z, score_func)
    idx, info = select_experts(s, bias, n_groups, topk_groups, topk)
    w = routing_weights(s, idx, score_func, route_scale)
    info.update(z=z, s=s)
    return w, idx, info


def brute_force_select(s, bias, n_groups, topk_groups, topk):
    """Selection by exhaustive enumeration (tiny E only; used to pin select_experts).

    Among all topk_groups-subsets of groups take the one with the largest total
    group score, then among all topk-subsets of their experts the one with the
    largest total s'.  For inputs without near-ties this is the same set as the
    sorted selection; returns a list of frozensets.
    """
    T, E = s.shape
    sp = (s + bias.astype(F32)).astype(F32) if bias is not None else s
    out = []
    gsz = E // n_groups
    for t in range(T):
        row = sp[t].astype(np.float64)
        if n_groups > 1:
            grp = row.reshape(n_groups, gsz)
            if bias is not None:
                gs = [max(a + b for a, b in itertools.combinations(g, 2)) for g in grp]
            else:
                gs = [max(g) for g in grp]
            best = max(itertools.combinations(range(n_groups), topk_groups),
                       key=lambda c: sum(gs[j] for j in c))
            cand = [j * gsz + i for j in best for i in range(gsz)]
        else:
            cand = list(range(E))
        bsel = max(itertools.combinations(cand, topk), key=lambda c: sum(row[i] for i in c))
        out.append(frozenset(bsel))
    return out


# ---------------------------------------------------------------------------
# dispatch  ([combine]: a count per expert, then each expert's (token, slot)
#            pairs in row-major order)
# ---------------------------------------------------------------------------


def permute(idx: np.ndarray, E: int):
    """Expert-contiguous order of the (token, slot) assignments.

    counts[e] = number of assignments to e; offsets = exclusive prefix sum;
    inside expert e's segment the tokens appear in ascending order (the order
    a row-major search of the index matrix yields); row_of[t, k] is the position of
    assignment (t, k).  Returns int32 arrays.
    """
    T, K = idx.shape
    counts = np.bincount(idx.ravel().astype(np.int64), minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_token = np.empty(T * K, dtype=np.int32)
    row_of = np.empty((T, K), dtype=np.int32)
    for e in range(E):
        toks, slots = np.nonzero(idx == e)
        pos = offsets[e] + np.arange(toks.size)
        sorted_token[pos] = toks
        row_of[toks, slots] = pos
    return counts, offsets, sorted_token, row_of


# ---------------------------------------------------------------------------
# experts  (R1, R3, R4)
# ---------------------------------------------------------------------------


def silu(a):
    return a / (1.0 + np.exp(-a))


def swiglu(a1: np.ndarray, a3: np.ndarray) -> np.ndarray:
    """h = silu(A) * B (fp64)."""
    return silu(a1) * a3


def expert_ffn(xv: np.ndarray, w1, w3, w2, w_dtype: str, act_dtype: str,
               w1_s=None, w3_s=None, w2_s=None, xq=None) -> np.ndarray:
    """One SwiGLU expert on rows xv (fp64 values of the layer input).

    Returns the expert output rounded to the layer dtype (as fp64 values).
    For fp8 weights the activations are quantised per 1x128 block first
    (xq may pass x already quantised, since the blocks do not depend on the
    expert).
    """
    W1 = decode_weights(w1, w_dtype, w1_s)
    W3 = decode_weights(w3, w_dtype, w3_s)
    W2 = decode_weights(w2, w_dtype, w2_s)
    if w_dtype == "fp8":
        xin = xq if xq is not None else quantize_act_1x128(xv)[2]
        h32 = swiglu(xin @ W1.T, xin @ W3.T).astype(F32)
        hin = quantize_act_1x128(h32)[2]
    else:
        hin = round_to(swiglu(xv @ W1.T, xv @ W3.T), act_dtype)
    return round_to(hin @ W2.T, act_dtype)


# ---------------------------------------------------------------------------
# layer  ([combine]: MoE.forward excerpt; [v3] constructor)
# ---------------------------------------------------------------------------


def combine(outs: np.ndarray, w: np.ndarray, idx: np.ndarray, shared_out=None,
            experts=None) -> np.ndarray:
    """fp32 accumulator y = 0; for each expert in ascending id, y[t] += out[t,k] * w[t,k]
    (product then sum, each rounded to fp32); then y += shared output.

    outs [T, topk, dim]: each assignment's expert output (layer-dtype values);
    w [T, topk] fp32; idx [T, topk]; shared_out [T, dim] or None.
    experts: optional (b, e) - only experts b..e-1 contribute ([v3]: a rank's
    forward loops over its own experts only).
    Returns the fp32 accumulator (cast it with round_to).
    """
    T, K, dim = outs.shape
    y = np.zeros((T, dim), dtype=F32)
    order = np.argsort(idx, axis=1, kind="stable")            # ascending expert id per token
    for j in range(K):
        k = order[:, j]
        o = outs[np.arange(T), k].astype(F32)
        contrib = (o * w[np.arange(T), k][:, None].astype(F32)).astype(F32)
        if experts is None:
            y = (y + contrib).astype(F32)
        else:
            e = idx[np.arange(T), k]
            keep = ((e >= experts[0]) & (e < experts[1]))[:, None]
            y = np.where(keep, (y + contrib).astype(F32), y)
    if shared_out is not None:
        y = (y + np.asarray(shared_out).astype(F32)).astype(F32)
    return y


def combine_layer(outs: np.ndarray, w: np.ndarray, idx: np.ndarray, shared_out,
                  act_dtype: str, experts=None) -> np.ndarray:
    """[v3] MoE.forward with y held in the layer dtype (R9): y = 0; for each
    expert in ascending id, y[t] = cast(y[t] + out[t,k] * w[t,k]) where the
    product and the sum are fp32 and cast rounds to the layer dtype; then
    y = cast(y + shared output).

    outs [T, topk, dim] layer-dtype values; w [T, topk] fp32; idx [T, topk];
    shared_out [T, dim] or None.  Returns fp64 values of the layer-dtype y.
    """
    T, K, dim = outs.shape
    y = np.zeros((T, dim), dtype=F32)
    order = np.argsort(idx, axis=1, kind="stable")            # ascending expert id per token
    for j in range(K):
        k = order[:, j]
        o = outs[np.arange(T), k].astype(F32)
        contrib = (o * w[np.arange(T), k][:, None].astype(F32)).astype(F32)
        upd = round_to((y + contrib).astype(F32), act_dtype).astype(F32)
        if experts is None:
            y = upd
        else:
            e = idx[np.arange(T), k]
            y = np.where(((e >= experts[0]) & (e < experts[1]))[:, None], upd, y)
    if shared_out is not None:
        y = round_to((y + np.asarray(shared_out).astype(F32)).astype(F32), act_dtype).astype(F32)
    return y.astype(np.float64)


def moe_forward(x, wr, bias, expert_weights: Callable, shared, *, act_dtype, w_dtype,
                router_dtype, E, n_groups, topk_groups, topk, score_func, route_scale,
                tokens=None, route=None, accumulate="f32", experts=None):
    """y = cast( sum_k w[t,k] * FFN_{idx[t,k]}(x_t) + FFN_shared(x_t) ).

    x, wr: storage-format arrays; expert_weights(e) -> (w1, w3, w2, w1_s, w3_s,
    w2_s); shared: the same tuple or None.  tokens: optional subset of token
    ids (the gate still runs on exactly those rows: routing is per token).
    route: optional (weights, idx) to use instead of the gate's own (for tokens
    whose top-k is undecided within the margin).  accumulate: "f32" ([combine])
    or "layer" ([v3], R9).  experts: optional (b, e), the routed experts that
    contribute ([v3] constructor and forward: a rank holds and loops over
    experts_start_idx..experts_end_idx-1); the gate still sees all experts.

    Returns dict(y=[n, dim] fp64 values of the cast output, y32=fp32
    accumulator (None in the layer mode), w, idx, info).
    """
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    xv = decode_act(x[tok], act_dtype)
    wrv = decode_act(wr, router_dtype)
    if route is None:
        w, idx, info = gate(xv, wrv, bias, score_func=score_func, n_groups=n_groups,
                            topk_groups=topk_groups, topk=topk, route_scale=route_scale)
    else:
        w, idx = (np.asarray(route[0], F32), np.asarray(route[1], np.int32))
        info = {}
    xq = quantize_act_1x128(xv)[2] if w_dtype == "fp8" else None
    outs = np.zeros(idx.shape + (xv.shape[1],))             # FFN_{idx[t,k]}(x_t)
    lo, hi = (0, E) if experts is None else experts
    for e in range(lo, hi):                                 # ascending expert order
        rows, slots = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        w1, w3, w2, s1, s3, s2 = expert_weights(e)
        outs[rows, slots] = expert_ffn(xv[rows], w1, w3, w2, w_dtype, act_dtype, s1, s3, s2,
                                       None if xq is None else xq[rows])
    sh = None
    if shared is not None:
        w1, w3, w2, s1, s3, s2 = shared
        sh = expert_ffn(xv, w1, w3, w2, w_dtype, act_dtype, s1, s3, s2, xq)
    if accumulate == "layer":
        return {"y": combine_layer(outs, w, idx, sh, act_dtype, experts), "y32": None, "w": w,
                "idx": idx, "info": info, "tokens": tok}
    if accumulate != "f32":
        raise ValueError(accumulate)
    y = combine(outs, w, idx, sh, experts)
    return {"y": round_to(y.astype(np.float64), act_dtype), "y32": y, "w": w, "idx": idx,
            "info": info, "tokens": tok}


def moe_forward_dense(x, wr, bias, expert_weights, shared, *, act_dtype, w_dtype,
                      router_dtype, E, n_groups, topk_groups, topk, score_func,
                      route_scale):
    """The weighted-sum formula read literally: y_routed = sum_i G_i E_i.

    Every expert runs on every token; G is the dense [T, E] gate matrix, zero
    off each token's top-k.  Everything after the gate is fp64 with the same
    per-module rounding of expert outputs; no fp32 accumulation emulation.
    Tiny shapes only.
    """
    xv = decode_act(x, act_dtype)
    wrv = decode_act(wr, router_dtype)
    w, idx, _ = gate(xv, wrv, bias, score_func=score_func, n_groups=n_groups,
                     topk_groups=topk_groups, topk=topk, route_scale=route_scale)
    T = xv.shape[0]
    G = np.zeros((T, E))
    np.put_along_axis(G, idx.astype(np.int64), w.astype(np.float64), axis=1)
    y = np.zeros(xv.shape)
    for e in range(E):
        w1, w3, w2, s1, s3, s2 = expert_weights(e)
        y += G[:, e:e + 1] * expert_ffn(xv, w1, w3, w2, w_dtype, act_dtype, s1, s3, s2)
    if shared is not None:
        w1, w3, w2, s1, s3, s2 = shared
        y += expert_ffn(xv, w1, w3, w2, w_dtype, act_dtype, s1, s3, s2)
    return {"y_exact": y, "w": w, "idx": idx}
