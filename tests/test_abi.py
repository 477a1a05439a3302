"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/moe.h declares, and rejects invalid calls on the host before any HIP
call (nothing is enqueued, so NULL device pointers are never touched)."""

import ctypes
import os
import re

import pytest

from mixture_experts_layer_11_amd import moe
from mixture_experts_layer_11_amd.inputs import SMALL_CONFIGS, config_by_name

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_steps():
    d = declared_functions()
    for name in ("moe_gate", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
                 "moe_workspace_size", "moe_status_string", "moe_last_error", "moe_abi_version"):
        assert name in d


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(moe.EXPORTS) == set(declared_functions())
    assert L.moe_abi_version() == 3


def test_status_strings():
    assert moe.status_string(0) == "MOE_OK"
    assert moe.status_string(3) == "MOE_ERR_WORKSPACE"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"


def _p(**kw):
    base = moe.Params.from_config(config_by_name("c1"))
    for k, v in kw.items():
        setattr(base, k, v)
    return base


def _ws_status(p, T=16):
    n = ctypes.c_size_t()
    return moe.lib().moe_workspace_size(ctypes.byref(p.c()), T, ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(n_groups=3), moe.MOE_ERR_INVALID_ARG),             # 256 % 3 != 0
    (dict(topk_groups=9), moe.MOE_ERR_INVALID_ARG),          # > n_groups
    (dict(topk_groups=0), moe.MOE_ERR_INVALID_ARG),
    (dict(topk=0), moe.MOE_ERR_INVALID_ARG),
    (dict(topk=129), moe.MOE_ERR_INVALID_ARG),               # > topk_groups * E / n_groups
    (dict(n_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=1024, n_groups=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(dim=7100), moe.MOE_ERR_UNSUPPORTED),               # not a multiple of 64
    (dict(inter=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype="f32"), moe.MOE_ERR_UNSUPPORTED),        # mixed dtypes
    (dict(weight_dtype="fp8", inter=2000), moe.MOE_ERR_UNSUPPORTED),
    (dict(topk=40, topk_groups=8), moe.MOE_ERR_UNSUPPORTED),  # topk > 32
    (dict(dim=65600), moe.MOE_ERR_UNSUPPORTED),              # wider than 65536
    (dict(inter=65600), moe.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=65600), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_params_rejected_on_host(kw, status):
    s, _ = _ws_status(_p(**kw))
    assert s == status
    assert moe.lib().moe_last_error().decode() != ""


def test_token_count_limit():
    # the combine runs one 256-thread workgroup per token: 2^24 of them would
    # need 2^32 work-items, one more than a dispatch counts
    assert _ws_status(_p(), (1 << 24) - 1)[0] == moe.MOE_OK
    assert _ws_status(_p(), 1 << 24)[0] == moe.MOE_ERR_UNSUPPORTED


def test_oversized_expert_launch_rejected_before_enqueue():
    # 8 experts of 2^21 rows each on 256-token tiles, 512 column tiles of a
    # 65536-wide expert: far beyond 2^32 work-items.  The pointers are never
    # dereferenced because the call returns first.
    p = _p(n_experts=8, n_groups=1, topk_groups=1, topk=8, dim=64, inter=65536,
           shared_inter=65536)
    fake = ctypes.c_void_p(256)
    w = moe.moe_weights(w_router=256, w1=256, w3=256, w2=256, ws1=256, ws3=256, ws2=256)
    L = moe.lib()
    T = (1 << 24) - 1
    assert _ws_status(p, T)[0] == moe.MOE_OK          # the shapes themselves are valid
    s = L.moe_expert_ffn(ctypes.byref(p.c()), T, fake, fake, fake, ctypes.byref(w), fake,
                         fake, 1 << 62, None)
    assert s == moe.MOE_ERR_UNSUPPORTED and "work-items" in L.moe_last_error().decode()
    s = L.moe_combine(ctypes.byref(p.c()), T, fake, fake, fake, fake, ctypes.byref(w), fake,
                      fake, 1 << 62, None)
    assert s == moe.MOE_ERR_UNSUPPORTED and "work-items" in L.moe_last_error().decode()
    s = L.moe_forward(ctypes.byref(p.c()), T, fake, ctypes.byref(w), fake, None, None, None,
                      fake, 1 << 62, None)
    assert s == moe.MOE_ERR_UNSUPPORTED and "work-items" in L.moe_last_error().decode()
    # a decode-sized batch of the same layer passes the check and stops at the
    # (deliberately too small) workspace instead
    s = L.moe_expert_ffn(ctypes.byref(p.c()), 16, fake, fake, fake, ctypes.byref(w), fake,
                         fake, 16, None)
    assert s == moe.MOE_ERR_WORKSPACE


def test_quant_fp8_block_limit():
    fake = ctypes.c_void_p(256)
    L = moe.lib()
    # 16 work-items per block, rounded up to 256-thread workgroups
    assert L.moe_quant_fp8(fake, (1 << 28) - 15, 128, fake, fake, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_fp8(fake, 1 << 25, 1024, fake, fake, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_fp8(fake, 100, 100, fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quant_fp8(fake, 0, 128, fake, fake, None) == moe.MOE_OK


def test_unknown_accumulate_mode_rejected():
    pc = _p().c()
    pc.accumulate = 7
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_size(ctypes.byref(pc), 16, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    pc.accumulate = 1
    assert moe.lib().moe_workspace_size(ctypes.byref(pc), 16, ctypes.byref(n)) == moe.MOE_OK


@pytest.mark.parametrize("b,e,status", [(0, 0, 0), (0, 256, 0), (32, 64, 0), (5, 5, 0),
                                         (-1, 8, 1), (9, 8, 1), (0, 257, 1)])
def test_expert_range_validation(b, e, status):
    pc = _p().c()
    pc.expert_begin, pc.expert_end = b, e
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_size(ctypes.byref(pc), 16, ctypes.byref(n)) == status


def test_combine_needs_full_expert_range():
    pc = _p().c()
    pc.expert_begin, pc.expert_end = 0, 32
    fake = ctypes.c_void_p(256)
    w = moe.moe_weights(ws1=256, ws3=256, ws2=256)
    s = moe.lib().moe_combine(ctypes.byref(pc), 16, fake, fake, fake, fake, ctypes.byref(w), fake,
                              fake, 1 << 30, None)
    assert s == moe.MOE_ERR_UNSUPPORTED


def test_workspace_size_grows_with_T_and_is_aligned():
    p = _p()
    s1, n1 = _ws_status(p, 16)
    s2, n2 = _ws_status(p, 4096)
    assert s1 == s2 == moe.MOE_OK and 0 < n1 < n2 and n1 % 256 == 0
    s, _ = _ws_status(p, -1)
    assert s == moe.MOE_ERR_INVALID_ARG


def test_null_and_workspace_errors_enqueue_nothing():
    p = _p()
    L = moe.lib()
    pc = p.c()
    i64 = 16
    # NULL pointers -> invalid argument
    s = L.moe_gate(ctypes.byref(pc), i64, None, None, None, None, None, None, 0, None)
    assert s == moe.MOE_ERR_INVALID_ARG
    # non-NULL (never dereferenced) pointers but no workspace -> workspace error
    fake = ctypes.c_void_p(256)
    s = L.moe_gate(ctypes.byref(pc), i64, fake, fake, None, fake, fake, None, 0, None)
    assert s == moe.MOE_ERR_WORKSPACE
    s = L.moe_permute(ctypes.byref(pc), i64, fake, fake, fake, fake, fake, fake, 10, None)
    assert s == moe.MOE_ERR_WORKSPACE
    # bias with groups of one expert is rejected (the group score needs a top-2)
    p1 = _p(n_experts=8, n_groups=8, topk_groups=4, topk=4)
    s = L.moe_gate(ctypes.byref(p1.c()), i64, fake, fake, fake, fake, fake, None, 0, None)
    assert s == moe.MOE_ERR_INVALID_ARG
    # a shared expert without its weights, and a combine without x for it
    w = moe.moe_weights(w1=256, w3=256, w2=256)
    s = L.moe_combine(ctypes.byref(pc), i64, fake, fake, fake, fake, ctypes.byref(w), fake,
                      fake, 1 << 30, None)
    assert s == moe.MOE_ERR_INVALID_ARG and "ws1" in L.moe_last_error().decode()
    ws = moe.moe_weights(ws1=256, ws3=256, ws2=256)
    s = L.moe_combine(ctypes.byref(pc), i64, None, fake, fake, fake, ctypes.byref(ws), fake,
                      fake, 1 << 30, None)
    assert s == moe.MOE_ERR_INVALID_ARG and "x is NULL" in L.moe_last_error().decode()
    # without a shared expert the combine needs neither x nor weights
    p0 = _p(shared_inter=0)
    s = L.moe_combine(ctypes.byref(p0.c()), i64, None, fake, fake, fake, None, fake,
                      None, 0, None)
    assert s == moe.MOE_ERR_WORKSPACE
    # fp8 weights without scales
    p8 = _p(weight_dtype="fp8")
    s = L.moe_forward(ctypes.byref(p8.c()), i64, fake, ctypes.byref(w), fake, None, None, None,
                      fake, 1 << 30, None)
    assert s in (moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED)


@pytest.mark.parametrize("rows,row_bytes", [(15, 64), (16, 32), (16, 0), (-16, 64), (32, 100)])
def test_pack_weights_rejects_bad_shapes(rows, row_bytes):
    fake = ctypes.c_void_p(256)
    other = ctypes.c_void_p(512)
    assert moe.lib().moe_pack_weights(fake, rows, row_bytes, other, None) == moe.MOE_ERR_INVALID_ARG


def test_pack_weights_rejects_null_and_aliasing():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    assert L.moe_pack_weights(None, 16, 64, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(fake, 16, 64, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(None, 0, 64, None, None) == moe.MOE_OK     # nothing to do


def test_stream_read_rejects_bad_arguments():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    assert L.moe_stream_read(None, 64, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(fake, 64, None, None) == moe.MOE_ERR_INVALID_ARG
    for n in (0, 8, 100):
        assert L.moe_stream_read(fake, n, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert "multiple of 16" in moe.lib().moe_last_error().decode()


def test_zero_tokens_is_a_noop():
    L = moe.lib()
    for cfg in SMALL_CONFIGS:
        p = moe.Params.from_config(cfg)
        if p.weight_dtype == "fp8":
            continue
        pc = p.c()
        w = moe.moe_weights(w_router=256, w1=256, w3=256, w2=256, ws1=256, ws3=256, ws2=256)
        assert L.moe_forward(ctypes.byref(pc), 0, None, ctypes.byref(w), None, None, None, None,
                             None, 0, None) == moe.MOE_OK
        assert L.moe_gate(ctypes.byref(pc), 0, None, None, None, None, None, None, 0, None) == moe.MOE_OK


def test_noalloc_limits_checked_before_any_device_work():
    # the DeepSeek-V3 prefill shape needs far more than the fixed scratch:
    # refused on the host, naming the limit; T = 0 is a no-op
    p = _p()
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    w = moe.moe_weights(w_router=256, w1=256, w3=256, w2=256, ws1=256, ws3=256, ws2=256)
    s = L.moe_forward_noalloc(ctypes.byref(p.c()), 4096, fake, ctypes.byref(w), fake, None, None,
                              None, None)
    assert s == moe.MOE_ERR_UNSUPPORTED
    assert str(64 << 20) in L.moe_last_error().decode()
    assert L.moe_forward_noalloc(ctypes.byref(p.c()), 0, None, ctypes.byref(w), None, None, None,
                                 None, None) == moe.MOE_OK
    assert _ws_status(p, 128)[1] <= 64 << 20      # the decode shape fits
