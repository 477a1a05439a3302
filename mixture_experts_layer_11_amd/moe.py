"""ctypes binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's kernels.
If the library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX = range(2)

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
_SCORE = {"sigmoid": MOE_SCORE_SIGMOID, "softmax": MOE_SCORE_SOFTMAX}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


class moe_params(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("score_func", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("accumulate", ctypes.c_int32), ("expert_begin", ctypes.c_int32),
                ("expert_end", ctypes.c_int32)]


_VP = ctypes.c_void_p
_ACC = {"f32": 0, "layer": 1}


class moe_weights(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("w_router", "bias", "w1", "w3", "w2", "w1_scale",
                                   "w3_scale", "w2_scale", "ws1", "ws3", "ws2", "ws1_scale",
                                   "ws3_scale", "ws2_scale")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so once.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m mixture_experts_layer_11_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    st, i64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER(moe_params)
    W = ctypes.POINTER(moe_weights)
    sigs = {
        "moe_workspace_size": (st, [P, i64, ctypes.POINTER(sz)]),
        "moe_gate": (st, [P, i64, _VP, _VP, _VP, _VP, _VP, _VP, sz, _VP]),
        "moe_permute": (st, [P, i64, _VP, _VP, _VP, _VP, _VP, _VP, sz, _VP]),
        "moe_expert_ffn": (st, [P, i64, _VP, _VP, _VP, W, _VP, _VP, sz, _VP]),
        "moe_combine": (st, [P, i64, _VP, _VP, _VP, _VP, W, _VP, _VP, sz, _VP]),
        "moe_forward": (st, [P, i64, _VP, W, _VP, _VP, _VP, _VP, _VP, sz, _VP]),
        "moe_forward_noalloc": (st, [P, i64, _VP, W, _VP, _VP, _VP, _VP, _VP]),
        "moe_status_string": (ctypes.c_char_p, [st]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (ctypes.c_int32, []),
        "moe_quant_fp8": (st, [_VP, i64, ctypes.c_int32, _VP, _VP, _VP]),
        "moe_pack_weights": (st, [_VP, i64, i64, _VP, _VP]),
        "moe_stream_read": (st, [_VP, sz, _VP, _VP]),
        "moe_profile_start": (st, [ctypes.c_int32]),
        "moe_profile_stop": (st, [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float)]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTS = ("moe_workspace_size", "moe_gate", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_status_string", "moe_last_error", "moe_abi_version",
           "moe_profile_start", "moe_profile_stop", "moe_quant_fp8", "moe_pack_weights",
           "moe_stream_read")


def status_string(s: int) -> str:
    return lib().moe_status_string(s).decode()


def _check(s: int):
    if s != MOE_OK:
        raise MoeError(s, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


@dataclass
class Params:
    dim: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    inter: int
    shared_inter: int
    score_func: str
    route_scale: float
    act_dtype: str
    router_dtype: str
    weight_dtype: str
    accumulate: str = "f32"   # "f32" or "layer" (moe_accumulate)
    expert_begin: int = 0     # routed experts computed: [expert_begin, expert_end)
    expert_end: int = 0       # 0 = n_experts

    @staticmethod
    def from_config(cfg) -> "Params":
        return Params(cfg.dim, cfg.E, cfg.n_groups, cfg.topk_groups, cfg.topk, cfg.inter,
                      cfg.inter_shared, cfg.score_func, cfg.route_scale, cfg.act_dtype,
                      cfg.router_dtype, cfg.w_dtype, getattr(cfg, "accumulate", "f32"))

    def c(self) -> moe_params:
        return moe_params(self.dim, self.n_experts, self.n_groups, self.topk_groups, self.topk,
                          self.inter, self.shared_inter, _SCORE[self.score_func],
                          self.route_scale, _DT[self.act_dtype], _DT[self.router_dtype],
                          _DT[self.weight_dtype], _ACC[self.accumulate], self.expert_begin,
                          self.expert_end)

    @property
    def act_torch(self):
        return torch.float32 if self.act_dtype == "f32" else torch.bfloat16


def workspace_size(p: Params, T: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(p.c()), T, ctypes.byref(n)))
    return n.value


def alloc_workspace(p: Params, T: int, device="cuda") -> torch.Tensor:
    n = workspace_size(p, T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_gate(p: Params, x, w_router, bias, workspace, topk_idx=None, topk_w=None, stream=None):
    T = x.shape[0]
    dev = x.device
    topk_idx = topk_idx if topk_idx is not None else torch.empty((T, p.topk), dtype=torch.int32, device=dev)
    topk_w = topk_w if topk_w is not None else torch.empty((T, p.topk), dtype=torch.float32, device=dev)
    _check(lib().moe_gate(ctypes.byref(p.c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                          _ptr(topk_idx), _ptr(topk_w), _ptr(workspace), workspace.numel(),
                          _stream(stream)))
    return topk_idx, topk_w


def moe_permute(p: Params, topk_idx, workspace, stream=None):
    T = topk_idx.shape[0]
    dev = topk_idx.device
    i32 = dict(dtype=torch.int32, device=dev)
    counts = torch.empty(p.n_experts, **i32)
    offsets = torch.empty(p.n_experts + 1, **i32)
    sorted_token = torch.empty(T * p.topk, **i32)
    row_of = torch.empty((T, p.topk), **i32)
    _check(lib().moe_permute(ctypes.byref(p.c()), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                             _ptr(sorted_token), _ptr(row_of), _ptr(workspace), workspace.numel(),
                             _stream(stream)))
    return counts, offsets, sorted_token, row_of


@dataclass
class DeviceWeights:
    """Device copies of one layer's weights (storage format) and the C struct."""
    w_router: torch.Tensor
    bias: Optional[torch.Tensor]
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    w1_scale: Optional[torch.Tensor] = None
    w3_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None
    ws1: Optional[torch.Tensor] = None
    ws3: Optional[torch.Tensor] = None
    ws2: Optional[torch.Tensor] = None
    ws1_scale: Optional[torch.Tensor] = None
    ws3_scale: Optional[torch.Tensor] = None
    ws2_scale: Optional[torch.Tensor] = None

    def c(self) -> moe_weights:
        return moe_weights(*[_ptr(getattr(self, f)) for f, _ in moe_weights._fields_])


def moe_expert_ffn(p: Params, x, sorted_token, offsets, w: DeviceWeights, workspace, out=None,
                   stream=None):
    """Routed experts -> expert_out [T*topk, dim] in the expert-contiguous order."""
    T = x.shape[0]
    out = out if out is not None else torch.empty((T * p.topk, p.dim), dtype=p.act_torch,
                                                  device=x.device)
    cw = w.c()
    _check(lib().moe_expert_ffn(ctypes.byref(p.c()), T, _ptr(x), _ptr(sorted_token),
                                _ptr(offsets), ctypes.byref(cw), _ptr(out),
                                _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def moe_combine(p: Params, x, expert_out, row_of, topk_w, w: Optional[DeviceWeights], workspace,
                y=None, stream=None):
    """Shared expert on x plus the weighted combine of the routed outputs -> y [T, dim].
    w supplies the shared weights (may be None when p.shared_inter == 0)."""
    T = row_of.shape[0]
    y = y if y is not None else torch.empty((T, p.dim), dtype=p.act_torch, device=row_of.device)
    cw = None if w is None else w.c()
    _check(lib().moe_combine(ctypes.byref(p.c()), T, _ptr(x), _ptr(expert_out), _ptr(row_of),
                             _ptr(topk_w), None if cw is None else ctypes.byref(cw), _ptr(y),
                             _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def moe_forward(p: Params, x, w: DeviceWeights, workspace, y=None, topk_idx=None, topk_w=None,
                counts=None, stream=None):
    T = x.shape[0]
    y = y if y is not None else torch.empty((T, p.dim), dtype=p.act_torch, device=x.device)
    cw = w.c()
    _check(lib().moe_forward(ctypes.byref(p.c()), T, _ptr(x), ctypes.byref(cw), _ptr(y),
                             _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    return y


def moe_forward_noalloc(p: Params, x, w: DeviceWeights, y=None, topk_idx=None, topk_w=None,
                        counts=None, stream=None):
    """moe_forward on the library's own device scratch (no workspace argument)."""
    T = x.shape[0]
    y = y if y is not None else torch.empty((T, p.dim), dtype=p.act_torch, device=x.device)
    cw = w.c()
    _check(lib().moe_forward_noalloc(ctypes.byref(p.c()), T, _ptr(x), ctypes.byref(cw), _ptr(y),
                                     _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _stream(stream)))
    return y


def moe_quant_fp8(x, stream=None):
    """bf16 [rows, cols] -> (e4m3fn codes uint8 [rows, cols], fp32 scales [rows, cols/128])."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sc = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    _check(lib().moe_quant_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(sc), _stream(stream)))
    return q, sc


def moe_pack_weights(w, stream=None):
    """Row-major expert matrix (device tensor whose last dim is the input width;
    leading dims are stacked rows) -> a new tensor of the same shape and dtype
    holding the tiled layout the expert kernels read."""
    w = w.contiguous()
    row_bytes = w.shape[-1] * w.element_size()
    rows = w.numel() // w.shape[-1]
    out = torch.empty_like(w)
    _check(lib().moe_pack_weights(_ptr(w), rows, row_bytes, _ptr(out), _stream(stream)))
    return out


def moe_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Enqueue one streaming read of every byte of buf (measurement helper)."""
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(stream)))


def moe_profile_start(max_calls: int):
    _check(lib().moe_profile_start(max_calls))


def moe_profile_stop():
    """-> (calls recorded, summed up-projection ms, summed down-projection ms)."""
    n, up, dn = ctypes.c_int32(), ctypes.c_float(), ctypes.c_float()
    _check(lib().moe_profile_stop(ctypes.byref(n), ctypes.byref(up), ctypes.byref(dn)))
    return n.value, up.value, dn.value


# ---------------------------------------------------------------------------
# host <-> device helpers for storage-format arrays (numpy in, torch out)
# ---------------------------------------------------------------------------

def to_device(a, dtype_tag: str, device="cuda") -> torch.Tensor:
    """numpy storage array -> device tensor of the matching torch dtype (bit copy)."""
    import numpy as np
    if dtype_tag == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype_tag == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn)
    elif dtype_tag in ("f32", "i32", "u8"):
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        raise ValueError(dtype_tag)
    return t.to(device)


def upload_layer(layer, device="cuda", experts=None) -> DeviceWeights:
    """Copy a drawn layer's weights (storage format) to the device; the expert
    matrices are rewritten into the tiled layout (moe_pack_weights).
    experts=(b, e): only the routed experts b..e-1 are uploaded (an expert
    range, see Params.expert_begin / expert_end)."""
    cfg = layer.cfg
    wd = cfg.w_dtype
    sl = slice(None) if experts is None else slice(experts[0], experts[1])
    f32 = lambda a: None if a is None else to_device(a[sl] if a.ndim == 3 else a, "f32", device)

    def mat(a):
        t = to_device(a, wd, device)
        packed = moe_pack_weights(t)
        del t
        return packed
    bias = None if layer.bias is None else to_device(layer.bias, "f32", device)
    dw = DeviceWeights(to_device(layer.wr, cfg.router_dtype, device), bias,
                       mat(layer.w1[sl]), mat(layer.w3[sl]), mat(layer.w2[sl]), f32(layer.w1_s),
                       f32(layer.w3_s), f32(layer.w2_s))
    if layer.shared is not None:
        s = layer.shared
        dw.ws1, dw.ws3, dw.ws2 = mat(s.w1), mat(s.w3), mat(s.w2)
        g = lambda a: None if a is None else to_device(a, "f32", device)
        dw.ws1_scale, dw.ws3_scale, dw.ws2_scale = g(s.w1_s), g(s.w3_s), g(s.w2_s)
    return dw


def to_host_values(t: torch.Tensor):
    """Device tensor (bf16 / f32) -> numpy fp32 values."""
    return t.detach().float().cpu().numpy()
