"""moe_forward_noalloc (the library's own device scratch, no workspace
argument) against moe_forward (a caller workspace): the same kernels on the
same inputs, so the outputs must be bitwise equal.  Two no-alloc calls in a
row, the second with fewer tokens, so the second runs on scratch the first
left behind."""

import pytest
import torch

from mixture_experts_layer_11_amd import inputs, moe

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("ci", [0, 1, 3, 7])     # fp32, bf16, fp8 stream tiles, fp8 decode
def test_noalloc_matches_forward_on_two_calls(ci):
    cfg = inputs.SMALL_CONFIGS[ci]
    layer = inputs.draw_layer(cfg)
    dw = moe.upload_layer(layer)
    p = moe.Params.from_config(cfg)
    x = moe.to_device(layer.x, cfg.act_dtype)
    sizes = (cfg.T, max(1, cfg.T // 3))
    refs = []
    for T in sizes:
        ws = moe.alloc_workspace(p, T)
        refs.append((moe.moe_forward(p, x[:T], dw, ws), ws))
    torch.cuda.synchronize()
    got = []
    for T in sizes:                                 # back to back on one stream
        idx = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
        got.append((moe.moe_forward_noalloc(p, x[:T], dw, topk_idx=idx), idx))
    torch.cuda.synchronize()
    for (y, _), (g, idx) in zip(refs, got):
        assert torch.equal(_bits(g), _bits(y))
        assert int(idx.min()) >= 0 and int(idx.max()) < cfg.E
