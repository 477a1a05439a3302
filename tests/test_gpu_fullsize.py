"""Whole-layer parity at the five workload sizes (the launch configuration the
benchmark times), on sampled tokens the oracle computes one by one, plus the
routing of every token."""

import os
import time

import numpy as np
import pytest
import torch

from mixture_experts_layer_11_amd import inputs, moe
from tests.test_gpu_parity import forward_and_check

pytestmark = pytest.mark.gpu

SAMPLE = {0: None, 1: 24, 2: 12, 3: 384, 4: 12}


def progress(msg):
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(d):
        with open(os.path.join(d, "progress.log"), "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_forward_full_size(ci):
    cfg = inputs.CONFIGS[ci]
    progress(f"{cfg.name}: drawing inputs")
    layer = inputs.draw_layer(cfg)
    progress(f"{cfg.name}: uploading")
    dw = moe.upload_layer(layer)
    n = SAMPLE[ci]
    tokens = None
    if n is not None:
        rng = np.random.default_rng(ci)
        tokens = np.sort(rng.choice(cfg.T, n, replace=False))
    progress(f"{cfg.name}: forward + oracle on {n or cfg.T} tokens")
    try:
        _, same = forward_and_check(cfg, layer, dw, tokens=tokens)
    except moe.MoeError as e:
        if e.status == moe.MOE_ERR_UNSUPPORTED:
            pytest.skip(str(e))
        raise
    progress(f"{cfg.name}: done, routing agreed on {same.mean():.4f}")
    del dw, layer
    torch.cuda.empty_cache()
