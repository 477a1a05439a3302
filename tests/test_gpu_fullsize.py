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

# sampled tokens per workload (None: every token)
SAMPLE = {"c0": None, "c1": 24, "c2": 12, "c3": 384, "c4": 12}


def progress(msg):
    """Progress lines for long runs, appended to $MOE_PROGRESS_FILE when set."""
    path = os.environ.get("MOE_PROGRESS_FILE")
    if path:
        with open(path, "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(SAMPLE))
def test_forward_full_size(name):
    cfg = inputs.config_by_name(name)
    ci = list(SAMPLE).index(name)
    progress(f"{cfg.name}: drawing inputs")
    layer = inputs.draw_layer(cfg)
    progress(f"{cfg.name}: uploading")
    dw = moe.upload_layer(layer)
    n = SAMPLE[name]
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
