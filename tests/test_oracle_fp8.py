"""Pins of the oracle's fp8 expert path (the block scheme of the fp8 workload).

The scheme (weights: e4m3fn codes with one fp32 scale per 128x128 block;
activations, i.e. x before W1/W3 and h before W2, quantised per 1x128 block
with scale = amax/448) is the plainest reading of the workload description
and of the "DeepSeek-V3.2-Exp · Expert scores" dtype note (the block's other
linears run in FP8).  Two kinds of pin, neither of which re-types the oracle:

  * a worked example by hand: identity weights, so every intermediate value
    is a closed form (silu from math.exp) and every rounding decision is a
    position on the e4m3 grid that the comments below work out;
  * a structural property on random inputs: with W2 the identity, the expert
    output is the quantised h itself, so every 1x128 block of it must lie on
    an e4m3 grid scaled by that block's own maximum / 448.

test_oracle_mutations.py plants three plausible mistakes (h unquantised, h
quantised along tokens instead of along its row, x unquantised) and checks
that these pins catch each.
"""

import math

import numpy as np

import oracle
from mixture_experts_layer_11_amd import inputs

F32 = np.float32
E4M3_ONE = 0x38        # e4m3fn code of 1.0: exponent field 7 (bias 7), mantissa 0


def _silu(a):
    return a / (1.0 + math.exp(-a))


def _identity_fp8(n):
    """n x n identity as e4m3 codes with every 128x128 block scale 1.0."""
    q = np.zeros((n, n), np.uint8)
    q[np.arange(n), np.arange(n)] = E4M3_ONE
    return q, np.ones((n // 128, n // 128), F32)


def _bf16_vals(v):
    return inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.asarray(v, F32))).astype(np.float64)


def check_fp8_hand_example():
    """dim = inter = 128, W1 = W3 = W2 = identity (scale 1), two token rows.

    Row 0: x = [3.5, 0.8984375, 0, ...] (0.8984375 is 0.9 in bf16).
      x block: amax 3.5, scale 3.5/448 = 2^-7 (exact).  0.8984375 / 2^-7 = 115
      lies between the e4m3 values 112 and 120 (spacing 8 in [64, 128)) and is
      closer to 112, so x1 enters the matmuls as 112 * 2^-7 = 0.875.
      h = silu(x) * x elementwise (identity W1, W3): h0 = silu(3.5) 3.5,
      h1 = silu(0.875) 0.875.  h block: scale s0 = h0/448, h0 maps to 448;
      448 h1/h0 = 20.36 lies between 20 and 22 (spacing 2 in [16, 32)), so h1
      enters W2 as 20 s0.
    Row 1: x = [1.75, 0.8984375, 0, ...].
      scale 2^-8; 0.8984375 / 2^-8 = 230 lies between 224 and 240 (spacing 16
      in [128, 256)), closer to 224: x1 = 224 * 2^-8 = 0.875 again.
      h0 = silu(1.75) 1.75, s1 = h0/448; 448 h1/h0 = 92.78 lies between 88 and
      96 (spacing 8), closer to 96: h1 enters W2 as 96 s1.
    W2 = identity, so the output row is h as it entered W2, rounded to bf16.
    """
    n = 128
    x = np.zeros((2, n), F32)
    x[0, 0], x[1, 0] = 3.5, 1.75
    x[:, 1] = 0.8984375
    xv = _bf16_vals(x)
    assert xv[0, 1] == 0.8984375
    q, s = _identity_fp8(n)
    got = oracle.expert_ffn(xv, q, q, q, "fp8", "bf16", s, s, s)

    h1 = _silu(0.875) * 0.875                       # the same in both rows
    want = np.zeros((2, n))
    for r, (a0, code1, half_gap) in enumerate([(3.5, 20.0, 1.0), (1.75, 96.0, 4.0)]):
        h0 = _silu(a0) * a0
        scale = F32(F32(h0) / F32(448.0))            # fp32 amax / 448
        assert abs(448.0 * h1 / h0 - code1) < half_gap    # the grid position worked out above
        want[r, 0] = 448.0 * float(scale)
        want[r, 1] = code1 * float(scale)
    want = _bf16_vals(want)
    np.testing.assert_allclose(got[:, :2], want[:, :2], rtol=1e-3)
    assert not np.any(got[:, 2:])
    return got


def test_fp8_hand_example():
    check_fp8_hand_example()


def _on_scaled_e4m3_grid(v):
    """Each 1x128 block of v (bf16-rounded values) must be e4m3 codes times one
    scale, with the block's largest magnitude at code 448.  Returns the
    fraction of elements that are not."""
    grid = oracle.e4m3_table()[:0x7F]                # non-negative finite values, ascending
    M, K = v.shape
    bad = 0
    for r in range(M):
        for b in range(K // 128):
            blk = np.abs(v[r, b * 128:(b + 1) * 128])
            amax = blk.max()
            if amax == 0:
                continue
            u = blk * (448.0 / amax)                 # scale estimated from the block maximum
            j = np.clip(np.searchsorted(grid, u), 1, grid.size - 1)
            near = np.where(u - grid[j - 1] < grid[j] - u, grid[j - 1], grid[j])
            # bf16 rounding (at most 2^-8 relative) of the value and of the
            # block maximum; e4m3 values are 2^-3 to 2^-4 apart (relative)
            tol = 2.0 ** -7 * np.maximum(near, 1.0) + 1e-12
            bad += int(np.count_nonzero(np.abs(u - near) > tol))
    return bad / v.size


def check_fp8_h_on_block_grid(seed=0, M=24, dim=256):
    """Random x, W1, W3; W2 = identity: the output is the quantised h itself."""
    rng = np.random.default_rng(seed)
    x = _bf16_vals(rng.standard_normal((M, dim)))
    x[3, :128] *= 1e-3                               # one block of small values
    q1, s1 = inputs.quantize_weight_blocks((rng.standard_normal((dim, dim)) / 16).astype(F32))
    q3, s3 = inputs.quantize_weight_blocks((rng.standard_normal((dim, dim)) / 16).astype(F32))
    q2, s2 = _identity_fp8(dim)
    out = oracle.expert_ffn(x, q1, q3, q2, "fp8", "bf16", s1, s3, s2)
    frac = _on_scaled_e4m3_grid(out)
    assert frac == 0.0, frac
    return out


def test_fp8_h_lies_on_its_block_grid():
    check_fp8_h_on_block_grid()


def test_fp8_block_grid_check_rejects_unquantised_values():
    # the property is not vacuous: plain bf16 values of the same h are off-grid
    rng = np.random.default_rng(1)
    v = _bf16_vals(rng.standard_normal((8, 256)))
    assert _on_scaled_e4m3_grid(v) > 0.5
