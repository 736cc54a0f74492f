"""Pins of the oracle's fused forward (in_proj followed by the ShortConv prefill) to values fixed outside it:
a hand-worked example, numpy's matmul for the linear map, and an independent torch pipeline (F.linear, a split,
a grouped conv1d) for the whole composition."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))["fused"]


def test_golden_in_proj():
    ip = oracle.in_proj(GOLD["x"], GOLD["W_in"])
    np.testing.assert_array_equal(ip, np.array(GOLD["expected_in_proj"]))


def test_golden_fused_one_sequence():
    c = GOLD["one_sequence_zero_state"]
    y, pool, ip = oracle.fused_prefill(np.array(GOLD["x"])[:c["rows"]], GOLD["W_in"], c["cu"], GOLD["w"])
    np.testing.assert_array_equal(y, np.array(c["expected_y"]))
    assert pool is None


def test_golden_fused_bias_and_state():
    c = GOLD["two_sequences_bias_state"]
    y, pool, ip = oracle.fused_prefill(GOLD["x"], GOLD["W_in"], c["cu"], GOLD["w"], pool=c["pool"],
                                       slot_idx=c["slot_idx"], bias=c["bias"])
    np.testing.assert_array_equal(y, np.array(c["expected_y"]))
    np.testing.assert_array_equal(pool, np.array(c["expected_pool"]))


@pytest.mark.parametrize("rows,D,n_out", [(37, 64, 24), (1, 8, 3), (0, 16, 6), (5, 2048, 12)])
def test_in_proj_matches_numpy_matmul(rows, D, n_out):
    rng = np.random.default_rng(rows * 7 + D)
    x = rng.standard_normal((rows, D))
    W = rng.standard_normal((n_out, D))
    np.testing.assert_allclose(oracle.in_proj(x, W), x @ W.T, rtol=1e-12, atol=1e-12)


def test_in_proj_padded_rows():
    """x rows wider than D (a padded buffer): only the first D columns enter the product."""
    rng = np.random.default_rng(3)
    xp = rng.standard_normal((9, 40))
    W = rng.standard_normal((12, 32))
    np.testing.assert_allclose(oracle.in_proj(xp, W), xp[:, :32] @ W.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_fused_matches_torch_pipeline(K):
    """Zero initial state, one sequence: y = C * conv1d(B*xv) with in_proj = F.linear(x, W_in), computed by torch
    in float64 with a causal (left-padded) grouped convolution."""
    T, D, H = 29, 48, 16
    g = torch.Generator().manual_seed(40 + K)
    x = torch.randn(T, D, generator=g, dtype=torch.float64)
    W = torch.randn(3 * H, D, generator=g, dtype=torch.float64) / D ** 0.5
    w = torch.rand(H, K, generator=g, dtype=torch.float64) - 0.5
    b = torch.randn(H, generator=g, dtype=torch.float64)
    ip = F.linear(x, W)
    B, C, xv = ip[:, :H], ip[:, H:2 * H], ip[:, 2 * H:]
    bx = (B * xv).t().unsqueeze(0)                                   # [1, H, T]
    conv = F.conv1d(F.pad(bx, (K - 1, 0)), w.unsqueeze(1), bias=b, groups=H)[0].t()
    y_ref = C * conv
    y, _, ip_o = oracle.fused_prefill(x.numpy(), W.numpy(), [0, T], w.numpy(), bias=b.numpy())
    np.testing.assert_allclose(ip_o, ip.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, y_ref.numpy(), rtol=1e-10, atol=1e-10)
