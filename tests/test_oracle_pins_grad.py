"""Pins of the oracle's conv bias and state-gradient paths (CPU only).

Bias: conv gets a per-channel bias before the C gate; the backward returns dbias.
State gradients: the backward returns the gradient of each sequence's initial
state and accepts a gradient arriving at its final state, so a long sequence
can be trained in chunks.  Each is pinned to hand-worked values, to torch fp64
autograd through an independent formulation, to exact finite differences, and
to the chunked-training invariant.
"""
import json
import os

import numpy as np
import pytest
import torch

from gated_short_causal_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-worked values

def test_golden_bias_forward_backward(oracle_mod):
    g = _g()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    b = g["bias"]["b"]
    y, newpool = oracle_mod.prefill(g["in"], [0, 4], g["w"], pool=pool, slot_idx=[0], bias=b)
    np.testing.assert_array_equal(y, np.array(g["bias"]["expected_y"], dtype=np.float64))
    np.testing.assert_array_equal(newpool[0], np.array(g["expected_state"], dtype=np.float64))
    d_in, dW, dbias, _ = oracle_mod.backward(g["in"], [0, 4], g["w"], g["dy"], pool=pool, slot_idx=[0], bias=b,
                                             full=True)
    expect = np.array(g["expected_d_in"], dtype=np.float64)
    expect[:, 2:4] = np.array(g["bias"]["expected_dC"], dtype=np.float64)
    np.testing.assert_array_equal(d_in, expect)
    np.testing.assert_array_equal(dW, np.array(g["expected_dW"], dtype=np.float64))
    np.testing.assert_array_equal(dbias, np.array(g["bias"]["expected_dbias"], dtype=np.float64))


def test_golden_bias_decode_and_verify(oracle_mod):
    g = _g()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    b = np.array(g["bias"]["b"], dtype=np.float64)
    yv, _ = oracle_mod.verify(np.array(g["in"])[:2], g["w"], pool, [0], 2, bias=b)
    np.testing.assert_array_equal(yv, np.array(g["bias"]["expected_y"], dtype=np.float64)[:2])
    yd, _ = oracle_mod.decode(np.array(g["in"])[:1], g["w"], pool, [0], bias=b)
    np.testing.assert_array_equal(yd, np.array(g["bias"]["expected_y"], dtype=np.float64)[:1])


def test_golden_state_gradients(oracle_mod):
    g = _g()
    sg = g["state_grads"]
    pool = np.array(g["state0"], dtype=np.float64)[None]
    d_in, dW, _, d_init = oracle_mod.backward(g["in"], [0, 4], g["w"], g["dy"], pool=pool, slot_idx=[0], full=True)
    np.testing.assert_array_equal(d_init[0], np.array(sg["expected_dS0"], dtype=np.float64))
    dF = np.array(sg["dF"], dtype=np.float64)[None]
    d_in, dW2, _, d_init = oracle_mod.backward(g["in"], [0, 4], g["w"], g["dy"], pool=pool, slot_idx=[0],
                                               d_final=dF, full=True)
    np.testing.assert_array_equal(d_in, np.array(sg["expected_d_in_with_dF"], dtype=np.float64))
    np.testing.assert_array_equal(d_init[0], np.array(sg["expected_dS0"], dtype=np.float64))
    np.testing.assert_array_equal(dW2, np.array(g["expected_dW"], dtype=np.float64))
    one = sg["one_token"]
    d_in, dW, _, d_init = oracle_mod.backward(np.array(g["in"])[:1], [0, 1], g["w"], np.array(g["dy"])[:1],
                                              pool=pool, slot_idx=[0], d_final=dF, full=True)
    np.testing.assert_array_equal(d_init[0], np.array(one["expected_dS0"], dtype=np.float64))
    np.testing.assert_array_equal(d_in, np.array(one["expected_d_in"], dtype=np.float64))
    np.testing.assert_array_equal(dW, np.array(one["expected_dW"], dtype=np.float64))


# ---------------------------------------------------------------- library routine: torch autograd

def _torch_loss(inp, cu, w, bias, S0, dy, dF):
    """sum(dy*y) + sum(dF*final_state) through torch's grouped conv1d over the explicit history
    [S0 | B*xv] (no padding), in float64; the final state is the last K history columns."""
    H, K = w.shape
    loss = 0.0
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        T = b - a
        B, C, xv = inp[a:b, :H], inp[a:b, H:2 * H], inp[a:b, 2 * H:3 * H]
        X = torch.cat([S0[i], (B * xv).T], dim=1)                       # [H, K+T]
        if T:
            conv = torch.nn.functional.conv1d(X[None, :, 1:], w[:, None, :], bias=bias, groups=H)[0]  # [H, T]
            loss = loss + (dy[a:b] * C * conv.T).sum()
        loss = loss + (dF[i] * X[:, T:T + K]).sum()
    return loss


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_full_backward_matches_torch_autograd(oracle_mod, K):
    lens = [7, 0, 1, 2, 5]
    case = wl.random_case(300 + K, lens, H=6, K=K, dtype=torch.float32, slots=7, with_dy=True)
    gen = torch.Generator().manual_seed(400 + K)
    bias = torch.randn(6, generator=gen, dtype=torch.float64)
    dF = torch.randn(len(lens), 6, K, generator=gen, dtype=torch.float64)
    inp = case.inp.double().clone().requires_grad_(True)
    w = case.w.double().clone().requires_grad_(True)
    b = bias.clone().requires_grad_(True)
    S0 = case.pool.double()[case.slot_idx.long()].clone().requires_grad_(True)
    loss = _torch_loss(inp, case.cu.tolist(), w, b, S0, case.dy.double(), dF)
    loss.backward()
    d_in, dW, dbias, d_init = oracle_mod.backward(case.inp, case.cu, case.w, case.dy, case.pool, case.slot_idx,
                                                  bias=bias, d_final=dF, full=True)
    np.testing.assert_allclose(d_in, inp.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW, w.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dbias, b.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d_init, S0.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_bias_forward_matches_torch_conv1d(oracle_mod):
    case = wl.random_case(310, [9, 1, 4], H=5, K=3, dtype=torch.float32, slots=3)
    bias = np.random.default_rng(1).standard_normal(5)
    y, _ = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx, bias=bias)
    inp = case.inp.double()
    S0 = case.pool.double()[case.slot_idx.long()]
    cu = case.cu.tolist()
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        X = torch.cat([S0[i], (inp[a:b, :5] * inp[a:b, 10:15]).T], dim=1)
        conv = torch.nn.functional.conv1d(X[None, :, 1:], case.w.double()[:, None, :],
                                          bias=torch.from_numpy(bias), groups=5)[0]
        np.testing.assert_allclose(y[a:b], (inp[a:b, 5:10] * conv.T).numpy(), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- exact finite differences

def _loss(oracle_mod, inp, cu, w, bias, pool, slots, dy, dF):
    y, newpool = oracle_mod.prefill(inp, cu, w, pool, slots, bias=bias)
    final = newpool[np.asarray(slots)]
    return float(np.sum(dy * y) + np.sum(dF * final))


def test_bias_and_state_directional_derivatives(oracle_mod):
    """The loss is linear in the bias and in the initial states taken alone, so central differences along
    random directions are exact up to fp64 rounding."""
    lens = [6, 1, 0, 3, 2]
    case = wl.random_case(320, lens, H=8, K=3, dtype=torch.float32, slots=8, with_dy=True)
    rng = np.random.default_rng(3)
    bias = rng.standard_normal(8)
    dF = rng.standard_normal((5, 8, 3))
    inp, w, dy = oracle_mod.f64(case.inp), oracle_mod.f64(case.w), oracle_mod.f64(case.dy)
    pool = oracle_mod.f64(case.pool)
    slots = case.slot_idx.numpy()
    d_in, dW, dbias, d_init = oracle_mod.backward(inp, case.cu, w, dy, pool, slots, bias=bias, d_final=dF, full=True)
    eps = 0.5
    vb = rng.standard_normal(8)
    fd = (_loss(oracle_mod, inp, case.cu, w, bias + eps * vb, pool, slots, dy, dF)
          - _loss(oracle_mod, inp, case.cu, w, bias - eps * vb, pool, slots, dy, dF)) / (2 * eps)
    assert abs(fd - float(np.sum(dbias * vb))) < 1e-10 * max(1.0, abs(fd))
    vs = rng.standard_normal(pool.shape)
    p_plus, p_minus = pool + eps * vs, pool - eps * vs
    fd = (_loss(oracle_mod, inp, case.cu, w, bias, p_plus, slots, dy, dF)
          - _loss(oracle_mod, inp, case.cu, w, bias, p_minus, slots, dy, dF)) / (2 * eps)
    an = float(np.sum(d_init * vs[slots]))
    assert abs(fd - an) < 1e-10 * max(1.0, abs(fd)), (fd, an)
    for part in range(3):
        V = np.zeros_like(inp)
        V[:, part * 8:(part + 1) * 8] = rng.standard_normal((inp.shape[0], 8))
        fd = (_loss(oracle_mod, inp + eps * V, case.cu, w, bias, pool, slots, dy, dF)
              - _loss(oracle_mod, inp - eps * V, case.cu, w, bias, pool, slots, dy, dF)) / (2 * eps)
        an = float(np.sum(d_in * V))
        assert abs(fd - an) < 1e-10 * max(1.0, abs(fd)), (part, fd, an)


# ---------------------------------------------------------------- chunked training invariant

def test_chunked_backward_equals_whole_sequence(oracle_mod):
    """Backward of [chunk 1 | chunk 2]: chunk 2 runs from chunk 1's final state and its initial-state
    gradient feeds chunk 1 as the final-state gradient; the pieces must reassemble the whole backward
    (including cuts shorter than K, where chunk 2's history reaches into chunk 1's initial state)."""
    case = wl.random_case(330, [13], H=6, K=4, dtype=torch.float32, slots=2, with_dy=True)
    rng = np.random.default_rng(4)
    bias = rng.standard_normal(6)
    dF = rng.standard_normal((1, 6, 4))
    inp, w, dy = oracle_mod.f64(case.inp), oracle_mod.f64(case.w), oracle_mod.f64(case.dy)
    pool = oracle_mod.f64(case.pool)
    sl = case.slot_idx.numpy()
    whole = oracle_mod.backward(inp, [0, 13], w, dy, pool, sl, bias=bias, d_final=dF, full=True)
    for cut in range(0, 14):
        _, p1 = oracle_mod.prefill(inp[:cut], [0, cut], w, pool, sl, bias=bias)
        b2 = oracle_mod.backward(inp[cut:], [0, 13 - cut], w, dy[cut:], p1, sl, bias=bias, d_final=dF, full=True)
        b1 = oracle_mod.backward(inp[:cut], [0, cut], w, dy[:cut], pool, sl, bias=bias, d_final=b2[3], full=True)
        np.testing.assert_allclose(np.concatenate([b1[0], b2[0]]), whole[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b1[1] + b2[1], whole[1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b1[2] + b2[2], whole[2], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b1[3], whole[3], rtol=1e-12, atol=1e-12)
