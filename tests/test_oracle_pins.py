"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

Each test pins one part of the oracle to something it cannot share a mistake
with: a hand-worked fixture, a library routine (torch conv1d / autograd in
float64), a closed form, an invariant between two differently coded entry
points (the padded-history prefill vs the shift-coded decode and verify), or
finite differences that are exact because the loss is linear in each operand.
"""
import json
import os

import numpy as np
import pytest
import torch

from gated_short_causal_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        return json.load(f)


def _split(inp, H):
    inp = np.asarray(inp, dtype=np.float64)
    return inp[:, :H], inp[:, H:2 * H], inp[:, 2 * H:3 * H]


def _conv1d_forward(inp, cu, w):
    """Zero-state forward through torch's grouped conv1d in float64 (library routine):
    y[t] = C[t] * sum_k w[k] * bx[t-(K-1)+k], i.e. left padding K-1 and the first T outputs."""
    H, K = w.shape
    B, C, xv = _split(inp, H)
    y = np.zeros((inp.shape[0], H))
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        bx = torch.from_numpy((B[a:b] * xv[a:b]).T.copy())[None]          # [1, H, T]
        wt = torch.from_numpy(np.asarray(w, dtype=np.float64))[:, None, :]  # [H, 1, K]
        conv = torch.nn.functional.conv1d(bx, wt, padding=K - 1, groups=H)[0, :, : b - a]
        y[a:b] = C[a:b] * conv.T.numpy()
    return y


# ---------------------------------------------------------------- hand-worked fixture

def test_golden_prefill_with_state(oracle_mod):
    g = _golden()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    y, newpool = oracle_mod.prefill(g["in"], [0, 4], g["w"], pool=pool, slot_idx=[0])
    np.testing.assert_array_equal(y, np.array(g["expected_y"], dtype=np.float64))
    np.testing.assert_array_equal(newpool[0], np.array(g["expected_state"], dtype=np.float64))


def test_golden_prefill_zero_state(oracle_mod):
    g = _golden()
    y, newpool = oracle_mod.prefill(g["in"], [0, 4], g["w"])
    assert newpool is None
    np.testing.assert_array_equal(y, np.array(g["expected_y_zero_state"], dtype=np.float64))


def test_golden_backward(oracle_mod):
    g = _golden()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    d_in, dW = oracle_mod.backward(g["in"], [0, 4], g["w"], g["dy"], pool=pool, slot_idx=[0])
    np.testing.assert_array_equal(d_in, np.array(g["expected_d_in"], dtype=np.float64))
    np.testing.assert_array_equal(dW, np.array(g["expected_dW"], dtype=np.float64))


def test_golden_decode(oracle_mod):
    g = _golden()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    y, newpool = oracle_mod.decode(g["decode"]["in"], g["w"], pool, [0])
    np.testing.assert_array_equal(y, np.array(g["decode"]["expected_y"], dtype=np.float64))
    np.testing.assert_array_equal(newpool[0], np.array(g["decode"]["expected_state"], dtype=np.float64))


def test_golden_verify_and_commit(oracle_mod):
    g = _golden()
    pool = np.array(g["state0"], dtype=np.float64)[None]
    L = g["verify"]["L"]
    y, tape = oracle_mod.verify(np.array(g["in"])[:L], g["w"], pool, [0], L)
    np.testing.assert_array_equal(tape[0], np.array(g["verify"]["expected_tape"], dtype=np.float64))
    np.testing.assert_array_equal(y, np.array(g["verify"]["expected_y"], dtype=np.float64))
    for a in range(L + 1):
        newpool = oracle_mod.commit(tape, [a], pool, [0])
        want = pool[0] if a == 0 else tape[0, a - 1]
        np.testing.assert_array_equal(newpool[0], want)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_prefill_zero_state_matches_conv1d(oracle_mod, K):
    lens = [7, 0, 1, 2, 13, 5]
    case = wl.random_case(100 + K, lens, H=12, K=K, dtype=torch.float32)
    y, _ = oracle_mod.prefill(case.inp, case.cu, case.w)
    ref = _conv1d_forward(oracle_mod.f64(case.inp), case.cu.numpy(), oracle_mod.f64(case.w))
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_prefill_bf16_inputs_match_conv1d(oracle_mod):
    case = wl.random_case(7, [33, 64, 1], H=16, K=3, dtype=torch.bfloat16)
    y, _ = oracle_mod.prefill(case.inp, case.cu, case.w)
    ref = _conv1d_forward(oracle_mod.f64(case.inp), case.cu.numpy(), oracle_mod.f64(case.w))
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_backward_matches_torch_autograd(oracle_mod):
    """Gradients of sum(dy * y) through the conv1d formulation, by torch autograd in float64."""
    for K in (1, 3, 4):
        case = wl.random_case(200 + K, [9, 3, 1, 0, 6], H=8, K=K, dtype=torch.float32, with_dy=True)
        H = case.H
        inp = case.inp.double().clone().requires_grad_(True)
        w = case.w.double().clone().requires_grad_(True)
        dy = case.dy.double()
        cu = case.cu.tolist()
        loss = 0.0
        for i in range(len(cu) - 1):
            a, b = cu[i], cu[i + 1]
            if a == b:
                continue
            B, C, xv = inp[a:b, :H], inp[a:b, H:2 * H], inp[a:b, 2 * H:3 * H]
            conv = torch.nn.functional.conv1d((B * xv).T[None], w[:, None, :], padding=K - 1, groups=H)[0, :, : b - a].T
            loss = loss + (dy[a:b] * C * conv).sum()
        loss.backward()
        d_in, dW = oracle_mod.backward(case.inp, case.cu, case.w, case.dy)
        np.testing.assert_allclose(d_in, inp.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, w.grad.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_k1_closed_form(oracle_mod):
    """K = 1: the state is just the last bx, so y = C * w * B * xv and the final state is bx[T-1]."""
    case = wl.random_case(11, [5, 1, 8], H=8, K=1, dtype=torch.float32, slots=5)
    y, newpool = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    B, C, xv = _split(oracle_mod.f64(case.inp), case.H)
    w = oracle_mod.f64(case.w)[:, 0]
    np.testing.assert_allclose(y, C * w * B * xv, rtol=1e-15, atol=0)
    cu = case.cu.tolist()
    for i, s in enumerate(case.slot_idx.tolist()):
        last = cu[i + 1] - 1
        np.testing.assert_array_equal(newpool[s][:, 0], B[last] * xv[last])


def test_t1_zero_state_backward_closed_form(oracle_mod):
    """T = 1 from a zero state: only tap K-1 sees data, so dW[:, K-1] = g * bx and the other taps are 0;
    dC = dy * w[K-1] * bx, dB = w[K-1] * g * xv, dxv = w[K-1] * g * B."""
    case = wl.random_case(12, [1], H=16, K=3, dtype=torch.float32, with_dy=True)
    d_in, dW = oracle_mod.backward(case.inp, case.cu, case.w, case.dy)
    B, C, xv = _split(oracle_mod.f64(case.inp), case.H)
    w = oracle_mod.f64(case.w)
    dy = oracle_mod.f64(case.dy)
    g = dy * C
    bx = B * xv
    np.testing.assert_allclose(dW[:, 2], (g * bx)[0], rtol=1e-15)
    np.testing.assert_array_equal(dW[:, :2], 0.0)
    np.testing.assert_allclose(d_in[:, 16:32], dy * w[:, 2] * bx, rtol=1e-14)
    np.testing.assert_allclose(d_in[:, :16], w[:, 2] * g * xv, rtol=1e-14)
    np.testing.assert_allclose(d_in[:, 32:], w[:, 2] * g * B, rtol=1e-14)


# ---------------------------------------------------------------- invariants

def test_chained_decode_equals_prefill(oracle_mod):
    """Prefill of 56 tokens then 8 decode steps == one 64-token prefill (the 'full vs prefill+decode'
    check of the InfiniLM PR); prefill is coded through the padded history, decode through the shift."""
    case = wl.tiny_fp32()
    H, K = case.H, case.K
    pool0 = np.zeros((1, H, K))
    y_full, pool_full = oracle_mod.prefill(case.inp, [0, 64], case.w, pool=pool0, slot_idx=[0])
    y_a, pool = oracle_mod.prefill(case.inp[:56], [0, 56], case.w, pool=pool0, slot_idx=[0])
    ys = [y_a]
    for t in range(56, 64):
        y_t, pool = oracle_mod.decode(case.inp[t:t + 1], case.w, pool, [0])
        ys.append(y_t)
    np.testing.assert_allclose(np.concatenate(ys), y_full, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(pool, pool_full)


def test_chained_decode_equals_prefill_random_state(oracle_mod):
    case = wl.random_case(13, [20], H=8, K=4, dtype=torch.float32, slots=3)
    y_full, pool_full = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    pool = oracle_mod.f64(case.pool)
    ys = []
    for t in range(20):
        y_t, pool = oracle_mod.decode(case.inp[t:t + 1], case.w, pool, case.slot_idx)
        ys.append(y_t)
    np.testing.assert_allclose(np.concatenate(ys), y_full, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(pool, pool_full)


def test_prefill_split_invariance(oracle_mod):
    """prefill(T1) then prefill(T2) from the returned state == prefill(T1 + T2), for every split,
    including splits shorter than K (T1 < K mixes the old state into the new one)."""
    case = wl.random_case(14, [11], H=8, K=4, dtype=torch.float32, slots=2)
    y_full, pool_full = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    for t1 in range(0, 12):
        y1, p1 = oracle_mod.prefill(case.inp[:t1], [0, t1], case.w, case.pool, case.slot_idx)
        y2, p2 = oracle_mod.prefill(case.inp[t1:], [0, 11 - t1], case.w, p1, case.slot_idx)
        np.testing.assert_allclose(np.concatenate([y1, y2]), y_full, rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(p2, pool_full)


def test_empty_prefill_is_noop(oracle_mod):
    case = wl.random_case(15, [0, 0], H=8, K=3, dtype=torch.float32, slots=4)
    y, newpool = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    assert y.shape == (0, 8)
    np.testing.assert_array_equal(newpool, oracle_mod.f64(case.pool))


def test_ragged_isolation(oracle_mod):
    """Packed prefill == each sequence alone: no history crosses a sequence boundary (the hazard the
    InfiniLM PR avoids by rejecting packed prefill of different lengths)."""
    lens = [5, 1, 0, 9, 2, 3]
    case = wl.random_case(16, lens, H=8, K=3, dtype=torch.float32, slots=10)
    y, pool = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    cu = case.cu.tolist()
    for i, s in enumerate(case.slot_idx.tolist()):
        a, b = cu[i], cu[i + 1]
        yi, pi = oracle_mod.prefill(case.inp[a:b], [0, b - a], case.w, case.pool[s:s + 1], [0])
        np.testing.assert_array_equal(y[a:b], yi)
        np.testing.assert_array_equal(pool[s], pi[0])
    untouched = sorted(set(range(10)) - set(case.slot_idx.tolist()))
    np.testing.assert_array_equal(pool[untouched], oracle_mod.f64(case.pool)[untouched])


def test_dead_state_entry(oracle_mod):
    """Entry 0 of an incoming state is shifted out before any product: changing it changes no output
    (and no final state once at least one token is consumed); changing any other entry changes y[0]."""
    case = wl.random_case(17, [6, 1], H=8, K=3, dtype=torch.float32, slots=2)
    y0, p0 = oracle_mod.prefill(case.inp, case.cu, case.w, case.pool, case.slot_idx)
    pool = oracle_mod.f64(case.pool).copy()
    pool[:, :, 0] += 1000.0
    y1, p1 = oracle_mod.prefill(case.inp, case.cu, case.w, pool, case.slot_idx)
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(p0, p1)
    for k in (1, 2):
        pool = oracle_mod.f64(case.pool).copy()
        pool[:, :, k] += 1.0
        y2, _ = oracle_mod.prefill(case.inp, case.cu, case.w, pool, case.slot_idx)
        assert np.all(y2[0] != y0[0])


def test_verify_equals_decode_steps(oracle_mod):
    """tape[i][s] == state after s+1 decode steps, y == the decode outputs, pool untouched."""
    N, L, H, K = 3, 5, 8, 3
    g = torch.Generator().manual_seed(18)
    inp = torch.randn(N * L, 3 * H, generator=g)
    w = torch.rand(H, K, generator=g) - 0.5
    pool = torch.randn(6, H, K, generator=g)
    slots = [4, 0, 2]
    pool_before = oracle_mod.f64(pool).copy()
    y, tape = oracle_mod.verify(inp, w, pool, slots, L)
    np.testing.assert_array_equal(oracle_mod.f64(pool), pool_before)
    p = pool_before
    for s in range(L):
        rows = [i * L + s for i in range(N)]
        y_s, p = oracle_mod.decode(inp[rows], w, p, slots)
        np.testing.assert_allclose(y[rows], y_s, rtol=1e-15, atol=1e-15)
        for i in range(N):
            np.testing.assert_array_equal(tape[i, s], p[slots[i]])


def test_commit_equals_accepted_decode_steps(oracle_mod):
    N, L, H, K = 4, 6, 8, 3
    g = torch.Generator().manual_seed(19)
    inp = torch.randn(N * L, 3 * H, generator=g)
    w = torch.rand(H, K, generator=g) - 0.5
    pool = oracle_mod.f64(torch.randn(8, H, K, generator=g))
    slots = [7, 1, 3, 5]
    accept = [0, 1, 6, 3]
    _, tape = oracle_mod.verify(inp, w, pool, slots, L)
    committed = oracle_mod.commit(tape, accept, pool, slots)
    for i in range(N):
        p = pool.copy()
        for s in range(accept[i]):
            _, p = oracle_mod.decode(inp[i * L + s:i * L + s + 1], w, p, [slots[i]])
        np.testing.assert_array_equal(committed[slots[i]], p[slots[i]])
    untouched = [0, 2, 4, 6]
    np.testing.assert_array_equal(committed[untouched], pool[untouched])


# ---------------------------------------------------------------- backward by exact finite differences

def _loss(oracle_mod, inp, cu, w, dy, pool, slots):
    y, _ = oracle_mod.prefill(inp, cu, w, pool, slots)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("with_state", [False, True])
def test_backward_exact_directional_derivatives(oracle_mod, with_state):
    """L = sum(dy * y) is linear in each of B, C, xv and w taken alone, so a central difference along
    a direction that moves one of them is exact up to fp64 rounding; it must equal <grad, direction>."""
    lens = [6, 1, 0, 4, 2]
    case = wl.random_case(20 + with_state, lens, H=8, K=3, dtype=torch.float32, slots=6 if with_state else 0,
                          with_dy=True)
    H = case.H
    inp, w, dy = oracle_mod.f64(case.inp), oracle_mod.f64(case.w), oracle_mod.f64(case.dy)
    pool = oracle_mod.f64(case.pool) if with_state else None
    slots = case.slot_idx if with_state else None
    d_in, dW = oracle_mod.backward(inp, case.cu, w, dy, pool, slots)
    rng = np.random.default_rng(5)
    eps = 0.5
    for part in range(3):
        V = np.zeros_like(inp)
        V[:, part * H:(part + 1) * H] = rng.standard_normal((inp.shape[0], H))
        fd = (_loss(oracle_mod, inp + eps * V, case.cu, w, dy, pool, slots)
              - _loss(oracle_mod, inp - eps * V, case.cu, w, dy, pool, slots)) / (2 * eps)
        an = float(np.sum(d_in * V))
        assert abs(fd - an) <= 1e-10 * max(1.0, abs(an)), (part, fd, an)
    Vw = rng.standard_normal(w.shape)
    fd = (_loss(oracle_mod, inp, case.cu, w + eps * Vw, dy, pool, slots)
          - _loss(oracle_mod, inp, case.cu, w - eps * Vw, dy, pool, slots)) / (2 * eps)
    an = float(np.sum(dW * Vw))
    assert abs(fd - an) <= 1e-10 * max(1.0, abs(an)), (fd, an)


def test_backward_elementwise_fd_tiny(oracle_mod):
    """Every single input element on a tiny case: gradient entry == exact central difference."""
    case = wl.random_case(22, [3, 2], H=2, K=3, dtype=torch.float32, slots=2, with_dy=True)
    inp, w, dy = oracle_mod.f64(case.inp), oracle_mod.f64(case.w), oracle_mod.f64(case.dy)
    pool = oracle_mod.f64(case.pool)
    d_in, dW = oracle_mod.backward(inp, case.cu, w, dy, pool, case.slot_idx)
    for idx in np.ndindex(*inp.shape):
        e = np.zeros_like(inp)
        e[idx] = 1.0
        fd = (_loss(oracle_mod, inp + e, case.cu, w, dy, pool, case.slot_idx)
              - _loss(oracle_mod, inp - e, case.cu, w, dy, pool, case.slot_idx)) / 2
        assert abs(fd - d_in[idx]) < 1e-12, (idx, fd, d_in[idx])
    for idx in np.ndindex(*w.shape):
        e = np.zeros_like(w)
        e[idx] = 1.0
        fd = (_loss(oracle_mod, inp, case.cu, w + e, dy, pool, case.slot_idx)
              - _loss(oracle_mod, inp, case.cu, w - e, dy, pool, case.slot_idx)) / 2
        assert abs(fd - dW[idx]) < 1e-12, (idx, fd, dW[idx])


def test_backward_ragged_isolation(oracle_mod):
    lens = [4, 0, 7, 1]
    case = wl.random_case(23, lens, H=8, K=3, dtype=torch.float32, slots=5, with_dy=True)
    d_in, dW = oracle_mod.backward(case.inp, case.cu, case.w, case.dy, case.pool, case.slot_idx)
    cu = case.cu.tolist()
    dW_sum = np.zeros_like(dW)
    for i, s in enumerate(case.slot_idx.tolist()):
        a, b = cu[i], cu[i + 1]
        di, dWi = oracle_mod.backward(case.inp[a:b], [0, b - a], case.w, case.dy[a:b], case.pool[s:s + 1], [0])
        np.testing.assert_array_equal(d_in[a:b], di)
        dW_sum += dWi
    np.testing.assert_allclose(dW, dW_sum, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- argument checks and threads

def test_oracle_rejects_bad_arguments(oracle_mod):
    case = wl.random_case(24, [3], H=8, K=3, dtype=torch.float32, slots=2)
    with pytest.raises(ValueError):
        oracle_mod.prefill(case.inp, [0, 5], case.w)             # cu past the rows
    with pytest.raises(ValueError):
        oracle_mod.prefill(case.inp, [0, 3], case.w, case.pool, [7])  # slot out of range
    with pytest.raises(ValueError):
        oracle_mod.commit(np.zeros((1, 2, 8, 3)), [3], case.pool, [0])  # accept > L


def test_thread_count_does_not_change_results(oracle_mod):
    case = wl.random_case(25, [40, 17], H=64, K=3, dtype=torch.float32, slots=3, with_dy=True)
    old = oracle_mod.get_threads()
    try:
        oracle_mod.set_threads(1)
        a = oracle_mod.backward(case.inp, case.cu, case.w, case.dy, case.pool, case.slot_idx)
        oracle_mod.set_threads(4)
        b = oracle_mod.backward(case.inp, case.cu, case.w, case.dy, case.pool, case.slot_idx)
    finally:
        oracle_mod.set_threads(old)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
