"""Pins of the oracle's conv update on gated inputs (oracle.conv_update): a hand-worked example, the separately
written verify and decode functions of the oracle (which see bx as B*xv with C = 1), and torch's conv1d over the
padded history."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))["conv_update"]


def test_golden_with_tape():
    out, tape, pool = oracle.conv_update(GOLD["bx"], GOLD["w"], GOLD["pool"], GOLD["slot_idx"])
    np.testing.assert_array_equal(out, np.array(GOLD["expected_out"]))
    np.testing.assert_array_equal(tape, np.array(GOLD["expected_tape"]))
    np.testing.assert_array_equal(pool, np.array(GOLD["pool"]))          # untouched with a tape


def test_golden_without_tape_and_bias():
    out, tape, pool = oracle.conv_update(GOLD["bx"], GOLD["w"], GOLD["pool"], GOLD["slot_idx"], with_tape=False)
    assert tape is None
    np.testing.assert_array_equal(pool, np.array(GOLD["expected_pool_without_tape"]))
    out_b, _, _ = oracle.conv_update(GOLD["bx"], GOLD["w"], GOLD["pool"], GOLD["slot_idx"], bias=GOLD["bias"])
    np.testing.assert_array_equal(out_b, np.array(GOLD["expected_out_with_bias"]))


def _case(seed, N, H, K, L, slots):
    rng = np.random.default_rng(seed)
    bx = rng.standard_normal((N, H, L))
    w = rng.uniform(-0.5, 0.5, (H, K))
    b = rng.standard_normal(H)
    pool = rng.standard_normal((slots, H, K))
    sl = rng.permutation(slots)[:N].astype(np.int32)
    return bx, w, b, pool, sl


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_matches_verify_with_unit_gates(K):
    """verify() on in_proj rows [B = bx | C = 1 | xv = 1] sees the same bx and an identity gate."""
    N, H, L = 5, 12, 6
    bx, w, b, pool, sl = _case(10 + K, N, H, K, L, 9)
    rows = bx.transpose(0, 2, 1).reshape(N * L, H)          # token-major rows of sequence-major blocks
    inp = np.concatenate([rows, np.ones_like(rows), np.ones_like(rows)], axis=1)
    y_ref, tape_ref = oracle.verify(inp, w, pool, sl, L, bias=b)
    out, tape, newpool = oracle.conv_update(bx, w, pool, sl, bias=b)
    np.testing.assert_allclose(out.transpose(0, 2, 1).reshape(N * L, H), y_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(tape, tape_ref.reshape(N, L, H, K), rtol=0, atol=0)
    np.testing.assert_array_equal(newpool, pool)


def test_without_tape_equals_chained_decode():
    N, H, K, L = 4, 10, 3, 5
    bx, w, b, pool, sl = _case(20, N, H, K, L, 7)
    out, _, newpool = oracle.conv_update(bx, w, pool, sl, bias=b, with_tape=False)
    p = pool.copy()
    for s in range(L):
        inp = np.concatenate([bx[:, :, s], np.ones((N, H)), np.ones((N, H))], axis=1)
        y, p = oracle.decode(inp, w, p, sl, bias=b)
        np.testing.assert_allclose(out[:, :, s], y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(newpool, p, rtol=0, atol=0)


@pytest.mark.parametrize("K", [1, 3, 4])
def test_matches_torch_conv1d_on_padded_history(K):
    N, H, L = 3, 8, 7
    bx, w, b, pool, sl = _case(30 + K, N, H, K, L, 5)
    out, _, _ = oracle.conv_update(bx, w, pool, sl, bias=b)
    for i in range(N):
        X = torch.cat([torch.from_numpy(pool[sl[i]][:, 1:]), torch.from_numpy(bx[i])], dim=1)   # [H, K-1+L]
        ref = F.conv1d(X.unsqueeze(0), torch.from_numpy(w).unsqueeze(1), bias=torch.from_numpy(b), groups=H)[0]
        np.testing.assert_allclose(out[i], ref.numpy(), rtol=1e-12, atol=1e-12)
