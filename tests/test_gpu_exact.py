"""GPU parity at full width and bit for bit.

* The headline training step (one sequence, T=65536, H=2048, K=3, bf16) compared
  with the fp64 oracle on every one of the 2048 channels (channels are
  independent, so the oracle runs on channel blocks of 512 and each block is
  exact for its channels).
* Integer-valued inputs (small nonzero integers, exact in bf16): every product
  and sum of the op is then an exact integer far below 2^24, held exactly by
  fp32 arithmetic, so y, d_in, the states, the initial-state gradient, dW and
  dbias have exactly one correct bit pattern (the exact value, rounded once).  Any dropped, doubled or misplaced token -- at a
  window boundary, in the head rows, in the remainder of a batch of rows in
  flight -- changes dW by a nonzero integer and fails the bitwise compare.
* Rows outside [cu[0], cu[N]) are never written.

The op: MAX Pipelines LFM2 article, "ShortConv implementation (LFM2ShortConv)";
its backward per the Liger-Kernel LFM2 PR, "Kernel changes / Gated short
convolution" (the gradient formulas are derived from the forward definition).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from gated_short_causal_amd import workloads as wl
from gated_short_causal_amd import lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_prefill_ragged
from tests.parity_util import assert_bits, assert_close, rounded

pytestmark = pytest.mark.gpu
DEV = "cuda"
BLOCK = 512   # channels per oracle call in the full-width compares


def _say(msg):
    print(msg, flush=True)


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _sub(c, chans):
    """The workload restricted to channels `chans` (in_proj columns of B, C and xv, dy, weight, pool)."""
    H = c.H
    cols = torch.cat([chans, chans + H, chans + 2 * H])
    pool = None if c.pool is None else c.pool[:, chans].contiguous()
    sub = wl.Workload(c.name + "_sub", c.dtype, len(chans), c.K, c.inp[:, cols].contiguous(), c.w[chans].contiguous(),
                      cu=c.cu, pool=pool, slot_idx=c.slot_idx, dy=c.dy[:, chans].contiguous())
    return sub, cols


def _run_step(g, pool=None, slot_idx=None, bias=None, d_final=None, state_grads=False):
    """Forward into y (pool advanced in place when given), then the backward from the initial pool."""
    T, H, K = g.inp.shape[0], g.H, g.K
    N = g.cu.numel() - 1
    pool0 = None if pool is None else pool.clone()
    y = _nan((T, H), g.dtype)
    lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, pool, slot_idx, bias=bias)
    d_in = _nan((T, 3 * H), g.dtype)
    dW = torch.full((H, K), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV) if state_grads else None
    di = _nan((N, H, K), g.dtype) if state_grads else None
    ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(g.dtype, H, K, T, N)), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, pool0, slot_idx, bias=bias, d_final_state=d_final,
                    dbias=db, d_init_state=di)
    torch.cuda.synchronize()
    return y, d_in, dW, db, di


def test_train_T65536_all_channels():
    """The bench's training step at full size, y / d_in / dW on all 2048 channels within the bf16 tolerance."""
    _say("case: train bf16 T=65536 H=2048 K=3, all 2048 channels")
    c = wl.train_lfm2(T=65536)
    g = c.to(DEV)
    y, d_in, dW, _, _ = _run_step(g)
    oracle.set_threads(_threads())
    for b0 in range(0, c.H, BLOCK):
        chans = torch.arange(b0, b0 + BLOCK)
        sub, cols = _sub(c, chans)
        y_ref, _ = oracle.prefill(sub.inp, sub.cu, sub.w)
        assert_close(y[:, b0:b0 + BLOCK], y_ref, c.dtype, f"y channels {b0}..{b0 + BLOCK - 1}")
        d_ref, dW_ref = oracle.backward(sub.inp, sub.cu, sub.w, sub.dy)
        assert_close(d_in[:, cols.to(DEV)], d_ref, c.dtype, f"d_in channels {b0}..{b0 + BLOCK - 1}")
        assert_close(dW[b0:b0 + BLOCK], dW_ref, c.dtype, f"dW channels {b0}..{b0 + BLOCK - 1}")
        _say(f"  channels {b0}..{b0 + BLOCK - 1} match")


def _exact_compare(c, y, d_in, dW, db=None, di=None, pool_after=None, rows=None):
    """Every output of the integer workload equals the oracle's exact value, bit for bit, on every channel
    (on the token rows `rows` when given: the rows that belong to a sequence)."""
    rsel = slice(None) if rows is None else rows
    oracle.set_threads(_threads())
    bias = c.extra.get("bias")
    dF = c.extra.get("d_final")
    for b0 in range(0, c.H, BLOCK):
        b1 = min(c.H, b0 + BLOCK)
        chans = torch.arange(b0, b1)
        sub, cols = _sub(c, chans)
        sb = None if bias is None else bias[chans]
        sdF = None if dF is None else dF[:, chans].contiguous()
        y_ref, p_ref = oracle.prefill(sub.inp, sub.cu, sub.w, sub.pool, sub.slot_idx, bias=sb)
        d_ref, dW_ref, db_ref, di_ref = oracle.backward(sub.inp, sub.cu, sub.w, sub.dy, sub.pool, sub.slot_idx,
                                                        bias=sb, d_final=sdF, full=True)
        # the premise of the bitwise compare: every reference value is an integer below 2^24, so the kernels'
        # fp32 arithmetic holds it exactly and both sides round the same exact value once at the store
        for name, r in (("y", y_ref), ("d_in", d_ref), ("dW", dW_ref), ("d_init", di_ref), ("dbias", db_ref)):
            fin = r[np.isfinite(r)]
            assert np.all(fin == np.round(fin)) and np.all(np.abs(fin) < (1 << 24)), f"{name}: reference not exact"
        tag = f"channels {b0}..{b1 - 1}"
        assert_bits(y[rsel, b0:b1], rounded(y_ref[rsel], c.dtype), f"y {tag}")
        assert_bits(d_in[rsel][:, cols.to(DEV)], rounded(d_ref[rsel], c.dtype), f"d_in {tag}")
        assert_bits(dW[b0:b1], rounded(dW_ref, torch.float32), f"dW {tag}")
        if db is not None:
            assert_bits(db[b0:b1], rounded(db_ref, torch.float32), f"dbias {tag}")
        if di is not None:
            assert_bits(di[:, b0:b1], rounded(di_ref, c.dtype), f"d_init {tag}")
        if pool_after is not None:
            assert_bits(pool_after[:, b0:b1], rounded(p_ref, c.dtype), f"states {tag}")
        _say(f"  {tag} bit-exact")


def test_train_T65536_integer_bit_exact():
    """The headline launch configuration (one 65,536-token sequence, zero state, bf16) on integer inputs: y,
    d_in and dW bit-exact on all 2048 channels.  Each wave's window of ~261 tokens ends in a partial batch of
    rows in flight, so window starts, head rows and batch remainders are all exercised."""
    _say("case: train bf16 T=65536 H=2048 K=3, integer inputs, bit-exact")
    c = wl.integer_case(501, [65536])
    g = c.to(DEV)
    y, d_in, dW, _, _ = _run_step(g)
    _exact_compare(c, y, d_in, dW)


RAGGED_INT = [
    # (lens, H, K): many sequences split over several windows each, with every remainder of the batched rows,
    # sequences shorter than K, an empty one, and channel counts that leave a partial 512-channel group
    ([1, 2, 3, 1000, 4097, 0, 5, 777, 10001, 64, 2, 3333], 2048, 3),
    ([7, 2049, 1, 300, 5000, 2], 1032, 4),
    ([2, 9, 4099, 1, 643], 520, 2),
    # window lengths from the measured rate tables of 3 KiB and 2 KiB rows (one round of windows of ~132 and
    # ~81 tokens, then the table's pick a few tokens longer), with sequence gaps on the virtual axis
    ([9000, 13, 17000, 3, 14000], 1536, 3),
    ([25000, 5, 15000, 1], 1024, 3),
]


@pytest.mark.parametrize("lens,H,K", RAGGED_INT)
def test_ragged_integer_bit_exact(lens, H, K):
    """Ragged multi-window training step from integer initial states, with bias and a final-state gradient: y,
    final states, d_in, dW, dbias and the initial-state gradient all bit-exact."""
    _say(f"case: ragged integer bit-exact lens={lens} H={H} K={K}")
    c = wl.integer_case(600 + H + K, lens, H=H, K=K, slots=len(lens) + 5, bias=True, d_final=True)
    g = c.to(DEV)
    pool = g.pool.clone()
    y, d_in, dW, db, di = _run_step(g, pool, g.slot_idx, bias=c.extra["bias"].to(DEV),
                                    d_final=c.extra["d_final"].to(DEV), state_grads=True)
    _exact_compare(c, y, d_in, dW, db, di, pool_after=pool)


def test_rows_outside_cu_untouched():
    """cu[0] > 0 and cu[N] < total_T: rows before the first sequence and after the last one stay unwritten in y
    (prefill) and d_in (backward); the rows inside match the oracle bit for bit (integer inputs)."""
    _say("case: rows outside [cu[0], cu[N]) untouched")
    lens = [300, 1, 2047, 5]
    H, K, lead, tail = 1024, 3, 37, 29
    c0 = wl.integer_case(700, [lead] + lens + [tail], H=H, K=K, slots=8)
    # drop the first and last "sequences": their rows become rows that belong to no sequence
    cu = c0.cu[1:-1].contiguous()
    c = wl.Workload("outside", c0.dtype, H, K, c0.inp, c0.w, cu=cu, pool=c0.pool,
                    slot_idx=c0.slot_idx[1:len(lens) + 1].contiguous(), dy=c0.dy)
    assert int(cu[0]) == lead and int(cu[-1]) == c.inp.shape[0] - tail
    g = c.to(DEV)
    pool = g.pool.clone()
    pool0 = g.pool.clone()
    y, d_in, dW, _, _ = _run_step(g, pool, g.slot_idx)
    T = c.inp.shape[0]
    outside = torch.cat([torch.arange(lead), torch.arange(T - tail, T)]).to(DEV)
    assert torch.isnan(y[outside]).all(), "y rows outside the sequences were written"
    assert torch.isnan(d_in[outside]).all(), "d_in rows outside the sequences were written"
    _exact_compare(c, y, d_in, dW, pool_after=pool, rows=slice(lead, T - tail))
    untouched = torch.ones(8, dtype=torch.bool)
    untouched[c.slot_idx.long()] = False
    assert_bits(pool[untouched.to(DEV)], pool0[untouched.to(DEV)], "slots not named keep their bytes")
