"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Values must match within |gpu - ref| <= max(atol, rtol*|ref|) (2e-2 for bf16
I/O, 1e-5 for fp32).  State, tape and slot handling are bit-exact: a written
state or tape entry equals the oracle value rounded once to the I/O dtype, and
every slot not named by a call keeps its bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_short_causal_amd import workloads as wl
from gated_short_causal_amd import (lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_commit_window,
                                    lfm2sc_decode_step, lfm2sc_prefill_ragged, lfm2sc_verify_window)
from tests.parity_util import assert_bits, assert_close, rounded

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def gpu_prefill(case, pool=None, slot_idx=None, y_pad=0):
    y = _nan_like((case.inp.shape[0], case.H + y_pad), case.dtype)
    lfm2sc_prefill_ragged(case.inp, case.cu, case.w, y[:, :case.H] if y_pad else y, pool, slot_idx)
    torch.cuda.synchronize()
    return y[:, :case.H]


def gpu_backward(case, pool=None, slot_idx=None):
    T = case.inp.shape[0]
    N = case.cu.numel() - 1
    d_in = _nan_like((T, 3 * case.H), case.dtype)
    dW = torch.full((case.H, case.K), float("nan"), dtype=torch.float32, device=DEV)
    nb = lfm2sc_backward_workspace_bytes(case.dtype, case.H, case.K, T, N)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(case.inp, case.cu, case.w, case.dy, d_in, dW, ws, pool, slot_idx)
    torch.cuda.synchronize()
    return d_in, dW


# ------------------------------------------------------------------ tiny fp32 (full vs prefill + decode)

def test_tiny_fp32_prefill_decode_backward():
    _say("case: tiny fp32 T=64 H=256 K=3")
    c = wl.tiny_fp32()
    g = c.to(DEV)
    y_ref, _ = oracle.prefill(c.inp, c.cu, c.w)
    y = gpu_prefill(g)
    assert_close(y, y_ref, torch.float32, "tiny prefill y")

    # 56-token prefill into a zeroed slot, then 8 decode steps == the 64-token prefill
    pool = torch.zeros(3, c.H, c.K, dtype=torch.float32, device=DEV)
    slot = torch.tensor([1], dtype=torch.int32, device=DEV)
    y56 = _nan_like((56, c.H), torch.float32)
    lfm2sc_prefill_ragged(g.inp[:56], torch.tensor([0, 56], dtype=torch.int32, device=DEV), g.w, y56, pool, slot)
    ys = [y56]
    for t in range(56, 64):
        yt = _nan_like((1, c.H), torch.float32)
        lfm2sc_decode_step(g.inp[t:t + 1], g.w, pool, slot, yt)
        ys.append(yt)
    torch.cuda.synchronize()
    y_chain = torch.cat(ys)
    assert_close(y_chain, y_ref, torch.float32, "prefill(56)+8 decodes vs oracle prefill(64)")
    # fp32: the carried state is the exact fp32 product either way, so the chain equals the GPU prefill bitwise
    assert_bits(y_chain, y, "GPU chained decode vs GPU prefill")
    _, pool_ref = oracle.prefill(c.inp, c.cu, c.w, np.zeros((1, c.H, c.K)), [0])
    assert_bits(pool[1], rounded(pool_ref[0], torch.float32), "final state after chain")
    assert_bits(pool[0], torch.zeros(c.H, c.K), "untouched slot 0")
    assert_bits(pool[2], torch.zeros(c.H, c.K), "untouched slot 2")

    d_ref, dW_ref = oracle.backward(c.inp, c.cu, c.w, c.dy)
    d_in, dW = gpu_backward(g)
    assert_close(d_in, d_ref, torch.float32, "tiny d_in")
    assert_close(dW, dW_ref, torch.float32, "tiny dW")


# ------------------------------------------------------------------ decode, LFM2-1.2B shape

def test_decode_lfm2_bf16():
    _say("case: decode bf16 N=256 pool=1024 H=2048 K=3")
    c = wl.decode_lfm2()
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan_like((256, c.H), c.dtype)
    lfm2sc_decode_step(g.inp, g.w, g.pool, g.slot_idx, y)
    torch.cuda.synchronize()
    y_ref, pool_ref = oracle.decode(c.inp, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "decode y")
    used = c.slot_idx.long()
    assert_bits(g.pool[used.to(DEV)], rounded(pool_ref[used.numpy()], c.dtype), "decode written slots")
    mask = torch.ones(1024, dtype=torch.bool)
    mask[used] = False
    assert_bits(g.pool[mask.to(DEV)], pool0[mask.to(DEV)], "decode untouched slots")


def test_decode_lfm2_bf16_N4096():
    """The larger decode batch bench.py times: 4096 sequences of an 8192-slot pool, full compare."""
    _say("case: decode bf16 N=4096 pool=8192 H=2048 K=3")
    c = wl.decode_lfm2(seed=250, N=4096, slots=8192)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan_like((4096, c.H), c.dtype)
    lfm2sc_decode_step(g.inp, g.w, g.pool, g.slot_idx, y)
    torch.cuda.synchronize()
    y_ref, pool_ref = oracle.decode(c.inp, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "decode y")
    used = c.slot_idx.long()
    assert_bits(g.pool[used.to(DEV)], rounded(pool_ref[used.numpy()], c.dtype), "decode written slots")
    mask = torch.ones(8192, dtype=torch.bool)
    mask[used] = False
    assert_bits(g.pool[mask.to(DEV)], pool0[mask.to(DEV)], "decode untouched slots")


# ------------------------------------------------------------------ ragged prefill

def test_ragged_prefill_lfm2_bf16():
    c = wl.ragged_prefill_lfm2()
    _say(f"case: ragged prefill bf16 lens={c.extra['lens']} H=2048 K=3")
    g = c.to(DEV)
    y = gpu_prefill(g, g.pool, g.slot_idx)
    y_ref, pool_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "ragged prefill y")
    assert_bits(g.pool, rounded(pool_ref, c.dtype), "ragged prefill final states")


def test_ragged_prefill_guard_slots_and_chunking():
    """A 16-slot pool with 8 used, short and long sequences: untouched slots keep their bytes."""
    c = wl.ragged_prefill_lfm2(seed=31, N=8, lo=1, hi=300, slots=16)
    _say(f"case: ragged prefill guard lens={c.extra['lens']}")
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = gpu_prefill(g, g.pool, g.slot_idx)
    y_ref, pool_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "y")
    used = c.slot_idx.long()
    assert_bits(g.pool[used.to(DEV)], rounded(pool_ref[used.numpy()], c.dtype), "written slots")
    mask = torch.ones(16, dtype=torch.bool)
    mask[used] = False
    assert_bits(g.pool[mask.to(DEV)], pool0[mask.to(DEV)], "untouched slots")


# ------------------------------------------------------------------ verify + commit

def test_verify_and_commit_lfm2_bf16():
    _say("case: verify bf16 N=64 L=8 pool=256")
    c = wl.verify_lfm2()
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan_like((512, c.H), c.dtype)
    win = _nan_like((64, 8, c.H, c.K), c.dtype)
    lfm2sc_verify_window(g.inp, g.w, g.pool, g.slot_idx, 8, win, y)
    torch.cuda.synchronize()
    y_ref, tape_ref = oracle.verify(c.inp, c.w, c.pool, c.slot_idx, 8)
    assert_close(y, y_ref, c.dtype, "verify y")
    assert_bits(win, rounded(tape_ref, c.dtype), "verify tape")
    assert_bits(g.pool, pool0, "pool untouched by verify")

    lfm2sc_commit_window(win, g.accept, g.pool, g.slot_idx)
    torch.cuda.synchronize()
    # the oracle commits its own tape (rounded as stored); the GPU tape was just shown equal to it bitwise
    pool_ref = oracle.commit(rounded(tape_ref, c.dtype), c.accept, c.pool, c.slot_idx)
    assert_bits(g.pool, rounded(pool_ref, c.dtype), "pool after commit")


# ------------------------------------------------------------------ training fwd + bwd

def test_train_T4096_full():
    _say("case: train bf16 T=4096 H=2048 K=3 (full compare)")
    c = wl.train_lfm2(T=4096)
    g = c.to(DEV)
    y = gpu_prefill(g)
    y_ref, _ = oracle.prefill(c.inp, c.cu, c.w)
    assert_close(y, y_ref, c.dtype, "train y")
    d_in, dW = gpu_backward(g)
    d_ref, dW_ref = oracle.backward(c.inp, c.cu, c.w, c.dy)
    assert_close(d_in, d_ref, c.dtype, "train d_in")
    assert_close(dW, dW_ref, c.dtype, "train dW")


def _channel_subset(c, chans):
    """Channels are independent: the oracle on a column subset is exact for those channels."""
    H = c.H
    cols = torch.cat([chans, chans + H, chans + 2 * H])
    sub = wl.Workload(c.name + "_sub", c.dtype, len(chans), c.K, c.inp[:, cols].contiguous(), c.w[chans].contiguous(),
                      cu=c.cu, dy=c.dy[:, chans].contiguous())
    return sub, cols


def _train_sampled(c, n_random, seed):
    """The training step on the device at full size, then the oracle on the first and last 8 channels plus
    `n_random` others (channels are independent, so the subset is exact for them)."""
    H = c.H
    g = c.to(DEV)
    y = gpu_prefill(g)
    d_in, dW = gpu_backward(g)
    assert torch.isfinite(y).all() and torch.isfinite(d_in).all() and torch.isfinite(dW).all()
    gen = torch.Generator().manual_seed(seed)
    chans = torch.cat([torch.arange(8), torch.arange(H - 8, H), torch.randperm(H - 16, generator=gen)[:n_random] + 8])
    chans = torch.sort(chans).values
    sub, cols = _channel_subset(c, chans)
    T = c.inp.shape[0]
    y_ref, _ = oracle.prefill(sub.inp, sub.cu, sub.w)
    assert_close(y[:, chans.to(DEV)], y_ref, c.dtype, f"T={T} y (sampled channels)")
    d_ref, dW_ref = oracle.backward(sub.inp, sub.cu, sub.w, sub.dy)
    assert_close(d_in[:, cols.to(DEV)], d_ref, c.dtype, f"T={T} d_in (sampled channels)")
    assert_close(dW[chans.to(DEV)], dW_ref, c.dtype, f"T={T} dW (sampled channels)")


def test_train_T65536_sampled_channels():
    _say("case: train bf16 T=65536 H=2048 K=3 (sampled channels + whole-output properties)")
    _train_sampled(wl.train_lfm2(T=65536), 112, 55)


@pytest.mark.parametrize("H,K,dtype", [(1024, 3, torch.bfloat16), (1536, 3, torch.bfloat16), (2048, 2, torch.bfloat16),
                                       (2048, 4, torch.bfloat16), (2048, 3, torch.float32)])
def test_train_T65536_other_shapes_sampled(H, K, dtype):
    """The other channel counts, tap counts and I/O type that bench.py times at T=65536, in that launch
    configuration (one 65,536-token sequence, zero state): sampled channels against the oracle."""
    _say(f"case: train T=65536 H={H} K={K} {dtype} (sampled channels)")
    _train_sampled(wl.train_lfm2(seed=60 + K, T=65536, H=H, K=K, dtype=dtype), 24, 56 + H + K)


# ------------------------------------------------------------------ edge cases

EDGE = [
    # (lens, H, K, dtype, slots, in_pad)
    ([1], 8, 3, torch.float32, 2, 0),
    ([2, 1, 0, 3], 8, 3, torch.float32, 6, 8),
    ([0, 0, 5], 24, 2, torch.bfloat16, 4, 0),
    ([5, 17, 64, 1, 2, 200, 333], 520, 3, torch.bfloat16, 9, 16),
    ([31, 7, 129], 2056, 4, torch.bfloat16, 3, 0),
    ([100, 3], 264, 1, torch.float32, 2, 0),
    ([1000, 1, 1, 999], 1024, 3, torch.float32, 5, 8),
    ([65, 3, 300], 512, 4, torch.float32, 0, 0),
]


@pytest.mark.parametrize("lens,H,K,dtype,slots,pad", EDGE)
def test_edge_prefill_backward(lens, H, K, dtype, slots, pad):
    _say(f"case: edge lens={lens} H={H} K={K} {dtype} slots={slots} pad={pad}")
    c = wl.random_case(1000 + H + K, lens, H=H, K=K, dtype=dtype, slots=slots, with_dy=True, in_pad=pad)
    g = c.to(DEV)
    pool_args = (g.pool, g.slot_idx) if slots else (None, None)
    pool0 = g.pool.clone() if slots else None
    y = gpu_prefill(g, *pool_args, y_pad=8)
    y_ref, pool_ref = oracle.prefill(c.inp[:, :3 * H], c.cu, c.w, c.pool, c.slot_idx)
    if c.inp.shape[0]:
        assert_close(y, y_ref, dtype, "edge y")
    d_in, dW = gpu_backward(g, pool0, g.slot_idx if slots else None)
    d_ref, dW_ref = oracle.backward(c.inp[:, :3 * H], c.cu, c.w, c.dy, c.pool, c.slot_idx)
    if c.inp.shape[0]:
        assert_close(d_in, d_ref, dtype, "edge d_in")
    assert_close(dW, dW_ref, dtype, "edge dW")
    if slots:
        assert_bits(g.pool, rounded(pool_ref, dtype), "edge pool (written + untouched slots)")


def test_empty_calls():
    _say("case: empty calls")
    H, K = 16, 3
    w = torch.zeros(H, K, dtype=torch.bfloat16, device=DEV)
    inp = torch.zeros(0, 3 * H, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(0, H, dtype=torch.bfloat16, device=DEV)
    lfm2sc_prefill_ragged(inp, torch.zeros(1, dtype=torch.int32, device=DEV), w, y)
    lfm2sc_prefill_ragged(inp, torch.zeros(3, dtype=torch.int32, device=DEV), w, y)
    dW = torch.full((H, K), float("nan"), device=DEV)
    lfm2sc_backward(inp, torch.zeros(3, dtype=torch.int32, device=DEV), w, y, torch.zeros(0, 3 * H, dtype=torch.bfloat16,
                    device=DEV), dW, None)
    torch.cuda.synchronize()
    assert torch.equal(dW, torch.zeros_like(dW)), "dW of an empty batch is zero"


def test_backward_deterministic():
    _say("case: backward determinism bf16 T=8192")
    c = wl.train_lfm2(seed=9, T=8192)
    g = c.to(DEV)
    a_in, a_w = gpu_backward(g)
    b_in, b_w = gpu_backward(g)
    assert_bits(a_in, b_in, "d_in rerun")
    assert_bits(a_w, b_w, "dW rerun")


def test_decode_chain_equals_verify_tape_fp32():
    """GPU decode steps reproduce the GPU verify tape and outputs bitwise (fp32)."""
    _say("case: decode chain vs verify fp32")
    c = wl.verify_lfm2(seed=41, N=5, L=6, slots=9, H=264, dtype=torch.float32)
    g = c.to(DEV)
    y_v = _nan_like((30, c.H), torch.float32)
    win = _nan_like((5, 6, c.H, c.K), torch.float32)
    lfm2sc_verify_window(g.inp, g.w, g.pool, g.slot_idx, 6, win, y_v)
    pool = g.pool.clone()
    for s in range(6):
        rows = torch.arange(5, device=DEV) * 6 + s
        ys = _nan_like((5, c.H), torch.float32)
        lfm2sc_decode_step(g.inp[rows].contiguous(), g.w, pool, g.slot_idx, ys)
        torch.cuda.synchronize()
        assert_bits(ys, y_v[rows], f"y step {s}")
        assert_bits(pool[g.slot_idx.long()], win[:, s], f"state step {s}")
