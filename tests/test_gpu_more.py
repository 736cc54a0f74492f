"""More GPU parity and robustness cases through the C ABI (fp64 oracle as reference)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_short_causal_amd import workloads as wl
from gated_short_causal_amd import (Lfm2scError, lfm2sc_backward, lfm2sc_backward_workspace_bytes,
                                    lfm2sc_commit_window, lfm2sc_conv_update, lfm2sc_decode_step,
                                    lfm2sc_prefill_ragged, lfm2sc_verify_window)
from tests.parity_util import assert_bits, assert_close, rounded

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _say(msg):
    print(msg, flush=True)


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


@pytest.mark.parametrize("K,dtype,H,N,L", [
    (1, torch.bfloat16, 512, 3, 1), (2, torch.float32, 520, 5, 3), (4, torch.bfloat16, 1024, 7, 8),
    (3, torch.float32, 2048, 4, 5), (4, torch.float32, 24, 9, 2),
])
def test_decode_verify_commit_variants(K, dtype, H, N, L):
    _say(f"case: decode/verify/commit K={K} {dtype} H={H} N={N} L={L}")
    c = wl.verify_lfm2(seed=60 + K, N=N, L=L, slots=N + 5, H=H, K=K, dtype=dtype)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    # decode of the first token of each sequence
    rows = torch.arange(N) * L
    y = _nan((N, H), dtype)
    lfm2sc_decode_step(g.inp[rows.to(DEV)].contiguous(), g.w, g.pool, g.slot_idx, y)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.decode(c.inp[rows], c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, dtype, "decode y")
    assert_bits(g.pool, rounded(p_ref, dtype), "decode pool")
    # verify from the original pool, then commit every accept length
    g.pool.copy_(pool0)
    yv = _nan((N * L, H), dtype)
    win = _nan((N, L, H, K), dtype)
    lfm2sc_verify_window(g.inp, g.w, g.pool, g.slot_idx, L, win, yv)
    torch.cuda.synchronize()
    yv_ref, tape_ref = oracle.verify(c.inp, c.w, c.pool, c.slot_idx, L)
    assert_close(yv, yv_ref, dtype, "verify y")
    assert_bits(win, rounded(tape_ref, dtype), "verify tape")
    assert_bits(g.pool, pool0, "pool untouched by verify")
    acc = torch.arange(N, dtype=torch.int32) % (L + 1)
    lfm2sc_commit_window(win, acc.to(DEV), g.pool, g.slot_idx)
    torch.cuda.synchronize()
    p_ref = oracle.commit(rounded(tape_ref, dtype), acc, c.pool, c.slot_idx)
    assert_bits(g.pool, rounded(p_ref, dtype), "pool after commit")


def test_commit_all_accept_lengths_bf16():
    _say("case: commit accept lengths 0..L")
    c = wl.verify_lfm2(seed=71, N=9, L=8, slots=20)
    g = c.to(DEV)
    win = _nan((9, 8, c.H, c.K), c.dtype)
    y = _nan((72, c.H), c.dtype)
    lfm2sc_verify_window(g.inp, g.w, g.pool, g.slot_idx, 8, win, y)
    acc = torch.arange(9, dtype=torch.int32)
    lfm2sc_commit_window(win, acc.to(DEV), g.pool, g.slot_idx)
    torch.cuda.synchronize()
    _, tape_ref = oracle.verify(c.inp, c.w, c.pool, c.slot_idx, 8)
    p_ref = oracle.commit(rounded(tape_ref, c.dtype), acc, c.pool, c.slot_idx)
    assert_bits(g.pool, rounded(p_ref, c.dtype), "pool after commit")


def test_many_short_sequences_multi_round_tiling():
    """More sequences than resident workgroup windows: the tiling falls back to several rounds."""
    gen = torch.Generator().manual_seed(72)
    lens = torch.randint(0, 41, (300,), generator=gen).tolist()
    _say(f"case: 300 short sequences, total {sum(lens)}")
    c = wl.random_case(73, lens, H=2048, K=3, dtype=torch.bfloat16, slots=310, with_dy=True)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan((sum(lens), 2048), c.dtype)
    lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, g.pool, g.slot_idx)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "y")
    assert_bits(g.pool, rounded(p_ref, c.dtype), "pool")
    d_in = _nan((sum(lens), 6144), c.dtype)
    dW = _nan((2048, 3), torch.float32)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(c.dtype, 2048, 3, sum(lens), 300), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, pool0, g.slot_idx)
    torch.cuda.synchronize()
    d_ref, dW_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx)
    assert_close(d_in, d_ref, c.dtype, "d_in")
    assert_close(dW, dW_ref, c.dtype, "dW")


def test_wide_channels_h8192():
    _say("case: H=8192 K=3 bf16 ragged")
    c = wl.random_case(74, [37, 300, 5], H=8192, K=3, dtype=torch.bfloat16, slots=4, with_dy=True)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan((342, 8192), c.dtype)
    lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, g.pool, g.slot_idx)
    d_in = _nan((342, 3 * 8192), c.dtype)
    dW = _nan((8192, 3), torch.float32)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(c.dtype, 8192, 3, 342, 3), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, pool0, g.slot_idx)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    d_ref, dW_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "y")
    assert_bits(g.pool, rounded(p_ref, c.dtype), "pool")
    assert_close(d_in, d_ref, c.dtype, "d_in")
    assert_close(dW, dW_ref, c.dtype, "dW")


def test_chunked_prefill_equals_oracle():
    """Prefill of a ragged batch in two chunks (state carried through the pool) against the oracle of the
    whole sequences; final states bit-exact, outputs within tolerance (the carried bf16 state is rounded)."""
    lens = [50, 3, 200, 1]
    cut = [20, 1, 199, 0]
    _say(f"case: chunked prefill lens={lens} cut={cut}")
    c = wl.random_case(75, lens, H=1024, K=3, dtype=torch.bfloat16, slots=6)
    g = c.to(DEV)
    cu = c.cu.tolist()
    first = torch.cat([torch.arange(cu[i], cu[i] + cut[i]) for i in range(4)])
    second = torch.cat([torch.arange(cu[i] + cut[i], cu[i + 1]) for i in range(4)])
    cu1 = torch.tensor([0] + list(np.cumsum(cut)), dtype=torch.int32)
    cu2 = torch.tensor([0] + list(np.cumsum([l - k for l, k in zip(lens, cut)])), dtype=torch.int32)
    y1 = _nan((len(first), 1024), c.dtype)
    y2 = _nan((len(second), 1024), c.dtype)
    lfm2sc_prefill_ragged(g.inp[first.to(DEV)].contiguous(), cu1.to(DEV), g.w, y1, g.pool, g.slot_idx)
    lfm2sc_prefill_ragged(g.inp[second.to(DEV)].contiguous(), cu2.to(DEV), g.w, y2, g.pool, g.slot_idx)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    y = torch.empty(sum(lens), 1024, dtype=c.dtype)
    y[first] = y1.cpu()
    y[second] = y2.cpu()
    assert_close(y, y_ref, c.dtype, "chunked y")
    assert_bits(g.pool, rounded(p_ref, c.dtype), "chunked final states")


def test_out_of_range_slots_are_skipped():
    """A slot id outside [0, num_slots) makes that sequence use a zero state and write nothing (the kernels
    check every slot before touching the pool); other sequences are unaffected."""
    _say("case: out-of-range slot ids")
    c = wl.decode_lfm2(seed=76, N=4, slots=6, H=512)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    bad = torch.tensor([2, 6, -1, 4], dtype=torch.int32)
    y = _nan((4, 512), c.dtype)
    lfm2sc_decode_step(g.inp, g.w, g.pool, bad.to(DEV), y)
    torch.cuda.synchronize()
    zero_pool = np.zeros((1, 512, 3))
    ok_rows = [0, 3]
    y_ok, p_ok = oracle.decode(c.inp[ok_rows], c.w, c.pool, bad[ok_rows])
    y_zero, _ = oracle.decode(c.inp[[1, 2]], c.w, zero_pool.repeat(2, 0), [0, 1])
    assert_close(y[ok_rows], y_ok, c.dtype, "valid rows")
    assert_close(y[[1, 2]], y_zero, c.dtype, "skipped rows use a zero state")
    expect = pool0.cpu().clone()
    expect[[2, 4]] = rounded(p_ok[[2, 4]], c.dtype)
    assert_bits(g.pool, expect, "pool: only valid slots written")


@pytest.mark.parametrize("K,dtype,H", [(1, torch.bfloat16, 2048), (2, torch.float32, 520), (3, torch.bfloat16, 520),
                                         (4, torch.bfloat16, 1024), (4, torch.float32, 24), (3, torch.float32, 2048)])
def test_decode_batches_staging_states(K, dtype, H):
    """Batches large enough that decode stages each wave's state block through LDS (600 sequences): every K,
    both dtypes, a channel count that leaves a partial wave group, some slot ids out of range (zero state,
    nothing written), and a conv bias.  y against the oracle, the pool bit for bit."""
    _say(f"case: staged decode K={K} {dtype} H={H} N=600")
    N, slots = 600, 700
    c = wl.decode_lfm2(seed=90 + K + H, N=N, slots=slots, H=H, K=K, dtype=dtype)
    slot_idx = c.slot_idx.clone()
    slot_idx[5] = slots          # past the pool
    slot_idx[77] = -3            # negative
    bias = (torch.rand(H, generator=torch.Generator().manual_seed(K)) - 0.5).to(dtype)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    y = _nan((N, H), dtype)
    lfm2sc_decode_step(g.inp, g.w, g.pool, slot_idx.to(DEV), y, bias=bias.to(DEV))
    torch.cuda.synchronize()
    ok = [i for i in range(N) if 0 <= int(slot_idx[i]) < slots]
    bad = [5, 77]
    y_ok, p_ok = oracle.decode(c.inp[ok], c.w, c.pool, slot_idx[ok], bias=bias)
    y_bad, _ = oracle.decode(c.inp[bad], c.w, np.zeros((2, H, K)), [0, 1], bias=bias)
    assert_close(y[ok], y_ok, dtype, "y, valid slots")
    assert_close(y[bad], y_bad, dtype, "y, skipped slots use a zero state")
    expect = pool0.cpu().clone()
    used = slot_idx[ok].long()
    expect[used] = rounded(p_ok[used.numpy()], dtype)
    assert_bits(g.pool, expect, "pool: valid slots advanced, every other slot untouched")


def test_decode_staged_padded_pool():
    """Staged decode (600 sequences) on a pool whose slots are padded apart (slot stride H*K + 72 elements):
    the slot blocks are advanced bit for bit and the padding between them stays untouched."""
    _say("case: staged decode, padded pool")
    N, slots, H, K = 600, 650, 2048, 3
    c = wl.decode_lfm2(seed=133, N=N, slots=slots, H=H, K=K)
    stride = H * K + 72
    big = torch.full((slots, stride), float("nan"), dtype=c.dtype)
    big[:, :H * K] = c.pool.reshape(slots, H * K)
    gbig = big.to(DEV)
    pool = torch.as_strided(gbig, (slots, H, K), (stride, K, 1))
    g = c.to(DEV)
    y = _nan((N, H), c.dtype)
    lfm2sc_decode_step(g.inp, g.w, pool, g.slot_idx, y)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.decode(c.inp, c.w, c.pool, c.slot_idx)
    assert_close(y, y_ref, c.dtype, "y")
    expect = big.clone()
    used = c.slot_idx.long()
    expect[used, :H * K] = rounded(p_ref[used.numpy()], c.dtype).reshape(len(used), H * K)
    assert_bits(gbig, expect, "padded pool: slots advanced, padding untouched")


def test_graph_capture_replays_match_eager():
    """Prefill + backward + decode captured in one HIP graph; each replay (with eager work and syncs in
    between) must reproduce the eager results bitwise."""
    _say("case: graph capture")
    c = wl.ragged_prefill_lfm2(seed=77, N=3, lo=5, hi=300, H=1024, slots=5)
    c.dy = torch.randn(c.inp.shape[0], 1024, generator=torch.Generator().manual_seed(78)).to(c.dtype)
    g = c.to(DEV)
    T, N = c.inp.shape[0], 3
    pool0 = g.pool.clone()
    y = torch.empty(T, 1024, dtype=c.dtype, device=DEV)
    d_in = torch.empty(T, 3072, dtype=c.dtype, device=DEV)
    dW = torch.empty(1024, 3, device=DEV)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(c.dtype, 1024, 3, T, N), dtype=torch.uint8, device=DEV)
    yd = torch.empty(N, 1024, dtype=c.dtype, device=DEV)
    dec_in = g.inp[:N].contiguous()

    def step():
        lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, g.pool, g.slot_idx)
        lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, g.pool, g.slot_idx)
        lfm2sc_decode_step(dec_in, g.w, g.pool, g.slot_idx, yd)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, d_in, dW, yd, g.pool)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.pool.copy_(pool0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    g.pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (y, d_in, dW, yd):
            t.fill_(float("nan"))
        g.pool.copy_(pool0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "d_in", "dW", "decode y", "pool"), (y, d_in, dW, yd, g.pool), ref):
            assert_bits(a, b, f"replay {rep}: {name}")


def test_graph_capture_staged_small_calls():
    """The small calls whose state or tape blocks go through LDS -- a 600-sequence decode, a verify window and
    a verify-shaped conv update on the transposed view -- captured in one graph; every replay (with eager work
    and syncs in between) reproduces the eager results bitwise."""
    _say("case: graph capture, staged small calls")
    H, K, N, L = 2048, 3, 600, 4
    d = wl.decode_lfm2(seed=141, N=N, slots=N + 40, H=H, K=K).to(DEV)
    v = wl.verify_lfm2(seed=142, N=48, L=L, slots=64, H=H, K=K).to(DEV)
    dpool0, vpool0 = d.pool.clone(), v.pool.clone()
    yd = torch.empty(N, H, dtype=d.dtype, device=DEV)
    yv = torch.empty(48 * L, H, dtype=v.dtype, device=DEV)
    win = torch.empty(48, L, H, K, dtype=v.dtype, device=DEV)
    bx = v.inp[:, :H].contiguous().view(48, L, H).transpose(1, 2)
    out = torch.empty(48, L, H, dtype=v.dtype, device=DEV).transpose(1, 2)
    tape = torch.empty(48, L, H, K, dtype=v.dtype, device=DEV)

    def step():
        lfm2sc_decode_step(d.inp, d.w, d.pool, d.slot_idx, yd)
        lfm2sc_verify_window(v.inp, v.w, v.pool, v.slot_idx, L, win, yv)
        lfm2sc_conv_update(bx, v.w, v.pool, v.slot_idx, out, windows=tape)

    step()
    torch.cuda.synchronize()
    outs = (yd, d.pool, yv, win, out, tape)
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.pool.copy_(dpool0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    d.pool.copy_(dpool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (yd, yv, win, out, tape):
            t.fill_(float("nan"))
        d.pool.copy_(dpool0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("decode y", "decode pool", "verify y", "verify tape", "conv update out",
                               "conv update tape"), outs, ref):
            assert_bits(a, b, f"replay {rep}: {name}")
    assert_bits(v.pool, vpool0, "verify and the tape-mode conv update leave the pool untouched")


_CHECK_SCRIPT = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from gated_short_causal_amd import lfm2sc_decode_step, lfm2sc_prefill_ragged, lfm2sc_commit_window, Lfm2scError
from gated_short_causal_amd import workloads as wl
dev = "cuda"
c = wl.decode_lfm2(seed=80, N=4, slots=8, H=512).to(dev)
y = torch.empty(4, 512, dtype=torch.bfloat16, device=dev)
def status(fn):
    try:
        fn(); torch.cuda.synchronize(); return 0
    except Lfm2scError as e:
        return e.status
res = []
res.append(status(lambda: lfm2sc_decode_step(c.inp, c.w, c.pool, c.slot_idx, y)))
dup = torch.tensor([1, 2, 1, 3], dtype=torch.int32, device=dev)
res.append(status(lambda: lfm2sc_decode_step(c.inp, c.w, c.pool, dup, y)))
oob = torch.tensor([1, 2, 8, 3], dtype=torch.int32, device=dev)
res.append(status(lambda: lfm2sc_decode_step(c.inp, c.w, c.pool, oob, y)))
badcu = torch.tensor([0, 3, 2, 4, 4], dtype=torch.int32, device=dev)
res.append(status(lambda: lfm2sc_prefill_ragged(c.inp, badcu, c.w, y, c.pool, c.slot_idx)))
win = torch.zeros(4, 2, 512, 3, dtype=torch.bfloat16, device=dev)
acc = torch.tensor([0, 1, 3, 2], dtype=torch.int32, device=dev)
res.append(status(lambda: lfm2sc_commit_window(win, acc, c.pool, c.slot_idx)))
from gated_short_causal_amd import lfm2sc_fused_prefill, lfm2sc_fused_prefill_workspace_bytes
f = wl.fused_case(81, [3, 5, 2, 6], H=512, K=3, D=1024, slots=8).to(dev)
yf = torch.empty(16, 512, dtype=torch.bfloat16, device=dev)
ws = torch.empty(lfm2sc_fused_prefill_workspace_bytes(torch.bfloat16, 512, 3, 4, True), dtype=torch.uint8, device=dev)
res.append(status(lambda: lfm2sc_fused_prefill(f.x, f.W_in, f.cu, f.w, yf, f.pool, f.slot_idx, workspace=ws)))
res.append(status(lambda: lfm2sc_fused_prefill(f.x, f.W_in, f.cu, f.w, yf, f.pool, dup, workspace=ws)))
badcu16 = torch.tensor([0, 3, 2, 10, 16], dtype=torch.int32, device=dev)
res.append(status(lambda: lfm2sc_fused_prefill(f.x, f.W_in, badcu16, f.w, yf, f.pool, f.slot_idx, workspace=ws)))
print("STATUS", res, flush=True)
"""


def test_check_mode_reports_bad_device_data():
    """With LFM2SC_CHECK=1 (read once per process, hence a child process) bad slot ids, row offsets and
    accept lengths are reported as LFM2SC_ERR_PRECONDITION (6) and nothing is launched for them: decode, ragged
    prefill, commit and the fused forward (valid inputs first, then duplicate slot ids, then bad row offsets)."""
    _say("case: LFM2SC_CHECK=1 in a child process")
    env = dict(os.environ, LFM2SC_CHECK="1")
    r = subprocess.run([sys.executable, "-c", _CHECK_SCRIPT, ROOT], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("STATUS")][0]
    assert line == "STATUS [0, 6, 6, 6, 6, 0, 6, 6]", line


# ------------------------------------------------------------------ conv bias and state gradients (ABI v2)

def _bias(H, dtype, seed):
    return (torch.randn(H, generator=torch.Generator().manual_seed(seed)) * 0.5).to(dtype)


@pytest.mark.parametrize("K,dtype", [(3, torch.bfloat16), (4, torch.float32), (1, torch.bfloat16)])
def test_bias_all_entry_points(K, dtype):
    _say(f"case: conv bias K={K} {dtype}")
    H = 520
    lens = [9, 1, 0, 40, 2]
    c = wl.random_case(90 + K, lens, H=H, K=K, dtype=dtype, slots=8, with_dy=True)
    b = _bias(H, dtype, 91)
    g = c.to(DEV)
    bd = b.to(DEV)
    pool0 = g.pool.clone()
    T, N = sum(lens), len(lens)
    y = _nan((T, H), dtype)
    lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, g.pool, g.slot_idx, bias=bd)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx, bias=b)
    assert_close(y, y_ref, dtype, "prefill y with bias")
    assert_bits(g.pool, rounded(p_ref, dtype), "prefill states with bias")
    # decode and verify on the original pool
    g.pool.copy_(pool0)
    yd = _nan((N, H), dtype)
    rows = torch.arange(N)
    lfm2sc_decode_step(g.inp[rows.to(DEV)].contiguous(), g.w, g.pool, g.slot_idx, yd, bias=bd)
    torch.cuda.synchronize()
    yd_ref, pd_ref = oracle.decode(c.inp[rows], c.w, c.pool, c.slot_idx, bias=b)
    assert_close(yd, yd_ref, dtype, "decode y with bias")
    assert_bits(g.pool, rounded(pd_ref, dtype), "decode states with bias")
    g.pool.copy_(pool0)
    L = 2
    vin = g.inp[:N * L].contiguous()
    yv = _nan((N * L, H), dtype)
    win = _nan((N, L, H, K), dtype)
    lfm2sc_verify_window(vin, g.w, g.pool, g.slot_idx, L, win, yv, bias=bd)
    torch.cuda.synchronize()
    yv_ref, tape_ref = oracle.verify(c.inp[:N * L], c.w, c.pool, c.slot_idx, L, bias=b)
    assert_close(yv, yv_ref, dtype, "verify y with bias")
    assert_bits(win, rounded(tape_ref, dtype), "verify tape with bias")
    # backward with bias: dC includes it, dbias = sum of g
    d_in = _nan((T, 3 * H), dtype)
    dW = _nan((H, K), torch.float32)
    db = _nan((H,), torch.float32)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(dtype, H, K, T, N), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, pool0, g.slot_idx, bias=bd, dbias=db)
    torch.cuda.synchronize()
    d_ref, dW_ref, db_ref, _ = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx, bias=b, full=True)
    assert_close(d_in, d_ref, dtype, "d_in with bias")
    assert_close(dW, dW_ref, dtype, "dW with bias")
    assert_close(db, db_ref, dtype, "dbias")


@pytest.mark.parametrize("K,dtype,lens", [
    (3, torch.bfloat16, [50, 1, 0, 2, 300, 3]),
    (4, torch.float32, [7, 0, 3, 129, 1]),
    (2, torch.bfloat16, [1, 64, 0]),
    (1, torch.float32, [5, 0, 2]),
])
def test_state_gradients(K, dtype, lens):
    _say(f"case: state gradients K={K} {dtype} lens={lens}")
    H = 264
    c = wl.random_case(95 + K, lens, H=H, K=K, dtype=dtype, slots=len(lens) + 3, with_dy=True)
    T, N = sum(lens), len(lens)
    dF = torch.randn(N, H, K, generator=torch.Generator().manual_seed(96)).to(dtype)
    g = c.to(DEV)
    d_in = _nan((T, 3 * H), dtype)
    dW = _nan((H, K), torch.float32)
    db = _nan((H,), torch.float32)
    dinit = _nan((N, H, K), dtype)
    ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(dtype, H, K, T, N)), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, g.pool, g.slot_idx, d_final_state=dF.to(DEV), dbias=db,
                    d_init_state=dinit)
    torch.cuda.synchronize()
    d_ref, dW_ref, db_ref, di_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx, d_final=dF, full=True)
    assert_close(d_in, d_ref, dtype, "d_in with d_final")
    assert_close(dW, dW_ref, dtype, "dW")
    assert_close(db, db_ref, dtype, "dbias")
    assert_close(dinit, di_ref, dtype, "d_init")
    # without d_final: the initial-state gradient comes from the conv terms alone
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, g.pool, g.slot_idx, d_init_state=dinit)
    torch.cuda.synchronize()
    d_ref, _, _, di_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx, full=True)
    assert_close(d_in, d_ref, dtype, "d_in without d_final")
    assert_close(dinit, di_ref, dtype, "d_init without d_final")


def test_chunked_training_on_gpu():
    """A long sequence trained in two chunks on the GPU (forward chunk 1, forward chunk 2 from its state,
    backward chunk 2, backward chunk 1 with chunk 2's d_init as d_final) against the oracle's backward of the
    whole sequence."""
    _say("case: chunked training on the GPU")
    H, K, T, cut = 1024, 3, 3000, 1234
    c = wl.random_case(97, [T], H=H, K=K, dtype=torch.bfloat16, slots=2, with_dy=True)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    cu1 = torch.tensor([0, cut], dtype=torch.int32, device=DEV)
    cu2 = torch.tensor([0, T - cut], dtype=torch.int32, device=DEV)
    in1, in2 = g.inp[:cut].contiguous(), g.inp[cut:].contiguous()
    y1 = _nan((cut, H), c.dtype)
    y2 = _nan((T - cut, H), c.dtype)
    lfm2sc_prefill_ragged(in1, cu1, g.w, y1, g.pool, g.slot_idx)
    pool_mid = g.pool.clone()
    lfm2sc_prefill_ragged(in2, cu2, g.w, y2, g.pool, g.slot_idx)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(c.dtype, H, K, T, 1), dtype=torch.uint8, device=DEV)
    d2 = _nan((T - cut, 3 * H), c.dtype)
    dW2 = _nan((H, K), torch.float32)
    dS_mid = _nan((1, H, K), c.dtype)
    lfm2sc_backward(in2, cu2, g.w, g.dy[cut:].contiguous(), d2, dW2, ws, pool_mid, g.slot_idx, d_init_state=dS_mid)
    d1 = _nan((cut, 3 * H), c.dtype)
    dW1 = _nan((H, K), torch.float32)
    dS0 = _nan((1, H, K), c.dtype)
    lfm2sc_backward(in1, cu1, g.w, g.dy[:cut].contiguous(), d1, dW1, ws, pool0, g.slot_idx, d_final_state=dS_mid,
                    d_init_state=dS0)
    torch.cuda.synchronize()
    d_ref, dW_ref, _, di_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx, full=True)
    assert_close(torch.cat([d1, d2]), d_ref, c.dtype, "chunked d_in")
    assert_close(dW1 + dW2, dW_ref, c.dtype, "chunked dW")
    assert_close(dS0, di_ref, c.dtype, "chunked d_init")


@pytest.mark.parametrize("H,K,dtype", [(1024, 2, torch.bfloat16), (1536, 4, torch.bfloat16), (1536, 3, torch.float32)])
def test_other_sizes_training_step(H, K, dtype):
    """Training step (prefill forward + backward) at other channel and tap counts, two sequences, full parity."""
    _say(f"case: training step H={H} K={K} {dtype}")
    c = wl.random_case(120 + K, [1700, 301], H=H, K=K, dtype=dtype, slots=3, with_dy=True)
    g = c.to(DEV)
    pool0 = g.pool.clone()
    T = 2001
    y = _nan((T, H), dtype)
    lfm2sc_prefill_ragged(g.inp, g.cu, g.w, y, g.pool, g.slot_idx)
    d_in = _nan((T, 3 * H), dtype)
    dW = _nan((H, K), torch.float32)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(dtype, H, K, T, 2), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, pool0, g.slot_idx)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.prefill(c.inp, c.cu, c.w, c.pool, c.slot_idx)
    d_ref, dW_ref = oracle.backward(c.inp, c.cu, c.w, c.dy, c.pool, c.slot_idx)
    assert_close(y, y_ref, dtype, "y")
    assert_bits(g.pool, rounded(p_ref, dtype), "states")
    assert_close(d_in, d_ref, dtype, "d_in")
    assert_close(dW, dW_ref, dtype, "dW")
