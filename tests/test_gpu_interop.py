"""GPU parity of lfm2sc_conv_update (gated inputs in [batch][channel][token] order, any strides) against the fp64
oracle (oracle.conv_update).  Tape entries and slot states are copies of inputs and so are compared bit for bit;
the conv outputs within the dtype's tolerance."""
import pytest
import torch

import oracle
from gated_short_causal_amd import lfm2sc_conv_update
from tests.parity_util import assert_bits, assert_close, rounded

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _inputs(seed, N, H, K, L, slots, dtype):
    g = torch.Generator().manual_seed(seed)
    rows = torch.randn(N * L, H, generator=g).to(dtype)                 # token-major gated rows
    w = (torch.rand(H, K, generator=g) - 0.5).to(dtype)
    b = torch.randn(H, generator=g).to(dtype)
    pool = torch.randn(slots, H, K, generator=g).to(dtype)
    sl = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    return rows, w, b, pool, sl


def _layout(rows, N, L, H, kind):
    """bx as [N, H, L] in the requested memory layout, plus an output tensor of the same layout."""
    if kind == "sglang_view":                      # transposed view of token-major rows: strides (L*H, 1, H)
        bx = rows.to(DEV).view(N, L, H).transpose(1, 2)
        out = torch.full((N, L, H), float("nan"), dtype=rows.dtype, device=DEV).transpose(1, 2)
    elif kind == "dense_nhl":                      # contiguous [N][H][L]: strides (H*L, L, 1)
        bx = rows.view(N, L, H).transpose(1, 2).contiguous().to(DEV)
        out = torch.full((N, H, L), float("nan"), dtype=rows.dtype, device=DEV)
    else:                                          # padded channel stride: strides (H*L*2, 2, H*2)
        big = torch.zeros(N, L, H, 2, dtype=rows.dtype)
        big[..., 0] = rows.view(N, L, H)
        bx = big.to(DEV).permute(0, 2, 1, 3)[..., 0]
        out = torch.full((N, L, H, 2), float("nan"), dtype=rows.dtype, device=DEV).permute(0, 2, 1, 3)[..., 1]
    return bx, out


@pytest.mark.parametrize("kind", ["sglang_view", "dense_nhl", "padded"])
@pytest.mark.parametrize("K,L,dtype,H", [(3, 8, torch.bfloat16, 2048), (4, 13, torch.float32, 520),
                                         (1, 1, torch.bfloat16, 64), (2, 5, torch.bfloat16, 1032)])
def test_conv_update_with_tape(kind, K, L, dtype, H):
    N = 6
    _say(f"case: conv_update tape {kind} K={K} L={L} {dtype} H={H}")
    rows, w, b, pool, sl = _inputs(800 + K + L, N, H, K, L, N + 3, dtype)
    bx, out = _layout(rows, N, L, H, kind)
    gpool = pool.to(DEV)
    win = torch.full((N, L, H, K), float("nan"), dtype=dtype, device=DEV)
    lfm2sc_conv_update(bx, w.to(DEV), gpool, sl.to(DEV), out, windows=win, bias=b.to(DEV))
    torch.cuda.synchronize()
    out_ref, tape_ref, _ = oracle.conv_update(rows.view(N, L, H).transpose(1, 2), w, pool, sl, bias=b)
    assert_close(out, out_ref, dtype, "out")
    assert_bits(win, rounded(tape_ref, dtype), "tape")
    assert_bits(gpool, pool, "pool untouched with a tape")


@pytest.mark.parametrize("kind", ["sglang_view", "dense_nhl"])
def test_conv_update_bench_shape(kind):
    """The shape bench.py times (64 sequences x 8 tokens, H = 2048, K = 3, bf16, a tape, no bias, 64 of 256
    slots), in both of its layouts: every output against the oracle, the tape bit for bit."""
    N, L, H, K, dtype = 64, 8, 2048, 3, torch.bfloat16
    _say(f"case: conv_update bench shape {kind} N={N} L={L} H={H} K={K}")
    rows, w, _, pool, sl = _inputs(870, N, H, K, L, 256, dtype)
    bx, out = _layout(rows, N, L, H, kind)
    gpool = pool.to(DEV)
    win = torch.full((N, L, H, K), float("nan"), dtype=dtype, device=DEV)
    lfm2sc_conv_update(bx, w.to(DEV), gpool, sl.to(DEV), out, windows=win)
    torch.cuda.synchronize()
    out_ref, tape_ref, _ = oracle.conv_update(rows.view(N, L, H).transpose(1, 2), w, pool, sl)
    assert_close(out, out_ref, dtype, "out")
    assert_bits(win, rounded(tape_ref, dtype), "tape")
    assert_bits(gpool, pool, "pool untouched with a tape")


@pytest.mark.parametrize("kind", ["sglang_view", "dense_nhl"])
@pytest.mark.parametrize("K,L,dtype", [(3, 1, torch.bfloat16), (3, 9, torch.bfloat16), (4, 3, torch.float32)])
def test_conv_update_in_place(kind, K, L, dtype):
    N, H = 5, 1024
    _say(f"case: conv_update in place {kind} K={K} L={L} {dtype}")
    rows, w, b, pool, sl = _inputs(900 + K + L, N, H, K, L, N + 4, dtype)
    bx, out = _layout(rows, N, L, H, kind)
    gpool = pool.to(DEV)
    lfm2sc_conv_update(bx, w.to(DEV), gpool, sl.to(DEV), out, bias=b.to(DEV))
    torch.cuda.synchronize()
    out_ref, _, pool_ref = oracle.conv_update(rows.view(N, L, H).transpose(1, 2), w, pool, sl, bias=b,
                                              with_tape=False)
    assert_close(out, out_ref, dtype, "out")
    assert_bits(gpool, rounded(pool_ref, dtype), "advanced slots (others untouched)")


def test_conv_update_out_of_range_slots():
    N, H, K, L = 3, 512, 3, 4
    _say("case: conv_update out-of-range slots")
    rows, w, b, pool, sl = _inputs(950, N, H, K, L, 5, torch.bfloat16)
    sl = torch.tensor([2, 5, -1], dtype=torch.int32)
    bx, out = _layout(rows, N, L, H, "sglang_view")
    gpool = pool.to(DEV)
    lfm2sc_conv_update(bx, w.to(DEV), gpool, sl.to(DEV), out)
    torch.cuda.synchronize()
    zero = torch.zeros(2, H, K, dtype=torch.bfloat16)
    x = rows.view(N, L, H).transpose(1, 2)
    ref0, _, p0 = oracle.conv_update(x[:1], w, pool, sl[:1], with_tape=False)
    ref12, _, _ = oracle.conv_update(x[1:], w, zero, torch.tensor([0, 1]), with_tape=False)
    assert_close(out[:1], ref0, torch.bfloat16, "valid slot")
    assert_close(out[1:], ref12, torch.bfloat16, "out-of-range slots use a zero state")
    assert_bits(gpool, rounded(p0, torch.bfloat16), "only slot 2 advanced")
