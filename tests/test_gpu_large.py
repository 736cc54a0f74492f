"""Maximum-size cases: byte offsets beyond 4 GiB in the streamed rows, element offsets beyond 2^31 in the state
pool, and a fused forward over ~300k tokens.  Inputs are drawn on the device (workloads.large_*_on); the oracle
checks sampled channels (channels are independent once in_proj is formed), and the states of every sequence."""
import pytest
import torch

import oracle
from gated_short_causal_amd import (lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_decode_step,
                                    lfm2sc_fused_prefill, lfm2sc_fused_prefill_workspace_bytes,
                                    lfm2sc_prefill_ragged)
from gated_short_causal_amd import workloads as wl
from tests.parity_util import assert_bits, assert_close, rounded

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16
CH = torch.tensor([0, 1, 7, 8, 511, 512, 1000, 1535, 1536, 2040, 2047])


def _say(msg):
    print(msg, flush=True)


def _cols(H):
    return torch.cat([CH, CH + H, CH + 2 * H])


def test_training_step_beyond_4gib_rows():
    """~1.05M tokens in two sequences: in_proj and d_in are 12.9 GB each, so row byte offsets pass 2^32."""
    lens = [(1 << 20) + 37, 1000]
    _say(f"case: training step lens={lens} H=2048 (multi-GB rows)")
    c = wl.large_train_on(DEV, 700, lens, slots=4)
    H, K = c.H, c.K
    T, N = sum(lens), len(lens)
    pool0 = c.pool.clone()
    y = torch.empty(T, H, dtype=BF, device=DEV)
    lfm2sc_prefill_ragged(c.inp, c.cu, c.w, y, c.pool, c.slot_idx)
    d_in = torch.empty(T, 3 * H, dtype=BF, device=DEV)
    dW = torch.empty(H, K, dtype=torch.float32, device=DEV)
    ws = torch.empty(lfm2sc_backward_workspace_bytes(BF, H, K, T, N), dtype=torch.uint8, device=DEV)
    lfm2sc_backward(c.inp, c.cu, c.w, c.dy, d_in, dW, ws, pool0, c.slot_idx)
    torch.cuda.synchronize()
    cols = _cols(H).to(DEV)
    inp_s = c.inp[:, cols].cpu()
    dy_s = c.dy[:, CH.to(DEV)].cpu()
    w_s, p_s = c.w[CH.to(DEV)].cpu(), pool0[:, CH.to(DEV), :].cpu()
    cu, sl = c.cu.cpu(), c.slot_idx.cpu()
    y_ref, pool_ref = oracle.prefill(inp_s, cu, w_s, p_s, sl)
    d_ref, dW_ref = oracle.backward(inp_s, cu, w_s, dy_s, p_s, sl)
    assert_close(y[:, CH.to(DEV)].cpu(), y_ref, BF, "y (sampled)")
    assert_bits(c.pool[:, CH.to(DEV), :].cpu(), rounded(pool_ref, BF), "final states (sampled)")
    assert_close(d_in[:, cols].cpu(), d_ref, BF, "d_in (sampled)")
    assert_close(dW[CH.to(DEV)].cpu(), dW_ref, BF, "dW (sampled)")


def test_decode_pool_beyond_2g_elements():
    """A 400k-slot pool: slot * slot_stride passes 2^31 elements for the upper slots."""
    slots, N, H, K = 400_000, 256, 2048, 3
    _say(f"case: decode N={N} pool of {slots} slots")
    g = torch.Generator(device=DEV).manual_seed(710)
    pool = torch.randn(slots, H, K, generator=g, device=DEV).to(BF)
    inp = torch.randn(N, 3 * H, generator=g, device=DEV).to(BF)
    w = (torch.rand(H, K, generator=g, device=DEV) - 0.5).to(BF)
    sl = torch.cat([torch.arange(slots - 128, slots, device=DEV),
                    torch.randperm(slots - 128, generator=g, device=DEV)[:128]]).to(torch.int32)
    before = pool[sl.long()].cpu()
    y = torch.empty(N, H, dtype=BF, device=DEV)
    lfm2sc_decode_step(inp, w, pool, sl, y)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.decode(inp.cpu(), w.cpu(), before, torch.arange(N, dtype=torch.int32))
    assert_close(y.cpu(), y_ref, BF, "y")
    assert_bits(pool[sl.long()].cpu(), rounded(p_ref, BF), "states of the named slots")


@pytest.mark.parametrize("form", ["overlap", "halo", "split32", "split64", "mid"])
def test_fused_forward_300k_tokens(form, monkeypatch):
    """Every tile form (wide tiles overlapping or with halo rows, split tiles of 32 or 64 channels, mid tiles)
    at ~300k tokens: tile and row offsets in 64 bits."""
    split = {"split32": "32", "split64": "64", "mid": "128"}.get(form, "0")
    monkeypatch.setenv("LFM2SC_FUSED_SPLIT", split)
    monkeypatch.setenv("LFM2SC_FUSED_HALO", "1" if form == "halo" else "0")
    lens = [300_000, 4097, 1]
    _say(f"case: fused forward lens={lens} D=H=2048 form={form}, sampled channels")
    c = wl.large_fused_on(DEV, 720, lens, slots=5)
    H, T = c.H, sum(lens)
    y = torch.empty(T, H, dtype=BF, device=DEV)
    ws = torch.empty(lfm2sc_fused_prefill_workspace_bytes(BF, H, c.K, len(lens), True), dtype=torch.uint8,
                     device=DEV)
    pool0 = c.pool.clone()
    lfm2sc_fused_prefill(c.x, c.W_in, c.cu, c.w, y, c.pool, c.slot_idx, workspace=ws)
    torch.cuda.synchronize()
    ch = CH[[0, 3, 5, 9, 10]]
    rows = torch.cat([ch, ch + H, ch + 2 * H]).to(DEV)
    y_ref, p_ref, _ = oracle.fused_prefill(c.x.cpu(), c.W_in[rows].cpu(), c.cu.cpu(), c.w[ch.to(DEV)].cpu(),
                                           pool0[:, ch.to(DEV), :].cpu(), c.slot_idx.cpu())
    assert_close(y[:, ch.to(DEV)].cpu(), y_ref, BF, "y (sampled)")
    assert_close(c.pool[:, ch.to(DEV), :].cpu(), p_ref, BF, "final states (sampled)")
