"""Host checks of the Python binding (no GPU): a call whose tensors do not cover what the kernels touch, sit on
another device, or carry another dtype is rejected before the library is called; a well-formed call reaches the
library with the sizes and strides of its tensors.

The library is replaced by a recorder, and the GPU-residency test by one that accepts CPU tensors, so that the
extent and dtype checks can run here on CPU tensors.
"""
import pytest
import torch

from gated_short_causal_amd import binding

H, K = 64, 3
BF = torch.bfloat16


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append((name, args))
            return 0
        return fn


@pytest.fixture
def lib(monkeypatch):
    rec = _Recorder()
    monkeypatch.setattr(binding._lib, "lib", lambda: rec)
    monkeypatch.setattr(binding, "_is_gpu", lambda t: True)
    monkeypatch.setattr(binding, "_stream", lambda device: 0)
    return rec


def _w(dtype=BF):
    return torch.zeros(H, K, dtype=dtype)


def _cu(*v):
    return torch.tensor(v, dtype=torch.int32)


def test_prefill_accepts_and_marshals(lib):
    inp = torch.zeros(10, 3 * H + 8, dtype=BF)
    y = torch.zeros(10, H, dtype=BF)
    pool = torch.zeros(4, H, K, dtype=BF)
    binding.lfm2sc_prefill_ragged(inp, _cu(0, 4, 10), _w(), y, pool, torch.tensor([1, 3], dtype=torch.int32))
    (name, args), = lib.calls
    assert name == "lfm2sc_prefill_ragged"
    assert args[1:3] == (H, K) and args[4] == 3 * H + 8 and args[5] == 10 and args[7] == 2
    assert args[11] == 4 and args[12] == H * K and args[15] == H


@pytest.mark.parametrize("bad", ["y_rows", "y_cols", "in_cols", "dtype", "cu_dtype", "slots", "no_slots", "bias"])
def test_prefill_rejections(lib, bad):
    inp = torch.zeros(10, 3 * H, dtype=BF)
    y = torch.zeros(10, H, dtype=BF)
    cu = _cu(0, 4, 10)
    pool = torch.zeros(4, H, K, dtype=BF)
    slots = torch.tensor([1, 3], dtype=torch.int32)
    bias = None
    if bad == "y_rows":
        y = torch.zeros(9, H, dtype=BF)
    elif bad == "y_cols":
        y = torch.zeros(10, H - 8, dtype=BF)
    elif bad == "in_cols":
        inp = torch.zeros(10, 3 * H - 8, dtype=BF)
    elif bad == "dtype":
        y = torch.zeros(10, H, dtype=torch.float32)
    elif bad == "cu_dtype":
        cu = cu.long()
    elif bad == "slots":
        slots = slots[:1]
    elif bad == "no_slots":
        slots = None
    elif bad == "bias":
        bias = torch.zeros(H - 8, dtype=BF)
    with pytest.raises((ValueError, TypeError)):
        binding.lfm2sc_prefill_ragged(inp, cu, _w(), y, pool, slots, bias=bias)
    assert lib.calls == []


def test_rejects_tensor_on_another_device(monkeypatch, lib):
    # residency is judged per tensor: a host tensor among device tensors is refused before any call
    monkeypatch.setattr(binding, "_is_gpu", lambda t: t.dtype != torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens must be on"):
        binding.lfm2sc_prefill_ragged(torch.zeros(4, 3 * H, dtype=BF), _cu(0, 4), _w(), torch.zeros(4, H, dtype=BF))
    assert lib.calls == []


def test_decode_verify_commit_extents(lib):
    pool = torch.zeros(8, H, K, dtype=BF)
    slots = torch.tensor([0, 5, 7], dtype=torch.int32)
    with pytest.raises(ValueError):   # 3 sequences need 3 in_proj rows
        binding.lfm2sc_decode_step(torch.zeros(2, 3 * H, dtype=BF), _w(), pool, slots, torch.zeros(3, H, dtype=BF))
    with pytest.raises(ValueError):   # and 3 y rows
        binding.lfm2sc_decode_step(torch.zeros(3, 3 * H, dtype=BF), _w(), pool, slots, torch.zeros(2, H, dtype=BF))
    binding.lfm2sc_decode_step(torch.zeros(3, 3 * H, dtype=BF), _w(), pool, slots, torch.zeros(3, H, dtype=BF))
    L = 4
    win = torch.zeros(3, L, H, K, dtype=BF)
    with pytest.raises(ValueError):   # 3 x 4 draft tokens need 12 rows
        binding.lfm2sc_verify_window(torch.zeros(11, 3 * H, dtype=BF), _w(), pool, slots, L, win,
                                     torch.zeros(12, H, dtype=BF))
    with pytest.raises(ValueError):   # tape too small
        binding.lfm2sc_verify_window(torch.zeros(12, 3 * H, dtype=BF), _w(), pool, slots, L, win[:2],
                                     torch.zeros(12, H, dtype=BF))
    binding.lfm2sc_verify_window(torch.zeros(12, 3 * H, dtype=BF), _w(), pool, slots, L, win,
                                 torch.zeros(12, H, dtype=BF))
    with pytest.raises(ValueError):   # one accept length per sequence
        binding.lfm2sc_commit_window(win, torch.zeros(2, dtype=torch.int32), pool, slots)
    with pytest.raises(TypeError):    # pool of another dtype
        binding.lfm2sc_commit_window(win, torch.zeros(3, dtype=torch.int32), pool.float(), slots)
    binding.lfm2sc_commit_window(win, torch.zeros(3, dtype=torch.int32), pool, slots)
    assert [n for n, _ in lib.calls] == ["lfm2sc_decode_step", "lfm2sc_verify_window", "lfm2sc_commit_window"]


def _bwd_args(T=10, N=2):
    return dict(in_proj=torch.zeros(T, 3 * H, dtype=BF), cu_seqlens=_cu(0, 3, T) if N == 2 else _cu(0, T),
                weight=_w(), dy=torch.zeros(T, H, dtype=BF), d_in_proj=torch.zeros(T, 3 * H, dtype=BF),
                dW=torch.zeros(H, K), workspace=torch.zeros(256, dtype=torch.uint8))


@pytest.mark.parametrize("bad", ["dy_rows", "din_rows", "din_cols", "dW_dtype", "dW_size", "dfinal", "dinit",
                                 "dbias", "dy_dtype"])
def test_backward_rejections(lib, bad):
    a = _bwd_args()
    extra = {}
    if bad == "dy_rows":
        a["dy"] = torch.zeros(9, H, dtype=BF)
    elif bad == "din_rows":
        a["d_in_proj"] = torch.zeros(9, 3 * H, dtype=BF)
    elif bad == "din_cols":
        a["d_in_proj"] = torch.zeros(10, 3 * H - 8, dtype=BF)
    elif bad == "dW_dtype":
        a["dW"] = torch.zeros(H, K, dtype=BF)
    elif bad == "dW_size":
        a["dW"] = torch.zeros(H - 1, K)
    elif bad == "dfinal":
        extra["d_final_state"] = torch.zeros(1, H, K, dtype=BF)
    elif bad == "dinit":
        extra["d_init_state"] = torch.zeros(2, H, K - 1, dtype=BF)
    elif bad == "dbias":
        extra["dbias"] = torch.zeros(H - 8)
    elif bad == "dy_dtype":
        a["dy"] = torch.zeros(10, H)
    with pytest.raises((ValueError, TypeError)):
        binding.lfm2sc_backward(**a, **extra)
    assert lib.calls == []


def test_backward_accepts(lib):
    a = _bwd_args()
    binding.lfm2sc_backward(**a, d_final_state=torch.zeros(2, H, K, dtype=BF), dbias=torch.zeros(H),
                            d_init_state=torch.zeros(2, H, K, dtype=BF))
    (name, args), = lib.calls
    assert name == "lfm2sc_backward" and args[5] == 10 and args[7] == 2 and args[-2] == 256


def test_fused_and_conv_update_extents(lib):
    x = torch.zeros(10, 128, dtype=BF)
    W_in = torch.zeros(3 * H, 128, dtype=BF)
    with pytest.raises(ValueError):   # y rows < x rows
        binding.lfm2sc_fused_prefill(x, W_in, _cu(0, 10), _w(), torch.zeros(9, H, dtype=BF))
    with pytest.raises(ValueError):   # in_proj output too narrow
        binding.lfm2sc_fused_prefill(x, W_in, _cu(0, 10), _w(), torch.zeros(10, H, dtype=BF),
                                     in_proj_out=torch.zeros(10, 2 * H, dtype=BF))
    binding.lfm2sc_fused_prefill(x, W_in, _cu(0, 10), _w(), torch.zeros(10, H, dtype=BF))
    pool = torch.zeros(4, H, K, dtype=BF)
    slots = torch.tensor([2, 3], dtype=torch.int32)
    bx = torch.zeros(2, 5, H, dtype=BF).transpose(1, 2)
    out = torch.zeros(2, H, 5, dtype=BF)
    with pytest.raises(ValueError):   # tape too small
        binding.lfm2sc_conv_update(bx, _w(), pool, slots, out, windows=torch.zeros(2, 4, H, K, dtype=BF))
    with pytest.raises(ValueError):   # one slot for two sequences
        binding.lfm2sc_conv_update(bx, _w(), pool, slots[:1], out)
    binding.lfm2sc_conv_update(bx, _w(), pool, slots, out)
    assert [n for n, _ in lib.calls] == ["lfm2sc_fused_prefill", "lfm2sc_conv_update"]
