"""Seeded synthetic workloads for the LFM2 ShortConv hot path.

This module only draws random inputs; it holds none of the op's arithmetic.
It is shared by the tests, the benchmark and the smoke check, and is the one
piece of code that both the HIP path and the CPU oracle consume (the oracle
reads the very tensors drawn here, widened exactly to float64).

Recipe for every workload: a CPU ``torch.Generator`` seeded with the workload's
seed; every floating tensor is drawn in float32 (``randn`` for N(0,1),
``rand`` rescaled for U(-0.5, 0.5)) and then cast to the I/O dtype, and the cast
values are the inputs of both sides.  Integer draws (lengths, slot choices,
accept lengths) come from the same generator.  Shapes follow the LFM2-1.2B
layer shape from the "LFM2-1.2B" inference-research record (conv_dim 2048,
conv_L_cache 3): H = 2048, K = 3, in_proj rows of width 3H.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

H_LFM2 = 2048   # conv_dim of LFM2-1.2B
K_LFM2 = 3      # conv_L_cache of LFM2-1.2B


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    H: int
    K: int
    inp: torch.Tensor                  # [rows, 3H]  B | C | xv
    w: torch.Tensor                    # [H, K]
    cu: Optional[torch.Tensor] = None  # int32 [N+1] row offsets (prefill / backward)
    pool: Optional[torch.Tensor] = None        # [slots, H, K]
    slot_idx: Optional[torch.Tensor] = None    # int32 [N]
    dy: Optional[torch.Tensor] = None          # [rows, H]
    accept: Optional[torch.Tensor] = None      # int32 [N] accept lengths (verify)
    L: int = 0                                 # verify block
    extra: Dict[str, object] = field(default_factory=dict)

    def to(self, device):
        out = Workload(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("inp", "w", "cu", "pool", "slot_idx", "dy", "accept"):
            v = getattr(out, k)
            if v is not None:
                setattr(out, k, v.to(device))
        return out


def _normal(g, shape, dtype):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def _uniform_half(g, shape, dtype):
    return (torch.rand(shape, generator=g, dtype=torch.float32) - 0.5).to(dtype)


def tiny_fp32(seed: int = 1, T: int = 64, H: int = 256, K: int = 3) -> Workload:
    """1 sequence, T=64, H=256, K=3, fp32, zero initial state, with dy."""
    g = torch.Generator().manual_seed(seed)
    inp = _normal(g, (T, 3 * H), torch.float32)
    w = _uniform_half(g, (H, K), torch.float32)
    dy = _normal(g, (T, H), torch.float32)
    cu = torch.tensor([0, T], dtype=torch.int32)
    return Workload("tiny_fp32", torch.float32, H, K, inp, w, cu=cu, dy=dy)


def decode_lfm2(seed: int = 2, N: int = 256, slots: int = 1024, H: int = H_LFM2, K: int = K_LFM2,
                dtype=torch.bfloat16) -> Workload:
    """N sequences x 1 token; pool [slots, H, K] ~N(0,1); N distinct slots drawn without replacement."""
    g = torch.Generator().manual_seed(seed)
    inp = _normal(g, (N, 3 * H), dtype)
    pool = _normal(g, (slots, H, K), dtype)
    slot_idx = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    w = _uniform_half(g, (H, K), dtype)
    return Workload("decode", dtype, H, K, inp, w, pool=pool, slot_idx=slot_idx)


def ragged_prefill_lfm2(seed: int = 3, N: int = 8, lo: int = 64, hi: int = 2048, H: int = H_LFM2,
                        K: int = K_LFM2, dtype=torch.bfloat16, slots: Optional[int] = None) -> Workload:
    """N sequences, lengths uniform on the integers [lo, hi], packed; random states in N pool slots."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(lo, hi + 1, (N,), generator=g)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    inp = _normal(g, (total, 3 * H), dtype)
    nslots = N if slots is None else slots
    pool = _normal(g, (nslots, H, K), dtype)
    slot_idx = torch.randperm(nslots, generator=g)[:N].to(torch.int32)
    w = _uniform_half(g, (H, K), dtype)
    return Workload("ragged_prefill", dtype, H, K, inp, w, cu=cu, pool=pool, slot_idx=slot_idx,
                    extra={"lens": lens.tolist()})


def verify_lfm2(seed: int = 4, N: int = 64, L: int = 8, slots: int = 256, H: int = H_LFM2,
                K: int = K_LFM2, dtype=torch.bfloat16) -> Workload:
    """N sequences x L draft tokens (row i*L+s); pool [slots, H, K]; accept lengths in [0, L]."""
    g = torch.Generator().manual_seed(seed)
    inp = _normal(g, (N * L, 3 * H), dtype)
    pool = _normal(g, (slots, H, K), dtype)
    slot_idx = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    accept = torch.randint(0, L + 1, (N,), generator=g).to(torch.int32)
    w = _uniform_half(g, (H, K), dtype)
    return Workload("verify", dtype, H, K, inp, w, pool=pool, slot_idx=slot_idx, accept=accept, L=L)


def train_lfm2(seed: int = 5, T: int = 65536, H: int = H_LFM2, K: int = K_LFM2,
               dtype=torch.bfloat16) -> Workload:
    """Single sequence of T tokens, zero initial state; inputs and dy ~N(0,1), weight ~U(-0.5,0.5)."""
    g = torch.Generator().manual_seed(seed)
    inp = _normal(g, (T, 3 * H), dtype)
    w = _uniform_half(g, (H, K), dtype)
    dy = _normal(g, (T, H), dtype)
    cu = torch.tensor([0, T], dtype=torch.int32)
    return Workload(f"train_T{T}", dtype, H, K, inp, w, cu=cu, dy=dy)


def random_case(seed: int, lens, H: int, K: int, dtype, slots: int = 0, with_dy: bool = False,
                in_pad: int = 0) -> Workload:
    """Small ragged case for edge-case tests: given sequence lengths (zeros allowed), optional pool
    with `slots` slots (0 = no pool), optional extra in_proj columns (stride padding)."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(list(lens), dtype=torch.int64)
    N = lens.numel()
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    inp = _normal(g, (total, 3 * H + in_pad), dtype)
    w = _uniform_half(g, (H, K), dtype)
    pool = slot_idx = None
    if slots:
        pool = _normal(g, (slots, H, K), dtype)
        slot_idx = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    dy = _normal(g, (total, H), dtype) if with_dy else None
    return Workload("random_case", dtype, H, K, inp, w, cu=cu, pool=pool, slot_idx=slot_idx, dy=dy)


@dataclass
class FusedWorkload:
    """Inputs of the fused in_proj + ShortConv forward: hidden states x [rows, >=D], in_proj weight W_in [3H, D]
    (rows 0..H-1 give B, H..2H-1 C, 2H..3H-1 xv), conv weight w [H, K], optional bias, ragged offsets and slots."""
    name: str
    H: int
    K: int
    D: int
    x: torch.Tensor
    W_in: torch.Tensor
    w: torch.Tensor
    cu: torch.Tensor
    bias: Optional[torch.Tensor] = None
    pool: Optional[torch.Tensor] = None
    slot_idx: Optional[torch.Tensor] = None

    def to(self, device):
        out = FusedWorkload(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("x", "W_in", "w", "cu", "bias", "pool", "slot_idx"):
            v = getattr(out, k)
            if v is not None:
                setattr(out, k, v.to(device))
        return out


def fused_case(seed: int, lens, H: int, K: int, D: int, slots: int = 0, bias: bool = False, x_pad: int = 0,
               tail_rows: int = 0) -> FusedWorkload:
    """bf16 hidden states x ~ N(0,1) and W_in ~ N(0, 1/D) (so in_proj entries are about N(0,1), like the
    other workloads' in_proj rows), w ~ U(-0.5,0.5), optional bias ~ N(0,1) and pool ~ N(0,1).  `tail_rows`
    extra rows after the last sequence belong to no sequence; `x_pad` extra columns pad the x rows."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(list(lens), dtype=torch.int64)
    N = lens.numel()
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    rows = int(cu[-1]) + tail_rows
    dt = torch.bfloat16
    x = _normal(g, (rows, D + x_pad), dt)
    W_in = (torch.randn((3 * H, D), generator=g, dtype=torch.float32) * D ** -0.5).to(dt)
    w = _uniform_half(g, (H, K), dt)
    b = _normal(g, (H,), dt) if bias else None
    pool = slot_idx = None
    if slots:
        pool = _normal(g, (slots, H, K), dt)
        slot_idx = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    return FusedWorkload("fused_case", H, K, D, x, W_in, w, cu, bias=b, pool=pool, slot_idx=slot_idx)


def fused_train_lfm2(seed: int = 6, T: int = 65536, H: int = H_LFM2, K: int = K_LFM2, D: int = H_LFM2) -> FusedWorkload:
    """Training forward of one ShortConv layer through the fused path: one sequence of T tokens, hidden size
    D = 2048 (LFM2-1.2B: hidden size = conv_dim), zero initial state."""
    return fused_case(seed, [T], H, K, D)


def fused_one_token_lfm2(seed: int = 8, N: int = 256, H: int = H_LFM2, K: int = K_LFM2,
                         D: int = H_LFM2) -> FusedWorkload:
    """N one-token sequences, each with its own slot (a decode-shaped batch through the fused prefill: every
    conv history comes from the pool)."""
    return fused_case(seed, [1] * N, H, K, D, slots=N + 16)


def fused_ragged_lfm2(seed: int = 7, N: int = 8, lo: int = 64, hi: int = 2048, H: int = H_LFM2, K: int = K_LFM2,
                      D: int = H_LFM2) -> FusedWorkload:
    """Ragged prefill through the fused path: N sequences with lengths uniform on [lo, hi], one pool slot each."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(lo, hi + 1, (N,), generator=g).tolist()
    return fused_case(seed + 1000, lens, H, K, D, slots=N)


def _normal_on(g, shape, dtype, device):
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dtype)


def large_train_on(device, seed: int, lens, H: int = H_LFM2, K: int = K_LFM2, slots: int = 0,
                   dtype=torch.bfloat16) -> Workload:
    """Maximum-size cases drawn directly on `device` (a generator of that device, same recipe: N(0,1) inputs,
    dy and pool, U(-0.5,0.5) weight), so that multi-GB inputs need no host copy."""
    g = torch.Generator(device=device).manual_seed(seed)
    lens = torch.as_tensor(list(lens), dtype=torch.int64)
    N = lens.numel()
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    inp = _normal_on(g, (total, 3 * H), dtype, device)
    w = (torch.rand((H, K), generator=g, dtype=torch.float32, device=device) - 0.5).to(dtype)
    dy = _normal_on(g, (total, H), dtype, device)
    pool = slot_idx = None
    if slots:
        pool = _normal_on(g, (slots, H, K), dtype, device)
        slot_idx = torch.randperm(slots, generator=g, device=device)[:N].to(torch.int32)
    return Workload("large_train", dtype, H, K, inp, w, cu=cu.to(device), pool=pool, slot_idx=slot_idx, dy=dy)


def large_fused_on(device, seed: int, lens, H: int = H_LFM2, K: int = K_LFM2, D: int = H_LFM2,
                   slots: int = 0) -> FusedWorkload:
    """Maximum-size fused-forward case drawn on `device`: x ~ N(0,1), W_in ~ N(0, 1/D), w ~ U(-0.5,0.5)."""
    g = torch.Generator(device=device).manual_seed(seed)
    lens = torch.as_tensor(list(lens), dtype=torch.int64)
    N = lens.numel()
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    dt = torch.bfloat16
    x = _normal_on(g, (total, D), dt, device)
    W_in = (torch.randn((3 * H, D), generator=g, dtype=torch.float32, device=device) * D ** -0.5).to(dt)
    w = (torch.rand((H, K), generator=g, dtype=torch.float32, device=device) - 0.5).to(dt)
    pool = slot_idx = None
    if slots:
        pool = _normal_on(g, (slots, H, K), dt, device)
        slot_idx = torch.randperm(slots, generator=g, device=device)[:N].to(torch.int32)
    return FusedWorkload("large_fused", H, K, D, x, W_in, w, cu.to(device), pool=pool, slot_idx=slot_idx)


def _small_int(g, shape, dtype, levels):
    """Integers drawn uniformly from {-levels, ..., -1, 1, ..., levels} (no zero), as `dtype`."""
    mag = torch.randint(1, levels + 1, shape, generator=g)
    sign = torch.randint(0, 2, shape, generator=g) * 2 - 1
    return (mag * sign).to(torch.float32).to(dtype)


def integer_case(seed: int, lens, H: int = H_LFM2, K: int = K_LFM2, dtype=torch.bfloat16, slots: int = 0,
                 levels: int = 3, bias: bool = False, d_final: bool = False) -> Workload:
    """Inputs, dy, weight, optional bias, pool and final-state gradient drawn as small nonzero integers
    ({-3..-1, 1..3} by default).  Such values are exact in bf16, and with |values| <= 3 every product and every
    sum the op forms stays an integer below 2^8 per output element (below 2^24 for dW over 65,536 tokens), so
    the exact result is representable and any correct implementation must reproduce it bit for bit.  A dropped
    or doubled token changes dW by a nonzero integer.  `extra` holds "bias" and "d_final" when asked for."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(list(lens), dtype=torch.int64)
    N = lens.numel()
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    inp = _small_int(g, (total, 3 * H), dtype, levels)
    w = _small_int(g, (H, K), dtype, levels)
    dy = _small_int(g, (total, H), dtype, levels)
    pool = slot_idx = None
    if slots:
        pool = _small_int(g, (slots, H, K), dtype, levels)
        slot_idx = torch.randperm(slots, generator=g)[:N].to(torch.int32)
    extra = {"lens": lens.tolist()}
    if bias:
        extra["bias"] = _small_int(g, (H,), dtype, levels)
    if d_final:
        extra["d_final"] = _small_int(g, (N, H, K), dtype, levels)
    return Workload("integer_case", dtype, H, K, inp, w, cu=cu, pool=pool, slot_idx=slot_idx, dy=dy, extra=extra)
