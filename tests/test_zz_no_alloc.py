"""lfm2sc_backward_noalloc (the backward whose partial sums live in the library's fixed device array) against
lfm2sc_backward with a caller workspace: bit-identical d_in, dW, dbias and initial-state gradients, on calls in
a row whose sizes shrink (so the second call runs over what the first one left in the array), and against the
fp64 oracle within the stated tolerances."""
import pytest
import torch

import oracle
from gated_short_causal_amd import workloads as wl
from gated_short_causal_amd import lfm2sc_backward, lfm2sc_backward_noalloc, lfm2sc_backward_workspace_bytes
from tests.parity_util import assert_bits, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _both(c, with_extras):
    g = c.to(DEV)
    T, H, K = c.inp.shape[0], c.H, c.K
    N = c.cu.numel() - 1
    bias = c.extra.get("bias")
    dF = c.extra.get("d_final")
    kw = {}
    if with_extras:
        kw = dict(init_state_pool=g.pool, slot_idx=g.slot_idx, bias=bias.to(DEV), d_final_state=dF.to(DEV))
    outs = []
    for noalloc in (False, True):
        d_in = _nan((T, 3 * H), c.dtype)
        dW = torch.full((H, K), float("nan"), dtype=torch.float32, device=DEV)
        db = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV) if with_extras else None
        di = _nan((N, H, K), c.dtype) if with_extras else None
        if noalloc:
            lfm2sc_backward_noalloc(g.inp, g.cu, g.w, g.dy, d_in, dW, dbias=db, d_init_state=di, **kw)
        else:
            ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(c.dtype, H, K, T, N)), dtype=torch.uint8,
                             device=DEV)
            lfm2sc_backward(g.inp, g.cu, g.w, g.dy, d_in, dW, ws, dbias=db, d_init_state=di, **kw)
        torch.cuda.synchronize()
        outs.append((d_in, dW, db, di))
    (a_in, a_w, a_b, a_i), (b_in, b_w, b_b, b_i) = outs
    assert_bits(b_in, a_in, "d_in: no-alloc vs workspace")
    assert_bits(b_w, a_w, "dW: no-alloc vs workspace")
    if with_extras:
        assert_bits(b_b, a_b, "dbias: no-alloc vs workspace")
        assert_bits(b_i, a_i, "d_init: no-alloc vs workspace")
    return b_in, b_w, b_b, b_i


def test_noalloc_matches_workspace_entry_point():
    # 1: the training step's shape (one 65,536-token sequence, H=2048, bf16): the largest use of the array
    print("case: no-alloc backward, T=65536 H=2048 K=3 bf16", flush=True)
    c1 = wl.train_lfm2(seed=71, T=65536)
    _both(c1, False)
    # 2: a smaller ragged batch with initial states, bias and final-state gradient (fewer partial rows than call 1)
    print("case: no-alloc backward, ragged lens=[700, 1, 0, 2500, 31] H=2048 K=3 bf16", flush=True)
    c2 = wl.integer_case(72, [700, 1, 0, 2500, 31], H=2048, K=3, slots=9, bias=True, d_final=True)
    d_in, dW, db, di = _both(c2, True)
    d_ref, dW_ref, db_ref, di_ref = oracle.backward(c2.inp, c2.cu, c2.w, c2.dy, c2.pool, c2.slot_idx,
                                                    bias=c2.extra["bias"], d_final=c2.extra["d_final"], full=True)
    assert_close(d_in, d_ref, c2.dtype, "d_in vs oracle")
    assert_close(dW, dW_ref, c2.dtype, "dW vs oracle")
    assert_close(db, db_ref, c2.dtype, "dbias vs oracle")
    assert_close(di, di_ref, c2.dtype, "d_init vs oracle")
    # 3: smaller still, fp32, another channel count and tap count
    print("case: no-alloc backward, T=300 H=520 K=4 fp32", flush=True)
    c3 = wl.random_case(73, [300], H=520, K=4, dtype=torch.float32, with_dy=True)
    d_in, dW, _, _ = _both(c3, False)
    d_ref, dW_ref = oracle.backward(c3.inp, c3.cu, c3.w, c3.dy)
    assert_close(d_in, d_ref, torch.float32, "fp32 d_in vs oracle")
    assert_close(dW, dW_ref, torch.float32, "fp32 dW vs oracle")
