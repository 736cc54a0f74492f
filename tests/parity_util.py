"""Comparison helpers for the GPU parity tests (no arithmetic of the op here)."""
import numpy as np
import torch

# Tolerances: an element passes iff |gpu - ref| <= max(atol, rtol * |ref|), with the fp64 oracle as ref.
TOL = {torch.bfloat16: (2e-2, 2e-2), torch.float32: (1e-5, 1e-5)}


def assert_close(gpu, ref, dtype, what):
    atol, rtol = TOL[dtype]
    g = gpu.detach().cpu().double().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    ok = err <= np.maximum(atol, rtol * np.abs(r))
    max_abs = float(np.nanmax(err)) if err.size else 0.0
    rel = err / np.maximum(np.abs(r), 1e-30)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} elements out of tolerance; first at {i}: "
                             f"gpu={g[i]!r} ref={r[i]!r}; max_abs={max_abs:.3e}")
    return max_abs, float(np.nanmax(np.where(np.abs(r) > atol, rel, 0.0))) if rel.size else 0.0


def rounded(ref_f64, dtype):
    """The oracle value rounded to the I/O dtype (round-to-nearest-even), as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(ref_f64)).to(dtype)


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def assert_bits(gpu, expected, what):
    a, b = _bits(gpu), _bits(expected)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    neq = (a != b)
    if neq.any():
        idx = neq.nonzero()[0].tolist()
        raise AssertionError(f"{what}: {int(neq.sum())} of {neq.numel()} entries differ bitwise; first at {idx}: "
                             f"gpu={gpu.detach().cpu()[tuple(idx)].item()!r} "
                             f"expected={expected.detach().cpu()[tuple(idx)].item()!r}")
