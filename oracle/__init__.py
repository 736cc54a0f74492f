"""fp64 CPU oracle for the LFM2 gated short causal convolution.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package; the product
path (``gated_short_causal_amd``) never does, and the two share no code.

Thin ctypes wrapper around ``liboracle.so`` (built from ``oracle.c`` by
``oracle/build.py``).  Every function takes array-likes (numpy arrays, or CPU
torch tensors of any float dtype, widened exactly to float64) and returns new
float64 numpy arrays; inputs are never modified.  The arithmetic and the
passages it follows are documented in ``oracle.h`` / ``oracle.c``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LFM2SC_ORACLE_LIB may name another build of the same source (the sanitizer build of the host tests).
_LIB_PATH = os.environ.get("LFM2SC_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"oracle library missing: build it with `python oracle/build.py` ({_LIB_PATH})")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_set_threads.argtypes = [_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_get_threads.argtypes = []
    lib.oracle_get_threads.restype = _int
    lib.oracle_prefill.argtypes = [_int, _int, _i64, _dp, _i64, _ip, _int, _dp, _dp, _dp, _i64, _ip, _dp]
    lib.oracle_decode.argtypes = [_int, _int, _int, _dp, _i64, _dp, _dp, _dp, _i64, _ip, _dp]
    lib.oracle_verify.argtypes = [_int, _int, _int, _int, _dp, _i64, _dp, _dp, _dp, _i64, _ip, _dp, _dp]
    lib.oracle_commit.argtypes = [_int, _int, _int, _int, _dp, _ip, _dp, _i64, _ip]
    lib.oracle_backward.argtypes = [_int, _int, _i64, _dp, _i64, _ip, _int, _dp, _dp, _dp, _i64, _ip, _dp, _dp, _dp,
                                    _dp, _dp, _dp]
    for name in ("oracle_prefill", "oracle_decode", "oracle_verify", "oracle_commit", "oracle_backward"):
        getattr(lib, name).restype = _int
    _lib = lib
    lib.oracle_in_proj.argtypes = [_i64, _int, _int, _dp, _i64, _dp, _dp]
    lib.oracle_conv_update.argtypes = [_int, _int, _int, _int, _dp, _dp, _dp, _dp, _i64, _ip, _dp, _dp]
    return lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def f64(x):
    """Exact widening to a C-contiguous float64 numpy array (None passes through)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen on the CPU (bf16 -> f64 is exact)
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: arguments rejected by the oracle (rc={rc})")


def _pool3(pool, H, K):
    """Pool as a dense float64 [slots][H][K] copy (any [slots][>=H*K] layout accepted)."""
    p = f64(pool)
    p = p.reshape(p.shape[0], -1)[:, : H * K]
    return np.ascontiguousarray(p).reshape(-1, H, K).copy()


def prefill(inp, cu, w, pool=None, slot_idx=None, bias=None):
    """Ragged prefill.  Returns (y [total_T, H], new_pool or None)."""
    inp, w, cu, bias = f64(inp), f64(w), i32(cu), f64(bias)
    H, K = w.shape
    total_T = inp.shape[0]
    N = cu.shape[0] - 1
    y = np.full((total_T, H), np.nan)
    newpool = None
    sl = None
    if pool is not None:
        newpool = _pool3(pool, H, K)
        sl = i32(slot_idx)
    _check(_load().oracle_prefill(H, K, total_T, _p(inp), inp.shape[1], _p(cu, _ip), N, _p(w), _p(bias),
                                  _p(newpool), 0 if newpool is None else newpool.shape[0],
                                  _p(sl, _ip), _p(y)), "prefill")
    return y, newpool


def decode(inp, w, pool, slot_idx, bias=None):
    """One decode token per sequence (row i = sequence i).  Returns (y [N, H], new_pool)."""
    inp, w, bias = f64(inp), f64(w), f64(bias)
    H, K = w.shape
    sl = i32(slot_idx)
    N = sl.shape[0]
    newpool = _pool3(pool, H, K)
    y = np.full((N, H), np.nan)
    _check(_load().oracle_decode(H, K, N, _p(inp), inp.shape[1], _p(w), _p(bias), _p(newpool), newpool.shape[0],
                                 _p(sl, _ip), _p(y)), "decode")
    return y, newpool


def verify(inp, w, pool, slot_idx, L, bias=None):
    """Verify window (row i*L+s).  Returns (y [N*L, H], tape [N, L, H, K]); pool untouched."""
    inp, w, bias = f64(inp), f64(w), f64(bias)
    H, K = w.shape
    sl = i32(slot_idx)
    N = sl.shape[0]
    p = _pool3(pool, H, K)
    y = np.full((N * L, H), np.nan)
    tape = np.full((N, L, H, K), np.nan)
    _check(_load().oracle_verify(H, K, N, L, _p(inp), inp.shape[1], _p(w), _p(bias), _p(p), p.shape[0],
                                 _p(sl, _ip), _p(tape), _p(y)), "verify")
    return y, tape


def commit(tape, accept, pool, slot_idx):
    """Post-verify commit.  Returns the new pool [slots, H, K]."""
    tape = f64(tape)
    N, L, H, K = tape.shape
    acc, sl = i32(accept), i32(slot_idx)
    newpool = _pool3(pool, H, K)
    _check(_load().oracle_commit(H, K, N, L, _p(tape), _p(acc, _ip), _p(newpool), newpool.shape[0],
                                 _p(sl, _ip)), "commit")
    return newpool


def backward(inp, cu, w, dy, pool=None, slot_idx=None, bias=None, d_final=None, full=False):
    """Backward of prefill.  Returns (d_in [total_T, 3H] = dB|dC|dxv, dW [H, K]), or with full=True
    (d_in, dW, dbias [H], d_init [N, H, K]).  d_final: gradient of each sequence's final state [N, H, K]."""
    inp, w, cu, dy, bias = f64(inp), f64(w), i32(cu), f64(dy), f64(bias)
    H, K = w.shape
    total_T = inp.shape[0]
    N = cu.shape[0] - 1
    dF = None if d_final is None else f64(d_final).reshape(N, H, K)
    d_in = np.full((total_T, 3 * H), np.nan)
    dW = np.full((H, K), np.nan)
    dbias = np.full((H,), np.nan)
    d_init = np.full((N, H, K), np.nan)
    p, sl = None, None
    if pool is not None:
        p = _pool3(pool, H, K)
        sl = i32(slot_idx)
    _check(_load().oracle_backward(H, K, total_T, _p(inp), inp.shape[1], _p(cu, _ip), N, _p(w), _p(bias),
                                   _p(p), 0 if p is None else p.shape[0], _p(sl, _ip), _p(dy), _p(dF),
                                   _p(d_in), _p(dW), _p(dbias), _p(d_init)), "backward")
    return (d_in, dW, dbias, d_init) if full else (d_in, dW)


def in_proj(x, W_in):
    """x [rows, >=D] @ W_in[3H, D]^T -> [rows, 3H] (B | C | xv), fp64."""
    x, W_in = f64(x), f64(W_in)
    n_out, D = W_in.shape
    rows = x.shape[0]
    out = np.full((rows, n_out), np.nan)
    _check(_load().oracle_in_proj(rows, D, n_out, _p(x), x.shape[1] if x.ndim == 2 else D, _p(W_in), _p(out)),
           "in_proj")
    return out


def fused_prefill(x, W_in, cu, w, pool=None, slot_idx=None, bias=None):
    """in_proj followed by the ragged prefill.  Returns (y [rows, H], new_pool or None, in_proj [rows, 3H])."""
    ip = in_proj(x, W_in)
    y, newpool = prefill(ip, cu, w, pool, slot_idx, bias)
    return y, newpool, ip


def conv_update(bx, w, pool, slot_idx, bias=None, with_tape=True):
    """Conv update of gated inputs bx [N, H, L] (any strides; copied dense).  Returns (out [N, H, L], tape
    [N, L, H, K] or None, new_pool): with a tape the pool is returned unchanged, without one each named slot
    holds the state after the L tokens."""
    bx, w, bias = f64(bx), f64(w), f64(bias)
    H, K = w.shape
    N, Hb, L = bx.shape
    assert Hb == H
    newpool = _pool3(pool, H, K)
    sl = i32(slot_idx)
    out = np.full((N, H, L), np.nan)
    tape = np.full((N, L, H, K), np.nan) if with_tape else None
    _check(_load().oracle_conv_update(H, K, N, L, _p(bx), _p(w), _p(bias), _p(newpool), newpool.shape[0],
                                      _p(sl, _ip), _p(tape), _p(out)), "conv_update")
    return out, tape, newpool

