"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

Every call below is built to fail host validation (or to hit an early no-work
return), so none of them reaches a kernel launch: the pointers are fake.
"""
import ctypes
import os
import re

import pytest

from gated_short_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lfm2sc.h")

OK, NULLP, SHAPE, ALIGN, UNSUP, WS, PRECOND, HIP = range(8)

P = 0x10000      # fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x10002    # fake, misaligned


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(lfm2sc_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) == 14, names
    assert set(names) == set(_lib.SIGNATURES), (names, sorted(_lib.SIGNATURES))
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_matches_header(L):
    m = re.search(r"#define\s+LFM2SC_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert L.lfm2sc_abi_version() == int(m.group(1))


def test_status_strings(L):
    names = ["LFM2SC_OK", "LFM2SC_ERR_NULL_POINTER", "LFM2SC_ERR_BAD_SHAPE", "LFM2SC_ERR_ALIGNMENT",
             "LFM2SC_ERR_UNSUPPORTED", "LFM2SC_ERR_WORKSPACE", "LFM2SC_ERR_PRECONDITION", "LFM2SC_ERR_HIP"]
    for code, name in enumerate(names):
        assert L.lfm2sc_status_string(code).decode() == name
    assert L.lfm2sc_status_string(99).decode() == "LFM2SC_UNKNOWN_STATUS"


def _prefill(L, **kw):
    a = dict(dtype=0, H=256, K=3, in_proj=P, in_stride=768, total_T=64, cu=P, N=1, w=P, bias=None,
             pool=None, num_slots=0, slot_stride=0, slot_idx=None, y=P, y_stride=256, stream=None)
    a.update(kw)
    return L.lfm2sc_prefill_ragged(a["dtype"], a["H"], a["K"], a["in_proj"], a["in_stride"], a["total_T"], a["cu"],
                                   a["N"], a["w"], a["bias"], a["pool"], a["num_slots"], a["slot_stride"],
                                   a["slot_idx"], a["y"], a["y_stride"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), UNSUP), (dict(H=0), SHAPE), (dict(H=12), SHAPE), (dict(H=4), SHAPE),
    (dict(K=0), UNSUP), (dict(K=5), UNSUP), (dict(bias=MIS), ALIGN),
    (dict(N=-1), SHAPE), (dict(total_T=-1), SHAPE), (dict(total_T=1 << 31), SHAPE),
    (dict(in_stride=700), SHAPE), (dict(in_stride=772), ALIGN), (dict(y_stride=100), SHAPE), (dict(y_stride=260), ALIGN),
    (dict(in_proj=None), NULLP), (dict(cu=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP),
    (dict(in_proj=MIS), ALIGN), (dict(w=MIS), ALIGN), (dict(y=MIS), ALIGN), (dict(cu=P + 2), ALIGN),
    (dict(pool=P, num_slots=4, slot_stride=768, slot_idx=None), NULLP),
    (dict(pool=P, num_slots=0, slot_stride=768, slot_idx=P), SHAPE),
    (dict(pool=P, num_slots=4, slot_stride=760, slot_idx=P), SHAPE),
    (dict(pool=P, num_slots=4, slot_stride=772, slot_idx=P), ALIGN),
    (dict(pool=MIS, num_slots=4, slot_stride=768, slot_idx=P), ALIGN),
])
def test_prefill_rejects(L, kw, code):
    assert _prefill(L, **kw) == code
    assert L.lfm2sc_last_error().decode().startswith("lfm2sc_prefill_ragged")


def test_prefill_no_work_is_ok_without_launch(L):
    # no sequence, or no token: returns OK before touching any pointer
    assert _prefill(L, N=0, in_proj=None, cu=None, y=None) == OK
    assert _prefill(L, total_T=0, in_proj=None, cu=None, y=None) == OK
    assert L.lfm2sc_last_error().decode() == ""


def _decode(L, **kw):
    a = dict(dtype=0, H=2048, K=3, in_proj=P, in_stride=6144, N=256, w=P, bias=None, pool=P, num_slots=1024,
             slot_stride=6144, slot_idx=P, y=P, y_stride=2048, stream=None)
    a.update(kw)
    return L.lfm2sc_decode_step(a["dtype"], a["H"], a["K"], a["in_proj"], a["in_stride"], a["N"], a["w"], a["bias"],
                                a["pool"], a["num_slots"], a["slot_stride"], a["slot_idx"], a["y"], a["y_stride"],
                                a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pool=None), NULLP), (dict(slot_idx=None), NULLP), (dict(y=None), NULLP), (dict(in_proj=None), NULLP),
    (dict(N=-3), SHAPE), (dict(num_slots=0), SHAPE), (dict(slot_stride=6136), SHAPE), (dict(dtype=7), UNSUP),
    (dict(bias=P + 8), ALIGN), (dict(in_stride=6148), ALIGN), (dict(pool=MIS), ALIGN), (dict(slot_idx=P + 1), ALIGN),
])
def test_decode_rejects(L, kw, code):
    assert _decode(L, **kw) == code


def _verify(L, **kw):
    a = dict(dtype=0, H=2048, K=3, in_proj=P, in_stride=6144, N=64, Lb=8, w=P, bias=None, pool=P, num_slots=256,
             slot_stride=6144, slot_idx=P, win=P, y=P, y_stride=2048, stream=None)
    a.update(kw)
    return L.lfm2sc_verify_window(a["dtype"], a["H"], a["K"], a["in_proj"], a["in_stride"], a["N"], a["Lb"], a["w"],
                                  a["bias"], a["pool"], a["num_slots"], a["slot_stride"], a["slot_idx"], a["win"],
                                  a["y"], a["y_stride"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(win=None), NULLP), (dict(win=None, N=0), NULLP),   # the tape is mandatory, even for an empty batch
    (dict(win=MIS), ALIGN), (dict(Lb=-1), SHAPE), (dict(pool=None), NULLP), (dict(K=9), UNSUP),
])
def test_verify_rejects(L, kw, code):
    assert _verify(L, **kw) == code


def _commit(L, **kw):
    a = dict(dtype=0, H=2048, K=3, win=P, N=64, Lb=8, acc=P, pool=P, num_slots=256, slot_stride=6144, slot_idx=P,
             stream=None)
    a.update(kw)
    return L.lfm2sc_commit_window(a["dtype"], a["H"], a["K"], a["win"], a["N"], a["Lb"], a["acc"], a["pool"],
                                  a["num_slots"], a["slot_stride"], a["slot_idx"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(win=None), NULLP), (dict(acc=None), NULLP), (dict(pool=None), NULLP), (dict(slot_idx=None), NULLP),
    (dict(N=-1), SHAPE), (dict(acc=P + 2), ALIGN), (dict(H=7), SHAPE),
])
def test_commit_rejects(L, kw, code):
    assert _commit(L, **kw) == code


def test_commit_no_work(L):
    assert _commit(L, N=0, win=None, acc=None, pool=None, slot_idx=None) == OK
    assert _commit(L, Lb=0, win=None, acc=None) == OK


def _bwd(L, **kw):
    a = dict(dtype=0, H=2048, K=3, in_proj=P, in_stride=6144, total_T=4096, cu=P, N=1, w=P, bias=None, pool=None,
             num_slots=0, slot_stride=0, slot_idx=None, dy=P, dy_stride=2048, dfinal=None, din=P, din_stride=6144,
             dW=P, dbias=None, dinit=None, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.lfm2sc_backward(a["dtype"], a["H"], a["K"], a["in_proj"], a["in_stride"], a["total_T"], a["cu"], a["N"],
                             a["w"], a["bias"], a["pool"], a["num_slots"], a["slot_stride"], a["slot_idx"], a["dy"],
                             a["dy_stride"], a["dfinal"], a["din"], a["din_stride"], a["dW"], a["dbias"], a["dinit"],
                             a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dW=None), NULLP), (dict(dW=P + 2), ALIGN), (dict(dy=None), NULLP), (dict(din=None), NULLP),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS), (dict(ws=P + 8), ALIGN), (dict(din_stride=6000), SHAPE),
    (dict(dy_stride=2044), SHAPE), (dict(dy_stride=2052), ALIGN), (dict(cu=None), NULLP),
    (dict(pool=P, num_slots=2, slot_stride=6144, slot_idx=None), NULLP), (dict(K=0), UNSUP),
    (dict(bias=P + 4, dW=None), ALIGN), (dict(dbias=P + 2), ALIGN), (dict(dfinal=P + 8), ALIGN),
    (dict(dinit=P + 8), ALIGN),
])
def test_backward_rejects(L, kw, code):
    assert _bwd(L, **kw) == code


def test_workspace_bytes(L):
    f = L.lfm2sc_backward_workspace_bytes
    assert f(0, 2048, 3, 0, 0) == 0
    assert f(0, 2048, 3, 65536, 1) > 0
    assert f(0, 2048, 3, 65536, 1) % 256 == 0
    # whole partial rows of H*K fp32 values (fp64 for fp32 I/O); never fewer for more tokens
    assert f(0, 2048, 3, 65536, 1) >= 2048 * 3 * 4
    # every sequence holds at least one window, each window one partial row of H x (K+1) fp32 sums
    assert f(0, 2048, 3, 65536, 8) >= 8 * 2048 * 4 * 4
    assert f(0, 2048, 3, 1 << 20, 1) >= f(0, 2048, 3, 65536, 1)
    assert f(1, 2048, 3, 65536, 1) >= 2 * f(0, 2048, 3, 65536, 1) - 256
    assert f(9, 2048, 3, 64, 1) == 0 and f(0, 12, 3, 64, 1) == 0 and f(0, 2048, 5, 64, 1) == 0


def test_window_tables_pick_measured_lengths(L):
    """The backward's window length at T=65536, one sequence, seen through its workspace (one partial row of
    H x (K+1) sums per window of 4 waves).  Row geometries with a measured rate table take the best-rated
    length up to 1/8 above the shortest one-round length; the others keep the shortest."""
    f = L.lfm2sc_backward_workspace_bytes
    T = 65536

    def windows(sub):
        return -(-T // (4 * sub))

    # (dtype, H, window length picked, accumulator bytes): 2 KiB, 3 KiB and 4 KiB bf16 rows have tables
    cases = [(0, 1024, 137, 4), (0, 1536, 228, 4), (0, 2048, 273, 4),
             (1, 2048, 256, 8),   # 8 KiB fp32 rows: no table
             (1, 1024, 128, 8),   # 4 KiB rows in 2 channel groups: the 4 KiB table is for 4 groups only
             (0, 512, 64, 4)]     # 1 KiB rows: no table
    for dtype, H, sub, acc in cases:
        got = f(dtype, H, 3, T, 1)
        want = windows(sub) * H * 4 * acc
        assert got == (want + 255) // 256 * 256, (dtype, H, got, want)


def test_binding_names_match_c_abi():
    import gated_short_causal_amd as g
    for n in ("lfm2sc_prefill_ragged", "lfm2sc_decode_step", "lfm2sc_verify_window", "lfm2sc_commit_window",
              "lfm2sc_backward", "lfm2sc_backward_workspace_bytes"):
        assert callable(getattr(g, n)) and n in _lib.SIGNATURES


def _fused(L, **kw):
    a = dict(dtype=0, H=2048, K=3, D=2048, x=P, x_stride=2048, total_T=4096, cu=P, N=1, W=P, w=P, bias=None,
             pool=None, num_slots=0, slot_stride=0, slot_idx=None, y=P, y_stride=2048, io=None, io_stride=0,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.lfm2sc_fused_prefill(a["dtype"], a["H"], a["K"], a["D"], a["x"], a["x_stride"], a["total_T"], a["cu"],
                                  a["N"], a["W"], a["w"], a["bias"], a["pool"], a["num_slots"], a["slot_stride"],
                                  a["slot_idx"], a["y"], a["y_stride"], a["io"], a["io_stride"], a["ws"],
                                  a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=1), UNSUP), (dict(dtype=2), UNSUP), (dict(K=5), UNSUP), (dict(bias=MIS), ALIGN),
    (dict(H=1000), SHAPE), (dict(H=72), SHAPE), (dict(D=0), SHAPE), (dict(D=1000), SHAPE), (dict(D=32), SHAPE),
    (dict(D=192), SHAPE), (dict(D=64), SHAPE),
    (dict(H=8192, D=65536, x_stride=65536), SHAPE),
    (dict(N=-1), SHAPE), (dict(total_T=-1), SHAPE), (dict(total_T=1 << 31), SHAPE),
    (dict(x_stride=2040), SHAPE), (dict(x_stride=2052), ALIGN), (dict(x_stride=1 << 22), SHAPE),
    (dict(y_stride=2047), SHAPE), (dict(io=P, io_stride=6000), SHAPE), (dict(io=P, io_stride=6148), ALIGN),
    (dict(x=None), NULLP), (dict(x=MIS), ALIGN), (dict(cu=None), NULLP), (dict(W=None), NULLP), (dict(W=MIS), ALIGN),
    (dict(w=None), NULLP), (dict(y=None), NULLP), (dict(io=MIS, io_stride=6144), ALIGN),
    (dict(pool=P, num_slots=4, slot_stride=6144, slot_idx=None), NULLP),
    (dict(pool=P, num_slots=4, slot_stride=6000, slot_idx=P), SHAPE),
    (dict(pool=P, num_slots=4, slot_stride=6144, slot_idx=P), WS),
    (dict(pool=P, num_slots=4, slot_stride=6144, slot_idx=P, ws=P, ws_bytes=100), WS),
    (dict(pool=P, num_slots=4, slot_stride=6144, slot_idx=P, ws=MIS, ws_bytes=1 << 20), ALIGN),
])
def test_fused_rejects(L, kw, code):
    assert _fused(L, **kw) == code
    assert L.lfm2sc_last_error().decode().startswith("lfm2sc_fused_prefill")


def test_fused_no_work_is_ok_without_launch(L):
    assert _fused(L, N=0, x=None, cu=None, W=None, y=None) == OK
    assert _fused(L, total_T=0, x=None, cu=None, W=None, y=None) == OK


def test_fused_workspace_bytes(L):
    assert L.lfm2sc_fused_prefill_workspace_bytes(0, 2048, 3, 8, 0) == 0
    assert L.lfm2sc_fused_prefill_workspace_bytes(0, 2048, 3, 8, 1) == 8 * 2048 * 3 * 2
    assert L.lfm2sc_fused_prefill_workspace_bytes(0, 64, 1, 1, 1) == 256
    assert L.lfm2sc_fused_prefill_workspace_bytes(1, 2048, 3, 8, 1) == 0     # fp32 unsupported
    assert L.lfm2sc_fused_prefill_workspace_bytes(0, 72, 3, 8, 1) == 0       # H % 64 != 0


def _cu(lib, **kw):
    a = dict(dtype=0, H=2048, K=3, N=64, L=8, bx=P, bsn=8 * 2048, bsh=1, bst=2048, w=P, bias=None, pool=P,
             num_slots=256, slot_stride=6144, slot_idx=P, win=None, out=P, osn=8 * 2048, osh=1, ost=2048,
             stream=None)
    a.update(kw)
    return lib.lfm2sc_conv_update(a["dtype"], a["H"], a["K"], a["N"], a["L"], a["bx"], a["bsn"], a["bsh"], a["bst"],
                                  a["w"], a["bias"], a["pool"], a["num_slots"], a["slot_stride"], a["slot_idx"],
                                  a["win"], a["out"], a["osn"], a["osh"], a["ost"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), UNSUP), (dict(K=5), UNSUP), (dict(H=12), SHAPE), (dict(bias=MIS), ALIGN),
    (dict(N=-1), SHAPE), (dict(L=-1), SHAPE), (dict(N=1 << 20, L=1 << 12), SHAPE),
    (dict(bsn=-1), SHAPE), (dict(bsh=-8), SHAPE), (dict(ost=-1), SHAPE),
    (dict(bx=None), NULLP), (dict(out=None), NULLP), (dict(bx=P + 1), ALIGN), (dict(dtype=1, out=P + 2), ALIGN),
    (dict(w=None), NULLP), (dict(pool=None), NULLP), (dict(slot_idx=None), NULLP),
    (dict(slot_stride=6000), SHAPE), (dict(win=P + 8), ALIGN),
])
def test_conv_update_rejects(L, kw, code):
    assert _cu(L, **kw) == code
    assert L.lfm2sc_last_error().decode().startswith("lfm2sc_conv_update")


def test_conv_update_no_work_is_ok(L):
    assert _cu(L, N=0, bx=None, out=None, pool=None, slot_idx=None) == OK
    assert _cu(L, L=0, bx=None, out=None, pool=None, slot_idx=None) == OK



def _bwd_noalloc(L, **kw):
    a = dict(dtype=0, H=2048, K=3, in_proj=P, in_stride=6144, total_T=65536, cu=P, N=1, w=P, bias=None, pool=None,
             num_slots=0, slot_stride=0, slot_idx=None, dy=P, dy_stride=2048, dF=None, din=P, din_stride=6144, dW=P,
             dbias=None, dinit=None, stream=None)
    a.update(kw)
    return L.lfm2sc_backward_noalloc(a["dtype"], a["H"], a["K"], a["in_proj"], a["in_stride"], a["total_T"], a["cu"],
                                     a["N"], a["w"], a["bias"], a["pool"], a["num_slots"], a["slot_stride"],
                                     a["slot_idx"], a["dy"], a["dy_stride"], a["dF"], a["din"], a["din_stride"],
                                     a["dW"], a["dbias"], a["dinit"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(din=None), NULLP), (dict(dW=None), NULLP), (dict(H=12), SHAPE), (dict(dy_stride=2040), SHAPE),
    (dict(din_stride=6150), ALIGN), (dict(dtype=3), UNSUP), (dict(in_proj=MIS), ALIGN),
    # more windows than the fixed scratch array holds partial rows for
    (dict(N=5000, total_T=1 << 20), WS), (dict(H=131072, total_T=1 << 20, in_stride=3 * 131072,
                                                dy_stride=131072, din_stride=3 * 131072), WS),
])
def test_backward_noalloc_rejects(L, kw, code):
    assert _bwd_noalloc(L, **kw) == code
    if code == WS:
        assert b"LFM2SC_NOALLOC_SCRATCH_BYTES" in L.lfm2sc_last_error()


def test_noalloc_limit_matches_header():
    from gated_short_causal_amd import binding
    m = re.search(r"#define\s+LFM2SC_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and binding.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_noalloc_headline_call_fits(L):
    """One 65,536-token sequence at H=2048 (the training step) fits the fixed scratch array."""
    from gated_short_causal_amd import binding
    need = L.lfm2sc_backward_workspace_bytes(0, 2048, 3, 65536, 1)
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
