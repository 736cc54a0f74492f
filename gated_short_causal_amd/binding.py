"""Python binding of the C ABI: the same entry-point names, taking torch tensors.

Argument marshalling only -- device pointers, strides, sizes and the current
HIP stream are read from the tensors and handed to liblfm2sc.so; every step of
the computation runs in the library's HIP kernels.  Outputs are caller-owned
tensors, written in place, exactly as the C calls do.

The C ABI sees plain pointers and cannot check what lies behind them, so each
binding first checks what it can see in the tensors and raises ValueError or
TypeError before any library call when one fails: every tensor is a GPU tensor
on the weight's device, every I/O tensor has the weight's dtype, index tensors
are int32, and every tensor covers the rows, columns and entries the kernels of
that call will touch (sizes the library derives from the other arguments).

Tensor conventions (see include/lfm2sc.h for the full contract):
  in_proj   [rows, >=3H]  bf16 or fp32, unit column stride (B | C | xv)
  weight    [H, K]        same dtype, contiguous
  state pool [slots, H, K] (or [slots, >=H*K]) same dtype, each slot contiguous
  cu_seqlens, slot_idx, accept_len: int32 device tensors
"""
import torch

from . import _lib

LFM2SC_BF16 = 0
LFM2SC_F32 = 1

_DTYPES = {torch.bfloat16: LFM2SC_BF16, torch.float32: LFM2SC_F32}


class Lfm2scError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = _lib.lib().lfm2sc_status_string(status).decode()
        super().__init__(f"{name}: {detail}")


def _check(rc: int):
    if rc != 0:
        raise Lfm2scError(rc, _lib.lib().lfm2sc_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")
    return _DTYPES[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _is_gpu(t: torch.Tensor) -> bool:
    return t.is_cuda


def _same_device(ref: torch.Tensor, **tensors):
    """Every given tensor lives on ref's GPU (the library dereferences their pointers on that device)."""
    if not _is_gpu(ref):
        raise ValueError(f"weight must be a GPU tensor, got device {ref.device}")
    for name, t in tensors.items():
        if t is not None and (not _is_gpu(t) or t.device != ref.device):
            raise ValueError(f"{name} must be on {ref.device} (the weight's device), got {t.device}")


def _same_dtype(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}; every I/O tensor must have the weight's dtype {ref.dtype}")


def _rows(t: torch.Tensor, name: str, min_rows: int = 0, min_cols: int = 0):
    """Row stride of a 2-D row-major tensor with unit column stride and at least min_rows x min_cols."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride, got shape {tuple(t.shape)} strides {t.stride()}")
    if t.shape[0] < min_rows or t.shape[1] < min_cols:
        raise ValueError(f"{name} of shape {tuple(t.shape)} is smaller than the [{min_rows}, {min_cols}] the call "
                         "touches")
    return t.stride(0)


def _pool_stride(pool: torch.Tensor, H: int, K: int) -> int:
    if pool.dim() == 3:
        if pool.shape[1:] != (H, K) or pool.stride(2) != 1 or pool.stride(1) != K:
            raise ValueError(f"state pool must be [slots, {H}, {K}] with contiguous slots")
    elif pool.dim() == 2:
        if pool.shape[1] < H * K or pool.stride(1) != 1:
            raise ValueError(f"state pool must be [slots, >= {H * K}] with unit column stride")
    else:
        raise ValueError("state pool must be 2-D or 3-D")
    if pool.shape[0] < 1:
        raise ValueError("state pool has no slot")
    return pool.stride(0)


def _i32(t, name, min_numel: int = 0):
    if t is None:
        return t
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    if not t.is_contiguous() or t.numel() < min_numel:
        raise ValueError(f"{name} must be a contiguous int32 tensor of at least {min_numel} entries, "
                         f"got {t.numel()}")
    return t


def _dense(t, name, numel: int, dtype=None):
    """A contiguous tensor of at least `numel` entries (and the given dtype)."""
    if t is None:
        return t
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name} must be contiguous with at least {numel} entries, got shape {tuple(t.shape)}")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _hk(weight: torch.Tensor):
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [H, K] tensor")
    return weight.shape[0], weight.shape[1]


def _pool_args(pool, slot_idx, N, H, K, name="state_pool"):
    """(num_slots, slot_stride) of an optional pool; slot_idx must then name N slots."""
    if pool is None:
        return 0, 0
    stride = _pool_stride(pool, H, K)
    if slot_idx is None:
        raise ValueError(f"slot_idx is required with {name}")
    _i32(slot_idx, "slot_idx", N)
    return pool.shape[0], stride


def _cu(cu_seqlens):
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 row offsets")
    _i32(cu_seqlens, "cu_seqlens", 1)
    return cu_seqlens.numel() - 1


def lfm2sc_prefill_ragged(in_proj, cu_seqlens, weight, y, state_pool=None, slot_idx=None, bias=None):
    H, K = _hk(weight)
    _same_device(weight, in_proj=in_proj, cu_seqlens=cu_seqlens, y=y, state_pool=state_pool, slot_idx=slot_idx,
                 bias=bias)
    _same_dtype(weight, in_proj=in_proj, y=y, state_pool=state_pool, bias=bias)
    N = _cu(cu_seqlens)
    T = in_proj.shape[0]
    in_stride = _rows(in_proj, "in_proj", 0, 3 * H)
    y_stride = _rows(y, "y", T, H)
    _dense(bias, "bias", H)
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    _check(_lib.lib().lfm2sc_prefill_ragged(
        _dtype_code(weight), H, K, _ptr(in_proj), in_stride, T,
        _ptr(cu_seqlens), N, _ptr(weight), _ptr(bias),
        _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(y), y_stride, _stream(weight.device)))
    return y


def lfm2sc_decode_step(in_proj, weight, state_pool, slot_idx, y, bias=None):
    H, K = _hk(weight)
    _same_device(weight, in_proj=in_proj, state_pool=state_pool, slot_idx=slot_idx, y=y, bias=bias)
    _same_dtype(weight, in_proj=in_proj, state_pool=state_pool, y=y, bias=bias)
    if state_pool is None or slot_idx is None:
        raise ValueError("decode needs a state pool and slot_idx")
    N = _i32(slot_idx, "slot_idx").numel()
    in_stride = _rows(in_proj, "in_proj", N, 3 * H)
    y_stride = _rows(y, "y", N, H)
    _dense(bias, "bias", H)
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    _check(_lib.lib().lfm2sc_decode_step(
        _dtype_code(weight), H, K, _ptr(in_proj), in_stride, N,
        _ptr(weight), _ptr(bias), _ptr(state_pool), num_slots, slot_stride,
        _ptr(slot_idx), _ptr(y), y_stride, _stream(weight.device)))
    return y


def lfm2sc_verify_window(in_proj, weight, state_pool, slot_idx, L, windows, y, bias=None):
    H, K = _hk(weight)
    _same_device(weight, in_proj=in_proj, state_pool=state_pool, slot_idx=slot_idx, windows=windows, y=y, bias=bias)
    _same_dtype(weight, in_proj=in_proj, state_pool=state_pool, windows=windows, y=y, bias=bias)
    if state_pool is None or slot_idx is None:
        raise ValueError("verify needs a state pool and slot_idx")
    N = _i32(slot_idx, "slot_idx").numel()
    L = int(L)
    if L < 0:
        raise ValueError(f"L={L} must be >= 0")
    if windows is not None and (not windows.is_contiguous() or windows.numel() < N * L * H * K):
        raise ValueError(f"windows must be a contiguous [{N}, {L}, {H}, {K}] tensor")
    in_stride = _rows(in_proj, "in_proj", N * L, 3 * H)
    y_stride = _rows(y, "y", N * L, H)
    _dense(bias, "bias", H)
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    _check(_lib.lib().lfm2sc_verify_window(
        _dtype_code(weight), H, K, _ptr(in_proj), in_stride, N, L,
        _ptr(weight), _ptr(bias), _ptr(state_pool), num_slots, slot_stride,
        _ptr(slot_idx), _ptr(windows), _ptr(y), y_stride, _stream(weight.device)))
    return y, windows


def lfm2sc_commit_window(windows, accept_len, state_pool, slot_idx):
    if windows.dim() != 4 or not windows.is_contiguous():
        raise ValueError("windows must be contiguous [N, L, H, K]")
    N, L, H, K = windows.shape
    _same_device(windows, accept_len=accept_len, state_pool=state_pool, slot_idx=slot_idx)
    _same_dtype(windows, state_pool=state_pool)
    _i32(accept_len, "accept_len", N)
    if state_pool is None or slot_idx is None or accept_len is None:
        raise ValueError("commit needs accept_len, a state pool and slot_idx")
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    _check(_lib.lib().lfm2sc_commit_window(
        _dtype_code(windows), H, K, _ptr(windows), N, L, _ptr(accept_len),
        _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _stream(windows.device)))
    return state_pool


def lfm2sc_backward_workspace_bytes(dtype, H, K, total_T, num_seqs) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().lfm2sc_backward_workspace_bytes(code, H, K, total_T, num_seqs))


def _backward_args(in_proj, cu_seqlens, weight, dy, d_in_proj, dW, workspace, init_state_pool, slot_idx, bias,
                   d_final_state, dbias, d_init_state):
    """Checks shared by the backward entry points; returns the marshalled sizes and strides."""
    H, K = _hk(weight)
    _same_device(weight, in_proj=in_proj, cu_seqlens=cu_seqlens, dy=dy, d_in_proj=d_in_proj, dW=dW,
                 workspace=workspace, init_state_pool=init_state_pool, slot_idx=slot_idx, bias=bias,
                 d_final_state=d_final_state, dbias=dbias, d_init_state=d_init_state)
    _same_dtype(weight, in_proj=in_proj, dy=dy, d_in_proj=d_in_proj, init_state_pool=init_state_pool, bias=bias,
                d_final_state=d_final_state, d_init_state=d_init_state)
    N = _cu(cu_seqlens)
    T = in_proj.shape[0]
    if dW.dtype != torch.float32 or not dW.is_contiguous() or dW.numel() < H * K:
        raise TypeError(f"dW must be a contiguous float32 [{H}, {K}] tensor")
    if dbias is not None and (dbias.dtype != torch.float32 or not dbias.is_contiguous() or dbias.numel() < H):
        raise TypeError(f"dbias must be a contiguous float32 [{H}] tensor")
    for name, t in (("d_final_state", d_final_state), ("d_init_state", d_init_state)):
        if t is not None and (not t.is_contiguous() or t.numel() < N * H * K):
            raise ValueError(f"{name} must be a contiguous [{N}, {H}, {K}] tensor of the I/O dtype")
    _dense(bias, "bias", H)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    num_slots, slot_stride = _pool_args(init_state_pool, slot_idx, N, H, K, "init_state_pool")
    strides = (_rows(in_proj, "in_proj", 0, 3 * H), _rows(dy, "dy", T, H), _rows(d_in_proj, "d_in_proj", T, 3 * H))
    return H, K, N, T, num_slots, slot_stride, strides


def lfm2sc_backward(in_proj, cu_seqlens, weight, dy, d_in_proj, dW, workspace,
                    init_state_pool=None, slot_idx=None, bias=None, d_final_state=None, dbias=None,
                    d_init_state=None):
    """Backward of lfm2sc_prefill_ragged.  Writes d_in_proj (dB | dC | dxv), dW (fp32), and when given dbias
    (fp32 [H]) and d_init_state ([N, H, K], I/O dtype).  d_final_state: gradient of the final states [N, H, K]."""
    H, K, N, T, num_slots, slot_stride, (in_s, dy_s, din_s) = _backward_args(
        in_proj, cu_seqlens, weight, dy, d_in_proj, dW, workspace, init_state_pool, slot_idx, bias, d_final_state,
        dbias, d_init_state)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lib().lfm2sc_backward(
        _dtype_code(weight), H, K, _ptr(in_proj), in_s, T,
        _ptr(cu_seqlens), N, _ptr(weight), _ptr(bias),
        _ptr(init_state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(dy), dy_s, _ptr(d_final_state), _ptr(d_in_proj), din_s, _ptr(dW),
        _ptr(dbias), _ptr(d_init_state), _ptr(workspace), ws_bytes, _stream(weight.device)))
    return d_in_proj, dW


# LFM2SC_NOALLOC_SCRATCH_BYTES of include/lfm2sc.h: the most workspace lfm2sc_backward_noalloc can stand in for
NOALLOC_SCRATCH_BYTES = 8 << 20


def lfm2sc_backward_noalloc(in_proj, cu_seqlens, weight, dy, d_in_proj, dW, init_state_pool=None, slot_idx=None,
                            bias=None, d_final_state=None, dbias=None, d_init_state=None):
    """lfm2sc_backward without a workspace argument, for callers that cannot allocate: the library keeps the
    partial sums in a fixed device array of NOALLOC_SCRATCH_BYTES per GPU.  Calls that overlap on one GPU race."""
    H, K, N, T, num_slots, slot_stride, (in_s, dy_s, din_s) = _backward_args(
        in_proj, cu_seqlens, weight, dy, d_in_proj, dW, None, init_state_pool, slot_idx, bias, d_final_state,
        dbias, d_init_state)
    _check(_lib.lib().lfm2sc_backward_noalloc(
        _dtype_code(weight), H, K, _ptr(in_proj), in_s, T,
        _ptr(cu_seqlens), N, _ptr(weight), _ptr(bias),
        _ptr(init_state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(dy), dy_s, _ptr(d_final_state), _ptr(d_in_proj), din_s, _ptr(dW),
        _ptr(dbias), _ptr(d_init_state), _stream(weight.device)))
    return d_in_proj, dW


def lfm2sc_fused_prefill_workspace_bytes(dtype, H, K, num_seqs, with_pool) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().lfm2sc_fused_prefill_workspace_bytes(code, H, K, num_seqs, int(bool(with_pool))))


def lfm2sc_fused_prefill_plan(H, K, D, total_T) -> int:
    """The tiling lfm2sc_fused_prefill takes for these sizes: 1 wide tiles, 2 wide tiles with halo rows, 3 the
    4-wave tile, 32 / 64 split tiles, 128 mid tiles, 0 for no token; negative for sizes it rejects."""
    return int(_lib.lib().lfm2sc_fused_prefill_plan(H, K, D, total_T))


def lfm2sc_fused_prefill(x, W_in, cu_seqlens, weight, y, state_pool=None, slot_idx=None, bias=None,
                         in_proj_out=None, workspace=None):
    """in_proj (x @ W_in^T, on the matrix cores) fused with the ShortConv prefill.  x [rows, >=D] bf16,
    W_in [3H, D] bf16.  Writes y (and in_proj_out when given); with a pool, the final states go through
    `workspace` (lfm2sc_fused_prefill_workspace_bytes bytes) into the slots."""
    H, K = _hk(weight)
    _same_device(weight, x=x, W_in=W_in, cu_seqlens=cu_seqlens, y=y, state_pool=state_pool, slot_idx=slot_idx,
                 bias=bias, in_proj_out=in_proj_out, workspace=workspace)
    _same_dtype(weight, x=x, W_in=W_in, y=y, state_pool=state_pool, bias=bias, in_proj_out=in_proj_out)
    if W_in.dim() != 2 or not W_in.is_contiguous() or W_in.shape[0] != 3 * H:
        raise ValueError(f"W_in must be a contiguous [{3 * H}, D] tensor")
    D = W_in.shape[1]
    N = _cu(cu_seqlens)
    T = x.shape[0]
    x_stride = _rows(x, "x", 0, D)
    y_stride = _rows(y, "y", T, H)
    io_stride = 0 if in_proj_out is None else _rows(in_proj_out, "in_proj_out", T, 3 * H)
    _dense(bias, "bias", H)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lib().lfm2sc_fused_prefill(
        _dtype_code(weight), H, K, D, _ptr(x), x_stride, T, _ptr(cu_seqlens), N,
        _ptr(W_in), _ptr(weight), _ptr(bias), _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(y), y_stride, _ptr(in_proj_out), io_stride, _ptr(workspace), ws_bytes, _stream(weight.device)))
    return y


def _span_ok(t: torch.Tensor) -> bool:
    """Every element of a (possibly strided) view lies inside its storage."""
    if t.numel() == 0:
        return True
    last = t.storage_offset() + sum((n - 1) * s for n, s in zip(t.shape, t.stride()))
    return min(t.stride()) >= 0 and last < t.untyped_storage().nbytes() // t.element_size()


def lfm2sc_conv_update(bx, weight, state_pool, slot_idx, out, windows=None, bias=None):
    """Conv update of gated inputs bx [N, H, L] (any element strides, e.g. a transposed view of token-major rows)
    into out [N, H, L] (any strides).  With `windows` ([N, L, H, K], contiguous) the pool is only read and every
    step's window is written; without, each named slot advances by the L tokens."""
    H, K = _hk(weight)
    _same_device(weight, bx=bx, state_pool=state_pool, slot_idx=slot_idx, out=out, windows=windows, bias=bias)
    _same_dtype(weight, bx=bx, state_pool=state_pool, out=out, windows=windows, bias=bias)
    if bx.dim() != 3 or out.dim() != 3 or bx.shape != out.shape or bx.shape[1] != H:
        raise ValueError(f"bx and out must both be [N, {H}, L] tensors")
    if not _span_ok(bx) or not _span_ok(out):
        raise ValueError("bx and out must be views inside their storage with non-negative strides")
    N, _, L = bx.shape
    if state_pool is None or slot_idx is None:
        raise ValueError("conv update needs a state pool and slot_idx")
    if windows is not None and (not windows.is_contiguous() or windows.numel() < N * L * H * K):
        raise ValueError(f"windows must be a contiguous [{N}, {L}, {H}, {K}] tensor")
    _dense(bias, "bias", H)
    num_slots, slot_stride = _pool_args(state_pool, slot_idx, N, H, K)
    _check(_lib.lib().lfm2sc_conv_update(
        _dtype_code(weight), H, K, N, L, _ptr(bx), bx.stride(0), bx.stride(1), bx.stride(2), _ptr(weight),
        _ptr(bias), _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(windows), _ptr(out), out.stride(0), out.stride(1), out.stride(2), _stream(weight.device)))
    return out


def abi_version() -> int:
    return int(_lib.lib().lfm2sc_abi_version())
