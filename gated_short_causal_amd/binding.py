"""Python binding of the C ABI: the same entry-point names, taking torch tensors.

Argument marshalling only -- device pointers, strides, sizes and the current
HIP stream are read from the tensors and handed to liblfm2sc.so; every step of
the computation runs in the library's HIP kernels.  Outputs are caller-owned
tensors, written in place, exactly as the C calls do.

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


def _rows(t: torch.Tensor, name: str):
    """(row stride) of a 2-D row-major tensor with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride, got shape {tuple(t.shape)} strides {t.stride()}")
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
    return pool.stride(0)


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _hk(weight: torch.Tensor):
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [H, K] tensor")
    return weight.shape[0], weight.shape[1]


def lfm2sc_prefill_ragged(in_proj, cu_seqlens, weight, y, state_pool=None, slot_idx=None, bias=None):
    H, K = _hk(weight)
    _i32(cu_seqlens, "cu_seqlens"); _i32(slot_idx, "slot_idx")
    num_slots = slot_stride = 0
    if state_pool is not None:
        slot_stride = _pool_stride(state_pool, H, K)
        num_slots = state_pool.shape[0]
    _check(_lib.lib().lfm2sc_prefill_ragged(
        _dtype_code(weight), H, K, _ptr(in_proj), _rows(in_proj, "in_proj"), in_proj.shape[0],
        _ptr(cu_seqlens), cu_seqlens.numel() - 1, _ptr(weight), _ptr(bias),
        _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(y), _rows(y, "y"), _stream(in_proj.device)))
    return y


def lfm2sc_decode_step(in_proj, weight, state_pool, slot_idx, y, bias=None):
    H, K = _hk(weight)
    _i32(slot_idx, "slot_idx")
    _check(_lib.lib().lfm2sc_decode_step(
        _dtype_code(weight), H, K, _ptr(in_proj), _rows(in_proj, "in_proj"), slot_idx.numel(),
        _ptr(weight), _ptr(bias), _ptr(state_pool), state_pool.shape[0], _pool_stride(state_pool, H, K),
        _ptr(slot_idx), _ptr(y), _rows(y, "y"), _stream(in_proj.device)))
    return y


def lfm2sc_verify_window(in_proj, weight, state_pool, slot_idx, L, windows, y, bias=None):
    H, K = _hk(weight)
    _i32(slot_idx, "slot_idx")
    N = slot_idx.numel()
    if windows is not None and (not windows.is_contiguous() or windows.numel() < N * L * H * K):
        raise ValueError(f"windows must be a contiguous [{N}, {L}, {H}, {K}] tensor")
    _check(_lib.lib().lfm2sc_verify_window(
        _dtype_code(weight), H, K, _ptr(in_proj), _rows(in_proj, "in_proj"), N, L,
        _ptr(weight), _ptr(bias), _ptr(state_pool), state_pool.shape[0], _pool_stride(state_pool, H, K),
        _ptr(slot_idx), _ptr(windows), _ptr(y), _rows(y, "y"), _stream(in_proj.device)))
    return y, windows


def lfm2sc_commit_window(windows, accept_len, state_pool, slot_idx):
    N, L, H, K = windows.shape
    if not windows.is_contiguous():
        raise ValueError("windows must be contiguous [N, L, H, K]")
    _i32(accept_len, "accept_len"); _i32(slot_idx, "slot_idx")
    _check(_lib.lib().lfm2sc_commit_window(
        _dtype_code(windows), H, K, _ptr(windows), N, L, _ptr(accept_len),
        _ptr(state_pool), state_pool.shape[0], _pool_stride(state_pool, H, K), _ptr(slot_idx),
        _stream(windows.device)))
    return state_pool


def lfm2sc_backward_workspace_bytes(dtype, H, K, total_T, num_seqs) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().lfm2sc_backward_workspace_bytes(code, H, K, total_T, num_seqs))


def lfm2sc_backward(in_proj, cu_seqlens, weight, dy, d_in_proj, dW, workspace,
                    init_state_pool=None, slot_idx=None, bias=None, d_final_state=None, dbias=None,
                    d_init_state=None):
    """Backward of lfm2sc_prefill_ragged.  Writes d_in_proj (dB | dC | dxv), dW (fp32), and when given dbias
    (fp32 [H]) and d_init_state ([N, H, K], I/O dtype).  d_final_state: gradient of the final states [N, H, K]."""
    H, K = _hk(weight)
    N = cu_seqlens.numel() - 1
    _i32(cu_seqlens, "cu_seqlens"); _i32(slot_idx, "slot_idx")
    if dW.dtype != torch.float32 or not dW.is_contiguous():
        raise TypeError("dW must be a contiguous float32 [H, K] tensor")
    if dbias is not None and (dbias.dtype != torch.float32 or not dbias.is_contiguous()):
        raise TypeError("dbias must be a contiguous float32 [H] tensor")
    for name, t in (("d_final_state", d_final_state), ("d_init_state", d_init_state)):
        if t is not None and (t.dtype != weight.dtype or not t.is_contiguous() or t.numel() < N * H * K):
            raise ValueError(f"{name} must be a contiguous [{N}, {H}, {K}] tensor of the I/O dtype")
    num_slots = slot_stride = 0
    if init_state_pool is not None:
        slot_stride = _pool_stride(init_state_pool, H, K)
        num_slots = init_state_pool.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lib().lfm2sc_backward(
        _dtype_code(weight), H, K, _ptr(in_proj), _rows(in_proj, "in_proj"), in_proj.shape[0],
        _ptr(cu_seqlens), N, _ptr(weight), _ptr(bias),
        _ptr(init_state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(dy), _rows(dy, "dy"), _ptr(d_final_state), _ptr(d_in_proj), _rows(d_in_proj, "d_in_proj"), _ptr(dW),
        _ptr(dbias), _ptr(d_init_state), _ptr(workspace), ws_bytes, _stream(in_proj.device)))
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
    if W_in.dim() != 2 or not W_in.is_contiguous() or W_in.shape[0] != 3 * H:
        raise ValueError(f"W_in must be a contiguous [{3 * H}, D] tensor")
    D = W_in.shape[1]
    _i32(cu_seqlens, "cu_seqlens"); _i32(slot_idx, "slot_idx")
    num_slots = slot_stride = 0
    if state_pool is not None:
        slot_stride = _pool_stride(state_pool, H, K)
        num_slots = state_pool.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    io_stride = 0 if in_proj_out is None else _rows(in_proj_out, "in_proj_out")
    _check(_lib.lib().lfm2sc_fused_prefill(
        _dtype_code(weight), H, K, D, _ptr(x), _rows(x, "x"), x.shape[0], _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        _ptr(W_in), _ptr(weight), _ptr(bias), _ptr(state_pool), num_slots, slot_stride, _ptr(slot_idx),
        _ptr(y), _rows(y, "y"), _ptr(in_proj_out), io_stride, _ptr(workspace), ws_bytes, _stream(x.device)))
    return y


def lfm2sc_conv_update(bx, weight, state_pool, slot_idx, out, windows=None, bias=None):
    """Conv update of gated inputs bx [N, H, L] (any element strides, e.g. a transposed view of token-major rows)
    into out [N, H, L] (any strides).  With `windows` ([N, L, H, K], contiguous) the pool is only read and every
    step's window is written; without, each named slot advances by the L tokens."""
    H, K = _hk(weight)
    _i32(slot_idx, "slot_idx")
    if bx.dim() != 3 or out.dim() != 3 or bx.shape != out.shape or bx.shape[1] != H:
        raise ValueError(f"bx and out must both be [N, {H}, L] tensors")
    N, _, L = bx.shape
    if windows is not None and (not windows.is_contiguous() or windows.numel() < N * L * H * K):
        raise ValueError(f"windows must be a contiguous [{N}, {L}, {H}, {K}] tensor")
    _check(_lib.lib().lfm2sc_conv_update(
        _dtype_code(weight), H, K, N, L, _ptr(bx), bx.stride(0), bx.stride(1), bx.stride(2), _ptr(weight),
        _ptr(bias), _ptr(state_pool), state_pool.shape[0], _pool_stride(state_pool, H, K), _ptr(slot_idx),
        _ptr(windows), _ptr(out), out.stride(0), out.stride(1), out.stride(2), _stream(bx.device)))
    return out


def abi_version() -> int:
    return int(_lib.lib().lfm2sc_abi_version())
