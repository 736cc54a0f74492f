"""MI355X-native LFM2 gated short causal convolution (ShortConv).

The computation lives in liblfm2sc.so (hand-written HIP kernels for gfx950
behind the C ABI of include/lfm2sc.h); this package only loads it and
marshals torch tensors into its calls.  Build the library with
``python -m gated_short_causal_amd.build``.
"""
from .binding import (  # noqa: F401
    LFM2SC_BF16,
    LFM2SC_F32,
    Lfm2scError,
    abi_version,
    lfm2sc_backward,
    lfm2sc_backward_noalloc,
    lfm2sc_backward_workspace_bytes,
    lfm2sc_commit_window,
    lfm2sc_conv_update,
    lfm2sc_decode_step,
    lfm2sc_fused_prefill,
    lfm2sc_fused_prefill_plan,
    lfm2sc_fused_prefill_workspace_bytes,
    lfm2sc_prefill_ragged,
    lfm2sc_verify_window,
)
