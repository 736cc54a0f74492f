// kernels.hpp -- argument blocks and launchers of the ShortConv kernels.
// Host-side only declarations; definitions live in fwd.hip / bwd.hip / check.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lfm2sc {

template <typename E>
struct PrefillArgs {
    const E* in; int64_t in_stride; int64_t total_T;
    const int32_t* cu; int N;
    const E* w; const E* bias;
    E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    E* y; int64_t y_stride;
    int H;
    int sub;      // tokens per wave window (a workgroup window is 4 * sub); set by the launcher
    int ntiles;   // number of workgroup windows; set by the launcher
};

template <typename E>
struct DecodeArgs {
    const E* in; int64_t in_stride; int N;
    const E* w; const E* bias;
    E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    E* y; int64_t y_stride;
    int H;
};

template <typename E>
struct VerifyArgs {
    const E* in; int64_t in_stride; int N; int L;
    const E* w; const E* bias;
    const E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    E* win;
    E* y; int64_t y_stride;
    int H;
};

template <typename E>
struct CommitArgs {
    const E* win; int N; int L; const int32_t* accept;
    E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    int H;
};

template <typename E>
struct BackwardArgs {
    const E* in; int64_t in_stride; int64_t total_T;
    const int32_t* cu; int N;
    const E* w; const E* bias;
    const E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    const E* dy; int64_t dy_stride;
    const E* dfinal;  // [N][H][K] gradient of the final states, or nullptr
    E* din; int64_t din_stride;
    void* partial;    // [ntiles][H][K+1] per-window dW/dbias sums (fp32 for bf16 I/O, fp64 for fp32 I/O)
    float* dW;        // [H][K]
    float* dbias;     // [H] or nullptr
    E* dinit;         // [N][H][K] gradient of the initial states, or nullptr
    int H;
    int sub;
    int ntiles;
};

// Conv update of gated inputs bx[n][h][t] (element strides sn, sh, st) into
// out[n][h][t]; tape win [N][L][H][K] or nullptr (then the slot advances).
template <typename E>
struct ConvUpdateArgs {
    const E* bx; int64_t bx_sn, bx_sh, bx_st;
    int N, L;
    const E* w; const E* bias;
    E* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    E* win;
    E* out; int64_t out_sn, out_sh, out_st;
    int H;
};
// Memory layout of bx and out (both): channel stride 1 (with 16-byte aligned
// rows: Vec), token stride 1 (Vec: L and the channel and batch strides are
// multiples of 8 elements, bases 16-byte aligned), or anything else.
enum class ConvLayout { kChannelsVec, kRowsVec, kRows, kGeneric };
template <typename E> hipError_t launch_conv_update(const ConvUpdateArgs<E>& a, int K, ConvLayout lay, hipStream_t s);

// Fused in_proj GEMM + ShortConv forward (bf16 only).  x [total_T][x_stride]
// (D used), W [3H][D]; y [total_T][y_stride]; io: optional in_proj output
// [total_T][io_stride] (B | C | xv, bf16); fin: [N][H][K] staging for the final
// states when a pool is given (then installed into the slots), else nullptr.
struct FusedArgs {
    const uint16_t* x; int64_t x_stride; int64_t total_T; int D;
    const uint16_t* W;
    const int32_t* cu; int N;
    const uint16_t* w; const uint16_t* bias;
    uint16_t* pool; int64_t num_slots; int64_t slot_stride; const int32_t* slot_idx;
    uint16_t* y; int64_t y_stride;
    uint16_t* io; int64_t io_stride;
    uint16_t* fin;
    int H;
    int tiles_m, tiles_n;   // set by the launcher
};
hipError_t launch_fused_prefill(const FusedArgs& a, int K, hipStream_t s);
// Tiles of a fused launch (host-side size checks).
int64_t fused_tiles(int64_t total_T, int H, int K);
// D must be a positive multiple of this (the reduction's stage depth times its ring depth).
int fused_depth_multiple();

// Rows of dW/dbias partials (one per workgroup window, H*(K+1) elements each)
// a backward launch of these sizes writes to its workspace, and the bytes of
// one partial element; the launcher and the workspace-size query share this.
int64_t backward_partial_rows(int dtype_is_f32, int H, int K, int64_t total_T, int N);
int backward_partial_bytes(int dtype_is_f32);
// Upper bound on ragged windows for any tiling (host-side size checks).
int64_t ragged_tiles_bound(int64_t total_T, int N);

template <typename E> hipError_t launch_prefill(const PrefillArgs<E>& a, int K, hipStream_t s);
template <typename E> hipError_t launch_decode(const DecodeArgs<E>& a, int K, hipStream_t s);
template <typename E> hipError_t launch_verify(const VerifyArgs<E>& a, int K, hipStream_t s);
template <typename E> hipError_t launch_commit(const CommitArgs<E>& a, int K, hipStream_t s);
template <typename E> hipError_t launch_backward(const BackwardArgs<E>& a, int K, hipStream_t s);

// The fixed device array behind lfm2sc_backward_noalloc: its size, and its
// address on the device of `stream` (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t stream, void** out);

// Debug precondition checks (LFM2SC_CHECK=1).  Each returns 0 when the device
// data satisfies the precondition, a nonzero mask otherwise; synchronises `s`.
enum CheckBits { kBadSlotRange = 1, kDupSlot = 2, kBadCu = 4, kBadAccept = 8 };
int check_device_preconditions(hipStream_t s, const int32_t* slot_idx, int N, int64_t num_slots,
                               const int32_t* cu, int64_t total_T,
                               const int32_t* accept, int L, hipError_t* err);

}  // namespace lfm2sc
