// api.cpp -- the exported C ABI (include/lfm2sc.h): host-side argument
// validation, error reporting and dispatch to the HIP launchers.
//
// Every check here runs before the first HIP call of an entry point, so all
// error paths can be exercised on a machine without a GPU.
#include <type_traits>
#include "lfm2sc.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fused_common.hpp"
#include "kernels.hpp"

namespace {

using namespace lfm2sc;

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return LFM2SC_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool check_mode() {
    static const bool on = [] {
        const char* e = std::getenv("LFM2SC_CHECK");
        return e != nullptr && e[0] == '1';
    }();
    return on;
}

constexpr int kMaxH = 1 << 20;
constexpr int64_t kMaxRows = (int64_t)1 << 31;   // row offsets are int32

#define TRY(expr)                       \
    do {                                \
        const int rc_ = (expr);         \
        if (rc_ != LFM2SC_OK) return rc_; \
    } while (0)

int check_common(const char* fn, int dtype, int H, int K, const void* bias) {
    if (dtype != LFM2SC_BF16 && dtype != LFM2SC_F32)
        return fail(LFM2SC_ERR_UNSUPPORTED, "%s: dtype %d is neither LFM2SC_BF16 (0) nor LFM2SC_F32 (1)", fn, dtype);
    if (H < 8 || H % 8 != 0 || H > kMaxH)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: H=%d must be a multiple of 8 in [8, %d]", fn, H, kMaxH);
    if (K < 1 || K > 4) return fail(LFM2SC_ERR_UNSUPPORTED, "%s: K=%d is not in 1..4", fn, K);
    if (bias != nullptr && !aligned(bias, 16))
        return fail(LFM2SC_ERR_ALIGNMENT, "%s: bias=%p is not 16-byte aligned", fn, bias);
    return LFM2SC_OK;
}

int check_stride(const char* fn, const char* name, int64_t stride, int64_t min) {
    if (stride < min) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: %s=%lld is below the minimum %lld", fn, name,
                                  (long long)stride, (long long)min);
    if (stride % 8 != 0) return fail(LFM2SC_ERR_ALIGNMENT, "%s: %s=%lld is not a multiple of 8 elements", fn, name,
                                     (long long)stride);
    return LFM2SC_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, uintptr_t align) {
    if (p == nullptr) return fail(LFM2SC_ERR_NULL_POINTER, "%s: %s is NULL", fn, name);
    if (!aligned(p, align)) return fail(LFM2SC_ERR_ALIGNMENT, "%s: %s=%p is not %u-byte aligned", fn, name, p,
                                        (unsigned)align);
    return LFM2SC_OK;
}

int check_pool(const char* fn, const void* pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
               int H, int K) {
    TRY(check_ptr(fn, "state_pool", pool, 16));
    TRY(check_ptr(fn, "slot_idx", slot_idx, 4));
    if (num_slots < 1) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_slots=%lld must be >= 1", fn, (long long)num_slots);
    TRY(check_stride(fn, "slot_stride", slot_stride, (int64_t)H * K));
    return LFM2SC_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(LFM2SC_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
    return ok();
}

int device_check(const char* fn, hipStream_t s, const int32_t* slot_idx, int N, int64_t num_slots, const int32_t* cu,
                 int64_t total_T, const int32_t* accept, int L) {
    if (!check_mode()) return LFM2SC_OK;
    hipError_t e;
    const int bad = check_device_preconditions(s, slot_idx, N, num_slots, cu, total_T, accept, L, &e);
    if (e != hipSuccess) return launched(fn, e);
    if (bad)
        return fail(LFM2SC_ERR_PRECONDITION, "%s: device data breaks a precondition:%s%s%s%s", fn,
                    (bad & kBadSlotRange) ? " slot index out of range;" : "",
                    (bad & kDupSlot) ? " duplicate slot index;" : "",
                    (bad & kBadCu) ? " cu_seqlens not non-decreasing within [0, total_T];" : "",
                    (bad & kBadAccept) ? " accept length outside [0, L];" : "");
    return LFM2SC_OK;
}

template <typename E>
int prefill_impl(int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T, const int32_t* cu, int N,
                 const void* weight, const void* bias, void* pool, int64_t num_slots, int64_t slot_stride,
                 const int32_t* slot_idx, void* y, int64_t y_stride, hipStream_t s) {
    PrefillArgs<E> a;
    a.in = static_cast<const E*>(in_proj); a.in_stride = in_stride; a.total_T = total_T;
    a.cu = cu; a.N = N;
    a.w = static_cast<const E*>(weight); a.bias = static_cast<const E*>(bias);
    a.pool = static_cast<E*>(pool); a.num_slots = num_slots; a.slot_stride = slot_stride; a.slot_idx = slot_idx;
    a.y = static_cast<E*>(y); a.y_stride = y_stride;
    a.H = H;
    a.sub = 0;
    a.ntiles = 0;
    return launched("lfm2sc_prefill_ragged", launch_prefill<E>(a, K, s));
}

template <typename E>
int decode_impl(int H, int K, const void* in_proj, int64_t in_stride, int N, const void* weight, const void* bias,
                void* pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx, void* y, int64_t y_stride,
                hipStream_t s) {
    DecodeArgs<E> a;
    a.in = static_cast<const E*>(in_proj); a.in_stride = in_stride; a.N = N;
    a.w = static_cast<const E*>(weight); a.bias = static_cast<const E*>(bias);
    a.pool = static_cast<E*>(pool); a.num_slots = num_slots; a.slot_stride = slot_stride; a.slot_idx = slot_idx;
    a.y = static_cast<E*>(y); a.y_stride = y_stride;
    a.H = H;
    return launched("lfm2sc_decode_step", launch_decode<E>(a, K, s));
}

template <typename E>
int verify_impl(int H, int K, const void* in_proj, int64_t in_stride, int N, int L, const void* weight,
                const void* bias, const void* pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
                void* windows, void* y, int64_t y_stride, hipStream_t s) {
    VerifyArgs<E> a;
    a.in = static_cast<const E*>(in_proj); a.in_stride = in_stride; a.N = N; a.L = L;
    a.w = static_cast<const E*>(weight); a.bias = static_cast<const E*>(bias);
    a.pool = static_cast<const E*>(pool); a.num_slots = num_slots; a.slot_stride = slot_stride;
    a.slot_idx = slot_idx;
    a.win = static_cast<E*>(windows);
    a.y = static_cast<E*>(y); a.y_stride = y_stride;
    a.H = H;
    return launched("lfm2sc_verify_window", launch_verify<E>(a, K, s));
}

template <typename E>
int commit_impl(int H, int K, const void* windows, int N, int L, const int32_t* accept, void* pool, int64_t num_slots,
                int64_t slot_stride, const int32_t* slot_idx, hipStream_t s) {
    CommitArgs<E> a;
    a.win = static_cast<const E*>(windows); a.N = N; a.L = L; a.accept = accept;
    a.pool = static_cast<E*>(pool); a.num_slots = num_slots; a.slot_stride = slot_stride; a.slot_idx = slot_idx;
    a.H = H;
    return launched("lfm2sc_commit_window", launch_commit<E>(a, K, s));
}

template <typename E>
int backward_impl(const char* fn, int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T, const int32_t* cu, int N,
                  const void* weight, const void* bias, const void* pool, int64_t num_slots, int64_t slot_stride,
                  const int32_t* slot_idx, const void* dy, int64_t dy_stride, const void* dfinal, void* din,
                  int64_t din_stride, float* dW, float* dbias, void* dinit, void* ws, hipStream_t s) {
    BackwardArgs<E> a;
    a.in = static_cast<const E*>(in_proj); a.in_stride = in_stride; a.total_T = total_T;
    a.cu = cu; a.N = N;
    a.w = static_cast<const E*>(weight); a.bias = static_cast<const E*>(bias);
    a.pool = static_cast<const E*>(pool); a.num_slots = num_slots; a.slot_stride = slot_stride; a.slot_idx = slot_idx;
    a.dy = static_cast<const E*>(dy); a.dy_stride = dy_stride;
    a.dfinal = static_cast<const E*>(dfinal);
    a.din = static_cast<E*>(din); a.din_stride = din_stride;
    a.partial = ws;
    a.dW = dW; a.dbias = dbias;
    a.dinit = static_cast<E*>(dinit);
    a.H = H;
    a.sub = 0;
    a.ntiles = 0;
    return launched(fn, launch_backward<E>(a, K, s));
}

size_t workspace_bytes(int dtype, int H, int K, int64_t total_T, int N) {
    if (N <= 0 || total_T <= 0) return 0;
    const int64_t nt = backward_partial_rows(dtype == LFM2SC_F32, H, K, total_T, N);
    const size_t bytes = (size_t)nt * (size_t)H * (size_t)(K + 1) * (size_t)backward_partial_bytes(dtype == LFM2SC_F32);
    return (bytes + 255) / 256 * 256;
}

// lfm2sc_backward and lfm2sc_backward_noalloc: the same validation; the second takes its workspace from the
// library's fixed device array instead of the caller.
int backward_entry(const char* fn, int dtype, int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T,
                   const int32_t* cu_seqlens, int num_seqs, const void* weight, const void* bias,
                   const void* init_state_pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
                   const void* dy, int64_t dy_stride, const void* d_final_state, void* d_in_proj, int64_t din_stride,
                   float* dW, float* dbias, void* d_init_state, void* workspace, size_t workspace_bytes_, bool noalloc,
                   void* stream) {
    TRY(check_common(fn, dtype, H, K, bias));
    if (num_seqs < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d is negative", fn, num_seqs);
    if (total_T < 0 || total_T >= kMaxRows)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: total_T=%lld outside [0, 2^31)", fn, (long long)total_T);
    TRY(check_stride(fn, "in_stride", in_stride, 3 * (int64_t)H));
    TRY(check_stride(fn, "dy_stride", dy_stride, H));
    TRY(check_stride(fn, "din_stride", din_stride, 3 * (int64_t)H));
    TRY(check_ptr(fn, "dW", dW, 4));
    if (dbias != nullptr && !aligned(dbias, 4)) return fail(LFM2SC_ERR_ALIGNMENT, "%s: dbias is not 4-byte aligned", fn);
    if (d_final_state != nullptr && !aligned(d_final_state, 16))
        return fail(LFM2SC_ERR_ALIGNMENT, "%s: d_final_state is not 16-byte aligned", fn);
    if (d_init_state != nullptr && !aligned(d_init_state, 16))
        return fail(LFM2SC_ERR_ALIGNMENT, "%s: d_init_state is not 16-byte aligned", fn);
    const bool work = num_seqs > 0 && total_T > 0;
    if (num_seqs > 0) TRY(check_ptr(fn, "cu_seqlens", cu_seqlens, 4));
    if (work) {
        TRY(check_ptr(fn, "in_proj", in_proj, 16));
        TRY(check_ptr(fn, "weight", weight, 16));
        TRY(check_ptr(fn, "dy", dy, 16));
        TRY(check_ptr(fn, "d_in_proj", d_in_proj, 16));
        if (init_state_pool != nullptr)
            TRY(check_pool(fn, init_state_pool, num_slots, slot_stride, slot_idx, H, K));
        if (ragged_tiles_bound(total_T, num_seqs) >= (1 << 30))
            return fail(LFM2SC_ERR_BAD_SHAPE, "%s: too many sequences/tokens for one launch", fn);
        const size_t need = workspace_bytes(dtype, H, K, total_T, num_seqs);
        if (noalloc) {
            if (need > noalloc_scratch_bytes())
                return fail(LFM2SC_ERR_WORKSPACE,
                            "%s: this call needs %zu bytes of workspace; the no-alloc entry point holds %zu "
                            "(LFM2SC_NOALLOC_SCRATCH_BYTES): use lfm2sc_backward with a caller workspace",
                            fn, need, noalloc_scratch_bytes());
        } else {
            if (workspace == nullptr || workspace_bytes_ < need)
                return fail(LFM2SC_ERR_WORKSPACE, "%s: workspace %p of %zu bytes, %zu needed", fn, workspace,
                            workspace_bytes_, need);
            if (!aligned(workspace, 16))
                return fail(LFM2SC_ERR_ALIGNMENT, "%s: workspace is not 16-byte aligned", fn);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (noalloc && work) {
        const hipError_t e = noalloc_scratch(s, &workspace);
        if (e != hipSuccess) return launched(fn, e);
    }
    if (num_seqs > 0)
        TRY(device_check(fn, s, (work && init_state_pool) ? slot_idx : nullptr, num_seqs, num_slots, cu_seqlens,
                         total_T, nullptr, 0));
    // With no token the launch still runs the reduction over zero windows (dW = 0, dbias = 0) and, when asked,
    // writes d_init_state = d_final_state (or 0) for every (empty) sequence.
    const int64_t T_eff = work ? total_T : 0;
    if (dtype == LFM2SC_BF16)
        return backward_impl<uint16_t>(fn, H, K, in_proj, in_stride, T_eff, cu_seqlens, num_seqs, weight, bias,
                                       init_state_pool, num_slots, slot_stride, slot_idx, dy, dy_stride, d_final_state,
                                       d_in_proj, din_stride, dW, dbias, d_init_state, workspace, s);
    return backward_impl<float>(fn, H, K, in_proj, in_stride, T_eff, cu_seqlens, num_seqs, weight, bias, init_state_pool,
                                num_slots, slot_stride, slot_idx, dy, dy_stride, d_final_state, d_in_proj, din_stride,
                                dW, dbias, d_init_state, workspace, s);
}

}  // namespace

extern "C" {

int lfm2sc_abi_version(void) { return LFM2SC_ABI_VERSION; }

const char* lfm2sc_last_error(void) { return g_err; }

const char* lfm2sc_status_string(int status) {
    switch (status) {
        case LFM2SC_OK: return "LFM2SC_OK";
        case LFM2SC_ERR_NULL_POINTER: return "LFM2SC_ERR_NULL_POINTER";
        case LFM2SC_ERR_BAD_SHAPE: return "LFM2SC_ERR_BAD_SHAPE";
        case LFM2SC_ERR_ALIGNMENT: return "LFM2SC_ERR_ALIGNMENT";
        case LFM2SC_ERR_UNSUPPORTED: return "LFM2SC_ERR_UNSUPPORTED";
        case LFM2SC_ERR_WORKSPACE: return "LFM2SC_ERR_WORKSPACE";
        case LFM2SC_ERR_PRECONDITION: return "LFM2SC_ERR_PRECONDITION";
        case LFM2SC_ERR_HIP: return "LFM2SC_ERR_HIP";
    }
    return "LFM2SC_UNKNOWN_STATUS";
}

int lfm2sc_prefill_ragged(int dtype, int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T,
                          const int32_t* cu_seqlens, int num_seqs, const void* weight, const void* bias,
                          void* state_pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx, void* y,
                          int64_t y_stride, void* stream) {
    const char* fn = "lfm2sc_prefill_ragged";
    TRY(check_common(fn, dtype, H, K, bias));
    if (num_seqs < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d is negative", fn, num_seqs);
    if (total_T < 0 || total_T >= kMaxRows)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: total_T=%lld outside [0, 2^31)", fn, (long long)total_T);
    TRY(check_stride(fn, "in_stride", in_stride, 3 * (int64_t)H));
    TRY(check_stride(fn, "y_stride", y_stride, H));
    if (num_seqs == 0 || total_T == 0) return ok();   // no token: nothing computed, no state changes
    TRY(check_ptr(fn, "in_proj", in_proj, 16));
    TRY(check_ptr(fn, "cu_seqlens", cu_seqlens, 4));
    TRY(check_ptr(fn, "weight", weight, 16));
    TRY(check_ptr(fn, "y", y, 16));
    if (state_pool != nullptr) TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
    if (ragged_tiles_bound(total_T, num_seqs) >= (1 << 30))
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: too many sequences/tokens for one launch", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, state_pool ? slot_idx : nullptr, num_seqs, num_slots, cu_seqlens, total_T, nullptr, 0));
    if (dtype == LFM2SC_BF16)
        return prefill_impl<uint16_t>(H, K, in_proj, in_stride, total_T, cu_seqlens, num_seqs, weight, bias,
                                      state_pool, num_slots, slot_stride, slot_idx, y, y_stride, s);
    return prefill_impl<float>(H, K, in_proj, in_stride, total_T, cu_seqlens, num_seqs, weight, bias, state_pool,
                               num_slots, slot_stride, slot_idx, y, y_stride, s);
}

int lfm2sc_decode_step(int dtype, int H, int K, const void* in_proj, int64_t in_stride, int num_seqs,
                       const void* weight, const void* bias, void* state_pool, int64_t num_slots, int64_t slot_stride,
                       const int32_t* slot_idx, void* y, int64_t y_stride, void* stream) {
    const char* fn = "lfm2sc_decode_step";
    TRY(check_common(fn, dtype, H, K, bias));
    if (num_seqs < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d is negative", fn, num_seqs);
    TRY(check_stride(fn, "in_stride", in_stride, 3 * (int64_t)H));
    TRY(check_stride(fn, "y_stride", y_stride, H));
    if (num_seqs == 0) return ok();
    TRY(check_ptr(fn, "in_proj", in_proj, 16));
    TRY(check_ptr(fn, "weight", weight, 16));
    TRY(check_ptr(fn, "y", y, 16));
    TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, slot_idx, num_seqs, num_slots, nullptr, 0, nullptr, 0));
    if (dtype == LFM2SC_BF16)
        return decode_impl<uint16_t>(H, K, in_proj, in_stride, num_seqs, weight, bias, state_pool, num_slots,
                                     slot_stride, slot_idx, y, y_stride, s);
    return decode_impl<float>(H, K, in_proj, in_stride, num_seqs, weight, bias, state_pool, num_slots, slot_stride,
                              slot_idx, y, y_stride, s);
}

int lfm2sc_verify_window(int dtype, int H, int K, const void* in_proj, int64_t in_stride, int num_seqs, int L,
                         const void* weight, const void* bias, const void* state_pool, int64_t num_slots,
                         int64_t slot_stride, const int32_t* slot_idx, void* windows, void* y, int64_t y_stride,
                         void* stream) {
    const char* fn = "lfm2sc_verify_window";
    TRY(check_common(fn, dtype, H, K, bias));
    if (windows == nullptr)
        return fail(LFM2SC_ERR_NULL_POINTER, "%s: the per-step window tape is required (windows is NULL)", fn);
    if (num_seqs < 0 || L < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d, L=%d must be >= 0", fn, num_seqs, L);
    if ((int64_t)num_seqs * L >= kMaxRows) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs*L too large", fn);
    TRY(check_stride(fn, "in_stride", in_stride, 3 * (int64_t)H));
    TRY(check_stride(fn, "y_stride", y_stride, H));
    if (num_seqs == 0 || L == 0) return ok();
    TRY(check_ptr(fn, "windows", windows, 16));
    TRY(check_ptr(fn, "in_proj", in_proj, 16));
    TRY(check_ptr(fn, "weight", weight, 16));
    TRY(check_ptr(fn, "y", y, 16));
    TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, slot_idx, num_seqs, num_slots, nullptr, 0, nullptr, 0));
    if (dtype == LFM2SC_BF16)
        return verify_impl<uint16_t>(H, K, in_proj, in_stride, num_seqs, L, weight, bias, state_pool, num_slots,
                                     slot_stride, slot_idx, windows, y, y_stride, s);
    return verify_impl<float>(H, K, in_proj, in_stride, num_seqs, L, weight, bias, state_pool, num_slots, slot_stride,
                              slot_idx, windows, y, y_stride, s);
}

int lfm2sc_commit_window(int dtype, int H, int K, const void* windows, int num_seqs, int L, const int32_t* accept_len,
                         void* state_pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
                         void* stream) {
    const char* fn = "lfm2sc_commit_window";
    TRY(check_common(fn, dtype, H, K, nullptr));
    if (num_seqs < 0 || L < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d, L=%d must be >= 0", fn, num_seqs, L);
    if (num_seqs == 0 || L == 0) return ok();   // with L = 0 every accept length is 0: nothing to install
    TRY(check_ptr(fn, "windows", windows, 16));
    TRY(check_ptr(fn, "accept_len", accept_len, 4));
    TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, slot_idx, num_seqs, num_slots, nullptr, 0, accept_len, L));
    if (dtype == LFM2SC_BF16)
        return commit_impl<uint16_t>(H, K, windows, num_seqs, L, accept_len, state_pool, num_slots, slot_stride,
                                     slot_idx, s);
    return commit_impl<float>(H, K, windows, num_seqs, L, accept_len, state_pool, num_slots, slot_stride, slot_idx, s);
}

size_t lfm2sc_backward_workspace_bytes(int dtype, int H, int K, int64_t total_T, int num_seqs) {
    if (dtype != LFM2SC_BF16 && dtype != LFM2SC_F32) return 0;
    if (H < 8 || H % 8 != 0 || H > kMaxH || K < 1 || K > 4) return 0;
    if (total_T < 0 || total_T >= kMaxRows || num_seqs < 0) return 0;
    return workspace_bytes(dtype, H, K, total_T, num_seqs);
}

int lfm2sc_backward(int dtype, int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T,
                    const int32_t* cu_seqlens, int num_seqs, const void* weight, const void* bias,
                    const void* init_state_pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
                    const void* dy, int64_t dy_stride, const void* d_final_state, void* d_in_proj, int64_t din_stride,
                    float* dW, float* dbias, void* d_init_state, void* workspace, size_t workspace_bytes_,
                    void* stream) {
    return backward_entry("lfm2sc_backward", dtype, H, K, in_proj, in_stride, total_T, cu_seqlens, num_seqs, weight,
                          bias, init_state_pool, num_slots, slot_stride, slot_idx, dy, dy_stride, d_final_state,
                          d_in_proj, din_stride, dW, dbias, d_init_state, workspace, workspace_bytes_, false, stream);
}

int lfm2sc_backward_noalloc(int dtype, int H, int K, const void* in_proj, int64_t in_stride, int64_t total_T,
                            const int32_t* cu_seqlens, int num_seqs, const void* weight, const void* bias,
                            const void* init_state_pool, int64_t num_slots, int64_t slot_stride,
                            const int32_t* slot_idx, const void* dy, int64_t dy_stride, const void* d_final_state,
                            void* d_in_proj, int64_t din_stride, float* dW, float* dbias, void* d_init_state,
                            void* stream) {
    return backward_entry("lfm2sc_backward_noalloc", dtype, H, K, in_proj, in_stride, total_T, cu_seqlens, num_seqs,
                          weight, bias, init_state_pool, num_slots, slot_stride, slot_idx, dy, dy_stride,
                          d_final_state, d_in_proj, din_stride, dW, dbias, d_init_state, nullptr, 0, true, stream);
}

int lfm2sc_conv_update(int dtype, int H, int K, int num_seqs, int L, const void* bx, int64_t bx_stride_n,
                       int64_t bx_stride_h, int64_t bx_stride_t, const void* weight, const void* bias,
                       void* state_pool, int64_t num_slots, int64_t slot_stride, const int32_t* slot_idx,
                       void* windows, void* out, int64_t out_stride_n, int64_t out_stride_h, int64_t out_stride_t,
                       void* stream) {
    const char* fn = "lfm2sc_conv_update";
    TRY(check_common(fn, dtype, H, K, bias));
    if (num_seqs < 0 || L < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d, L=%d", fn, num_seqs, L);
    if ((int64_t)num_seqs * L >= kMaxRows) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs*L too large", fn);
    if (bx_stride_n < 0 || bx_stride_h < 0 || bx_stride_t < 0 || out_stride_n < 0 || out_stride_h < 0 ||
        out_stride_t < 0)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: negative stride", fn);
    if (num_seqs == 0 || L == 0) return ok();
    const uintptr_t esz = dtype == LFM2SC_BF16 ? 2 : 4;
    TRY(check_ptr(fn, "bx", bx, esz));
    TRY(check_ptr(fn, "out", out, esz));
    TRY(check_ptr(fn, "weight", weight, 16));
    TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
    if (windows != nullptr && !aligned(windows, 16))
        return fail(LFM2SC_ERR_ALIGNMENT, "%s: windows is not 16-byte aligned", fn);
    // channel-contiguous (the transposed view of token-major rows), token-contiguous (a dense [N][H][L]
    // tensor), or neither
    const bool chan_vec = bx_stride_h == 1 && out_stride_h == 1 && bx_stride_n % 8 == 0 && bx_stride_t % 8 == 0 &&
                          out_stride_n % 8 == 0 && out_stride_t % 8 == 0 && aligned(bx, 16) && aligned(out, 16);
    const bool rows = bx_stride_t == 1 && out_stride_t == 1;
    const bool rows_vec = rows && L % 8 == 0 && bx_stride_h % 8 == 0 && out_stride_h % 8 == 0 &&
                          bx_stride_n % 8 == 0 && out_stride_n % 8 == 0 && aligned(bx, 16) && aligned(out, 16);
    const ConvLayout lay = chan_vec ? ConvLayout::kChannelsVec
                                    : rows_vec ? ConvLayout::kRowsVec : rows ? ConvLayout::kRows : ConvLayout::kGeneric;
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, slot_idx, num_seqs, num_slots, nullptr, 0, nullptr, 0));
    auto fill = [&](auto* tag) {
        using E = std::remove_pointer_t<decltype(tag)>;
        ConvUpdateArgs<E> a;
        a.bx = static_cast<const E*>(bx); a.bx_sn = bx_stride_n; a.bx_sh = bx_stride_h; a.bx_st = bx_stride_t;
        a.N = num_seqs; a.L = L;
        a.w = static_cast<const E*>(weight); a.bias = static_cast<const E*>(bias);
        a.pool = static_cast<E*>(state_pool); a.num_slots = num_slots; a.slot_stride = slot_stride;
        a.slot_idx = slot_idx;
        a.win = static_cast<E*>(windows);
        a.out = static_cast<E*>(out); a.out_sn = out_stride_n; a.out_sh = out_stride_h; a.out_st = out_stride_t;
        a.H = H;
        return launched(fn, launch_conv_update<E>(a, K, lay, s));
    };
    if (dtype == LFM2SC_BF16) return fill(static_cast<uint16_t*>(nullptr));
    return fill(static_cast<float*>(nullptr));
}

size_t lfm2sc_fused_prefill_workspace_bytes(int dtype, int H, int K, int num_seqs, int with_pool) {
    if (dtype != LFM2SC_BF16 || H < 64 || H % 64 != 0 || H > kMaxH || K < 1 || K > 4 || num_seqs < 0) return 0;
    if (!with_pool) return 0;
    return ((size_t)num_seqs * (size_t)H * (size_t)K * 2 + 255) / 256 * 256;
}

int lfm2sc_fused_prefill_plan(int H, int K, int D, int64_t total_T) {
    if (H < 64 || H % 64 != 0 || H > kMaxH || K < 1 || K > 4 || D < fused_depth_multiple() ||
        D % fused_depth_multiple() != 0 || (int64_t)3 * H * D * 2 >= ((int64_t)1 << 31) || total_T < 0 ||
        total_T >= kMaxRows)
        return -LFM2SC_ERR_BAD_SHAPE;
    if (total_T == 0) return 0;
    return fused_plan(K, total_T, H, D);
}

int lfm2sc_fused_prefill(int dtype, int H, int K, int D, const void* x, int64_t x_stride, int64_t total_T,
                         const int32_t* cu_seqlens, int num_seqs, const void* W_in, const void* weight,
                         const void* bias, void* state_pool, int64_t num_slots, int64_t slot_stride,
                         const int32_t* slot_idx, void* y, int64_t y_stride, void* in_proj_out, int64_t io_stride,
                         void* workspace, size_t workspace_bytes_, void* stream) {
    const char* fn = "lfm2sc_fused_prefill";
    TRY(check_common(fn, dtype, H, K, bias));
    if (dtype != LFM2SC_BF16) return fail(LFM2SC_ERR_UNSUPPORTED, "%s: only LFM2SC_BF16 is supported", fn);
    if (H % 64 != 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: H=%d is not a multiple of 64", fn, H);
    if (D < fused_depth_multiple() || D % fused_depth_multiple() != 0)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: D=%d is not a positive multiple of %d", fn, D, fused_depth_multiple());
    if ((int64_t)3 * H * D * 2 >= kMaxRows)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: W_in of 3H x D = %d x %d is 2 GiB or more", fn, 3 * H, D);
    if (num_seqs < 0) return fail(LFM2SC_ERR_BAD_SHAPE, "%s: num_seqs=%d is negative", fn, num_seqs);
    if (total_T < 0 || total_T >= kMaxRows)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: total_T=%lld outside [0, 2^31)", fn, (long long)total_T);
    TRY(check_stride(fn, "x_stride", x_stride, D));
    if (x_stride * 2 * 256 >= kMaxRows)
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: x_stride=%lld too large", fn, (long long)x_stride);
    TRY(check_stride(fn, "y_stride", y_stride, H));
    if (in_proj_out != nullptr) TRY(check_stride(fn, "io_stride", io_stride, 3 * (int64_t)H));
    if (num_seqs == 0 || total_T == 0) return ok();   // no token: nothing computed, no state changes
    TRY(check_ptr(fn, "x", x, 16));
    TRY(check_ptr(fn, "cu_seqlens", cu_seqlens, 4));
    TRY(check_ptr(fn, "W_in", W_in, 16));
    TRY(check_ptr(fn, "weight", weight, 16));
    TRY(check_ptr(fn, "y", y, 16));
    if (in_proj_out != nullptr) TRY(check_ptr(fn, "in_proj_out", in_proj_out, 16));
    if (state_pool != nullptr) {
        TRY(check_pool(fn, state_pool, num_slots, slot_stride, slot_idx, H, K));
        const size_t need = lfm2sc_fused_prefill_workspace_bytes(dtype, H, K, num_seqs, 1);
        if (workspace == nullptr || workspace_bytes_ < need)
            return fail(LFM2SC_ERR_WORKSPACE, "%s: workspace %p of %zu bytes, %zu needed", fn, workspace,
                        workspace_bytes_, need);
        if (!aligned(workspace, 16)) return fail(LFM2SC_ERR_ALIGNMENT, "%s: workspace is not 16-byte aligned", fn);
    }
    if (fused_tiles(total_T, H, K) >= (1 << 30))
        return fail(LFM2SC_ERR_BAD_SHAPE, "%s: too many tokens for one launch", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    TRY(device_check(fn, s, state_pool ? slot_idx : nullptr, num_seqs, num_slots, cu_seqlens, total_T, nullptr, 0));
    FusedArgs a;
    a.x = static_cast<const uint16_t*>(x); a.x_stride = x_stride; a.total_T = total_T; a.D = D;
    a.W = static_cast<const uint16_t*>(W_in);
    a.cu = cu_seqlens; a.N = num_seqs;
    a.w = static_cast<const uint16_t*>(weight); a.bias = static_cast<const uint16_t*>(bias);
    a.pool = static_cast<uint16_t*>(state_pool); a.num_slots = num_slots; a.slot_stride = slot_stride;
    a.slot_idx = slot_idx;
    a.y = static_cast<uint16_t*>(y); a.y_stride = y_stride;
    a.io = static_cast<uint16_t*>(in_proj_out); a.io_stride = io_stride;
    a.fin = state_pool != nullptr ? static_cast<uint16_t*>(workspace) : nullptr;
    a.H = H;
    a.tiles_m = a.tiles_n = 0;
    return launched(fn, launch_fused_prefill(a, K, s));
}

}  // extern "C\"
