// check.hip -- optional device-side precondition checks (LFM2SC_CHECK=1).
//
// The kernels of this library never read or write outside the buffers the
// size arguments describe, whatever the device-side index data holds; these
// checks only turn bad index data into an error code instead of silently
// skipped or wrong work.  They synchronise the stream, so they are for
// debugging only.  The result travels through one device flag per process,
// so a process-wide lock keeps each call's reset, checks and read-back
// together: calls from several host threads take turns.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace lfm2sc {

__device__ int g_check_flags;

__global__ void check_reset_kernel() {
    if (threadIdx.x == 0) g_check_flags = 0;
}

__global__ void check_slots_kernel(const int32_t* __restrict__ slot, int N, int64_t num_slots) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int32_t s = slot[i];
    int bad = 0;
    if (s < 0 || (int64_t)s >= num_slots) bad |= kBadSlotRange;
    for (int j = 0; j < i; ++j)
        if (slot[j] == s) { bad |= kDupSlot; break; }
    if (bad) atomicOr(&g_check_flags, bad);
}

__global__ void check_cu_kernel(const int32_t* __restrict__ cu, int N, int64_t total_T) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i > N) return;
    const int32_t v = cu[i];
    bool bad = v < 0 || (int64_t)v > total_T;
    if (i < N && cu[i + 1] < v) bad = true;
    if (bad) atomicOr(&g_check_flags, (int)kBadCu);
}

__global__ void check_accept_kernel(const int32_t* __restrict__ acc, int N, int L) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    if (acc[i] < 0 || acc[i] > L) atomicOr(&g_check_flags, (int)kBadAccept);
}

int check_device_preconditions(hipStream_t s, const int32_t* slot_idx, int N, int64_t num_slots,
                               const int32_t* cu, int64_t total_T, const int32_t* accept, int L, hipError_t* err) {
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    *err = hipSuccess;
    const int tb = 256;
    hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(64), 0, s);
    if (slot_idx && N > 0)
        hipLaunchKernelGGL(check_slots_kernel, dim3((N + tb - 1) / tb), dim3(tb), 0, s, slot_idx, N, num_slots);
    if (cu)
        hipLaunchKernelGGL(check_cu_kernel, dim3((N + 1 + tb - 1) / tb), dim3(tb), 0, s, cu, N, total_T);
    if (accept && N > 0)
        hipLaunchKernelGGL(check_accept_kernel, dim3((N + tb - 1) / tb), dim3(tb), 0, s, accept, N, L);
    int flags = 0;
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyFromSymbolAsync(&flags, HIP_SYMBOL(g_check_flags), sizeof(int), 0,
                                                      hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    *err = e;
    return flags;
}

}  // namespace lfm2sc
