// bwd.hip -- ShortConv backward for gfx950: input gradients (dB, dC, dxv) and
// the weight gradient dW, reduced deterministically in fp32.
//
// Derivatives of the forward (Liger-Kernel PR 1317, "Kernel changes / Gated
// short convolution" describes a fused B/C-gate + conv input backward and a
// weight backward that gathers all K taps of a channel; the formulas are ours,
// from the forward definition).  Per channel of one sequence, with X the padded
// history [state | bx...] and g = dy * C:
//   dC[t]  = dy[t] * conv[t],            conv[t] = sum_k w[k] X[t+1+k]
//   dbx[u] = sum_k w[k] g[u+K-1-k]       (g = 0 past the sequence end)
//   dB[u]  = dbx[u] * xv[u],  dxv[u] = dbx[u] * B[u]
//   dW[k]  = sum_t g[t] X[t+1+k]
//
// Pass structure (one read of dy and in_proj, one write of d_in): each lane
// streams the tokens of its window in order.  At row r it forms g[r], bx[r],
// conv[r] (from the K-1 bx values carried in registers), stores dC[r] and
// accumulates dW; dbx needs the K-1 FUTURE g values, so dB/dxv are emitted
// K-1 rows behind, at u = r-K+1, with B[u], xv[u] kept in a register FIFO.
// The window re-reads K-1 rows behind it (B, xv: the halo) and K-1 rows
// ahead of it (dy, C).  dW: each lane accumulates its 8 channels x K taps over
// its window, the 4 waves of a workgroup are summed through LDS in a fixed
// order, one fp32 partial row per workgroup window goes to the workspace,
// and a second small kernel sums the rows in a fixed order.  No atomics, so
// dW is bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace lfm2sc {

// Internal arithmetic type of the backward: fp32 for bf16 I/O (products of
// two bf16 values are exact in fp32), fp64 for fp32 I/O (products of two fp32
// values are exact in fp64).  dW is a reduction over every token of a
// sequence, so this keeps its only rounding at the final fp32 store even when
// thousands of terms cancel.
template <typename E> struct BwdAcc { using type = float; };
template <> struct BwdAcc<float> { using type = double; };

template <typename E, int K>
struct BwdState {
    using A = typename BwdAcc<E>::type;
    static constexpr int KH = K > 1 ? K - 1 : 1;
    A wf[kChPerLane][K];
    A hist[kChPerLane][KH];       // X[r+1 .. r+K-1] for the current row r
    A gw[kChPerLane][K];          // gw[c][a] = g[r-a]
    Raw8<E> fb[KH], fx[KH];       // fb[a] = B of row r-1-a (same for xv)
    A acc[kChPerLane][K];         // dW partial
};

template <typename A>
__device__ __forceinline__ A fma_a(A a, A b, A c) { return a * b + c; }
template <> __device__ __forceinline__ float fma_a<float>(float a, float b, float c) { return fmaf(a, b, c); }
template <> __device__ __forceinline__ double fma_a<double>(double a, double b, double c) { return fma(a, b, c); }

// Row r of the window: all four operands loaded.  Emits dC[r] and, if `emit`,
// dB/dxv of u = r-K+1.
// Per-lane byte offsets of the lane's 8 channels in a d_in row (dB | dC | dxv).
struct DinOffsets { uint32_t b, c, x; };

template <typename E, int K>
__device__ __forceinline__ void bwd_row(BwdState<E, K>& st, const Raw8<E>& rdy, const Raw8<E>& rb, const Raw8<E>& rc,
                                        const Raw8<E>& rx, rsrc_t dc_row, bool emit, rsrc_t du_row,
                                        const DinOffsets& o) {
    using A = typename BwdState<E, K>::A;
    float dy[8], b[8], c[8], x[8], dC[8];
    to_f32(rdy, dy); to_f32(rb, b); to_f32(rc, c); to_f32(rx, x);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const A g = (A)dy[ch] * (A)c[ch];
        const A bx = (A)b[ch] * (A)x[ch];
        A conv = st.wf[ch][K - 1] * bx;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fma_a<A>(st.wf[ch][k], st.hist[ch][k], conv);
        dC[ch] = (float)((A)dy[ch] * conv);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) st.acc[ch][k] = fma_a<A>(g, st.hist[ch][k], st.acc[ch][k]);
        st.acc[ch][K - 1] = fma_a<A>(g, bx, st.acc[ch][K - 1]);
        if constexpr (K > 1) {
#pragma unroll
            for (int k = 0; k < K - 2; ++k) st.hist[ch][k] = st.hist[ch][k + 1];
            st.hist[ch][K - 2] = bx;
        }
#pragma unroll
        for (int a = K - 1; a > 0; --a) st.gw[ch][a] = st.gw[ch][a - 1];
        st.gw[ch][0] = g;
    }
    bst8f<E, LFM2SC_BWD_NT>(dc_row, o.c, dC);
    if (emit) {
        float bu[8], xu[8];
        if constexpr (K > 1) { to_f32(st.fb[K - 2], bu); to_f32(st.fx[K - 2], xu); }
        else { to_f32(rb, bu); to_f32(rx, xu); }
        float dB[8], dX[8];
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            A dbx = st.wf[ch][0] * st.gw[ch][0];
#pragma unroll
            for (int k = 1; k < K; ++k) dbx = fma_a<A>(st.wf[ch][k], st.gw[ch][k], dbx);
            dB[ch] = (float)(dbx * (A)xu[ch]);
            dX[ch] = (float)(dbx * (A)bu[ch]);
        }
        bst8f<E, LFM2SC_BWD_NT>(du_row, o.b, dB);
        bst8f<E, LFM2SC_BWD_NT>(du_row, o.x, dX);
    }
    if constexpr (K > 1) {
#pragma unroll
        for (int a = K - 2; a > 0; --a) { st.fb[a] = st.fb[a - 1]; st.fx[a] = st.fx[a - 1]; }
        st.fb[0] = rb; st.fx[0] = rx;
    }
}

// Row r at or past the window end: only g[r] is needed (0 past the sequence
// end); emits dB/dxv of u = r-K+1 when u is inside the window.
template <typename E, int K>
__device__ __forceinline__ void bwd_tail_row(BwdState<E, K>& st, const typename BwdState<E, K>::A* g, bool emit,
                                             rsrc_t du_row, const DinOffsets& o) {
    using A = typename BwdState<E, K>::A;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
#pragma unroll
        for (int a = K - 1; a > 0; --a) st.gw[ch][a] = st.gw[ch][a - 1];
        st.gw[ch][0] = g[ch];
    }
    if (emit) {
        float bu[8], xu[8];
        to_f32(st.fb[K - 2 >= 0 ? K - 2 : 0], bu);
        to_f32(st.fx[K - 2 >= 0 ? K - 2 : 0], xu);
        float dB[8], dX[8];
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            A dbx = st.wf[ch][0] * st.gw[ch][0];
#pragma unroll
            for (int k = 1; k < K; ++k) dbx = fma_a<A>(st.wf[ch][k], st.gw[ch][k], dbx);
            dB[ch] = (float)(dbx * (A)xu[ch]);
            dX[ch] = (float)(dbx * (A)bu[ch]);
        }
        bst8f<E, LFM2SC_BWD_NT>(du_row, o.b, dB);
        bst8f<E, LFM2SC_BWD_NT>(du_row, o.x, dX);
    }
    if constexpr (K > 1) {
#pragma unroll
        for (int a = K - 2; a > 0; --a) { st.fb[a] = st.fb[a - 1]; st.fx[a] = st.fx[a - 1]; }
    }
}

template <typename E, int K, int U>
__device__ __forceinline__ void bwd_window(const BackwardArgs<E>& a, const SeqSpan& sp, int ch0, BwdState<E, K>& st) {
    const int H = a.H;
    const int64_t lo = sp.lo, hi = sp.hi, T = sp.T, r0 = sp.r0;
    const E* ib = a.in + ch0;

    // History X[lo+1 .. lo+K-1]: initial-state entries (index < K) or bx of
    // earlier rows of this sequence.
    using A = typename BwdState<E, K>::A;
    if constexpr (K > 1) {
        float s0[kChPerLane][K];
        bool have_s0 = false;
        if (lo < K - 1 && a.pool != nullptr) {
            const int64_t slot = a.slot_idx[sp.seq];
            if (slot_ok(slot, a.num_slots)) {
                load_block<E, K>(a.pool + slot * a.slot_stride + (int64_t)ch0 * K, s0);
                have_s0 = true;
            }
        }
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            const int64_t j = lo + 1 + k;
            if (j < K) {
#pragma unroll
                for (int c = 0; c < 8; ++c) st.hist[c][k] = have_s0 ? (A)s0[c][j] : (A)0;
            } else {
                const E* row = ib + (r0 + j - K) * a.in_stride;
                float b[8], x[8];
                load_f32x8<E>(row, b);
                load_f32x8<E>(row + 2 * H, x);
#pragma unroll
                for (int c = 0; c < 8; ++c) st.hist[c][k] = (A)b[c] * (A)x[c];
            }
        }
    }

    // Streamed rows go through buffer descriptors (see row_rsrc).
    const uint32_t eb = sizeof(E);
    const DinOffsets o{(uint32_t)ch0 * eb, (uint32_t)(ch0 + H) * eb, (uint32_t)(ch0 + 2 * H) * eb};
    const uint32_t in_bytes = 3u * (uint32_t)H * eb, dy_bytes = (uint32_t)H * eb;
    const E* in_rows = a.in + r0 * a.in_stride;
    const E* dy_rows = a.dy + r0 * a.dy_stride;
    E* din_rows = a.din + r0 * a.din_stride;
    auto in_row = [&](int64_t t) { return row_rsrc(in_rows + t * a.in_stride, in_bytes); };
    auto dy_row = [&](int64_t t) { return row_rsrc(dy_rows + t * a.dy_stride, dy_bytes); };
    auto din_row = [&](int64_t t) { return row_rsrc(din_rows + t * a.din_stride, in_bytes); };
    auto load_batch = [&](Raw8<E> (&rdy)[U], Raw8<E> (&rb)[U], Raw8<E> (&rc)[U], Raw8<E> (&rx)[U], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const rsrc_t ir = in_row(t0 + u);
            rdy[u] = bld8<E, LFM2SC_BWD_NT>(dy_row(t0 + u), o.b);
            rb[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.b);
            rc[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.c);
            rx[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.x);
        }
    };
    auto use_batch = [&](const Raw8<E> (&rdy)[U], const Raw8<E> (&rb)[U], const Raw8<E> (&rc)[U],
                         const Raw8<E> (&rx)[U], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            bwd_row<E, K>(st, rdy[u], rb[u], rc[u], rx[u], din_row(t0 + u), true, din_row(t0 + u - (K - 1)), o);
    };

    // Rows whose u = r-K+1 is still before the window: no dB/dxv emitted.
    int64_t r = lo;
    const int64_t head_end = (lo + K - 1 < hi) ? lo + K - 1 : hi;
    for (; r < head_end; ++r) {
        const rsrc_t ir = in_row(r);
        bwd_row<E, K>(st, bld8<E, LFM2SC_BWD_NT>(dy_row(r), o.b), bld8<E, LFM2SC_BWD_NT>(ir, o.b),
                      bld8<E, LFM2SC_BWD_NT>(ir, o.c), bld8<E, LFM2SC_BWD_NT>(ir, o.x), din_row(r), false, din_row(r),
                      o);
    }
    // Steady state: batches of U rows, all loads of a batch issued together.
    for (; r + U <= hi; r += U) {
        Raw8<E> rdy[U], rb[U], rc[U], rx[U];
        load_batch(rdy, rb, rc, rx, r);
        use_batch(rdy, rb, rc, rx, r);
    }
    // Remainder (< U rows): one partial batch, all its loads issued together.
    if (r < hi) {
        const int n = (int)(hi - r);
        Raw8<E> rdy[U], rb[U], rc[U], rx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < n) {
                const rsrc_t ir = in_row(r + u);
                rdy[u] = bld8<E, LFM2SC_BWD_NT>(dy_row(r + u), o.b);
                rb[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.b);
                rc[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.c);
                rx[u] = bld8<E, LFM2SC_BWD_NT>(ir, o.x);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < n)
                bwd_row<E, K>(st, rdy[u], rb[u], rc[u], rx[u], din_row(r + u), true, din_row(r + u - (K - 1)), o);
        r = hi;
    }
    // K-1 rows past the window: g only, from the next rows of the sequence.
    if constexpr (K > 1) {
        for (; r < hi + K - 1; ++r) {
            A g[8];
            if (r < T) {
                float dyv[8], cv[8];
                to_f32(bld8<E, 0>(dy_row(r), o.b), dyv);
                to_f32(bld8<E, 0>(in_row(r), o.c), cv);
#pragma unroll
                for (int c = 0; c < 8; ++c) g[c] = (A)dyv[c] * (A)cv[c];
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) g[c] = (A)0;
            }
            const int64_t u = r - (K - 1);
            bwd_tail_row<E, K>(st, g, u >= lo, din_row(u), o);
        }
    }
}

template <typename E, int K, int U>
__global__ __launch_bounds__(kThreads) void backward_kernel(const BackwardArgs<E> a) {
    using A = typename BwdState<E, K>::A;
    constexpr int TW = LFM2SC_BWD_TW;
    using Lay = WgLayout<TW>;
    const int wave = wave_id();
    const int lane = threadIdx.x % kWave;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int ch0 = ((blockIdx.y * Lay::kCW + wave / TW) * kWave + lane) * kChPerLane;
    const bool lane_on = tile < a.ntiles && ch0 < a.H;

    BwdState<E, K> st;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) { st.acc[c][k] = (A)0; st.gw[c][k] = (A)0; }

    if (lane_on) {
        const int64_t gap = (int64_t)a.sub * TW;
        const int64_t v0 = (int64_t)tile * gap + (int64_t)(wave % TW) * a.sub;
        SeqSpan sp;
        if (find_span(a.cu, a.N, a.total_T, gap, v0, v0 + a.sub, sp)) {
            float wf[kChPerLane][K];
            load_block<E, K>(a.w + (int64_t)ch0 * K, wf);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int k = 0; k < K; ++k) st.wf[c][k] = (A)wf[c][k];
            bwd_window<E, K, U>(a, sp, ch0, st);
        }
    }

    // dW partial of this workgroup window: the TW waves that share channels
    // (consecutive windows) are summed through LDS in a fixed order; one
    // partial row [H*K] per workgroup window goes to the workspace.
    A* dst = static_cast<A*>(a.partial) + (int64_t)tile * a.H * K + (int64_t)ch0 * K;
    if constexpr (TW == 1) {
        if (lane_on) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int k = 0; k < K; ++k) dst[c * K + k] = st.acc[c][k];
        }
    } else {
        __shared__ A red[kWavesPerBlock][kChPerLane * K][kWave];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int k = 0; k < K; ++k) red[wave][c * K + k][lane] = st.acc[c][k];
        __syncthreads();
        if (wave % TW == 0 && lane_on) {
#pragma unroll
            for (int e = 0; e < kChPerLane * K; ++e) {
                A v = red[wave][e][lane];
#pragma unroll
                for (int q = 1; q < TW; ++q) v += red[wave + q][e][lane];
                dst[e] = v;
            }
        }
    }
}

// dW[j] = sum over windows of partial[window][j], j in [0, H*K): 32 columns x
// 32 row groups per workgroup, then a fixed-order sum of the 32 row groups;
// one rounding to fp32 at the store.
constexpr int kFinCols = 32;
constexpr int kFinRows = 32;

template <typename A>
__global__ __launch_bounds__(kFinCols * kFinRows) void dw_finish_kernel(const A* __restrict__ partial, int64_t ntiles,
                                                                       int64_t HK, float* __restrict__ dW) {
    const int col = threadIdx.x % kFinCols;
    const int rg = threadIdx.x / kFinCols;
    const int64_t j = (int64_t)blockIdx.x * kFinCols + col;
    A s = (A)0;
    if (j < HK) {
#pragma unroll 8
        for (int64_t r = rg; r < ntiles; r += kFinRows) s += partial[r * HK + j];
    }
    __shared__ A red[kFinRows][kFinCols + 1];
    red[rg][col] = s;
    __syncthreads();
    if (rg == 0 && j < HK) {
        A t = (A)0;
#pragma unroll
        for (int q = 0; q < kFinRows; ++q) t += red[q][col];
        dW[j] = (float)t;
    }
}

// fp32 I/O carries fp64 state: fewer rows in flight keep it in registers.
template <typename E> constexpr int bwd_unroll() { return sizeof(typename BwdAcc<E>::type) == 8 ? 2 : LFM2SC_BWD_U; }

template <typename E, int K>
static Tiling backward_tiling(int64_t total_T, int N, int H) {
    constexpr auto kernel = backward_kernel<E, K, bwd_unroll<E>()>;
    static const int resident = resident_workgroups(kernel, LFM2SC_BWD_LDS);
    return ragged_tiling(total_T, N, WgLayout<LFM2SC_BWD_TW>::groups(H), resident, LFM2SC_BWD_TW);
}

template <typename E, int K>
static hipError_t backward_k(BackwardArgs<E> a, hipStream_t s) {
    using A = typename BwdAcc<E>::type;
    if (a.N > 0 && a.total_T > 0) {
        const Tiling t = backward_tiling<E, K>(a.total_T, a.N, a.H);
        a.sub = t.sub;
        a.ntiles = (int)t.ntiles;
        const int gy = WgLayout<LFM2SC_BWD_TW>::groups(a.H);
        hipLaunchKernelGGL((backward_kernel<E, K, bwd_unroll<E>()>), dim3(pad_xcd(a.ntiles), gy), dim3(kThreads),
                           LFM2SC_BWD_LDS, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        a.ntiles = 0;
    }
    const int64_t HK = (int64_t)a.H * K;
    hipLaunchKernelGGL((dw_finish_kernel<A>), dim3((unsigned)((HK + kFinCols - 1) / kFinCols)),
                       dim3(kFinCols * kFinRows), 0, s, (const A*)a.partial, (int64_t)a.ntiles, HK, a.dW);
    return hipGetLastError();
}

template <typename E>
static int64_t partial_rows_e(int K, int64_t total_T, int N, int H) {
    switch (K) {
        case 1: return backward_tiling<E, 1>(total_T, N, H).ntiles;
        case 2: return backward_tiling<E, 2>(total_T, N, H).ntiles;
        case 3: return backward_tiling<E, 3>(total_T, N, H).ntiles;
        case 4: return backward_tiling<E, 4>(total_T, N, H).ntiles;
    }
    return 0;
}

int64_t backward_partial_rows(int dtype_is_f32, int H, int K, int64_t total_T, int N) {
    if (N <= 0 || total_T <= 0) return 0;
    return dtype_is_f32 ? partial_rows_e<float>(K, total_T, N, H) : partial_rows_e<uint16_t>(K, total_T, N, H);
}

int backward_partial_bytes(int dtype_is_f32) { return dtype_is_f32 ? (int)sizeof(double) : (int)sizeof(float); }

template <typename E>
hipError_t launch_backward(const BackwardArgs<E>& a, int K, hipStream_t s) {
    switch (K) {
        case 1: return backward_k<E, 1>(a, s);
        case 2: return backward_k<E, 2>(a, s);
        case 3: return backward_k<E, 3>(a, s);
        case 4: return backward_k<E, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template hipError_t launch_backward<uint16_t>(const BackwardArgs<uint16_t>&, int, hipStream_t);
template hipError_t launch_backward<float>(const BackwardArgs<float>&, int, hipStream_t);

}  // namespace lfm2sc
