// bwd.hip -- ShortConv backward for gfx950: input gradients (dB, dC, dxv), the
// weight and bias gradients (dW, dbias, reduced deterministically), and the
// gradient of each sequence's initial state.
//
// The chain rule on the forward (Liger-Kernel PR 1317, "Kernel changes / Gated
// short convolution" describes a fused B/C-gate + conv input backward and a
// weight backward that gathers all K taps of a channel; the formulas are ours,
// from the forward definition).  Per channel of one sequence, with X the padded
// history [initial state | bx...], g = dy * C and dF the gradient arriving at
// the final state X[T .. T+K-1]:
//   dC[t]  = dy[t] * conv[t],           conv[t] = bias + sum_k w[k] X[t+1+k]
//   dbx[u] = sum_k w[k] g[u+K-1-k]      (g = 0 past the sequence end)
//            + dF[K+u-T]                (the last K tokens only)
//   dB[u]  = dbx[u] * xv[u],  dxv[u] = dbx[u] * B[u]
//   dS0[j] = sum_{k<j} w[k] g[j-1-k] + dF[j-T] (j >= T)       (j < K)
//   dW[k]  = sum_t g[t] X[t+1+k],       dbias = sum_t g[t]
//
// Pass structure (one read of dy and in_proj, one write of d_in): each lane
// streams the tokens of its window in order.  At row r it forms g[r], bx[r],
// conv[r] (from the K-1 bx values carried in registers), stores dC[r] and
// accumulates dW and dbias; dbx needs the K-1 FUTURE g values, so dB/dxv are
// emitted K-1 rows behind, at u = r-K+1, with B[u], xv[u] kept in a register
// FIFO.  The window re-reads K-1 rows behind it (B, xv: the halo) and K-1 rows
// ahead of it (dy, C).  The window holding a sequence's token 0 forms dS0 once
// it has g[0 .. K-2].  dW/dbias: each lane accumulates its 8 channels over its
// window, the waves of a workgroup that share channels are summed through LDS
// in a fixed order, one partial row per workgroup window goes to the
// workspace, and a second small kernel sums the rows in a fixed order.  No
// atomics, so every output is bitwise reproducible.
#include <type_traits>

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

// Per channel, the partial row holds the K taps of dW and then dbias.
template <int K> constexpr int kPartCols = K + 1;

template <typename E, int K>
struct BwdState {
    using A = typename BwdAcc<E>::type;
    static constexpr int KH = K > 1 ? K - 1 : 1;
    A wf[kChPerLane][K];
    A bv[kChPerLane];             // conv bias (0 without one)
    A hist[kChPerLane][KH];       // X[r+1 .. r+K-1] for the current row r
    A gw[kChPerLane][K];          // gw[c][a] = g[r-a]
    Raw8<E> fb[KH], fx[KH];       // fb[a] = B of row r-1-a (same for xv)
    A acc[kChPerLane][K + 1];     // dW partial (K taps) and dbias partial
};

template <typename A>
__device__ __forceinline__ A fma_a(A a, A b, A c) { return a * b + c; }
template <> __device__ __forceinline__ float fma_a<float>(float a, float b, float c) { return fmaf(a, b, c); }
template <> __device__ __forceinline__ double fma_a<double>(double a, double b, double c) { return fma(a, b, c); }

// Per-lane byte offsets of the lane's 8 channels in a d_in row (dB | dC | dxv).
struct DinOffsets { uint32_t b, c, x; };

// Where the final-state gradient enters dbx: the lane's dF block of its
// sequence (nullptr without one) and the first token it reaches.
template <typename E>
struct FinalGrad {
    const E* blk;      // 8*K contiguous elements, or nullptr
    int64_t u_first;   // dbx[u] gets dF[K+u-T] for u >= u_first = T-K
    int64_t T;
};

// Emit dB, dxv of token u from the K g values in st.gw (gw[a] = g[u+K-1-a]).
// DF = false is the batched loop's form: it never meets the last K tokens of
// a sequence while a final-state gradient is given.
template <typename E, int K, bool DF>
__device__ __forceinline__ void emit_dbx(BwdState<E, K>& st, const float* bu, const float* xu, int64_t u,
                                         const FinalGrad<E>& fg, rsrc_t du_row, const DinOffsets& o) {
    using A = typename BwdState<E, K>::A;
    A dbx[8];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        A v = st.wf[ch][0] * st.gw[ch][0];
#pragma unroll
        for (int k = 1; k < K; ++k) v = fma_a<A>(st.wf[ch][k], st.gw[ch][k], v);
        dbx[ch] = v;
    }
    if (DF && fg.blk != nullptr && u >= fg.u_first) {
        // token u is among the last K: its bx is entry K+u-T of the final state
        float df[kChPerLane][K];
        load_block<E, K>(fg.blk, df);
        const int64_t j = K + u - fg.T;
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (k == j)
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) dbx[ch] += (A)df[ch][k];
    }
    float dB[8], dX[8];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        dB[ch] = (float)(dbx[ch] * (A)xu[ch]);
        dX[ch] = (float)(dbx[ch] * (A)bu[ch]);
    }
    bst8f<E, LFM2SC_BWD_NT>(du_row, o.b, dB);
    bst8f<E, LFM2SC_BWD_NT>(du_row, o.x, dX);
}

// Row r of the window: all four operands loaded.  Emits dC[r] and, if `emit`,
// dB/dxv of u = r-K+1.
template <typename E, int K, bool DF>
__device__ __forceinline__ void bwd_row(BwdState<E, K>& st, const Raw8<E>& rdy, const Raw8<E>& rb, const Raw8<E>& rc,
                                        const Raw8<E>& rx, rsrc_t dc_row, bool emit, int64_t u, const FinalGrad<E>& fg,
                                        rsrc_t du_row, const DinOffsets& o) {
    using A = typename BwdState<E, K>::A;
    float dy[8], b[8], c[8], x[8], dC[8];
    to_f32(rdy, dy); to_f32(rb, b); to_f32(rc, c); to_f32(rx, x);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const A g = (A)dy[ch] * (A)c[ch];
        const A bx = (A)b[ch] * (A)x[ch];
        A conv = fma_a<A>(st.wf[ch][K - 1], bx, st.bv[ch]);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fma_a<A>(st.wf[ch][k], st.hist[ch][k], conv);
        dC[ch] = (float)((A)dy[ch] * conv);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) st.acc[ch][k] = fma_a<A>(g, st.hist[ch][k], st.acc[ch][k]);
        st.acc[ch][K - 1] = fma_a<A>(g, bx, st.acc[ch][K - 1]);
        st.acc[ch][K] += g;
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
        emit_dbx<E, K, DF>(st, bu, xu, u, fg, du_row, o);
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
                                             int64_t u, const FinalGrad<E>& fg, rsrc_t du_row, const DinOffsets& o) {
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
        emit_dbx<E, K, true>(st, bu, xu, u, fg, du_row, o);
    }
    if constexpr (K > 1) {
#pragma unroll
        for (int a = K - 2; a > 0; --a) { st.fb[a] = st.fb[a - 1]; st.fx[a] = st.fx[a - 1]; }
    }
}

// Initial-state gradient of the lane's 8 channels, formed by the window that
// holds token 0 right after row K-2 (st.gw[a] then holds g[K-2-a]):
// dS0[j] = sum_{k<j} w[k] g[j-1-k] (+ dF[j-T] for j >= T), stored once.
template <typename E, int K>
__device__ __forceinline__ void store_dinit(const BwdState<E, K>& st, const BackwardArgs<E>& a, int seq, int ch0,
                                            int64_t T) {
    using A = typename BwdState<E, K>::A;
    float out[kChPerLane][K];
    float df[kChPerLane][K];
    const bool have_df = a.dfinal != nullptr && T < K;
    if (have_df) load_block<E, K>(a.dfinal + (int64_t)seq * a.H * K + (int64_t)ch0 * K, df);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            A v = (A)0;
#pragma unroll
            for (int k = 0; k < j; ++k) v = fma_a<A>(st.wf[c][k], st.gw[c][K - 1 - j + k], v);
            if (have_df && j >= T) v += (A)df[c][j - T];
            out[c][j] = (float)v;
        }
    }
    store_block<E, K>(a.dinit + (int64_t)seq * a.H * K + (int64_t)ch0 * K, out);
}

template <typename E, int K, int U>
__device__ __forceinline__ void bwd_window(const BackwardArgs<E>& a, const SeqSpan& sp, int ch0, BwdState<E, K>& st) {
    using A = typename BwdState<E, K>::A;
    const int H = a.H;
    const int64_t lo = sp.lo, hi = sp.hi, T = sp.T, r0 = sp.r0;
    const E* ib = a.in + ch0;
    const bool want_dinit = (lo == 0) && a.dinit != nullptr;

    // History X[lo+1 .. lo+K-1]: initial-state entries (index < K) or bx of
    // earlier rows of this sequence.
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
    } else {
        // K = 1: no history entry reaches an output, so dS0 = 0 (dF passes
        // through only for an empty sequence, which no window holds).
        if (want_dinit) {
            float z[kChPerLane][1] = {};
            store_block<E, 1>(a.dinit + (int64_t)sp.seq * H + ch0, z);
        }
    }

    const FinalGrad<E> fg{a.dfinal != nullptr ? a.dfinal + (int64_t)sp.seq * H * K + (int64_t)ch0 * K : nullptr,
                          T - K, T};

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
        for (int u = 0; u < U; ++u) {
            const int64_t rr = t0 + u;
            bwd_row<E, K, false>(st, rdy[u], rb[u], rc[u], rx[u], din_row(rr), true, rr - (K - 1), fg,
                                 din_row(rr - (K - 1)), o);
        }
    };
    // One row on its own (u = r-K+1 emitted when inside the window).
    auto single_row = [&](auto df, int64_t r) {
        const rsrc_t ir = in_row(r);
        const int64_t u = r - (K - 1);
        bwd_row<E, K, decltype(df)::value>(st, bld8<E, LFM2SC_BWD_NT>(dy_row(r), o.b), bld8<E, LFM2SC_BWD_NT>(ir, o.b),
                                           bld8<E, LFM2SC_BWD_NT>(ir, o.c), bld8<E, LFM2SC_BWD_NT>(ir, o.x),
                                           din_row(r), u >= lo, u, fg, din_row(u >= lo ? u : r), o);
        if constexpr (K > 1)
            if (want_dinit && r == K - 2) store_dinit<E, K>(st, a, sp.seq, ch0, T);
    };
    // With a final-state gradient, the row that emits the first of the last K
    // tokens (the sequence's last row) is taken after the batched rows; the
    // later K-1 of them are emitted by the rows past the window.
    const int64_t main_hi = (a.dfinal != nullptr && hi == T && hi > lo) ? hi - 1 : hi;

    // Rows whose u = r-K+1 is still before the window: no dB/dxv emitted.
    int64_t r = lo;
    const int64_t head_end = (lo + K - 1 < main_hi) ? lo + K - 1 : main_hi;
    for (; r < head_end; ++r) single_row(std::false_type{}, r);
    // Steady state: batches of U rows, all loads of a batch issued together.
    for (; r + U <= main_hi; r += U) {
        Raw8<E> rdy[U], rb[U], rc[U], rx[U];
        load_batch(rdy, rb, rc, rx, r);
        use_batch(rdy, rb, rc, rx, r);
    }
    // Remainder (< U rows): one partial batch, all its loads issued together.
    if (r < main_hi) {
        const int n = (int)(main_hi - r);
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
        for (int u = 0; u < U; ++u) {
            if (u < n) {
                const int64_t rr = r + u;
                bwd_row<E, K, false>(st, rdy[u], rb[u], rc[u], rx[u], din_row(rr), true, rr - (K - 1), fg,
                                     din_row(rr - (K - 1)), o);
            }
        }
        r = main_hi;
    }
    if (r < hi) single_row(std::true_type{}, r++);
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
            bwd_tail_row<E, K>(st, g, u >= lo, u, fg, din_row(u >= lo ? u : r), o);
            if (want_dinit && r == K - 2) store_dinit<E, K>(st, a, sp.seq, ch0, T);
        }
    }
}

// Static LDS of the workgroup's dW/dbias reduction, and the dynamic LDS that
// brings the total to LFM2SC_BWD_LDS (so one workgroup runs per CU).
template <typename E, int K>
constexpr size_t bwd_static_lds() {
    return LFM2SC_BWD_TW > 1 ? (size_t)kWavesPerBlock * kChPerLane * kPartCols<K> * kWave *
                                   sizeof(typename BwdAcc<E>::type)
                             : 0;
}
template <typename E, int K>
constexpr size_t bwd_dyn_lds() {
    return (size_t)LFM2SC_BWD_LDS > bwd_static_lds<E, K>() ? (size_t)LFM2SC_BWD_LDS - bwd_static_lds<E, K>() : 0;
}

template <typename E, int K, int U>
__global__ __launch_bounds__(kThreads) void backward_kernel(const BackwardArgs<E> a) {
    using A = typename BwdState<E, K>::A;
    constexpr int TW = LFM2SC_BWD_TW;
    constexpr int PC = kPartCols<K>;
    using Lay = WgLayout<TW>;
    const int wave = wave_id();
    const int lane = threadIdx.x % kWave;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int ch0 = ((blockIdx.y * Lay::kCW + wave / TW) * kWave + lane) * kChPerLane;
    const bool lane_on = tile < a.ntiles && ch0 < a.H;
    const bool tile_on = tile < a.ntiles;   // wave-uniform

    BwdState<E, K> st;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int k = 0; k < K; ++k) st.gw[c][k] = (A)0;
#pragma unroll
        for (int k = 0; k < PC; ++k) st.acc[c][k] = (A)0;
    }

    if (tile_on) {
        const int64_t gap = (int64_t)a.sub * TW;
        const int64_t v0 = (int64_t)tile * gap + (int64_t)(wave % TW) * a.sub;
        SeqSpan sp;
        // the span search runs with every lane of the wave active; lanes past H then stay idle
        if (find_span(a.cu, a.N, a.total_T, gap, v0, v0 + a.sub, sp) && lane_on) {
            float wf[kChPerLane][K];
            load_block<E, K>(a.w + (int64_t)ch0 * K, wf);
            float bv[8] = {};
            if (a.bias != nullptr) load_f32x8<E>(a.bias + ch0, bv);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st.bv[c] = (A)bv[c];
#pragma unroll
                for (int k = 0; k < K; ++k) st.wf[c][k] = (A)wf[c][k];
            }
            bwd_window<E, K, U>(a, sp, ch0, st);
        }
    }

    // dW / dbias partial of this workgroup window: the TW waves that share
    // channels (consecutive windows) are summed through LDS in a fixed order;
    // one partial row [H][K+1] per workgroup window goes to the workspace.
    A* dst = static_cast<A*>(a.partial) + (int64_t)tile * a.H * PC + (int64_t)ch0 * PC;
    if constexpr (TW == 1) {
        if (lane_on) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int k = 0; k < PC; ++k) dst[c * PC + k] = st.acc[c][k];
        }
    } else {
        __shared__ A red[kWavesPerBlock][kChPerLane * PC][kWave];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int k = 0; k < PC; ++k) red[wave][c * PC + k][lane] = st.acc[c][k];
        __syncthreads();
        if (wave % TW == 0 && lane_on) {
#pragma unroll
            for (int e = 0; e < kChPerLane * PC; ++e) {
                A v = red[wave][e][lane];
#pragma unroll
                for (int q = 1; q < TW; ++q) v += red[wave + q][e][lane];
                dst[e] = v;
            }
        }
    }
}

// dW[h][k] (and dbias[h]) = sum over windows of the partial rows, column
// h*(K+1)+k (+K).  A workgroup takes 16 chunks of 16 bytes of columns (64 fp32
// or 32 fp64 columns) and 16 row groups: each thread sums the rows rg, rg+16,
// ... of its chunk in that order, then 16 partial sums per column meet in LDS
// and are added in row-group order.  Fixed order, one rounding to fp32 at the
// store.
constexpr int kFinQ = 16;    // 16-byte column chunks per workgroup
constexpr int kFinRG = 16;   // row groups per workgroup
constexpr int kFinThreads = kFinQ * kFinRG;

template <typename A>
__global__ __launch_bounds__(kFinThreads) void dw_finish_kernel(const A* __restrict__ partial, int64_t ntiles,
                                                                 int64_t H, int K, float* __restrict__ dW,
                                                                 float* __restrict__ dbias) {
    constexpr int V = 16 / (int)sizeof(A);   // columns per 16-byte chunk
    constexpr int kCols = kFinQ * V;         // columns per workgroup
    const int PC = K + 1;
    const int64_t cols = H * PC;             // a multiple of 8 (H % 8 == 0): chunks never straddle its end
    const int q = threadIdx.x % kFinQ;
    const int rg = threadIdx.x / kFinQ;
    const int64_t c0 = (int64_t)blockIdx.x * kCols + (int64_t)q * V;
    A s[V];
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] = (A)0;
    if (c0 < cols) {
#pragma unroll 4
        for (int64_t r = rg; r < ntiles; r += kFinRG) {
            const uint4 raw = *reinterpret_cast<const uint4*>(partial + r * cols + c0);
            const A* e = reinterpret_cast<const A*>(&raw);
#pragma unroll
            for (int v = 0; v < V; ++v) s[v] += e[v];
        }
    }
    __shared__ A red[kFinRG][kCols + 1];
#pragma unroll
    for (int v = 0; v < V; ++v) red[rg][q * V + v] = s[v];
    __syncthreads();
    if (threadIdx.x < kCols) {
        const int64_t j = (int64_t)blockIdx.x * kCols + threadIdx.x;
        if (j < cols) {
            A t = (A)0;
#pragma unroll
            for (int g = 0; g < kFinRG; ++g) t += red[g][threadIdx.x];
            const int64_t h = j / PC;
            const int k = (int)(j % PC);
            if (k < K) dW[h * K + k] = (float)t;
            else if (dbias != nullptr) dbias[h] = (float)t;
        }
    }
}

// d_init of sequences with no token (no window holds them): dS0 = dF, or 0.
template <typename E>
__global__ __launch_bounds__(kSmallBlock) void dinit_empty_kernel(const int32_t* __restrict__ cu, int64_t total_T,
                                                                 int64_t HK, const E* __restrict__ dfinal,
                                                                 E* __restrict__ dinit) {
    const int i = blockIdx.x;
    const int64_t e0 = ((int64_t)blockIdx.y * kSmallBlock + threadIdx.x) * 8;
    if (e0 >= HK) return;
    const int64_t r0 = clamp64(cu[i], 0, total_T);
    const int64_t r1 = clamp64(cu[i + 1], r0, total_T);
    if (r1 > r0) return;
    Raw8<E> v;
    if (dfinal != nullptr) {
        v = ld8<E>(dfinal + (int64_t)i * HK + e0);
    } else {
        const float z[8] = {};
        v = from_f32<E>(z);
    }
    st8<E>(dinit + (int64_t)i * HK + e0, v);
}

// fp32 I/O carries fp64 state: fewer rows in flight keep it in registers.
template <typename E, int K> constexpr int bwd_unroll() {
    return sizeof(typename BwdAcc<E>::type) == 8 ? (K >= 3 ? 1 : 2) : LFM2SC_BWD_U;
}

template <typename E, int K>
static Tiling backward_tiling(int64_t total_T, int N, int H) {
    constexpr auto kernel = backward_kernel<E, K, bwd_unroll<E, K>()>;
    static const int resident_long = resident_workgroups(kernel, bwd_dyn_lds<E, K>());
    static const int resident_short = resident_workgroups(kernel, 0);
    return ragged_tiling(total_T, N, WgLayout<LFM2SC_BWD_TW>::groups(H),
                         total_T < LFM2SC_SHORT_T ? resident_short : resident_long, LFM2SC_BWD_TW,
                         (int64_t)H * (int64_t)sizeof(E), kWinSpanBwd);
}

template <typename E, int K>
static hipError_t backward_k(BackwardArgs<E> a, hipStream_t s) {
    using A = typename BwdAcc<E>::type;
    if (a.N > 0 && a.total_T > 0) {
        const Tiling t = backward_tiling<E, K>(a.total_T, a.N, a.H);
        a.sub = t.sub;
        a.ntiles = (int)t.ntiles;
        const int gy = WgLayout<LFM2SC_BWD_TW>::groups(a.H);
        const size_t dyn_lds = a.total_T < LFM2SC_SHORT_T ? 0 : bwd_dyn_lds<E, K>();
        hipLaunchKernelGGL((backward_kernel<E, K, bwd_unroll<E, K>()>), dim3(pad_xcd(a.ntiles), gy), dim3(kThreads),
                           dyn_lds, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        a.ntiles = 0;
    }
    const int64_t cols = (int64_t)a.H * kPartCols<K>;
    const int64_t fin_cols = (int64_t)kFinQ * (16 / (int64_t)sizeof(A));
    hipLaunchKernelGGL((dw_finish_kernel<A>), dim3((unsigned)((cols + fin_cols - 1) / fin_cols)), dim3(kFinThreads), 0,
                       s, (const A*)a.partial, (int64_t)a.ntiles, (int64_t)a.H, K, a.dW, a.dbias);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.dinit != nullptr && a.N > 0) {
        const int64_t HK = (int64_t)a.H * K;
        hipLaunchKernelGGL((dinit_empty_kernel<E>), dim3(a.N, (unsigned)((HK / 8 + kSmallBlock - 1) / kSmallBlock)),
                           dim3(kSmallBlock), 0, s, a.cu, a.total_T, HK, a.dfinal, a.dinit);
        e = hipGetLastError();
    }
    return e;
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
