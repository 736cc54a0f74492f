/*
 * oracle.c -- fp64 CPU oracle for the LFM2 gated short causal convolution.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU baseline, never by the product path.  Shares no code with
 * the HIP library.  The definitions and the readings behind them are listed in
 * oracle.h; each function below names the passage it follows.
 *
 * Style: plain loops over (sequence, channel, token), one output element at a
 * time, in the order the definition states them.  OpenMP splits the channel
 * loop only, so thread count never changes any result.
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void oracle_set_threads(int n) {
    if (n < 1) n = 1;
#ifdef _OPENMP
    g_threads = n;
#else
    g_threads = 1;
#endif
}

int oracle_get_threads(void) { return g_threads; }

/* Row-range sanity so that every access below stays in bounds. */
static int check_cu(const int32_t* cu, int N, int64_t total_T) {
    if (N < 0) return -1;
    if (N == 0) return 0;
    if (!cu || cu[0] < 0) return -1;
    for (int i = 0; i < N; ++i)
        if (cu[i + 1] < cu[i]) return -1;
    if ((int64_t)cu[N] > total_T) return -1;
    return 0;
}

static int check_slots(const int32_t* slot_idx, int N, int64_t num_slots) {
    if (N > 0 && !slot_idx) return -1;
    for (int i = 0; i < N; ++i)
        if (slot_idx[i] < 0 || (int64_t)slot_idx[i] >= num_slots) return -1;
    return 0;
}

/*
 * Ragged prefill.
 *
 * MAX Pipelines LFM2 article, section "ShortConv implementation
 * (LFM2ShortConv)": bx = b * xv from the three-way split of in_proj; the
 * per-token loop shifts bx into the [H, K] state and takes
 * conv_out = sum_k state * w, then y = c * conv_out.  Section "Batching and
 * weight adaptation" / the graph inputs: tokens of all requests are packed
 * with row offsets, and each conv layer receives one [H, K] state per request.
 *
 * The token loop is written here through the padded history of one channel,
 *     X = [S0[0], ..., S0[K-1], bx[0], ..., bx[T-1]],
 * in which the state after token t is X[t+1 .. t+K]; hence
 *     conv[t] = sum_k w[k] * X[t+1+k]
 * and the final state is X[T .. T+K-1].  (Decode and verify below use the
 * shift form instead, so that the two codings can be checked against each
 * other.)  All final states are written after all initial states are read.
 */
int oracle_prefill(int H, int K, int64_t total_T,
                   const double* in, int64_t in_stride,
                   const int32_t* cu, int N,
                   const double* w, const double* bias,
                   double* pool, int64_t num_slots, const int32_t* slot_idx,
                   double* y) {
    if (H <= 0 || K <= 0 || total_T < 0 || in_stride < 3 * (int64_t)H) return -1;
    if (check_cu(cu, N, total_T)) return -1;
    if (pool && check_slots(slot_idx, N, num_slots)) return -1;
    if (N == 0) return 0;
    if ((cu[N] > 0 && (!in || !y)) || !w) return -1;

    const int64_t HK = (int64_t)H * K;
    double* fin = NULL;
    if (pool) {
        fin = (double*)malloc(sizeof(double) * (size_t)N * (size_t)HK);
        if (!fin) return -1;
    }
    int fail = 0;
    for (int i = 0; i < N; ++i) {
        const int64_t r0 = cu[i];
        const int64_t T = (int64_t)cu[i + 1] - cu[i];
#pragma omp parallel for num_threads(g_threads) schedule(static)
        for (int h = 0; h < H; ++h) {
            double* X = (double*)malloc(sizeof(double) * (size_t)(K + T));
            if (!X) { fail = 1; continue; }
            for (int k = 0; k < K; ++k)
                X[k] = pool ? pool[(int64_t)slot_idx[i] * HK + (int64_t)h * K + k] : 0.0;
            for (int64_t u = 0; u < T; ++u) {
                const double* row = in + (r0 + u) * in_stride;
                X[K + u] = row[h] * row[2 * H + h];              /* bx = B * xv */
            }
            for (int64_t t = 0; t < T; ++t) {
                const double* row = in + (r0 + t) * in_stride;
                double conv = 0.0;
                for (int k = 0; k < K; ++k) conv += w[(int64_t)h * K + k] * X[t + 1 + k];
                if (bias) conv += bias[h];
                y[(r0 + t) * H + h] = row[H + h] * conv;        /* y = C * conv */
            }
            if (fin)
                for (int k = 0; k < K; ++k) fin[(int64_t)i * HK + (int64_t)h * K + k] = X[T + k];
            free(X);
        }
    }
    if (fin) {
        if (!fail)
            for (int i = 0; i < N; ++i)
                memcpy(pool + (int64_t)slot_idx[i] * HK, fin + (int64_t)i * HK, sizeof(double) * (size_t)HK);
        free(fin);
    }
    return fail ? -1 : 0;
}

/*
 * One decode step per sequence.
 *
 * MAX Pipelines LFM2 article, section "ShortConv implementation
 * (LFM2ShortConv)": the request's [H, K] state is taken from its slot, the
 * oldest column is dropped and bx of the new token appended, conv_out is the
 * tap-weighted sum of the new state, y = c * conv_out, and the new state goes
 * back to the same slot (section "Inference state management").
 */
int oracle_decode(int H, int K, int N,
                  const double* in, int64_t in_stride,
                  const double* w, const double* bias,
                  double* pool, int64_t num_slots, const int32_t* slot_idx,
                  double* y) {
    if (H <= 0 || K <= 0 || N < 0 || in_stride < 3 * (int64_t)H) return -1;
    if (N == 0) return 0;
    if (!in || !w || !pool || !y) return -1;
    if (check_slots(slot_idx, N, num_slots)) return -1;
    const int64_t HK = (int64_t)H * K;
    int fail = 0;
    for (int i = 0; i < N; ++i) {
        const double* row = in + (int64_t)i * in_stride;
        double* S_all = pool + (int64_t)slot_idx[i] * HK;
#pragma omp parallel for num_threads(g_threads) schedule(static)
        for (int h = 0; h < H; ++h) {
            double* S = S_all + (int64_t)h * K;
            for (int k = 0; k + 1 < K; ++k) S[k] = S[k + 1];  /* drop the oldest */
            S[K - 1] = row[h] * row[2 * H + h];                /* append bx      */
            double conv = 0.0;
            for (int k = 0; k < K; ++k) conv += w[(int64_t)h * K + k] * S[k];
            if (bias) conv += bias[h];
            y[(int64_t)i * H + h] = row[H + h] * conv;
        }
    }
    return fail;
}

/*
 * Speculative verify window.
 *
 * SGLang PR 31041 summary, implementation item 2 and the shortconv_target_verify
 * excerpt: the block of draft tokens of each request is run through the conv
 * update from the request's slot state, and the conv window after every step
 * is recorded in a tape indexed by batch row (the tape index buffer is
 * arange(bs)), so that the state can later be rolled back to the accept
 * boundary.  Reading: the slot pool itself is not written here.
 */
int oracle_verify(int H, int K, int N, int L,
                  const double* in, int64_t in_stride,
                  const double* w, const double* bias,
                  const double* pool, int64_t num_slots, const int32_t* slot_idx,
                  double* tape, double* y) {
    if (H <= 0 || K <= 0 || N < 0 || L < 0 || in_stride < 3 * (int64_t)H) return -1;
    if (N == 0 || L == 0) return 0;
    if (!in || !w || !pool || !tape || !y) return -1;
    if (check_slots(slot_idx, N, num_slots)) return -1;
    const int64_t HK = (int64_t)H * K;
    int fail = 0;
    for (int i = 0; i < N; ++i) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
        for (int h = 0; h < H; ++h) {
            double S[64];
            if (K > 64) { fail = 1; continue; }
            for (int k = 0; k < K; ++k) S[k] = pool[(int64_t)slot_idx[i] * HK + (int64_t)h * K + k];
            for (int s = 0; s < L; ++s) {
                const int64_t r = (int64_t)i * L + s;
                const double* row = in + r * in_stride;
                for (int k = 0; k + 1 < K; ++k) S[k] = S[k + 1];
                S[K - 1] = row[h] * row[2 * H + h];
                double conv = 0.0;
                for (int k = 0; k < K; ++k) conv += w[(int64_t)h * K + k] * S[k];
                if (bias) conv += bias[h];
                y[r * H + h] = row[H + h] * conv;
                for (int k = 0; k < K; ++k) tape[(r * H + h) * K + k] = S[k];
            }
        }
    }
    return fail ? -1 : 0;
}

/*
 * Post-verify commit at the accept boundary.
 *
 * SGLang PR 31041 summary: the tape exists so the state can be rolled back to
 * the accept boundary; the commit itself is the generic post-verify hybrid
 * state commit (related PR 32828).  Reading: with accept length a, tokens
 * 0..a-1 are kept, so the slot receives tape[i][a-1]; a = 0 keeps the state
 * the slot already holds.
 */
int oracle_commit(int H, int K, int N, int L,
                  const double* tape, const int32_t* accept,
                  double* pool, int64_t num_slots, const int32_t* slot_idx) {
    if (H <= 0 || K <= 0 || N < 0 || L < 0) return -1;
    if (N == 0) return 0;
    if (!accept || !pool) return -1;
    if (check_slots(slot_idx, N, num_slots)) return -1;
    for (int i = 0; i < N; ++i)
        if (accept[i] < 0 || accept[i] > L) return -1;
    const int64_t HK = (int64_t)H * K;
    for (int i = 0; i < N; ++i) {
        const int a = accept[i];
        if (a == 0) continue;
        if (!tape) return -1;
        const double* src = tape + ((int64_t)i * L + (a - 1)) * HK;
        memcpy(pool + (int64_t)slot_idx[i] * HK, src, sizeof(double) * (size_t)HK);
    }
    return 0;
}

/*
 * Backward of the prefill forward.
 *
 * Liger-Kernel PR 1317, section "Kernel changes / Gated short convolution":
 * the op's backward gives the input gradient through the fused B and C gates
 * and a weight gradient with all K taps of a channel together.  The formulas
 * are the chain rule applied to the forward definition (the pages print
 * none).  With X the padded history used in oracle_prefill, for one channel
 * of one sequence:
 *     conv[t] = bias + sum_k w[k] X[t+1+k],  y[t] = C[t] conv[t],
 *     X[k] = S0[k] (k < K),  X[K+u] = B[u] xv[u],  final state F = X[T .. T+K-1].
 * With g[t] = dy[t] C[t] the chain rule gives, term by term:
 *     dC[t]  = dy[t] conv[t]
 *     dX[j]  = sum over (t, k) with t+1+k = j of w[k] g[t]   (every conv term)
 *              + dF[j-T] for j >= T                          (the final state)
 *     dB[u]  = dX[K+u] xv[u],   dxv[u] = dX[K+u] B[u]
 *     dS0[k] = dX[k]            (k < K)
 *     dW[k]  = sum over sequences and t of g[t] X[t+1+k]
 *     dbias  = sum over sequences and t of g[t]
 * dX is accumulated by scattering each conv term, in token order.
 */
int oracle_backward(int H, int K, int64_t total_T,
                    const double* in, int64_t in_stride,
                    const int32_t* cu, int N,
                    const double* w, const double* bias,
                    const double* pool, int64_t num_slots, const int32_t* slot_idx,
                    const double* dy, const double* d_final,
                    double* d_in, double* dW, double* dbias, double* d_init) {
    if (H <= 0 || K <= 0 || total_T < 0 || in_stride < 3 * (int64_t)H) return -1;
    if (check_cu(cu, N, total_T)) return -1;
    if (pool && check_slots(slot_idx, N, num_slots)) return -1;
    if (!w || !dW) return -1;
    const int64_t HK = (int64_t)H * K;
    int64_t maxT = 0;
    for (int i = 0; i < N; ++i) {
        const int64_t T = (int64_t)cu[i + 1] - cu[i];
        if (T > maxT) maxT = T;
    }
    if (maxT > 0 && (!in || !dy || !d_in)) return -1;
    int fail = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int h = 0; h < H; ++h) {
        double* X = (double*)malloc(sizeof(double) * (size_t)(K + maxT));
        double* dX = (double*)malloc(sizeof(double) * (size_t)(K + maxT));
        if (!X || !dX) { fail = 1; free(X); free(dX); continue; }
        const double b = bias ? bias[h] : 0.0;
        double db = 0.0;
        for (int k = 0; k < K; ++k) dW[(int64_t)h * K + k] = 0.0;
        for (int i = 0; i < N; ++i) {
            const int64_t r0 = cu[i];
            const int64_t T = (int64_t)cu[i + 1] - cu[i];
            for (int k = 0; k < K; ++k)
                X[k] = pool ? pool[(int64_t)slot_idx[i] * HK + (int64_t)h * K + k] : 0.0;
            for (int64_t u = 0; u < T; ++u) {
                const double* row = in + (r0 + u) * in_stride;
                X[K + u] = row[h] * row[2 * H + h];
            }
            for (int64_t j = 0; j < K + T; ++j) dX[j] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double* row = in + (r0 + t) * in_stride;
                const double dyt = dy[(r0 + t) * H + h];
                double conv = b;
                for (int k = 0; k < K; ++k) conv += w[(int64_t)h * K + k] * X[t + 1 + k];
                const double g = dyt * row[H + h];
                d_in[(r0 + t) * 3 * H + H + h] = dyt * conv;             /* dC */
                for (int k = 0; k < K; ++k) {
                    dX[t + 1 + k] += w[(int64_t)h * K + k] * g;
                    dW[(int64_t)h * K + k] += g * X[t + 1 + k];
                }
                db += g;
            }
            if (d_final)
                for (int k = 0; k < K; ++k) dX[T + k] += d_final[(int64_t)i * HK + (int64_t)h * K + k];
            for (int64_t u = 0; u < T; ++u) {
                const double* row = in + (r0 + u) * in_stride;
                d_in[(r0 + u) * 3 * H + h] = dX[K + u] * row[2 * H + h];          /* dB  */
                d_in[(r0 + u) * 3 * H + 2 * H + h] = dX[K + u] * row[h];          /* dxv */
            }
            if (d_init)
                for (int k = 0; k < K; ++k) d_init[(int64_t)i * HK + (int64_t)h * K + k] = dX[k];
        }
        if (dbias) dbias[h] = db;
        free(X);
        free(dX);
    }
    return fail ? -1 : 0;
}

/* MAX Pipelines LFM2 article, "ShortConv implementation (LFM2ShortConv)": the
 * in_proj layer projects the hidden state into the three parts b, c, xv.  The
 * plain definition of that linear map, one dot product per output element. */
int oracle_in_proj(int64_t rows, int D, int n_out,
                   const double* x, int64_t x_stride, const double* W_in,
                   double* out) {
    if (rows < 0 || D <= 0 || n_out <= 0 || x_stride < D) return -1;
    if (rows == 0) return 0;
    if (!x || !W_in || !out) return -1;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t t = 0; t < rows; ++t) {
        const double* xr = x + t * x_stride;
        for (int j = 0; j < n_out; ++j) {
            const double* wr = W_in + (int64_t)j * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += xr[d] * wr[d];
            out[t * n_out + j] = acc;
        }
    }
    return 0;
}

/* SGLang PR 31041 summary, implementation item 2 and its shortconv_target_verify
 * excerpt: the conv update there takes Bx (already gated; the C gate is left to
 * out_proj) as a [batch, channels, block] tensor, the slot pool, the weight and
 * bias, and returns the conv output in the same layout, writing one conv window
 * per draft token to the tape.  Written here on the padded history X = [state |
 * bx], as the prefill above is. */
int oracle_conv_update(int H, int K, int N, int L,
                       const double* bx, const double* w, const double* bias,
                       double* pool, int64_t num_slots, const int32_t* slot_idx,
                       double* tape, double* out) {
    if (H <= 0 || K <= 0 || N < 0 || L < 0) return -1;
    if (N == 0 || L == 0) return 0;
    if (!bx || !w || !pool || !out) return -1;
    if (check_slots(slot_idx, N, num_slots)) return -1;
    const int64_t HK = (int64_t)H * K;
    int fail = 0;
    for (int i = 0; i < N; ++i) {
        double* S = pool + (int64_t)slot_idx[i] * HK;
#pragma omp parallel for num_threads(g_threads) schedule(static)
        for (int h = 0; h < H; ++h) {
            double* X = (double*)malloc(sizeof(double) * (size_t)(K + L));
            if (!X) { fail = 1; continue; }
            for (int k = 0; k < K; ++k) X[k] = S[(int64_t)h * K + k];
            for (int s = 0; s < L; ++s) X[K + s] = bx[((int64_t)i * H + h) * L + s];
            for (int s = 0; s < L; ++s) {
                double conv = 0.0;
                for (int k = 0; k < K; ++k) conv += w[(int64_t)h * K + k] * X[s + 1 + k];
                if (bias) conv += bias[h];
                out[((int64_t)i * H + h) * L + s] = conv;
                if (tape)
                    for (int k = 0; k < K; ++k) tape[(((int64_t)i * L + s) * H + h) * K + k] = X[s + 1 + k];
            }
            if (!tape)
                for (int k = 0; k < K; ++k) S[(int64_t)h * K + k] = X[L + k];
            free(X);
        }
    }
    return fail ? -1 : 0;
}
