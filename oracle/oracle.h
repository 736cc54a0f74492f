/*
 * oracle.h -- fp64 CPU oracle for the LFM2 gated short causal convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library, and it never calls the library.
 *
 * What it computes (all arithmetic in double on the exact input values):
 *
 *   MAX Pipelines LFM2 architecture article, section "ShortConv implementation
 *   (LFM2ShortConv)": the in_proj output row of a token is split, in order,
 *   into three H-wide parts b, c and xv; bx = b * xv; the conv weight has shape
 *   [H, 1, K] with K = conv_L_cache; a per-request state [H, K] is advanced one
 *   token at a time by dropping its oldest column and appending bx; the conv
 *   output of the token is the sum over the K columns of state * weight, and
 *   the op returns y = c * conv_out together with the new state.
 *
 *   Same article, section "Inference state management (ConvStateCache)": each
 *   slot holds a zero-initialised [H, K] buffer per conv layer; requests own
 *   slots; the new states are written back to the request's slot.
 *
 *   SGLang PR 31041 summary ("DSpark speculative decoding for LFM2 and
 *   LFM2-MoE"), implementation item 2 and its source excerpt of
 *   shortconv_target_verify: in TARGET_VERIFY a block of draft tokens per
 *   request is convolved from the slot state and every step's conv window is
 *   written to a tape indexed by batch row, so that the state can be rolled
 *   back to the accept boundary after verification; a separate post-verify
 *   commit then installs the accepted window.
 *
 *   Liger-Kernel PR 1317 ("Add LFM2, LFM2-MoE, and LFM2-VL support"), section
 *   "Kernel changes / Gated short convolution": the op has a backward pass that
 *   returns the gradients through both gates (B and C) and the input, and a
 *   weight gradient that gathers all K taps of a channel.  The pages print no
 *   gradient formulas; the ones below are the derivatives of the forward
 *   definition.
 *
 * Readings where the pages leave a step open (each repeated at its function):
 *   - in_proj row layout: three contiguous H-wide blocks B | C | xv.
 *   - The state holds K entries, oldest first; weight tap K-1 multiplies the
 *     current token's bx.  Entry 0 of an incoming state never reaches an output.
 *   - Prefill continues from the slot state (zero for a new request, or when no
 *     pool is given); its final state is the last K entries of
 *     [state | bx of the sequence's tokens].
 *   - Verify leaves the pool untouched; tape[i][s] is the state after token s
 *     of batch row i; commit with accept length a > 0 installs tape[i][a-1],
 *     a = 0 keeps the old state.
 *   - Conv bias (optional, [H]): added to conv before the C gate.  The MAX
 *     article's weight-name mapping carries a conv bias and SGLang's excerpt
 *     passes one to its conv update; the released LFM2 checkpoints are
 *     bias-free (Liger-Kernel PR, "Gated short convolution").
 *   - in_proj (the fused forward only): a linear map of the hidden state x
 *     [rows][D] by a weight W_in [3H][D] in the usual out-by-in layout, no
 *     bias: column j of the in_proj row is sum_d x[d] * W_in[j][d].  The MAX
 *     article says only that in_proj projects the hidden state into the three
 *     parts; it names no in_proj bias.
 *   - Backward: the gradient of the initial state is returned on request, and a
 *     gradient arriving at the returned final state may be given (chunked
 *     training: chunk c+1's initial-state gradient is chunk c's final-state
 *     gradient).
 *
 * Layouts (all row-major, strides in elements):
 *   in     [rows][in_stride]   columns 0..H-1 = B, H..2H-1 = C, 2H..3H-1 = xv
 *   w      [H][K]
 *   pool   [num_slots][H][K]   (dense: slot stride H*K)
 *   y      [rows][H]
 *   tape   [N][L][H][K]
 *   dy     [rows][H]
 *   d_in   [rows][3H]          dB | dC | dxv
 *   dW     [H][K]
 *   bias   [H] (NULL = no bias), dbias [H]
 *   d_final, d_init  [N][H][K]  (gradients of each sequence's final / initial state)
 *   x      [rows][x_stride]    hidden states (D used), W_in [3H][D]
 *
 * Every function returns 0 on success and -1 if an argument is out of range
 * (the oracle checks what it needs to stay in bounds; it is not a validator).
 */
#ifndef LFM2SC_ORACLE_H
#define LFM2SC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP).
 * Parallelism is over channels only; the arithmetic of every output element
 * is the same whatever the thread count. */
void oracle_set_threads(int n);
int oracle_get_threads(void);

/* Ragged prefill.  Sequences are the row ranges [cu[i], cu[i+1]).  pool may be
 * NULL: zero initial state and no state written.  Otherwise the initial state
 * of sequence i is pool[slot_idx[i]], and after all outputs are computed the
 * final state is written back to that slot (a sequence of length 0 leaves its
 * slot unchanged). */
int oracle_prefill(int H, int K, int64_t total_T,
                   const double* in, int64_t in_stride,
                   const int32_t* cu, int N,
                   const double* w, const double* bias,
                   double* pool, int64_t num_slots, const int32_t* slot_idx,
                   double* y);

/* One decode token per sequence: row i of in belongs to sequence i, whose
 * state lives in pool[slot_idx[i]] and is advanced in place. */
int oracle_decode(int H, int K, int N,
                  const double* in, int64_t in_stride,
                  const double* w, const double* bias,
                  double* pool, int64_t num_slots, const int32_t* slot_idx,
                  double* y);

/* Verify window: L draft tokens per sequence, row i*L+s.  The pool is read
 * only; tape[i][s] receives the state after token s. */
int oracle_verify(int H, int K, int N, int L,
                  const double* in, int64_t in_stride,
                  const double* w, const double* bias,
                  const double* pool, int64_t num_slots, const int32_t* slot_idx,
                  double* tape, double* y);

/* Post-verify commit: for accept[i] > 0, pool[slot_idx[i]] = tape[i][accept[i]-1]. */
int oracle_commit(int H, int K, int N, int L,
                  const double* tape, const int32_t* accept,
                  double* pool, int64_t num_slots, const int32_t* slot_idx);

/* Backward of the prefill forward (same sequence and state conventions; pool
 * is read only and may be NULL for zero initial states).  dy is the gradient
 * of y; d_final (may be NULL = zero) the gradient of each sequence's returned
 * final state.  Writes d_in [total_T][3H] = dB | dC | dxv and dW [H][K], and,
 * when non-NULL, dbias [H] and d_init [N][H][K] (all overwritten). */
int oracle_backward(int H, int K, int64_t total_T,
                    const double* in, int64_t in_stride,
                    const int32_t* cu, int N,
                    const double* w, const double* bias,
                    const double* pool, int64_t num_slots, const int32_t* slot_idx,
                    const double* dy, const double* d_final,
                    double* d_in, double* dW, double* dbias, double* d_init);

/* Conv update on gated inputs in the [batch][channel][token] order (the layout
 * SGLang's verify path hands its conv update, with the C gate left to
 * out_proj): X = [state | bx of the L tokens] per channel, out[i][h][s] =
 * bias[h] + sum_k w[h][k] X[s+1+k].  With a tape, tape[i][s] = X[s+1 .. s+K]
 * and the pool is left as it is; with tape NULL, the slot receives
 * X[L .. L+K-1].  bx and out dense [N][H][L], tape [N][L][H][K]. */
int oracle_conv_update(int H, int K, int N, int L,
                       const double* bx, const double* w, const double* bias,
                       double* pool, int64_t num_slots, const int32_t* slot_idx,
                       double* tape, double* out);

/* in_proj = x W_in^T for the fused forward: out[t][j] = sum over d (ascending) of
 * x[t][d] * W_in[j][d], for t < rows, j < n_out; out is dense [rows][n_out]. */
int oracle_in_proj(int64_t rows, int D, int n_out,
                   const double* x, int64_t x_stride, const double* W_in,
                   double* out);

#ifdef __cplusplus
}
#endif
#endif
