/*
 * lfm2sc.h -- C ABI of liblfm2sc.so: the LFM2 gated short causal convolution
 * ("ShortConv") on AMD Instinct MI355X (gfx950).
 *
 * The op (MAX Pipelines LFM2 architecture article, section "ShortConv
 * implementation (LFM2ShortConv)"): the in_proj output row of a token is split,
 * in order, into three H-wide parts B, C and xv; bx = B * xv; a per-sequence
 * state of K columns per channel (K = conv_L_cache, 3 for LFM2-1.2B) is
 * advanced by dropping its oldest column and appending bx; the conv output is
 * the tap-weighted sum of the state with weight [H, K] (the [H, 1, K] depthwise
 * kernel with its unit axis dropped); y = C * conv; the new state is returned.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers unless stated otherwise; the caller
 *    owns every buffer.  The library allocates no device memory and keeps no
 *    device state between calls (lfm2sc_backward_noalloc's fixed scratch array
 *    aside), and is safe to call from several host threads.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *    the null stream).  The return code covers host-side argument checks and
 *    launch errors only; a fault inside a kernel surfaces at the caller's next
 *    synchronisation.
 *  - dtype: LFM2SC_BF16 or LFM2SC_F32.  It applies to the in_proj rows, the
 *    weight, the state pool, y, the tape, dy and d_in alike.  Arithmetic is
 *    fp32 in registers (fp64 in the backward with fp32 I/O, where products of
 *    two fp32 values are exact); each output element is rounded once (RNE)
 *    when stored.
 *    In bf16 mode B*xv and dy*C are exact in fp32, so every stored state or
 *    tape entry equals the exact value rounded to bf16.
 *  - Layouts are row-major; every "stride" is in ELEMENTS between consecutive
 *    rows.  in_proj rows hold B in columns [0, H), C in [H, 2H), xv in
 *    [2H, 3H) (the split order b, c, xv of the ShortConv section above).
 *  - The state pool is [num_slots][slot_stride] with slot s holding an [H][K]
 *    block (channel-major, the K columns of a channel contiguous, oldest
 *    first), i.e. the per-slot [1, hidden, conv_L_cache] buffer of the article's
 *    section "Inference state management (ConvStateCache)".  Sequences name
 *    their slot through slot_idx; slots must be distinct within a call and are
 *    claimed and released by the caller (the library does no slot allocation).
 *  - Requirements checked on the host: 8 <= H, H % 8 == 0; 1 <= K <= 4; every
 *    device base pointer 16-byte aligned (dW: 4-byte); every stride a multiple
 *    of 8 elements; in_stride >= 3H, y_stride >= H, dy_stride >= H,
 *    din_stride >= 3H, slot_stride >= H*K.
 *  - bias: optional conv bias [H] (same dtype as the weight, 16-byte aligned),
 *    added to conv before the C gate; NULL = none.  The MAX article's
 *    weight-name mapping carries a conv bias and SGLang's verify excerpt passes
 *    one to its conv update; the released LFM2 checkpoints are bias-free
 *    (Liger-Kernel LFM2 PR, "Gated short convolution").
 *  - Device-side data (slot indices, row offsets, accept lengths) cannot be
 *    checked on the host without a synchronisation.  Kernels never access
 *    memory outside the buffers described by the size arguments: a slot index
 *    outside [0, num_slots) makes that sequence skip every state read and write
 *    (treated as a zero state, nothing written back); row offsets are clamped
 *    to [0, total_T]; an accept length outside [0, L] commits nothing.  Set the
 *    environment variable LFM2SC_CHECK=1 to have each call verify these
 *    preconditions on the device, synchronise, and return
 *    LFM2SC_ERR_PRECONDITION when one fails (slow; for debugging).  The check
 *    reads its verdict back through one device flag of the library, so
 *    checking calls from several host threads take turns on a process-wide
 *    lock (they stay correct, and each one synchronises its own stream).
 *  - Outputs must not overlap inputs.  Nothing is accumulated into an output:
 *    y, tape, d_in and dW are overwritten.  Rows of y / d_in that belong to no
 *    sequence (outside [cu_seqlens[0], cu_seqlens[N])) are not written.
 */
#ifndef LFM2SC_H
#define LFM2SC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LFM2SC_ABI_VERSION 6

enum lfm2sc_dtype { LFM2SC_BF16 = 0, LFM2SC_F32 = 1 };

enum lfm2sc_status {
    LFM2SC_OK = 0,
    LFM2SC_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                          */
    LFM2SC_ERR_BAD_SHAPE = 2,      /* H, K, a count, a stride or a size is out of range   */
    LFM2SC_ERR_ALIGNMENT = 3,      /* a pointer or stride breaks the alignment rules      */
    LFM2SC_ERR_UNSUPPORTED = 4,    /* dtype, K or bias not supported by this version      */
    LFM2SC_ERR_WORKSPACE = 5,      /* workspace NULL or smaller than required             */
    LFM2SC_ERR_PRECONDITION = 6,   /* LFM2SC_CHECK=1 found bad device-side data           */
    LFM2SC_ERR_HIP = 7             /* the HIP runtime reported an error at launch         */
};

/*
 * Ragged (packed) prefill.
 *
 * Passage: MAX Pipelines LFM2 article, "ShortConv implementation
 * (LFM2ShortConv)" (per-token state update, conv, C gate, new state) and
 * "Batching and weight adaptation" / the graph's packed tokens with row
 * offsets and one [H, K] state per request.
 *
 * in_proj    [total_T][in_stride]  packed rows of all sequences (B | C | xv).
 * cu_seqlens [num_seqs+1] int32    sequence i owns rows [cu[i], cu[i+1]);
 *                                  non-decreasing; cu[N] <= total_T.
 * weight     [H][K].  bias: [H] or NULL.
 * state_pool [num_slots][slot_stride] or NULL.  NULL: every sequence starts
 *            from a zero state and no state is written (training forward).
 *            Otherwise sequence i starts from pool[slot_idx[i]] and, in
 *            place, that slot receives the last K columns of
 *            [initial state | bx of the sequence's tokens] (a sequence of
 *            length 0 leaves it unchanged, one shorter than K keeps part of the
 *            old state).  Slots not named in slot_idx are never touched.
 * slot_idx   [num_seqs] int32, distinct (ignored when state_pool is NULL).
 * y          [total_T][y_stride]   y = C * conv.
 * Packed sequences never share history: a sequence's first token sees only its
 * own initial state (the hazard the InfiniLM LFM2 PR, "Notes for reviewers",
 * avoids by rejecting packed prefill).
 */
int lfm2sc_prefill_ragged(int dtype, int H, int K,
                          const void* in_proj, int64_t in_stride, int64_t total_T,
                          const int32_t* cu_seqlens, int num_seqs,
                          const void* weight, const void* bias,
                          void* state_pool, int64_t num_slots, int64_t slot_stride,
                          const int32_t* slot_idx,
                          void* y, int64_t y_stride, void* stream);

/*
 * One decode token per sequence.
 *
 * Passage: MAX Pipelines LFM2 article, "ShortConv implementation" (take the
 * request's [H, K] state, shift in bx, conv, gate, write the state back with a
 * scatter by slot) and "Inference state management" (the slot pool).
 *
 * in_proj    [num_seqs][in_stride]  row i is the new token of sequence i.
 * state_pool [num_slots][slot_stride] required; pool[slot_idx[i]] is advanced
 *            in place by one token.  Slots not named are never touched.
 * y          [num_seqs][y_stride].
 */
int lfm2sc_decode_step(int dtype, int H, int K,
                       const void* in_proj, int64_t in_stride, int num_seqs,
                       const void* weight, const void* bias,
                       void* state_pool, int64_t num_slots, int64_t slot_stride,
                       const int32_t* slot_idx,
                       void* y, int64_t y_stride, void* stream);

/*
 * Speculative-decoding verify window.
 *
 * Passage: SGLang PR 31041 summary (DSpark speculative decoding for LFM2),
 * implementation item 2 and its shortconv_target_verify excerpt: a block of L
 * draft tokens per request is convolved from the request's slot state, and the
 * conv window after every step is stored in a tape indexed by batch row so the
 * state can be rolled back to the accept boundary; the tape is mandatory (the
 * excerpt refuses to run without one).
 *
 * in_proj    [num_seqs*L][in_stride]  row i*L+s is draft token s of sequence i.
 * state_pool read only: nothing is written to the pool by this call.
 * windows    [num_seqs][L][H][K] (dense) required: windows[i][s] = the state of
 *            sequence i after draft token s.  NULL -> LFM2SC_ERR_NULL_POINTER.
 * y          [num_seqs*L][y_stride].
 */
int lfm2sc_verify_window(int dtype, int H, int K,
                         const void* in_proj, int64_t in_stride, int num_seqs, int L,
                         const void* weight, const void* bias,
                         const void* state_pool, int64_t num_slots, int64_t slot_stride,
                         const int32_t* slot_idx,
                         void* windows,
                         void* y, int64_t y_stride, void* stream);

/*
 * Post-verify commit (rollback to the accept boundary).
 *
 * Passage: SGLang PR 31041 summary, implementation item 2 (the tape exists for
 * rollback at the accept boundary) and its related-work note on the generic
 * post-verify hybrid-state commit.
 *
 * windows    [num_seqs][L][H][K] as written by lfm2sc_verify_window.
 * accept_len [num_seqs] int32 in [0, L]: a > 0 copies windows[i][a-1] into
 *            pool[slot_idx[i]] (tokens 0..a-1 kept); a == 0 leaves the slot.
 */
int lfm2sc_commit_window(int dtype, int H, int K,
                         const void* windows, int num_seqs, int L,
                         const int32_t* accept_len,
                         void* state_pool, int64_t num_slots, int64_t slot_stride,
                         const int32_t* slot_idx, void* stream);

/*
 * Bytes of device workspace lfm2sc_backward needs for these sizes (it holds
 * per-window partial sums of dW and dbias).  Returns 0 for invalid sizes.
 */
size_t lfm2sc_backward_workspace_bytes(int dtype, int H, int K, int64_t total_T, int num_seqs);

/*
 * Backward of lfm2sc_prefill_ragged (training).
 *
 * Passage: Liger-Kernel PR 1317 ("Add LFM2, LFM2-MoE, and LFM2-VL support"),
 * "Kernel changes / Gated short convolution": gradients through both gates and
 * the conv input, and a weight gradient that gathers all K taps of a channel.
 * The formulas are the chain rule on the forward: with X = [initial state |
 * bx of the sequence], conv[t] = bias + sum_k w[k] X[t+1+k], g = dy*C,
 *   dC = dy * conv;  dX[j] = sum over (t, k) with t+1+k = j of w[k] g[t]
 *   (+ the final-state gradient on the last K entries of X);
 *   dB = dX[K+u] * xv;  dxv = dX[K+u] * B;  d_init = dX[0..K-1];
 *   dW[h][k] = sum over tokens of g * X[t+1+k];  dbias[h] = sum over tokens of g.
 *
 * in_proj, cu_seqlens, weight, bias: as for the forward call (bias may be NULL).
 * init_state_pool / num_slots / slot_stride / slot_idx: the initial states the
 *            forward started from (read only); NULL pool = zero states.
 * dy         [total_T][dy_stride].
 * d_final_state [num_seqs][H][K] dense, or NULL (= zero): gradient arriving at
 *            each sequence's returned final state (chunked training: the
 *            d_init_state of the next chunk of the same sequences).
 * d_in_proj  [total_T][din_stride]  columns dB | dC | dxv (overwritten).
 * dW         [H][K] fp32 (overwritten); dbias [H] fp32 or NULL (overwritten).
 *            Both are reduced over all sequences and tokens in a fixed order,
 *            so results are bitwise reproducible.
 * d_init_state [num_seqs][H][K] dense, I/O dtype, or NULL: gradient of each
 *            sequence's initial state (overwritten; entry 0 of a sequence with
 *            at least one token is always 0, that entry being shifted out).
 * workspace  device buffer of at least lfm2sc_backward_workspace_bytes(...)
 *            bytes, 16-byte aligned; contents on entry are ignored.
 */
int lfm2sc_backward(int dtype, int H, int K,
                    const void* in_proj, int64_t in_stride, int64_t total_T,
                    const int32_t* cu_seqlens, int num_seqs,
                    const void* weight, const void* bias,
                    const void* init_state_pool, int64_t num_slots, int64_t slot_stride,
                    const int32_t* slot_idx,
                    const void* dy, int64_t dy_stride,
                    const void* d_final_state,
                    void* d_in_proj, int64_t din_stride,
                    float* dW, float* dbias,
                    void* d_init_state,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * lfm2sc_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and determinism as lfm2sc_backward,
 * without the workspace: the per-window partial sums live in a fixed array of
 * LFM2SC_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends (its address is looked up once per
 * device on the first call there).  The call itself allocates nothing.
 *
 * Limit: the call must need at most LFM2SC_NOALLOC_SCRATCH_BYTES of workspace,
 * i.e. lfm2sc_backward_workspace_bytes(...) <= LFM2SC_NOALLOC_SCRATCH_BYTES
 * (one 65,536-token sequence at H = 2048 needs 2 MiB; the workspace grows with
 * the number of sequences); a larger call returns LFM2SC_ERR_WORKSPACE before
 * any launch.  Every call on one GPU uses that GPU's one array: calls that
 * overlap on a GPU (other streams or host threads without ordering) race and
 * may return wrong dW / dbias.  Nothing in the array needs clearing between
 * calls (each call writes all of what it reads).
 */
#define LFM2SC_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int lfm2sc_backward_noalloc(int dtype, int H, int K,
                            const void* in_proj, int64_t in_stride, int64_t total_T,
                            const int32_t* cu_seqlens, int num_seqs,
                            const void* weight, const void* bias,
                            const void* init_state_pool, int64_t num_slots, int64_t slot_stride,
                            const int32_t* slot_idx,
                            const void* dy, int64_t dy_stride,
                            const void* d_final_state,
                            void* d_in_proj, int64_t din_stride,
                            float* dW, float* dbias,
                            void* d_init_state, void* stream);

/* Static text for a status code (never NULL). */
const char* lfm2sc_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* lfm2sc_last_error(void);

/*
 * Fused in_proj + ShortConv forward (bf16 only): the in_proj GEMM runs on the
 * matrix cores and the gated conv of lfm2sc_prefill_ragged runs in its
 * epilogue, so in_proj never has to be written to memory and read back.
 *
 * Passage: MAX Pipelines LFM2 article, "ShortConv implementation
 * (LFM2ShortConv)": in_proj projects each token's hidden state into b, c and
 * xv, which then go through the gated conv.  Reading: in_proj is the linear
 * map in_proj[t][j] = sum_d x[t][d] * W_in[j][d] with no bias (the article
 * names none).
 *
 * x           [total_T][x_stride] bf16 hidden states (the first D columns).
 * W_in        [3H][D] bf16, row-major (the usual out-by-in weight layout):
 *             rows [0, H) produce B, [H, 2H) C, [2H, 3H) xv.
 * cu_seqlens, weight, bias, state_pool, num_slots, slot_stride, slot_idx, y:
 *             as in lfm2sc_prefill_ragged (same state semantics).
 * in_proj_out [total_T][io_stride] bf16, or NULL: when given, receives
 *             B | C | xv rounded to bf16 (the in_proj the backward takes).
 * workspace   needed only when state_pool is given: at least
 *             lfm2sc_fused_prefill_workspace_bytes(...) bytes, 16-byte
 *             aligned.  The final states are staged there and a second kernel
 *             installs them into the slots once every tile has read its
 *             initial states.
 * Requirements beyond the shared ones: dtype LFM2SC_BF16 (else
 * LFM2SC_ERR_UNSUPPORTED); H % 64 == 0, D % 128 == 0, 3H*D*2 < 2^31 and
 * 256*x_stride*2 < 2^31 (else LFM2SC_ERR_BAD_SHAPE); x_stride >= D and
 * io_stride >= 3H, multiples of 8.
 * Accuracy: B, C and xv are fp32 sums over D and are not rounded before the
 * conv, so y and the final states carry one bf16 rounding of an fp32 result:
 * within the bf16 tolerance of the exact value, but not bit-equal to running
 * a GEMM into bf16 in_proj and then lfm2sc_prefill_ragged.  For D in {1024,
 * 1536, 2048} the call picks a tiling by size: wide tiles (H % 128 == 0) with
 * or without halo rows, or, for short inputs, split tiles whose waves each sum
 * a quarter of D, or mid tiles whose waves each sum half of it (the fp32 sums,
 * and so the results, may differ by rounding between tilings; each is
 * deterministic).  For testing, the environment variables LFM2SC_FUSED_SPLIT
 * (0: never split or mid tiles, 1: always, 32 or 64: split tiles with that
 * many channels, 128: mid tiles), LFM2SC_FUSED_HALO (0 or 1) and
 * LFM2SC_FUSED_WIDE (0: the 4-wave tile instead of the wide one) force one.
 * When to call it (measured on MI355X, D = H = 2048, K = 3, against a bf16
 * library GEMM into in_proj followed by lfm2sc_prefill_ragged): the fused call
 * is faster for short inputs (T <= 256, and 256 one-token sequences with a
 * pool: 20-55%) and for long forward-only inputs (T = 65,536 with y only: 5%),
 * level around T = 1,024 and T = 4,096, and slower between T ~ 1,280 and
 * 2,048 (12-34%), at T = 512-768 (4-7%), on a ragged batch of 8 sequences of
 * 64-2,048 tokens (~12%) and when in_proj_out is also wanted for the backward
 * (~7% at T = 65,536).  Callers should take the two-step path for those
 * shapes; the call does not switch to it by itself (it never runs a library
 * GEMM).
 */
int lfm2sc_fused_prefill(int dtype, int H, int K, int D,
                         const void* x, int64_t x_stride, int64_t total_T,
                         const int32_t* cu_seqlens, int num_seqs,
                         const void* W_in, const void* weight, const void* bias,
                         void* state_pool, int64_t num_slots, int64_t slot_stride,
                         const int32_t* slot_idx,
                         void* y, int64_t y_stride, void* in_proj_out, int64_t io_stride,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of lfm2sc_fused_prefill (0 when with_pool is 0). */
size_t lfm2sc_fused_prefill_workspace_bytes(int dtype, int H, int K, int num_seqs, int with_pool);

/*
 * The tiling lfm2sc_fused_prefill takes for these sizes, for tests and tuning
 * (host only: the one device query, the number of resident workgroups, falls
 * back to 256 without a device).  1: wide tiles (256 rows x 128 channels),
 * 2: wide tiles with halo rows, 3: the 4-wave tile (256 rows x 64 channels),
 * 32 or 64: split tiles of 64 rows and that many channels, 128: mid tiles
 * (128 rows x 64 channels); 0 when total_T == 0 (nothing is launched).  The
 * environment overrides named at lfm2sc_fused_prefill apply.  Returns
 * -LFM2SC_ERR_BAD_SHAPE for sizes lfm2sc_fused_prefill rejects (H, K, D as
 * there; total_T outside [0, 2^31)).
 */
int lfm2sc_fused_prefill_plan(int H, int K, int D, int64_t total_T);

/*
 * Conv update of gated inputs in [batch][channel][token] order with arbitrary
 * element strides: the layout-interop form of the verify / multi-token decode
 * step, for engines that gate B and xv themselves and keep the C gate for
 * out_proj.
 *
 * Passage: SGLang PR 31041 summary, implementation item 2 and its
 * shortconv_target_verify excerpt (the conv update takes Bx as a [batch,
 * channels, block] tensor -- there a transposed view of token-major rows --
 * with the slot pool, weight and bias, returns the conv output in the same
 * layout and writes one window per draft token to the tape).
 *
 * bx     element (n, h, t) at bx[n*bx_stride_n + h*bx_stride_h + t*bx_stride_t],
 *        n < num_seqs, h < H, t < L: the gated input B*xv of token t.
 * out    element (n, h, t) at out[n*out_stride_n + h*out_stride_h + t*out_stride_t]:
 *        bias[h] + sum_k weight[h][k] * X[t+1+k] with X = [slot state | bx of
 *        tokens 0..L-1] (no C gate).  out must not overlap bx.
 * state_pool, num_slots, slot_stride, slot_idx: as in lfm2sc_verify_window.
 * windows [num_seqs][L][H][K] (16-byte aligned) or NULL.  Given: windows[n][t]
 *        receives X[t+1 .. t+K] (the state after token t) and the pool is only
 *        read; commit with lfm2sc_commit_window.  NULL: each named slot
 *        receives X[L .. L+K-1] in place (the state after the L tokens).
 * Strides are in elements and must be >= 0; bx and out need only element
 * alignment.  When bx_stride_h == out_stride_h == 1, the other strides are
 * multiples of 8 and bx, out are 16-byte aligned, the kernel moves 16-byte
 * vectors; otherwise it accesses single elements (slower, same results).
 */
int lfm2sc_conv_update(int dtype, int H, int K, int num_seqs, int L,
                       const void* bx, int64_t bx_stride_n, int64_t bx_stride_h, int64_t bx_stride_t,
                       const void* weight, const void* bias,
                       void* state_pool, int64_t num_slots, int64_t slot_stride,
                       const int32_t* slot_idx, void* windows,
                       void* out, int64_t out_stride_n, int64_t out_stride_h, int64_t out_stride_t,
                       void* stream);

/* LFM2SC_ABI_VERSION of the loaded library. */
int lfm2sc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LFM2SC_H */
