// fwd.hip -- forward ShortConv kernels for gfx950: ragged prefill, decode,
// speculative verify window and post-verify commit.
//
// The op (MAX Pipelines LFM2 architecture article, "ShortConv implementation
// (LFM2ShortConv)"): bx = B * xv; the [H, K] state drops its oldest column and
// appends bx; conv = sum_k w[:, k] * state[:, k]; y = C * conv.
//
// All four kernels are HBM-streaming with a handful of FMAs per byte, so they
// are written for memory-level parallelism: 16-byte accesses, several token
// rows of loads issued before any arithmetic, no LDS and no barriers.
#include "common.hpp"
#include "kernels.hpp"

namespace lfm2sc {

// One token of one lane: bx = B*xv; conv over the K-1 history entries and bx;
// y = C*conv; the history shifts by one.  hist[c][k] holds X[t+1+k] (k < K-1)
// of the padded history X = [state | bx...] for the current token t.
template <typename E, int K>
__device__ __forceinline__ void fwd_token(const Raw8<E>& rb, const Raw8<E>& rc, const Raw8<E>& rx,
                                          const float (&wf)[kChPerLane][K], const float (&bv)[kChPerLane],
                                          float (&hist)[kChPerLane][K > 1 ? K - 1 : 1], rsrc_t yrow, uint32_t yoff) {
    float b[8], c[8], x[8], yv[8];
    to_f32(rb, b); to_f32(rc, c); to_f32(rx, x);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const float bx = b[ch] * x[ch];
        float conv = fmaf(wf[ch][K - 1], bx, bv[ch]);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fmaf(wf[ch][k], hist[ch][k], conv);
        yv[ch] = c[ch] * conv;
        if constexpr (K > 1) {
#pragma unroll
            for (int k = 0; k < K - 2; ++k) hist[ch][k] = hist[ch][k + 1];
            hist[ch][K - 2] = bx;
        }
    }
    bst8f<E, LFM2SC_FWD_NT>(yrow, yoff, yv);
}

// ------------------------------------------------------------------ prefill
// Work unit: one wave x one window of `sub` tokens x 512 channels.  A
// workgroup is 4 consecutive windows of the virtual ragged axis (see
// find_span), grid.y splits the channels.  Each lane streams its window's
// tokens in order, carrying the K-1 previous bx values in registers (the
// halo), so bx never reaches memory.
//
// In-place state update without a race: only the window holding a sequence's
// token 0 (the "owner") reads the slot; it also handles tokens 0..K-2 (the
// only ones that see the initial state) and writes the final state, which it
// forms from the slot (for entries the sequence does not overwrite) and the
// B, xv rows of the sequence's last K tokens.  No other wave touches the slot.
template <typename E, int K, int U, int TW>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs<E> a) {
    using Lay = WgLayout<TW>;
    const int wave = wave_id();
    const int lane = threadIdx.x % kWave;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= a.ntiles) return;
    const int ch0 = ((blockIdx.y * Lay::kCW + wave / TW) * kWave + lane) * kChPerLane;
    const int64_t gap = (int64_t)a.sub * TW;
    const int64_t v0 = (int64_t)tile * gap + (int64_t)(wave % TW) * a.sub;
    SeqSpan sp;
    if (!find_span(a.cu, a.N, a.total_T, gap, v0, v0 + a.sub, sp)) return;   // all lanes still active here
    if (ch0 >= a.H) return;
    int64_t lo = sp.lo, hi = sp.hi;
    const bool owner = (lo == 0);
    if (owner) {
        const int64_t m = (K - 1) < sp.T ? (K - 1) : sp.T;
        if (hi < m) hi = m;
    } else if (lo < K - 1) {
        lo = K - 1;
        if (lo >= hi) return;
    }
    const int H = a.H;
    const E* base = a.in + ch0;

    float wf[kChPerLane][K];
    load_block<E, K>(a.w + (int64_t)ch0 * K, wf);
    float bv[kChPerLane] = {};
    if (a.bias != nullptr) load_f32x8<E>(a.bias + ch0, bv);

    E* slotp = nullptr;
    if (owner && a.pool != nullptr) {
        const int64_t slot = a.slot_idx[sp.seq];
        if (slot_ok(slot, a.num_slots)) slotp = a.pool + slot * a.slot_stride + (int64_t)ch0 * K;
    }

    // The owner's final state needs bx of the sequence's last K tokens: those
    // loads are independent of everything else, so they are issued here, at the
    // window start, instead of costing an extra round trip after the last batch.
    Raw8<E> fin_b[K], fin_x[K];
    if (slotp) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t j = sp.T + k;   // index in the padded history [state | bx...]
            if (j >= K) {
                const E* row = base + (sp.r0 + j - K) * a.in_stride;
                fin_b[k] = ld8<E>(row);
                fin_x[k] = ld8<E>(row + 2 * H);
            }
        }
    }

    float hist[kChPerLane][K > 1 ? K - 1 : 1];
    if constexpr (K > 1) {
        if (owner) {
            float s0[kChPerLane][K];
            if (slotp) {
                load_block<E, K>(slotp, s0);
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int k = 0; k < K; ++k) s0[c][k] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int k = 0; k < K - 1; ++k) hist[c][k] = s0[c][k + 1];
        } else {
            // lo >= K-1: the K-1 tokens before lo are rows of this sequence.
#pragma unroll
            for (int k = 0; k < K - 1; ++k) {
                const E* row = base + (sp.r0 + lo - (K - 1) + k) * a.in_stride;
                float b[8], x[8];
                load_f32x8<E>(row, b);
                load_f32x8<E>(row + 2 * H, x);
#pragma unroll
                for (int c = 0; c < 8; ++c) hist[c][k] = b[c] * x[c];
            }
        }
    }

    // Streamed rows through buffer descriptors: per-lane byte offsets of this
    // lane's 8 channels in the B, C and xv blocks of an in_proj row and in a y row.
    const uint32_t offB = (uint32_t)ch0 * sizeof(E);
    const uint32_t offC = offB + (uint32_t)H * sizeof(E);
    const uint32_t offX = offB + 2u * (uint32_t)H * sizeof(E);
    const uint32_t in_row_bytes = 3u * (uint32_t)H * sizeof(E);
    const uint32_t y_row_bytes = (uint32_t)H * sizeof(E);
    const E* in_rows = a.in + sp.r0 * a.in_stride;
    E* y_rows = a.y + sp.r0 * a.y_stride;
    int64_t t = lo;
    // Rows in flight: batches of U rows, all loads of a batch issued together.
    auto load_batch = [&](Raw8<E> (&rb)[U], Raw8<E> (&rc)[U], Raw8<E> (&rx)[U], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const rsrc_t row = row_rsrc(in_rows + (t0 + u) * a.in_stride, in_row_bytes);
            rb[u] = bld8<E, LFM2SC_FWD_NT>(row, offB);
            rc[u] = bld8<E, LFM2SC_FWD_NT>(row, offC);
            rx[u] = bld8<E, LFM2SC_FWD_NT>(row, offX);
        }
    };
    auto use_batch = [&](const Raw8<E> (&rb)[U], const Raw8<E> (&rc)[U], const Raw8<E> (&rx)[U], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            fwd_token<E, K>(rb[u], rc[u], rx[u], wf, bv, hist, row_rsrc(y_rows + (t0 + u) * a.y_stride, y_row_bytes), offB);
    };
    for (; t + U <= hi; t += U) {
        Raw8<E> rb[U], rc[U], rx[U];
        load_batch(rb, rc, rx, t);
        use_batch(rb, rc, rx, t);
    }
    // Remainder (< U rows): one partial batch, all its loads issued together.
    if (t < hi) {
        const int n = (int)(hi - t);
        Raw8<E> rb[U], rc[U], rx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < n) {
                const rsrc_t row = row_rsrc(in_rows + (t + u) * a.in_stride, in_row_bytes);
                rb[u] = bld8<E, LFM2SC_FWD_NT>(row, offB);
                rc[u] = bld8<E, LFM2SC_FWD_NT>(row, offC);
                rx[u] = bld8<E, LFM2SC_FWD_NT>(row, offX);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < n)
                fwd_token<E, K>(rb[u], rc[u], rx[u], wf, bv, hist, row_rsrc(y_rows + (t + u) * a.y_stride, y_row_bytes),
                                offB);
    }

    if (slotp) {
        // Final state = X[T .. T+K-1] of the padded history [state | bx...].
        const int64_t T = sp.T;
        float s0[kChPerLane][K];
        if (T < K) load_block<E, K>(slotp, s0);
        float fin[kChPerLane][K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t j = T + k;
            if (j < K) {
#pragma unroll
                for (int c = 0; c < 8; ++c) fin[c][k] = s0[c][j];
            } else {
                float b[8], x[8];
                to_f32(fin_b[k], b);
                to_f32(fin_x[k], x);
#pragma unroll
                for (int c = 0; c < 8; ++c) fin[c][k] = b[c] * x[c];
            }
        }
        store_block<E, K>(slotp, fin);
    }
}

// ------------------------------------------------------------------ small calls
// Decode, verify and commit run one wave per 512-channel group of a sequence
// (and, for verify, of a draft step), on a flat grid of work items with a
// grid-stride loop for counts above the grid limit.  Decode and commit take
// the channel group fastest (b = i * groups + g): the waves touching one
// in_proj row and one slot block are consecutive workgroups and run together,
// so each row and block is read and written whole at one time (4% faster
// than one pass per channel group over every sequence).  Verify keeps the
// sequence fastest (b = (z * groups + g) * N + i), measured 4% faster for it.
struct SmallIdx { int i, g, z; };
__device__ __forceinline__ SmallIdx small_idx(int64_t b, int groups) {
    return SmallIdx{(int)(b / groups), (int)(b % groups), 0};
}
__device__ __forceinline__ SmallIdx small_idx_seq_fastest(int64_t b, int N, int groups) {
    const int64_t q = b / N;
    return SmallIdx{(int)(b % N), (int)(q % groups), (int)(q / groups)};
}
inline unsigned small_grid(int64_t items) { return (unsigned)(items < (1 << 30) ? items : (1 << 30)); }
inline int small_groups(int64_t lanes) { return (int)((lanes + kSmallBlock - 1) / kSmallBlock); }

// ------------------------------------------------------------------ decode
// One token per sequence, a lane = 8 channels.  Every load of a lane is
// independent of the others except the state, whose address needs the
// (wave-uniform, scalar-loaded) slot index.
// Decode with the state block staged through LDS (StateStage).
template <typename E, int K>
__device__ __forceinline__ void decode_one_staged(const DecodeArgs<E>& a, int i, int g) {
    const int lane = (int)threadIdx.x;
    const int ch0 = (g * kSmallBlock + lane) * kChPerLane;
    const bool on = ch0 < a.H;
    const int H = a.H;
    const int64_t slot = a.slot_idx[i];
    const bool ok = slot_ok(slot, a.num_slots);
    const int chw = g * kSmallBlock * kChPerLane;   // the wave's first channel
    const int nch = H - chw < kSmallBlock * kChPerLane ? H - chw : kSmallBlock * kChPerLane;
    const rsrc_t blk = row_rsrc(ok ? (const void*)(a.pool + slot * a.slot_stride + (int64_t)chw * K) : (const void*)a.w,
                                ok ? (uint32_t)nch * K * (uint32_t)sizeof(E) : 0u);
    const int chl = on ? ch0 : chw;   // lanes past H work on a valid address and store nothing
    const E* row = a.in + (int64_t)i * a.in_stride + chl;
    const Raw8<E> rb = ld8s<E, LFM2SC_DEC_NT>(row), rc = ld8s<E, LFM2SC_DEC_NT>(row + H),
                  rx = ld8s<E, LFM2SC_DEC_NT>(row + 2 * H);
    float wf[kChPerLane][K];
    load_block<E, K>(a.w + (int64_t)chl * K, wf);
    float bv[kChPerLane] = {};
    if (a.bias != nullptr) load_f32x8<E>(a.bias + chl, bv);
    __shared__ StateStage<E, K> stage;
    float s[kChPerLane][K];
    stage_load<E, K>(stage, blk, lane, s);
    float b[8], c8[8], x[8], yv[8];
    to_f32(rb, b); to_f32(rc, c8); to_f32(rx, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int k = 0; k < K - 1; ++k) s[c][k] = s[c][k + 1];
        s[c][K - 1] = b[c] * x[c];
        float conv = fmaf(wf[c][K - 1], s[c][K - 1], bv[c]);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fmaf(wf[c][k], s[c][k], conv);
        yv[c] = c8[c] * conv;
    }
    if (on) store_f32x8s<E, LFM2SC_DEC_NT>(a.y + (int64_t)i * a.y_stride + ch0, yv);
    stage_store<E, K>(stage, blk, lane, s);
}

// Decode with each lane loading and storing its own 8 x K state elements.
template <typename E, int K>
__device__ __forceinline__ void decode_one(const DecodeArgs<E>& a, int i, int g) {
    const int ch0 = (g * kSmallBlock + threadIdx.x) * kChPerLane;
    if (ch0 >= a.H) return;
    const int H = a.H;
    const int64_t slot = a.slot_idx[i];
    const bool ok = slot_ok(slot, a.num_slots);
    const E* row = a.in + (int64_t)i * a.in_stride + ch0;
    const Raw8<E> rb = ld8s<E, LFM2SC_DEC_NT>(row), rc = ld8s<E, LFM2SC_DEC_NT>(row + H),
                  rx = ld8s<E, LFM2SC_DEC_NT>(row + 2 * H);
    float wf[kChPerLane][K];
    load_block<E, K>(a.w + (int64_t)ch0 * K, wf);
    float bv[kChPerLane] = {};
    if (a.bias != nullptr) load_f32x8<E>(a.bias + ch0, bv);
    E* sp = ok ? a.pool + slot * a.slot_stride + (int64_t)ch0 * K : nullptr;
    float s[kChPerLane][K];
    if (ok) {
        load_block_s<E, K, (LFM2SC_DEC_NT & 4) ? 1 : 0>(sp, s);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int k = 0; k < K; ++k) s[c][k] = 0.f;
    }
    float b[8], c8[8], x[8], yv[8];
    to_f32(rb, b); to_f32(rc, c8); to_f32(rx, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int k = 0; k < K - 1; ++k) s[c][k] = s[c][k + 1];
        s[c][K - 1] = b[c] * x[c];
        float conv = fmaf(wf[c][K - 1], s[c][K - 1], bv[c]);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fmaf(wf[c][k], s[c][k], conv);
        yv[c] = c8[c] * conv;
    }
    store_f32x8s<E, LFM2SC_DEC_NT>(a.y + (int64_t)i * a.y_stride + ch0, yv);
    if (ok) store_block_s<E, K, (LFM2SC_DEC_NT & 8) ? 2 : 0>(sp, s);
}

template <typename E, int K, bool STAGED>
__global__ __launch_bounds__(kSmallBlock) void decode_kernel(const DecodeArgs<E> a, int groups) {
    const int64_t items = (int64_t)a.N * groups;
    for (int64_t b = blockIdx.x; b < items; b += gridDim.x) {
        const SmallIdx ix = small_idx(b, groups);
        if constexpr (STAGED) decode_one_staged<E, K>(a, ix.i, ix.g);
        else decode_one<E, K>(a, ix.i, ix.g);
    }
}

// ------------------------------------------------------------------ verify
// L draft tokens per sequence from the slot state (read only); after each
// token the lane's 8 x K window goes to the tape windows[i][s].  The steps are
// split over work items z in blocks of U: the window entering a block's first
// step s0 is X[s0 .. s0+K-1] of X = [state | bx of the draft tokens] (entry
// s0 is shifted out before use), i.e. state entries for the first K-1 steps
// and otherwise bx of the K-1 tokens before s0, recomputed from their B and
// xv rows.  Only blocks that start inside the first K-1 steps read the slot,
// so most waves skip the slot -> state round trip, and more waves share the
// work of one sequence.
template <typename E, int K, int U, bool STAGED>
__device__ __forceinline__ void verify_one(const VerifyArgs<E>& a, int i, int g, int z) {
    constexpr int KH = K > 1 ? K - 1 : 1;
    const int lane = (int)threadIdx.x;
    const int chw = g * kSmallBlock * kChPerLane;   // the wave's first channel
    int ch0 = chw + lane * kChPerLane;
    const bool on = ch0 < a.H;
    if (!STAGED && !on) return;
    if (!on) ch0 = chw;   // staged: lanes past H work on a valid address and store nothing
    const int s0 = z * U;
    const int n = a.L - s0 < U ? a.L - s0 : U;
    if (n <= 0) return;   // wave-uniform
    const int H = a.H;
    const int64_t HK = (int64_t)H * K;
    const E* base = a.in + (int64_t)i * a.L * a.in_stride + ch0;
    // Loads first, all independent: the K-1 history rows (B, xv), the block's rows (B, C, xv), the state.
    Raw8<E> hb[KH], hx[KH];
#pragma unroll
    for (int k = 1; k < K; ++k) {
        const int t = s0 + k - K;                      // token whose bx is window entry k
        if (t >= 0) {
            const E* row = base + (int64_t)t * a.in_stride;
            hb[k - 1] = ld8s<E, LFM2SC_VER_NT>(row); hx[k - 1] = ld8s<E, LFM2SC_VER_NT>(row + 2 * H);
        }
    }
    Raw8<E> rb[U], rc[U], rx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u < n) {
            const E* row = base + (int64_t)(s0 + u) * a.in_stride;
            rb[u] = ld8s<E, LFM2SC_VER_NT>(row); rc[u] = ld8s<E, LFM2SC_VER_NT>(row + H);
            rx[u] = ld8s<E, LFM2SC_VER_NT>(row + 2 * H);
        }
    }
    float st[kChPerLane][K];
    const bool need_state = s0 + 1 < K;
    if (need_state) {
        const int64_t slot = a.slot_idx[i];
        if (slot_ok(slot, a.num_slots)) {
            load_block_s<E, K, (LFM2SC_VER_NT & 4) ? 1 : 0>(a.pool + slot * a.slot_stride + (int64_t)ch0 * K, st);
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int k = 0; k < K; ++k) st[c][k] = 0.f;
        }
    }
    float wf[kChPerLane][K];
    load_block<E, K>(a.w + (int64_t)ch0 * K, wf);
    float bv[kChPerLane] = {};
    if (a.bias != nullptr) load_f32x8<E>(a.bias + ch0, bv);

    // window entering step s0: s[c][k] = X[s0 + k] for k >= 1
    float s[kChPerLane][K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = s0 + k;                        // index into X
        if (k == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) s[c][0] = 0.f; // shifted out before it is used
        } else if (idx < K) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float v = 0.f;
#pragma unroll
                for (int m = 1; m < K; ++m) v = (m == idx) ? st[c][m] : v;
                s[c][k] = v;
            }
        } else {
            float b[8], x[8];
            to_f32(hb[k - 1], b); to_f32(hx[k - 1], x);
#pragma unroll
            for (int c = 0; c < 8; ++c) s[c][k] = b[c] * x[c];
        }
    }
    E* ybase = a.y + (int64_t)i * a.L * a.y_stride + ch0;
    E* tbase = a.win + (int64_t)i * a.L * HK + (int64_t)ch0 * K;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u < n) {
            float b[8], c8[8], x[8], yv[8];
            to_f32(rb[u], b); to_f32(rc[u], c8); to_f32(rx[u], x);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
#pragma unroll
                for (int k = 0; k < K - 1; ++k) s[c][k] = s[c][k + 1];
                s[c][K - 1] = b[c] * x[c];
                float conv = fmaf(wf[c][K - 1], s[c][K - 1], bv[c]);
#pragma unroll
                for (int k = 0; k < K - 1; ++k) conv = fmaf(wf[c][k], s[c][k], conv);
                yv[c] = c8[c] * conv;
            }
            if (on) store_f32x8s<E, LFM2SC_VER_NT>(ybase + (int64_t)(s0 + u) * a.y_stride, yv);
            if constexpr (STAGED) {
                // the tape row of this step through LDS: contiguous 1 KiB per store instruction
                __shared__ StateStage<E, K> stage;
                const int nch = H - chw < kSmallBlock * kChPerLane ? H - chw : kSmallBlock * kChPerLane;
                const rsrc_t blk = row_rsrc(a.win + ((int64_t)i * a.L + s0 + u) * HK + (int64_t)chw * K,
                                            (uint32_t)nch * K * (uint32_t)sizeof(E));
                stage_store<E, K, (LFM2SC_VER_NT & 8) ? kPolicyNt : 0>(stage, blk, lane, s);
            } else {
                store_block_s<E, K, (LFM2SC_VER_NT & 8) ? 2 : 0>(tbase + (int64_t)(s0 + u) * HK, s);
            }
        }
    }
}

template <typename E, int K, int U, bool STAGED>
__global__ __launch_bounds__(kSmallBlock) void verify_kernel(const VerifyArgs<E> a, int groups, int nz) {
    const int64_t items = (int64_t)a.N * nz * groups;
    for (int64_t b = blockIdx.x; b < items; b += gridDim.x) {
        const SmallIdx ix = small_idx_seq_fastest(b, a.N, groups);
        verify_one<E, K, U, STAGED>(a, ix.i, ix.g, ix.z);
    }
}

// ------------------------------------------------------------------ commit
// pool[slot[i]] <- windows[i][accept[i]-1] for accept[i] in [1, L]: a plain
// 16-byte-per-lane copy of the accepted [H, K] window.
template <typename E>
__global__ __launch_bounds__(kSmallBlock) void commit_kernel(const CommitArgs<E> a, int64_t HK, int groups) {
    const int64_t items = (int64_t)a.N * groups;
    for (int64_t b = blockIdx.x; b < items; b += gridDim.x) {
        const SmallIdx ix = small_idx(b, groups);
        const int i = ix.i;
        const int64_t e0 = ((int64_t)ix.g * kSmallBlock + threadIdx.x) * 8;
        if (e0 >= HK) continue;
        const int acc = a.accept[i];
        if (acc < 1 || acc > a.L) continue;
        const int64_t slot = a.slot_idx[i];
        if (!slot_ok(slot, a.num_slots)) continue;
        const E* src = a.win + ((int64_t)i * a.L + (acc - 1)) * HK + e0;
        st8<E>(a.pool + slot * a.slot_stride + e0, ld8<E>(src));
    }
}

// ------------------------------------------------------------------ launchers
int64_t ragged_tiles_bound(int64_t total_T, int N) {
    const int64_t gap = (int64_t)LFM2SC_SUB_MIN;
    return (total_T + gap - 1) / gap + N;
}

// Rows of loads in flight per wave: measured on MI355X at T=65536, H=2048, 4
// for bf16 (6.1 TB/s; 12 rows: 5.9) and 2 for fp32 (5.1 TB/s; 12 rows: 4.8).
template <typename E> constexpr int fwd_unroll() { return sizeof(E) == 4 ? LFM2SC_FWD_U_F32 : LFM2SC_FWD_U; }

template <typename E, int K, int TW>
static hipError_t prefill_tw(PrefillArgs<E> a, hipStream_t s) {
    constexpr auto kernel = prefill_kernel<E, K, fwd_unroll<E>(), TW>;
    static const int resident_long = resident_workgroups(kernel, LFM2SC_FWD_LDS);
    static const int resident_short = resident_workgroups(kernel, 0);
    const bool short_call = a.total_T < LFM2SC_SHORT_T;
    const int gy = WgLayout<TW>::groups(a.H);
    const Tiling t = ragged_tiling(a.total_T, a.N, gy, short_call ? resident_short : resident_long, TW,
                                   (int64_t)a.H * (int64_t)sizeof(E), kWinSpanFwd);
    a.sub = t.sub;
    a.ntiles = (int)t.ntiles;
    hipLaunchKernelGGL(kernel, dim3(pad_xcd(a.ntiles), gy), dim3(kThreads), short_call ? 0 : LFM2SC_FWD_LDS, s, a);
    return hipGetLastError();
}

// One sequence: workgroups of LFM2SC_FWD_TW consecutive windows of one
// 512-channel group.  Several: one window per workgroup across 4 channel
// groups, so the gap the virtual axis leaves between two sequences is one
// window instead of LFM2SC_FWD_TW (with 8 sequences the gaps took 7 of 64
// window slots per channel group; measured ragged prefill of 8 sequences,
// ~7,000 tokens: 27.7 -> 26.9 us per call; a single 65,536-token sequence
// is 1% slower that way, 200 vs 202 us).
template <typename E, int K>
static hipError_t prefill_k(PrefillArgs<E> a, hipStream_t s) {
    if (a.N > 1 && LFM2SC_FWD_TW_RAGGED != LFM2SC_FWD_TW) return prefill_tw<E, K, LFM2SC_FWD_TW_RAGGED>(a, s);
    return prefill_tw<E, K, LFM2SC_FWD_TW>(a, s);
}

template <typename E>
hipError_t launch_prefill(const PrefillArgs<E>& a, int K, hipStream_t s) {
    switch (K) {
        case 1: return prefill_k<E, 1>(a, s);
        case 2: return prefill_k<E, 2>(a, s);
        case 3: return prefill_k<E, 3>(a, s);
        case 4: return prefill_k<E, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename E, int K>
static hipError_t decode_k(const DecodeArgs<E>& a, hipStream_t s) {
    const int groups = small_groups(a.H / kChPerLane);
    if (a.N >= LFM2SC_DEC_STAGE_N)
        hipLaunchKernelGGL((decode_kernel<E, K, true>), dim3(small_grid((int64_t)a.N * groups)), dim3(kSmallBlock), 0,
                           s, a, groups);
    else
        hipLaunchKernelGGL((decode_kernel<E, K, false>), dim3(small_grid((int64_t)a.N * groups)), dim3(kSmallBlock), 0,
                           s, a, groups);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_decode(const DecodeArgs<E>& a, int K, hipStream_t s) {
    switch (K) {
        case 1: return decode_k<E, 1>(a, s);
        case 2: return decode_k<E, 2>(a, s);
        case 3: return decode_k<E, 3>(a, s);
        case 4: return decode_k<E, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename E, int K>
static hipError_t verify_k(const VerifyArgs<E>& a, hipStream_t s) {
    constexpr int U = LFM2SC_VERIFY_U;
    const int groups = small_groups(a.H / kChPerLane);
    const int nz = (a.L + U - 1) / U;
    hipLaunchKernelGGL((verify_kernel<E, K, U, LFM2SC_VER_STAGE != 0>), dim3(small_grid((int64_t)a.N * nz * groups)),
                       dim3(kSmallBlock), 0, s, a, groups, nz);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_verify(const VerifyArgs<E>& a, int K, hipStream_t s) {
    switch (K) {
        case 1: return verify_k<E, 1>(a, s);
        case 2: return verify_k<E, 2>(a, s);
        case 3: return verify_k<E, 3>(a, s);
        case 4: return verify_k<E, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_commit(const CommitArgs<E>& a, int K, hipStream_t s) {
    const int64_t HK = (int64_t)a.H * K;
    const int groups = small_groups(HK / 8);
    hipLaunchKernelGGL((commit_kernel<E>), dim3(small_grid((int64_t)a.N * groups)), dim3(kSmallBlock), 0, s, a, HK,
                       groups);
    return hipGetLastError();
}

template hipError_t launch_prefill<uint16_t>(const PrefillArgs<uint16_t>&, int, hipStream_t);
template hipError_t launch_prefill<float>(const PrefillArgs<float>&, int, hipStream_t);
template hipError_t launch_decode<uint16_t>(const DecodeArgs<uint16_t>&, int, hipStream_t);
template hipError_t launch_decode<float>(const DecodeArgs<float>&, int, hipStream_t);
template hipError_t launch_verify<uint16_t>(const VerifyArgs<uint16_t>&, int, hipStream_t);
template hipError_t launch_verify<float>(const VerifyArgs<float>&, int, hipStream_t);
template hipError_t launch_commit<uint16_t>(const CommitArgs<uint16_t>&, int, hipStream_t);
template hipError_t launch_commit<float>(const CommitArgs<float>&, int, hipStream_t);

}  // namespace lfm2sc
