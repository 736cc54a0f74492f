// fused.hip -- in_proj GEMM on the matrix cores with the ShortConv forward in
// its epilogue (bf16 I/O, fp32 accumulation).
//
// What it computes (MAX Pipelines LFM2 article, "ShortConv implementation
// (LFM2ShortConv)"): in_proj projects each token's hidden state x[t] (D wide)
// into B | C | xv (3 x H); bx = B * xv; the K-tap depthwise causal conv runs
// over [initial state | bx] per sequence; y = C * conv.  Unfused, in_proj is a
// [T][3H] tensor written by a GEMM and read back by the conv kernel (12 KiB per
// token each way at H = 2048); here it never leaves the chip unless the caller
// asks for it (training keeps it for the backward).
//
// Tiling.  A workgroup computes a tile of kFBM = 256 token rows by kFNC = 64
// channels; its GEMM columns gather the B, C and xv columns of those channels
// (3 x 64 = 192 rows of W_in).  Four waves, 2 x 2: wave (wm, wn) owns rows
// wm*128 .. +128 and channels wn*32 .. +32, as 4 row tiles x 3 column tiles
// (B, C, xv) of v_mfma_f32_32x32x16_bf16, so every lane ends up holding B, C
// and xv of the same channel and rows in its accumulators.  Consecutive tiles
// overlap by K-1 rows: a tile outputs rows K-1 .. 255 of the rows it computes,
// so the conv history of every output row is inside the tile (0.8% extra MFMA
// work at K = 3).  When H % 128 == 0 and D is one of the LFM2 hidden sizes a
// wide variant (fused_wide_kernel) covers 128 channels with 8 waves instead,
// the same 128 x 32 block per wave, which halves the x rows fetched per FLOP.
// Short inputs, which fill too few of these tiles, take the split and mid
// tiles of fused_split.hip; fused_k below picks the form per call.
//
// Reduction.  Stages of kFBK = 32 along D.  The x rows and W_in rows of a stage
// go from global memory straight into one slot of a 4-deep LDS ring (buffer
// loads with an LDS destination, no registers in between), 3 stages ahead of
// the one being consumed.  The ring slots are separate LDS arrays, so the
// compiler can tell that a refill never overlaps the slot being read and does
// not wait for it; the reduction is fully unrolled for the usual hidden sizes
// (straight-line code keeps the wait counts exact), with a loop for the rest.
// (Loading each wave's W_in operands straight into registers instead was
// slower on MI355X: both row halves then fetch them, and the vector-memory
// path, not LDS, is what this loop runs short of.)
//
// Epilogue.  Each lane holds B, C, xv of one channel for runs of 4 consecutive
// rows; the K-1 rows before a run live in the partner lane (lane ^ 32), or for
// the first run of the second row half in the other wave (through a small LDS
// buffer).  y = C * conv is rounded once to bf16 and staged in LDS so that the
// stores to y are 16-byte row segments.  Final states are the last K entries
// of [initial state | bx]: the tile that holds a sequence's last token writes
// them to a per-sequence staging block, and a second small kernel installs
// them into the slots after every tile has read its initial states (a slot may
// be read by one tile and written by another).
#include <cstdlib>
#include <type_traits>

#include "fused_common.hpp"

namespace lfm2sc {


constexpr int kFNC = 64;               // channels per tile
constexpr int kFBK = 32;               // reduction depth per stage
constexpr int kFStages = 4;            // ring depth: 3 stages in flight ahead of the one in use
constexpr int kFThreads = 256;         // 4 waves
constexpr int kFRowBytes = kFBK * 2;   // one staged x row: 32 bf16 = 64 B = 4 chunks of 16 B
constexpr int kFStageA = kFBM * kFRowBytes;           // 16 KiB of x rows per stage
constexpr int kFStageB = 3 * kFNC * kFRowBytes;       // 12 KiB of W_in rows per stage
// One global->LDS instruction moves 64 lanes x 16 B = 16 staged rows; per stage
// the 4 waves move 16 x blocks and 12 W_in blocks, 4 + 3 per wave.
constexpr int kFDmaA = kFBM / 16 / 4, kFDmaB = 3 * kFNC / 16 / 4;
constexpr int kFVmPerStage = kFDmaA + kFDmaB;
// Output staging tile [256][kFOutStride] bf16: the two row halves of a wave
// (hl = 0, 1: rows 4 apart) land 576 B apart, i.e. in different banks.
constexpr int kFOutStride = kFNC + 8;

template <int K> constexpr int fused_out_rows() { return kFBM - (K - 1); }


typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// c + sum of the 8 products a[e] * b[e] (bf16 operands, fp32 accumulation)
__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const bf16x8& b, float c) {
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), c, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), c,
                                           false);
}

// Swizzled byte offset of 16-byte chunk c of staged row r: rows r, r+4, r+8,
// r+12 put chunk c in four different positions, so the 16 lanes of a
// ds_read_b128 quarter (16 consecutive rows, one chunk) hit all 64 banks once.
__device__ __forceinline__ uint32_t lds_chunk(int r, int c) {
    return (uint32_t)r * kFRowBytes + (uint32_t)((c ^ ((r >> 2) & 3)) << 4);
}







// Per-row sequence data of a tile's epilogue (LDS): position in the sequence
// (-1 outside every sequence), sequence length and index, and the row's slot
// when a pool is given and the slot id is in range (else -1).
struct RowMap {
    const int* pos;
    const int* len;
    const int* seq;
    const int* slot;
};

// Does the quad R0..R0+3 need the general epilogue below?  Only when one of
// its output rows is among a sequence's first K-1 (its history starts from
// the initial state, not from the rows before it) or ends a sequence whose
// final state is wanted; every other quad of a multi-sequence tile takes the
// plain conv over the rows before it, the same code as a one-sequence tile.
template <int K>
__device__ __forceinline__ bool quad_special(const FusedArgs& a, const RowMap& rm, int R0, int first_out) {
    const int4 p4 = *reinterpret_cast<const int4*>(rm.pos + R0);
    const int4 l4 = *reinterpret_cast<const int4*>(rm.len + R0);
    const int pos[4] = {p4.x, p4.y, p4.z, p4.w};
    const int len[4] = {l4.x, l4.y, l4.z, l4.w};
    bool sp = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool out = R0 + j >= first_out && pos[j] >= 0;
        sp = sp || (out && (pos[j] < K - 1 || (a.fin != nullptr && pos[j] == len[j] - 1)));
    }
    return sp;
}

// The general (multi-sequence) epilogue for the 4 consecutive rows R0..R0+3
// that one lane holds in an accumulator quad (rows before first_out are the
// tile's history rows, not outputs).  hx holds bx of rows R0-(K-1) ..
// R0+3; cgate the rows' C.  Rows whose conv history reaches before their
// sequence start take initial-state entries instead (X[pos+1+k], k < K-1);
// those entries are fetched first, all together, from an address chosen
// without branching (an entry that is not needed reads the channel's weight
// instead), so the loads overlap rather than queue one behind another.  Each
// row's effective history then serves both its conv and, at a sequence end,
// its final state X[len .. len+K-1].
template <int K, typename Out>
__device__ __forceinline__ void quad_general(const FusedArgs& a, const RowMap& rm, int R0, int first_out, int ch,
                                             const float (&wk)[K], float bv, const float* hx, const float* cgate,
                                             Out&& out) {
    constexpr int KH = K > 1 ? K - 1 : 1;
    // the quad's positions and lengths in two 16-byte LDS reads (read row by
    // row, each length check waited on the LDS before the next row)
    const int4 p4 = *reinterpret_cast<const int4*>(rm.pos + R0);
    const int4 l4 = *reinterpret_cast<const int4*>(rm.len + R0);
    const int pos[4] = {p4.x, p4.y, p4.z, p4.w};
    const int len[4] = {l4.x, l4.y, l4.z, l4.w};
    float sv[4][KH];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < KH; ++k) sv[j][k] = 0.f;
    if (a.pool != nullptr) {
        const int4 s4 = *reinterpret_cast<const int4*>(rm.slot + R0);
        const int slot[4] = {s4.x, s4.y, s4.z, s4.w};
        // Only a sequence's first K-1 rows take state entries: a quad without
        // one skips the fetch (a wave none of whose lanes has one branches
        // around it), so the other quads do not wait on loads.
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) any = any || (pos[j] >= 0 && pos[j] < K - 1 && R0 + j >= first_out && slot[j] >= 0);
        if (any) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < K - 1; ++k) {
                    const bool need = pos[j] >= 0 && pos[j] < K - 1 - k && R0 + j >= first_out && slot[j] >= 0;
                    const uint16_t* src = need ? a.pool + (int64_t)slot[j] * a.slot_stride + (int64_t)ch * K + pos[j] +
                                                     1 + k
                                               : a.w + (int64_t)ch * K;
                    sv[j][k] = need ? bf16_val(*src) : 0.f;
                }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float h[KH];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) h[k] = pos[j] < K - 1 - k ? sv[j][k] : hx[j + k];
        float conv = fmaf(wk[K - 1], hx[K - 1 + j], bv);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], h[k], conv);
        out(j, cgate[j] * conv);
        const int row = R0 + j;
        if (a.fin != nullptr && row >= first_out && pos[j] >= 0 && pos[j] == len[j] - 1) {
            uint16_t* f = a.fin + (int64_t)rm.seq[row] * a.H * K + (int64_t)ch * K;
#pragma unroll
            for (int e = 0; e < K - 1; ++e) f[e] = bf16_bits(h[e]);
            f[K - 1] = bf16_bits(hx[K - 1 + j]);
        }
    }
}

// NK: number of kFBK stages along D when it is known at compile time (the
// reduction is then straight-line code), 0 for the loop form.
template <int K, int NK>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_prefill_kernel(const FusedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kFStageA], ring1[kFStageA], ring2[kFStageA], ring3[kFStageA];
    __shared__ __attribute__((aligned(16))) uint8_t wring0[kFStageB], wring1[kFStageB], wring2[kFStageB],
        wring3[kFStageB];
    __shared__ __attribute__((aligned(16))) uint16_t ost[kFBM * kFOutStride];
    __shared__ __attribute__((aligned(16))) int s_pos[kFBM];
    __shared__ __attribute__((aligned(16))) int s_len[kFBM];
    __shared__ int s_seq[kFBM];
    __shared__ __attribute__((aligned(16))) int s_slot[kFBM];
    __shared__ float s_edge[2][32][4];        // bx of rows 125..127 of each channel (the second half's history)

    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    if (lin >= a.tiles_m * a.tiles_n) return;
    int mt, nt;
    fused_tile(lin, a.tiles_m, a.tiles_n, mt, nt);
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int q = lane & 31, hl = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int H = a.H;
    const int64_t T = a.total_T;
    const int64_t row0 = (int64_t)mt * fused_out_rows<K>() - (K - 1);   // token of computed row 0
    const int n0 = nt * kFNC;                                           // first channel of the tile

    // Row -> (sequence, position, length, slot) map of the tile, for the epilogue.
    {
        const TileSeq f = tile_first_seq(a, row0);
        int pos, len, seq, sid;
        tile_row(a, f, row0, kFBM, tid, pos, len, seq, sid);
        s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq; s_slot[tid] = sid;
    }

    // ---------------------------------------------------------------- reduction
    // x rows: each lane of a 16-row block fetches the chunk that the swizzle
    // places at its LDS slot (row lane/4, position lane%4).  Rows outside
    // [0, T) are clamped to a valid row: they are never stored and never feed
    // another row's conv history.
    // W_in rows the same way: staged row n of a slot is W_in row
    // (n / 64) * H + n0 + n % 64 (the B, C, xv rows of the tile's channels).
    const int64_t vlo = row0 < 0 ? 0 : row0;
    const int64_t vhi = (row0 + kFBM < T) ? row0 + kFBM : T;     // > vlo for every launched tile
    const rsrc_t xr = row_rsrc(a.x + vlo * a.x_stride, (uint32_t)((vhi - vlo) * a.x_stride * 2));
    const rsrc_t wr = row_rsrc(a.W, (uint32_t)((int64_t)3 * H * a.D * 2));
    const int brow = lane >> 2;                                    // row within a 16-row block
    const uint32_t bchunk = (uint32_t)(((lane & 3) ^ ((brow >> 2) & 3)) << 4);
    uint32_t xoff[kFDmaA], woff[kFDmaB];
#pragma unroll
    for (int i = 0; i < kFDmaA; ++i) {
        int64_t t = row0 + (wave + 4 * i) * 16 + brow;
        t = t < vlo ? vlo : (t >= vhi ? vhi - 1 : t);
        xoff[i] = (uint32_t)((t - vlo) * a.x_stride * 2) + bchunk;
    }
#pragma unroll
    for (int i = 0; i < kFDmaB; ++i) {
        const int n = (wave + 4 * i) * 16 + brow;
        woff[i] = (uint32_t)(((int64_t)(n / kFNC) * H + n0 + (n % kFNC)) * a.D * 2) + bchunk;
    }

    auto slot = [&](auto u_c) -> uint8_t* {
        constexpr int u = decltype(u_c)::value;
        if constexpr (u == 0) return ring0;
        else if constexpr (u == 1) return ring1;
        else if constexpr (u == 2) return ring2;
        else return ring3;
    };
    auto wslot = [&](auto u_c) -> uint8_t* {
        constexpr int u = decltype(u_c)::value;
        if constexpr (u == 0) return wring0;
        else if constexpr (u == 1) return wring1;
        else if constexpr (u == 2) return wring2;
        else return wring3;
    };
    auto issue = [&](auto u_c, int kt) { // loads of stage kt into ring slot u
        uint8_t* st = slot(u_c);
        uint8_t* sw = wslot(u_c);
        const uint32_t ko = (uint32_t)kt * kFRowBytes;
#pragma unroll
        for (int i = 0; i < kFDmaA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(st + (wave + 4 * i) * 1024), 16, xoff[i] + ko,
                                                     0, 0, 0);
#pragma unroll
        for (int i = 0; i < kFDmaB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(sw + (wave + 4 * i) * 1024), 16,
                                                     woff[i] + ko, 0, 0, 0);
    };

    f32x16 acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // One stage: wait for its loads (this wave's; `later` stages after it may
    // still be in flight), meet the workgroup, refill the slot the previous
    // stage used, then feed the matrix cores from slot u.
    auto stage = [&](auto u_c, int kt, auto later_c, auto refill_c) {
        constexpr int u = decltype(u_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<decltype(later_c)::value * kFVmPerStage>();
        stage_barrier();
        if constexpr (decltype(refill_c)::value) issue(IC<(u + kFStages - 1) % kFStages>{}, kt + kFStages - 1);
        // the refill goes out first: left to itself the scheduler may sink it
        // below the MFMAs, shortening the prefetch
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* sa = slot(u_c);
        const uint8_t* sb = wslot(u_c);
#pragma unroll
        for (int kk = 0; kk < kFBK / 16; ++kk) {
            const int c = kk * 2 + hl;
            bf16x8 fa[4], fb[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(sa + lds_chunk(wm * 128 + i * 32 + q, c));
#pragma unroll
            for (int j = 0; j < 3; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(sb + lds_chunk(j * kFNC + wn * 32 + q, c));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Four stages at a time (ring slots 0..3); the last group only refills
    // once (the final stage) and then drains the ring.
    auto group = [&](int kb) {
        stage(IC<0>{}, kb + 0, IC<2>{}, std::true_type{});
        stage(IC<1>{}, kb + 1, IC<2>{}, std::true_type{});
        stage(IC<2>{}, kb + 2, IC<2>{}, std::true_type{});
        stage(IC<3>{}, kb + 3, IC<2>{}, std::true_type{});
    };
    auto last_group = [&](int kb) {
        stage(IC<0>{}, kb + 0, IC<2>{}, std::true_type{});
        stage(IC<1>{}, kb + 1, IC<2>{}, std::false_type{});
        stage(IC<2>{}, kb + 2, IC<1>{}, std::false_type{});
        stage(IC<3>{}, kb + 3, IC<0>{}, std::false_type{});
    };
    static_assert(kFStages == 4, "the stage groups above are written for a 4-deep ring");
    issue(IC<0>{}, 0);
    issue(IC<1>{}, 1);
    issue(IC<2>{}, 2);
    if constexpr (NK > 0) {
        static_assert(NK % kFStages == 0 && NK >= kFStages, "whole stage groups");
#pragma unroll
        for (int kb = 0; kb + kFStages < NK; kb += kFStages) group(kb);
        last_group(NK - kFStages);
    } else {
        const int nk = a.D / kFBK;      // a multiple of kFStages, at least kFStages (checked on the host)
        int kb = 0;
        for (; kb + kFStages < nk; kb += kFStages) group(kb);
        last_group(kb);
    }

    // ---------------------------------------------------------------- epilogue
    // Accumulator register r of row tile i holds computed row
    // R = wm*128 + i*32 + 8*(r/4) + 4*hl + (r%4) of channel ch = n0 + lcn:
    // lane-local runs of 4 consecutive rows ("quads"), quad (i, g = r/4)
    // starting at R0 = wm*128 + i*32 + 8g + 4hl.  The K-1 rows before a quad
    // end the partner lane's (lane ^ 32) quad: the same quad for hl = 1, the
    // previous one for hl = 0 (for the wave's first quad: the other wave of
    // the same channels, rows 125..127, or rows before the tile for wm = 0,
    // which are never outputs).
    const int lcn = wn * 32 + q;
    const int ch = n0 + lcn;
    float bx[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) bx[i][r] = acc[i][0][r] * acc[i][2][r];
    // tail[i][g][m]: the partner's rows 4g + 4 - (K-1) + m of its tile i
    float tail[4][4][K > 1 ? K - 1 : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int m = 0; m < K - 1; ++m) tail[i][g][m] = __shfl_xor(bx[i][4 * g + 4 - (K - 1) + m], 32);
    if (wm == 0 && hl == 1) {
#pragma unroll
        for (int m = 0; m < K - 1; ++m) s_edge[wn][q][m] = bx[3][12 + 4 - (K - 1) + m];
    }

    // Output rows of the tile go out through `ost` with 16-byte stores: chunk
    // (row, cc) holds channels n0 + 8cc .. +8 of computed row `row`.
    auto flush_rows = [&](uint16_t* dst, int64_t stride, bool last) {
        lds_barrier();
#pragma unroll
        for (int k = 0; k < kFBM * 8 / kFThreads; ++k) {
            const int id = tid + kFThreads * k;
            const int row = id >> 3, cc = id & 7;
            if (row >= K - 1 && s_pos[row] >= 0) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(ost + row * kFOutStride + cc * 8);
                *reinterpret_cast<u32x4*>(dst + (row0 + row) * stride + n0 + cc * 8) = v;
            }
        }
        if (!last) lds_barrier();   // `ost` is refilled next
    };
    auto stage_out = [&](int i, int r, float v) {
        const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        ost[row * kFOutStride + lcn] = bf16_bits(v);
    };

    if (a.io != nullptr) {          // in_proj for the backward: B, C, xv rounded to bf16
#pragma unroll
        for (int j = 0; j < 3; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) stage_out(i, r, acc[i][j][r]);
            flush_rows(a.io + (int64_t)j * H, a.io_stride, false);
        }
    }
    lds_barrier();                  // s_edge written

    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = bf16_val(a.w[(int64_t)ch * K + k]);
    const float bv = a.bias != nullptr ? bf16_val(a.bias[ch]) : 0.f;
    const RowMap rm{s_pos, s_len, s_seq, s_slot};
    // hx[m] = bx of row R0 - (K-1) + m for quad (i, g): K-1 history rows, then the quad's own 4
    auto history = [&](int i, int g, float* hx) {
#pragma unroll
        for (int m = 0; m < K - 1; ++m) {
            float prev;
            if (g > 0) prev = tail[i][g - 1][m];
            else if (i > 0) prev = tail[i - 1][3][m];
            else prev = wm == 1 ? s_edge[wn][q][m] : 0.f;
            hx[m] = hl ? tail[i][g][m] : prev;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) hx[K - 1 + j] = bx[i][4 * g + j];
    };
    // One sequence covers every computed row (and does not end inside the tile
    // when final states are wanted): no per-row sequence logic.
    const int p0 = s_pos[0], pl = s_pos[kFBM - 1];
    const bool simple = p0 >= 0 && pl == p0 + kFBM - 1 && !(a.fin != nullptr && pl == s_len[kFBM - 1] - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int R0 = wm * 128 + i * 32 + 8 * g + 4 * hl;
            float hx[K - 1 + 4];
            history(i, g, hx);
            if (simple || !quad_special<K>(a, rm, R0, K - 1)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float conv = fmaf(wk[K - 1], hx[K - 1 + j], bv);
#pragma unroll
                    for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], hx[j + k], conv);
                    stage_out(i, 4 * g + j, acc[i][1][4 * g + j] * conv);
                }
            } else {
                float cg[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) cg[j] = acc[i][1][4 * g + j];
                quad_general<K>(a, rm, R0, K - 1, ch, wk, bv, hx, cg, [&](int j, float v) { stage_out(i, 4 * g + j, v); });
            }
        }
    flush_rows(a.y, a.y_stride, true);
}

// ---------------------------------------------------------------- wide tiles
// The tile above fetches 28 KiB per 32-deep stage for its MFMA work; on
// MI355X its loop waits on those loads (they do not hide under the MFMA work,
// though L2 could deliver them three times faster).  Wide tiles cover 128
// channels with 8 waves (two per SIMD), each wave still 128 rows x 32
// channels, so a stage moves 1.4x fewer bytes per FLOP.  Used when H % 128 ==
// 0 and D is one of the unrolled hidden sizes.
//
// Two forms (HALO).  Without, consecutive tiles overlap by K-1 rows as above;
// the reduction runs in 64-deep stages through a 2-slot ring that fills the
// whole 160 KiB of LDS (each staged row is then a whole 128-byte line, and a
// tile meets half as many stage barriers as with 32-deep stages: ~4% faster).
// With HALO, a tile outputs all 256 of its rows, so T = 4096 fills exactly
// one round of 256 CUs instead of spilling 16 tiles into a second; the conv
// history of its first K-1 rows is bx of the K-1 x rows just before it ("halo
// rows"): they are staged in LDS once per tile, and the waves of the first row
// half form their B and xv with bf16 dot products against the W_in fragments
// they already hold for the MFMAs, stage by stage (fp32 accumulation, no extra
// W_in traffic).  The halo rows need LDS, so this form keeps 32-deep stages in
// a 3-slot ring; with those and the dot products a tile is ~21% slower on
// MI355X, and the launcher takes the halo form only when it saves enough
// rounds of tiles.
constexpr int kWThreads = 512;                     // 8 waves: 2 row halves x 4 channel groups of 32
constexpr int kWRegion = 128 * 32 * 2;             // one wave's bf16 output block: 128 rows x 32 channels


// LDS of one wide tile: the ring slots (separate arrays, so that the compiler
// sees that a refill never touches the slot being read), the halo rows, the
// row map [4][kFBM] (position, length, sequence, slot) and the row-half
// hand-off [4][32][4] (bx of rows 125..127 of the first half, per channel).
struct WideLds {
    uint8_t* ra[3];
    uint8_t* rb[3];
    uint8_t* halo;
    int* map;
    float* edge;
};

// Stage loads of a wide tile: the wave's x blocks and W_in blocks, global ->
// LDS slot (sa, sb); xoff / woff are the lanes' byte offsets in stage 0.
template <class S>
__device__ __forceinline__ void wide_issue(rsrc_t xr, rsrc_t wr, uint8_t* sa, uint8_t* sb, const uint32_t* xoff,
                                           const uint32_t* woff, int wave, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < S::kDmaA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(sa + (wave + 8 * i) * 1024), 16, xoff[i] + ko, 0, 0,
                                                 0);
#pragma unroll
    for (int i = 0; i < S::kDmaB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(sb + (wave + 8 * i) * 1024), 16, woff[i] + ko, 0, 0,
                                                 0);
}

template <int K, int D, bool HALO, int BK, int NSLOT>
__device__ __forceinline__ void wide_tile(const FusedArgs& a, const WideLds& L) {
    using S = WideStage<BK>;
    constexpr int NK = D / BK;                         // stages
    static_assert(NK >= NSLOT && NSLOT >= 2, "at least a full ring of stages");
    constexpr int KH = K > 1 ? K - 1 : 1;
    constexpr int kRowBytes = D * 2;                   // one x row
    constexpr int kFirstOut = HALO ? 0 : K - 1;        // rows before it are history, not outputs
    // Without halo rows the ring fills the LDS: the row map waits in registers
    // (threads 0..255, one row each) and moves into the idle ring afterwards.
    constexpr bool kMapLate = !HALO;

    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    if (lin >= a.tiles_m * a.tiles_n) return;
    int mt, nt;
    fused_tile(lin, a.tiles_m, a.tiles_n, mt, nt);
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int q = lane & 31, hl = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;
    const int H = a.H;
    const int64_t T = a.total_T;
    const int64_t row0 = HALO ? (int64_t)mt * kFBM : (int64_t)mt * fused_out_rows<K>() - (K - 1);
    const int n0 = nt * kWNC;
    int* s_pos = L.map;
    int* s_len = L.map + kFBM;
    int* s_seq = L.map + 2 * kFBM;
    int* s_slot = L.map + 3 * kFBM;

    // row -> (sequence, position, length, slot) map, before any load of the
    // reduction (as in the kernel above)
    int m_pos = -1, m_len = 0, m_seq = 0, m_slot = -1;
    {
        const TileSeq f = tile_first_seq(a, row0);
        if (tid < kFBM) {
            int pos, len, seq, sid;
            tile_row(a, f, row0, kFBM, tid, pos, len, seq, sid);
            if constexpr (kMapLate) {
                m_pos = pos; m_len = len; m_seq = seq; m_slot = sid;
            } else {
                s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq; s_slot[tid] = sid;
            }
        }
    }

    // ---------------------------------------------------------------- reduction
    const int64_t vlo = row0 < 0 ? 0 : row0;
    const int64_t vhi = (row0 + kFBM < T) ? row0 + kFBM : T;
    // The row map above is filled under a branch that splits the waves; the
    // descriptor size is taken through readfirstlane so that the compiler keeps
    // it in SGPRs (otherwise every load gets a loop over distinct descriptors).
    const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)((vhi - vlo) * a.x_stride * 2));
    const rsrc_t xr = row_rsrc(a.x + vlo * a.x_stride, xbytes);
    const rsrc_t wr = row_rsrc(a.W, (uint32_t)((int64_t)3 * H * a.D * 2));
    const int brow = lane / S::kChunks;                // row within a block of kRowsPerDma
    uint32_t xoff[S::kDmaA], woff[S::kDmaB];
#pragma unroll
    for (int i = 0; i < S::kDmaA; ++i) {
        const int r = (wave + 8 * i) * S::kRowsPerDma + brow;
        int64_t t = row0 + r;
        t = t < vlo ? vlo : (t >= vhi ? vhi - 1 : t);
        xoff[i] = (uint32_t)((t - vlo) * a.x_stride * 2) + S::dma_chunk(lane, r);
    }
#pragma unroll
    for (int i = 0; i < S::kDmaB; ++i) {
        const int n = (wave + 8 * i) * S::kRowsPerDma + brow;   // staged W_in row: part n / 128, channel n % 128
        const int chn = n0 + n % kWNC;                 // H % 128 == 0: every channel of the tile exists
        woff[i] = (uint32_t)(((int64_t)(n / kWNC) * H + chn) * a.D * 2) + S::dma_chunk(lane, n);
    }
    auto issue = [&](uint8_t* sa, uint8_t* sb, int kt) {     // stage kt's loads into ring slot (sa, sb)
        wide_issue<S>(xr, wr, sa, sb, xoff, woff, wave, (uint32_t)kt * S::kRowB);
    };

    f32x16 acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Halo rows first (the oldest loads, so the first stage's wait covers
    // them): (K-1) x D bf16 in 1 KiB pieces, row max(t, 0) for a tile at the
    // start (its first rows take their history from the initial states).
    if constexpr (HALO) {
        constexpr int kPerRow = kRowBytes / 1024;
        constexpr int kPieces = (K - 1) * kPerRow;
#pragma unroll
        for (int i = 0; i < (kPieces + 7) / 8; ++i) {
            const int pc = wave + 8 * i;
            if (pc < kPieces) {
                const int m = pc / kPerRow;
                const int64_t hr = row0 - (K - 1) + m < 0 ? 0 : row0 - (K - 1) + m;
                const rsrc_t hs = row_rsrc(a.x + hr * a.x_stride, (uint32_t)kRowBytes);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(hs, (lds_ptr_t)(L.halo + pc * 1024), 16,
                                                         (uint32_t)((pc % kPerRow) * 1024 + lane * 16), 0, 0, 0);
            }
        }
    }
    float hacc[KH][2];                                 // partial B, xv of the halo rows (first row half)
#pragma unroll
    for (int m = 0; m < KH; ++m) hacc[m][0] = hacc[m][1] = 0.f;

    issue(L.ra[0], L.rb[0], 0);                        // the first NSLOT - 1 stages
    if constexpr (NSLOT > 2) issue(L.ra[1], L.rb[1], 1);
    static_assert(NSLOT <= 3, "prologue issues at most two stages");
    auto stage = [&](auto kt_c) {
        constexpr int kt = decltype(kt_c)::value;
        constexpr int u = kt % NSLOT;
        constexpr int later = NK - 1 - kt < NSLOT - 2 ? NK - 1 - kt : NSLOT - 2;   // stages after kt in flight
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<later * S::kVm>();
        stage_barrier();
        if constexpr (kt + NSLOT - 1 < NK)
            issue(L.ra[(kt + NSLOT - 1) % NSLOT], L.rb[(kt + NSLOT - 1) % NSLOT], kt + NSLOT - 1);
        const uint8_t* sa = L.ra[u];
        const uint8_t* sb = L.rb[u];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + hl;
            bf16x8 fa[4], fb[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(sa + S::chunk(wm * 128 + i * 32 + q, c));
#pragma unroll
            for (int j = 0; j < 3; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(sb + S::chunk(j * kWNC + wn * 32 + q, c));
            if constexpr (HALO) {
                if (wm == 0) {                         // halo rows: the same k values as this lane's fragments
#pragma unroll
                    for (int m = 0; m < K - 1; ++m) {
                        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(
                            L.halo + m * kRowBytes + (kt * BK + kk * 16 + 8 * hl) * 2);
                        hacc[m][0] = dot8_bf16(xh, fb[0], hacc[m][0]);
                        hacc[m][1] = dot8_bf16(xh, fb[2], hacc[m][1]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if constexpr (kt + NSLOT - 1 < NK) {
            // the refill loads spread over the stage's MFMAs: issued in a burst
            // they stall the wave on a full address queue (2-4% slower)
#pragma unroll
            for (int g = 0; g < S::kVm; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, S::kMfma / S::kVm, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    unroll_stages<0, NK>(stage);

    // ---------------------------------------------------------------- epilogue
    // As in the kernel above, one 32-row tile i at a time, which keeps the
    // working set beside the 192 accumulator registers small.  Each wave stages
    // its 128 x 32 outputs in its own 8 KiB of the x slots of the (now idle) ring
    // (and, with three 16 KiB slots, of the first W_in slot).
    __syncthreads();
    if constexpr (kMapLate) {
        if (tid < kFBM) {
            s_pos[tid] = m_pos; s_len[tid] = m_len; s_seq[tid] = m_seq; s_slot[tid] = m_slot;
        }
    }
    float (*s_edge)[32][4] = reinterpret_cast<float (*)[32][4]>(L.edge);
    if (wm == 0 && hl == 1) {
#pragma unroll
        for (int m = 0; m < K - 1; ++m) {
            const int r = 12 + 4 - (K - 1) + m;
            s_edge[wn][q][m] = acc[3][0][r] * acc[3][2][r];
        }
    }
    lds_barrier();
    uint8_t* region;
    if constexpr (NSLOT == 2) {                        // 32 KiB x slots: four waves each
        static_assert(S::kStageA == 4 * kWRegion, "x slot holds four output blocks");
        region = (wave < 4 ? L.ra[0] : L.ra[1]) + (wave & 3) * kWRegion;
    } else {                                           // 16 KiB x slots: two waves each, the last two in rb[0]
        static_assert(S::kStageA == 2 * kWRegion && NSLOT == 3, "x slot holds two output blocks");
        region = (wave < 2 ? L.ra[0] : (wave < 4 ? L.ra[1] : (wave < 6 ? L.ra[2] : L.rb[0]))) + (wave & 1) * kWRegion;
    }
    uint16_t* wout = reinterpret_cast<uint16_t*>(region);   // [128][32]
    const int lcn = wn * 32 + q;
    const int ch = n0 + lcn;
    const int rbase = wm * 128;
    auto stage_out = [&](int i, int r, float v) {
        wout[(i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3)) * 32 + q] = bf16_bits(v);
    };
    auto flush = [&](uint16_t* dst, int64_t stride) {
        __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));   // this wave's LDS writes
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < 128 * 4 / 64; ++k) {
            const int id = lane + 64 * k;
            const int rw = id >> 2, cc = id & 3;
            const int row = rbase + rw;
            if (row >= kFirstOut && s_pos[row] >= 0) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(wout + rw * 32 + cc * 8);
                *reinterpret_cast<u32x4*>(dst + (row0 + row) * stride + n0 + wn * 32 + cc * 8) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));
        __builtin_amdgcn_wave_barrier();
    };
    if (a.io != nullptr) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) stage_out(i, r, acc[i][j][r]);
            flush(a.io + (int64_t)j * H, a.io_stride);
        }
    }

    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = bf16_val(a.w[(int64_t)ch * K + k]);
    const float bv = a.bias != nullptr ? bf16_val(a.bias[ch]) : 0.f;
    const RowMap rm{s_pos, s_len, s_seq, s_slot};
    // one sequence holds every computed row (and, with halo rows, those too)
    const int p0 = s_pos[0], pl = s_pos[kFBM - 1];
    const bool simple = p0 >= (HALO ? K - 1 : 0) && pl == p0 + kFBM - 1 &&
                        !(a.fin != nullptr && pl == s_len[kFBM - 1] - 1);
    float prev[KH];                                    // the partner's last K-1 rows of the previous quad
#pragma unroll
    for (int m = 0; m < K - 1; ++m) {
        // first row half: bx of the halo rows, from the two lane halves' partial sums
        float hb = 0.f;
        if constexpr (HALO)
            hb = (hacc[m][0] + __shfl_xor(hacc[m][0], 32)) * (hacc[m][1] + __shfl_xor(hacc[m][1], 32));
        prev[m] = wm == 1 ? s_edge[wn][q][m] : hb;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float bx[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) bx[r] = acc[i][0][r] * acc[i][2][r];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float tl[KH];
#pragma unroll
            for (int m = 0; m < K - 1; ++m) tl[m] = __shfl_xor(bx[4 * g + 4 - (K - 1) + m], 32);
            float hx[K - 1 + 4];
#pragma unroll
            for (int m = 0; m < K - 1; ++m) hx[m] = hl ? tl[m] : prev[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) hx[K - 1 + j] = bx[4 * g + j];
#pragma unroll
            for (int m = 0; m < K - 1; ++m) prev[m] = tl[m];
            const int R0 = rbase + i * 32 + 8 * g + 4 * hl;
            if (simple || !quad_special<K>(a, rm, R0, kFirstOut)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float conv = fmaf(wk[K - 1], hx[K - 1 + j], bv);
#pragma unroll
                    for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], hx[j + k], conv);
                    stage_out(i, 4 * g + j, acc[i][1][4 * g + j] * conv);
                }
            } else {
                float cg[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) cg[j] = acc[i][1][4 * g + j];
                quad_general<K>(a, rm, R0, kFirstOut, ch, wk, bv, hx, cg,
                                [&](int j, float v) { stage_out(i, 4 * g + j, v); });
            }
        }
    }
    flush(a.y, a.y_stride);
}

// The wide tile's kernel: its LDS arrays per form (the halo form's 32-deep
// 3-slot ring plus halo rows, row map and hand-off; or the 64-deep 2-slot
// ring alone, exactly 160 KiB, the row map and hand-off going into its second
// W_in slot after the reduction).
template <int K, int D, bool HALO>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fused_wide_kernel(const FusedArgs a) {
    if constexpr (HALO && K > 1) {
        using S = WideStage<32>;
        __shared__ __attribute__((aligned(16))) uint8_t ra0[S::kStageA], ra1[S::kStageA], ra2[S::kStageA];
        __shared__ __attribute__((aligned(16))) uint8_t rb0[S::kStageB], rb1[S::kStageB], rb2[S::kStageB];
        __shared__ __attribute__((aligned(16))) uint8_t halo[(K - 1) * D * 2];
        __shared__ __attribute__((aligned(16))) int map[4 * kFBM];
        __shared__ __attribute__((aligned(16))) float edge[4 * 32 * 4];
        wide_tile<K, D, true, 32, 3>(a, WideLds{{ra0, ra1, ra2}, {rb0, rb1, rb2}, halo, map, edge});
    } else {
        using S = WideStage<64>;
        static_assert(2 * (S::kStageA + S::kStageB) == 160 * 1024, "the ring fills the LDS");
        __shared__ __attribute__((aligned(16))) uint8_t ra0[S::kStageA], ra1[S::kStageA];
        __shared__ __attribute__((aligned(16))) uint8_t rb0[S::kStageB], rb1[S::kStageB];
        wide_tile<K, D, false, 64, 2>(a, WideLds{{ra0, ra1, nullptr}, {rb0, rb1, nullptr}, nullptr,
                                                reinterpret_cast<int*>(rb1),
                                                reinterpret_cast<float*>(rb1 + 4 * kFBM * sizeof(int))});
    }
}


// Installs the staged final states: slot_idx[i] <- fin[i] for every sequence
// with at least one token (an empty sequence leaves its slot as it was).
__global__ __launch_bounds__(kSmallBlock) void fused_state_commit_kernel(const FusedArgs a, int K) {
    const int i = blockIdx.x;
    const int64_t HK = (int64_t)a.H * K;
    const int64_t e = ((int64_t)blockIdx.y * kSmallBlock + threadIdx.x) * 8;
    if (e >= HK) return;
    if (a.cu[i + 1] <= a.cu[i]) return;
    const int64_t slot = a.slot_idx[i];
    if (!slot_ok(slot, a.num_slots)) return;
    const uint4 v = *reinterpret_cast<const uint4*>(a.fin + (int64_t)i * HK + e);
    *reinterpret_cast<uint4*>(a.pool + slot * a.slot_stride + e) = v;
}

int64_t fused_tiles(int64_t total_T, int H, int K) {
    const int64_t out = kFBM - (K - 1);
    return (total_T + out - 1) / out * (H / kFNC);
}

int fused_depth_multiple() { return kFBK * kFStages; }

// After the tile kernel: installs the final states when a pool is given.
static hipError_t fused_commit(const FusedArgs& a, int K, hipStream_t s) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.fin == nullptr) return e;
    const int64_t chunks = (int64_t)a.H * K / 8;
    hipLaunchKernelGGL(fused_state_commit_kernel, dim3(a.N, (unsigned)((chunks + kSmallBlock - 1) / kSmallBlock)),
                       dim3(kSmallBlock), 0, s, a, K);
    return hipGetLastError();
}

template <int K, int NK>
static void fused_launch_main(const FusedArgs& a, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((fused_prefill_kernel<K, NK>), dim3(blocks), dim3(kFThreads), 0, s, a);
}

template <int K, int D, bool HALO>
static void fused_launch_wide(const FusedArgs& a, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((fused_wide_kernel<K, D, HALO>), dim3(blocks), dim3(kWThreads), 0, s, a);
}

// Halo or overlapping wide tiles: the one with the shorter expected span, in
// rounds of resident workgroups, a halo tile counting kHaloTileCost of an
// overlapping one (measured on MI355X, D=H=2048: 88-90 us against 73-74 us
// per round at T=32768 and 65536).  T up to 16384 takes halo tiles (T=4096:
// 1 round instead of 2, 0.098 against 0.137 ms), larger T overlapping ones.
// LFM2SC_FUSED_HALO=0 or 1 in the environment forces a form (and
// LFM2SC_FUSED_WIDE=0 the 4-wave tile instead of the wide one).
constexpr double kHaloTileCost = 1.21;
// A 4-wave tile's cost relative to a wide overlapping tile (1.8 against 2.6 MB
// staged per tile; used only against split and mid tiles).
constexpr double kMainTileCost = 0.80;
// Wide tiles resident on the device at once.
template <int K>
static int wide_resident() {
    static const int resident = [] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_wide_kernel<K, 2048, true>, kWThreads, 0) !=
                hipSuccess || cus <= 0 || per <= 0) {
            (void)hipGetLastError();
            return 256;
        }
        return cus * per;
    }();
    return resident;
}
template <int K>
static bool fused_use_halo(int64_t total_T, int tiles_n) {
    if (K == 1) return false;
    if (const char* e = getenv("LFM2SC_FUSED_HALO")) {
        if (e[0] == '0') return false;
        if (e[0] == '1') return true;
    }
    const int resident = wide_resident<K>();
    const int64_t halo = (total_T + kFBM - 1) / kFBM * tiles_n;
    const int64_t ovl = (total_T + fused_out_rows<K>() - 1) / fused_out_rows<K>() * tiles_n;
    const double rounds_halo = (double)((halo + resident - 1) / resident) * kHaloTileCost;
    const double rounds_ovl = (double)((ovl + resident - 1) / resident);
    return rounds_halo < rounds_ovl;
}


// The tiling of a call: kPlanWide, kPlanWideHalo, kPlanMain (the 4-wave tile),
// or a split / mid tile's channel-or-row code from fused_split_choice (32, 64,
// 128).
constexpr int kPlanWide = 1, kPlanWideHalo = 2, kPlanMain = 3;
template <int K>
static int fused_plan_k(int64_t total_T, int H, int D) {
    const bool unrolled = D == 1024 || D == 1536 || D == 2048;
    bool wide = H % kWNC == 0 && unrolled;
    if (const char* e = getenv("LFM2SC_FUSED_WIDE")) wide = wide && e[0] != '0';   // 0: the 4-wave tile
    const int tiles_n = H / (wide ? kWNC : kFNC);
    const bool halo = wide && fused_use_halo<K>(total_T, tiles_n);
    const int64_t out = halo ? kFBM : fused_out_rows<K>();     // halo tiles output all their rows
    if (unrolled) {   // split or mid tiles when their expected span is shorter (short inputs)
        const int64_t tiles = (total_T + out - 1) / out * tiles_n, res = wide_resident<K>();
        const double other = (double)((tiles + res - 1) / res) * (wide ? (halo ? kHaloTileCost : 1.0) : kMainTileCost);
        const int nc = fused_split_choice(total_T, H, other);
        if (nc != 0) return nc;
    }
    return wide ? (halo ? kPlanWideHalo : kPlanWide) : kPlanMain;
}

int fused_plan(int K, int64_t total_T, int H, int D) {
    switch (K) {
        case 1: return fused_plan_k<1>(total_T, H, D);
        case 2: return fused_plan_k<2>(total_T, H, D);
        case 3: return fused_plan_k<3>(total_T, H, D);
        case 4: return fused_plan_k<4>(total_T, H, D);
    }
    return -1;
}

template <int K>
static hipError_t fused_k(FusedArgs a, hipStream_t s) {
    const int plan = fused_plan_k<K>(a.total_T, a.H, a.D);
    if (plan != kPlanWide && plan != kPlanWideHalo && plan != kPlanMain) {
        const hipError_t e = launch_fused_split(a, K, plan, s);
        return e != hipSuccess ? e : fused_commit(a, K, s);
    }
    const bool wide = plan != kPlanMain, halo = plan == kPlanWideHalo;
    a.tiles_n = a.H / (wide ? kWNC : kFNC);
    const int64_t out = halo ? kFBM : fused_out_rows<K>();
    a.tiles_m = (int)((a.total_T + out - 1) / out);
    const int blocks = pad_xcd(a.tiles_m * a.tiles_n);
    if (wide) {
        auto go = [&](auto halo_c) {
            constexpr bool H = decltype(halo_c)::value;
            switch (a.D) {
                case 1024: fused_launch_wide<K, 1024, H>(a, blocks, s); break;
                case 1536: fused_launch_wide<K, 1536, H>(a, blocks, s); break;
                default: fused_launch_wide<K, 2048, H>(a, blocks, s); break;
            }
        };
        if (halo) go(std::true_type{}); else go(std::false_type{});
    } else {
        switch (a.D) {      // straight-line reductions for the LFM2 hidden sizes
            case 1024: fused_launch_main<K, 1024 / kFBK>(a, blocks, s); break;
            case 1536: fused_launch_main<K, 1536 / kFBK>(a, blocks, s); break;
            case 2048: fused_launch_main<K, 2048 / kFBK>(a, blocks, s); break;
            default: fused_launch_main<K, 0>(a, blocks, s); break;
        }
    }
    return fused_commit(a, K, s);
}

hipError_t launch_fused_prefill(const FusedArgs& a, int K, hipStream_t s) {
    switch (K) {
        case 1: return fused_k<1>(a, s);
        case 2: return fused_k<2>(a, s);
        case 3: return fused_k<3>(a, s);
        case 4: return fused_k<4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace lfm2sc
