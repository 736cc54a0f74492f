// fused_split.hip -- split tiles of the fused in_proj + ShortConv forward
// (bf16 I/O, fp32 accumulation) for inputs too short to fill the chip with the
// wide tiles of fused.hip.  It computes what those do (MAX Pipelines LFM2
// article, "ShortConv implementation (LFM2ShortConv)"): in_proj projects x[t]
// into B | C | xv, bx = B * xv, the K-tap causal conv over [initial state | bx]
// per sequence, y = C * conv; final states go to the same per-sequence staging
// block, installed into the slots by fused.hip's second kernel.
#include <algorithm>
#include <cstdlib>
#include <string>

#include "fused_common.hpp"

namespace lfm2sc {

// ---------------------------------------------------------------- split tiles
// A tile's time follows the bytes it stages (x rows and W_in rows over all of
// D), which these loops draw at a roughly fixed rate per CU on MI355X (about a
// third of what L2 delivers): a wide tile stages 2.6 MB at D = 2048 (~75 us).  Short inputs fill few tiles (T = 256:
// 16 wide tiles for 256 CUs; any T up to 4096 one round or less), so their
// time is that of one tile.  A split tile is 64 rows x NC channels (NC = 64:
// 1.1 MB at D = 2048; NC = 32: 0.7 MB), and its 4 waves each reduce their own
// quarter of D: a wave stages its quarter-rows through a private 2-slot LDS
// ring, reads the next stage's fragments into registers while the matrix cores
// work on the current one, and meets no other wave until its reduction ends.
// Every row of a split tile is an output (T = 512 at NC = 64, or T = 256 at
// NC = 32, is exactly 256 tiles): the conv history of its first K-1 rows is bx
// of the K-1 x rows before the tile, staged beside the tile's rows, whose B and
// xv come from one more row tile of MFMAs against the same W_in fragments (the
// matrix cores are mostly idle in this load-bound loop).  The four partial sums
// then go through LDS one row tile (32 rows) at a time, added in a fixed order,
// and each thread runs the conv for one channel and NC/8 consecutive rows
// straight from them.
constexpr int kSBM = 64;                       // token rows per split tile (all of them outputs)
constexpr int kSWaves = 4;                     // each reduces a quarter of D
constexpr int kSThreads = kSWaves * 64;
constexpr int kSStageA = kSBM * 64;            // one wave's stage: 64 x rows of 32 bf16 (4 KiB)
constexpr int kSStageH = 16 * 64;              // and a block of 16 rows for the K-1 halo rows
constexpr int kSDmaA = kSBM / 16;              // 1 KiB loads of x rows per wave and stage
constexpr int64_t split_tiles(int64_t total_T, int H, int nc) { return (total_T + kSBM - 1) / kSBM * (H / nc); }

template <int NC>
struct SplitGeom {
    static_assert(NC == 32 || NC == 64, "32 or 64 channels");
    static constexpr int kCT = 3 * NC / 32;    // column tiles: B, C, xv of the NC channels
    static constexpr int kHT = 2 * NC / 32;    // the halo row tile needs B and xv only
    static constexpr int kStageB = 3 * NC * 64;
    static constexpr int kDmaB = 3 * NC / 16;
    static constexpr int kVm = kSDmaA + 1 + kDmaB;
    static constexpr int kCols = 3 * NC;       // partial sums per row: B | C | xv
    static constexpr int kRpt = 32 * NC / kSThreads;    // epilogue rows per thread and row tile
    // halo column tile h -> column tile: the B tiles, then the xv tiles
    __device__ static constexpr int halo_tile(int h) { return h < NC / 32 ? h : h + NC / 32; }
    // Partial sum (row, col) of a [32][kCols] block.  NC = 64: the column of
    // rows 4..7 mod 8 is XOR-ed with 32, so the two lane halves of a store (rows
    // 4 apart, same columns) hit different banks; NC = 32: plain.
    __device__ static int pidx(int row, int col) {
        if constexpr (NC == 64) return row * kCols + (col ^ (((row >> 2) & 1) << 5));
        else return row * kCols + col;
    }
};

__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));
}

// One wave's stage loads, global -> LDS: its 4 blocks of x rows, the halo block
// and the W_in blocks.
template <int NC>
__device__ __forceinline__ void split_issue(rsrc_t xr, rsrc_t hr, rsrc_t wr, uint8_t* sa, uint8_t* sh, uint8_t* sb,
                                            const uint32_t* xoff, uint32_t hoff, const uint32_t* woff, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < kSDmaA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(sa + i * 1024), 16, xoff[i] + ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, (lds_ptr_t)sh, 16, hoff + ko, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < SplitGeom<NC>::kDmaB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(sb + i * 1024), 16, woff[i] + ko, 0, 0, 0);
}

// A stage's MFMA operands: [row tile][k step] of x, [k step] of the halo rows,
// [column tile][k step] of W_in.
template <int NC>
struct SplitFrags {
    bf16x8 a[2][2];
    bf16x8 h[2];
    bf16x8 b[SplitGeom<NC>::kCT][2];
};
template <int NC>
__device__ __forceinline__ void split_read(SplitFrags<NC>& f, const uint8_t* sa, const uint8_t* sh, const uint8_t* sb,
                                           int q, int hl) {
    using S = WideStage<32>;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int c = kk * 2 + hl;
#pragma unroll
        for (int i = 0; i < 2; ++i) f.a[i][kk] = *reinterpret_cast<const bf16x8*>(sa + S::chunk(i * 32 + q, c));
        // rows 16..31 of the halo row tile repeat rows 0..15: their sums are never read
        f.h[kk] = *reinterpret_cast<const bf16x8*>(sh + S::chunk(q & 15, c));
#pragma unroll
        for (int j = 0; j < SplitGeom<NC>::kCT; ++j)
            f.b[j][kk] = *reinterpret_cast<const bf16x8*>(sb + S::chunk(j * 32 + q, c));
    }
}

template <int K, int D, int NC>
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_split_kernel(const FusedArgs a) {
    using S = WideStage<32>;                           // 64-byte staged rows: its swizzle and chunk map
    using G = SplitGeom<NC>;
    constexpr int NKW = D / kSWaves / 32;              // stages per wave
    static_assert(D % (kSWaves * 32) == 0 && NKW >= 3, "whole stages, at least three per wave");
    constexpr int KH = K > 1 ? K - 1 : 1;
    constexpr int CT = G::kCT, HT = G::kHT, RPT = G::kRpt;
    constexpr int HTK = K > 1 ? HT : 0;                // halo MFMAs per k step (none without history)
    constexpr int kMf = 2 * (2 * CT + HTK);            // MFMAs per wave and stage
    static_assert(KH < RPT, "a thread's history rows lie in the group before it");
    __shared__ __attribute__((aligned(16))) uint8_t sa0[kSWaves * kSStageA], sa1[kSWaves * kSStageA];
    __shared__ __attribute__((aligned(16))) uint8_t sh0[kSWaves * kSStageH], sh1[kSWaves * kSStageH];
    __shared__ __attribute__((aligned(16))) uint8_t sb0[kSWaves * G::kStageB], sb1[kSWaves * G::kStageB];
    __shared__ int s_pos[kSBM], s_len[kSBM], s_seq[kSBM], s_slot[kSBM];
    __shared__ float s_hpart[kSWaves][KH][2 * NC];     // halo rows' B | xv partial sums per wave
    __shared__ float s_edge[KH][NC];                   // bx of rows 32-(K-1) .. 31 (the second row tile's history)

    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    if (lin >= a.tiles_m * a.tiles_n) return;
    int mt, nt;
    fused_tile(lin, a.tiles_m, a.tiles_n, mt, nt);
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int q = lane & 31, hl = lane >> 5;
    const int H = a.H;
    const int64_t T = a.total_T;
    const int64_t row0 = (int64_t)mt * kSBM;           // token of row 0 of the tile
    const int n0 = nt * NC;

    {   // row map, before any load of the reduction
        const TileSeq f = tile_first_seq(a, row0);
        if (tid < kSBM) {
            int pos, len, seq, sid;
            tile_row(a, f, row0, kSBM, tid, pos, len, seq, sid);
            s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq; s_slot[tid] = sid;
        }
    }

    // ---------------------------------------------------------------- reduction
    // Wave w reduces k in [w*D/4, (w+1)*D/4).  Staged rows: the tile's x rows
    // (rows at or past T clamped to a valid row: never outputs, never history
    // of an output); the halo block, whose rows e < K-1 are x rows row0-(K-1)+e
    // when those exist (the rest lie outside its descriptor and read as zero
    // without a memory access); W_in rows (n / NC) * H + n0 + n % NC.
    const int64_t vhi = (row0 + kSBM < T) ? row0 + kSBM : T;     // > row0 for every launched tile
    const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)((vhi - row0) * a.x_stride * 2));
    const rsrc_t xr = row_rsrc(a.x + row0 * a.x_stride, xbytes);
    const int64_t hlo = row0 - (K - 1) < 0 ? 0 : row0 - (K - 1);
    const uint32_t hbytes = __builtin_amdgcn_readfirstlane((uint32_t)((row0 - hlo) * a.x_stride * 2));
    const rsrc_t hr = row_rsrc(a.x + hlo * a.x_stride, hbytes);
    const rsrc_t wr = row_rsrc(a.W, (uint32_t)((int64_t)3 * H * D * 2));
    const int brow = lane >> 2;
    const uint32_t kq = (uint32_t)wave * (D / kSWaves) * 2;      // byte offset of the wave's k range
    uint32_t xoff[kSDmaA], woff[G::kDmaB];
#pragma unroll
    for (int i = 0; i < kSDmaA; ++i) {
        const int r = 16 * i + brow;
        int64_t t = row0 + r;
        t = t >= vhi ? vhi - 1 : t;
        xoff[i] = (uint32_t)((t - row0) * a.x_stride * 2) + kq + S::dma_chunk(lane, r);
    }
    uint32_t hoff;
    {
        const int64_t t = row0 - (K - 1) + brow;
        hoff = (brow < K - 1 && t >= hlo) ? (uint32_t)((t - hlo) * a.x_stride * 2) + kq + S::dma_chunk(lane, brow)
                                          : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < G::kDmaB; ++i) {
        const int n = 16 * i + brow;
        woff[i] = (uint32_t)(((int64_t)(n / NC) * H + n0 + (n % NC)) * D * 2) + kq + S::dma_chunk(lane, n);
    }
    uint8_t* const xa0 = sa0 + wave * kSStageA;
    uint8_t* const xa1 = sa1 + wave * kSStageA;
    uint8_t* const ha0 = sh0 + wave * kSStageH;
    uint8_t* const ha1 = sh1 + wave * kSStageH;
    uint8_t* const wb0 = sb0 + wave * G::kStageB;
    uint8_t* const wb1 = sb1 + wave * G::kStageB;

    f32x16 acc[2][CT], acch[HT];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < CT; ++j) acc[i][j][r] = 0.f;
#pragma unroll
        for (int j = 0; j < HT; ++j) acch[j][r] = 0.f;
    }
    SplitFrags<NC> fr[2];
    auto mfma = [&](const SplitFrags<NC>& f, int m) {   // MFMA m of a stage, k step major
        constexpr int per = 2 * CT + HTK;
        const int kk = m / per, t = m % per;
        if (t < 2 * CT)
            acc[t / CT][t % CT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[t / CT][kk], f.b[t % CT][kk],
                                                                        acc[t / CT][t % CT], 0, 0, 0);
        else
            acch[t - 2 * CT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                f.h[kk], f.b[G::halo_tile(t - 2 * CT)][kk], acch[t - 2 * CT], 0, 0, 0);
    };

    // Stage s computes from fr[s & 1] (read during stage s-1); meanwhile it
    // reads stage s+1 from its slot into fr[(s+1) & 1], then refills that slot
    // with stage s+3.  Stages s+1 and s+2 are in flight when it starts.
    split_issue<NC>(xr, hr, wr, xa0, ha0, wb0, xoff, hoff, woff, 0);
    split_issue<NC>(xr, hr, wr, xa1, ha1, wb1, xoff, hoff, woff, 64);
    wait_vm<G::kVm>();
    split_read<NC>(fr[0], xa0, ha0, wb0, q, hl);
    wait_lgkm0();
    split_issue<NC>(xr, hr, wr, xa0, ha0, wb0, xoff, hoff, woff, 2 * 64);
    auto stage = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int cur = s & 1, nxt = cur ^ 1;
        constexpr int kLead = 8;                       // MFMAs before the refill: the reads above land meanwhile
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s + 1 < NKW) {
            wait_vm<(s + 2 < NKW) ? G::kVm : 0>();
            split_read<NC>(fr[nxt], nxt ? xa1 : xa0, nxt ? ha1 : ha0, nxt ? wb1 : wb0, q, hl);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < kLead; ++m) mfma(fr[cur], m);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s + 3 < NKW) {
            wait_lgkm0();
            __builtin_amdgcn_sched_barrier(0);
            split_issue<NC>(xr, hr, wr, nxt ? xa1 : xa0, nxt ? ha1 : ha0, nxt ? wb1 : wb0, xoff, hoff, woff,
                            (uint32_t)(s + 3) * 64);
        }
#pragma unroll
        for (int m = kLead; m < kMf; ++m) mfma(fr[cur], m);
        if constexpr (s + 3 < NKW) {
            constexpr int per = (kMf - kLead) / G::kVm;        // refill loads spread over the MFMAs
#pragma unroll
            for (int m = 0; m < G::kVm; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, per > 0 ? per : 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    unroll_stages<0, NKW>(stage);

    // ---------------------------------------------------------------- epilogue
    // Accumulator register r of row tile i, column tile j holds row
    // i*32 + 8*(r/4) + 4*hl + (r%4), column j*32 + q (columns: B of the NC
    // channels, then C, then xv); of the halo row tile, registers r < K-1 of the
    // lanes hl = 0 hold halo rows r.  Partials [32][3NC] fp32 per wave, in the
    // W_in halves of the ring.
    if (hl == 0) {
#pragma unroll
        for (int j = 0; j < HT; ++j)
#pragma unroll
            for (int e = 0; e < K - 1; ++e) s_hpart[wave][e][j * 32 + q] = acch[j][e];
    }
    lds_barrier();                                     // every wave's reduction is done
    float* const part0 = reinterpret_cast<float*>(sb0);
    float* const part1 = part0 + 32 * G::kCols;
    float* const part2 = reinterpret_cast<float*>(sb1);
    float* const part3 = part2 + 32 * G::kCols;
    float* const mine = wave == 0 ? part0 : wave == 1 ? part1 : wave == 2 ? part2 : part3;
    auto psum = [&](int row, int col) {
        const int o = G::pidx(row, col);
        return ((part0[o] + part1[o]) + part2[o]) + part3[o];
    };
    const int c = tid % NC;                            // epilogue thread: channel n0 + c,
    const int grp = tid / NC;                          // rows RPT*grp .. +RPT of each row tile
    const int ch = n0 + c;
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = bf16_val(a.w[(int64_t)ch * K + k]);
    const float bv = a.bias != nullptr ? bf16_val(a.bias[ch]) : 0.f;

#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[G::pidx(8 * (r >> 2) + 4 * hl + (r & 3), 32 * j + q)] = acc[p][j][r];
        lds_barrier();
        // Initial-state entries the rows need, fetched together first from
        // addresses chosen without branching (an entry not needed reads the
        // channel's weight instead).
        float sv[RPT][KH];
        bool any = false;                              // does a row of this thread start a sequence?
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int pos = s_pos[32 * p + RPT * grp + i];
            any = any || (pos >= 0 && pos < K - 1 && s_slot[32 * p + RPT * grp + i] >= 0);
#pragma unroll
            for (int k = 0; k < KH; ++k) sv[i][k] = 0.f;
        }
        if (any) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int R = 32 * p + RPT * grp + i;
                const int pos = s_pos[R], slot = s_slot[R];
#pragma unroll
                for (int k = 0; k < KH; ++k) {
                    const bool need = k < K - 1 && pos >= 0 && pos < K - 1 - k && slot >= 0;
                    const uint16_t* src = need ? a.pool + (int64_t)slot * a.slot_stride + (int64_t)ch * K + pos + 1 + k
                                               : a.w + (int64_t)ch * K;
                    sv[i][k] = need ? bf16_val(*src) : 0.f;
                }
            }
        }
        // hb[m]: bx of row RPT*grp - (K-1) + m of this row tile
        float hb[KH + RPT];
#pragma unroll
        for (int m = 0; m < K - 1; ++m) {
            const int rr = RPT * grp - (K - 1) + m;
            float v;
            if (rr >= 0) v = psum(rr, c) * psum(rr, 2 * NC + c);
            else if (p == 1) v = s_edge[m][c];         // rr < 0 only for grp 0: rows 32-(K-1)+m of row tile 0
            else                                       // p == 0, grp 0: halo row m
                v = (((s_hpart[0][m][c] + s_hpart[1][m][c]) + s_hpart[2][m][c]) + s_hpart[3][m][c]) *
                    (((s_hpart[0][m][NC + c] + s_hpart[1][m][NC + c]) + s_hpart[2][m][NC + c]) + s_hpart[3][m][NC + c]);
            hb[m] = v;
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) hb[K - 1 + i] = psum(RPT * grp + i, c) * psum(RPT * grp + i, 2 * NC + c);
        if (p == 0 && grp == kSThreads / NC - 1) {
#pragma unroll
            for (int e = 0; e < K - 1; ++e) s_edge[e][c] = hb[RPT + e];
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int R = 32 * p + RPT * grp + i;      // row of the tile
            const int pos = s_pos[R];
            if (pos < 0) continue;                     // no sequence's token
            const float bxr = hb[K - 1 + i];
            float h[KH];
#pragma unroll
            for (int k = 0; k < K - 1; ++k) h[k] = pos < K - 1 - k ? sv[i][k] : hb[i + k];
            float conv = fmaf(wk[K - 1], bxr, bv);
#pragma unroll
            for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], h[k], conv);
            const int64_t t = row0 + R;
            const float cg = psum(RPT * grp + i, NC + c);
            a.y[t * a.y_stride + ch] = bf16_bits(cg * conv);
            if (a.io != nullptr) {
                uint16_t* io = a.io + t * a.io_stride + ch;
                io[0] = bf16_bits(psum(RPT * grp + i, c));
                io[H] = bf16_bits(cg);
                io[2 * H] = bf16_bits(psum(RPT * grp + i, 2 * NC + c));
            }
            if (a.fin != nullptr && pos == s_len[R] - 1) {
                uint16_t* f = a.fin + (int64_t)s_seq[R] * H * K + (int64_t)ch * K;
#pragma unroll
                for (int e = 0; e < K - 1; ++e) f[e] = bf16_bits(h[e]);
                f[K - 1] = bf16_bits(bxr);
            }
        }
        if (p == 0) lds_barrier();                     // partials are overwritten next; s_edge written
    }
}

// ---------------------------------------------------------------- mid tiles
// Between the split tiles and the wide ones (T ~ 512 .. 1024 at H = 2048) a CU
// has ~25k GEMM outputs to produce; the tile that stages the fewest bytes for
// that is 128 rows x 64 channels (1.3 MB at D = 2048, one round at T = 1024,
// against 2 rounds of 64-row split tiles or a 2.6 MB wide tile).  8 waves: k
// half x row half x channel half, each wave 64 rows x 32 channels over its half
// of D; the waves of a k half share its staged x and W_in rows, so the stages
// meet at a workgroup barrier (3-slot ring, 2 stages in flight, as in the halo
// form of the wide tile).  The halo rows' B and xv come from one more MFMA row
// tile per k step, B in the row half 0 waves and xv in the row half 1 waves;
// the two k halves' partial sums and the LDS epilogue work as in the split
// tiles.
constexpr int kMBM = 128;                      // token rows per mid tile (all of them outputs)
constexpr int kMNC = 64;                       // channels per mid tile
constexpr int kMThreads = 512;
constexpr int kMHalf = 21 * 1024;              // one k half of a stage: x 8 KiB, halo block 1 KiB, W_in 12 KiB
constexpr int kMHalo = 8 * 1024, kMW = 9 * 1024;
constexpr int kMSlot = 48 * 1024;              // a ring slot (both k halves); after the reduction, 64 rows of partials
constexpr int kMVm = 5;                        // loads per wave and stage (the halo block: one more for wave 0 of a half)
constexpr int64_t mid_tiles(int64_t total_T, int H) { return (total_T + kMBM - 1) / kMBM * (H / kMNC); }

// One wave's loads of a stage: blocks gi, gi+4 of the half's 8 x blocks, gi, gi+4,
// gi+8 of its 12 W_in blocks, and for gi == 0 the halo block.
__device__ __forceinline__ void mid_issue(rsrc_t xr, rsrc_t hr, rsrc_t wr, uint8_t* half, int gi,
                                          const uint32_t* xoff, uint32_t hoff, const uint32_t* woff, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(half + (gi + 4 * i) * 1024), 16, xoff[i] + ko, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 3; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(half + kMW + (gi + 4 * i) * 1024), 16, woff[i] + ko, 0,
                                                 0, 0);
    if (gi == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, (lds_ptr_t)(half + kMHalo), 16, hoff + ko, 0, 0, 0);
}

template <int K, int D>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fused_mid_kernel(const FusedArgs a) {
    using S = WideStage<32>;
    using G = SplitGeom<kMNC>;                         // partial-sum layout of 64-row blocks
    constexpr int NKH = D / 2 / 32;                    // stages (each covers 32 k of both halves)
    static_assert(D % 64 == 0 && NKH >= 3, "whole stages, at least three");
    constexpr int KH = K > 1 ? K - 1 : 1;
    constexpr int kRpt = kMBM / (kMThreads / kMNC);    // epilogue rows per thread (16)
    __shared__ __attribute__((aligned(16))) uint8_t r0[kMSlot], r1[kMSlot], r2[kMSlot];
    __shared__ int s_pos[kMBM], s_len[kMBM], s_seq[kMBM], s_slot[kMBM];
    __shared__ float s_hpart[KH][2 * kMNC];            // halo rows' B | xv (partials, then sums)

    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    if (lin >= a.tiles_m * a.tiles_n) return;
    int mt, nt;
    fused_tile(lin, a.tiles_m, a.tiles_n, mt, nt);
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int q = lane & 31, hl = lane >> 5;
    const int kh = wave >> 2, rh = (wave >> 1) & 1, chh = wave & 1, gi = wave & 3;
    const int H = a.H;
    const int64_t T = a.total_T;
    const int64_t row0 = (int64_t)mt * kMBM;
    const int n0 = nt * kMNC;

    {   // row map, before any load of the reduction
        const TileSeq f = tile_first_seq(a, row0);
        if (tid < kMBM) {
            int pos, len, seq, sid;
            tile_row(a, f, row0, kMBM, tid, pos, len, seq, sid);
            s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq; s_slot[tid] = sid;
        }
    }

    // ---------------------------------------------------------------- reduction
    const int64_t vhi = (row0 + kMBM < T) ? row0 + kMBM : T;
    const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)((vhi - row0) * a.x_stride * 2));
    const rsrc_t xr = row_rsrc(a.x + row0 * a.x_stride, xbytes);
    const int64_t hlo = row0 - (K - 1) < 0 ? 0 : row0 - (K - 1);
    const uint32_t hbytes = __builtin_amdgcn_readfirstlane((uint32_t)((row0 - hlo) * a.x_stride * 2));
    const rsrc_t hr = row_rsrc(a.x + hlo * a.x_stride, hbytes);
    const rsrc_t wr = row_rsrc(a.W, (uint32_t)((int64_t)3 * H * D * 2));
    const int brow = lane >> 2;
    const uint32_t kq = (uint32_t)kh * D;              // byte offset of the half's k range (D/2 bf16)
    uint32_t xoff[2], woff[3];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * (gi + 4 * i) + brow;
        int64_t t = row0 + r;
        t = t >= vhi ? vhi - 1 : t;
        xoff[i] = (uint32_t)((t - row0) * a.x_stride * 2) + kq + S::dma_chunk(lane, r);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int n = 16 * (gi + 4 * i) + brow;
        woff[i] = (uint32_t)(((int64_t)(n / kMNC) * H + n0 + (n % kMNC)) * D * 2) + kq + S::dma_chunk(lane, n);
    }
    uint32_t hoff;
    {
        const int64_t t = row0 - (K - 1) + brow;
        hoff = (brow < K - 1 && t >= hlo) ? (uint32_t)((t - hlo) * a.x_stride * 2) + kq + S::dma_chunk(lane, brow)
                                          : 0x80000000u;
    }
    auto half = [&](int u) -> uint8_t* { return (u == 0 ? r0 : u == 1 ? r1 : r2) + kh * kMHalf; };

    f32x16 acc[2][3], acch;                            // acch: halo rows, B (row half 0) or xv (row half 1)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) acc[i][j][r] = 0.f;
        acch[r] = 0.f;
    }

    // Each stage's two k steps alternate between two fragment sets so that the
    // LDS reads of one land under the MFMAs of the other: k step 1 of stage s is
    // read during k step 0; then (barrier: stage s+1 has landed and every wave
    // is done with stage s's slot) the slot is refilled with stage s+3 and k
    // step 0 of stage s+1 is read during k step 1.  Two stages stay in flight
    // (the three slots: one read, two landing).
    struct Frags { bf16x8 a[2], b[3], h; };
    auto read = [&](Frags& f, const uint8_t* h, int kk) {
        const int c = kk * 2 + hl;
#pragma unroll
        for (int i = 0; i < 2; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(h + S::chunk(rh * 64 + i * 32 + q, c));
#pragma unroll
        for (int j = 0; j < 3; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(h + kMW + S::chunk(j * kMNC + chh * 32 + q, c));
        if (K > 1) f.h = *reinterpret_cast<const bf16x8*>(h + kMHalo + S::chunk(q & 15, c));
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        if (K > 1)                                     // halo rows: the row halves split B and xv, balancing the SIMDs
            acch = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.h, rh == 0 ? f.b[0] : f.b[2], acch, 0, 0, 0);
    };
    Frags f0, f1;
    mid_issue(xr, hr, wr, half(0), gi, xoff, hoff, woff, 0);
    mid_issue(xr, hr, wr, half(1), gi, xoff, hoff, woff, 64);
    mid_issue(xr, hr, wr, half(2), gi, xoff, hoff, woff, 2 * 64);
    if (gi == 0) wait_vm<2 * (kMVm + 1)>(); else wait_vm<2 * kMVm>();
    stage_barrier();
    read(f0, half(0), 0);
    wait_lgkm0();
    auto stage = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        read(f1, half(s % 3), 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(f0);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        if constexpr (s + 1 < NKH) {
            constexpr int later = s + 2 < NKH ? 1 : 0;     // stages after s+1 still in flight
            if (gi == 0) wait_vm<later * (kMVm + 1)>(); else wait_vm<later * kMVm>();
            stage_barrier();                               // stage s+1 landed; slot s % 3 read by every wave
            if constexpr (s + 3 < NKH)
                mid_issue(xr, hr, wr, half(s % 3), gi, xoff, hoff, woff, (uint32_t)(s + 3) * 64);
            read(f0, half((s + 1) % 3), 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mma(f1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s + 1 < NKH) wait_lgkm0();
    };
    unroll_stages<0, NKH>(stage);

    // ---------------------------------------------------------------- epilogue
    // Row half rh's partials [64][192] live in slot rh (after the ring drains):
    // the k half 1 waves store theirs, the k half 0 waves add their own in place
    // (each element read and written by the same lane), then every thread runs
    // the conv for one channel and 16 consecutive rows.
    lds_barrier();
    float* const prt = reinterpret_cast<float*>(rh == 0 ? r0 : r1);
    if (kh == 1) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    prt[G::pidx(i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3), j * kMNC + chh * 32 + q)] = acc[i][j][r];
        if (hl == 0) {
#pragma unroll
            for (int e = 0; e < K - 1; ++e) s_hpart[e][rh * kMNC + chh * 32 + q] = acch[e];
        }
    }
    lds_barrier();
    if (kh == 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float* p = prt + G::pidx(i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3), j * kMNC + chh * 32 + q);
                    *p = acc[i][j][r] + *p;
                }
        if (hl == 0) {
#pragma unroll
            for (int e = 0; e < K - 1; ++e)
                s_hpart[e][rh * kMNC + chh * 32 + q] = acch[e] + s_hpart[e][rh * kMNC + chh * 32 + q];
        }
    }
    lds_barrier();

    const float* const p0 = reinterpret_cast<const float*>(r0);
    const float* const p1 = reinterpret_cast<const float*>(r1);
    auto psum = [&](int row, int col) { return (row < 64 ? p0 : p1)[G::pidx(row & 63, col)]; };
    const int c = tid % kMNC;
    const int grp = tid / kMNC;                        // rows kRpt*grp .. +kRpt
    const int ch = n0 + c;
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = bf16_val(a.w[(int64_t)ch * K + k]);
    const float bv = a.bias != nullptr ? bf16_val(a.bias[ch]) : 0.f;
    float sv[kRpt][KH];
    bool any = false;                                  // does a row of this thread start a sequence?
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
        const int pos = s_pos[kRpt * grp + i];
        any = any || (pos >= 0 && pos < K - 1 && s_slot[kRpt * grp + i] >= 0);
#pragma unroll
        for (int k = 0; k < KH; ++k) sv[i][k] = 0.f;
    }
    if (any) {
#pragma unroll
        for (int i = 0; i < kRpt; ++i) {
            const int R = kRpt * grp + i;
            const int pos = s_pos[R], slot = s_slot[R];
#pragma unroll
            for (int k = 0; k < KH; ++k) {
                const bool need = k < K - 1 && pos >= 0 && pos < K - 1 - k && slot >= 0;
                const uint16_t* src = need ? a.pool + (int64_t)slot * a.slot_stride + (int64_t)ch * K + pos + 1 + k
                                           : a.w + (int64_t)ch * K;
                sv[i][k] = need ? bf16_val(*src) : 0.f;
            }
        }
    }
    float hb[KH + kRpt];                               // bx of rows kRpt*grp - (K-1) .. kRpt*grp + kRpt - 1
#pragma unroll
    for (int m = 0; m < K - 1; ++m) {
        const int rr = kRpt * grp - (K - 1) + m;
        hb[m] = rr >= 0 ? psum(rr, c) * psum(rr, 2 * kMNC + c) : s_hpart[m][c] * s_hpart[m][kMNC + c];
    }
#pragma unroll
    for (int i = 0; i < kRpt; ++i) hb[K - 1 + i] = psum(kRpt * grp + i, c) * psum(kRpt * grp + i, 2 * kMNC + c);
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
        const int R = kRpt * grp + i;
        const int pos = s_pos[R];
        if (pos < 0) continue;
        const float bxr = hb[K - 1 + i];
        float h[KH];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) h[k] = pos < K - 1 - k ? sv[i][k] : hb[i + k];
        float conv = fmaf(wk[K - 1], bxr, bv);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], h[k], conv);
        const int64_t t = row0 + R;
        const float cg = psum(R, kMNC + c);
        a.y[t * a.y_stride + ch] = bf16_bits(cg * conv);
        if (a.io != nullptr) {
            uint16_t* io = a.io + t * a.io_stride + ch;
            io[0] = bf16_bits(psum(R, c));
            io[H] = bf16_bits(cg);
            io[2 * H] = bf16_bits(psum(R, 2 * kMNC + c));
        }
        if (a.fin != nullptr && pos == s_len[R] - 1) {
            uint16_t* f = a.fin + (int64_t)s_seq[R] * H * K + (int64_t)ch * K;
#pragma unroll
            for (int e = 0; e < K - 1; ++e) f[e] = bf16_bits(h[e]);
            f[K - 1] = bf16_bits(bxr);
        }
    }
}

template <int K, int D, int NC>
static void split_launch(const FusedArgs& a, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((fused_split_kernel<K, D, NC>), dim3(blocks), dim3(kSThreads), 0, s, a);
}

template <int K, int NC>
static void split_k(const FusedArgs& a, int blocks, hipStream_t s) {
    switch (a.D) {
        case 1024: split_launch<K, 1024, NC>(a, blocks, s); break;
        case 1536: split_launch<K, 1536, NC>(a, blocks, s); break;
        default: split_launch<K, 2048, NC>(a, blocks, s); break;
    }
}

template <int K>
static void mid_k(const FusedArgs& a, int blocks, hipStream_t s) {
    switch (a.D) {
        case 1024: hipLaunchKernelGGL((fused_mid_kernel<K, 1024>), dim3(blocks), dim3(kMThreads), 0, s, a); break;
        case 1536: hipLaunchKernelGGL((fused_mid_kernel<K, 1536>), dim3(blocks), dim3(kMThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((fused_mid_kernel<K, 2048>), dim3(blocks), dim3(kMThreads), 0, s, a); break;
    }
}

hipError_t launch_fused_split(FusedArgs a, int K, int nc, hipStream_t s) {
    if (nc == kMBM) {                                  // mid tiles: 128 rows x 64 channels
        a.tiles_n = a.H / kMNC;
        a.tiles_m = (int)((a.total_T + kMBM - 1) / kMBM);
        const int blocks = pad_xcd(a.tiles_m * a.tiles_n);
        switch (K) {
            case 1: mid_k<1>(a, blocks, s); break;
            case 2: mid_k<2>(a, blocks, s); break;
            case 3: mid_k<3>(a, blocks, s); break;
            case 4: mid_k<4>(a, blocks, s); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    a.tiles_n = a.H / nc;
    a.tiles_m = (int)((a.total_T + kSBM - 1) / kSBM);
    const int blocks = pad_xcd(a.tiles_m * a.tiles_n);
    switch (K * 100 + nc) {
        case 132: split_k<1, 32>(a, blocks, s); break;
        case 164: split_k<1, 64>(a, blocks, s); break;
        case 232: split_k<2, 32>(a, blocks, s); break;
        case 264: split_k<2, 64>(a, blocks, s); break;
        case 332: split_k<3, 32>(a, blocks, s); break;
        case 364: split_k<3, 64>(a, blocks, s); break;
        case 432: split_k<4, 32>(a, blocks, s); break;
        case 464: split_k<4, 64>(a, blocks, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// A split or mid tile's cost relative to a wide overlapping tile, measured on
// MI355X at D = H = 2048 (it follows the bytes a tile stages: 1.1 MB for a split
// tile of 64 channels, 0.7 MB at 32, 1.3 MB for a mid tile, 2.6 MB for the wide
// tile).
constexpr double kSplitTileCost64 = 0.45, kSplitTileCost32 = 0.30, kMidTileCost = 0.60;

int fused_split_choice(int64_t total_T, int H, double other) {
    const bool ok64 = H % 64 == 0 && split_tiles(total_T, H, 64) < (1 << 30);
    const bool ok32 = H % 32 == 0 && split_tiles(total_T, H, 32) < (1 << 30);
    const bool okm = H % kMNC == 0 && mid_tiles(total_T, H) < (1 << 30);
    bool force = false;
    if (const char* e = getenv("LFM2SC_FUSED_SPLIT")) {
        const std::string v(e);
        if (v == "0") return 0;
        if (v == "64") return ok64 ? 64 : 0;
        if (v == "32") return ok32 ? 32 : 0;
        if (v == "128") return okm ? kMBM : 0;
        force = v == "1";
    }
    // workgroups resident at once: split and mid tiles both fit one per CU (LDS)
    static const int resident = [] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_split_kernel<3, 2048, 64>, kSThreads, 0) !=
                hipSuccess || cus <= 0 || per <= 0) {
            (void)hipGetLastError();
            return 256;
        }
        return cus * per;
    }();
    auto span = [&](int64_t tiles, double cost) { return (double)((tiles + resident - 1) / resident) * cost; };
    const double s64 = ok64 ? span(split_tiles(total_T, H, 64), kSplitTileCost64) : 1e300;
    const double s32 = ok32 ? span(split_tiles(total_T, H, 32), kSplitTileCost32) : 1e300;
    const double sm = okm ? span(mid_tiles(total_T, H), kMidTileCost) : 1e300;
    if (!ok64 && !ok32 && !okm) return 0;
    int best = s32 < s64 ? 32 : 64;
    double bs = std::min(s32, s64);
    if (sm < bs) { best = kMBM; bs = sm; }
    if (force) return best;
    return bs < other ? best : 0;
}

}  // namespace lfm2sc
