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
// work at K = 3).  The reduction runs in stages of kFBK = 64, double-buffered
// in LDS: the next stage's global loads are in flight while the current stage
// feeds the matrix cores.
//
// LDS layout.  A stage holds x rows [256][64] and W_in rows [192][64] (bf16,
// 128 B per row).  16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7):
// the 16 lanes of a ds_read_b128 quarter (16 consecutive rows, one chunk) and
// of a ds_write_b128 quarter (2 rows, all chunks) then touch all 64 banks once.
//
// Epilogue.  bx of every computed row goes to LDS (fp32, reusing the stage
// buffers); each lane then forms conv for its own rows from bx of the K-1
// previous rows (LDS) or, for the first K-1 tokens of a sequence, from the
// initial state; y = C * conv is rounded once to bf16.  Final states are the
// last K entries of [initial state | bx]: the tile that holds a sequence's
// last token writes them to a per-sequence staging block, and a second small
// kernel installs them into the slots after every tile has read its initial
// states (a slot may be read by one tile and written by another).
#include "common.hpp"
#include "kernels.hpp"

namespace lfm2sc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFBM = 256;              // token rows computed per tile
constexpr int kFNC = 64;               // channels per tile
constexpr int kFBN = 3 * kFNC;         // GEMM columns per tile (B | C | xv)
constexpr int kFBK = 32;               // reduction depth per LDS stage
#ifndef LFM2SC_FUSED_STAGES
#define LFM2SC_FUSED_STAGES 4
#endif
constexpr int kFStages = LFM2SC_FUSED_STAGES;   // LDS ring depth: kFStages-1 stages in flight ahead of the one in use
constexpr int kFThreads = 256;         // 4 waves
constexpr int kFRowBytes = kFBK * 2;   // one staged row: 32 bf16 = 64 B = 4 chunks of 16 B
constexpr int kFStageA = kFBM * kFRowBytes;   // 16 KiB
constexpr int kFStageB = kFBN * kFRowBytes;   // 12 KiB
constexpr int kFStage = kFStageA + kFStageB;
constexpr int kFRing = kFStages * kFStage;    // 112 KiB at 4 stages
// One global->LDS instruction moves 64 lanes x 16 B = 16 staged rows; per stage
// the 4 waves move 16 A blocks and 12 B blocks, i.e. 4 + 3 per wave.
constexpr int kFDmaA = kFBM / 16 / 4, kFDmaB = kFBN / 16 / 4, kFDmaPerStage = kFDmaA + kFDmaB;
// Epilogue buffers, carved from the ring once the reduction is done:
// bx channel-major [64][kFBxStride] fp32 (rows at offset kFBxPad, so the K-1
// rows before row 0 exist), then an output staging tile [256][kFOutStride] bf16.
constexpr int kFBxPad = 4;
constexpr int kFBxStride = kFBM + kFBxPad;            // 260 floats: lanes 0..15 of a quarter hit distinct banks
constexpr int kFBxBytes = kFNC * kFBxStride * 4;
constexpr int kFOutStride = kFNC + 8;                  // 72 bf16 = 144 B per staged output row
constexpr int kFOutBytes = kFBM * kFOutStride * 2;
static_assert(kFBxBytes + kFOutBytes <= kFRing, "epilogue buffers must fit in the ring");

template <int K> constexpr int fused_out_rows() { return kFBM - (K - 1); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    f32x2 v = {f, 0.f};
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)) & 0xffffu);
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Swizzled byte offset of 16-byte chunk c of staged row r: rows r, r+4, r+8,
// r+12 put chunk c in four different positions, so the 16 lanes of a
// ds_read_b128 quarter (16 consecutive rows, one chunk) hit all 64 banks once.
__device__ __forceinline__ uint32_t lds_chunk(int r, int c) {
    return (uint32_t)r * kFRowBytes + (uint32_t)((c ^ ((r >> 2) & 3)) << 4);
}

// s_waitcnt that waits until at most n vector-memory operations are outstanding
// (expcnt and lgkmcnt left unconstrained).
template <int n> __device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Workgroup -> (m, n) tile: XCD-contiguous runs of the linear tile order, in
// groups of kFGroupM row tiles that sweep every channel tile, so the workgroups
// an XCD runs at once share x rows and W_in rows in its L2.
#ifndef LFM2SC_FUSED_GROUP_M
#define LFM2SC_FUSED_GROUP_M 4
#endif
constexpr int kFGroupM = LFM2SC_FUSED_GROUP_M;
__device__ __forceinline__ void fused_tile(int lin, int tiles_m, int tiles_n, int& m, int& n) {
    const int per_group = kFGroupM * tiles_n;
    const int g = lin / per_group;
    const int idx = lin - g * per_group;
    const int gm = min(kFGroupM, tiles_m - g * kFGroupM);
    m = g * kFGroupM + idx % gm;
    n = idx / gm;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier between reduction stages without __syncthreads' release
// fence: that fence waits for every outstanding vector-memory operation, i.e.
// for the global->LDS loads of the stages still in flight, which would drain
// the ring at every stage.  It is not needed here: before the barrier each wave
// has waited (wait_vm) for its own loads of the stage about to be read, and
// its LDS reads of the buffer about to be refilled were consumed by its MFMAs.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier for LDS hand-offs in the epilogue: the wave's LDS accesses complete
// (lgkmcnt 0), then the workgroup meets; global stores in flight are not waited
// for (they touch no LDS).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int K>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_prefill_kernel(const FusedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kFRing];
    __shared__ __attribute__((aligned(16))) int s_pos[kFBM];
    __shared__ int s_len[kFBM], s_seq[kFBM];

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

    // Row -> (sequence, position, length) map of the tile, for the epilogue.  It
    // is built before any global->LDS load is issued: waiting on a vector load
    // would also wait on every load issued before it.  The sequence of the
    // tile's first row comes from a wave-uniform (scalar) search; when that
    // sequence covers every computed row, the map is arithmetic, otherwise each
    // row searches cu_seqlens itself.
    {
        const int64_t tf = row0 < 0 ? 0 : row0;
        int lo = 0, hi = a.N;                      // largest s in [0, N) with cu[s] <= tf
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int64_t)a.cu[mid] <= tf) lo = mid; else hi = mid;
        }
        const int64_t c0 = a.cu[lo], c1 = a.cu[lo + 1];
        const int64_t t = row0 + tid;
        int pos = -1, len = 0, seq = lo;
        if (c0 <= tf && c1 >= row0 + kFBM) {       // one sequence holds rows [tf, row0 + 256)
            if (t >= tf) { pos = (int)(t - c0); len = (int)(c1 - c0); }
        } else if (t >= 0 && t < T) {
            int l2 = 0, h2 = a.N;
            while (h2 - l2 > 1) {
                const int mid = (l2 + h2) >> 1;
                if ((int64_t)a.cu[mid] <= t) l2 = mid; else h2 = mid;
            }
            seq = l2;
            const int64_t s0 = a.cu[l2], s1 = a.cu[l2 + 1];
            if (t >= s0 && t < s1) { pos = (int)(t - s0); len = (int)(s1 - s0); }
        }
        s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq;
    }

    // ---------------------------------------------------------------- reduction
    // Global -> LDS, no registers in between: each lane of a 16-row block
    // fetches the chunk that the swizzle places at its LDS slot (row lane/4,
    // position lane%4).  Rows outside [0, T) are clamped to a valid row: they
    // are never stored and never feed another row's conv history.
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
        const int n = (wave + 4 * i) * 16 + brow;                 // staged W_in row: part n / 64, channel n % 64
        const int64_t wrow = (int64_t)(n / kFNC) * H + n0 + (n % kFNC);
        woff[i] = (uint32_t)(wrow * a.D * 2) + bchunk;
    }
    auto issue = [&](int kt) {
        uint8_t* st = smem + (kt % kFStages) * kFStage;
        const uint32_t ko = (uint32_t)kt * kFRowBytes;
#pragma unroll
        for (int i = 0; i < kFDmaA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(st + (wave + 4 * i) * 1024), 16, xoff[i] + ko,
                                                     0, 0, 0);
#pragma unroll
        for (int i = 0; i < kFDmaB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(st + kFStageA + (wave + 4 * i) * 1024), 16,
                                                     woff[i] + ko, 0, 0, 0);
    };

    f32x16 acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = a.D / kFBK;
#pragma unroll
    for (int s = 0; s < kFStages - 1; ++s)
        if (s < nk) issue(s);

    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most the later stages already issued are outstanding
        const int later = min(kFStages - 2, nk - 1 - kt);
        static_assert(kFStages <= 5, "wait cases below cover up to 3 later stages");
        if (later >= 3) wait_vm<3 * kFDmaPerStage>();
        else if (later == 2) wait_vm<2 * kFDmaPerStage>();
        else if (later == 1) wait_vm<kFDmaPerStage>();
        else wait_vm<0>();
        stage_barrier();
        // the buffer of stage kt-1 is free now (every wave is past its reads)
        if (kt + kFStages - 1 < nk) issue(kt + kFStages - 1);
        const uint8_t* sa = smem + (kt % kFStages) * kFStage;
        const uint8_t* sb = sa + kFStageA;
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
    }
    __syncthreads();   // every wave is done with the ring; its space now holds the epilogue buffers

    // ---------------------------------------------------------------- epilogue
    // Accumulator register r of row tile i holds computed row
    // R = wm*128 + i*32 + 8*(r/4) + 4*hl + (r%4) of channel n0 + lcn: lane-local
    // runs of 4 consecutive rows ("quads"), quad (i, g = r/4) starting at
    // R0 = wm*128 + i*32 + 8g + 4hl.
    float* bxT = reinterpret_cast<float*>(smem);                       // [64][kFBxStride], row R at kFBxPad + R
    uint16_t* ost = reinterpret_cast<uint16_t*>(smem + kFBxBytes);     // [256][kFOutStride] bf16
    const int lcn = wn * 32 + q;
    const int ch = n0 + lcn;
    float* bxc = bxT + lcn * kFBxStride + kFBxPad;

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

    // bx of every computed row, channel-major
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int R0 = wm * 128 + i * 32 + 8 * g + 4 * hl;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = acc[i][0][4 * g + j] * acc[i][2][4 * g + j];
            *reinterpret_cast<f32x4*>(bxc + R0) = v;
        }
    lds_barrier();

    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = bf16_val(a.w[(int64_t)ch * K + k]);
    const float bv = a.bias != nullptr ? bf16_val(a.bias[ch]) : 0.f;
    // Entry idx (1 <= idx < K) of sequence seq's initial state for this channel.
    auto s0 = [&](int seq, int idx) -> float {
        if (a.pool == nullptr) return 0.f;
        const int64_t slot = a.slot_idx[seq];
        if (!slot_ok(slot, a.num_slots)) return 0.f;
        return bf16_val(a.pool[slot * a.slot_stride + (int64_t)ch * K + idx]);
    };
    // One sequence covers every computed row (and does not end inside the tile
    // when final states are wanted): no per-row sequence logic.
    const int p0 = s_pos[0], pl = s_pos[kFBM - 1];
    const bool simple = p0 >= 0 && pl == p0 + kFBM - 1 && !(a.fin != nullptr && pl == s_len[kFBM - 1] - 1);

    if (simple) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int R0 = wm * 128 + i * 32 + 8 * g + 4 * hl;
                float hx[K - 1 + 4];
#pragma unroll
                for (int k = 0; k < K - 1; ++k) hx[k] = bxc[R0 - (K - 1) + k];
#pragma unroll
                for (int j = 0; j < 4; ++j) hx[K - 1 + j] = acc[i][0][4 * g + j] * acc[i][2][4 * g + j];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float conv = fmaf(wk[K - 1], hx[K - 1 + j], bv);   // same order as the general path
#pragma unroll
                    for (int k = 0; k < K - 1; ++k) conv = fmaf(wk[k], hx[j + k], conv);
                    stage_out(i, 4 * g + j, acc[i][1][4 * g + j] * conv);
                }
            }
    } else {
    #pragma unroll
        for (int i = 0; i < 4; ++i)
    #pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int R0 = wm * 128 + i * 32 + 8 * g + 4 * hl;
                // bx of rows R0-(K-1) .. R0+3 of this channel: K-1 from LDS, 4 from registers
                float hx[K - 1 + 4];
    #pragma unroll
                for (int k = 0; k < K - 1; ++k) hx[k] = bxc[R0 - (K - 1) + k];
    #pragma unroll
                for (int j = 0; j < 4; ++j) hx[K - 1 + j] = acc[i][0][4 * g + j] * acc[i][2][4 * g + j];
                const int4 p = *reinterpret_cast<const int4*>(s_pos + R0);
                const int pos4[4] = {p.x, p.y, p.z, p.w};
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = R0 + j;
                    const int pos = pos4[j];
                    float conv = fmaf(wk[K - 1], hx[K - 1 + j], bv);
    #pragma unroll
                    for (int k = 0; k < K - 1; ++k) {
                        const int d = K - 1 - k;             // X[pos+1+k] is bx of the token d rows back
                        float h = hx[K - 1 + j - d];
                        if (pos < d) h = (pos >= 0 && row >= K - 1) ? s0(s_seq[row], pos + 1 + k) : 0.f;
                        conv = fmaf(wk[k], h, conv);
                    }
                    stage_out(i, 4 * g + j, acc[i][1][4 * g + j] * conv);
                    if (a.fin != nullptr && row >= K - 1 && pos >= 0 && pos == s_len[row] - 1) {
                        // final state X[len .. len+K-1]: bx of the last tokens, or initial-state entries
                        const int len = pos + 1, seq = s_seq[row];
                        uint16_t* f = a.fin + (int64_t)seq * H * K + (int64_t)ch * K;
    #pragma unroll
                        for (int e = 0; e < K; ++e) {
                            const int idx = len + e;
                            f[e] = bf16_bits(idx >= K ? bxc[row + 1 + e - K] : s0(seq, idx));
                        }
                    }
                }
            }
    }
    flush_rows(a.y, a.y_stride, true);
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

template <int K>
static hipError_t fused_k(FusedArgs a, hipStream_t s) {
    const int64_t out = fused_out_rows<K>();
    a.tiles_m = (int)((a.total_T + out - 1) / out);
    a.tiles_n = a.H / kFNC;
    const int blocks = pad_xcd(a.tiles_m * a.tiles_n);
    hipLaunchKernelGGL((fused_prefill_kernel<K>), dim3(blocks), dim3(kFThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.fin == nullptr) return e;
    const int64_t chunks = (int64_t)a.H * K / 8;
    hipLaunchKernelGGL(fused_state_commit_kernel, dim3(a.N, (unsigned)((chunks + kSmallBlock - 1) / kSmallBlock)),
                       dim3(kSmallBlock), 0, s, a, K);
    return hipGetLastError();
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
