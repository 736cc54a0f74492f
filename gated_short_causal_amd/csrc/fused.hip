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

constexpr int kFBM = 256;              // token rows computed per tile
constexpr int kFNC = 64;               // channels per tile
constexpr int kFBN = 3 * kFNC;         // GEMM columns per tile (B | C | xv)
constexpr int kFBK = 64;               // reduction depth per LDS stage
constexpr int kFThreads = 256;         // 4 waves
constexpr int kFRowBytes = kFBK * 2;   // one staged row: 64 bf16 = 128 B
constexpr int kFStageA = kFBM * kFRowBytes;   // 32 KiB
constexpr int kFStageB = kFBN * kFRowBytes;   // 24 KiB
constexpr int kFStage = kFStageA + kFStageB;
constexpr int kFLds = 2 * kFStage;            // 112 KiB, double-buffered
static_assert(kFBM * kFNC * 4 <= kFLds, "bx tile must fit in the stage buffers");

template <int K> constexpr int fused_out_rows() { return kFBM - (K - 1); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    f32x2 v = {f, 0.f};
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)) & 0xffffu);
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Swizzled byte offset of 16-byte chunk c of staged row r.
__device__ __forceinline__ uint32_t lds_chunk(int r, int c) {
    return (uint32_t)r * kFRowBytes + (uint32_t)((c ^ ((r >> 1) & 7)) << 4);
}

// Workgroup -> (m, n) tile: XCD-contiguous runs of the linear tile order, in
// groups of kFGroupM row tiles that sweep every channel tile, so the workgroups
// an XCD runs at once share x rows and W_in rows in its L2.
constexpr int kFGroupM = 4;
__device__ __forceinline__ void fused_tile(int lin, int tiles_m, int tiles_n, int& m, int& n) {
    const int per_group = kFGroupM * tiles_n;
    const int g = lin / per_group;
    const int idx = lin - g * per_group;
    const int gm = min(kFGroupM, tiles_m - g * kFGroupM);
    m = g * kFGroupM + idx % gm;
    n = idx / gm;
}

template <int K>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_prefill_kernel(const FusedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kFLds];
    __shared__ int s_pos[kFBM], s_len[kFBM], s_seq[kFBM];

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

    // Row -> (sequence, position, length) map of the tile, for the epilogue.
    {
        const int64_t t = row0 + tid;
        int pos = -1, len = 0, seq = 0;
        if (t >= 0 && t < T && a.N > 0) {
            int lo = 0, hi = a.N;                  // largest s in [0, N) with cu[s] <= t
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)a.cu[mid] <= t) lo = mid; else hi = mid;
            }
            seq = lo;
            const int64_t s0 = a.cu[lo], s1 = a.cu[lo + 1];
            if (t >= s0 && t < s1) { pos = (int)(t - s0); len = (int)(s1 - s0); }
        }
        s_pos[tid] = pos; s_len[tid] = len; s_seq[tid] = seq;
    }

    // Global -> LDS staging: thread tid moves 16-byte chunk (tid & 7) of rows
    // (tid >> 3) + 32 i: 8 x rows and 6 W_in rows per stage.
    const int lc = tid & 7, lr = tid >> 3;
    const int64_t vrow_lo = row0 < 0 ? 0 : row0;
    const int64_t vrow_hi = (row0 + kFBM < T) ? row0 + kFBM : T;
    const rsrc_t xr = row_rsrc(a.x + vrow_lo * a.x_stride,
                               (uint32_t)((vrow_hi > vrow_lo ? vrow_hi - vrow_lo : 0) * a.x_stride * 2));
    const rsrc_t wr = row_rsrc(a.W, (uint32_t)((int64_t)3 * H * a.D * 2));
    uint32_t xoff[8], woff[6];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t t = row0 + lr + 32 * i;
        xoff[i] = (t >= vrow_lo && t < vrow_hi) ? (uint32_t)((t - vrow_lo) * a.x_stride * 2) + lc * 16u : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int n = lr + 32 * i;                          // staged W_in row: part n / 64, channel n % 64
        const int64_t wrow = (int64_t)(n / kFNC) * H + n0 + (n % kFNC);
        woff[i] = (uint32_t)(wrow * a.D * 2) + lc * 16u;
    }
    const uint32_t sw_a = lds_chunk(lr, lc);   // same swizzle for every row lr + 32 i
    u32x4 ga[8], gb[6];
    auto gload = [&](int kt) {
        const uint32_t ko = (uint32_t)kt * kFRowBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) ga[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i] + ko, 0, 0);
#pragma unroll
        for (int i = 0; i < 6; ++i) gb[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[i] + ko, 0, 0);
    };
    auto lstore = [&](int buf) {
        uint8_t* base = smem + buf * kFStage;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4*>(base + sw_a + (uint32_t)(32 * i) * kFRowBytes) = ga[i];
#pragma unroll
        for (int i = 0; i < 6; ++i)
            *reinterpret_cast<u32x4*>(base + kFStageA + sw_a + (uint32_t)(32 * i) * kFRowBytes) = gb[i];
    };

    f32x16 acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = a.D / kFBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* sa = smem + cur * kFStage;
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
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // Accumulator register r of row tile i holds computed row
    // wm*128 + i*32 + 8*(r/4) + 4*hl + (r%4), channel n0 + wn*32 + q.
    float* bxs = reinterpret_cast<float*>(smem);   // [256][64] fp32
    const int lcn = wn * 32 + q;                   // channel within the tile
    const int ch = n0 + lcn;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            bxs[row * kFNC + lcn] = acc[i][0][r] * acc[i][2][r];
        }
    if (a.io != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                const int64_t t = row0 + row;
                if (row >= K - 1 && t < T) {
                    uint16_t* o = a.io + t * a.io_stride + ch;
                    o[0] = bf16_bits(acc[i][0][r]);
                    o[H] = bf16_bits(acc[i][1][r]);
                    o[2 * H] = bf16_bits(acc[i][2][r]);
                }
            }
    }
    __syncthreads();

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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const int64_t t = row0 + row;
            const int pos = s_pos[row];
            if (row < K - 1 || pos < 0) continue;      // overlap row, or not a token
            const int seq = s_seq[row];
            const float bx = acc[i][0][r] * acc[i][2][r];
            float conv = fmaf(wk[K - 1], bx, bv);
#pragma unroll
            for (int k = 0; k < K - 1; ++k) {
                const int d = K - 1 - k;                 // X[pos+1+k] is bx of the token d rows back
                const float h = pos >= d ? bxs[(row - d) * kFNC + lcn] : s0(seq, pos + 1 + k);
                conv = fmaf(wk[k], h, conv);
            }
            a.y[t * a.y_stride + ch] = bf16_bits(acc[i][1][r] * conv);
            const int len = s_len[row];
            if (a.fin != nullptr && pos == len - 1) {
                // final state X[len .. len+K-1]: bx of the last tokens, or initial-state entries
                uint16_t* f = a.fin + (int64_t)seq * H * K + (int64_t)ch * K;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const int idx = len + j;
                    f[j] = bf16_bits(idx >= K ? bxs[(row + 1 + j - K) * kFNC + lcn] : s0(seq, idx));
                }
            }
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
