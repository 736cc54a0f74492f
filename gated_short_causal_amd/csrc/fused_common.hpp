// fused_common.hpp -- pieces shared by the fused in_proj + ShortConv kernels
// (fused.hip: the 4-wave and wide tiles; fused_split.hip: the split tiles):
// bf16 helpers, wait counts and barriers, the tile order, the geometry of
// staged rows; and the host entry points of the split tiles.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lfm2sc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kFBM = 256;              // token rows computed per tile

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    f32x2 v = {f, 0.f};
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)) & 0xffffu);
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// s_waitcnt that waits until at most n vector-memory operations are outstanding
// (expcnt and lgkmcnt left unconstrained).
template <int n> __device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier between reduction stages without __syncthreads' release
// fence: that fence waits for every outstanding vector-memory operation, i.e.
// for the loads of the stages still in flight, which would drain the ring at
// every stage.  It is not needed here: before the barrier each wave has waited
// (wait_vm) for its own loads of the stage about to be read, and its LDS reads
// of the slot about to be refilled were consumed by its MFMAs.  The empty asm
// statements keep the compiler from moving memory accesses across it.
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

template <int v> using IC = std::integral_constant<int, v>;

constexpr int kWNC = 128;                          // channels per wide tile

// Stage geometry for a reduction depth of BK per stage.  One global->LDS
// instruction moves 64 lanes x 16 B = 1 KiB = kRowsPerDma staged rows.  The
// swizzle places the 16-byte chunks of consecutive rows so that the 16 lanes
// of a ds_read_b128 quarter (16 consecutive rows, one chunk) hit all 64 banks
// once: rows 4 apart (64-byte rows) or 2 apart (128-byte rows) rotate the
// chunk position.
template <int BK>
struct WideStage {
    static_assert(BK == 32 || BK == 64, "32- or 64-deep stages");
    static constexpr int kRowB = 2 * BK;                        // one staged row: BK bf16
    static constexpr int kChunks = kRowB / 16;
    static constexpr int kRowsPerDma = 1024 / kRowB;
    static constexpr int kDmaA = kFBM / kRowsPerDma / 8;        // x blocks per wave per stage
    static constexpr int kDmaB = 3 * kWNC / kRowsPerDma / 8;    // W_in blocks per wave per stage
    static constexpr int kVm = kDmaA + kDmaB;
    static constexpr int kStageA = kFBM * kRowB;
    static constexpr int kStageB = 3 * kWNC * kRowB;
    static constexpr int kMfma = BK / 16 * 12;                  // MFMAs per wave per stage
    __device__ static int rot(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
    __device__ static uint32_t chunk(int r, int c) { return (uint32_t)r * kRowB + (uint32_t)((c ^ rot(r)) << 4); }
    // global byte offset, within its staged row r, of the chunk that lane `lane` writes
    __device__ static uint32_t dma_chunk(int lane, int r) { return (uint32_t)(((lane % kChunks) ^ rot(r)) << 4); }
};

template <int KT, int NK, typename F>
__device__ __forceinline__ void unroll_stages(F& f) {
    if constexpr (KT < NK) {
        f(IC<KT>{});
        unroll_stages<KT + 1, NK>(f);
    }
}

// Row map of a tile, built before any load of its reduction (waiting on a
// vector load would also wait on every load issued before it).  The sequence
// of the tile's first row comes from a wave-uniform (scalar) search; when that
// sequence covers every row of the tile, each row's entry is arithmetic,
// otherwise each row searches cu_seqlens itself.
// Sequence of the first token row of a tile (wave-uniform search of cu_seqlens).
struct TileSeq {
    int lo;
    int64_t c0, c1;
    int slot_lo;
};
__device__ __forceinline__ TileSeq tile_first_seq(const FusedArgs& a, int64_t row0) {
    const int64_t tf = row0 < 0 ? 0 : row0;
    int lo = 0, hi = a.N;                          // largest s in [0, N) with cu[s] <= tf
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)a.cu[mid] <= tf) lo = mid; else hi = mid;
    }
    return TileSeq{lo, a.cu[lo], a.cu[lo + 1], a.pool != nullptr ? a.slot_idx[lo] : -1};
}

// Row r of a tile of `rows` rows from token row0: position in its sequence (-1
// outside every sequence), length, sequence, slot (-1 without a pool or out of
// range).  Arithmetic when the first row's sequence covers the tile, else a
// per-row search.
__device__ __forceinline__ void tile_row(const FusedArgs& a, const TileSeq& f, int64_t row0, int rows, int r,
                                         int& pos, int& len, int& seq, int& sid) {
    const int64_t tf = row0 < 0 ? 0 : row0;
    const int64_t t = row0 + r;
    pos = -1; len = 0; seq = f.lo;
    if (f.c0 <= tf && f.c1 >= row0 + rows) {
        if (t >= tf) { pos = (int)(t - f.c0); len = (int)(f.c1 - f.c0); }
    } else if (t >= 0 && t < a.total_T) {
        int l2 = 0, h2 = a.N;
        while (h2 - l2 > 1) {
            const int mid = (l2 + h2) >> 1;
            if ((int64_t)a.cu[mid] <= t) l2 = mid; else h2 = mid;
        }
        seq = l2;
        const int64_t s0 = a.cu[l2], s1 = a.cu[l2 + 1];
        if (t >= s0 && t < s1) { pos = (int)(t - s0); len = (int)(s1 - s0); }
    }
    sid = -1;
    if (a.pool != nullptr && pos >= 0) {
        const int64_t v = seq == f.lo ? f.slot_lo : a.slot_idx[seq];
        sid = slot_ok(v, a.num_slots) ? (int)v : -1;
    }
}

// Split tiles (fused_split.hip), for D in {1024, 1536, 2048}.
// fused_split_choice: 32 or 64 (split tiles of 64 rows and that many channels)
// or 128 (mid tiles: 128 rows x 64 channels) when that form's expected span is
// shorter than `other`, the span of the other tile forms in rounds of wide
// overlapping tiles; 0 otherwise.  LFM2SC_FUSED_SPLIT in the environment
// overrides it: 0 never, 1 always (the best of the three), 32, 64 or 128 always
// that form.
int fused_split_choice(int64_t total_T, int H, double other);
// Sets the tile counts and launches the split-tile (nc = 32, 64) or mid-tile
// (nc = 128) kernel.
hipError_t launch_fused_split(FusedArgs a, int K, int nc, hipStream_t s);
// The tiling lfm2sc_fused_prefill takes (fused.hip): 1 wide tiles, 2 wide tiles
// with halo rows, 3 the 4-wave tile, 32 / 64 split tiles, 128 mid tiles.
int fused_plan(int K, int64_t total_T, int H, int D);

}  // namespace lfm2sc
