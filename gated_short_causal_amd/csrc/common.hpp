// common.hpp -- shared device helpers for the ShortConv kernels (gfx950).
//
// Data layout used by every kernel:
//   * a lane owns 8 consecutive channels, so every bf16 operand row segment it
//     touches is one 16-byte access (fp32: two), and a 64-lane wave covers
//     512 contiguous channels = 1 KiB (bf16) per operand per token row;
//   * state entries of a lane's 8 channels are 8*K contiguous elements of the
//     channel-major [H][K] slot block (48 bytes for bf16, K = 3), so pool
//     traffic is already fully coalesced without any transpose;
//   * values are widened to fp32 in registers and rounded once (RNE) when
//     stored; gfx950 has a hardware packed fp32->bf16 RNE convert.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef LFM2SC_VERIFY_U
#define LFM2SC_VERIFY_U 1      // draft steps per verify wave (the steps of a sequence are split over waves)
#endif
#ifndef LFM2SC_ROUNDS
#define LFM2SC_ROUNDS 1        // ragged grids are sized to this many full rounds of resident workgroups
#endif
#ifndef LFM2SC_SUB_MIN
#define LFM2SC_SUB_MIN 8       // shortest per-wave token window
#endif
#ifndef LFM2SC_FWD_U
#define LFM2SC_FWD_U 4         // token rows of loads in flight per wave (forward, bf16 I/O)
#endif
#ifndef LFM2SC_FWD_U_F32
#define LFM2SC_FWD_U_F32 2     // same for fp32 I/O (twice the bytes per row)
#endif
#ifndef LFM2SC_FWD_TW
#define LFM2SC_FWD_TW 4        // forward workgroup: waves along time (4: 4 consecutive windows of one 512-channel
#endif                         // group; 1: one window across 4 x 512 channels)
#ifndef LFM2SC_BWD_TW
#define LFM2SC_BWD_TW 4        // same for the backward
#endif
#ifndef LFM2SC_FWD_LDS
#define LFM2SC_FWD_LDS 82944   // dynamic LDS bytes reserved per forward workgroup: more than half of a CU's
#endif                         // 160 KiB, so one workgroup (4 long row streams) runs per CU
#ifndef LFM2SC_BWD_LDS
#define LFM2SC_BWD_LDS 82944   // same for the backward (its static LDS stays within 160 KiB with it)
#endif
#ifndef LFM2SC_SHORT_T
#define LFM2SC_SHORT_T 0       // ragged calls with fewer tokens than this launch without the LDS reservation
#endif                         // (several workgroups per CU, shorter windows); 0 = never
#ifndef LFM2SC_BWD_U
#define LFM2SC_BWD_U 3         // token rows of loads in flight per wave (backward, bf16 I/O)
#endif
#ifndef LFM2SC_FWD_NT
#define LFM2SC_FWD_NT 1        // non-temporal hints on streamed rows, forward: 1 = loads, 2 = stores, 3 = both
#endif
#ifndef LFM2SC_DEC_NT
#define LFM2SC_DEC_NT 3        // non-temporal hints in decode (bits): 1 in_proj loads, 2 y stores, 4 state loads,
#endif                         // 8 state stores.  Measured at N=4096: 0 -> 38.6 us, 3 -> 32.2, 7 -> 40.2, 15 -> 50.1
#ifndef LFM2SC_VER_NT
#define LFM2SC_VER_NT 11       // same for verify: 1 in_proj loads, 2 y stores, 4 state loads, 8 tape stores.
#endif                         // Measured at 64 x 8: 0 -> 6.24 us, 2 -> 6.10, 10 -> 5.95, 11 -> 5.89
#ifndef LFM2SC_CVU_NT
#define LFM2SC_CVU_NT 3        // same for the interop conv update (vector layouts): 1 bx loads, 2 out stores,
#endif                         // 8 tape stores.  Measured at 64 x 8 (view / dense): 0 -> 6.25 / 6.56 us,
                               // 3 -> 5.83 / 6.02, 11 -> 6.48 / 6.00
#ifndef LFM2SC_BWD_NT
#define LFM2SC_BWD_NT 3        // same for the backward
#endif

namespace lfm2sc {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kChPerLane = 8;      // channels per lane
constexpr int kChPerWave = kWave * kChPerLane;   // 512
constexpr int kThreads = 256;      // 4 waves per workgroup
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSmallBlock = kWave;   // decode / verify / commit: one wave per workgroup, spread over every CU

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element traits
// uint16_t carries bf16 bit patterns; float is fp32.  Both expose 8-element
// vector access on 16-byte aligned addresses.
template <typename E> struct Elem;

template <> struct Elem<uint16_t> {
    static constexpr int kChunks = 1;   // 16-byte chunks per 8 elements
    __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
        f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
        f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
    }
    __device__ __forceinline__ static uint32_t pack2(float a, float b) {
        f32x2 f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    __device__ __forceinline__ static uint4 pack(const float* f) {
        uint4 v;
        v.x = pack2(f[0], f[1]); v.y = pack2(f[2], f[3]);
        v.z = pack2(f[4], f[5]); v.w = pack2(f[6], f[7]);
        return v;
    }
};

template <> struct Elem<float> {
    static constexpr int kChunks = 2;
    __device__ __forceinline__ static void unpack(const uint4* v, float* f) {
        f[0] = __uint_as_float(v[0].x); f[1] = __uint_as_float(v[0].y);
        f[2] = __uint_as_float(v[0].z); f[3] = __uint_as_float(v[0].w);
        f[4] = __uint_as_float(v[1].x); f[5] = __uint_as_float(v[1].y);
        f[6] = __uint_as_float(v[1].z); f[7] = __uint_as_float(v[1].w);
    }
};

// Raw 8-element register image (kept packed until used to save VGPRs).
template <typename E> struct Raw8 { uint4 c[Elem<E>::kChunks]; };

template <typename E>
__device__ __forceinline__ Raw8<E> ld8(const E* p) {
    Raw8<E> r;
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) r.c[i] = q[i];
    return r;
}

// Streamed rows (in_proj, dy, y, d_in): touched once, optionally hinted
// non-temporal so they do not evict reused data (halo rows, state, weights).
template <typename E, int NT>
__device__ __forceinline__ Raw8<E> ld8s(const E* p) {
    if constexpr ((NT & 1) != 0) {
    Raw8<E> r;
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 v = __builtin_nontemporal_load(q + i);
        r.c[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
    return r;
    } else {
        return ld8<E>(p);
    }
}

template <typename E>
__device__ __forceinline__ void st8(E* p, const Raw8<E>& r) {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) q[i] = r.c[i];
}

__device__ __forceinline__ void to_f32(const Raw8<uint16_t>& r, float* f) { Elem<uint16_t>::unpack(r.c[0], f); }
__device__ __forceinline__ void to_f32(const Raw8<float>& r, float* f) { Elem<float>::unpack(r.c, f); }

template <typename E> __device__ __forceinline__ Raw8<E> from_f32(const float* f);
template <> __device__ __forceinline__ Raw8<uint16_t> from_f32<uint16_t>(const float* f) {
    Raw8<uint16_t> r; r.c[0] = Elem<uint16_t>::pack(f); return r;
}
template <> __device__ __forceinline__ Raw8<float> from_f32<float>(const float* f) {
    Raw8<float> r;
    r.c[0] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    r.c[1] = make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7]));
    return r;
}

template <typename E, int NT>
__device__ __forceinline__ void st8s(E* p, const Raw8<E>& r) {
    if constexpr ((NT & 2) != 0) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 v = {r.c[i].x, r.c[i].y, r.c[i].z, r.c[i].w};
        __builtin_nontemporal_store(v, q + i);
    }
    } else {
        st8<E>(p, r);
    }
}

template <typename E> __device__ __forceinline__ void load_f32x8(const E* p, float* f) { to_f32(ld8<E>(p), f); }
template <typename E> __device__ __forceinline__ void store_f32x8(E* p, const float* f) { st8<E>(p, from_f32<E>(f)); }
template <typename E, int NT>
__device__ __forceinline__ void store_f32x8s(E* p, const float* f) { st8s<E, NT>(p, from_f32<E>(f)); }

// 8*K contiguous elements (a lane's state block) <-> float s[8][K].
template <typename E, int K>
__device__ __forceinline__ void load_block(const E* p, float (&s)[kChPerLane][K]) {
    float f[8 * K];
#pragma unroll
    for (int j = 0; j < K; ++j) load_f32x8<E>(p + 8 * j, f + 8 * j);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) s[c][k] = f[c * K + k];
}

// The same with non-temporal hints (NT bit 1: loads, bit 2: stores, as ld8s / st8s).
template <typename E, int K, int NT>
__device__ __forceinline__ void load_block_s(const E* p, float (&s)[kChPerLane][K]) {
    float f[8 * K];
#pragma unroll
    for (int j = 0; j < K; ++j) to_f32(ld8s<E, NT>(p + 8 * j), f + 8 * j);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) s[c][k] = f[c * K + k];
}

template <typename E, int K, int NT>
__device__ __forceinline__ void store_block_s(E* p, const float (&s)[kChPerLane][K]) {
    float f[8 * K];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) f[c * K + k] = s[c][k];
#pragma unroll
    for (int j = 0; j < K; ++j) st8s<E, NT>(p + 8 * j, from_f32<E>(f + 8 * j));
}

template <typename E, int K>
__device__ __forceinline__ void store_block(E* p, const float (&s)[kChPerLane][K]) {
    float f[8 * K];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) f[c * K + k] = s[c][k];
#pragma unroll
    for (int j = 0; j < K; ++j) store_f32x8<E>(p + 8 * j, f + 8 * j);
}

// Wave index inside the workgroup, as a wave-uniform (scalar) value so that
// everything derived from it -- window bounds, row offsets, loop counts --
// stays in SGPRs and addresses become scalar base + per-lane offset.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// ---------------------------------------------------------------- buffer access to streamed rows
// A streamed row (in_proj, dy, y, d_in) is addressed through a raw buffer
// descriptor built on the (wave-uniform) row start, with num_records = the
// row's width in bytes, plus a 32-bit per-lane byte offset.  The descriptor
// lives in SGPRs, so a load costs no VGPRs for its address, and the hardware
// range check turns any access past the row into a zero read / dropped write.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;   // gfx9-family raw (untyped) buffer

__device__ __forceinline__ rsrc_t row_rsrc(const void* row, uint32_t row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, (int)row_bytes, kRawBufferWord3);
}

template <typename E, int NT>
__device__ __forceinline__ Raw8<E> bld8(rsrc_t r, uint32_t voff) {
    Raw8<E> out;
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16u * i, 0, (NT & 1) ? 2 : 0);
        out.c[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
    return out;
}

template <typename E, int NT>
__device__ __forceinline__ void bst8(rsrc_t r, uint32_t voff, const Raw8<E>& v) {
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 w = {v.c[i].x, v.c[i].y, v.c[i].z, v.c[i].w};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, voff + 16u * i, 0, (NT & 2) ? 2 : 0);
    }
}

template <typename E, int NT>
__device__ __forceinline__ void bst8f(rsrc_t r, uint32_t voff, const float* f) { bst8<E, NT>(r, voff, from_f32<E>(f)); }

// ---------------------------------------------------------------- XCD-aware block order
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Remap so that XCD x receives a contiguous run of tiles:
// neighbouring tiles share halo rows, which then hit in that XCD's L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
    const int per = nblocks / kXcds;          // host pads nblocks to a multiple of 8
    return (bid % kXcds) * per + bid / kXcds;
}
inline int pad_xcd(int n) { return (n + kXcds - 1) / kXcds * kXcds; }

// ---------------------------------------------------------------- ragged tiling
// Packed sequences are laid on a virtual axis on which sequence i occupies
// [cu[i] + i*gap, cu[i+1] + i*gap): consecutive sequences are separated by
// `gap` empty positions, so any window of at most `gap` positions meets at
// most one sequence.  Fixed-size windows of that axis are the work units.  The
// last sequence ends at most at total_T + (N-1)*gap, so ceil(total_T / gap) +
// N - 1 windows of `gap` positions cover every sequence; that count is known
// on the host without reading cu_seqlens.  Row offsets are clamped to
// [0, total_T], so a malformed cu_seqlens can produce wrong results but never
// an out-of-bounds access.
struct SeqSpan {
    int seq;        // sequence index
    int64_t r0;     // first packed row of the sequence
    int64_t T;      // sequence length
    int64_t lo, hi; // the window's part of the sequence, in sequence-local tokens
};

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t a, int64_t b) { return v < a ? a : (v > b ? b : v); }

// The sequence a window [v0, v1) meets: the last i with vstart(i) <= v1 - 1.
// Fewer than 64 sequences: every lane loads one row offset (one memory round
// trip for the whole search, instead of one per step of a binary search over
// scalar loads), a ballot finds i and readlane brings its offsets back to
// scalar registers.  Call it with every lane of the wave active.  More
// sequences: binary search.  Both give the same i for valid offsets; for
// invalid ones any i may result, and the clamps still keep every row in
// [0, total_T].
__device__ __forceinline__ bool find_span(const int32_t* __restrict__ cu, int N, int64_t total_T, int64_t gap,
                                          int64_t v0, int64_t v1, SeqSpan& s) {
    if (N < kWave) {
        const int lane = (int)(threadIdx.x % kWave);
        const int c = lane <= N ? (int)clamp64(cu[lane], 0, total_T) : (int)total_T;
        const bool cand = lane < N && (int64_t)c + (int64_t)lane * gap <= v1 - 1;
        const uint64_t m = __ballot(cand);
        if (m == 0) return false;
        const int i = 63 - __builtin_clzll(m);
        const int64_t r0 = __builtin_amdgcn_readlane(c, i);
        const int64_t r1 = clamp64(__builtin_amdgcn_readlane(c, i + 1), r0, total_T);
        const int64_t vs = r0 + (int64_t)i * gap;
        s.seq = i; s.r0 = r0; s.T = r1 - r0;
        s.lo = v0 - vs > 0 ? v0 - vs : 0;
        s.hi = v1 - vs < s.T ? v1 - vs : s.T;
        return s.hi > s.lo;
    }
    int a = 0, b = N - 1, ans = -1;
    while (a <= b) {
        const int mid = (a + b) >> 1;
        const int64_t vs = clamp64(cu[mid], 0, total_T) + (int64_t)mid * gap;
        if (vs <= v1 - 1) { ans = mid; a = mid + 1; } else { b = mid - 1; }
    }
    if (ans < 0) return false;
    const int64_t r0 = clamp64(cu[ans], 0, total_T);
    const int64_t r1 = clamp64(cu[ans + 1], r0, total_T);
    const int64_t vs = r0 + (int64_t)ans * gap;
    s.seq = ans; s.r0 = r0; s.T = r1 - r0;
    s.lo = v0 - vs > 0 ? v0 - vs : 0;
    s.hi = v1 - vs < s.T ? v1 - vs : s.T;
    return s.hi > s.lo;
}

__device__ __forceinline__ bool slot_ok(int64_t slot, int64_t num_slots) { return slot >= 0 && slot < num_slots; }

// Window length for a ragged launch.  Every window of `kWavesPerBlock * sub`
// virtual positions is one workgroup per channel group; the grid holds
// ceil(total_T / gap) + N windows per group.  The windows are sized so that
// the whole grid is LFM2SC_ROUNDS full rounds of the workgroups the device
// keeps resident (`resident`, from the occupancy of the kernel): a partial
// last round would leave most CUs idle while it drains.
struct Tiling { int sub; int64_t ntiles; };

// A workgroup is TW waves along time (consecutive windows of `sub` tokens) by
// kWavesPerBlock / TW waves along channels (512 channels each).
template <int TW>
struct WgLayout {
    static_assert(TW == 1 || TW == 2 || TW == 4, "waves along time must divide the workgroup");
    static constexpr int kCW = kWavesPerBlock / TW;
    static constexpr int kChPerBlock = kCW * kChPerWave;
    static int groups(int H) { return (H + kChPerBlock - 1) / kChPerBlock; }
};

// Window slots are counted per XCD: the launch pads the window count to a
// multiple of 8 and each XCD runs `groups` workgroups for each of its windows,
// so a chip-wide count (e.g. 85 windows x 3 groups = 255 <= 256) can still put
// 33 workgroups on an XCD of 32 CUs and push one into a second round.
// Window length and HBM conflicts.  All windows of a launch stream at once,
// their rows a fixed `sub` apart, so the HBM channels and banks that serve
// them at any moment follow from the spacing sub * row_bytes: at some
// spacings many windows land on the same ones and the kernels slow down by up
// to 25% (measured on MI355X with every base alignment of the buffers tried:
// the effect follows the spacing, not the addresses).  kWinRate holds the
// backward kernel's measured rate for bf16 rows of H = 2048 (4 KiB rows of
// dy and y, 12 KiB of in_proj and d_in) at one full round of windows, for
// window lengths kWinLo .. kWinHi-1: (TB/s - 4.0) * 100, median of three
// sweeps.  For that row geometry a launch takes, among the window lengths from
// the shortest that fits one round to 1/span above it, the one with the best
// measured rate.  A longer window leaves some CUs idle: the backward, bound by
// HBM, hardly notices (at 40 of 64 windows per channel group it still runs at
// 95% of the full round's rate) and searches 1/8 above; the forward loses
// ~0.6% per idle window and searches 1/64 above.  Other row geometries take
// the shortest window.
constexpr int kWinLo = 64;
constexpr int kWinHi = 1024;
constexpr unsigned char kWinRate[kWinHi - kWinLo] = {
     82, 100,  93,  86,  99,  93,  92,  96, 101,  97,  93,  85,  93,  98, 104, 100, 103,  95, 108, 103,
    114, 104,   0, 115, 116, 117, 109, 114, 108, 102, 106,  55,  95, 102, 108, 101,  82, 108, 103, 109,
    109, 115,  74, 108,  85,  89,  41, 111, 116, 108, 111, 113, 109,  96,  94,  77, 109, 103, 109, 102,
    115,  76,  96,  23,  87,  15, 108,  91, 110, 105, 103,  91, 119, 121, 100,  91, 115,  97, 113, 115,
    114, 104, 114, 115,  97,  99,  90,  67, 111,  20, 118,  67, 126, 101, 128, 125, 119, 133, 111, 136,
    135,  89,  99, 121, 135, 118, 113, 126,  66, 120, 123, 117, 120, 124, 133, 130, 134, 134, 137, 124,
    128, 126, 124, 109, 123, 125,  66, 110, 102,  12, 109, 117, 113,   0, 101, 107,  94, 105, 122, 128,
    120, 121, 113, 120, 118,  92, 114,  89,  60, 101, 102,  63,  99,  92, 109, 107,  90, 106, 121, 109,
    126, 116,  71, 112, 118,  78, 119, 123, 110, 112, 116, 108,  99, 115, 114, 119, 126, 121, 125, 118,
    112, 127, 119, 111, 129, 122, 111, 116, 116, 111,  78, 105, 101, 104,  65, 111, 120, 120, 111, 123,
    124, 118, 108, 125, 124, 121,  95, 105, 125, 135, 123,  96,  99, 114, 118, 116, 117, 119, 115, 119,
    123, 108, 123, 126, 118, 125,  70, 120, 116, 100, 108,  68,  78,  76,  86,  75,  87,  34,  81, 105,
    114, 116,  75, 120, 125, 122, 101, 118, 119, 119, 104, 118, 122, 122, 120, 124, 111, 132, 121, 124,
    113, 116, 128, 124, 129, 120, 108, 134, 111, 121, 120, 128, 127, 121, 103,  92, 117, 115, 113, 115,
     86, 112, 121, 129, 125, 127, 121, 132, 118, 115, 116, 119, 123, 122, 112, 117, 111, 123, 133, 124,
    133, 124, 123, 117, 130, 123, 121, 126, 127, 123, 126, 122, 124, 118, 121, 114,  89,  78,  80,  95,
     99,  79,  68,  14,  80, 112, 129, 125, 112,  81,  54, 119, 126, 127, 130, 130, 123, 112, 110, 128,
    128, 129, 134, 137, 127, 127, 130, 123, 111, 122, 130, 120, 128, 119, 111, 124, 132, 124, 115, 103,
    111, 127, 126, 124, 125, 121,  98, 113, 127, 124, 124, 122, 125, 129, 125, 125, 115, 124, 130, 126,
    125, 112, 107, 121, 135, 126, 126,  92,  50,  98, 118, 145, 134, 118,  61,  79, 123, 125, 131, 126,
    109,  94,  86, 119, 111, 120, 118, 106, 112,  94, 114, 128, 122, 130, 128, 121, 124, 129, 113,  96,
    106, 112, 125, 120, 117, 132, 127, 130, 110, 120, 119, 115, 126, 127, 123, 126, 120, 128, 126, 128,
    137, 132, 130, 123,  99, 118, 133, 134, 136, 133, 131, 122,  96, 120, 133, 135, 136, 131, 130, 128,
    123, 128, 122, 105, 119, 120, 122, 126, 129, 121, 124, 110, 107, 123, 120, 102, 116, 119, 107, 128,
    131, 133, 139, 134, 130, 124,  83, 102, 114, 117, 124, 133, 124, 130, 118,  99, 110, 123, 122, 127,
    133, 130, 130, 132, 130, 113, 119, 126, 134, 133, 136, 135, 127, 122, 121, 101,  54,  96, 125, 123,
    128, 132, 121, 116, 123, 100,  58,  66,  90,  74, 107, 111, 116, 119, 117, 114, 103,  97,  73,  72,
    103, 101, 128, 134, 118, 131, 121,  78, 105, 115, 129, 128, 135, 130, 124, 121, 122, 126, 128, 131,
    120, 127, 130, 124, 125, 126, 128, 130, 132, 123, 122, 113, 119, 132, 131, 132, 120, 128, 134, 130,
    108, 103, 120, 122, 117, 129, 124, 120, 130, 133, 129, 124, 128, 126, 122, 127, 121, 130, 134, 126,
    123, 125, 127, 127, 125, 129, 137, 134, 144, 141, 129, 123, 110,  51,  95, 124, 135, 131, 147, 139,
    135, 139, 126,  95,  64,  97, 108, 129, 129, 136, 138, 137, 130, 127, 121, 125, 125, 127, 130, 128,
    130, 122, 124, 119, 127, 125, 126, 129, 130, 126, 126, 115, 124, 133, 121, 120, 100, 130, 126, 133,
    135, 128, 131, 134, 135, 129, 115, 108, 113, 128, 124, 133, 134, 136, 128, 126, 133, 126, 129, 127,
    126, 132, 129, 133, 131, 124, 125, 125, 122,  89, 108, 120, 121, 132, 125, 117, 112,  92,  89,  87,
     78,  89,  94, 110, 128, 118, 102,  96,  99,  53,  50,  80,  97, 125, 125, 134, 141, 136, 132, 127,
    126, 118, 106,  80,  99, 128, 124, 129, 134, 134, 133, 130, 129, 126, 128, 127, 129, 117, 125, 122,
    105, 116, 127, 131, 127, 126, 124, 131, 125, 128, 134, 131, 122, 115, 119, 129, 128, 126, 132, 131,
    118, 112, 113, 123, 117,  89, 112, 129, 131, 128, 123, 133, 122, 125, 122, 122, 120, 119, 123, 126,
    124, 129, 124, 108, 127, 130, 135, 134, 132, 128, 131, 135, 132, 133, 131, 122, 116, 122, 129, 129,
    127, 129, 128, 126, 112, 118, 117, 114, 118, 130, 126, 125, 127, 131, 128, 126, 119, 122, 126, 121,
    122, 107, 112, 123, 113, 111, 116, 121, 118, 113, 126, 130, 131, 130, 125, 132, 129, 120,  94,  88,
     86, 104, 111, 131, 135, 135, 139, 138, 138, 134, 127, 118,  88,  69, 102, 119, 131, 130, 128, 135,
    134, 132, 128, 131, 122, 114, 115,  92, 110, 122, 123, 119, 120, 125, 128, 129, 125, 118, 121, 121,
    125, 120, 113, 117, 121, 126, 127, 127, 126, 126, 133, 135, 134, 129, 124, 129, 125, 131, 130, 117,
    116, 115,  79,  68,  94, 110, 112, 125, 122, 121, 112, 113, 121, 128, 127, 123, 114, 124, 117, 106,
    104,  96, 111, 110, 113, 109, 115, 116, 124, 120, 127, 122, 123, 128, 132, 123, 125, 120, 126, 128,
    127, 129, 128, 130, 133, 133, 127, 127, 128, 132, 132, 125, 112, 115, 124, 134, 133, 131, 129, 128,
};

constexpr int kWinSpanBwd = 8;
constexpr int kWinSpanFwd = 64;

inline int64_t pick_window(int64_t sub0, int64_t row_bytes, int span) {
    if (row_bytes != 4096 || sub0 < kWinLo || sub0 >= kWinHi || span < 1) return sub0;
    const int64_t last = sub0 + (sub0 + span - 1) / span;
    int64_t best = sub0;
    for (int64_t s = sub0 + 1; s <= last && s < kWinHi; ++s)
        if (kWinRate[s - kWinLo] > kWinRate[best - kWinLo]) best = s;
    return best;
}

// The N-1 gaps between sequences take N-1 of the window slots (one sequence,
// the training step, uses every slot: all CUs of the round get work).
// row_bytes = H * element size (the dy / y row); span: see pick_window.
inline Tiling ragged_tiling(int64_t total_T, int N, int groups, int resident, int tw, int64_t row_bytes, int span) {
    const int64_t g = groups > 0 ? groups : 1;
    const int64_t gaps = N > 1 ? N - 1 : 0;
    const int64_t per_xcd = (int64_t)resident * LFM2SC_ROUNDS / kXcds / g;
    const int64_t slots = (per_xcd > 0 ? per_xcd : 1) * kXcds;
    const int64_t free = slots - gaps;
    const int64_t denom = (int64_t)tw * (free >= 1 ? free : (slots > 0 ? slots : 1));
    int64_t sub = (total_T + denom - 1) / denom;
    if (sub < LFM2SC_SUB_MIN) sub = LFM2SC_SUB_MIN;
    if (sub > (1 << 24)) sub = 1 << 24;
    sub = pick_window(sub, row_bytes, span);

    const int64_t gap = sub * tw;
    return Tiling{(int)sub, (total_T + gap - 1) / gap + gaps};
}

// Workgroups of `kernel` (kThreads wide, no dynamic LDS) resident on the
// current device at once; a conservative default if the query fails.
template <typename KernelT>
inline int resident_workgroups(KernelT kernel, size_t dyn_lds = 0) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, dyn_lds) != hipSuccess || cus <= 0 ||
        per <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return cus * per;
}

}  // namespace lfm2sc
