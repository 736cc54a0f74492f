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
#ifndef LFM2SC_FWD_TW_RAGGED
#define LFM2SC_FWD_TW_RAGGED 1 // the same for forward calls of more than one sequence
#endif
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
#ifndef LFM2SC_WIN_TABLES
#define LFM2SC_WIN_TABLES 1    // 1: window lengths from the measured rate tables below; 0: always the shortest
#endif                         // window that fits one round (the setting those tables are measured with)
#ifndef LFM2SC_BWD_U
#define LFM2SC_BWD_U 3         // token rows of loads in flight per wave (backward, bf16 I/O)
#endif
#ifndef LFM2SC_FWD_NT
#define LFM2SC_FWD_NT 1        // non-temporal hints on streamed rows, forward: 1 = loads, 2 = stores, 3 = both
#endif
#ifndef LFM2SC_DEC_NT
#define LFM2SC_DEC_NT 3        // non-temporal hints in decode (bits): 1 in_proj loads, 2 y stores, 4 state loads,
#endif                         // 8 state stores.  Measured at N=4096: 0 -> 38.6 us, 3 -> 32.2, 7 -> 40.2, 15 -> 50.1
#ifndef LFM2SC_DEC_STAGE_N
#define LFM2SC_DEC_STAGE_N 512   // decode calls of at least this many sequences stage the slot states through LDS.
#endif                           // Per call by graph replay, lane-owned / staged: N=256 4.14 / 4.17 us, 512 6.01 /
                                 // 5.78, 1024 10.2 / 9.3, 2048 17.9 / 16.0, 4096 32.4 / 29.9
#ifndef LFM2SC_VER_STAGE
#define LFM2SC_VER_STAGE 1       // 1: verify writes each step's tape row through LDS, 1 KiB per store instruction
#endif                           // (64 x 8 draft tokens: 5.89 us per call with one lane per block, 4.55 staged)
#ifndef LFM2SC_CVU_STAGE
#define LFM2SC_CVU_STAGE 1       // 1: the tape-mode conv update writes its tape blocks through LDS, as verify
#endif                           // (64 x 8 on the transposed view: 5.85 us per call lane-owned, 4.99 staged)
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

// Cache-policy operands of the buffer loads and stores (gfx950: bit 0 sc0,
// bit 1 nt, bit 4 sc1).  Streamed loads take nt.  bf16 stores take sc1
// (system scope, i.e. written through), with nt where the NT knob asks for
// it.  Measured on MI355X (median of 3-4 runs each): the backward's d_in
// stores as nt sc1 take the T=65536 step from 533.8 to 530.3 us (nt alone is
// the former; sc1 alone 577 us); then the forward's y stores as sc1 take it to
// 525.8 us (forward 175.1 -> 168.5 us; nt sc1 196 us, sc0 sc1 the same as
// sc1), the T=4096 step from 43.9 to 42.5 us and the ragged prefill from 28.3
// to 27.8 us.  Written through, a store must cover whole cache lines: with
// fp32 I/O a lane holds two 16-byte chunks, so each store instruction of a
// wave covers every other 16 bytes of its 2 KiB, and sc1 made the fp32 step
// 2x slower (1.24 -> 2.55 ms at H=2048).  fp32 stores keep nt only.
constexpr int kPolicyNt = 2;
constexpr int kPolicySc1 = 16;
template <typename E>
constexpr int store_policy(bool nt) {
    return (nt ? kPolicyNt : 0) | (Elem<E>::kChunks == 1 ? kPolicySc1 : 0);
}

template <typename E, int NT>
__device__ __forceinline__ Raw8<E> bld8(rsrc_t r, uint32_t voff) {
    Raw8<E> out;
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 v =
            __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16u * i, 0, (NT & 1) ? kPolicyNt : 0);
        out.c[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
    return out;
}

template <typename E, int NT>
__device__ __forceinline__ void bst8(rsrc_t r, uint32_t voff, const Raw8<E>& v) {
#pragma unroll
    for (int i = 0; i < Elem<E>::kChunks; ++i) {
        const u32x4 w = {v.c[i].x, v.c[i].y, v.c[i].z, v.c[i].w};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, voff + 16u * i, 0, store_policy<E>((NT & 2) != 0));
    }
}

template <typename E, int NT>
__device__ __forceinline__ void bst8f(rsrc_t r, uint32_t voff, const float* f) { bst8<E, NT>(r, voff, from_f32<E>(f)); }

// A wave's slot-state block (its 512 channels x K, contiguous in the slot)
// moved between memory and the lanes through LDS.  A lane owns 8 channels x K
// taps, 16*K contiguous bytes (bf16), so when each lane loads its own block
// one load instruction of the wave touches every cache line of the wave's
// block at a 16*K-byte stride, and the K instructions each touch them all.
// Staged, instruction j moves the contiguous 1 KiB j of the block, and the
// lanes exchange their pieces through LDS.  For decode batches this cut the
// call at N=4096 from 32.4 to 29.9 us; it costs two barriers and an LDS round
// trip, which small batches (N=256: 4.14 vs 4.17 us) do not earn back.
template <typename E, int K>
struct StateStage {
    static constexpr int kCpl = K * Elem<E>::kChunks;   // 16-byte chunks per lane
    uint4 buf[kCpl * kWave];
};

template <typename E, int K>
__device__ __forceinline__ void stage_load(StateStage<E, K>& st, rsrc_t blk, int lane, float (&s)[kChPerLane][K]) {
    constexpr int C = StateStage<E, K>::kCpl;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(blk, (uint32_t)(j * kWave + lane) * 16u, 0, 0);
        st.buf[j * kWave + lane] = make_uint4(v.x, v.y, v.z, v.w);
    }
    __syncthreads();
    float f[8 * K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        Raw8<E> r;
#pragma unroll
        for (int q = 0; q < Elem<E>::kChunks; ++q) r.c[q] = st.buf[lane * C + j * Elem<E>::kChunks + q];
        to_f32(r, f + 8 * j);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) s[c][k] = f[c * K + k];
}

template <typename E, int K, int POLICY = 0>
__device__ __forceinline__ void stage_store(StateStage<E, K>& st, rsrc_t blk, int lane,
                                            const float (&s)[kChPerLane][K]) {
    constexpr int C = StateStage<E, K>::kCpl;
    float f[8 * K];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k) f[c * K + k] = s[c][k];
    __syncthreads();   // every lane has read its chunks of the load stage
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const Raw8<E> r = from_f32<E>(f + 8 * j);
#pragma unroll
        for (int q = 0; q < Elem<E>::kChunks; ++q) st.buf[lane * C + j * Elem<E>::kChunks + q] = r.c[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const uint4 v = st.buf[j * kWave + lane];
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(w, blk, (uint32_t)(j * kWave + lane) * 16u, 0, POLICY);
    }
    __syncthreads();   // the buffer is free for the next item
}


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
// to 30% (measured on MI355X with every base alignment of the buffers tried:
// the effect follows the spacing, not the addresses).  The tables below hold
// the backward kernel's measured rate at one full round of windows, for
// window lengths kWinLo .. kWinHi-1 and three row geometries (row_bytes is the
// dy / y row; in_proj and d_in rows are three times as long): (TB/s - 3.0) *
// 100, median of three sweeps.  For a measured geometry a launch takes, among
// the window lengths from the shortest that fits one round to 1/span above
// it, the one with the best rate.  A longer window leaves some CUs idle: the
// backward, bound by HBM, hardly notices (at 40 of 64 windows per channel
// group it still runs at 95% of the full round's rate) and searches 1/8
// above; the forward loses ~0.6% per idle window and searches 1/64 above (its
// conflicts fall at the same spacings).  Other geometries take the shortest
// window; so do 8 KiB rows (H = 2048, fp32), where the table's picks gained
// under 1% in the backward at T = 65536 and lost as much in the forward.
constexpr int kWinLo = 64;
constexpr int kWinHi = 1024;
// H = 1024, 2-byte elements: 2 KiB rows, 2 channel groups
constexpr unsigned char kWinRate2K[kWinHi - kWinLo] = {
    154, 181, 172, 173, 197, 177, 187, 186, 185, 180, 182, 177, 186, 180, 188, 186, 187, 183, 189, 203,
    199, 193,  41, 202, 202, 199, 192, 196, 191, 191, 185, 183, 189, 192, 194, 186, 172, 194, 183, 194,
    193, 197, 196, 198, 159, 162,  94, 203, 212, 203, 213, 212, 207, 176, 176, 152, 191, 194, 194, 184,
    200, 174, 187, 158, 174, 144, 203, 181, 194, 173, 184, 193, 204, 207, 194, 156, 199, 189, 199, 198,
    204, 180, 199, 200, 195, 197, 191, 198, 203, 148, 195, 165, 206, 187, 205, 196, 199, 214, 204, 214,
    209, 182, 196, 194, 222, 216, 208, 224, 130, 215, 221, 207, 214, 203, 212, 209, 210, 213, 215, 205,
    211, 209, 195, 189, 201, 207, 171, 197, 192, 163, 195, 209, 208, 134, 197, 182, 195, 174, 207, 211,
    203, 208, 207, 205, 205, 154, 212, 171, 173, 202, 207, 188, 198, 164, 185, 175, 142, 175, 204, 204,
    212, 202, 199, 199, 209, 204, 210, 209, 202, 207, 188, 195, 189, 193, 175, 191, 206, 191, 206, 210,
    205, 209, 195, 190, 216, 212, 173, 207, 203, 200, 130, 197, 186, 204, 128, 205, 212, 209, 187, 208,
    212, 207, 198, 205, 205, 208, 196, 187, 212, 219, 212, 189, 203, 200, 183, 198, 206, 200, 190, 197,
    208, 197, 210, 209, 208, 214, 205, 215, 200, 185, 209, 198, 198, 176, 192, 195, 193, 111, 196, 209,
    214, 199, 133, 200, 209, 206, 172, 212, 214, 213, 197, 210, 218, 219, 212, 202, 199, 220, 218, 221,
    208, 193, 222, 207, 219, 209, 182, 230, 192, 200, 198, 217, 225, 215, 206, 181, 225, 233, 232, 227,
    179, 213, 219, 232, 217, 222, 215, 222, 198, 188, 213, 200, 222, 207, 210, 191, 219, 200, 222, 219,
    223, 221, 210, 192, 220, 206, 213, 212, 205, 205, 197, 211, 209, 216, 211, 191, 175, 184, 197, 202,
    201, 183, 160,  82, 195, 205, 214, 210, 198, 153, 103, 181, 195, 194, 199, 203, 197, 184, 195, 208,
    215, 215, 218, 218, 206, 197, 212, 216, 204, 215, 206, 214, 209, 189, 189, 211, 216, 211, 188, 175,
    176, 208, 209, 213, 209, 205, 156, 187, 209, 202, 203, 203, 204, 215, 201, 210, 180, 199, 198, 193,
    210, 202, 196, 209, 209, 205, 200, 187, 169, 191, 206, 216, 215, 206, 173, 173, 214, 212, 209, 211,
    194, 195, 198, 209, 204, 189, 196, 185, 204, 196, 199, 214, 199, 211, 207, 189, 210, 208, 208, 205,
    209, 214, 202, 203, 196, 215, 211, 216, 209, 196, 204, 208, 212, 212, 213, 207, 196, 204, 207, 214,
    210, 205, 209, 193, 164, 186, 204, 204, 202, 204, 208, 197, 170, 197, 217, 217, 224, 219, 216, 212,
    205, 211, 213, 207, 215, 205, 205, 210, 203, 204, 215, 208, 214, 211, 210, 172, 193, 197, 182, 201,
    213, 214, 225, 215, 212, 213, 185, 181, 198, 175, 210, 216, 199, 208, 205, 200, 205, 201, 201, 200,
    199, 198, 205, 206, 208, 203, 204, 209, 216, 211, 214, 220, 205, 207, 209, 192, 190, 196, 213, 212,
    203, 208, 184, 203, 207, 178, 160, 178, 174, 149, 188, 167, 191, 191, 192, 186, 195, 172, 123, 127,
    189, 200, 211, 220, 210, 209, 197, 134, 168, 197, 211, 209, 208, 206, 200, 188, 188, 191, 203, 202,
    205, 201, 204, 196, 197, 197, 214, 212, 218, 207, 215, 197, 210, 216, 210, 212, 201, 213, 219, 218,
    208, 196, 215, 196, 198, 212, 203, 190, 215, 216, 212, 214, 214, 202, 208, 209, 197, 199, 214, 202,
    200, 216, 210, 202, 213, 213, 216, 206, 218, 212, 210, 207, 203, 147, 191, 207, 216, 210, 215, 213,
    213, 214, 221, 204, 147, 203, 216, 217, 213, 220, 223, 210, 214, 206, 214, 198, 216, 214, 215, 207,
    207, 213, 192, 185, 209, 210, 207, 209, 212, 210, 212, 200, 207, 209, 198, 208, 206, 213, 206, 216,
    217, 210, 205, 213, 214, 207, 208, 197, 204, 206, 193, 204, 207, 207, 199, 204, 208, 208, 213, 213,
    214, 213, 210, 204, 212, 208, 203, 210, 208, 185, 198, 198, 212, 203, 196, 192, 186, 177, 173, 163,
    174, 192, 193, 195, 211, 188, 182, 176, 174, 119, 115, 155, 177, 207, 210, 213, 220, 219, 213, 206,
    204, 190, 156, 135, 153, 186, 181, 200, 206, 200, 207, 211, 213, 211, 213, 210, 209, 196, 203, 199,
    209, 205, 217, 215, 216, 220, 215, 217, 215, 211, 220, 214, 213, 204, 212, 214, 212, 203, 209, 210,
    198, 195, 209, 215, 206, 186, 206, 214, 220, 204, 189, 211, 199, 205, 207, 212, 216, 211, 204, 201,
    194, 196, 187, 165, 192, 201, 210, 204, 208, 208, 209, 213, 207, 212, 213, 190, 178, 196, 208, 212,
    212, 214, 213, 202, 214, 211, 208, 213, 208, 214, 213, 211, 207, 216, 211, 201, 198, 188, 209, 208,
    209, 206, 213, 214, 213, 204, 208, 188, 194, 197, 205, 214, 217, 208, 206, 206, 200, 200, 178, 151,
    144, 181, 192, 203, 213, 218, 224, 225, 218, 215, 209, 185, 166, 144, 166, 181, 211, 208, 211, 212,
    217, 215, 213, 216, 201, 182, 184, 155, 180, 202, 203, 209, 205, 202, 211, 209, 204, 199, 197, 197,
    210, 200, 176, 194, 207, 208, 215, 210, 208, 206, 212, 211, 208, 195, 200, 209, 206, 205, 209, 209,
    207, 202, 172, 175, 199, 217, 210, 209, 208, 207, 209, 201, 199, 215, 217, 214, 210, 217, 203, 193,
    198, 176, 188, 205, 207, 205, 203, 188, 211, 220, 209, 200, 205, 216, 208, 206, 200, 193, 210, 213,
    208, 214, 216, 212, 220, 215, 216, 212, 213, 214, 210, 199, 178, 193, 207, 214, 216, 215, 217, 216,
};
// H = 1536, 2-byte elements: 3 KiB rows, 3 channel groups
constexpr unsigned char kWinRate3K[kWinHi - kWinLo] = {
    183, 190, 177, 157, 170, 185, 190, 188, 157, 151, 192, 199, 212, 211, 150, 155, 180, 195, 179, 196,
    182, 175, 128, 187, 187, 184, 190, 202, 182, 175, 181, 180, 200, 198, 195, 155, 179, 195, 116, 182,
    207, 182, 202, 212, 195, 205, 185, 205, 232, 116, 206, 214, 226, 215, 212, 200, 211, 210, 202, 202,
    196, 206, 205, 183, 194, 102, 194, 130, 192, 190, 186, 204, 194, 212, 197, 164, 217, 187, 206, 207,
    187, 204, 169, 187, 207, 205, 203, 218, 218, 196, 214, 211, 191, 137, 190, 199, 204, 183, 212, 206,
    195, 211, 207, 194, 203, 200, 188, 193, 106, 211, 209, 196, 214, 214, 204, 195, 191, 213, 222, 207,
    189, 211, 211, 205, 201, 214, 207, 211, 214, 199, 219, 203, 208, 200, 154, 196, 190,  86, 212, 185,
    105, 204, 198, 194, 214, 199, 204, 214, 220, 222, 227, 211, 206, 203, 214, 191, 183, 191, 223, 224,
    246, 224, 193, 235, 247, 203, 220, 233, 230, 205, 215, 229, 224, 208, 201, 218, 225, 205, 223, 226,
    214, 212, 213, 218, 216, 200, 215, 214, 218, 176, 184, 205, 199, 171,  83, 201, 221, 211, 133, 151,
    202, 207, 203, 169, 197, 214, 224, 215, 214, 212, 219, 210, 211, 220, 187, 210, 219, 216, 170, 196,
    209, 217, 198, 191, 209, 182, 210, 213, 196, 214, 197, 199, 220, 207, 218, 222, 209, 182, 211, 229,
    224, 205, 188, 222, 218, 216, 195, 210, 213, 197, 185, 216, 205, 220, 212, 187, 218, 203, 196, 220,
    209, 205, 220, 221, 214, 196, 208, 230, 212, 193, 209, 221, 222, 218, 222, 182, 216, 218, 212, 219,
    172, 226, 217, 230, 219, 215, 209, 219, 217, 214, 220, 200, 220, 204, 211, 205, 192, 191, 208, 213,
    235, 214, 215, 166, 189, 169, 219, 217, 209, 214, 212, 215, 211, 226, 222, 220, 211, 220, 220, 223,
    208, 220, 195, 165, 217, 215, 211, 211, 211, 187, 163, 146, 161, 186, 196, 191, 201, 153, 107, 192,
    221, 224, 217, 147, 162, 209, 222, 222, 219, 186, 210, 221, 218, 209, 200, 203, 217, 219, 209, 220,
    216, 212, 223, 211, 228, 225, 206, 218, 197, 210, 202, 216, 218, 219, 206, 212, 186, 206, 210, 216,
    216, 215, 219, 224, 232, 220, 226, 203, 177, 229, 222, 236, 231, 234, 203, 169, 208, 226, 228, 222,
    220, 220, 212, 216, 220, 203, 211, 205, 220, 218, 210, 220, 210, 212, 220, 193, 204, 210, 218, 212,
    209, 223, 221, 221, 218, 220, 221, 225, 209, 221, 218, 222, 218, 218, 208, 210, 209, 213, 178, 205,
    220, 211, 194, 173, 157, 150, 184, 198, 206, 194, 170, 127, 111, 166, 204, 216, 228, 224, 221, 208,
    162, 126, 190, 213, 219, 218, 225, 229, 224, 219, 199, 204, 206, 216, 221, 211, 219, 228, 220, 221,
    218, 212, 222, 200, 215, 218, 198, 222, 214, 214, 227, 221, 201, 214, 208, 205, 227, 220, 208, 206,
    191, 197, 221, 220, 217, 216, 224, 221, 211, 183, 198, 213, 220, 219, 209, 220, 212, 210, 219, 221,
    214, 220, 208, 209, 213, 216, 214, 222, 220, 209, 189, 182, 218, 222, 222, 217, 218, 198, 155, 162,
    206, 224, 230, 235, 231, 223, 199, 143, 158, 209, 212, 222, 226, 212, 221, 167, 172, 182, 190, 212,
    203, 207, 209, 210, 195, 209, 203, 175, 205, 212, 214, 207, 221, 224, 213, 216, 221, 222, 222, 216,
    164, 191, 220, 205, 216, 210, 202, 215, 223, 223, 221, 206, 212, 195, 197, 209, 205, 212, 231, 217,
    211, 221, 211, 205, 217, 217, 223, 218, 228, 221, 223, 225, 222, 173, 196, 218, 227, 221, 226, 227,
    226, 220, 228, 202, 182, 200, 223, 227, 224, 225, 220, 213, 223, 209, 224, 207, 222, 222, 202, 195,
    209, 222, 201, 201, 223, 221, 212, 216, 194, 207, 195, 215, 221, 212, 200, 194, 214, 219, 197, 199,
    221, 226, 223, 226, 233, 230, 221, 221, 219, 202, 170, 192, 213, 177, 195, 221, 223, 221, 216, 213,
    210, 184, 202, 205, 214, 221, 217, 219, 221, 225, 225, 222, 220, 215, 208, 214, 205, 210, 219, 226,
    222, 223, 222, 217, 219, 214, 212, 210, 196, 133, 162, 216, 211, 219, 221, 221, 220, 219, 222, 217,
    213, 198, 186, 152, 159, 191, 166, 194, 193, 192, 199, 208, 215, 211, 215, 209, 206, 196, 184, 151,
    155, 192, 208, 214, 220, 234, 228, 219, 223, 202, 196, 157, 199, 195, 215, 221, 220, 223, 226, 218,
    215, 218, 210, 217, 213, 219, 226, 218, 218, 218, 211, 222, 215, 217, 216, 219, 219, 223, 224, 221,
    215, 217, 204, 193, 206, 223, 221, 222, 221, 218, 218, 225, 225, 225, 215, 207, 188, 204, 214, 198,
    201, 223, 221, 206, 211, 221, 219, 221, 218, 214, 219, 222, 215, 218, 215, 216, 214, 202, 216, 206,
    216, 216, 214, 211, 217, 213, 219, 215, 218, 217, 228, 225, 229, 227, 223, 222, 202, 204, 189, 161,
    192, 218, 225, 229, 228, 234, 238, 235, 232, 228, 226, 208, 185, 162, 156, 179, 208, 215, 222, 223,
    228, 226, 223, 221, 216, 214, 216, 207, 212, 222, 218, 219, 218, 217, 214, 208, 213, 221, 217, 215,
    216, 220, 220, 218, 223, 220, 223, 219, 217, 218, 214, 223, 222, 209, 200, 197, 192, 211, 218, 214,
    223, 224, 216, 213, 217, 219, 227, 231, 219, 210, 202, 191, 196, 217, 215, 215, 222, 219, 222, 226,
    221, 217, 220, 217, 215, 219, 210, 213, 220, 218, 223, 220, 217, 226, 214, 217, 207, 213, 209, 210,
    184, 188, 204, 209, 222, 228, 226, 207, 213, 196, 202, 197, 181, 186, 166, 175, 184, 183, 207, 212,
};
// H = 2048, 2-byte elements: 4 KiB rows, 4 channel groups
constexpr unsigned char kWinRate4K[kWinHi - kWinLo] = {
    182, 200, 193, 186, 199, 193, 192, 196, 201, 197, 193, 185, 193, 198, 204, 200, 203, 195, 208, 203,
    214, 204,  82, 215, 216, 217, 209, 214, 208, 202, 206, 155, 195, 202, 208, 201, 182, 208, 203, 209,
    209, 215, 174, 208, 185, 189, 141, 211, 216, 208, 211, 213, 209, 196, 194, 177, 209, 203, 209, 202,
    215, 176, 196, 123, 187, 115, 208, 191, 210, 205, 203, 191, 219, 221, 200, 191, 215, 197, 213, 215,
    214, 204, 214, 215, 197, 199, 190, 167, 211, 120, 218, 167, 226, 201, 228, 224, 219, 233, 211, 236,
    235, 189, 199, 221, 235, 218, 213, 226, 166, 220, 223, 217, 220, 224, 233, 230, 234, 234, 237, 224,
    228, 226, 224, 209, 223, 226, 166, 210, 202, 112, 209, 217, 213,  90, 201, 207, 194, 205, 222, 228,
    220, 221, 213, 220, 218, 192, 214, 189, 160, 201, 202, 163, 199, 192, 209, 207, 190, 206, 221, 209,
    226, 216, 171, 212, 218, 178, 219, 223, 210, 212, 216, 208, 199, 215, 214, 219, 226, 221, 225, 218,
    212, 227, 219, 211, 229, 222, 211, 216, 216, 211, 178, 205, 201, 204, 165, 211, 220, 220, 211, 223,
    224, 218, 208, 225, 224, 221, 195, 205, 225, 235, 223, 196, 199, 214, 218, 216, 217, 219, 215, 219,
    223, 208, 223, 226, 218, 225, 170, 220, 216, 200, 208, 168, 178, 176, 186, 174, 187, 134, 181, 205,
    214, 216, 175, 220, 226, 222, 201, 218, 219, 219, 204, 218, 222, 222, 220, 224, 211, 232, 221, 224,
    213, 216, 228, 224, 229, 220, 208, 234, 211, 221, 220, 228, 227, 221, 203, 192, 217, 215, 213, 215,
    186, 212, 221, 229, 225, 227, 221, 232, 218, 215, 216, 219, 223, 222, 212, 217, 211, 223, 233, 224,
    233, 224, 223, 217, 230, 223, 222, 226, 227, 223, 226, 222, 224, 218, 221, 214, 189, 178, 180, 195,
    199, 179, 168, 114, 180, 212, 229, 225, 212, 181, 154, 219, 226, 227, 230, 230, 223, 212, 210, 228,
    228, 229, 234, 237, 227, 227, 230, 223, 211, 222, 230, 220, 228, 219, 211, 224, 232, 224, 215, 203,
    211, 227, 226, 224, 225, 221, 198, 213, 227, 224, 224, 222, 226, 229, 225, 224, 215, 224, 230, 226,
    225, 212, 207, 221, 235, 226, 226, 192, 150, 198, 218, 245, 234, 218, 161, 179, 223, 224, 231, 226,
    209, 194, 186, 219, 211, 220, 218, 206, 212, 194, 214, 228, 222, 230, 228, 221, 224, 229, 213, 196,
    206, 212, 225, 220, 217, 232, 227, 230, 210, 220, 219, 215, 226, 227, 223, 226, 220, 228, 226, 228,
    237, 232, 230, 223, 199, 218, 233, 234, 236, 233, 231, 222, 196, 220, 233, 235, 236, 231, 230, 228,
    223, 228, 222, 205, 219, 220, 222, 226, 229, 221, 224, 210, 207, 223, 220, 202, 216, 219, 207, 228,
    231, 233, 239, 234, 230, 224, 183, 202, 214, 217, 224, 233, 224, 230, 218, 199, 210, 223, 222, 227,
    233, 230, 230, 232, 230, 213, 219, 226, 234, 233, 236, 235, 227, 222, 221, 201, 154, 196, 225, 223,
    228, 232, 221, 216, 223, 200, 158, 166, 190, 174, 207, 211, 216, 219, 217, 214, 203, 197, 173, 172,
    203, 201, 228, 234, 218, 231, 221, 178, 205, 215, 229, 228, 235, 230, 224, 221, 222, 226, 228, 231,
    220, 227, 230, 224, 226, 226, 228, 230, 232, 223, 222, 213, 219, 232, 231, 232, 220, 228, 234, 230,
    208, 203, 220, 222, 217, 229, 224, 220, 230, 233, 229, 224, 228, 226, 222, 227, 221, 230, 234, 226,
    223, 225, 227, 227, 225, 229, 237, 234, 244, 241, 229, 223, 210, 151, 195, 224, 235, 231, 247, 239,
    235, 239, 226, 195, 164, 197, 208, 229, 229, 236, 238, 237, 230, 227, 221, 225, 225, 227, 230, 228,
    230, 222, 224, 219, 227, 225, 226, 229, 230, 226, 226, 215, 224, 233, 221, 220, 200, 230, 226, 233,
    235, 228, 231, 234, 235, 229, 215, 208, 213, 228, 224, 233, 234, 236, 228, 226, 233, 226, 229, 227,
    226, 232, 229, 233, 231, 224, 225, 225, 222, 189, 208, 220, 222, 232, 225, 217, 212, 192, 189, 187,
    178, 189, 194, 210, 228, 218, 202, 196, 199, 153, 150, 180, 197, 225, 224, 234, 241, 236, 232, 227,
    226, 218, 206, 180, 199, 228, 224, 229, 234, 234, 233, 230, 229, 226, 228, 227, 229, 217, 225, 222,
    205, 216, 227, 231, 227, 226, 224, 231, 225, 228, 234, 231, 222, 215, 219, 229, 228, 226, 232, 231,
    218, 212, 213, 223, 217, 189, 212, 229, 231, 228, 223, 233, 222, 225, 222, 222, 220, 219, 223, 226,
    224, 229, 224, 208, 227, 230, 235, 234, 232, 228, 231, 235, 232, 233, 231, 222, 216, 222, 229, 229,
    227, 229, 228, 226, 212, 218, 217, 214, 218, 230, 226, 225, 227, 231, 228, 226, 219, 222, 226, 221,
    222, 207, 212, 223, 213, 211, 216, 221, 218, 213, 226, 230, 231, 230, 225, 232, 229, 220, 194, 188,
    186, 204, 211, 231, 235, 235, 239, 238, 238, 234, 227, 218, 188, 169, 202, 219, 231, 230, 228, 235,
    234, 232, 228, 231, 222, 214, 215, 192, 210, 222, 223, 219, 220, 225, 228, 229, 225, 218, 221, 221,
    225, 220, 213, 217, 221, 226, 227, 227, 226, 226, 233, 235, 234, 229, 224, 229, 225, 231, 230, 217,
    216, 215, 179, 168, 194, 210, 212, 225, 222, 221, 212, 213, 222, 228, 227, 223, 214, 224, 217, 206,
    204, 196, 211, 210, 213, 209, 215, 216, 224, 220, 227, 222, 223, 228, 232, 223, 225, 220, 226, 228,
    227, 229, 228, 230, 233, 233, 227, 227, 228, 232, 232, 225, 212, 215, 224, 234, 233, 231, 229, 228,
};

constexpr int kWinSpanBwd = 8;
constexpr int kWinSpanFwd = 64;

// The measured table for rows of row_bytes split into `groups` channel groups,
// or nullptr.
inline const unsigned char* win_rate_table(int64_t row_bytes, int groups) {
    if (row_bytes == 2048 && groups == 2) return kWinRate2K;
    if (row_bytes == 3072 && groups == 3) return kWinRate3K;
    if (row_bytes == 4096 && groups == 4) return kWinRate4K;
    return nullptr;
}

inline int64_t pick_window(int64_t sub0, int64_t row_bytes, int groups, int span) {
    const unsigned char* rate = LFM2SC_WIN_TABLES ? win_rate_table(row_bytes, groups) : nullptr;
    if (rate == nullptr || sub0 < kWinLo || sub0 >= kWinHi || span < 1) return sub0;
    const int64_t last = sub0 + (sub0 + span - 1) / span;
    int64_t best = sub0;
    for (int64_t s = sub0 + 1; s <= last && s < kWinHi; ++s)
        if (rate[s - kWinLo] > rate[best - kWinLo]) best = s;
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
    sub = pick_window(sub, row_bytes, groups, span);

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
