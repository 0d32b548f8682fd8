// device.h -- gfx950 device helpers shared by the MoE decode FFN kernels.
//
// Conventions (all kernels):
//  * a weight row is read as 16-byte chunks; chunk c of a row is held by lane
//    (c % LPR) of an LPR-lane segment, in register slot c / LPR, so one wave
//    instruction reads LPR*16 contiguous bytes per segment (64 lanes = 1 KiB);
//  * each lane accumulates its chunks in a fixed order, then the segment is
//    reduced with DPP and cross-row shuffles; every lane of the segment ends
//    with the same bits, so results never depend on which lane writes them;
//  * no floating-point atomics anywhere: every sum has one fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeffn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ---- cross-lane ---------------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// quad_perm [3,2,1,0] (lane ^ 3), row_half_mirror (reverse within 8 lanes),
// row_mirror (reverse within 16), row_ror:8 (rotate a row of 16 by 8: lane ^ 8),
// row_shr:n (lane i of a row reads lane i - n of the same row).
constexpr int kDppXor1 = 0xb1;
constexpr int kDppXor2 = 0x4e;
constexpr int kDppRevQuad = 0x1b;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned segments of LPR lanes (LPR in 8, 16, 32, 64); the result is
// in every lane of the segment.  Each step adds a lane's value to its partner's
// (a + b in one lane, b + a in the other), so all lanes hold identical bits.  The
// steps run from the widest partner distance down: halves of the wave, rows of 16
// lanes (both with the gfx950 permlane swaps, no LDS round trip), then mirrored
// lanes inside 16 and 8, then lane ^ 2 and lane ^ 1.  After a swap of a register with
// itself, one copy holds the lower partner's value and the other the upper
// partner's in both lanes of every pair, and the step adds lower + upper.
__device__ __forceinline__ float swap32_add(float lo_keep, float hi_keep) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo_keep), __float_as_uint(hi_keep), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float swap16_add(float even_keep, float odd_keep) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(even_keep), __float_as_uint(odd_keep), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float sum_in16(float v) {
    v = v + dpp_f<kDppMirror>(v);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppXor2>(v);
    v = v + dpp_f<kDppXor1>(v);
    return v;
}

template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "segment size");
    if constexpr (LPR >= 64) v = swap32_add(v, v);
    if constexpr (LPR >= 32) v = swap16_add(v, v);
    if constexpr (LPR >= 16) v = v + dpp_f<kDppMirror>(v);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppXor2>(v);
    v = v + dpp_f<kDppXor1>(v);
    return v;
}

// Inclusive prefix sum of an integer over the 64 lanes of a wave (every lane active):
// shifts of 1, 2, 4 and 8 lanes inside each row of 16 (DPP row shifts; a lane with no
// source lane adds 0), then each row adds the totals of the rows below it, read from
// their last lanes.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, true);
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Whole-wave sums of N rows at once (N = 1, 2, 4 or 8 partial values per lane): the
// same additions as seg_sum<64> on every row, in fewer instructions.  Each swap across
// halves or rows of 16 takes two rows' registers, keeps one row in each half, and
// adds, so the register count halves at every such step; the steps inside 16 lanes
// then run on what is left.  Where the results sit: rows_lane<N>(i) is the first lane
// holding row i (the 16-lane row or half it starts holds it in every lane), in result
// register rows_reg<N>(i).
template <int N> constexpr int rows_regs() { return N >= 8 ? 2 : 1; }
template <int N> __host__ __device__ constexpr int rows_lane(int i) {
    return N == 1 ? 0 : N == 2 ? 32 * i : N == 4 ? 16 * i : 16 * (i >> 1);
}
template <int N> __host__ __device__ constexpr int rows_reg(int i) { return N >= 8 ? (i & 1) : 0; }

template <int N>
__device__ __forceinline__ void seg_sum_rows(const float (&v)[N], float (&r)[rows_regs<N>()]) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "rows at once");
    if constexpr (N == 1) {
        r[0] = seg_sum<64>(v[0]);
    } else if constexpr (N == 2) {  // lanes 0-31 row 0, 32-63 row 1
        const float h = swap32_add(v[0], v[1]);
        r[0] = sum_in16(swap16_add(h, h));
    } else if constexpr (N == 4) {  // 16-lane row q holds row q
        r[0] = sum_in16(swap16_add(swap32_add(v[0], v[2]), swap32_add(v[1], v[3])));
    } else {  // register c, 16-lane row q: row c + 2q
        const float s0 = swap32_add(v[0], v[4]), s1 = swap32_add(v[1], v[5]);
        const float s2 = swap32_add(v[2], v[6]), s3 = swap32_add(v[3], v[7]);
        r[0] = sum_in16(swap16_add(s0, s2));
        r[1] = sum_in16(swap16_add(s1, s3));
    }
}

// ---- activation functions --------------------------------------------------------
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---- 16-byte chunk loads ---------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Chunk loads of a 256-thread staging pass: thread tid takes chunks tid + 256q
// (q < MAXC, below n), every load issued before any is used, so a pass costs one
// memory round trip, not one per chunk (a plain loop waits for each load before
// the next).  src(i) gives chunk i's address; src(0) must be readable even when n is
// 0.  Every thread issues all MAXC loads (a chunk at or past n re-reads the address
// of chunk n - 1, or of chunk 0, and is to be ignored): with a fixed number of loads in
// flight the compiler waits for exactly the ones a later use needs, not for all
// (memory returns loads in issue order; a conditional load would make it wait for
// every load issued before the use).
template <int MAXC, typename Src>
__device__ __forceinline__ void load_chunks(uint4 (&v)[MAXC], int n, int tid, Src src) {
    const int last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
        const int i = tid + 256 * q;
        v[q] = ld16(src(i < n ? i : last));
    }
}

// ---- 4-bit blocks ------------------------------------------------------------------
// A chunk is one 32-element block: word i holds elements 8i..8i+7, element
// 8i+n in bits 4n..4n+3 (low nibble = even element), stored as u = q + 8.
// Nibbles become bf16 values 128 + u by placing them under the bf16 pattern
// 0x43 (2^7): the byte-permute picks a nibble byte for the low half of each
// bf16 and 0x43 for the high half.  Pairs come out as (e0,e2) (e4,e6) from
// the low nibbles and (e1,e3) (e5,e7) from the high nibbles of a word.
constexpr uint32_t kQ4Bias = 0x43434343u;
constexpr uint32_t kSelLo = 0x04010400u;  // bytes 0 and 1 of the nibble word
constexpr uint32_t kSelHi = 0x04030402u;  // bytes 2 and 3

__device__ __forceinline__ void q4_word_to_bf16_pairs(uint32_t w, uint32_t out[4]) {
    const uint32_t lo = w & 0x0f0f0f0fu;
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;
    out[0] = __builtin_amdgcn_perm(kQ4Bias, lo, kSelLo);  // (e0, e2)
    out[1] = __builtin_amdgcn_perm(kQ4Bias, lo, kSelHi);  // (e4, e6)
    out[2] = __builtin_amdgcn_perm(kQ4Bias, hi, kSelLo);  // (e1, e3)
    out[3] = __builtin_amdgcn_perm(kQ4Bias, hi, kSelHi);  // (e5, e7)
}

// Rearranges 8 consecutive bf16 activations (4 words, element pairs (0,1)
// (2,3) (4,5) (6,7)) into the pair order of q4_word_to_bf16_pairs.
__device__ __forceinline__ void bf16x8_to_q4_order(const uint32_t x[4], uint32_t out[4]) {
    out[0] = __builtin_amdgcn_perm(x[1], x[0], 0x05040100u);  // (x0, x2)
    out[1] = __builtin_amdgcn_perm(x[3], x[2], 0x05040100u);  // (x4, x6)
    out[2] = __builtin_amdgcn_perm(x[1], x[0], 0x07060302u);  // (x1, x3)
    out[3] = __builtin_amdgcn_perm(x[3], x[2], 0x07060302u);  // (x5, x7)
}

// Workgroup barrier ordering LDS accesses only: global loads and stores in flight
// are not waited for, as they would be by __syncthreads (which waits for every
// outstanding memory access of the wave before the barrier).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moeffn
