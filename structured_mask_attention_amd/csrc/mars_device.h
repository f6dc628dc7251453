// Device-side building blocks of libmars (gfx950 / CDNA4, wave64).
//
// The visibility predicate here is the one every kernel uses (attention forward, the
// debug mask and tile-map kernels).  It is the mask of "MARS: Enabling Autoregressive
// Models Multi-Token Generation", §3.2 Eq. 2, with a causal prompt in front, written
// 0-indexed as two key intervals per query row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mars {

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x2_ev __attribute__((ext_vector_type(2)));
typedef float f32x2_ev __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Visible keys of query row r are [0, hi1) and [lo2, r].
//  * prompt / clean row (r < P + L): hi1 = r + 1, and [lo2, r] is empty (lo2 = r + 1);
//  * noisy row, response offset t0 = r - P - L, block k = t0 / B: hi1 = P + k*B (prompt and
//    the clean tokens of blocks before k), lo2 = P + L + k*B (own block, causal).
struct RowBounds {
    int hi1;
    int lo2;
};

__host__ __device__ inline RowBounds row_bounds(int r, int P, int L, int B) {
    if (r < P + L) return RowBounds{r + 1, r + 1};
    const int kB = ((r - P - L) / B) * B;
    return RowBounds{P + kB, P + L + kB};
}

__host__ __device__ inline bool key_visible(int r, int j, RowBounds rb) {
    return j < rb.hi1 || (j >= rb.lo2 && j <= r);
}

// Some key of [c0, c1) is visible to row r (c0 < c1).
__host__ __device__ inline bool range_any(int r, int c0, int c1, RowBounds rb) {
    if (c0 < rb.hi1) return true;
    const int lo = c0 > rb.lo2 ? c0 : rb.lo2;
    const int hi = (c1 - 1) < r ? (c1 - 1) : r;
    return lo <= hi;
}

// Every key of [c0, c1) is visible to row r (c0 < c1).
__host__ __device__ inline bool range_all(int r, int c0, int c1, RowBounds rb) {
    if (c1 <= rb.hi1) return true;
    if (c0 >= rb.lo2 && c1 - 1 <= r) return true;
    // The two intervals touch only when hi1 == lo2 (no noisy stream), handled above.
    return false;
}

__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    f32x2_ev v = {a, b};
    bf16x2_ev r = __builtin_convertvector(v, bf16x2_ev);
    return __builtin_bit_cast(uint32_t, r);
}

// Max / sum across the two 32-lane halves of a wave (lane l with lane l ^ 32).
__device__ inline float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mars
