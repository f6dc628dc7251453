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

// Lane value from another lane of the same row of 16 by a DPP pattern (VALU, no LDS).
template <int CTRL>
__device__ inline float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 32 lanes, result in every lane of the group: quad swaps
// (DPP quad_perm [1,0,3,2] and [2,3,0,1]), half-row and row mirrors (DPP), then the two
// rows of 16 exchanged with v_permlane16_swap.
__device__ inline float sum32(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    x += dpp_f32<0x140>(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------------------
// K/V tiles in LDS: rows of D bf16 (2D bytes, no padding), 16-byte chunks XOR-swizzled by
// row so that the MFMA operand reads are free of bank conflicts:
//   * K (ds_read_b128, lane = row, same logical chunk): chunk c of row r at c ^ swz_k(r);
//   * V (ds_read_b64_tr_b16, 4 rows x 2 chunks per 16 lanes): chunk c of row r at c ^ swz_v(r);
//   * tiles read both ways (the backward's Q, dO and K tiles): chunk c of row r at
//     c ^ swz_kv(r), which is injective on every 16 consecutive rows of one parity class
//     (row reads) and gives the 4 rows of an aligned group disjoint chunk quads (transposed
//     reads).  Unlike swz_v it is not periodic in 8 rows: swz_kv(r + 8) = swz_kv(r) ^ 2 for
//     r % 16 < 8.
// Tiles are filled with global_load_lds_dwordx4: lane L of a 64-lane instruction writes LDS
// bytes [16L, 16L+16) of that instruction's 1 KB window, i.e. slot s = (row, position).
// ---------------------------------------------------------------------------------------
template <int D>
__device__ inline int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ inline int swz_v(int r) {
    return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}
template <int D>
__device__ inline int swz_kv(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Row-tile order of the training-layout kernels that walk keys per row tile (heaviest
// first): rank -> row tile, with T row tiles per (batch, kv head) and tN0 the first tile
// that starts at a noisy position.  Noisy tiles from the end interleaved with the other
// tiles from the end of the clean stream, then whatever remains, in descending order.
__device__ inline int rank_to_tile(int rank, int T, int tN0) {
    const int nN = T - tN0, nR = tN0;
    const int m = nN < nR ? nN : nR;
    if (rank < 2 * m) return (rank & 1) ? (tN0 - 1 - (rank >> 1)) : (T - 1 - (rank >> 1));
    const int rr = rank - 2 * m;
    return (nN > m) ? (T - 1 - m - rr) : (tN0 - 1 - m - rr);
}

// A pointer the whole wave holds the same value of, made visibly wave-uniform (SGPRs) for an
// inline-asm operand that must be scalar.
template <class T>
__device__ inline T* uniform_ptr(T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// LDS byte address of a __shared__ object (the low half of its generic address).
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane L writes LDS bytes
// [w + 16L, w + 16L + 16) where w = `lds_window` is the same for the whole wave.  Issued
// as inline asm so the copies are invisible to the compiler's wait insertion: the caller
// orders them with wait_vmcnt<>() and a barrier before reading the window.
// M0 is saved and restored around the copy, since the compiler reserves it.
__device__ inline void dma16(const void* gsrc, uint32_t lds_window) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_window), "v"(gsrc)
        : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte offset
// (global_load_lds_dwordx4 v_off, s_base): no per-lane 64-bit address arithmetic.
__device__ inline void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_window) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_window), "v"(voff), "s"(sbase)
        : "memory");
}

// s_waitcnt vmcnt(N) for the gfx9 encoding (expcnt/lgkmcnt left unconstrained).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace mars
