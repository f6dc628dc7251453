// Training-layout backward of the MARS structured-mask attention: dQ, dK, dV of the
// forward in attn_fwd.hip ("MARS: Enabling Autoregressive Models Multi-Token Generation",
// §3.2 Eq. 2 and Fig. 2 left; training takes the losses of Eq. 3 and Eq. 5 through this
// attention, so it needs these gradients).
//
// With P the forward's row probabilities, D_i = sum_d dO_id O_id, and in the log2 domain
// of the forward (scores s = c q.k, c = scale*log2(e); P = 2^(s - LSE*log2(e))):
//   dV = P^T dO,   dS = P o (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q,
// dK and dV of a KV head summed over its G query heads.  Three kernels:
//   1. prep (per row): -D and -LSE*log2(e) into the workspace, positions padded to a
//      multiple of 32 (zeros);
//   2. dK/dV (key-stationary): a workgroup owns a block of keys of one (batch, kv head) and
//      walks the (32-position, head) tiles of every row that sees one of its keys (a union
//      of at most three position intervals).  Q and dO tiles plus the two per-row scalars
//      stream through an LDS ring (global_load_lds_dwordx4, XOR-swizzled chunks).  The
//      key-stationary side carries the score scale: its K fragments are Kc = bf16(K*c),
//      rounded once per workgroup.  Per tile and 32-key group: S = Q Kc^T and dP = dO V^T
//      (MFMA accumulators start at -LSE2 and -D), P = 2^S, dS = P dP, then dV^T += dO^T P
//      and dK^T += Q^T dS (dK takes the scale at the end) with the transposed operands read
//      by ds_read_b64_tr_b16.  Head_dim 64: 128 keys, one wave per 32 keys with K and V
//      fragments in registers, a 3-stage ring.  Head_dim 128: 192 keys, two waves per 32
//      keys split by role (K, S, P, dV on one; V, dP, dS, dK on the other, P handed over
//      through LDS), three waves per SIMD, two steps per barrier over a 6-stage ring.  The
//      element mask is a per-key bitmask over the tile's 32 positions.  A heavy key block
//      (prompt keys are seen by every row) splits its walk
//      into up to 8 chunks on separate workgroups (chunk size from the layout's total work);
//      their fp32 partials are written through to memory and summed in chunk order by
//      whichever wave arrives last for a 32-key slice and gradient (one counter each), so
//      the result does not depend on the arrival order.
//   3. dQ (row-stationary): the forward's row packing, tile walk, tile classes and K/V
//      ring; each lane rounds its row's Qc = bf16(Q*c) in registers exactly as the forward
//      does; per tile S^T = K Qc^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// P and dS enter the MFMAs as bf16 (round to nearest even); statistics and accumulation
// are fp32; gradients are stored as bf16.
#include <cmath>
#include <type_traits>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kWavesB = 4;
constexpr int kThreadsB = 64 * kWavesB;
constexpr int kT = 32;               // keys per dQ tile; positions per dK/dV tile; rows or keys per wave
constexpr int kStagesB = 3;
constexpr int kKeysPerWG = kWavesB * kT;   // dK/dV at head_dim 64: 128 keys per workgroup
constexpr int kRowsPerWGB = kWavesB * kT;  // dQ: 128 packed rows per workgroup
constexpr int kChunkMax = 8;               // dK/dV: a key block's walk splits into at most 8 chunks
constexpr int kChunkMinTiles = 4;          //        of at least 4 position tiles each
constexpr int kOrderMax = 1024;            // dK/dV work list passed with the launch (entries)
constexpr int kNominalSlots64 = 512;       // workgroup slots the dK/dV chunk size aims at: 2 per CU at
constexpr int kNominalSlots128 = 192;      // head_dim 64 (3 fit; 768 measured the same); at head_dim 128
                                           // (one per CU) 3/4 of the CUs, measured best of 160-1024

// ---------------------------------------------------------------------------------------
// LDS rings.  One file-scope object per stage, array and head_dim.
//   dK/dV: Q tile, dO tile ([32 positions][D] bf16 each) and the scalars of the tile's
//          rows ([-LSE2 x 32][-D x 32] fp32).
//   dQ:    K tile and V tile ([32 keys][D] bf16 each).
// ---------------------------------------------------------------------------------------
#define MARS_BRING(NAME, ELEMS)                                                         \
    __shared__ __attribute__((aligned(16))) uint16_t NAME##0[ELEMS];                    \
    __shared__ __attribute__((aligned(16))) uint16_t NAME##1[ELEMS];                    \
    __shared__ __attribute__((aligned(16))) uint16_t NAME##2[ELEMS];
MARS_BRING(g_bq64_, kT * 64)
MARS_BRING(g_bo64_, kT * 64)
MARS_BRING(g_bs64_, 128)         // 256 bytes of fp32 scalars per stage
MARS_BRING(g_dk128_, kT * 128)
MARS_BRING(g_dv128_, kT * 128)
MARS_BRING(g_dk64_, kT * 64)
MARS_BRING(g_dv64_, kT * 64)
#undef MARS_BRING

#define MARS_SEL(FN, N128, N64)                                                          \
    template <int D, int ST>                                                             \
    __device__ inline uint16_t* FN() {                                                   \
        static_assert(ST >= 0 && ST < kStagesB, "stage");                                \
        if constexpr (D == 128) {                                                        \
            if constexpr (ST == 0) return N128##0;                                       \
            else if constexpr (ST == 1) return N128##1;                                  \
            else return N128##2;                                                         \
        } else {                                                                         \
            if constexpr (ST == 0) return N64##0;                                        \
            else if constexpr (ST == 1) return N64##1;                                   \
            else return N64##2;                                                          \
        }                                                                                \
    }
// The 4-wave dK/dV kernel runs at head_dim 64 only (its rings have no head_dim-128 copy).
template <int D, int ST>
__device__ inline uint16_t* ring_q() {
    static_assert(D == 64 && ST >= 0 && ST < kStagesB, "stage");
    if constexpr (ST == 0) return g_bq64_0;
    else if constexpr (ST == 1) return g_bq64_1;
    else return g_bq64_2;
}
template <int D, int ST>
__device__ inline uint16_t* ring_o() {
    static_assert(D == 64 && ST >= 0 && ST < kStagesB, "stage");
    if constexpr (ST == 0) return g_bo64_0;
    else if constexpr (ST == 1) return g_bo64_1;
    else return g_bo64_2;
}
template <int D, int ST>
__device__ inline uint16_t* ring_s() {
    static_assert(D == 64 && ST >= 0 && ST < kStagesB, "stage");
    if constexpr (ST == 0) return g_bs64_0;
    else if constexpr (ST == 1) return g_bs64_1;
    else return g_bs64_2;
}
MARS_SEL(ring_k, g_dk128_, g_dk64_)
MARS_SEL(ring_v, g_dv128_, g_dv64_)
#undef MARS_SEL

typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Element e of an MFMA 32x32 accumulator sits at row (or key) 4*g2 + o(e) of the tile.
__device__ constexpr int acc_off(int e) { return 8 * (e >> 2) + (e & 3); }

// The 16 accumulator elements as two bf16x8 B operands (k = the accumulator's row index,
// in the order acc_off gives; the A operands are read to match).
__device__ inline void pack_b(const f32x16_t& x, bf16x8_t out[2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[8 * kh + 2 * i], x[8 * kh + 2 * i + 1]);
        out[kh] = __builtin_bit_cast(bf16x8_t, w);
    }
}

// Element mask of a tile: vis bit o (o < 32) says whether tile row (or key) o is visible;
// elements of this lane (rows/keys 4*g2 + acc_off(e)) outside it become -inf.
__device__ inline void apply_mask(f32x16_t& s, uint32_t vis, int g2) {
    const uint32_t v = vis >> (4 * g2);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int o = acc_off(e);
        const uint32_t t = (uint32_t)((int32_t)(v << (31 - o)) >> 31);
        s[e] = __uint_as_float((__float_as_uint(s[e]) & t) | (0xff800000u & ~t));
    }
}

// Bits [a - base, b - base) of a 32-bit mask (clipped to [0, 32)).
__device__ inline uint32_t span_bits(int a, int b, int base) {
    auto low = [](int x) { return x >= 32 ? 0xffffffffu : (1u << (x > 0 ? x : 0)) - 1u; };
    return low(b - base) & ~low(a - base);
}

// A operand (rows of a [32][D] tile, lane = row hl, 8 columns per lane) and transposed A
// operand (ds_read_b64_tr_b16: 16 tile rows x 32 columns per instruction pair) offsets.
// Tiles read both ways are swizzled with swz_kv; rows 8..15 of a 16-row chunk have their
// own base offset (hi = 1) because that swizzle is not periodic in 8 rows.
template <int D>
__device__ inline int row_read_off(int hl, int g2, int swz) {
    return hl * (2 * D) + 16 * (g2 ^ swz);
}
template <int D>
__device__ inline int tr_read_off(int lane, int hi) {
    const int s16 = lane & 15, grp = lane >> 4;
    const int row = 8 * hi + 4 * (grp >> 1) + (s16 >> 2);
    const int col = 16 * (grp & 1) + 4 * (s16 & 3);
    return row * (2 * D) + 16 * ((col >> 3) ^ swz_kv<D>(row)) + 2 * (col & 7);
}
// Transposed fragment of column block db, 16-row chunk kh (rows in acc_off order).
template <int D>
__device__ inline bf16x8_t tr_frag(const char* tile, int off_lo, int off_hi, int db, int kh) {
    const char* pl = tile + (off_lo ^ (64 * db)) + kh * 16 * (2 * D);
    const char* ph = tile + (off_hi ^ (64 * db)) + kh * 16 * (2 * D);
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)pl);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)ph);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Position tiles (32 positions) that see some key of [kb0, kb1): sorted, merged ranges
// [rs[i], re[i]) of tile indices; returns their number (<= 3).  Prompt/clean keys are seen
// by the later prompt/clean rows and by the noisy rows of the blocks after the smallest
// key's own (every block for a prompt key); noisy keys by the later rows of their block.
__host__ __device__ inline int kblock_tile_ranges(int kb0, int kb1, int P, int L, int B, int N, int rs[3], int re[3]) {
    const int PL = P + L;
    int s[3], e[3], n = 0;
    if (kb0 < PL) {
        s[n] = kb0; e[n] = PL; ++n;
        const int n0 = PL + (kb0 < P ? 0 : B * ((kb0 - P) / B + 1));
        if (n0 < N) { s[n] = n0; e[n] = N; ++n; }
    }
    if (kb1 > PL) {
        const int kl = (kb1 - 1 - PL) / B;
        const int hi = PL + (kl + 1) * B;
        s[n] = kb0 > PL ? kb0 : PL; e[n] = hi < N ? hi : N; ++n;
    }
    for (int i = 0; i < n; ++i) { s[i] = s[i] / kT; e[i] = (e[i] + kT - 1) / kT; }
    for (int i = 1; i < n; ++i)
        for (int m = i; m > 0 && s[m] < s[m - 1]; --m) {
            const int ts = s[m], te = e[m];
            s[m] = s[m - 1]; e[m] = e[m - 1]; s[m - 1] = ts; e[m - 1] = te;
        }
    int nm = 0;
    for (int i = 0; i < n; ++i) {
        if (nm > 0 && s[i] <= re[nm - 1]) re[nm - 1] = re[nm - 1] > e[i] ? re[nm - 1] : e[i];
        else { rs[nm] = s[i]; re[nm] = e[i]; ++nm; }
    }
    return nm;
}

// bf16(x * c) of eight bf16 values: fp32 product, then round to nearest even.
__device__ inline bf16x8_t scale_bf16x8(bf16x8_t x, float c) {
    const u32x4_t w = __builtin_bit_cast(u32x4_t, x);
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(__uint_as_float(w[i] << 16) * c, __uint_as_float(w[i] & 0xffff0000u) * c);
    return __builtin_bit_cast(bf16x8_t, r);
}

// Chunks of a key block's walk of npt position tiles, at most tc tiles per chunk.
__host__ __device__ inline int walk_chunks(int npt, int tc) {
    const int c = (npt + tc - 1) / tc;
    return c < 1 ? 1 : (c > kChunkMax ? kChunkMax : c);
}

// ---------------------------------------------------------------------------------------
// 1. Row prologue.
// ---------------------------------------------------------------------------------------
struct PrepParams {
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    float* nlse;
    float* ndelta;
    int* cnt;            // dK/dV arrival counters, zeroed here
    int64_t os0, os1, os2, ds0, ds1, ds2;
    int batch, hq, N, Npad, ncnt;
};

constexpr int kPrepPasses = 4;   // rows per prep thread (their loads issued together)

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(PrepParams p) {
    constexpr int TPR = D / 8;          // lanes per (batch, head, position) row, 8 elements each
    constexpr int RPP = 256 / TPR;      // rows per workgroup pass
    // Rows in [batch][head][position] order, the order of the two scalars written, so their
    // stores and the LSE reads are contiguous; a thread takes the same lane of kPrepPasses
    // rows RPP apart and issues all of their loads before using any.
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < p.ncnt) p.cnt[t] = 0;
    const int c8 = (int)(threadIdx.x % TPR);
    const int64_t rows = (int64_t)p.batch * p.hq * p.Npad;
    const int64_t r0 = (int64_t)blockIdx.x * (RPP * kPrepPasses) + threadIdx.x / TPR;
    u32x4_t ow[kPrepPasses], dw[kPrepPasses];
#pragma unroll
    for (int k = 0; k < kPrepPasses; ++k) {
        const int64_t r = r0 + (int64_t)k * RPP;
        const int pos = (int)(r % p.Npad);
        const int64_t bh = r / p.Npad;
        ow[k] = u32x4_t{0u, 0u, 0u, 0u};
        dw[k] = u32x4_t{0u, 0u, 0u, 0u};
        if (r < rows && pos < p.N) {
            const int h = (int)(bh % p.hq), b = (int)(bh / p.hq);
            ow[k] = *reinterpret_cast<const u32x4_t*>(p.o + b * p.os0 + (int64_t)pos * p.os1 + (int64_t)h * p.os2 + 8 * c8);
            dw[k] = *reinterpret_cast<const u32x4_t*>(p.dout + b * p.ds0 + (int64_t)pos * p.ds1 + (int64_t)h * p.ds2 + 8 * c8);
        }
    }
#pragma unroll
    for (int k = 0; k < kPrepPasses; ++k) {
        const int64_t r = r0 + (int64_t)k * RPP;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dot = fmaf(__uint_as_float(ow[k][i] << 16), __uint_as_float(dw[k][i] << 16), dot);
            dot = fmaf(__uint_as_float(ow[k][i] & 0xffff0000u), __uint_as_float(dw[k][i] & 0xffff0000u), dot);
        }
#pragma unroll
        for (int m = TPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
        if (c8 == 0 && r < rows) {
            const int pos = (int)(r % p.Npad);
            const int64_t bh = r / p.Npad;
            p.nlse[r] = pos < p.N ? -p.lse[bh * p.N + pos] * kLog2e : 0.f;
            p.ndelta[r] = pos < p.N ? -dot : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------------------
// 2. dK / dV.
// ---------------------------------------------------------------------------------------
struct DkvParams {
    const uint16_t* q;
    const uint16_t* dout;
    const uint16_t* k;
    const uint16_t* v;
    const float* nlse;       // workspace [batch][hq][Npad]
    const float* ndelta;
    uint16_t* dk;
    uint16_t* dv;
    float* part;             // workspace [nch_max][kblocks][bg][key groups][32 keys x 2D] fp32
    int* cnt;                // workspace [kblocks][bg][key groups][dV, dK], zero on entry
    int64_t qs0, qs2, ds0, ds2, ks0, ks1, ks2, vs0, vs1, vs2, dks0, dks1, dks2, dvs0, dvs1, dvs2;
    int qs1, ds1;            // position strides of Q and dO (at most 2^25 elements)
    int hq, hkv, G, P, L, B, N, Npad;
    int bg_count, kblocks, nch_max, tc;
    int rot;                 // 1: chunk index rotated by the key block (see the launch)
    int nord;                // > 0: the grid follows ord (longest chunks first), bg_count
                             // workgroups per entry; 0: the closed-form order
    uint16_t ord[kOrderMax]; // entry = key block << 3 | chunk
    int kgroups;             // 32-key groups per key block (4 at head_dim 64, 6 at 128)
    float c, scale;          // scale * log2(e) (folded into K), scale (applied to dK)
};

// Work item of this workgroup.  With a work list (p.nord > 0): entry blockIdx.x / bg_count,
// pair blockIdx.x % bg_count, so the pairs of one (key block, chunk) go to consecutive XCDs
// and the longest chunks start first.  Without: chunk fastest (rotated by the key block when
// p.rot), then pair, then key block.
__device__ inline void dkdv_item(const DkvParams& p, int& bg, int& kblk, int& c) {
    if (p.nord > 0) {
        bg = (int)(blockIdx.x % (unsigned)p.bg_count);
        const int e = p.ord[blockIdx.x / (unsigned)p.bg_count];
        kblk = e >> 3;
        c = e & 7;
    } else {
        const int rest = (int)(blockIdx.x / (unsigned)p.nch_max);
        bg = rest % p.bg_count;
        kblk = rest / p.bg_count;
        c = ((int)(blockIdx.x % (unsigned)p.nch_max) + (p.rot ? p.nch_max - kblk % p.nch_max : 0)) % p.nch_max;
    }
}

// dV (part 0) or dK (part 1) of one wave's 32 keys (key group kg of the block; j = this
// lane's key), from its accumulator acc = dV^T or dK^T: stored directly when the walk is one
// chunk, else through the chunk partials and the per-(slice, part) arrival counter.
template <int D>
__device__ inline void dkdv_finish_part(const DkvParams& p, int part, int c, int nch, int kblk, int bg, int kg,
                                        int lane, int b, int g, int j, bool kvalid, f32x16_t (&acc)[D / 32]) {
    constexpr int NDB = D / 32;
    const int g2 = lane >> 5;
    if (nch > 1) {
        // A walk in several chunks: every chunk stores its fp32 partial for its 32 keys; the
        // wave that arrives last for this 32-key slice and part (one counter each) sums the
        // partials in chunk order (the same order whoever is last).  Slot of a slice:
        // [dV | dK][d block][4 element groups][64 lanes] x 16 bytes, so every store / load
        // instruction moves 1 KB of contiguous memory.  Both are system coherent (sc0 sc1):
        // written through to memory and read from it, so chunks on other XCDs see them
        // without cache maintenance.
        constexpr int kPartBytes = NDB * 4 * 64 * 16;
        constexpr int kSysCoherent = 1 | 16;   // sc0 | sc1
        auto part_rsrc = [&](int cc) __attribute__((always_inline)) {
            char* base = reinterpret_cast<char*>(p.part) +
                         ((((int64_t)cc * p.kblocks + kblk) * p.bg_count + bg) * p.kgroups + kg) * (int64_t)(2 * kPartBytes) +
                         part * kPartBytes;
            return __builtin_amdgcn_make_buffer_rsrc(base, 0, kPartBytes, 0x00020000);
        };
        {
            const __amdgpu_buffer_rsrc_t r = part_rsrc(c);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4_t x = {acc[db][4 * qd], acc[db][4 * qd + 1], acc[db][4 * qd + 2], acc[db][4 * qd + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(x, r, (db * 4 + qd) * 1024 + 16 * lane, 0, kSysCoherent);
                }
            }
        }
        // Every partial store of this wave completes before its arrival is counted.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(p.cnt + (((int64_t)kblk * p.bg_count + bg) * p.kgroups + kg) * 2 + part, 1,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        asm volatile("" ::: "memory");
        if (old != nch - 1) return;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
        }
#pragma unroll 1
        for (int cc = 0; cc < nch; ++cc) {
            const __amdgpu_buffer_rsrc_t r = part_rsrc(cc);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (db * 4 + qd) * 1024 + 16 * lane, 0, kSysCoherent);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[db][4 * qd + i] += x[i];
                }
            }
        }
    }
    // dV = dV^T^T; dK = scale * dK^T^T (the walk multiplies by Q itself).
    if (!kvalid) return;
    const float mul = part ? p.scale : 1.f;
    uint16_t* out = part ? p.dk + b * p.dks0 + (int64_t)j * p.dks1 + (int64_t)g * p.dks2
                         : p.dv + b * p.dvs0 + (int64_t)j * p.dvs1 + (int64_t)g * p.dvs2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int d = 32 * db + 8 * bb + 4 * g2;
            uint2 w;
            w.x = pack_bf16x2(acc[db][4 * bb + 0] * mul, acc[db][4 * bb + 1] * mul);
            w.y = pack_bf16x2(acc[db][4 * bb + 2] * mul, acc[db][4 * bb + 3] * mul);
            *reinterpret_cast<uint2*>(out + d) = w;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreadsB, D == 64 ? 3 : 1) void attn_bwd_dkdv_kernel(DkvParams p) {
    constexpr int NC = D / 16;                    // 16-wide d chunks of the S / dP contractions
    constexpr int NDB = D / 32;                   // 32-row d blocks of dK^T / dV^T
    constexpr int CPR = D / 8;                    // 16-byte chunks per tile row
    constexpr int PERW = kT * CPR / 64 / kWavesB; // 1 KB copy windows per wave and tile array
    constexpr int GROUPW = 2 * PERW + 1;          // copy instructions per wave and step
    static_assert(PERW >= 1 && (kT * CPR / 64) % kWavesB == 0, "tile copy split");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31, g2 = lane >> 5;
    // Work item: chunk c of the walk of key block kblk of pair bg.
    int bg, kblk, c;
    dkdv_item(p, bg, kblk, c);
    const int b = bg / p.hkv, g = bg % p.hkv;
    const int PL = p.P + p.L;
    const int kb0 = kblk * kKeysPerWG;
    const int kb1 = min(kb0 + kKeysPerWG, p.N);

    // Position tiles of the key block (union over its keys), then this chunk's share.
    int rs[3] = {0, 0, 0}, re[3] = {0, 0, 0};
    kblock_tile_ranges(kb0, kb1, p.P, p.L, p.B, p.N, rs, re);
    const int n0t = re[0] - rs[0], n1t = re[1] - rs[1], n2t = re[2] - rs[2];
    const int npt = n0t + n1t + n2t;
    const int nch = walk_chunks(npt, p.tc);
    if (c >= nch) return;
    const int ct0 = (int)((int64_t)c * npt / nch), ct1 = (int)((int64_t)(c + 1) * npt / nch);
    const int nsteps = (ct1 - ct0) * p.G;
    auto pos_tile = [&](int ti) __attribute__((always_inline)) {
        ti += ct0;
        return ti < n0t ? rs[0] + ti : (ti < n0t + n1t ? rs[1] + (ti - n0t) : rs[2] + (ti - n0t - n1t));
    };

    // This lane's key and its K / V rows as B operands (k = d: 8 values per lane per chunk).
    const int j = kb0 + wave * kT + hl;
    const bool kvalid = j < p.N;
    const int jj = kvalid ? j : p.N - 1;
    bf16x8_t kf[NC], vf[NC];
    {
        const uint16_t* kp = p.k + b * p.ks0 + (int64_t)jj * p.ks1 + (int64_t)g * p.ks2 + 8 * g2;
        const uint16_t* vp = p.v + b * p.vs0 + (int64_t)jj * p.vs1 + (int64_t)g * p.vs2 + 8 * g2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            kf[cc] = scale_bf16x8(*reinterpret_cast<const bf16x8_t*>(kp + 16 * cc), p.c);
            vf[cc] = *reinterpret_cast<const bf16x8_t*>(vp + 16 * cc);
        }
    }
    // Positions that see key j: [a1, b1) u [a2, b2).  A prompt or clean key is seen by the
    // later prompt/clean rows and by the noisy rows of the blocks after its own (every
    // block, for a prompt key); a noisy key by the later rows of its own block.
    int a1 = 0, b1 = 0, a2 = 0, b2 = 0;
    if (kvalid) {
        if (j < PL) {
            a1 = j;
            b1 = PL;
            a2 = min(PL + (j < p.P ? 0 : p.B * ((j - p.P) / p.B + 1)), p.N);
            b2 = p.N;
        } else {
            a1 = j;
            b1 = min(p.N, PL + ((j - PL) / p.B + 1) * p.B);
        }
    }

    // Copy of step `it` (position tile, head) into stage ST.  Window slot (row r,
    // position ps) holds logical chunk ps ^ swz_kv(r) of row r; Q and dO rows past N repeat
    // row N-1 (finite; such rows are always masked).  The scalar copy: wave w moves bytes
    // [64w, 64w + 64) of [-LSE2 x 32][-D x 32] with four lanes.
    uint32_t qgo[PERW], ogo[PERW];
#pragma unroll
    for (int w = 0; w < PERW; ++w) {
        const int slot = 64 * (wave * PERW + w) + lane;
        const int r = slot / CPR, ps = slot % CPR;
        qgo[w] = (uint32_t)(r * p.qs1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
        ogo[w] = (uint32_t)(r * p.ds1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
    }
    // Running position of the next copy (walk order: position tile, then head): tile index
    // iti, head ih, and that step's base pointers; a head step adds one head stride, a tile
    // step recomputes them.
    int iti = 0, ih = 0, ip0 = 0;
    const uint16_t* iq = nullptr;
    const uint16_t* io = nullptr;
    const float* isl = nullptr;
    auto seek = [&]() __attribute__((always_inline)) {
        ip0 = pos_tile(iti) * kT;
        const int head = g * p.G;
        iq = p.q + b * p.qs0 + (int64_t)ip0 * p.qs1 + (int64_t)head * p.qs2;
        io = p.dout + b * p.ds0 + (int64_t)ip0 * p.ds1 + (int64_t)head * p.ds2;
        isl = (wave < 2 ? p.nlse : p.ndelta) + ((int64_t)b * p.hq + head) * p.Npad + ip0 + 16 * (wave & 1);
    };
    seek();
    auto issue = [&](auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const bool full = ip0 + kT <= p.N;
#pragma unroll
        for (int w = 0; w < PERW; ++w) {
            const int jw = wave * PERW + w;
            uint32_t oq = qgo[w], oo = ogo[w];
            if (!full) {
                const int slot = 64 * jw + lane;
                const int r = slot / CPR, ps = slot % CPR;
                const int rr = min(r, p.N - 1 - ip0);
                oq = (uint32_t)(rr * p.qs1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
                oo = (uint32_t)(rr * p.ds1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
            }
            dma16_sv(iq, oq, lds_addr(ring_q<D, ST>()) + 1024 * jw);
            dma16_sv(io, oo, lds_addr(ring_o<D, ST>()) + 1024 * jw);
        }
        if (lane < 4) dma16_sv(isl, (uint32_t)(16 * lane), lds_addr(ring_s<D, ST>()) + 64 * wave);
        if (++ih == p.G) {
            ih = 0;
            ++iti;
            seek();
        } else {
            iq += p.qs2;
            io += p.ds2;
            isl += p.Npad;
        }
    };

    f32x16_t dva[NDB], dka[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dva[db][e] = 0.f;
            dka[db][e] = 0.f;
        }
    }
    const int roff = row_read_off<D>(hl, g2, swz_kv<D>(hl));
    const int troff = tr_read_off<D>(lane, 0), troff_hi = tr_read_off<D>(lane, 1);

    issue(S0{});
    if (nsteps > 1) issue(S1{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();

    uint32_t vis = 0;
    bool any = false, all = false;
    int cti = 0, ch = 0;   // position tile and head of the step being computed
    auto body = [&](const int it, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        if (it + 1 < nsteps) wait_vmcnt<GROUPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (it + 2 < nsteps) issue(std::integral_constant<int, (ST + 2) % kStagesB>{});

        if (ch == 0) {
            // New position tile: this lane's visibility bits and the wave's tile class.
            const int p0 = pos_tile(cti) * kT;
            vis = span_bits(a1, b1, p0) | span_bits(a2, b2, p0);
            any = __builtin_amdgcn_ballot_w64(kvalid && vis != 0u) != 0ull;
            all = __builtin_amdgcn_ballot_w64(kvalid && vis != 0xffffffffu) == 0ull;
        }
        if (++ch == p.G) {
            ch = 0;
            ++cti;
        }
        if (!any) return;

        const char* qt = reinterpret_cast<const char*>(ring_q<D, ST>());
        const char* ot = reinterpret_cast<const char*>(ring_o<D, ST>());
        const char* st = reinterpret_cast<const char*>(ring_s<D, ST>());
        // S = Q Kc^T - LSE2 and dP = dO V^T - D; element e is tile row 4*g2 + acc_off(e).
        f32x16_t s, dp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(st + 4 * (4 * g2 + 8 * i));
            const f32x4_t c = *reinterpret_cast<const f32x4_t*>(st + 128 + 4 * (4 * g2 + 8 * i));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[4 * i + e] = a[e];
                dp[4 * i + e] = c[e];
            }
        }
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qt + (roff ^ (32 * cc)));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[cc], s, 0, 0, 0);
        }
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const bf16x8_t oa = *reinterpret_cast<const bf16x8_t*>(ot + (roff ^ (32 * cc)));
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[cc], dp, 0, 0, 0);
        }
        if (!all) apply_mask(s, vis, g2);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[e] = __builtin_amdgcn_exp2f(s[e]);   // P
            dp[e] *= s[e];                          // dS
        }
        bf16x8_t pb[2], sb[2];
        pack_b(s, pb);
        pack_b(dp, sb);
        // dV^T += dO^T P,  dK^T += Q^T dS  (A operands: transposed tile reads).
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(ot, troff, troff_hi, db, kh), pb[kh], dva[db], 0, 0, 0);
                dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qt, troff, troff_hi, db, kh), sb[kh], dka[db], 0, 0, 0);
            }
        }
    };
    for (int t0 = 0; t0 < nsteps; t0 += kStagesB) {
        body(t0, S0{});
        if (t0 + 1 < nsteps) body(t0 + 1, S1{});
        if (t0 + 2 < nsteps) body(t0 + 2, S2{});
    }

    dkdv_finish_part<D>(p, 0, c, nch, kblk, bg, wave, lane, b, g, j, kvalid, dva);
    dkdv_finish_part<D>(p, 1, c, nch, kblk, bg, wave, lane, b, g, j, kvalid, dka);
}

// ---------------------------------------------------------------------------------------
// 2b. dK / dV at head_dim 128: role-split wave pairs, three waves per SIMD.
//   At head_dim 128 a wave's dK and dV sums plus its keys' K and V fragments need about
//   400 registers.  Split by role, a wave holds one sum and one fragment set (~160
//   registers), so three waves fit a SIMD.  A workgroup of 12 waves owns 192 keys; waves w
//   and w + 6 share key group w and split every step's products:
//     role 0 (wave w):     Kc fragments in registers; S = Q Kc^T - LSE2, P = 2^S,
//                          dV^T += dO^T P;
//     role 1 (wave w + 6): V fragments in registers; dP = dO V^T - D, dS = P o dP,
//                          dK^T += Q^T dS.
//   An iteration covers two steps and one barrier.  P goes from role 0 to role 1 in bf16
//   (the values the dV MFMAs take) through an LDS exchange of two parities, so role 1 runs
//   one iteration behind: in iteration t role 0 does steps 2t and 2t + 1, role 1 steps
//   2t - 2 and 2t - 1, forming each step's dP right before its dS.  K and V never go
//   through LDS; each step's Q / dO tiles serve 192 keys.  The tiles and row scalars
//   stream through a 6-stage ring (steps 2t - 2 .. 2t + 1 in use, 2t + 2 and 2t + 3 in
//   flight): role-0 waves 0..3 copy the tile windows, waves 4 and 5 the scalars.
// ---------------------------------------------------------------------------------------
constexpr int kGroupsR = 6;                  // 32-key groups per workgroup
constexpr int kWavesR = 2 * kGroupsR;
constexpr int kThreadsR = 64 * kWavesR;
constexpr int kKeysPerWGR = kGroupsR * kT;   // 192
constexpr int kStagesR = 6;
__shared__ __attribute__((aligned(16))) uint16_t g_rq[kStagesR][kT * 128];   // Q tiles
__shared__ __attribute__((aligned(16))) uint16_t g_ro[kStagesR][kT * 128];   // dO tiles
__shared__ __attribute__((aligned(16))) float g_rs[kStagesR][64];            // [-LSE2 x 32][-D x 32]
__shared__ __attribute__((aligned(16))) uint16_t g_rx[2][2][kGroupsR][16 * 64];   // bf16 P: [parity][step][key group][half][lane]

__global__ __launch_bounds__(kThreadsR, 1) void attn_bwd_dkdv_role_kernel(DkvParams p) {
    constexpr int D = 128;
    constexpr int NC = D / 16, NDB = D / 32, CPR = D / 8;
    constexpr int TSZ = kT * D * 2;                 // bytes of one Q or dO tile
    static_assert(kT * CPR / 64 == 8, "eight 1 KB copy windows per tile, two per copying wave");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave >= kGroupsR ? 1 : 0;
    const int kg = wave - kGroupsR * role;
    const int hl = lane & 31, g2 = lane >> 5;
    int bg, kblk, c;
    dkdv_item(p, bg, kblk, c);
    const int b = bg / p.hkv, g = bg % p.hkv;
    const int PL = p.P + p.L;
    const int kb0 = kblk * kKeysPerWGR;
    const int kb1 = min(kb0 + kKeysPerWGR, p.N);

    int rs[3] = {0, 0, 0}, re[3] = {0, 0, 0};
    kblock_tile_ranges(kb0, kb1, p.P, p.L, p.B, p.N, rs, re);
    const int n0t = re[0] - rs[0], n1t = re[1] - rs[1], n2t = re[2] - rs[2];
    const int npt = n0t + n1t + n2t;
    const int nch = walk_chunks(npt, p.tc);
    if (c >= nch) return;
    const int ct0 = (int)((int64_t)c * npt / nch), ct1 = (int)((int64_t)(c + 1) * npt / nch);
    const int nsteps = (ct1 - ct0) * p.G;
    auto pos_tile = [&](int ti) __attribute__((always_inline)) {
        ti += ct0;
        return ti < n0t ? rs[0] + ti : (ti < n0t + n1t ? rs[1] + (ti - n0t) : rs[2] + (ti - n0t - n1t));
    };

    // This lane's key and the positions that see it: [a1, b1) u [a2, b2) (as the 4-wave kernel).
    const int j = kb0 + kg * kT + hl;
    const bool kvalid = j < p.N;
    int a1 = 0, b1 = 0, a2 = 0, b2 = 0;
    if (kvalid) {
        if (j < PL) {
            a1 = j;
            b1 = PL;
            a2 = min(PL + (j < p.P ? 0 : p.B * ((j - p.P) / p.B + 1)), p.N);
            b2 = p.N;
        } else {
            a1 = j;
            b1 = min(p.N, PL + ((j - PL) / p.B + 1) * p.B);
        }
    }

    // B operand of the S (role 0) or dP (role 1) MFMAs: this lane's key row of K or V, chunk
    // cc = d in [16 cc + 8 g2, 16 cc + 8 g2 + 8); keys past N repeat row N - 1 (never visible).
    bf16x8_t bfr[NC];
    {
        const int jj = min(j, p.N - 1);
        const uint16_t* src = role == 0 ? p.k + b * p.ks0 + (int64_t)jj * p.ks1 + (int64_t)g * p.ks2
                                        : p.v + b * p.vs0 + (int64_t)jj * p.vs1 + (int64_t)g * p.vs2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(src + 16 * cc + 8 * g2);
            bfr[cc] = role == 0 ? scale_bf16x8(x, p.c) : x;
        }
    }

    // Step copies, by the role-0 waves only (role 1 has the longer step): wave w < 4 moves
    // windows 2w and 2w + 1 of the Q tile and of the dO tile, waves 4 and 5 the 128 bytes
    // of -LSE2 and of -D.  Walk order: position tile, then head; the next copy's step is
    // (iti, ih).  Q and dO rows past N repeat row N - 1 (finite; always masked).
    uint32_t qgo[2], ogo[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int slot = 64 * (2 * (wave & 3) + jj) + lane;
        const int r = slot / CPR, ps = slot % CPR;
        qgo[jj] = (uint32_t)(r * p.qs1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
        ogo[jj] = (uint32_t)(r * p.ds1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
    }
    int iti = 0, ih = 0, ip0 = 0;
    const uint16_t* iq = nullptr;
    const uint16_t* io = nullptr;
    const float* isl = nullptr;
    auto seek = [&]() __attribute__((always_inline)) {
        ip0 = pos_tile(iti) * kT;
        const int head = g * p.G;
        iq = p.q + b * p.qs0 + (int64_t)ip0 * p.qs1 + (int64_t)head * p.qs2;
        io = p.dout + b * p.ds0 + (int64_t)ip0 * p.ds1 + (int64_t)head * p.ds2;
        isl = (wave == 4 ? p.nlse : p.ndelta) + ((int64_t)b * p.hq + head) * p.Npad + ip0;
    };
    seek();
    auto issue = [&](const int st) __attribute__((always_inline)) {
        if (wave < 4) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int win = 2 * wave + jj;
                uint32_t oq = qgo[jj], oo = ogo[jj];
                if (ip0 + kT > p.N) {
                    const int slot = 64 * win + lane;
                    const int r = slot / CPR, ps = slot % CPR;
                    const int rr = min(r, p.N - 1 - ip0);
                    oq = (uint32_t)(rr * p.qs1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
                    oo = (uint32_t)(rr * p.ds1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
                }
                dma16_sv(iq, oq, lds_addr(&g_rq[0][0]) + st * TSZ + 1024 * win);
                dma16_sv(io, oo, lds_addr(&g_ro[0][0]) + st * TSZ + 1024 * win);
            }
        } else if (wave < 6 && lane < 8) {
            dma16_sv(isl, (uint32_t)(16 * lane), lds_addr(&g_rs[0][0]) + st * 256 + 128 * (wave - 4));
        }
        if (++ih == p.G) {
            ih = 0;
            ++iti;
            seek();
        } else {
            iq += p.qs2;
            io += p.ds2;
            isl += p.Npad;
        }
    };

    f32x16_t acc[NDB];   // dV^T (role 0) or dK^T (role 1)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
    }
    const int roff = row_read_off<D>(hl, g2, swz_kv<D>(hl));
    const int troff = tr_read_off<D>(lane, 0), troff_hi = tr_read_off<D>(lane, 1);
    char* const xw = reinterpret_cast<char*>(&g_rx[0][0][kg][0]) + 16 * lane;   // + (2 parity + step) * 12 KB + half * 1 KB

    // Prologue: the key fragments and steps 0, 1 in flight, all drained before the walk.
    for (int t = 0; t < 2 && t < nsteps; ++t) issue(t);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();

    // S (role 0) or dP (role 1) of a step: the accumulator starts at the rows' -LSE2 or -D
    // (scalars at byte offset 0 or 128 of the stage); its A operand (Q or dO rows) is read
    // PF MFMAs ahead with a scheduling fence per MFMA.
    auto row_product = [&](const char* at, const char* sp, f32x16_t& x) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4_t y = *reinterpret_cast<const f32x4_t*>(sp + 4 * (4 * g2 + 8 * i));
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * i + e] = y[e];
        }
        constexpr int PF = 3;
        bf16x8_t ar[PF + 1];
#pragma unroll
        for (int i = 0; i < PF; ++i) ar[i] = *reinterpret_cast<const bf16x8_t*>(at + (roff ^ (32 * i)));
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (i + PF < NC) ar[(i + PF) % (PF + 1)] = *reinterpret_cast<const bf16x8_t*>(at + (roff ^ (32 * (i + PF))));
            x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[i % (PF + 1)], bfr[i], x, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // acc += (tile^T) y, the transposed tile read as A operands (dO for dV, Q for dK).
    auto col_product = [&](const char* tt, const bf16x8_t (&y)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tt, troff, troff_hi, db, kh), y[kh], acc[db], 0, 0, 0);
        }
    };

    // Walk, two steps per iteration: iteration t handles steps 2t and 2t + 1 on role 0 and
    // steps 2t - 2 and 2t - 1 on role 1, which reads their P (bf16, as the dV MFMAs use it)
    // from the exchange buffers role 0 filled in iteration t - 1.  Copies: steps 2t + 2 and
    // 2t + 3 go into the stages of steps 2t - 4 and 2t - 3 (ring of 6: steps 2t - 2 ... 2t + 3).
    constexpr int XSTEP = kGroupsR * 2 * 1024;   // bytes between the (parity, step) buffers
    auto walk = [&](auto role_c) __attribute__((always_inline)) {
        constexpr int R = decltype(role_c)::value;
        int cti = 0, ch = 0;             // position tile / head of this role's next step
        uint32_t vis = 0;
        bool any = false, all = false;
        int vis_tile = -1;
        int st = 0;                      // ring stage of this role's next step
        int st_i = 2;                    // stage of the next issue (step 2t + 2)
        auto nxt = [](int x) { return x + 1 == kStagesR ? 0 : x + 1; };
        // Classify this role's next step, then advance the counters past it.
        auto classify = [&]() __attribute__((always_inline)) {
            if (cti != vis_tile) {
                const int p0 = pos_tile(cti) * kT;
                vis = span_bits(a1, b1, p0) | span_bits(a2, b2, p0);
                any = __builtin_amdgcn_ballot_w64(kvalid && vis != 0u) != 0ull;
                all = __builtin_amdgcn_ballot_w64(kvalid && vis != 0xffffffffu) == 0ull;
                vis_tile = cti;
            }
            if (++ch == p.G) {
                ch = 0;
                ++cti;
            }
        };
        const int npairs = (nsteps + 1) / 2;
        for (int t = 0; t <= npairs; ++t) {
            if (t > 0) {
                // Steps 2t and 2t + 1 land (issued at the start of iteration t - 1).
                wait_vmcnt<0>();
                __syncthreads();
            }
            if (2 * t + 2 < nsteps) {
                issue(st_i);
                st_i = nxt(st_i);
            }
            if (2 * t + 3 < nsteps) {
                issue(st_i);
                st_i = nxt(st_i);
            }
            if constexpr (R == 0) {
#pragma unroll
                for (int jx = 0; jx < 2; ++jx) {
                    if (2 * t + jx < nsteps) {
                        classify();
                        if (any) {
                            const char* const qt = reinterpret_cast<const char*>(&g_rq[0][0]) + st * TSZ;
                            const char* const ot = reinterpret_cast<const char*>(&g_ro[0][0]) + st * TSZ;
                            const char* const sp = reinterpret_cast<const char*>(&g_rs[0][0]) + st * 256;
                            f32x16_t sa;
                            row_product(qt, sp, sa);
                            if (!all) apply_mask(sa, vis, g2);
#pragma unroll
                            for (int e = 0; e < 16; ++e) sa[e] = __builtin_amdgcn_exp2f(sa[e]);   // P
                            bf16x8_t pb[2];
                            pack_b(sa, pb);
                            char* const xc = xw + (2 * (t & 1) + jx) * XSTEP;
                            *reinterpret_cast<bf16x8_t*>(xc) = pb[0];
                            *reinterpret_cast<bf16x8_t*>(xc + 1024) = pb[1];
                            col_product(ot, pb);
                        }
                        st = nxt(st);
                    }
                }
            } else {
#pragma unroll
                for (int jx = 0; jx < 2; ++jx) {
                    const int s = 2 * t - 2 + jx;
                    if (t > 0 && s < nsteps) {
                        classify();
                        if (any) {
                            const char* const qt = reinterpret_cast<const char*>(&g_rq[0][0]) + st * TSZ;
                            const char* const ot = reinterpret_cast<const char*>(&g_ro[0][0]) + st * TSZ;
                            const char* const sp = reinterpret_cast<const char*>(&g_rs[0][0]) + st * 256;
                            const char* const xp = xw + (2 * ((t - 1) & 1) + jx) * XSTEP;
                            const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xp);
                            const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xp + 1024);
                            f32x16_t dp;
                            row_product(ot, sp + 128, dp);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {   // dS = P (dP - D), P as the bf16 pairs role 0 packed
                                dp[2 * i] *= __uint_as_float(x0[i] << 16);
                                dp[2 * i + 1] *= __uint_as_float(x0[i] & 0xffff0000u);
                                dp[8 + 2 * i] *= __uint_as_float(x1[i] << 16);
                                dp[8 + 2 * i + 1] *= __uint_as_float(x1[i] & 0xffff0000u);
                            }
                            bf16x8_t sb[2];
                            pack_b(dp, sb);
                            col_product(qt, sb);
                        }
                        st = nxt(st);
                    }
                }
            }
        }
    };
    if (role == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});

    dkdv_finish_part<D>(p, role, c, nch, kblk, bg, kg, lane, b, g, j, kvalid, acc);
}

// ---------------------------------------------------------------------------------------
// 3. dQ.
// ---------------------------------------------------------------------------------------
struct DqParams {
    const uint16_t* q;
    const uint16_t* dout;
    const uint16_t* k;
    const uint16_t* v;
    const float* nlse;
    const float* ndelta;
    uint16_t* dq;
    int64_t qs0, qs1, qs2, ds0, ds1, ds2, ks0, ks1, ks2, vs0, vs1, vs2, dqs0, dqs1, dqs2;
    int hq, hkv, G, P, L, B, N, Npad;
    int rows_per_pair, tiles_per_pair, tN0, bg_count;
    float scale, c;
};

template <int D>
__global__ __launch_bounds__(kThreadsB, 2) void attn_bwd_dq_kernel(DqParams p) {
    constexpr int NC = D / 16;
    constexpr int NDB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int NINS = kT * CPR / 64;
    constexpr int PERW = NINS / kWavesB;
    constexpr int GROUPW = 2 * PERW;
    static_assert(PERW >= 1 && NINS % kWavesB == 0, "tile copy split");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31, g2 = lane >> 5;
    const int bg = blockIdx.x % p.bg_count;
    const int rank = blockIdx.x / p.bg_count;
    const int tile = rank_to_tile(rank, p.tiles_per_pair, p.tN0);
    const int b = bg / p.hkv, g = bg % p.hkv;
    const int row0 = tile * kRowsPerWGB;
    const int wrow0 = row0 + wave * kT;

    // This lane's packed row: position u / G, head g*G + u % G (as in the forward).
    const int u = wrow0 + hl;
    const bool valid = u < p.rows_per_pair;
    const int uu = valid ? u : p.rows_per_pair - 1;
    const int pos = uu / p.G;
    const int head = g * p.G + uu % p.G;
    const RowBounds rb = row_bounds(pos, p.P, p.L, p.B);
    // The lane's half row (d = 16 cc + 8 g2 + [0, 8)) of Qc = bf16(Q c), rounded as the
    // forward rounds its Q operand, and of dO.
    bf16x8_t qf[NC], of[NC];
    {
        const uint16_t* qp = p.q + b * p.qs0 + (int64_t)pos * p.qs1 + (int64_t)head * p.qs2 + 8 * g2;
        const uint16_t* op = p.dout + b * p.ds0 + (int64_t)pos * p.ds1 + (int64_t)head * p.ds2 + 8 * g2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            qf[cc] = scale_bf16x8(*reinterpret_cast<const bf16x8_t*>(qp + 16 * cc), p.c);
            of[cc] = *reinterpret_cast<const bf16x8_t*>(op + 16 * cc);
        }
    }
    const int64_t sidx = ((int64_t)b * p.hq + head) * p.Npad + pos;
    const float nl = p.nlse[sidx];
    const float nd = p.ndelta[sidx];

    // Key walk of the workgroup's rows: [0, endA) and [startC, endC) (forward's schedule).
    const int u_last = min(row0 + kRowsPerWGB, p.rows_per_pair) - 1;
    const int pf = row0 / p.G, pl = u_last / p.G;
    const int PL = p.P + p.L;
    int endA = 0, startC = 0, endC = 0;
    if (pf < PL) endA = min(pl, PL - 1) + 1;
    if (pl >= PL) {
        endA = max(endA, p.P + ((pl - PL) / p.B) * p.B);
        startC = PL + ((max(pf, PL) - PL) / p.B) * p.B;
        endC = pl + 1;
    }
    const int nA = (endA + kT - 1) / kT;
    int c0t = startC / kT;
    const int c1t = (endC + kT - 1) / kT;
    if (c0t < nA) c0t = nA;
    const int nCt = c1t > c0t ? c1t - c0t : 0;
    const int ntiles = nA + nCt;
    auto tile_of = [&](int it) { return it < nA ? it : c0t + (it - nA); };

    const uint16_t* kbase = p.k + b * p.ks0 + (int64_t)g * p.ks2;
    const uint16_t* vbase = p.v + b * p.vs0 + (int64_t)g * p.vs2;
    // K tile: row reads and transposed reads (swz_kv); V tile: row reads only (swz_k).
    uint32_t kgo[PERW], vgo[PERW];
#pragma unroll
    for (int w = 0; w < PERW; ++w) {
        const int slot = 64 * (wave * PERW + w) + lane;
        const int r = slot / CPR, ps = slot % CPR;
        kgo[w] = (uint32_t)(r * p.ks1 * 2 + 16 * (ps ^ swz_kv<D>(r)));
        vgo[w] = (uint32_t)(r * p.vs1 * 2 + 16 * (ps ^ swz_k<D>(r)));
    }
    const int nfull = p.N / kT;
    auto issue = [&](const int it, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const int kt = tile_of(it);
        const int k0 = kt * kT;
        const uint16_t* kb = kbase + (int64_t)k0 * p.ks1;
        const uint16_t* vb = vbase + (int64_t)k0 * p.vs1;
#pragma unroll
        for (int w = 0; w < PERW; ++w) {
            const int jw = wave * PERW + w;
            if (kt < nfull) {
                dma16_sv(kb, kgo[w], lds_addr(ring_k<D, ST>()) + 1024 * jw);
                dma16_sv(vb, vgo[w], lds_addr(ring_v<D, ST>()) + 1024 * jw);
            } else {
                const int slot = 64 * jw + lane;
                const int r = slot / CPR, ps = slot % CPR;
                const int rr = min(r, p.N - 1 - k0);
                dma16_sv(kb, (uint32_t)(rr * p.ks1 * 2 + 16 * (ps ^ swz_kv<D>(r))), lds_addr(ring_k<D, ST>()) + 1024 * jw);
                dma16_sv(vb, (uint32_t)(rr * p.vs1 * 2 + 16 * (ps ^ swz_k<D>(r))), lds_addr(ring_v<D, ST>()) + 1024 * jw);
            }
        }
    };

    // Tile classes of the wave's rows (the forward's union / intersection intervals).
    const bool wave_has_rows = wrow0 < p.rows_per_pair;
    int U_hi = 0, C0 = 0, Cend = 0, I_hi = 0, I2lo = 1, I2hi = 0;
    if (wave_has_rows) {
        const int u_hi = min(wrow0 + kT, p.rows_per_pair) - 1;
        const int p_lo = wrow0 / p.G, p_hi = u_hi / p.G;
        I_hi = 0x7fffffff;
        if (p_lo < PL) {
            U_hi = min(p_hi, PL - 1) + 1;
            I_hi = p_lo + 1;
        }
        if (p_hi >= PL) {
            const int n_lo = max(p_lo, PL);
            const int klo = (n_lo - PL) / p.B, khi = (p_hi - PL) / p.B;
            U_hi = max(U_hi, p.P + khi * p.B);
            I_hi = min(I_hi, p.P + klo * p.B);
            C0 = PL + klo * p.B;
            Cend = p_hi + 1;
            if (p_lo >= PL && klo == khi) {
                I2lo = C0;
                I2hi = n_lo + 1;
            }
        }
    }
    auto tile_class = [&](const int it) __attribute__((always_inline)) {
        const int kb = tile_of(it) * kT;
        const int ke = kb + kT;
        const bool any = (kb < U_hi) || (kb < Cend && ke > C0);
        const bool all = (ke <= p.N) && (ke <= I_hi || (kb >= I2lo && ke <= I2hi));
        return (any ? 1 : 0) | (all ? 2 : 0);
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
    }
    const int kroff = row_read_off<D>(hl, g2, swz_kv<D>(hl));
    const int vroff = row_read_off<D>(hl, g2, swz_k<D>(hl));
    const int troff = tr_read_off<D>(lane, 0), troff_hi = tr_read_off<D>(lane, 1);

    issue(0, S0{});
    if (ntiles > 1) issue(1, S1{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();

    auto body = [&](const int it, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        if (it + 1 < ntiles) wait_vmcnt<GROUPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (it + 2 < ntiles) issue(it + 2, std::integral_constant<int, (ST + 2) % kStagesB>{});
        const int cls = __builtin_amdgcn_readfirstlane(tile_class(it));
        if (!(cls & 1)) return;
        const int kb = tile_of(it) * kT;
        const char* kt_lds = reinterpret_cast<const char*>(ring_k<D, ST>());
        const char* vt_lds = reinterpret_cast<const char*>(ring_v<D, ST>());
        // S^T = K Qc^T - LSE2, dP^T = V dO^T - D; element e is key kb + 4*g2 + acc_off(e).
        f32x16_t s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[e] = nl;
            dp[e] = nd;
        }
        // S and dP chunks alternate (i even: S chunk i/2, odd: dP chunk i/2), each A operand
        // read PF MFMAs ahead with a scheduling fence per MFMA (near the register limit the
        // compiler would otherwise wait for each read right before its MFMA).
        {
            constexpr int NA = 2 * NC, PF = 3;
            bf16x8_t ar[PF + 1];
            auto opread = [&](const int i) __attribute__((always_inline)) {
                ar[i % (PF + 1)] = (i & 1) ? *reinterpret_cast<const bf16x8_t*>(vt_lds + (vroff ^ (32 * (i >> 1))))
                                           : *reinterpret_cast<const bf16x8_t*>(kt_lds + (kroff ^ (32 * (i >> 1))));
            };
#pragma unroll
            for (int i = 0; i < PF; ++i) opread(i);
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                if (i + PF < NA) opread(i + PF);
                if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[i % (PF + 1)], of[i >> 1], dp, 0, 0, 0);
                else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[i % (PF + 1)], qf[i >> 1], s, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (!(cls & 2)) {
            auto low = [](int x) { return x >= 32 ? 0xffffffffu : (1u << max(x, 0)) - 1u; };
            const int A = rb.hi1 - kb, Lo = rb.lo2 - kb, Hi = pos - kb;
            apply_mask(s, low(A) | (low(Hi + 1) & ~low(Lo)), g2);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[e] *= __builtin_amdgcn_exp2f(s[e]);   // dS = P (dP - D)
        bf16x8_t sb[2];
        pack_b(dp, sb);
        // dQ^T += K^T dS^T.
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(kt_lds, troff, troff_hi, db, kh), sb[kh], acc[db], 0, 0, 0);
        }
    };
    for (int t0 = 0; t0 < ntiles; t0 += kStagesB) {
        body(t0, S0{});
        if (t0 + 1 < ntiles) body(t0 + 1, S1{});
        if (t0 + 2 < ntiles) body(t0 + 2, S2{});
    }

    // dQ = scale * dQ^T^T (bf16).
    if (valid) {
        uint16_t* qo = p.dq + b * p.dqs0 + (int64_t)pos * p.dqs1 + (int64_t)head * p.dqs2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d = 32 * db + 8 * bb + 4 * g2;
                uint2 w;
                w.x = pack_bf16x2(acc[db][4 * bb + 0] * p.scale, acc[db][4 * bb + 1] * p.scale);
                w.y = pack_bf16x2(acc[db][4 * bb + 2] * p.scale, acc[db][4 * bb + 3] * p.scale);
                *reinterpret_cast<uint2*>(qo + d) = w;
            }
        }
    }
}

int pad32(int n) { return (n + kT - 1) / kT * kT; }

size_t r256(size_t x) { return (x + 255) / 256 * 256; }

// Chunk size of the dK/dV walks (position tiles): half the mean number of tiles per
// workgroup slot for a nominal slot count (kNominalSlots64 / kNominalSlots128, chosen by
// measurement: at head_dim 128 the 256 real slots would put chunks at half a slot's load,
// which packs worse than two thirds), at least kChunkMinTiles; and the largest chunk count
// over the key blocks (sizes the partial buffer).
void walk_plan(int P, int L, int B, int N, int bg, int d, int kpb, int* tc, int* nch_max) {
    int64_t total = 0;
    int maxnpt = 0;
    for (int kb0 = 0; kb0 < N; kb0 += kpb) {
        int rs[3] = {0, 0, 0}, re[3] = {0, 0, 0};
        const int n = kblock_tile_ranges(kb0, kb0 + kpb < N ? kb0 + kpb : N, P, L, B, N, rs, re);
        int npt = 0;
        for (int i = 0; i < n; ++i) npt += re[i] - rs[i];
        total += npt;
        maxnpt = npt > maxnpt ? npt : maxnpt;
    }
    const int64_t slots = d == 64 ? kNominalSlots64 : kNominalSlots128;
    const int64_t t = (total * bg + 2 * slots - 1) / (2 * slots);
    *tc = (int)(t < kChunkMinTiles ? kChunkMinTiles : t);
    *nch_max = walk_chunks(maxnpt, *tc);
}

// Workspace: -LSE2 [batch][hq][Npad] | -D [batch][hq][Npad] |
// counters [kblocks][batch*hkv][groups][2] int | partials [nch][kblocks][batch*hkv][groups][32 x 2D] fp32
// (groups = 32-key groups per key block: 4 at head_dim 64, 6 at head_dim 128)
// (partials only when some key block's walk is split).
struct BwdLayout {
    size_t nlse, ndelta, cnt, part, total;
    int Npad, kpb, kgroups, kblocks, nch, tc;
};
BwdLayout bwd_layout(int batch, int hq, int hkv, int d, int P, int L, int B, int N) {
    BwdLayout w;
    w.Npad = pad32(N);
    w.kpb = d == 128 ? kKeysPerWGR : kKeysPerWG;   // keys per dK/dV workgroup
    w.kgroups = w.kpb / kT;
    w.kblocks = (N + w.kpb - 1) / w.kpb;
    const size_t bg = (size_t)batch * hkv;
    walk_plan(P, L, B, N, (int)bg, d, w.kpb, &w.tc, &w.nch);
    w.nlse = 0;
    w.ndelta = w.nlse + r256((size_t)batch * hq * w.Npad * 4);
    w.cnt = w.ndelta + r256((size_t)batch * hq * w.Npad * 4);
    w.part = w.cnt + r256((size_t)w.kblocks * bg * w.kgroups * 2 * 4);
    w.total = w.part + (w.nch > 1 ? r256((size_t)w.nch * w.kblocks * bg * w.kpb * 2 * d * 4) : 0);
    return w;
}

// Position tiles the walk of key block kb visits.
int kblock_tiles(const BwdLayout& w, int kb, int P, int L, int B, int N) {
    const int kb0 = kb * w.kpb;
    int rs[3] = {0, 0, 0}, re[3] = {0, 0, 0};
    const int nr = kblock_tile_ranges(kb0, kb0 + w.kpb < N ? kb0 + w.kpb : N, P, L, B, N, rs, re);
    int npt = 0;
    for (int i = 0; i < nr; ++i) npt += re[i] - rs[i];
    return npt;
}

// (key block, chunk) entries of the dK/dV grid: the chunks that exist, which is fewer than
// key blocks x the largest chunk count wherever walks differ in length.
int64_t bwd_work_items(const BwdLayout& w, int P, int L, int B, int N) {
    int64_t n = 0;
    for (int kb = 0; kb < w.kblocks; ++kb) n += walk_chunks(kblock_tiles(w, kb, P, L, B, N), w.tc);
    return n;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int batch, int hq, int hkv, int d, int P, int L, int B) {
    return bwd_layout(batch, hq, hkv, d, P, L, B, P + 2 * L).total;
}

void attn_bwd_plan(int batch, int hq, int hkv, int d, int P, int L, int B, int* chunk_tiles, int* max_chunks,
                   int64_t* items, int* work_list) {
    const int N = P + 2 * L;
    const BwdLayout w = bwd_layout(batch, hq, hkv, d, P, L, B, N);
    *chunk_tiles = w.tc;
    *max_chunks = w.nch;
    *items = bwd_work_items(w, P, L, B, N);
    *work_list = *items <= kOrderMax ? 1 : 0;
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t s) {
    const BwdLayout w = bwd_layout(a.batch, a.hq, a.hkv, a.d, a.P, a.L, a.B, a.N);
    const int Npad = w.Npad;
    char* ws = static_cast<char*>(a.ws);
    float* nlse = reinterpret_cast<float*>(ws + w.nlse);
    float* ndelta = reinterpret_cast<float*>(ws + w.ndelta);
    int* cnt = reinterpret_cast<int*>(ws + w.cnt);
    float* part = reinterpret_cast<float*>(ws + w.part);
    const int G = a.hq / a.hkv;
    const float c = a.scale * kLog2e;
    const int bg_count = a.batch * a.hkv;

    PrepParams pp;
    pp.o = static_cast<const uint16_t*>(a.o);
    pp.dout = static_cast<const uint16_t*>(a.dout);
    pp.lse = a.lse;
    pp.nlse = nlse;
    pp.ndelta = ndelta;
    pp.cnt = cnt;
    pp.os0 = a.os[0]; pp.os1 = a.os[1]; pp.os2 = a.os[2];
    pp.ds0 = a.dos[0]; pp.ds1 = a.dos[1]; pp.ds2 = a.dos[2];
    pp.batch = a.batch;
    pp.hq = a.hq;
    pp.N = a.N;
    pp.Npad = Npad;
    pp.ncnt = w.kblocks * bg_count * w.kgroups * 2;
    const int64_t prep_rows = (int64_t)a.batch * a.hq * Npad;
    const int64_t rows_per_wg = (int64_t)(256 / (a.d / 8)) * kPrepPasses;
    int64_t prep_wgs = (prep_rows + rows_per_wg - 1) / rows_per_wg;
    if (prep_wgs * 256 < pp.ncnt) prep_wgs = ((int64_t)pp.ncnt + 255) / 256;
    const dim3 pg((unsigned)prep_wgs);
    if (a.d == 128) hipLaunchKernelGGL((attn_bwd_prep_kernel<128>), pg, dim3(256), 0, s, pp);
    else hipLaunchKernelGGL((attn_bwd_prep_kernel<64>), pg, dim3(256), 0, s, pp);

    DkvParams kp;
    kp.q = static_cast<const uint16_t*>(a.q);
    kp.dout = pp.dout;
    kp.k = static_cast<const uint16_t*>(a.k);
    kp.v = static_cast<const uint16_t*>(a.v);
    kp.nlse = nlse;
    kp.ndelta = ndelta;
    kp.dk = static_cast<uint16_t*>(a.dk);
    kp.dv = static_cast<uint16_t*>(a.dv);
    kp.part = part;
    kp.cnt = cnt;
    kp.qs0 = a.qs[0]; kp.qs1 = (int)a.qs[1]; kp.qs2 = a.qs[2];
    kp.ds0 = a.dos[0]; kp.ds1 = (int)a.dos[1]; kp.ds2 = a.dos[2];
    kp.ks0 = a.ks[0]; kp.ks1 = a.ks[1]; kp.ks2 = a.ks[2];
    kp.vs0 = a.vs[0]; kp.vs1 = a.vs[1]; kp.vs2 = a.vs[2];
    kp.dks0 = a.dks[0]; kp.dks1 = a.dks[1]; kp.dks2 = a.dks[2];
    kp.dvs0 = a.dvs[0]; kp.dvs1 = a.dvs[1]; kp.dvs2 = a.dvs[2];
    kp.hq = a.hq;
    kp.hkv = a.hkv;
    kp.G = G;
    kp.P = a.P;
    kp.L = a.L;
    kp.B = a.B;
    kp.N = a.N;
    kp.Npad = Npad;
    kp.bg_count = bg_count;
    kp.kblocks = w.kblocks;
    kp.kgroups = w.kgroups;
    kp.nch_max = w.nch;
    kp.tc = w.tc;
    kp.c = c;
    kp.scale = a.scale;
    // Grid order.  Workgroups are dispatched in index order, workgroup i to XCD i mod 8, so
    // the order decides both when a chunk starts and where it runs.  Work list: every
    // (key block, chunk) that exists, longest chunk first (a counting sort on the chunk's
    // tile count, ties in key block and chunk order), with the pairs of an entry on
    // consecutive workgroups: the heaviest chunks no longer start late and every XCD gets
    // a similar mix.
    kp.nord = 0;
    kp.rot = 0;
    int64_t kgrid = (int64_t)w.nch * w.kblocks * bg_count;
    const int64_t nent = bwd_work_items(w, a.P, a.L, a.B, a.N);
    if (nent <= kOrderMax) {
        int len[kOrderMax];
        int hist[kOrderMax + 2] = {0};
        int n = 0, maxlen = 0;
        for (int kb = 0; kb < w.kblocks; ++kb) {
            const int npt = kblock_tiles(w, kb, a.P, a.L, a.B, a.N);
            const int nch = walk_chunks(npt, w.tc);
            for (int cc = 0; cc < nch; ++cc) {
                len[n] = (int)((int64_t)(cc + 1) * npt / nch - (int64_t)cc * npt / nch);
                if (len[n] > kOrderMax) len[n] = kOrderMax;   // only the rank matters
                maxlen = len[n] > maxlen ? len[n] : maxlen;
                kp.ord[n++] = (uint16_t)(kb << 3 | cc);
            }
        }
        // start of each length's run, longest first
        for (int i = 0; i < n; ++i) ++hist[len[i]];
        int at = 0;
        for (int l = maxlen; l >= 0; --l) {
            const int cnt = hist[l];
            hist[l] = at;
            at += cnt;
        }
        uint16_t sorted[kOrderMax];
        for (int i = 0; i < n; ++i) sorted[hist[len[i]]++] = kp.ord[i];
        for (int i = 0; i < n; ++i) kp.ord[i] = sorted[i];
        kp.nord = n;
        kgrid = (int64_t)n * bg_count;
    } else {
        // Closed-form order: chunk fastest, then pair, then key block; it keeps a (pair, chunk)
        // of nearby key blocks on one XCD, but when it sends every walk's chunk 0 (a short
        // walk's only chunk) to some XCDs only, the chunk index is rotated by the key block.
        unsigned seen = 0;
        const int64_t S = (int64_t)bg_count * w.nch;
        for (int kb = 0; kb < w.kblocks && kb < 8; ++kb)
            for (int bi = 0; bi < bg_count && bi < 8; ++bi) seen |= 1u << (int)((kb * S + (int64_t)bi * w.nch) & 7);
        kp.rot = seen == 0xffu ? 0 : 1;
    }
    const dim3 kg((unsigned)kgrid);
    if (a.d == 128) hipLaunchKernelGGL(attn_bwd_dkdv_role_kernel, kg, dim3(kThreadsR), 0, s, kp);
    else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<64>), kg, dim3(kThreadsB), 0, s, kp);

    DqParams qp;
    qp.q = kp.q;
    qp.dout = pp.dout;
    qp.k = kp.k;
    qp.v = kp.v;
    qp.nlse = nlse;
    qp.ndelta = ndelta;
    qp.dq = static_cast<uint16_t*>(a.dq);
    qp.ds0 = a.dos[0]; qp.ds1 = a.dos[1]; qp.ds2 = a.dos[2];
    qp.ks0 = a.ks[0]; qp.ks1 = a.ks[1]; qp.ks2 = a.ks[2];
    qp.vs0 = a.vs[0]; qp.vs1 = a.vs[1]; qp.vs2 = a.vs[2];
    qp.qs0 = a.qs[0]; qp.qs1 = a.qs[1]; qp.qs2 = a.qs[2];
    qp.dqs0 = a.dqs[0]; qp.dqs1 = a.dqs[1]; qp.dqs2 = a.dqs[2];
    qp.hq = a.hq;
    qp.hkv = a.hkv;
    qp.G = G;
    qp.P = a.P;
    qp.L = a.L;
    qp.B = a.B;
    qp.N = a.N;
    qp.Npad = Npad;
    qp.rows_per_pair = a.N * G;
    qp.tiles_per_pair = (qp.rows_per_pair + kRowsPerWGB - 1) / kRowsPerWGB;
    const int64_t noisy_row0 = (int64_t)(a.P + a.L) * G;
    int tN0 = (int)((noisy_row0 + kRowsPerWGB - 1) / kRowsPerWGB);
    if (tN0 > qp.tiles_per_pair) tN0 = qp.tiles_per_pair;
    qp.tN0 = tN0;
    qp.bg_count = bg_count;
    qp.scale = a.scale;
    qp.c = c;
    const dim3 qg((unsigned)((int64_t)qp.tiles_per_pair * qp.bg_count));
    if (a.d == 128) hipLaunchKernelGGL((attn_bwd_dq_kernel<128>), qg, dim3(kThreadsB), 0, s, qp);
    else hipLaunchKernelGGL((attn_bwd_dq_kernel<64>), qg, dim3(kThreadsB), 0, s, qp);
    return hipGetLastError();
}

}  // namespace mars
