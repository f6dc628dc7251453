// Training-layout attention over [prompt ; x ; x~] with the MARS structured mask
// ("MARS: Enabling Autoregressive Models Multi-Token Generation", §3.2 Eq. 2 and Fig. 2
// left; the prompt is a causal prefix seen by every response row).
//
// bf16 path (gfx950 MFMA):
//   * Rows: the G = Hq/Hkv query heads of one KV head are packed as rows (row u of a
//     (batch, kv head) pair = position u / G, head kvh*G + u % G), so every K/V tile a
//     workgroup stages in LDS serves G heads.  A workgroup owns 128 such rows (4 waves x
//     32 rows): small enough that the heaviest row tiles (the longest key ranges) finish
//     early when dispatched first, and light enough on registers for 4 (head_dim 64) or 3
//     (head_dim 128) waves per SIMD.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the K
//     tile is the A operand (read from LDS), the wave's Q rows the B operand (registers for
//     the whole kernel).  In the output layout a lane owns one query row and 16 of the 32
//     keys, its partner lane (l ^ 32) the other 16, so row max/sum need one permlane32 swap.
//   * O^T += V^T P^T: P^T comes straight from the score registers (bf16, RNE); V^T is read
//     from the natural [key][d] LDS tile with ds_read_b64_tr_b16 (transposing 16-bit read).
//   * K/V tiles reach LDS by global_load_lds_dwordx4 into a ring: 3 stages with one tile per
//     barrier at head_dim 128, 4 stages with two tiles per barrier at head_dim 64; 16-byte
//     chunks are XOR-swizzled per row so operand reads are conflict-free.
//   * Keys are walked in 32-key tiles over at most two intervals per workgroup (the union
//     of its rows' visible keys, see mars_device.h); each wave classifies every tile for its
//     own rows: skipped, computed with the element mask, or computed without it.
//   * Online softmax in the log2 domain, fp32 statistics, fp32 MFMA accumulation.  Q is
//     multiplied by scale*log2(e) and rounded to bf16 once per wave, so P = 2^(s - off)
//     costs one v_exp_f32 per element.  The per-row offset `off` stays 0 while a row's
//     scores are moderate (|first max| <= 64, no tile whose P sum passes 2^64): the QK MFMA
//     output is then exponentiated as it is, with no max and no subtraction.  Rows with
//     larger scores move their offset to their max (and rescale O) only when needed.
//   * Copy addresses: one wave-uniform base per tile (SGPRs) plus fixed per-lane offsets.
//   * Workgroup order: heaviest row tiles first (noisy and clean tiles from the far end,
//     interleaved, then the prompt); the (batch, kv head) index is the fastest-varying part
//     of the workgroup id, so the round-robin dispatch over the 8 XCDs keeps each pair's
//     K/V on few L2s.
//
// fp32 path: one thread per query row on the vector ALUs, fp32 throughout (for fp32
// inputs; a correctness path, not a tuned one).
#include <atomic>
#include <cmath>
#include <type_traits>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kWaves = 4;
constexpr int kNcb = 1;                              // 32-row column blocks per wave
constexpr int kRowsPerWave = 32 * kNcb;              // == kAttnRowBlock
constexpr int kRowsPerWG = kWaves * kRowsPerWave;    // 128
constexpr int kThreads = 64 * kWaves;               // workgroup size
constexpr int kKT = kAttnKeyBlock;                   // 32 keys per LDS tile
static_assert(kRowsPerWave == kAttnRowBlock, "row block");

struct AttnKParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int8_t* tilelog;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
    int hq, hkv, G, P, L, B, N;
    int rows_per_pair;   // N * G
    int tiles_per_pair;  // ceil(rows_per_pair / 256)
    int tN0;             // first row tile whose first row is a noisy position
    int bg_count;        // batch * hkv
    int key_tiles;       // ceil(N / 32)
    int row_groups;      // ceil(rows_per_pair / 32)
    int lead;            // lightest items dispatched first
    float scale_log2;    // scale * log2(e)
};


// K/V ring: 3 stages at head_dim 128, 4 at head_dim 64 (two tiles per barrier); one
// file-scope __shared__ object per stage, tensor and head_dim, so every access names its
// array directly (no generic pointers to LDS).
template <int D> constexpr int fwd_stages() { return D == 64 ? 4 : 3; }
__shared__ __attribute__((aligned(16))) uint16_t g_ak0_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_ak1_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_ak2_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_av0_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_av1_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_av2_128[kKT * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_ak0_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_ak1_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_ak2_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_av0_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_av1_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_av2_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_ak3_64[kKT * 64];
__shared__ __attribute__((aligned(16))) uint16_t g_av3_64[kKT * 64];

template <int D, int ST>
__device__ inline uint16_t* att_k() {
    if constexpr (D == 128) {
        if constexpr (ST == 0) return g_ak0_128;
        else if constexpr (ST == 1) return g_ak1_128;
        else return g_ak2_128;
    } else {
        if constexpr (ST == 0) return g_ak0_64;
        else if constexpr (ST == 1) return g_ak1_64;
        else if constexpr (ST == 2) return g_ak2_64;
        else return g_ak3_64;
    }
}
template <int D, int ST>
__device__ inline uint16_t* att_v() {
    if constexpr (D == 128) {
        if constexpr (ST == 0) return g_av0_128;
        else if constexpr (ST == 1) return g_av1_128;
        else return g_av2_128;
    } else {
        if constexpr (ST == 0) return g_av0_64;
        else if constexpr (ST == 1) return g_av1_64;
        else if constexpr (ST == 2) return g_av2_64;
        else return g_av3_64;
    }
}

template <int D, bool LOG>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 3) void attn_fwd_bf16_kernel(AttnKParams p) {
    constexpr int NC = D / 16;          // 16-wide d chunks of the QK^T contraction
    constexpr int NDB = D / 32;         // 32-row d blocks of O^T
    constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
    constexpr int kStages = fwd_stages<D>();
    constexpr int NINS = kKT * CPR / 64;            // 1 KB copy windows per tile and tensor
    constexpr int PERW = NINS / kWaves;             // windows per wave and tensor
    constexpr int GROUPW = 2 * PERW;                // copy instructions per wave and tile
    static_assert(D <= 128 && NINS % kWaves == 0 && PERW >= 1, "tile copy split");
    constexpr float kLazy = 32.f;   // shifted score that moves a started row's offset
    constexpr float kMod = 64.f;    // first max within +-kMod: the row keeps offset 0
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane & 31, g2 = lane >> 5;

    // Work item in heaviest-first order ((batch, kv head) fastest); the first p.lead
    // workgroups take the lightest items instead (see the launcher).
    const int nitems = p.tiles_per_pair * p.bg_count;
    const int gi = (int)blockIdx.x < p.lead ? nitems - p.lead + (int)blockIdx.x : (int)blockIdx.x - p.lead;
    const int bg = gi % p.bg_count;
    const int rank = gi / p.bg_count;
    const int tile = rank_to_tile(rank, p.tiles_per_pair, p.tN0);
    const int b = bg / p.hkv, g = bg % p.hkv;
    const int row0 = tile * kRowsPerWG;
    const int wrow0 = row0 + wave * kRowsPerWave;

    // This lane's query rows (one per column block).
    int pos[kNcb], head[kNcb];
    bool valid[kNcb];
    RowBounds rb[kNcb];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
        const int u = wrow0 + cb * 32 + hl;
        valid[cb] = u < p.rows_per_pair;
        const int uu = valid[cb] ? u : p.rows_per_pair - 1;
        pos[cb] = uu / p.G;
        head[cb] = g * p.G + uu % p.G;
        rb[cb] = row_bounds(pos[cb], p.P, p.L, p.B);
    }

    // Q^T operand: lane holds Q[row][16c + 8*g2 .. +7] for every chunk c.  The raw rows are
    // loaded here (padding rows read the clamped last row) and converted below, after the
    // first K/V copies are issued, so the two latencies overlap.
    typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
    u32x4_t qraw[kNcb][NC];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
        const uint16_t* qp = p.q + b * p.qs0 + (int64_t)pos[cb] * p.qs1 + (int64_t)head[cb] * p.qs2 + 8 * g2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) qraw[cb][cc] = *reinterpret_cast<const u32x4_t*>(qp + 16 * cc);
    }

    // Union of the workgroup's visible keys: [0, endA) and [startC, endC).
    const int u_last = min(row0 + kRowsPerWG, p.rows_per_pair) - 1;
    const int pf = row0 / p.G, pl = u_last / p.G;
    const int PL = p.P + p.L;
    int endA = 0, startC = 0, endC = 0;
    if (pf < PL) endA = min(pl, PL - 1) + 1;
    if (pl >= PL) {
        endA = max(endA, p.P + ((pl - PL) / p.B) * p.B);
        startC = PL + ((max(pf, PL) - PL) / p.B) * p.B;
        endC = pl + 1;
    }
    const int nA = (endA + kKT - 1) / kKT;
    int c0t = startC / kKT;
    const int c1t = (endC + kKT - 1) / kKT;
    if (c0t < nA) c0t = nA;
    const int nCt = c1t > c0t ? c1t - c0t : 0;
    const int ntiles = nA + nCt;
    auto tile_of = [&](int it) { return it < nA ? it : c0t + (it - nA); };

    const uint16_t* kbase = p.k + b * p.ks0 + (int64_t)g * p.ks2;
    const uint16_t* vbase = p.v + b * p.vs0 + (int64_t)g * p.vs2;

    // Copy of key tile kt into stage ST: this wave fills PERW 1 KB windows of K and of V.
    // Window slot (row r, position pos) holds logical chunk pos ^ swz(r) of key kt*32 + r;
    // rows past N repeat key N-1 (finite values; such keys are always masked).  The tile's
    // first key row is a wave-uniform base; the per-lane byte offsets are fixed.
    uint32_t kgo[PERW], vgo[PERW];
#pragma unroll
    for (int jj = 0; jj < PERW; ++jj) {
        const int slot = 64 * (wave * PERW + jj) + lane;
        const int r = slot / CPR, ps = slot % CPR;
        kgo[jj] = (uint32_t)(r * p.ks1 * 2 + 16 * (ps ^ swz_k<D>(r)));
        vgo[jj] = (uint32_t)(r * p.vs1 * 2 + 16 * (ps ^ swz_v<D>(r)));
    }
    // Copies are issued in walk order; kq / vq point at the first key row of the next tile
    // to copy (tile tile_of(nq)) and advance by one tile, or jump to the second interval.
    const int64_t tbk = (int64_t)kKT * p.ks1, tbv = (int64_t)kKT * p.vs1;
    const int nfull = p.N / kKT;        // tiles entirely inside [0, N)
    int nq = 0;
    const uint16_t* kq = kbase;
    const uint16_t* vq = vbase;
    if (nA == 0) {
        kq = kbase + c0t * tbk;
        vq = vbase + c0t * tbv;
    }
    auto issue = [&](auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const int kt = tile_of(nq);
        const int k0 = kt * kKT;
        const uint16_t* kb = kq;
        const uint16_t* vb = vq;
        ++nq;
        if (nq == nA) {
            kq = kbase + c0t * tbk;
            vq = vbase + c0t * tbv;
        } else {
            kq += tbk;
            vq += tbv;
        }
        if (kt < nfull) {
#pragma unroll
            for (int jj = 0; jj < PERW; ++jj) {
                const uint32_t w = lds_addr(att_k<D, ST>()) + 1024 * (wave * PERW + jj);
                dma16_sv(kb, kgo[jj], w);
                dma16_sv(vb, vgo[jj], lds_addr(att_v<D, ST>()) + 1024 * (wave * PERW + jj));
            }
        } else {
            const int last = p.N - 1 - k0;
#pragma unroll
            for (int jj = 0; jj < PERW; ++jj) {
                const int j = wave * PERW + jj;
                const int slot = 64 * j + lane;
                const int r = slot / CPR, ps = slot % CPR;
                const int rr = min(r, last);
                dma16_sv(kb, (uint32_t)(rr * p.ks1 * 2 + 16 * (ps ^ swz_k<D>(r))), lds_addr(att_k<D, ST>()) + 1024 * j);
                dma16_sv(vb, (uint32_t)(rr * p.vs1 * 2 + 16 * (ps ^ swz_v<D>(r))), lds_addr(att_v<D, ST>()) + 1024 * j);
            }
        }
    };

    // Online softmax state per row (log2 domain): off = offset subtracted from the raw
    // scores, l_run = this lane's share of sum 2^(s - off), acc = O^T on the same scale,
    // m_run = -inf until the row's first visible key.  The offset stays 0 while a row's
    // scores are moderate (first visible tile's max within +-kMod, no later tile pushing a
    // P sum past 2^64): the QK MFMA output is then used as it is, and only a wave holding a
    // shifted row (`shifted`) subtracts.  thr is the largest shifted score that keeps the
    // offset: kLazy once the row has started, -inf before.
    float m_run[kNcb], l_run[kNcb], thr[kNcb], off[kNcb];
    bool shifted = false;
    f32x16_t acc[kNcb][NDB];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
        thr[cb] = -INFINITY;
        off[cb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[cb][db][e] = 0.f;
        }
    }

    const bool wave_has_rows = wrow0 < p.rows_per_pair;
    int8_t* logrow = nullptr;
    if (LOG && wave_has_rows)
        logrow = p.tilelog + ((int64_t)bg * p.row_groups + wrow0 / kRowsPerWave) * p.key_tiles;

    // Per-lane LDS byte offsets of the MFMA operands (the same for every stage).  The
    // swizzle only permutes 16-byte chunks within a row, so chunk pair cc of K sits at
    // koff0 ^ (32 cc) and the V^T fragment of d block db at voff0 ^ (64 db); the key half
    // (kh) and 8-row half (hf) of a V fragment are plain additive offsets.
    const int koff0 = hl * (2 * D) + 16 * (g2 ^ swz_k<D>(hl));
    const int s16 = lane & 15, grp = lane >> 4;
    int voff0;
    {
        const int row = 4 * (grp >> 1) + (s16 >> 2);
        const int col = 16 * (grp & 1) + 4 * (s16 & 3);
        voff0 = row * (2 * D) + 16 * ((col >> 3) ^ swz_v<D>(row)) + 2 * (col & 7);
    }

    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v ones2 = {(__bf16)1.0f, (__bf16)1.0f};

    issue(S0{});
    if (ntiles > 1) issue(S1{});
    // Drain Q (and the first copies) before Q is used: the compiler does not count the
    // copies, so a Q wait left to it would land inside the loop as a full vmcnt(0).  The
    // scheduling barrier keeps the conversion below the copies.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    // Q multiplied by scale*log2(e) and rounded to bf16 once, so the MFMA yields scores in
    // the log2 domain (padding rows are zero).
    const float c = p.scale_log2;
    bf16x8_t qf[kNcb][NC];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            u32x4_t ws;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = valid[cb] ? qraw[cb][cc][j] : 0u;
                ws[j] = pack_bf16x2(__uint_as_float(w << 16) * c, __uint_as_float(w & 0xffff0000u) * c);
            }
            qf[cb][cc] = __builtin_bit_cast(bf16x8_t, ws);
        }
    }

    // Tile classes from the wave's row range.  The wave's valid rows are consecutive
    // positions p_lo..p_hi, so the union U and the intersection I of their visible key
    // sets are each at most two intervals:
    //   U = [0, U_hi) u [C0, p_hi]      (C0 = lo2 of the first noisy row; empty if none)
    //   I = [0, I_hi) u [I2lo, I2hi)    (the second part only when every row is noisy and
    //                                    in one block: its causal own-block prefix)
    // A tile is visited iff it meets U, and needs no element mask iff it lies inside I.
    int U_hi = 0, C0 = 0, Cend = 0, I_hi = 0, I2lo = 1, I2hi = 0;
    if (wave_has_rows) {
        const int u_hi = min(wrow0 + kRowsPerWave, p.rows_per_pair) - 1;
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
    // Class code of tile `it` (bit 0: visit, bit 1: no mask needed).
    auto tile_class = [&](const int it) __attribute__((always_inline)) {
        const int kb = tile_of(it) * kKT;
        const int ke = kb + kKT;
        const bool any = (kb < U_hi) || (kb < Cend && ke > C0);
        const bool all = (ke <= p.N) && (ke <= I_hi || (kb >= I2lo && ke <= I2hi));
        return (any ? 1 : 0) | (all ? 2 : 0);
    };
    // The codes of tiles lane + 64 j (j < 16) are precomputed, two bits each, in one
    // register per lane; the loop reads them back with v_readlane (tiles beyond 1024 are
    // classified on the spot).
    uint32_t cls_bits = 0;
    for (int j = 0; j < 16 && 64 * j < ntiles; ++j) {
        const int it = lane + 64 * j;
        if (it < ntiles) cls_bits |= (uint32_t)tile_class(it) << (2 * j);
    }

    // The computation of tile `it` from ring stage ST (its copy has landed).
    auto tile_body = [&](const int it, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;

        const int kt = tile_of(it);
        const int kb = kt * kKT;
        const int cls = it < 1024 ? (int)(__builtin_amdgcn_readlane(cls_bits, it & 63) >> (2 * (it >> 6))) & 3
                                  : __builtin_amdgcn_readfirstlane(tile_class(it));
        const bool wany = cls & 1, wall = cls & 2;
        if constexpr (LOG) {
            if (logrow && lane == 0 && wany) logrow[kt] = wall ? 2 : 1;
        }
        if (!wany) return;

        const char* kt_lds = reinterpret_cast<const char*>(att_k<D, ST>());
        const char* vt_lds = reinterpret_cast<const char*>(att_v<D, ST>());

        // S^T = K Q^T - m_run (log2 domain) for this wave's column blocks, then the element
        // mask on tiles that are not entirely visible.  Element e of this lane holds key
        // kb + 4*g2 + o(e), o(e) = 8*(e/4) + e%4.
        f32x16_t s[kNcb];
        auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt_lds + (koff0 ^ (32 * cc)));
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb)
                    s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[cb][cc], cc == 0 ? f32x16_t{} : s[cb], 0, 0, 0);
            }
            if (shifted) {
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) s[cb][e] -= off[cb];
                }
            }
            if (!wall) {
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb) {
                    // Bit o of vis: key kb + o is visible to this lane's row (o < 32).
                    const int A = rb[cb].hi1 - kb, Lo = rb[cb].lo2 - kb, Hi = pos[cb] - kb;
                    auto low = [](int x) __attribute__((always_inline)) {
                        return x >= 32 ? 0xffffffffu : (1u << max(x, 0)) - 1u;
                    };
                    const uint32_t vis = (low(A) | (low(Hi + 1) & ~low(Lo))) >> (4 * g2);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int o = 8 * (e >> 2) + (e & 3);
                        const uint32_t t = (uint32_t)((int32_t)(vis << (31 - o)) >> 31);  // all ones iff visible
                        s[cb][e] = __uint_as_float((__float_as_uint(s[cb][e]) & t) | (0xff800000u & ~t));
                    }
                }
            }
        };
        scores();
        // V^T fragments of this tile.  Head_dim 64 reads them now (into the registers the K
        // fragments just released) so that their LDS latency overlaps the softmax below;
        // head_dim 128 reads them just before P V, which keeps the kernel within 168 VGPRs
        // (three waves per SIMD, whose interleaving hides that latency instead).
        bf16x8_t va[NDB][2];
        auto read_v = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const char* vb = vt_lds + (voff0 ^ (64 * db));
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(vb + kh * 16 * (2 * D)));
                const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(vb + kh * 16 * (2 * D) + 8 * (2 * D)));
                va[db][kh] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        };
        if constexpr (D == 64) read_v();
        // Lazy rescale.  The row max is computed while some row of the wave has no finite
        // running max yet (its first visible keys), or when this tile's P could overflow:
        // P = 2^s is formed first and its row sum checked against 2^64, which bounds every
        // term of acc and l far from the fp32 limit.  Otherwise scores above the running
        // max just give P > 1, which bf16 and the fp32 accumulators hold exactly as well.
        auto rescale = [&]() __attribute__((always_inline)) {
            float mx[kNcb];
            bool need = false;
#pragma unroll
            for (int cb = 0; cb < kNcb; ++cb) {
                float m = fmaxf(fmaxf(fmaxf(s[cb][0], s[cb][1]), fmaxf(s[cb][2], s[cb][3])),
                                fmaxf(fmaxf(s[cb][4], s[cb][5]), fmaxf(s[cb][6], s[cb][7])));
                m = fmaxf(m, fmaxf(fmaxf(fmaxf(s[cb][8], s[cb][9]), fmaxf(s[cb][10], s[cb][11])),
                                   fmaxf(fmaxf(s[cb][12], s[cb][13]), fmaxf(s[cb][14], s[cb][15]))));
                mx[cb] = half_swap_max(m);
                need |= mx[cb] > thr[cb];
            }
            if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
                // acc is still all zero while every row of the wave has m_run = -inf.
                bool started = false;
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb) started |= m_run[cb] != -INFINITY;
                started = __builtin_amdgcn_ballot_w64(started) != 0ull;
                bool any_off = false;
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb) {
                    if (mx[cb] > thr[cb]) {
                        // New offset: the row's max raw score in this tile, or 0 for a row
                        // starting with a moderate max.  A started row rescales its sums.
                        const float mnew = off[cb] + mx[cb];
                        const bool first = m_run[cb] == -INFINITY;
                        const float noff = (first && fabsf(mnew) <= kMod) ? 0.f : mnew;
                        const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(off[cb] - noff);
                        l_run[cb] *= alpha;
                        if (started) {
                            // One 16-register block at a time (scheduling barriers), so the
                            // rescale never needs all accumulators in flight at once.
#pragma unroll
                            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                                for (int e = 0; e < 16; ++e) acc[cb][db][e] *= alpha;
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                        const float delta = noff - off[cb];
#pragma unroll
                        for (int e = 0; e < 16; ++e) s[cb][e] -= delta;
                        off[cb] = noff;
                        m_run[cb] = mnew;
                        thr[cb] = kLazy;
                    }
                    any_off |= off[cb] != 0.f;
                }
                shifted = __builtin_amdgcn_ballot_w64(any_off) != 0ull;
            }
        };
        bf16x8_t pb[kNcb][2];
        float lt[kNcb];
        // P = 2^s in bf16 and its row sum (of the rounded P, dot2 with ones).
        auto make_p = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < kNcb; ++cb) {
                float pv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) pv[e] = __builtin_amdgcn_exp2f(s[cb][e]);
                float lsum = 0.f;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    // Scalar temporaries: element reads of a partially built vector in this
                    // unrolled loop were miscompiled (every dot2 read element 0).
                    const uint32_t w0 = pack_bf16x2(pv[8 * kh + 0], pv[8 * kh + 1]);
                    const uint32_t w1 = pack_bf16x2(pv[8 * kh + 2], pv[8 * kh + 3]);
                    const uint32_t w2 = pack_bf16x2(pv[8 * kh + 4], pv[8 * kh + 5]);
                    const uint32_t w3 = pack_bf16x2(pv[8 * kh + 6], pv[8 * kh + 7]);
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w0), ones2, lsum, false);
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w1), ones2, lsum, false);
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w2), ones2, lsum, false);
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w3), ones2, lsum, false);
                    typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
                    const u32x4_t w = {w0, w1, w2, w3};
                    pb[cb][kh] = __builtin_bit_cast(bf16x8_t, w);
                }
                lt[cb] = lsum;
            }
        };
        bool fresh = false;
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb) fresh |= m_run[cb] == -INFINITY;
        fresh = __builtin_amdgcn_ballot_w64(fresh) != 0ull;
        if (fresh) rescale();
        make_p();
        if (!fresh) {
            bool big = false;
#pragma unroll
            for (int cb = 0; cb < kNcb; ++cb) big |= !(lt[cb] <= 0x1p64f);
            if (__builtin_amdgcn_ballot_w64(big) != 0ull) {
                // Rare: the scores are formed again (the tile is still in LDS) rather than
                // kept alive next to P.
                scores();
                rescale();
                make_p();
            }
        }
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb) l_run[cb] += lt[cb];
        if constexpr (D == 128) read_v();
        // O^T += V^T P^T.
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int cb = 0; cb < kNcb; ++cb)
                    acc[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][kh], pb[cb][kh], acc[cb][db], 0, 0, 0);
            }
        }
    };

    if constexpr (D == 128) {
        // One tile per barrier: tile `it` is the oldest copy group in flight; once every wave
        // has it, the barrier also guarantees that the stage read for tile it-1 is free for
        // tile it+2.
        auto body = [&](const int it, auto stage) __attribute__((always_inline)) {
            constexpr int ST = decltype(stage)::value;
            if (it + 1 < ntiles) wait_vmcnt<GROUPW>();
            else wait_vmcnt<0>();
            __syncthreads();
            if (it + 2 < ntiles) issue(std::integral_constant<int, (ST + 2) % kStages>{});
            tile_body(it, stage);
        };
        for (int t0 = 0; t0 < ntiles; t0 += kStages) {
            body(t0, S0{});
            if (t0 + 1 < ntiles) body(t0 + 1, S1{});
            if (t0 + 2 < ntiles) body(t0 + 2, S2{});
        }
    } else {
        // Two tiles per barrier: tiles it and it+1 landed (issued before the previous
        // barrier); tiles it+2 and it+3 go into the stages tiles it-2 and it-1 used.
        auto body2 = [&](const int it, auto stage) __attribute__((always_inline)) {
            constexpr int ST = decltype(stage)::value;
            wait_vmcnt<0>();
            __syncthreads();
            if (it + 2 < ntiles) issue(std::integral_constant<int, (ST + 2) % kStages>{});
            if (it + 3 < ntiles) issue(std::integral_constant<int, (ST + 3) % kStages>{});
            tile_body(it, stage);
            if (it + 1 < ntiles) tile_body(it + 1, std::integral_constant<int, ST + 1>{});
        };
        for (int t0 = 0; t0 < ntiles; t0 += kStages) {
            body2(t0, S0{});
            if (t0 + 2 < ntiles) body2(t0 + 2, S2{});
        }
    }

    // Epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2.
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
        const float lt = half_swap_sum(l_run[cb]);
        const float inv = 1.f / lt;
        if (valid[cb]) {
            uint16_t* op = p.o + b * p.os0 + (int64_t)pos[cb] * p.os1 + (int64_t)head[cb] * p.os2;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int d = 32 * db + 8 * bb + 4 * g2;
                    uint2 w;
                    w.x = pack_bf16x2(acc[cb][db][4 * bb + 0] * inv, acc[cb][db][4 * bb + 1] * inv);
                    w.y = pack_bf16x2(acc[cb][db][4 * bb + 2] * inv, acc[cb][db][4 * bb + 3] * inv);
                    *reinterpret_cast<uint2*>(op + d) = w;
                }
            }
            if (p.lse && g2 == 0)
                p.lse[((int64_t)b * p.hq + head[cb]) * p.N + pos[cb]] = (off[cb] + log2f(lt)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------------------
// fp32 vector path: thread = query row; grid (ceil(N/64), Hq, batch).
// ---------------------------------------------------------------------------------------
struct AttnF32Params {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* lse;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
    int hq, G, P, L, B, N;
    float scale;
};

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnF32Params p) {
    // One 64-lane workgroup per 64 consecutive positions of one (batch, head), a row per
    // lane.  The workgroup walks the 64-key tiles of the union of its rows' two key intervals
    // ([0, hi1) and [lo2, r]), staged in LDS and read by broadcast; each lane forms dot
    // products only for the keys its own row sees (exact fp32, online softmax).
    constexpr int KT = 64;
    __shared__ float sk[KT][D];
    __shared__ float sv[KT][D];
    const int r0 = blockIdx.x * 64;
    const int r = r0 + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z, g = h / p.G;
    const bool valid = r < p.N;
    const int rr = valid ? r : p.N - 1;
    const RowBounds rb = row_bounds(rr, p.P, p.L, p.B);

    // Tiles of the workgroup's key union: [0, ahi) and [clo, chi).
    int ahi = rb.hi1, clo = rb.lo2 <= rr ? rb.lo2 : 0x7fffffff, chi = rb.lo2 <= rr ? rr + 1 : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        ahi = max(ahi, __shfl_xor(ahi, m));
        clo = min(clo, __shfl_xor(clo, m));
        chi = max(chi, __shfl_xor(chi, m));
    }
    const int nA = (ahi + KT - 1) / KT;
    const int c0 = clo < chi ? max(clo / KT, nA) : nA;
    const int c1 = clo < chi ? (chi + KT - 1) / KT : nA;
    const int ntiles = nA + (c1 > c0 ? c1 - c0 : 0);

    float q[D], acc[D];
    const float* qp = p.q + b * p.qs0 + (int64_t)rr * p.qs1 + (int64_t)h * p.qs2;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = qp[d];
        acc[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const float* kb = p.k + b * p.ks0 + (int64_t)g * p.ks2;
    const float* vb = p.v + b * p.vs0 + (int64_t)g * p.vs2;
    for (int ti = 0; ti < ntiles; ++ti) {
        const int k0 = (ti < nA ? ti : c0 + (ti - nA)) * KT;
        __syncthreads();   // the previous tile's readers are done
        {
            const int j = min(k0 + (int)threadIdx.x, p.N - 1);
            const float* kp = kb + (int64_t)j * p.ks1;
            const float* vp = vb + (int64_t)j * p.vs1;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                sk[threadIdx.x][d] = kp[d];
                sv[threadIdx.x][d] = vp[d];
            }
        }
        __syncthreads();
        const int kend = min(KT, p.N - k0);
        for (int jj = 0; jj < kend; ++jj) {
            const int j = k0 + jj;
            if (!key_visible(rr, j, rb)) continue;
            float sdot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) sdot = fmaf(q[d], sk[jj][d], sdot);
            const float sc = sdot * p.scale;
            const float mnew = fmaxf(m, sc);
            const float alpha = expf(m - mnew);
            const float pj = expf(sc - mnew);
            l = fmaf(l, alpha, pj);
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], alpha, pj * sv[jj][d]);
            m = mnew;
        }
    }
    if (valid) {
        float* op = p.o + b * p.os0 + (int64_t)r * p.os1 + (int64_t)h * p.os2;
        const float inv = 1.f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
        if (p.lse) p.lse[((int64_t)b * p.hq + h) * p.N + r] = m + logf(l);
    }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t s) {
    AttnKParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.tilelog = a.tilelog;
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.vs0 = a.vs[0]; p.vs1 = a.vs[1]; p.vs2 = a.vs[2];
    p.os0 = a.os[0]; p.os1 = a.os[1]; p.os2 = a.os[2];
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.P = a.P;
    p.L = a.L;
    p.B = a.B;
    p.N = a.N;
    p.rows_per_pair = a.N * p.G;
    p.tiles_per_pair = (p.rows_per_pair + kRowsPerWG - 1) / kRowsPerWG;
    const int64_t noisy_row0 = (int64_t)(a.P + a.L) * p.G;
    int tN0 = (int)((noisy_row0 + kRowsPerWG - 1) / kRowsPerWG);
    if (tN0 > p.tiles_per_pair) tN0 = p.tiles_per_pair;
    p.tN0 = tN0;
    p.bg_count = a.batch * a.hkv;
    p.key_tiles = (a.N + kKT - 1) / kKT;
    p.row_groups = (p.rows_per_pair + kRowsPerWave - 1) / kRowsPerWave;
    p.scale_log2 = a.scale * kLog2e;
    const int64_t grid = (int64_t)p.tiles_per_pair * p.bg_count;
    if (grid == 0) return hipSuccess;
    // When the grid is a little larger than what is resident at once, the items that do not
    // fit would start only when a first-round workgroup ends (late: the oldest waves have
    // issue priority).  Those lightest items are dispatched first instead; they finish
    // early and their slots take the rest.
    // Resident-slot count per (head_dim, device), computed once; atomics because callers
    // on several host threads may race to fill it (they all store the same value).
    static std::atomic<int> slot_cache[2][64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int di = a.d == 128 ? 1 : 0;
    int slots = (dev >= 0 && dev < 64) ? slot_cache[di][dev].load(std::memory_order_relaxed) : 0;
    if (slots <= 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = a.d == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_bf16_kernel<128, false>, kThreads, 0)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_bf16_kernel<64, false>, kThreads, 0);
        if (e != hipSuccess) return e;
        slots = cus * (per_cu > 0 ? per_cu : 1);
        if (dev >= 0 && dev < 64) slot_cache[di][dev].store(slots, std::memory_order_relaxed);
    }
    p.lead = (grid > slots && grid < 2 * (int64_t)slots) ? (int)(grid - slots) : 0;
    const dim3 g((unsigned)grid), blk(kThreads);
    if (a.d == 128) {
        if (p.tilelog) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), g, blk, 0, s, p);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), g, blk, 0, s, p);
    } else {
        if (p.tilelog) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), g, blk, 0, s, p);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), g, blk, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t s) {
    AttnF32Params p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.o = static_cast<float*>(a.o);
    p.lse = a.lse;
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.vs0 = a.vs[0]; p.vs1 = a.vs[1]; p.vs2 = a.vs[2];
    p.os0 = a.os[0]; p.os1 = a.os[1]; p.os2 = a.os[2];
    p.hq = a.hq;
    p.G = a.hq / a.hkv;
    p.P = a.P;
    p.L = a.L;
    p.B = a.B;
    p.N = a.N;
    p.scale = a.scale;
    if (a.N == 0 || a.batch == 0) return hipSuccess;
    dim3 grid((a.N + 63) / 64, a.hq, a.batch);
    if (a.d == 128) {
        hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(64), 0, s, p);
    } else {
        hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace mars
