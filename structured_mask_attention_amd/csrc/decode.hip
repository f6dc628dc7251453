// Sliding-window decode step ("MARS: Enabling Autoregressive Models Multi-Token
// Generation", Fig. 2 right): W window rows per sequence attend to the sequence's KV
// cache [0, len) and, causally and self-inclusively, to the window rows 0..i.
//
// Two kernels on the caller's stream:
//   1. split: one wave per (sequence, kv head, CH-key cache chunk).  The G*W query rows
//      of a kv head (G = Hq/Hkv query heads x W window rows, <= 64) form one or two
//      32-column MFMA blocks; S^T = K Q^T (K tile read from LDS as the A operand), online
//      softmax, O^T += V^T P^T (V read back transposed with ds_read_b64_tr_b16).  K and V
//      32-key steps stream into a 3-stage LDS ring by global_load_lds_dwordx4 (two steps
//      in flight; a wave-uniform base per step plus fixed per-lane offsets).  Each chunk
//      writes an unnormalised partial (acc, m, l) to the workspace.
//   2. combine: one workgroup per (sequence, query head): the window keys (at most W dot
//      products per row) and a log-sum-exp merge of the chunk partials.
// Chunks past a sequence's length exit at once, so the grid is fixed while the work is
// ragged; the cache is read exactly once.
#include <atomic>
#include <cmath>
#include <type_traits>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kCH = kDecodeChunk;   // cache keys per split workgroup
constexpr int kStep = 32;     // keys per MFMA step
constexpr int kStages = 3;    // LDS ring depth of the split kernel

struct DecodeKParams {
    const uint16_t* qw;
    const uint16_t* kw;
    const uint16_t* vw;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* cache_len;
    uint16_t* o;
    float* ws_acc;  // [batch*hkv][nchunk][R][D]
    float* ws_ml;   // [batch*hkv][nchunk][R][2]
    int64_t qws0, qws1, qws2, kws0, kws1, kws2, vws0, vws1, vws2;
    int64_t kcs0, kcs1, kcs2, vcs0, vcs1, vcs2, os0, os1, os2;
    int hq, hkv, G, W, R, cap, nchunk;
    float scale_log2;
};

__device__ inline int clamp_len(int len, int cap) { return len < 0 ? 0 : (len > cap ? cap : len); }

// LDS ring of the split kernel: one __shared__ object per stage and tensor (sized for
// D = 128), named directly at every access so no generic pointer to LDS is ever formed and
// the compiler's LDS-DMA wait tracking keeps the in-flight stages apart.
__shared__ __attribute__((aligned(16))) uint16_t g_dk0[kStep * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_dk1[kStep * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_dk2[kStep * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_dv0[kStep * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_dv1[kStep * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_dv2[kStep * 128];

template <int ST>
__device__ inline uint16_t* dec_k() {
    if constexpr (ST == 0) return g_dk0;
    else if constexpr (ST == 1) return g_dk1;
    else return g_dk2;
}
template <int ST>
__device__ inline uint16_t* dec_v() {
    if constexpr (ST == 0) return g_dv0;
    else if constexpr (ST == 1) return g_dv1;
    else return g_dv2;
}

template <int D, int NCB>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeKParams p) {
    constexpr int NC = D / 16;                 // 16-wide d chunks of the QK^T contraction
    constexpr int NDB = D / 32;                // 32-row d blocks of O^T
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int NINS = kStep * CPR / 64;     // 1 KB DMA instructions per tile (per tensor)
    constexpr int GROUP = 2 * NINS;            // DMA instructions per step (K and V)
    constexpr float kLazy = 8.f;
    static_assert(D <= 128, "ring sized for head_dim <= 128");

    // Grid: x = (sequence, kv head) pair, y = chunk.  With x fastest, every pair's chunk 0
    // is dispatched first, then chunk 1, ...: the chunks that exist (most have small c)
    // spread over all CUs instead of piling up behind the empty ones.
    const int c = blockIdx.y, b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv;
    const int len = clamp_len(p.cache_len[b], p.cap);
    const int k_begin = c * kCH;
    if (k_begin >= len) return;
    const int k_end = min(len, k_begin + kCH);
    const int nsteps = (k_end - k_begin + kStep - 1) / kStep;

    const int lane = threadIdx.x;
    const int hl = lane & 31, g2 = lane >> 5;

    const uint16_t* kbase = p.kc + b * p.kcs0 + (int64_t)g * p.kcs1;
    const uint16_t* vbase = p.vc + b * p.vcs0 + (int64_t)g * p.vcs1;

    // DMA of step `step` into stage arrays (sk, sv): slot (row r, position pos) holds logical
    // chunk pos ^ swz(r) of key k0 + r (keys past the chunk end repeat its last key; they are
    // masked to -inf, and repeating a real row keeps V finite).
    // Per-lane byte offsets of the copy windows relative to the step's first key row
    // (row r of window j = (64 j + lane) / CPR); the step base is a uniform pointer.
    uint32_t ko[NINS], vo[NINS];
#pragma unroll
    for (int j = 0; j < NINS; ++j) {
        const int slot = 64 * j + lane;
        const int r = slot / CPR, pos = slot % CPR;
        ko[j] = (uint32_t)(r * p.kcs2 * 2 + 16 * (pos ^ swz_k<D>(r)));
        vo[j] = (uint32_t)(r * p.vcs2 * 2 + 16 * (pos ^ swz_v<D>(r)));
    }
    auto issue = [&](int step, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const int k0 = k_begin + step * kStep;
        const uint16_t* kb = kbase + (int64_t)k0 * p.kcs2;
        const uint16_t* vb = vbase + (int64_t)k0 * p.vcs2;
        if (__builtin_amdgcn_readfirstlane(k0 + kStep <= k_end ? 1 : 0)) {
#pragma unroll
            for (int j = 0; j < NINS; ++j) {
                dma16_sv(kb, ko[j], lds_addr(dec_k<ST>()) + 1024 * j);
                dma16_sv(vb, vo[j], lds_addr(dec_v<ST>()) + 1024 * j);
            }
        } else {
            // Last, partial step of the chunk: rows past the end repeat the last key.
            const int last = k_end - 1 - k0;
#pragma unroll
            for (int j = 0; j < NINS; ++j) {
                const int slot = 64 * j + lane;
                const int r = slot / CPR, pos = slot % CPR;
                const int rr = min(r, last);
                dma16_sv(kb, (uint32_t)(rr * p.kcs2 * 2 + 16 * (pos ^ swz_k<D>(r))), lds_addr(dec_k<ST>()) + 1024 * j);
                dma16_sv(vb, (uint32_t)(rr * p.vcs2 * 2 + 16 * (pos ^ swz_v<D>(r))), lds_addr(dec_v<ST>()) + 1024 * j);
            }
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    // Query rows u = i*G + hh (window row i, query head g*G + hh): the B operand, in registers.
    bf16x8_t qf[NCB][NC];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int u = cb * 32 + hl;
        const bool ok = u < p.R;
        const int uu = ok ? u : 0;
        const uint16_t* qp = p.qw + b * p.qws0 + (int64_t)(uu / p.G) * p.qws1 +
                             (int64_t)(g * p.G + uu % p.G) * p.qws2 + 8 * g2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
            qf[cb][cc] = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 16 * cc) : bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
    issue(0, S0{});
    if (nsteps > 1) issue(1, S1{});
    // Drain the Q loads (issued before the copies, so their latencies overlap) here: the
    // compiler does not count the copies, so a Q wait left to it inside the loop would
    // become a full vmcnt(0).
    wait_vmcnt<0>();

    float m_run[NCB], l_run[NCB];
    f32x16_t acc[NCB][NDB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[cb][db][e] = 0.f;
        }
    }
    const float csc = p.scale_log2;
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v ones2 = {(__bf16)1.0f, (__bf16)1.0f};

    // Per-lane LDS byte offsets of the MFMA operands (independent of the stage).
    int koff[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) koff[cc] = hl * (2 * D) + 16 * ((2 * cc + g2) ^ swz_k<D>(hl));
    const int s16 = lane & 15, grp = lane >> 4;
    int voff[NDB][2][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 16 * kh + 8 * hf + 4 * (grp >> 1) + (s16 >> 2);
                const int col = 32 * db + 16 * (grp & 1) + 4 * (s16 & 3);
                voff[db][kh][hf] = row * (2 * D) + 16 * ((col >> 3) ^ swz_v<D>(row)) + 2 * (col & 7);
            }
        }
    }

    // One step on stage (ks, vs); step + 2 is issued into (nk, nv), the stage step - 1 used.
    auto body = [&](const int step, auto stage) __attribute__((always_inline)) {
                constexpr int ST = decltype(stage)::value;
                // Keep two steps in flight, then wait until this step's DMA group has landed.
                const int ahead = nsteps - 1 - step;   // groups issued after this one
                if (ahead >= 2) {
                    issue(step + 2, std::integral_constant<int, (ST + 2) % kStages>{});
                    wait_vmcnt<2 * GROUP>();
                } else if (ahead == 1) {
                    wait_vmcnt<GROUP>();
                } else {
                    wait_vmcnt<0>();
                }
                __syncthreads();
                const char* kt = reinterpret_cast<const char*>(dec_k<ST>());
                const char* vt = reinterpret_cast<const char*>(dec_v<ST>());
                const int k0 = k_begin + step * kStep;

                f32x16_t s[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) s[cb][e] = 0.f;
                }
#pragma unroll
                for (int cc = 0; cc < NC; ++cc) {
                    const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + koff[cc]);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[cb][cc], s[cb], 0, 0, 0);
                }
                if (__builtin_amdgcn_readfirstlane(k0 + kStep > k_end ? 1 : 0)) {
                    const int lim = k_end - k0 - 4 * g2;   // element o is a key iff o < lim
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int o = 8 * (e >> 2) + (e & 3);
                            s[cb][e] = (o < lim) ? s[cb][e] : -INFINITY;
                        }
                    }
                }
                float mx[NCB];
                bool need = false;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    float m = fmaxf(fmaxf(fmaxf(s[cb][0], s[cb][1]), fmaxf(s[cb][2], s[cb][3])),
                                    fmaxf(fmaxf(s[cb][4], s[cb][5]), fmaxf(s[cb][6], s[cb][7])));
                    m = fmaxf(m, fmaxf(fmaxf(fmaxf(s[cb][8], s[cb][9]), fmaxf(s[cb][10], s[cb][11])),
                                       fmaxf(fmaxf(s[cb][12], s[cb][13]), fmaxf(s[cb][14], s[cb][15]))));
                    mx[cb] = half_swap_max(m) * csc;
                    need |= mx[cb] > m_run[cb] + kLazy;
                }
                if (__builtin_amdgcn_readfirstlane(__ballot(need) != 0ull ? 1 : 0)) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const float mnew = fmaxf(m_run[cb], mx[cb]);
                        if (mnew > m_run[cb]) {
                            const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - mnew);
                            l_run[cb] *= alpha;
#pragma unroll
                            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                                for (int e = 0; e < 16; ++e) acc[cb][db][e] *= alpha;
                            }
                            m_run[cb] = mnew;
                        }
                    }
                }
                bf16x8_t pb[NCB][2];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const float msafe = (m_run[cb] == -INFINITY) ? 0.f : m_run[cb];
                    float pv[16];
#pragma unroll
                    for (int e = 0; e < 16; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[cb][e], csc, -msafe));
                    float lsum = l_run[cb];
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
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
                    l_run[cb] = lsum;
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
                        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(vt + voff[db][kh][0]));
                        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(vt + voff[db][kh][1]));
                        const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            acc[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[cb][kh], acc[cb][db], 0, 0, 0);
                    }
                }
                __syncthreads();   // this stage is refilled two steps later
    };
    for (int t0 = 0; t0 < nsteps; t0 += kStages) {
        body(t0, S0{});
        if (t0 + 1 < nsteps) body(t0 + 1, S1{});
        if (t0 + 2 < nsteps) body(t0 + 2, S2{});
    }

    // Unnormalised partial of this chunk.
    const int64_t slot = ((int64_t)(b * p.hkv + g) * p.nchunk + c) * p.R;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int u = cb * 32 + hl;
        const float lt = half_swap_sum(l_run[cb]);
        if (u < p.R) {
            float* ap = p.ws_acc + (slot + u) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    float4 w = {acc[cb][db][4 * bb + 0], acc[cb][db][4 * bb + 1], acc[cb][db][4 * bb + 2],
                                acc[cb][db][4 * bb + 3]};
                    *reinterpret_cast<float4*>(ap + 32 * db + 8 * bb + 4 * g2) = w;
                }
            }
            if (g2 == 0) {
                p.ws_ml[(slot + u) * 2 + 0] = m_run[cb];
                p.ws_ml[(slot + u) * 2 + 1] = lt;
            }
        }
    }
}

// DPT consecutive bf16 (DPT = 4 or 2) of one row, as fp32.
template <int DPT>
struct BfRow {
    uint32_t w[DPT / 2];
    __device__ inline void load(const uint16_t* src) {
        if constexpr (DPT == 4) {
            const uint2 q = *reinterpret_cast<const uint2*>(src);
            w[0] = q.x;
            w[1] = q.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(src);
        }
    }
    __device__ inline float operator[](int e) const {
        const uint32_t x = w[e >> 1];
        return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    }
};

// One 256-thread workgroup per (sequence, kv head, group of 8 query rows u = i*G + hh);
// 32 threads per row, each owning D/32 consecutive output columns.  The chunk partials
// and then the window keys 0..i (dot products reduced over the row's 32 threads) are
// merged online (max, rescale, accumulate), in batches of kPre whose loads are all issued
// before any of them is used.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeKParams p) {
    constexpr int DPT = D / 32;   // columns per thread (4 or 2)
    constexpr int kPre = 8;       // chunk partials / window rows fetched per batch
    const int rg = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x;
    const int u = rg * 8 + (t >> 5);
    const int l32 = t & 31;
    if (u >= p.R) return;   // whole 32-lane groups exit together; no barriers below
    const int i = u / p.G, h = g * p.G + u % p.G;
    const int len = clamp_len(p.cache_len[b], p.cap);
    const int nch = (len + kCH - 1) / kCH;
    const int d0 = l32 * DPT;

    BfRow<DPT> qv;
    qv.load(p.qw + b * p.qws0 + (int64_t)i * p.qws1 + (int64_t)h * p.qws2 + d0);
    // Chunk partials (unnormalised acc, running max m, sum l) and window rows are fetched
    // in batches of kPre; the first batch of each is issued before anything is used.
    const int64_t slot0 = ((int64_t)(b * p.hkv + g) * p.nchunk) * p.R + u;
    float a[kPre][DPT];
    float2 ml[kPre];
    auto load_chunks = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int64_t sl = slot0 + (int64_t)min(c0 + k, nch - 1) * p.R;
            ml[k] = *reinterpret_cast<const float2*>(p.ws_ml + sl * 2);
            if constexpr (DPT == 4) {
                const float4 q = *reinterpret_cast<const float4*>(p.ws_acc + sl * D + d0);
                a[k][0] = q.x; a[k][1] = q.y; a[k][2] = q.z; a[k][3] = q.w;
            } else {
                const float2 q = *reinterpret_cast<const float2*>(p.ws_acc + sl * D + d0);
                a[k][0] = q.x; a[k][1] = q.y;
            }
        }
    };
    if (nch > 0) load_chunks(0);
    BfRow<DPT> kr[kPre], vr[kPre];
    auto load_window = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int j = min(j0 + k, i);
            kr[k].load(p.kw + b * p.kws0 + (int64_t)j * p.kws1 + (int64_t)g * p.kws2 + d0);
            vr[k].load(p.vw + b * p.vws0 + (int64_t)j * p.vws1 + (int64_t)g * p.vws2 + d0);
        }
    };
    load_window(0);

    float M = -INFINITY, den = 0.f;
    float num[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) num[e] = 0.f;
    auto merge = [&](float mj, float lj, const float (&aj)[DPT]) __attribute__((always_inline)) {
        const float Mn = fmaxf(M, mj);
        const float r0 = __builtin_amdgcn_exp2f(M - Mn), rj = __builtin_amdgcn_exp2f(mj - Mn);
        den = den * r0 + lj * rj;
#pragma unroll
        for (int e = 0; e < DPT; ++e) num[e] = num[e] * r0 + aj[e] * rj;
        M = Mn;
    };

    for (int c0 = 0; c0 < nch; c0 += kPre) {
        if (c0 > 0) load_chunks(c0);
#pragma unroll
        for (int k = 0; k < kPre; ++k)
            if (c0 + k < nch) merge(ml[k].x, ml[k].y, a[k]);
    }

    // Window keys 0..i of this sequence (causal, self-inclusive).
    for (int j0 = 0; j0 <= i; j0 += kPre) {
        if (j0 > 0) load_window(j0);
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            if (j0 + k > i) break;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < DPT; ++e) part = fmaf(qv[e], kr[k][e], part);
            part = sum32(part);
            float vj[DPT];
#pragma unroll
            for (int e = 0; e < DPT; ++e) vj[e] = vr[k][e];
            merge(part * p.scale_log2, 1.f, vj);
        }
    }
    const float inv = 1.f / den;
    uint16_t* op = p.o + b * p.os0 + (int64_t)i * p.os1 + (int64_t)h * p.os2 + d0;
#pragma unroll
    for (int e = 0; e < DPT; e += 2) {
        const uint32_t pk = pack_bf16x2(num[e] * inv, num[e + 1] * inv);
        *reinterpret_cast<uint32_t*>(op + e) = pk;
    }
}

}  // namespace

// Scratch of the allocation-free decode step: the chunk partials of one call, on each device
// the library runs on (held until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address hipGetSymbolAddress reports for the
// current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

size_t decode_workspace_bytes(int batch, int hkv, int G, int W, int d, int cap) {
    const int64_t nchunk = (cap + kCH - 1) / kCH;
    const int64_t R = (int64_t)G * W;
    return (size_t)((int64_t)batch * hkv * nchunk * R * (d + 2) * (int64_t)sizeof(float));
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    DecodeKParams p;
    p.qw = static_cast<const uint16_t*>(a.qw);
    p.kw = static_cast<const uint16_t*>(a.kw);
    p.vw = static_cast<const uint16_t*>(a.vw);
    p.kc = static_cast<const uint16_t*>(a.kc);
    p.vc = static_cast<const uint16_t*>(a.vc);
    p.cache_len = a.cache_len;
    p.o = static_cast<uint16_t*>(a.o);
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.W = a.W;
    p.R = p.G * a.W;
    p.cap = a.cap;
    p.nchunk = (a.cap + kCH - 1) / kCH;
    const int64_t acc_elems = (int64_t)a.batch * a.hkv * p.nchunk * p.R * a.d;
    p.ws_acc = static_cast<float*>(a.ws);
    p.ws_ml = p.ws_acc + acc_elems;
    p.qws0 = a.qws[0]; p.qws1 = a.qws[1]; p.qws2 = a.qws[2];
    p.kws0 = a.kws[0]; p.kws1 = a.kws[1]; p.kws2 = a.kws[2];
    p.vws0 = a.vws[0]; p.vws1 = a.vws[1]; p.vws2 = a.vws[2];
    p.kcs0 = a.kcs[0]; p.kcs1 = a.kcs[1]; p.kcs2 = a.kcs[2];
    p.vcs0 = a.vcs[0]; p.vcs1 = a.vcs[1]; p.vcs2 = a.vcs[2];
    p.os0 = a.os[0]; p.os1 = a.os[1]; p.os2 = a.os[2];
    p.scale_log2 = a.scale * kLog2e;
    if (a.batch == 0) return hipSuccess;
    if (p.nchunk > 0) {
        dim3 grid((unsigned)(a.batch * a.hkv), (unsigned)p.nchunk);
        const bool two = p.R > 32;
        if (a.d == 128) {
            if (two) hipLaunchKernelGGL((decode_split_kernel<128, 2>), grid, dim3(64), 0, s, p);
            else hipLaunchKernelGGL((decode_split_kernel<128, 1>), grid, dim3(64), 0, s, p);
        } else {
            if (two) hipLaunchKernelGGL((decode_split_kernel<64, 2>), grid, dim3(64), 0, s, p);
            else hipLaunchKernelGGL((decode_split_kernel<64, 1>), grid, dim3(64), 0, s, p);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 cgrid((p.R + 7) / 8, a.hkv, a.batch);
    if (a.d == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, cgrid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(decode_combine_kernel<64>, cgrid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t s) {
    // The caller has checked that the workspace fits kDecodeScratchBytes.  The device's
    // address of `scratch` is looked up once per device (with that device current) and kept;
    // threads racing on the first call store the same address.
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    DecodeArgs b = a;
    b.ws = ptr;
    return launch_decode(b, s);
}

}  // namespace mars
