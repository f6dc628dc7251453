// Sliding-window decode step ("MARS: Enabling Autoregressive Models Multi-Token
// Generation", Fig. 2 right): W window rows per sequence attend to the sequence's KV
// cache [0, len) and, causally and self-inclusively, to the window rows 0..i.
//
// Two kernels on the caller's stream:
//   1. split: one wave per (sequence, kv head, CH-key cache chunk).  The G*W query rows
//      of a kv head (G = Hq/Hkv query heads x W window rows, <= 64) form one or two
//      32-column MFMA blocks; S^T = K Q^T (K fragments loaded straight from HBM as the A
//      operand), online softmax, O^T += V^T P^T (V staged through LDS and read back
//      transposed with ds_read_b64_tr_b16).  The next 32-key step is prefetched into
//      registers while the current one computes.  Each chunk writes an unnormalised
//      partial (acc, m, l) to the workspace.
//   2. combine: one workgroup per (sequence, query head): the window keys (at most W dot
//      products per row) and a log-sum-exp merge of the chunk partials.
// Chunks past a sequence's length exit at once, so the grid is fixed while the work is
// ragged; the cache is read exactly once.
#include <cmath>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kCH = 256;      // cache keys per split workgroup
constexpr int kStep = 32;     // keys per MFMA step
constexpr int kMaxRows = 64;  // G * W

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

template <int D, int NCB>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeKParams p) {
    constexpr int VSTR = D + 32;
    constexpr int NC = D / 16;
    constexpr int NDB = D / 32;
    constexpr int VL = (kStep * D / 8) / 64;   // 16-byte V loads per lane per step
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][kStep * VSTR];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int len = clamp_len(p.cache_len[b], p.cap);
    const int k_begin = c * kCH;
    if (k_begin >= len) return;
    const int k_end = min(len, k_begin + kCH);
    const int nsteps = (k_end - k_begin + kStep - 1) / kStep;

    const int lane = threadIdx.x;
    const int hl = lane & 31, g2 = lane >> 5;

    // Query rows u = i*G + hh (window row i, query head g*G + hh).
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

    const uint16_t* kbase = p.kc + b * p.kcs0 + (int64_t)g * p.kcs1;
    const uint16_t* vbase = p.vc + b * p.vcs0 + (int64_t)g * p.vcs1;

    bf16x8_t kreg[NC], vreg[VL];
    auto gload = [&](int step) {
        const int k0 = k_begin + step * kStep;
        const int key = k0 + hl;
        if (key < k_end) {
            const uint16_t* kp = kbase + (int64_t)key * p.kcs2 + 8 * g2;
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) kreg[cc] = *reinterpret_cast<const bf16x8_t*>(kp + 16 * cc);
        } else {
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) kreg[cc] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int idx = lane + 64 * i;
            const int kl = idx / (D / 8), ch = idx % (D / 8);
            if (k0 + kl < k_end)
                vreg[i] = *reinterpret_cast<const bf16x8_t*>(vbase + (int64_t)(k0 + kl) * p.vcs2 + 8 * ch);
            else
                vreg[i] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    };

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

    const int s16 = lane & 15, grp = lane >> 4;
    const int vkey = 4 * (grp >> 1) + (s16 >> 2);
    const int vcol = 16 * (grp & 1) + 4 * (s16 & 3);

    gload(0);
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        // Stage this step's V tile in LDS, then take K out of the load registers so the
        // next step's loads can be issued before the math.
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int idx = lane + 64 * i;
            const int kl = idx / (D / 8), ch = idx % (D / 8);
            *reinterpret_cast<bf16x8_t*>(&sV[buf][kl * VSTR + 8 * ch]) = vreg[i];
        }
        bf16x8_t kf[NC];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kf[cc] = kreg[cc];
        __syncthreads();
        if (step + 1 < nsteps) gload(step + 1);

        const int k0 = k_begin + step * kStep;
        f32x16_t s[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[cb][e] = 0.f;
        }
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], qf[cb][cc], s[cb], 0, 0, 0);
        }
        if (k0 + kStep > k_end) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = k0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                    if (j >= k_end) s[cb][e] = -INFINITY;
                }
            }
        }
        bf16x8_t pb[NCB][2];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            float mx = s[cb][0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[cb][e]);
            mx = half_swap_max(mx);
            const float mnew = fmaxf(m_run[cb], mx * p.scale_log2);
            const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = exp2f(m_run[cb] - msafe);
            m_run[cb] = mnew;
            float pv[16];
            float rs = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pv[e] = exp2f(fmaf(s[cb][e], p.scale_log2, -msafe));
                rs += pv[e];
            }
            l_run[cb] = fmaf(l_run[cb], alpha, rs);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[cb][db][e] *= alpha;
            }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
                u32x4_t w = {pack_bf16x2(pv[8 * kh + 0], pv[8 * kh + 1]), pack_bf16x2(pv[8 * kh + 2], pv[8 * kh + 3]),
                             pack_bf16x2(pv[8 * kh + 4], pv[8 * kh + 5]), pack_bf16x2(pv[8 * kh + 6], pv[8 * kh + 7])};
                pb[cb][kh] = __builtin_bit_cast(bf16x8_t, w);
            }
        }
        const uint16_t* vt = &sV[buf][0];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const uint16_t* a0 = vt + (16 * kh + vkey) * VSTR + 32 * db + vcol;
                const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(a0));
                const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(a0 + 8 * VSTR));
                const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[cb][kh], acc[cb][db], 0, 0, 0);
            }
        }
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

// One workgroup (64 threads) per (sequence, query head); thread t owns d = t, t + 64.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeKParams p) {
    constexpr int DPT = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int g = h / p.G, hh = h % p.G;
    const int t = threadIdx.x;
    const int len = clamp_len(p.cache_len[b], p.cap);
    const int nch = (len + kCH - 1) / kCH;

    for (int i = 0; i < p.W; ++i) {
        const int u = i * p.G + hh;
        const uint16_t* qp = p.qw + b * p.qws0 + (int64_t)i * p.qws1 + (int64_t)h * p.qws2;
        float qv[DPT];
#pragma unroll
        for (int e = 0; e < DPT; ++e) qv[e] = bf16_bits_to_f32(qp[t + 64 * e]);

        // Window scores (log2 domain), rows 0..i of this sequence's window.
        float sw[kMaxRows];
        float M = -INFINITY;
        for (int j = 0; j <= i; ++j) {
            const uint16_t* kp = p.kw + b * p.kws0 + (int64_t)j * p.kws1 + (int64_t)g * p.kws2;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < DPT; ++e) part = fmaf(qv[e], bf16_bits_to_f32(kp[t + 64 * e]), part);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
            sw[j] = part * p.scale_log2;
            M = fmaxf(M, sw[j]);
        }
        const int64_t slot0 = ((int64_t)(b * p.hkv + g) * p.nchunk) * p.R + u;
        for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, p.ws_ml[(slot0 + (int64_t)cc * p.R) * 2]);

        float num[DPT] = {};
        float den = 0.f;
        for (int cc = 0; cc < nch; ++cc) {
            const int64_t sl = slot0 + (int64_t)cc * p.R;
            const float w = exp2f(p.ws_ml[sl * 2] - M);
            den = fmaf(p.ws_ml[sl * 2 + 1], w, den);
            const float* ap = p.ws_acc + sl * D;
#pragma unroll
            for (int e = 0; e < DPT; ++e) num[e] = fmaf(ap[t + 64 * e], w, num[e]);
        }
        for (int j = 0; j <= i; ++j) {
            const float w = exp2f(sw[j] - M);
            den += w;
            const uint16_t* vp = p.vw + b * p.vws0 + (int64_t)j * p.vws1 + (int64_t)g * p.vws2;
#pragma unroll
            for (int e = 0; e < DPT; ++e) num[e] = fmaf(bf16_bits_to_f32(vp[t + 64 * e]), w, num[e]);
        }
        const float inv = 1.f / den;
        uint16_t* op = p.o + b * p.os0 + (int64_t)i * p.os1 + (int64_t)h * p.os2;
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
            const uint32_t pk = pack_bf16x2(num[e] * inv, 0.f);
            op[t + 64 * e] = (uint16_t)(pk & 0xffffu);
        }
    }
}

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
        dim3 grid(p.nchunk, a.hkv, a.batch);
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
    dim3 cgrid(a.hq, a.batch);
    if (a.d == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, cgrid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL(decode_combine_kernel<64>, cgrid, dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace mars
