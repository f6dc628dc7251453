// Training loss of MARS over the vocabulary ("MARS: Enabling Autoregressive Models
// Multi-Token Generation", §3.2 Eq. 3 and §3.3 Eq. 5): L = L_mask + L_AR with
// right-shifted logits (the row of position p predicts the token at p + 1, as in AR).
//   L_AR:   response token x_t from the clean row P - 1 + t (none for t = 0 without a prompt);
//   L_mask: x_t from the noisy row P + L + t - 1 inside its block; the first token of a
//           block (only fully clean context, §3.3 and Eq. 4) from the same clean row as L_AR.
// Per row with a target: CE = logsumexp(row) - row[target] (natural log).
//
// Two launches:
//   1. rows: one workgroup per (sequence, row).  The usual vocabularies (up to 160K
//      entries) take the register-resident kernel: 1024 threads load the whole bf16 row
//      once into registers (16-byte vectors, all loads in flight together), reduce
//      (max, sum of exp) per thread and then across the workgroup, write CE to the
//      workspace and, with a gradient output, dlogits = w * (softmax - onehot) straight
//      from the registers (w = w_AR + w_mask): 2 bytes read and 2 written per entry, the
//      least this loss can move.  Larger vocabularies take a streaming kernel that keeps
//      an online (max, sum) and reads the row a second time for the gradient.  Rows
//      without a target write CE 0 and a zero gradient row.
//   2. sums: one workgroup per sequence adds the per-row CE with its weights in a fixed
//      order (deterministic) into loss_mask[b] and loss_ar[b].
#include <cmath>
#include <utility>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte vectors in flight per thread

struct CeParams {
    const uint16_t* logits;
    const int32_t* tokens;
    float* loss_mask;
    float* loss_ar;
    uint16_t* dlogits;   // may be null
    float* ce;           // workspace [batch][N]
    int64_t ls0, ls1, ds0, ds1, ts0;
    int P, L, B, N, V;
};

// Target response offset of row r (-1: none) and its loss weights (MARS reading above).
__device__ __host__ inline int ce_target(int r, int P, int L, int B, float* w_ar, float* w_mask) {
    const int PL = P + L;
    *w_ar = 0.f;
    *w_mask = 0.f;
    if (r < PL) {
        const int t = r - P + 1;
        if (t < 0 || t >= L) return -1;
        *w_ar = 1.f;
        *w_mask = (t % B == 0) ? 1.f : 0.f;
        return t;
    }
    const int j = r - PL;
    if (j > L - 2 || (j + 1) % B == 0) return -1;
    *w_mask = 1.f;
    return j + 1;
}

__device__ inline float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr int kThreadsR = 1024;   // register-resident kernel
constexpr int kMaxVecR = 20;      // 16-byte vectors per thread: V <= 20 * 8 * 1024

// Sums of exps are taken relative to c = fl(m log2 e), the max's log2-domain image rounded
// once: terms exp2(fma(x, log2 e, -c)) (the product is exact inside the fma, so a term near
// the max carries no rounding at the magnitude of the logits), sums over different maxima
// rescaled by exp2(c_a - c_b), and lse2 = c + log2 S keeps c's rounding out of
// CE = (fma(x_t, -log2 e, c) + log2 S) ln 2.
// The product is rounded on its own (no fusing into a later subtraction), so every
// use sees the same fp32 value of c.
__device__ inline float exp_offset(float m) {
#pragma clang fp contract(off)
    return m * kLog2e;
}

// Merge two (max, sum of exp relative to that max) pairs.
__device__ inline void merge_ms(float& ma, float& sa, float mb, float sb) {
    const float mn = fmaxf(ma, mb);
    const float a = ma == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(exp_offset(ma) - exp_offset(mn));
    const float c = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(exp_offset(mb) - exp_offset(mn));
    sa = sa * a + sb * c;
    ma = mn;
}

// An empty asm that claims to rewrite the row registers: the bf16 -> fp32 unpacking is
// then redone in each pass instead of being kept alive across passes (8 floats per vector
// would not fit the 128 registers a 1024-thread workgroup allows).
template <int NV>
__device__ inline void pin_regs(uint4 (&q)[NV]) {
#pragma unroll
    for (int u = 0; u < NV; ++u) asm volatile("" : "+v"(q[u].x), "+v"(q[u].y), "+v"(q[u].z), "+v"(q[u].w));
}

// max(a, b, c) in one instruction.  The operands are finite floats unpacked from bf16 by
// bit moves, which fmaxf would first canonicalise one by one.
__device__ inline float max3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Workgroup max / sum of one value per thread (wave butterfly, then the 16 wave results
// from LDS in a fixed order).  `red` holds 16 floats; ends with every thread holding it.
__device__ inline float block_max(float x, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kThreadsR / 64; ++k) r = fmaxf(r, red[k]);
    return r;
}
__device__ inline float block_sum(float x, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kThreadsR / 64; ++k) r += red[k];
    return r;
}

// NV = ceil((V / 8) / 1024) exactly, so vectors u < NV - 1 are in range for every thread
// and only the last one needs a bounds check.
template <int NV>
__global__ __launch_bounds__(kThreadsR) void ce_row_reg_kernel(CeParams p) {
    __shared__ float red_m[kThreadsR / 64], red_s[kThreadsR / 64];
    __shared__ float s_tv;
    const int r = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    float w_ar, w_mask;
    const int t = ce_target(r, p.P, p.L, p.B, &w_ar, &w_mask);
    const uint16_t* row = p.logits + b * p.ls0 + (int64_t)r * p.ls1;
    uint16_t* drow = p.dlogits ? p.dlogits + b * p.ds0 + (int64_t)r * p.ds1 : nullptr;
    const int nvec = p.V / 8;
    const bool last_in = tid + (NV - 1) * kThreadsR < nvec;

    if (t < 0) {
        if (drow) {
#pragma unroll
            for (int u = 0; u < NV; ++u)
                if (u < NV - 1 || last_in)
                    *reinterpret_cast<uint4*>(drow + 8 * (tid + u * kThreadsR)) = uint4{0u, 0u, 0u, 0u};
        }
        if (tid == 0) p.ce[(int64_t)b * p.N + r] = 0.f;
        return;
    }
    const int target = p.tokens[b * p.ts0 + t];

    uint4 q[NV];
#pragma unroll
    for (int u = 0; u < NV - 1; ++u) q[u] = *reinterpret_cast<const uint4*>(row + 8 * (tid + u * kThreadsR));
    q[NV - 1] = last_in ? *reinterpret_cast<const uint4*>(row + 8 * (tid + (NV - 1) * kThreadsR)) : uint4{0u, 0u, 0u, 0u};
    if (tid == 0) s_tv = (target >= 0 && target < p.V) ? __uint_as_float((uint32_t)row[target] << 16) : -INFINITY;

    // One pass over the vectors as they arrive: a running (max, sum of exp relative to it)
    // per thread, rescaled once per vector.
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        if (u < NV - 1 || last_in) {   // past the row: nothing to add (with NV = 1, m stays -inf, s 0)
            const uint32_t wv[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
            float mn = m;
#pragma unroll
            for (int k = 0; k < 4; ++k) mn = max3_raw(mn, lo_bf(wv[k]), hi_bf(wv[k]));
            s *= __builtin_amdgcn_exp2f(exp_offset(m) - exp_offset(mn));   // 0 on the first vector (m = -inf, s = 0)
            m = mn;
            const float mb = exp_offset(m);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                s += __builtin_amdgcn_exp2f(fmaf(lo_bf(wv[k]), kLog2e, -mb));
                s += __builtin_amdgcn_exp2f(fmaf(hi_bf(wv[k]), kLog2e, -mb));
            }
            // Order the pass vector by vector: this vector's sum is complete before the next
            // vector is unpacked (left to itself the compiler computes every vector's max
            // first and keeps their unpacked entries in registers until the exps).
            if (u + 1 < NV)
                asm volatile("" : "+v"(s), "+v"(m), "+v"(q[u + 1].x), "+v"(q[u + 1].y), "+v"(q[u + 1].z),
                             "+v"(q[u + 1].w));
        }
    }
    // Workgroup max, each thread's sum moved to it (a thread without entries has s = 0 and
    // m = -inf: factor 0), workgroup sum.
    const float M = block_max(m, red_m);
    s = block_sum(s * __builtin_amdgcn_exp2f(exp_offset(m) - exp_offset(M)), red_s);
    const float C = exp_offset(M), ls2 = log2f(s);
    if (tid == 0) p.ce[(int64_t)b * p.N + r] = (fmaf(s_tv, -kLog2e, C) + ls2) * kLn2;

    if (drow) {
        // w * softmax = exp2(x log2e - (lse2 - log2 w)), w in {1, 2}; the target entry
        // then gets -w, added only by the thread that holds it.
        pin_regs<NV>(q);
        const float w = w_ar + w_mask;
        const float lb = C + (ls2 - (w > 1.5f ? 1.f : 0.f));
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + u * kThreadsR;
            if (u < NV - 1 || last_in) {
                const uint32_t wv[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
                float g[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    g[2 * k] = __builtin_amdgcn_exp2f(fmaf(lo_bf(wv[k]), kLog2e, -lb));
                    g[2 * k + 1] = __builtin_amdgcn_exp2f(fmaf(hi_bf(wv[k]), kLog2e, -lb));
                }
                *reinterpret_cast<uint4*>(drow + 8 * v) = uint4{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                                                                pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
            }
        }
        // The thread that wrote the target's vector rewrites its entry (same thread, same
        // address: the later store lands last), from the same formula minus w.
        if (target >= 0 && target < p.V && tid == (target >> 3) % kThreadsR) {
            const float gt = __builtin_amdgcn_exp2f(fmaf(s_tv, kLog2e, -lb)) - w;
            drow[target] = (uint16_t)(pack_bf16x2(gt, 0.f) & 0xffffu);
        }
    }
}

template <int NV>
hipError_t launch_reg(const CeParams& p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL(ce_row_reg_kernel<NV>, grid, dim3(kThreadsR), 0, s, p);
    return hipGetLastError();
}

template <int... I>
hipError_t launch_reg_nv(int nv, const CeParams& p, dim3 grid, hipStream_t s, std::integer_sequence<int, I...>) {
    // The instantiation whose vector count matches nv launches; the fold stops there.
    hipError_t e = hipErrorInvalidValue;
    const bool launched = ((nv == I + 1 ? (e = launch_reg<I + 1>(p, grid, s), true) : false) || ...);
    return launched ? e : hipErrorInvalidValue;
}

__global__ __launch_bounds__(kThreads) void ce_row_kernel(CeParams p) {
    __shared__ float red_m[kThreads / 64], red_s[kThreads / 64], red_t[kThreads / 64];
    const int r = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float w_ar, w_mask;
    const int t = ce_target(r, p.P, p.L, p.B, &w_ar, &w_mask);
    const uint16_t* row = p.logits + b * p.ls0 + (int64_t)r * p.ls1;
    const int nvec = p.V / 8;   // V % 8 == 0 (checked by the caller)

    if (t < 0) {
        if (p.dlogits) {
            uint16_t* drow = p.dlogits + b * p.ds0 + (int64_t)r * p.ds1;
            for (int v = tid; v < nvec; v += kThreads) *reinterpret_cast<uint4*>(drow + 8 * v) = uint4{0u, 0u, 0u, 0u};
        }
        if (tid == 0) p.ce[(int64_t)b * p.N + r] = 0.f;
        return;
    }
    const int target = p.tokens[b * p.ts0 + t];

    // Pass 1: (max, sum exp) per thread over vectors tid + 256k; the target entry.
    float m = -INFINITY, s = 0.f, tv = -INFINITY;
    for (int v0 = tid; v0 < nvec; v0 += kThreads * kUnroll) {
        uint4 q[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int v = v0 + u * kThreads;
            q[u] = v < nvec ? *reinterpret_cast<const uint4*>(row + 8 * v) : uint4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t wv[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
            float x[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = lo_bf(wv[k]);
                x[2 * k + 1] = hi_bf(wv[k]);
            }
            float vm = x[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) vm = fmaxf(vm, x[k]);
            if (vm > m) {
                s *= __builtin_amdgcn_exp2f(exp_offset(m) - exp_offset(vm));
                m = vm;
            }
            if (m != -INFINITY) {
                const float mb = exp_offset(m);
#pragma unroll
                for (int k = 0; k < 8; ++k) s += __builtin_amdgcn_exp2f(fmaf(x[k], kLog2e, -mb));
            }
            const int base = 8 * (v0 + u * kThreads);
            if (target >= base && target < base + 8) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (target - base == k) tv = x[k];   // no dynamic register indexing
            }
        }
    }
    // Workgroup merge of (m, s) and the target entry (one thread holds it).
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float mo = __shfl_xor(m, off), so = __shfl_xor(s, off), to = __shfl_xor(tv, off);
        merge_ms(m, s, mo, so);
        tv = fmaxf(tv, to);
    }
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
        red_t[wave] = tv;
    }
    __syncthreads();
    m = red_m[0];
    s = red_s[0];
    tv = red_t[0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) {
        merge_ms(m, s, red_m[k], red_s[k]);
        tv = fmaxf(tv, red_t[k]);
    }
    const float C = exp_offset(m), ls2 = log2f(s);
    if (tid == 0) p.ce[(int64_t)b * p.N + r] = (fmaf(tv, -kLog2e, C) + ls2) * kLn2;

    // Pass 2 (gradient): w * (exp(l - lse) - onehot(target)).
    if (p.dlogits) {
        const float w = w_ar + w_mask;
        const float lb = C + ls2;
        uint16_t* drow = p.dlogits + b * p.ds0 + (int64_t)r * p.ds1;
        for (int v = tid; v < nvec; v += kThreads) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + 8 * v);
            const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e0 = 8 * v + 2 * k;
                float g0 = __builtin_amdgcn_exp2f(fmaf(lo_bf(wv[k]), kLog2e, -lb));
                float g1 = __builtin_amdgcn_exp2f(fmaf(hi_bf(wv[k]), kLog2e, -lb));
                g0 = w * (g0 - (e0 == target ? 1.f : 0.f));
                g1 = w * (g1 - (e0 + 1 == target ? 1.f : 0.f));
                o[k] = pack_bf16x2(g0, g1);
            }
            *reinterpret_cast<uint4*>(drow + 8 * v) = uint4{o[0], o[1], o[2], o[3]};
        }
    }
}

// One 256-thread workgroup per sequence: weighted sums of the row CE.  Thread k adds
// rows k, k + 256, ... (loads issued together), then a fixed butterfly and the four wave
// sums in wave order: the same order on every call (deterministic).
constexpr int kSumThreads = 256;

__global__ __launch_bounds__(kSumThreads) void ce_sum_kernel(CeParams p) {
    __shared__ float red_a[kSumThreads / 64], red_m[kSumThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x;
    float sa = 0.f, sm = 0.f;
    for (int r0 = 0; r0 < p.N; r0 += 4 * kSumThreads) {
        float c[4], wa[4], wm[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = r0 + k * kSumThreads + tid;
            const bool has = r < p.N && ce_target(r, p.P, p.L, p.B, &wa[k], &wm[k]) >= 0;
            if (!has) wa[k] = wm[k] = 0.f;
            c[k] = has ? p.ce[(int64_t)b * p.N + r] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {   // a zero weight adds nothing (not 0 * inf)
            sa += wa[k] != 0.f ? wa[k] * c[k] : 0.f;
            sm += wm[k] != 0.f ? wm[k] * c[k] : 0.f;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sa += __shfl_xor(sa, off);
        sm += __shfl_xor(sm, off);
    }
    if ((tid & 63) == 0) {
        red_a[tid >> 6] = sa;
        red_m[tid >> 6] = sm;
    }
    __syncthreads();
    if (tid == 0) {
        float ta = red_a[0], tm = red_m[0];
#pragma unroll
        for (int w = 1; w < kSumThreads / 64; ++w) {
            ta += red_a[w];
            tm += red_m[w];
        }
        p.loss_ar[b] = ta;
        p.loss_mask[b] = tm;
    }
}

}  // namespace

hipError_t launch_shifted_ce(const CeArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    CeParams p;
    p.logits = static_cast<const uint16_t*>(a.logits);
    p.tokens = a.tokens;
    p.loss_mask = a.loss_mask;
    p.loss_ar = a.loss_ar;
    p.dlogits = static_cast<uint16_t*>(a.dlogits);
    p.ce = static_cast<float*>(a.ws);
    p.ls0 = a.ls[0];
    p.ls1 = a.ls[1];
    p.ds0 = a.ds[0];
    p.ds1 = a.ds[1];
    p.ts0 = a.ts0;
    p.P = a.P;
    p.L = a.L;
    p.B = a.B;
    p.N = a.P + 2 * a.L;
    p.V = a.V;
    if (p.N == 0) {
        hipLaunchKernelGGL(ce_sum_kernel, dim3((unsigned)a.batch), dim3(kSumThreads), 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)p.N, (unsigned)a.batch);
    const int nv = (p.V / 8 + kThreadsR - 1) / kThreadsR;   // vectors per thread, register kernel
    hipError_t e;
    if (nv <= kMaxVecR) {
        e = launch_reg_nv(nv, p, grid, s, std::make_integer_sequence<int, kMaxVecR>{});
    } else {
        hipLaunchKernelGGL(ce_row_kernel, grid, dim3(kThreads), 0, s, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ce_sum_kernel, dim3((unsigned)a.batch), dim3(kSumThreads), 0, s, p);
    return hipGetLastError();
}

size_t shifted_ce_workspace_bytes(int batch, int P, int L) { return (size_t)batch * (size_t)(P + 2 * L) * 4; }

}  // namespace mars
