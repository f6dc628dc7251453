// Confidence-threshold acceptance (MARS author blog, "Inference: a knob, not a mode
// switch"; greedy decoding): per window row the argmax (lowest index on ties) and the
// top-1 probability pmax = 1 / sum_v exp(l_v - max); per sequence the length of the
// leading run of rows with pmax >= tau, at least one (tau >= 1: exactly one).
//
// Two launches on the caller's stream; the kernel boundary orders them, so no device-scope
// fences or counters are needed and the workspace needs no initialisation.
//   1. slices: grid (rows = batch*W, slices); a 256-thread workgroup owns one 8192-entry
//      slice of one row.  Each thread issues all four of its 16-byte loads before any
//      math, converts bf16 -> fp32 with shifts/masks, takes the max with v_max3, finds the
//      lowest index attaining it hierarchically (vector max first) and sums
//      2^((l - m) log2 e) with the raw v_exp_f32.  (max, argmax, sum) triples are merged
//      across the wave (shuffles) and the workgroup (LDS) and written to the workspace.
//   2. finish: one workgroup per sequence merges the slices of each row in a fixed order
//      (one wave per row), writes tokens and pmax, and applies the tau-prefix rule.
#include <cmath>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;                              // 16-byte vectors per thread
constexpr int kSlice = kThreads * 8 * kVec;          // 8192 vocabulary entries per workgroup
constexpr int kMaxWindow = 64;

struct AcceptKParams {
    const uint16_t* logits;
    int32_t* tokens;
    float* pmax;
    int32_t* n_accept;
    float4* partial;     // [batch*W][split]: (max, sum, index bits, unused)
    int64_t bstride, rstride;
    int W, V, split;
    float tau;
};

struct Part {
    float m;
    float s;
    int idx;
};

// Merge two (max, lowest argmax, sum of exp relative to max) triples (branch-free).
__device__ inline Part merge(Part a, Part b) {
    const bool bw = b.m > a.m || (b.m == a.m && b.idx < a.idx);
    Part r;
    r.m = bw ? b.m : a.m;
    r.idx = bw ? b.idx : a.idx;
    const float lo_m = bw ? a.m : b.m;
    const float lo_s = bw ? a.s : b.s;
    const float hi_s = bw ? b.s : a.s;
    const float scale = (lo_m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((lo_m - r.m) * kLog2e);
    r.s = fmaf(lo_s, scale, hi_s);
    return r;
}

__device__ inline Part wave_reduce(Part x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Part y;
        y.m = __shfl_xor(x.m, off);
        y.s = __shfl_xor(x.s, off);
        y.idx = __shfl_xor(x.idx, off);
        x = merge(x, y);
    }
    return x;
}

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// RAGGED: V is not a multiple of 8, so the last vector of a row is read entry by entry.
template <bool RAGGED>
__global__ __launch_bounds__(kThreads) void accept_slice_kernel(AcceptKParams p) {
    __shared__ Part red[kThreads / 64];

    const int row = blockIdx.x, sl = blockIdx.y;
    const int b = row / p.W, i = row % p.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v0 = sl * kSlice;
    const int v1 = min(p.V, v0 + kSlice);
    const uint16_t* rowp = p.logits + b * p.bstride + (int64_t)i * p.rstride;

    // Loads: vector k of this thread covers entries e0(k) .. e0(k)+7, e0(k) increasing in k.
    uint32_t w[kVec][4];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const int e0 = v0 + 8 * (tid + kThreads * k);
        if (!RAGGED) {
            // V % 8 == 0: every vector is whole.  Vectors past the row end re-read the last
            // vector (always in bounds) and are replaced by -inf (bf16 0xff80) without a branch.
            const bool in = e0 < v1;
            const uint4 q = *reinterpret_cast<const uint4*>(rowp + (in ? e0 : v1 - 8));
            w[k][0] = in ? q.x : 0xff80ff80u;
            w[k][1] = in ? q.y : 0xff80ff80u;
            w[k][2] = in ? q.z : 0xff80ff80u;
            w[k][3] = in ? q.w : 0xff80ff80u;
        } else if (e0 + 8 <= v1) {
            const uint4 q = *reinterpret_cast<const uint4*>(rowp + e0);
            w[k][0] = q.x; w[k][1] = q.y; w[k][2] = q.z; w[k][3] = q.w;
        } else if (e0 >= v1) {
            w[k][0] = w[k][1] = w[k][2] = w[k][3] = 0xff80ff80u;
        } else {
            // Ragged last vector: entries past V read as -inf.
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ea = e0 + 2 * j, eb = ea + 1;
                const uint32_t lo = ea < v1 ? (uint32_t)rowp[ea] : 0xff80u;
                const uint32_t hi = eb < v1 ? (uint32_t)rowp[eb] : 0xff80u;
                w[k][j] = lo | (hi << 16);
            }
        }
    }

    float f[kVec][8];
    float vmax[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[k][2 * j] = lo_bf16(w[k][j]);
            f[k][2 * j + 1] = hi_bf16(w[k][j]);
        }
        vmax[k] = fmaxf(fmaxf(fmaxf(f[k][0], f[k][1]), fmaxf(f[k][2], f[k][3])),
                        fmaxf(fmaxf(f[k][4], f[k][5]), fmaxf(f[k][6], f[k][7])));
    }
    Part x;
    x.m = fmaxf(fmaxf(vmax[0], vmax[1]), fmaxf(vmax[2], vmax[3]));
    // Lowest index attaining the max: first vector holding it, then first entry in it.
    int kk = kVec - 1;
#pragma unroll
    for (int k = kVec - 2; k >= 0; --k) kk = (vmax[k] == x.m) ? k : kk;
    float gsel[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gsel[e] = kk == 0 ? f[0][e] : (kk == 1 ? f[1][e] : (kk == 2 ? f[2][e] : f[3][e]));
    int ee = 7;
#pragma unroll
    for (int e = 6; e >= 0; --e) ee = (gsel[e] == x.m) ? e : ee;
    x.idx = (x.m == -INFINITY) ? 0x7fffffff : v0 + 8 * (tid + kThreads * kk) + ee;
    // Sum of 2^((l - m) log2 e) over the thread's entries (two partial sums).
    x.s = 0.f;
    if (x.m != -INFINITY) {
        const float mb = x.m * kLog2e;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                s0 += __builtin_amdgcn_exp2f(fmaf(f[k][e], kLog2e, -mb));
                s1 += __builtin_amdgcn_exp2f(fmaf(f[k][e + 1], kLog2e, -mb));
            }
        }
        x.s = s0 + s1;
    }

    x = wave_reduce(x);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    if (tid == 0) {
        Part y = red[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) y = merge(y, red[k]);
        p.partial[(int64_t)row * p.split + sl] = float4{y.m, y.s, __int_as_float(y.idx), 0.f};
    }
}

// One workgroup per sequence: one wave per row, lanes over slices (fixed merge order).
__global__ __launch_bounds__(kThreads) void accept_finish_kernel(AcceptKParams p) {
    __shared__ float row_pmax[kMaxWindow];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < p.W; r += kThreads / 64) {
        Part y{-INFINITY, 0.f, 0x7fffffff};
        const float4* pr = p.partial + ((int64_t)b * p.W + r) * p.split;
        for (int s2 = lane; s2 < p.split; s2 += 64) {
            const float4 q = pr[s2];
            y = merge(y, Part{q.x, q.y, __float_as_int(q.z)});
        }
        y = wave_reduce(y);
        if (lane == 0) {
            const float pm = 1.f / y.s;
            row_pmax[r] = pm;
            p.tokens[(int64_t)b * p.W + r] = y.idx;
            p.pmax[(int64_t)b * p.W + r] = pm;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        if (p.tau < 1.f) {
            while (n < p.W && row_pmax[n] >= p.tau) ++n;
        }
        p.n_accept[b] = n > 1 ? n : 1;
    }
}

}  // namespace

static int accept_split(int V) { return (V + kSlice - 1) / kSlice; }

size_t accept_workspace_bytes(int batch, int W, int V) {
    return (size_t)((int64_t)batch * W * accept_split(V) * (int64_t)sizeof(float4));
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    AcceptKParams p;
    p.logits = static_cast<const uint16_t*>(a.logits);
    p.tokens = a.tokens;
    p.pmax = a.pmax;
    p.n_accept = a.n_accept;
    p.partial = static_cast<float4*>(a.ws);
    p.bstride = a.batch_stride;
    p.rstride = a.row_stride;
    p.W = a.W;
    p.V = a.V;
    p.split = accept_split(a.V);
    p.tau = a.tau;
    const dim3 grid((unsigned)(a.batch * a.W), (unsigned)p.split);
    if (a.V % 8 == 0) hipLaunchKernelGGL(accept_slice_kernel<false>, grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(accept_slice_kernel<true>, grid, dim3(kThreads), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_finish_kernel, dim3((unsigned)a.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mars
