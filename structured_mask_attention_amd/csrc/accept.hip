// Confidence-threshold acceptance (MARS author blog, "Inference: a knob, not a mode
// switch"; greedy decoding): per window row the argmax (lowest index on ties) and the
// top-1 probability pmax = 1 / sum_v exp(l_v - max); per sequence the length of the
// leading run of rows with pmax >= tau, at least one (tau >= 1: exactly one).
//
// One launch.  Grid (split, batch): each 256-thread workgroup streams one vocabulary
// slice of every window row of its sequence with 16-byte loads (all loads of a 4-row
// group are issued before any math), reduces (max, argmax, sum of exp) per row across
// the workgroup and writes a partial to the workspace.  The last workgroup of a sequence
// to finish (device-scope counter) merges the partials, writes tokens and pmax, applies
// the tau-prefix rule and resets the counter, leaving the workspace zeroed.
#include <cmath>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;                          // 16-byte vectors per row per thread
constexpr int kSlice = kThreads * 8 * kVecPerThread;      // 8192 vocabulary entries per slice
constexpr int kRowGroup = 4;                              // rows loaded together
constexpr int kMaxWindow = 64;

struct AcceptKParams {
    const uint16_t* logits;
    int32_t* tokens;
    float* pmax;
    int32_t* n_accept;
    int32_t* counters;   // [batch]
    float4* partial;     // [batch][split][W]: (max, sum, index bits, unused)
    int64_t bstride, rstride;
    int W, V, split;
    float tau;
};

struct Part {
    float m;
    float s;
    int idx;
};

// Merge two (max, lowest argmax, sum of exp relative to max) triples.
__device__ inline Part merge(Part a, Part b) {
    if (b.m > a.m || (b.m == a.m && b.idx < a.idx)) {
        Part t = a;
        a = b;
        b = t;
    }
    // a has the larger max (or the lower index at equal max).
    if (b.m == -INFINITY) return a;
    a.s += b.s * exp2f((b.m - a.m) * kLog2e);
    return a;
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

__global__ __launch_bounds__(kThreads) void accept_kernel(AcceptKParams p) {
    __shared__ Part red[kThreads / 64][kRowGroup];
    __shared__ int is_last;
    __shared__ float row_pmax[kMaxWindow];

    const int sl = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v0 = sl * kSlice;
    const int v1 = min(p.V, v0 + kSlice);
    const uint16_t* base = p.logits + b * p.bstride;

    for (int r0 = 0; r0 < p.W; r0 += kRowGroup) {
        uint4 vec[kRowGroup][kVecPerThread];
#pragma unroll
        for (int rr = 0; rr < kRowGroup; ++rr) {
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k) {
                const int e0 = v0 + 8 * (tid + kThreads * k);
                if (r0 + rr < p.W && e0 + 8 <= v1)
                    vec[rr][k] = *reinterpret_cast<const uint4*>(base + (int64_t)(r0 + rr) * p.rstride + e0);
                else
                    vec[rr][k] = uint4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int rr = 0; rr < kRowGroup; ++rr) {
            const int row = r0 + rr;
            Part x{-INFINITY, 0.f, 0x7fffffff};
            if (row < p.W) {
                const uint16_t* rowp = base + (int64_t)row * p.rstride;
                // Pass 1: max and lowest index attaining it (elements in increasing order).
#pragma unroll
                for (int k = 0; k < kVecPerThread; ++k) {
                    const int e0 = v0 + 8 * (tid + kThreads * k);
                    const uint32_t w[4] = {vec[rr][k].x, vec[rr][k].y, vec[rr][k].z, vec[rr][k].w};
                    if (e0 + 8 <= v1) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float f = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                            if (f > x.m) {
                                x.m = f;
                                x.idx = e0 + e;
                            }
                        }
                    } else if (e0 < v1) {  // ragged tail of the vocabulary
                        for (int e = 0; e < v1 - e0; ++e) {
                            const float f = bf16_bits_to_f32(rowp[e0 + e]);
                            if (f > x.m) {
                                x.m = f;
                                x.idx = e0 + e;
                            }
                        }
                    }
                }
                // Pass 2: sum of exp relative to the thread's max.
                if (x.m != -INFINITY) {
                    const float mb = x.m * kLog2e;
#pragma unroll
                    for (int k = 0; k < kVecPerThread; ++k) {
                        const int e0 = v0 + 8 * (tid + kThreads * k);
                        const uint32_t w[4] = {vec[rr][k].x, vec[rr][k].y, vec[rr][k].z, vec[rr][k].w};
                        if (e0 + 8 <= v1) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float f = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                                x.s += exp2f(fmaf(f, kLog2e, -mb));
                            }
                        } else if (e0 < v1) {
                            for (int e = 0; e < v1 - e0; ++e)
                                x.s += exp2f(fmaf(bf16_bits_to_f32(rowp[e0 + e]), kLog2e, -mb));
                        }
                    }
                }
            }
            x = wave_reduce(x);
            if (lane == 0) red[wave][rr] = x;
        }
        __syncthreads();
        if (tid < kRowGroup && r0 + tid < p.W) {
            Part x = red[0][tid];
#pragma unroll
            for (int w = 1; w < kThreads / 64; ++w) x = merge(x, red[w][tid]);
            p.partial[((int64_t)b * p.split + sl) * p.W + r0 + tid] = float4{x.m, x.s, __int_as_float(x.idx), 0.f};
        }
        __syncthreads();
    }

    // Publish the partials (every writer fences, then the workgroup syncs), then count
    // this workgroup in.
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(&p.counters[b], 1) == p.split - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    // Last workgroup of sequence b: one wave per row, lanes over slices.
    for (int row = wave; row < p.W; row += kThreads / 64) {
        Part x{-INFINITY, 0.f, 0x7fffffff};
        for (int s2 = lane; s2 < p.split; s2 += 64) {
            const float4 q = p.partial[((int64_t)b * p.split + s2) * p.W + row];
            x = merge(x, Part{q.x, q.y, __float_as_int(q.z)});
        }
        x = wave_reduce(x);
        if (lane == 0) {
            const float pm = 1.f / x.s;
            row_pmax[row] = pm;
            p.tokens[(int64_t)b * p.W + row] = x.idx;
            p.pmax[(int64_t)b * p.W + row] = pm;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        if (p.tau < 1.f) {
            while (n < p.W && row_pmax[n] >= p.tau) ++n;
        }
        p.n_accept[b] = n > 1 ? n : 1;
        atomicExch(&p.counters[b], 0);
    }
}

}  // namespace

static int accept_split(int V) { return (V + kSlice - 1) / kSlice; }

size_t accept_workspace_bytes(int batch, int W, int V) {
    const int64_t cnt = ((int64_t)batch * 4 + 255) / 256 * 256;
    return (size_t)(cnt + (int64_t)batch * accept_split(V) * W * (int64_t)sizeof(float4));
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    AcceptKParams p;
    p.logits = static_cast<const uint16_t*>(a.logits);
    p.tokens = a.tokens;
    p.pmax = a.pmax;
    p.n_accept = a.n_accept;
    p.counters = static_cast<int32_t*>(a.ws);
    const int64_t cnt = ((int64_t)a.batch * 4 + 255) / 256 * 256;
    p.partial = reinterpret_cast<float4*>(static_cast<char*>(a.ws) + cnt);
    p.bstride = a.batch_stride;
    p.rstride = a.row_stride;
    p.W = a.W;
    p.V = a.V;
    p.split = accept_split(a.V);
    p.tau = a.tau;
    hipLaunchKernelGGL(accept_kernel, dim3(p.split, a.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mars
