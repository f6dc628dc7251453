// Confidence-threshold acceptance (MARS author blog, "Inference: a knob, not a mode
// switch"; greedy decoding): per window row the argmax (lowest index on ties) and the
// top-1 probability pmax = 1 / sum_v exp(l_v - max); per sequence the length of the
// leading run of rows with pmax >= tau, at least one (tau >= 1: exactly one).
// The margin gate (same blog section: how far the top token is ahead) gates on
// margin = top-1 minus top-2 probability = (1 - exp(l2 - l1)) / sum_v exp(l_v - l1), with
// l2 the second largest entry counted with multiplicity; the slice kernel then also keeps
// each thread's two largest entries (v_med3 / v_max per entry).
//
// Two launches on the caller's stream; the kernel boundary orders them, so no device-scope
// fences or counters are needed and the workspace needs no initialisation.
//   1. slices: grid (rows = batch*W, slices); a 256-thread workgroup owns one 16384-entry
//      slice of one row (at the 152k vocabulary every workgroup is resident at once): all
//      of its loads are issued up front, then four 4096-entry chunks are reduced in order
//      as their data arrives.  Each thread keeps a
//      running (max, lowest argmax, sum of 2^((l - m) log2 e)) over its entries; values
//      stay packed bf16 until used (shift/mask to fp32), the sum uses the raw v_exp_f32
//      and is rescaled when the max grows.  The (max, argmax, sum) triples are merged
//      across the wave (shuffles) and the workgroup (LDS) and written to the workspace.
//   2. finish: one workgroup per sequence merges the slices of each row in a fixed order
//      (one wave per row), writes tokens and pmax, and applies the tau-prefix rule.
#include <cmath>

#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerChunk = 2;                      // 16-byte vectors per thread and chunk
constexpr int kChunk = kThreads * 8 * kVecPerChunk;  // 4096 vocabulary entries per chunk
constexpr int kChunks = 4;                           // chunks per workgroup
constexpr int kSlice = kChunk * kChunks;             // 16384 vocabulary entries per workgroup
constexpr int kMaxWindow = 64;

struct AcceptKParams {
    const uint16_t* logits;
    int32_t* tokens;
    float* pmax;
    int32_t* n_accept;
    float4* partial;     // [batch*W][split]: (max, sum, index bits, second largest)
    float* margin;       // margin gate only (may be null otherwise)
    int64_t bstride, rstride;
    int W, V, split;
    float tau;
};

// Every sum of exps is taken relative to c = fl(m log2 e), the max's log2-domain image
// rounded once to fp32: terms are exp2(fma(l, log2 e, -c)) (the product is exact inside
// the fma, so a term near the max carries no rounding at the magnitude of the logits),
// sums with different maxima are rescaled by exp2(c_a - c_b), and pmax = exp2(fma(m,
// log2 e, -c)) / S undoes the rounding of c itself.
// The product is rounded on its own (no fusing into a later subtraction), so every
// use sees the same fp32 value of c.
__device__ inline float exp_offset(float m) {
#pragma clang fp contract(off)
    return m * kLog2e;
}

struct Part {
    float m;
    float s;
    int idx;
    float m2;            // second largest entry with multiplicity (margin gate; else -inf)
};

// Merge two (max, lowest argmax, sum of exp relative to max, second largest) tuples
// (branch-free).  The union's second largest is the smaller maximum or the larger second.
__device__ inline Part merge(Part a, Part b) {
    const bool bw = b.m > a.m || (b.m == a.m && b.idx < a.idx);
    Part r;
    r.m = bw ? b.m : a.m;
    r.idx = bw ? b.idx : a.idx;
    r.m2 = fmaxf(fminf(a.m, b.m), fmaxf(a.m2, b.m2));
    const float lo_m = bw ? a.m : b.m;
    const float lo_s = bw ? a.s : b.s;
    const float hi_s = bw ? b.s : a.s;
    const float scale = (lo_m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(exp_offset(lo_m) - exp_offset(r.m));
    r.s = fmaf(lo_s, scale, hi_s);
    return r;
}

template <int CTRL>
__device__ inline Part dpp_part(Part x) {
    return Part{dpp_f32<CTRL>(x.m), dpp_f32<CTRL>(x.s), __float_as_int(dpp_f32<CTRL>(__int_as_float(x.idx))),
                dpp_f32<CTRL>(x.m2)};
}

// merge() is symmetric in its arguments, so each step may pair lanes by any involution:
// quad swaps, half-row and row mirrors (DPP), then rows of 16 and halves of 32 exchanged
// with v_permlane16_swap / v_permlane32_swap (which hand each lane both values).
__device__ inline Part wave_reduce(Part x) {
    x = merge(x, dpp_part<0xB1>(x));
    x = merge(x, dpp_part<0x4E>(x));
    x = merge(x, dpp_part<0x141>(x));
    x = merge(x, dpp_part<0x140>(x));
    {
        auto m = __builtin_amdgcn_permlane16_swap(__float_as_uint(x.m), __float_as_uint(x.m), false, false);
        auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x.s), __float_as_uint(x.s), false, false);
        auto i = __builtin_amdgcn_permlane16_swap((uint32_t)x.idx, (uint32_t)x.idx, false, false);
        auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x.m2), __float_as_uint(x.m2), false, false);
        x = merge(Part{__uint_as_float(m[0]), __uint_as_float(s[0]), (int)i[0], __uint_as_float(t[0])},
                  Part{__uint_as_float(m[1]), __uint_as_float(s[1]), (int)i[1], __uint_as_float(t[1])});
    }
    {
        auto m = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.m), __float_as_uint(x.m), false, false);
        auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.s), __float_as_uint(x.s), false, false);
        auto i = __builtin_amdgcn_permlane32_swap((uint32_t)x.idx, (uint32_t)x.idx, false, false);
        auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.m2), __float_as_uint(x.m2), false, false);
        x = merge(Part{__uint_as_float(m[0]), __uint_as_float(s[0]), (int)i[0], __uint_as_float(t[0])},
                  Part{__uint_as_float(m[1]), __uint_as_float(s[1]), (int)i[1], __uint_as_float(t[1])});
    }
    return x;
}

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Entry j (0..7) of a 16-byte vector held as four packed bf16 words, as fp32.
__device__ inline float entry(const uint32_t (&w)[4], int j) {
    return (j & 1) ? hi_bf16(w[j >> 1]) : lo_bf16(w[j >> 1]);
}

// Vectors of chunk c of this thread's slice: vector v covers entries e0 .. e0+7 with
// e0 = v0 + c*kChunk + 8*(tid + kThreads*v), increasing in (c, v).
__device__ inline int vec_start(int v0, int c, int tid, int k) { return v0 + c * kChunk + 8 * (tid + kThreads * k); }

// Issue the loads of chunk c; nothing here uses the loaded values, so no wait is needed
// until the chunk is reduced.  V % 8 == 0: every vector is whole, and vectors at or past
// v1 re-read the last vector (always in bounds); finish_chunk masks them to -inf.
// Otherwise (ragged V) the partial vector is read entry by entry, entries past v1 as -inf.
template <bool RAGGED>
__device__ inline void load_chunk(const uint16_t* rowp, int v0, int v1, int c, int tid, uint32_t (&w)[kVecPerChunk][4]) {
#pragma unroll
    for (int k = 0; k < kVecPerChunk; ++k) {
        const int e0 = vec_start(v0, c, tid, k);
        if (!RAGGED) {
            const uint4 q = *reinterpret_cast<const uint4*>(rowp + (e0 < v1 ? e0 : v1 - 8));
            w[k][0] = q.x; w[k][1] = q.y; w[k][2] = q.z; w[k][3] = q.w;
        } else if (e0 + 8 <= v1) {
            const uint4 q = *reinterpret_cast<const uint4*>(rowp + e0);
            w[k][0] = q.x; w[k][1] = q.y; w[k][2] = q.z; w[k][3] = q.w;
        } else if (e0 >= v1) {
            w[k][0] = w[k][1] = w[k][2] = w[k][3] = 0xff80ff80u;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ea = e0 + 2 * j, eb = ea + 1;
                const uint32_t lo = ea < v1 ? (uint32_t)rowp[ea] : 0xff80u;
                const uint32_t hi = eb < v1 ? (uint32_t)rowp[eb] : 0xff80u;
                w[k][j] = lo | (hi << 16);
            }
        }
    }
}

// Replace the re-read vectors past v1 by -inf (bf16 0xff80 pairs); a no-op for ragged V.
template <bool RAGGED>
__device__ inline void finish_chunk(int v0, int v1, int c, int tid, uint32_t (&w)[kVecPerChunk][4]) {
    if (RAGGED) return;
#pragma unroll
    for (int k = 0; k < kVecPerChunk; ++k) {
        const bool in = vec_start(v0, c, tid, k) < v1;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[k][j] = in ? w[k][j] : 0xff80ff80u;
    }
}

// RAGGED: V is not a multiple of 8, so the last vector of a row is read entry by entry.
// TOP2: also keep the second largest entry (margin gate).
template <bool RAGGED, bool TOP2>
__global__ __launch_bounds__(kThreads) void accept_slice_kernel(AcceptKParams p) {
    __shared__ Part red[kThreads / 64];

    const int row = blockIdx.x, sl = blockIdx.y;
    const int b = row / p.W, i = row % p.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v0 = sl * kSlice;
    const int v1 = min(p.V, v0 + kSlice);
    const uint16_t* rowp = p.logits + b * p.bstride + (int64_t)i * p.rstride;

    // All loads of the slice are issued first (32 KB in flight per workgroup); the chunks
    // are then reduced in order as their data arrives, into this thread's running (max,
    // lowest argmax, sum).  sched_barrier keeps the compiler from hoisting any use of the
    // loaded words above the later loads (which would wait for the data and serialise them).
    Part x{-INFINITY, 0.f, 0x7fffffff, -INFINITY};
    // Two independent (largest, second largest) chains over even / odd entries (TOP2).
    float ta1 = -INFINITY, ta2 = -INFINITY, tb1 = -INFINITY, tb2 = -INFINITY;
    uint32_t w[kChunks][kVecPerChunk][4];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) load_chunk<RAGGED>(rowp, v0, v1, c, tid, w[c]);
    __builtin_amdgcn_sched_barrier(0);
    auto reduce_chunk = [&](const int c, uint32_t (&w)[kVecPerChunk][4]) __attribute__((always_inline)) {
        finish_chunk<RAGGED>(v0, v1, c, tid, w);
        float vmax[kVecPerChunk];
#pragma unroll
        for (int k = 0; k < kVecPerChunk; ++k) {
            vmax[k] = fmaxf(fmaxf(fmaxf(entry(w[k], 0), entry(w[k], 1)), fmaxf(entry(w[k], 2), entry(w[k], 3))),
                            fmaxf(fmaxf(entry(w[k], 4), entry(w[k], 5)), fmaxf(entry(w[k], 6), entry(w[k], 7))));
        }
        float cm = vmax[0];
#pragma unroll
        for (int k = 1; k < kVecPerChunk; ++k) cm = fmaxf(cm, vmax[k]);
        if (cm > x.m) {
            // New running max: its lowest index in this chunk (first vector, first entry),
            // and the sum so far rescaled to it (0 while the old max is -inf).
            int kk = kVecPerChunk - 1;
#pragma unroll
            for (int k = kVecPerChunk - 2; k >= 0; --k) kk = (vmax[k] == cm) ? k : kk;
            uint32_t sel[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sel[j] = w[kVecPerChunk - 1][j];
#pragma unroll
                for (int k = kVecPerChunk - 2; k >= 0; --k) sel[j] = (kk == k) ? w[k][j] : sel[j];
            }
            int ee = 7;
#pragma unroll
            for (int e = 6; e >= 0; --e) ee = (entry(sel, e) == cm) ? e : ee;
            x.idx = v0 + c * kChunk + 8 * (tid + kThreads * kk) + ee;
            x.s *= __builtin_amdgcn_exp2f(exp_offset(x.m) - exp_offset(cm));   // 0 while x.m = -inf (s = 0)
            x.m = cm;
        }
        if constexpr (TOP2) {
#pragma unroll
            for (int k = 0; k < kVecPerChunk; ++k) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float va = entry(w[k], e), vb = entry(w[k], e + 1);
                    ta2 = __builtin_amdgcn_fmed3f(ta1, va, ta2);
                    ta1 = fmaxf(ta1, va);
                    tb2 = __builtin_amdgcn_fmed3f(tb1, vb, tb2);
                    tb1 = fmaxf(tb1, vb);
                }
            }
        }
        if (x.m != -INFINITY) {
            const float mb = exp_offset(x.m);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int k = 0; k < kVecPerChunk; ++k) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    s0 += __builtin_amdgcn_exp2f(fmaf(entry(w[k], e), kLog2e, -mb));
                    s1 += __builtin_amdgcn_exp2f(fmaf(entry(w[k], e + 1), kLog2e, -mb));
                }
            }
            x.s += s0 + s1;
        }
    };
#pragma unroll
    for (int c = 0; c < kChunks; ++c) reduce_chunk(c, w[c]);
    if constexpr (TOP2) x.m2 = fmaxf(fminf(ta1, tb1), fmaxf(ta2, tb2));

    x = wave_reduce(x);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    if (tid == 0) {
        Part y = red[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) y = merge(y, red[k]);
        p.partial[(int64_t)row * p.split + sl] = float4{y.m, y.s, __int_as_float(y.idx), y.m2};
    }
}

// One workgroup per sequence: one wave per row, lanes over slices (fixed merge order).
// MARGIN: gate on the top-1 minus top-2 probability instead of the top-1 probability.
template <bool MARGIN>
__global__ __launch_bounds__(kThreads) void accept_finish_kernel(AcceptKParams p) {
    __shared__ float row_gate[kMaxWindow];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < p.W; r += kThreads / 64) {
        Part y{-INFINITY, 0.f, 0x7fffffff, -INFINITY};
        const float4* pr = p.partial + ((int64_t)b * p.W + r) * p.split;
        for (int s2 = lane; s2 < p.split; s2 += 64) {
            const float4 q = pr[s2];
            y = merge(y, Part{q.x, q.y, __float_as_int(q.z), q.w});
        }
        y = wave_reduce(y);
        if (lane == 0) {
            const float pm = __builtin_amdgcn_exp2f(fmaf(y.m, kLog2e, -exp_offset(y.m))) / y.s;
            p.tokens[(int64_t)b * p.W + r] = y.idx;
            if (p.pmax) p.pmax[(int64_t)b * p.W + r] = pm;
            if constexpr (MARGIN) {
                // p1 - p2 = (1 - e^(l2 - l1)) / S (0 for a tied maximum)
                const float mg = (1.f - expf(y.m2 - y.m)) * pm;
                row_gate[r] = mg;
                p.margin[(int64_t)b * p.W + r] = mg;
            } else {
                row_gate[r] = pm;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        if (p.tau < 1.f) {
            while (n < p.W && row_gate[n] >= p.tau) ++n;
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
    p.margin = a.margin;
    const dim3 grid((unsigned)(a.batch * a.W), (unsigned)p.split);
    const bool ragged = a.V % 8 != 0;
    if (a.margin) {
        if (!ragged) hipLaunchKernelGGL((accept_slice_kernel<false, true>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((accept_slice_kernel<true, true>), grid, dim3(kThreads), 0, s, p);
    } else {
        if (!ragged) hipLaunchKernelGGL((accept_slice_kernel<false, false>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((accept_slice_kernel<true, false>), grid, dim3(kThreads), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.margin) hipLaunchKernelGGL(accept_finish_kernel<true>, dim3((unsigned)a.batch), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(accept_finish_kernel<false>, dim3((unsigned)a.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mars
