// KV commit and cursor advance for the sliding-window decode loop (MARS author blog,
// "Batching is where methods like this usually die": the block-level KV cache that
// advances at the batch-minimum acceptance, and the deferred-KV sampler with per-sample
// cursors and a cache-validity bitmask).
//
// After acceptance, sequence b appends its accepted window rows 0..n_b-1 (their K and V
// from the proposal forward) to its cache at its cursor cache_len[b] and advances the
// cursor by n_b; n_b = n_accept[b] (per-sample cursors) or the batch minimum of
// n_accept (every sequence advances together).  A sequence whose cache cannot hold n_b
// more rows commits nothing and reports an overflow.  valid[b] gets bit i set iff window
// row i was committed.
//
// One workgroup per sequence copies all of its KV heads (16-byte chunks, a handful of
// KB) and is the only writer of that sequence's cursor, so the cursor is read by every
// thread, the block synchronises, and one thread writes the new value.
#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

namespace {

constexpr int kThreads = 256;

struct CommitParams {
    const uint16_t* kw;
    const uint16_t* vw;
    const int32_t* n_accept;
    uint16_t* kc;
    uint16_t* vc;
    int32_t* cache_len;
    uint64_t* valid;     // may be null
    int32_t* overflow;   // may be null
    int64_t kws0, kws1, kws2, vws0, vws1, vws2, kcs0, kcs1, kcs2, vcs0, vcs1, vcs2;
    int batch, hkv, d, W, cap, batch_min;
};

__global__ __launch_bounds__(kThreads) void kv_commit_kernel(CommitParams p) {
    __shared__ int s_min[kThreads / 64];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;

    // n for this sequence: its own acceptance, or the batch minimum.
    int n;
    if (p.batch_min) {
        int m = 0x7fffffff;
        for (int i = tid; i < p.batch; i += kThreads) m = min(m, p.n_accept[i]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = min(m, __shfl_xor(m, off));
        if ((tid & 63) == 0) s_min[tid >> 6] = m;
        __syncthreads();
        m = s_min[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) m = min(m, s_min[w]);
        n = m;
    } else {
        n = p.n_accept[b];
    }
    n = max(0, min(n, p.W));
    int len = p.cache_len[b];
    len = max(0, min(len, p.cap));
    const bool fits = len + n <= p.cap;
    __syncthreads();   // every thread has read the cursor before it is rewritten

    if (fits) {
        const int cpr = p.d / 8;                        // 16-byte chunks per row
        const int total = n * p.hkv * cpr;
        for (int c = tid; c < total; c += kThreads) {
            const int ch = c % cpr;
            const int rg = c / cpr;
            const int g = rg % p.hkv, i = rg / p.hkv;
            const uint4 kx = *reinterpret_cast<const uint4*>(p.kw + b * p.kws0 + (int64_t)i * p.kws1 + (int64_t)g * p.kws2 + 8 * ch);
            const uint4 vx = *reinterpret_cast<const uint4*>(p.vw + b * p.vws0 + (int64_t)i * p.vws1 + (int64_t)g * p.vws2 + 8 * ch);
            *reinterpret_cast<uint4*>(p.kc + b * p.kcs0 + (int64_t)g * p.kcs1 + (int64_t)(len + i) * p.kcs2 + 8 * ch) = kx;
            *reinterpret_cast<uint4*>(p.vc + b * p.vcs0 + (int64_t)g * p.vcs1 + (int64_t)(len + i) * p.vcs2 + 8 * ch) = vx;
        }
    }
    if (tid == 0) {
        if (fits) p.cache_len[b] = len + n;
        if (p.valid) p.valid[b] = fits ? (n >= 64 ? ~0ull : ((1ull << n) - 1ull)) : 0ull;
        if (p.overflow) p.overflow[b] = fits ? 0 : 1;
    }
}

}  // namespace

hipError_t launch_kv_commit(const CommitArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    CommitParams p;
    p.kw = static_cast<const uint16_t*>(a.kw);
    p.vw = static_cast<const uint16_t*>(a.vw);
    p.n_accept = a.n_accept;
    p.kc = static_cast<uint16_t*>(a.kc);
    p.vc = static_cast<uint16_t*>(a.vc);
    p.cache_len = a.cache_len;
    p.valid = a.valid;
    p.overflow = a.overflow;
    p.kws0 = a.kws[0]; p.kws1 = a.kws[1]; p.kws2 = a.kws[2];
    p.vws0 = a.vws[0]; p.vws1 = a.vws[1]; p.vws2 = a.vws[2];
    p.kcs0 = a.kcs[0]; p.kcs1 = a.kcs[1]; p.kcs2 = a.kcs[2];
    p.vcs0 = a.vcs[0]; p.vcs1 = a.vcs[1]; p.vcs2 = a.vcs[2];
    p.batch = a.batch;
    p.hkv = a.hkv;
    p.d = a.d;
    p.W = a.W;
    p.cap = a.cap;
    p.batch_min = a.batch_min;
    hipLaunchKernelGGL(kv_commit_kernel, dim3((unsigned)a.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mars
