// Debug kernels that expose the device visibility predicate: the dense mask and the
// per-tile class map (MARS §3.2 Eq. 2 with a causal prompt; see mars_device.h).
#include "mars_device.h"
#include "mars_internal.h"

namespace mars {

// One thread per (row, 4 consecutive keys); writes uint8 [N][N].
__global__ void mask_materialize_kernel(int P, int L, int B, int N, uint8_t* __restrict__ mask) {
    const int r = blockIdx.y;
    const RowBounds rb = row_bounds(r, P, L, B);
    for (int j = (blockIdx.x * blockDim.x + threadIdx.x); j < N; j += gridDim.x * blockDim.x) {
        mask[(int64_t)r * N + j] = key_visible(r, j, rb) ? 1 : 0;
    }
}

// One workgroup per tile; every in-range element is evaluated.
__global__ void tile_map_kernel(int P, int L, int B, int N, int bm, int bn, int tiles_n,
                                int8_t* __restrict__ map) {
    const int ta = blockIdx.y, tc = blockIdx.x;
    const int r0 = ta * bm, c0 = tc * bn;
    const int r1 = min(N, r0 + bm), c1 = min(N, c0 + bn);
    const int w = c1 - c0;
    const int64_t elems = (int64_t)(r1 - r0) * w;
    int any = 0, all = 1;
    for (int64_t e = threadIdx.x; e < elems; e += blockDim.x) {
        const int r = r0 + (int)(e / w);
        const int j = c0 + (int)(e % w);
        const bool vis = key_visible(r, j, row_bounds(r, P, L, B));
        any |= vis;
        all &= vis;
    }
    any = __syncthreads_or(any);
    all = __syncthreads_and(all);
    if (threadIdx.x == 0) map[(int64_t)ta * tiles_n + tc] = all ? 2 : (any ? 1 : 0);
}

hipError_t launch_mask_materialize(int P, int L, int B, uint8_t* mask, hipStream_t s) {
    const int N = P + 2 * L;
    if (N == 0) return hipSuccess;
    dim3 grid((N + 255) / 256 < 64 ? (N + 255) / 256 : 64, N);
    hipLaunchKernelGGL(mask_materialize_kernel, grid, dim3(256), 0, s, P, L, B, N, mask);
    return hipGetLastError();
}

hipError_t launch_tile_map(int P, int L, int B, int bm, int bn, int8_t* map, hipStream_t s) {
    const int N = P + 2 * L;
    if (N == 0) return hipSuccess;
    const int ta = (N + bm - 1) / bm, tc = (N + bn - 1) / bn;
    hipLaunchKernelGGL(tile_map_kernel, dim3(tc, ta), dim3(256), 0, s, P, L, B, N, bm, bn, tc, map);
    return hipGetLastError();
}

}  // namespace mars
