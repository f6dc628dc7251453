// Internal launch interface between the C ABI layer (mars_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mars {

// Training-layout forward (attn_fwd.hip).
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // may be null
    int8_t* tilelog;   // may be null (bf16 path only)
    int64_t qs[3], ks[3], vs[3], os[3];
    int batch, hq, hkv, d, P, L, B, N;
    float scale;       // > 0
};

// Geometry of the bf16 forward's row/key grouping (for the tile log).
constexpr int kAttnRowBlock = 32;   // rows per wave
constexpr int kAttnKeyBlock = 32;   // keys per LDS tile

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t s);

// Training-layout backward (attn_bwd.hip): gradients of the bf16 forward.
struct AttnBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;    // fp32 [batch][hq][N], natural log (the forward's output)
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    void* ws;
    int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];
    int batch, hq, hkv, d, P, L, B, N;
    float scale;         // > 0
};
size_t attn_bwd_workspace_bytes(int batch, int hq, int hkv, int d, int P, int L, int B);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t s);
// The dK/dV schedule launch_attn_bwd_bf16 would use (host only).
void attn_bwd_plan(int batch, int hq, int hkv, int d, int P, int L, int B, int* chunk_tiles, int* max_chunks,
                   int64_t* items, int* work_list);

// Debug mask kernels (mask_kernels.hip).
hipError_t launch_mask_materialize(int P, int L, int B, uint8_t* mask, hipStream_t s);
hipError_t launch_tile_map(int P, int L, int B, int bm, int bn, int8_t* map, hipStream_t s);

// Decode step (decode.hip).
struct DecodeArgs {
    const void* qw;
    const void* kw;
    const void* vw;
    const void* kc;
    const void* vc;
    const int32_t* cache_len;
    void* o;
    void* ws;
    int64_t qws[3], kws[3], vws[3], kcs[3], vcs[3], os[3];
    int batch, hq, hkv, d, W, cap;
    float scale;
};
// Decode split: keys per cache chunk (one workgroup each) and the largest cache capacity
// whose chunk count fits the grid's y dimension.
constexpr int kDecodeChunk = 512;
constexpr int64_t kDecodeMaxCapacity = int64_t(65535) * kDecodeChunk;
size_t decode_workspace_bytes(int batch, int hkv, int G, int W, int d, int cap);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Decode step whose partials live in the library's own per-device scratch array (a.ws is
// ignored): at most kDecodeScratchBytes of workspace, no allocation.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t s);

// KV commit and cursor advance (kv_commit.hip).
struct CommitArgs {
    const void* kw;
    const void* vw;
    const int32_t* n_accept;
    void* kc;
    void* vc;
    int32_t* cache_len;
    uint64_t* valid;     // may be null
    int32_t* overflow;   // may be null
    int64_t kws[3], vws[3], kcs[3], vcs[3];
    int batch, hkv, d, W, cap, batch_min;
};
hipError_t launch_kv_commit(const CommitArgs& a, hipStream_t s);

// Right-shifted cross-entropy L_mask + L_AR (shifted_ce.hip).
struct CeArgs {
    const void* logits;
    const int32_t* tokens;
    float* loss_mask;
    float* loss_ar;
    void* dlogits;       // may be null
    void* ws;
    int64_t ls[2], ds[2], ts0;
    int batch, P, L, B, V;
};
size_t shifted_ce_workspace_bytes(int batch, int P, int L);
hipError_t launch_shifted_ce(const CeArgs& a, hipStream_t s);

// Acceptance (accept.hip).
struct AcceptArgs {
    const void* logits;
    int32_t* tokens;
    float* pmax;         // may be null for the margin gate
    float* margin;       // non-null: margin gate (gate on top-1 minus top-2 probability)
    int32_t* n_accept;
    void* ws;
    int64_t batch_stride, row_stride;
    int batch, W, V;
    float tau;
};
size_t accept_workspace_bytes(int batch, int W, int V);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t s);

}  // namespace mars
