// C ABI of libmars (include/mars.h): argument validation, then kernel launches on the
// caller's stream.  Validation is complete before anything is launched, so an error
// leaves every buffer untouched.  Nothing here allocates device memory; the state the library
// keeps is the forward launcher's per-device count of resident workgroups and the per-device
// address of the allocation-free decode step's scratch array.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/mars.h"
#include "mars_device.h"
#include "mars_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides: non-negative and keep 16-byte alignment of every row start.
bool strides_ok(const int64_t s[3], int elem_bytes) {
    const int64_t unit = 16 / elem_bytes;
    for (int i = 0; i < 3; ++i) {
        if (s[i] < 0 || s[i] % unit != 0) return false;
    }
    return true;
}

constexpr int64_t kMaxKeyPosStride = int64_t(1) << 25;

int map_hip(hipError_t e) { return e == hipSuccess ? MARS_OK : MARS_EHIP; }

int check_attn_desc(const mars_attn_desc* d) {
    if (!d) return MARS_EINVAL;
    if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1) return MARS_EINVAL;
    if (d->n_q_heads % d->n_kv_heads != 0) return MARS_EINVAL;
    if (d->prompt_len < 0 || d->resp_len < 0 || d->block < 1) return MARS_EINVAL;
    if (d->reserved != 0) return MARS_EINVAL;
    if (!isfinite(d->scale) || d->scale < 0.f) return MARS_EINVAL;
    if (d->dtype != MARS_DTYPE_BF16 && d->dtype != MARS_DTYPE_FP32) return MARS_EINVAL;
    const int64_t N = (int64_t)d->prompt_len + 2 * (int64_t)d->resp_len;
    if (N > (1 << 24)) return MARS_EUNSUPPORTED;
    if ((int64_t)N * (d->n_q_heads / d->n_kv_heads) > INT32_MAX / 2) return MARS_EUNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return MARS_EUNSUPPORTED;
    return MARS_OK;
}

int64_t attn_N(const mars_attn_desc* d) { return (int64_t)d->prompt_len + 2 * (int64_t)d->resp_len; }

float eff_scale(float scale, int head_dim) { return scale == 0.f ? 1.f / sqrtf((float)head_dim) : scale; }

int check_attn_tensors(const mars_attn_desc* d, const void* q, const void* k, const void* v, const void* o,
                       const float* lse) {
    if (!q || !k || !v || !o) return MARS_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MARS_EINVAL;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return MARS_EINVAL;
    const int eb = d->dtype == MARS_DTYPE_BF16 ? 2 : 4;
    if (!strides_ok(d->q_strides, eb) || !strides_ok(d->k_strides, eb) || !strides_ok(d->v_strides, eb) ||
        !strides_ok(d->o_strides, eb))
        return MARS_EINVAL;
    // The K/V tile copies address 32 positions from one base with 32-bit byte offsets.
    if (d->k_strides[1] > kMaxKeyPosStride || d->v_strides[1] > kMaxKeyPosStride) return MARS_EUNSUPPORTED;
    return MARS_OK;
}

mars::AttnArgs make_attn_args(const mars_attn_desc* d, const void* q, const void* k, const void* v, void* o,
                              float* lse, int8_t* tilelog) {
    mars::AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.tilelog = tilelog;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = d->q_strides[i];
        a.ks[i] = d->k_strides[i];
        a.vs[i] = d->v_strides[i];
        a.os[i] = d->o_strides[i];
    }
    a.batch = d->batch;
    a.hq = d->n_q_heads;
    a.hkv = d->n_kv_heads;
    a.d = d->head_dim;
    a.P = d->prompt_len;
    a.L = d->resp_len;
    a.B = d->block;
    a.N = (int)attn_N(d);
    a.scale = eff_scale(d->scale, d->head_dim);
    return a;
}

}  // namespace

extern "C" {

int mars_abi_version(void) { return MARS_ABI_VERSION; }

const char* mars_strerror(int status) {
    switch (status) {
        case MARS_OK: return "success";
        case MARS_EINVAL: return "invalid argument (shape, enum, tau, null pointer, alignment or stride)";
        case MARS_EUNSUPPORTED: return "unsupported configuration (head_dim, dtype, window or size)";
        case MARS_EWORKSPACE: return "workspace missing or too small";
        case MARS_EHIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int mars_attn_fwd(const mars_attn_desc* desc, const void* q, const void* k, const void* v, void* o, float* lse,
                  hipStream_t stream) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (desc->batch == 0 || attn_N(desc) == 0) return MARS_OK;
    st = check_attn_tensors(desc, q, k, v, o, lse);
    if (st) return st;
    const mars::AttnArgs a = make_attn_args(desc, q, k, v, o, lse, nullptr);
    if (desc->dtype == MARS_DTYPE_BF16) return map_hip(mars::launch_attn_fwd_bf16(a, stream));
    return map_hip(mars::launch_attn_fwd_f32(a, stream));
}

int mars_attn_bwd_workspace_bytes(const mars_attn_desc* desc, size_t* bytes) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (!bytes) return MARS_EINVAL;
    if (desc->dtype != MARS_DTYPE_BF16) return MARS_EUNSUPPORTED;
    *bytes = mars::attn_bwd_workspace_bytes(desc->batch, desc->n_q_heads, desc->n_kv_heads, desc->head_dim,
                                            desc->prompt_len, desc->resp_len, desc->block);
    return MARS_OK;
}

int mars_attn_bwd_plan(const mars_attn_desc* desc, int32_t* chunk_tiles, int32_t* max_chunks, int64_t* items,
                       int32_t* work_list) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (!chunk_tiles || !max_chunks || !items || !work_list) return MARS_EINVAL;
    if (desc->dtype != MARS_DTYPE_BF16) return MARS_EUNSUPPORTED;
    int tc = 0, nch = 0, list = 0;
    int64_t n = 0;
    mars::attn_bwd_plan(desc->batch, desc->n_q_heads, desc->n_kv_heads, desc->head_dim, desc->prompt_len,
                        desc->resp_len, desc->block, &tc, &nch, &n, &list);
    *chunk_tiles = tc;
    *max_chunks = nch;
    *items = n;
    *work_list = list;
    return MARS_OK;
}

int mars_attn_bwd(const mars_attn_desc* desc, const mars_attn_bwd_strides* gs, const void* q, const void* k,
                  const void* v, const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (!gs) return MARS_EINVAL;
    if (desc->dtype != MARS_DTYPE_BF16) return MARS_EUNSUPPORTED;
    if (desc->batch == 0 || attn_N(desc) == 0) return MARS_OK;
    st = check_attn_tensors(desc, q, k, v, o, lse);
    if (st) return st;
    if (!lse || !d_o || !dq || !dk || !dv) return MARS_EINVAL;
    if (!aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return MARS_EINVAL;
    if (!strides_ok(gs->do_strides, 2) || !strides_ok(gs->dq_strides, 2) || !strides_ok(gs->dk_strides, 2) ||
        !strides_ok(gs->dv_strides, 2))
        return MARS_EINVAL;
    // The backward's Q and dO tile copies address 32 positions with 32-bit byte offsets.
    if (gs->do_strides[1] > kMaxKeyPosStride || desc->q_strides[1] > kMaxKeyPosStride) return MARS_EUNSUPPORTED;
    const size_t need = mars::attn_bwd_workspace_bytes(desc->batch, desc->n_q_heads, desc->n_kv_heads,
                                                       desc->head_dim, desc->prompt_len, desc->resp_len, desc->block);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MARS_EWORKSPACE;
    mars::AttnBwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.dout = d_o;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ws = ws;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = desc->q_strides[i];
        a.ks[i] = desc->k_strides[i];
        a.vs[i] = desc->v_strides[i];
        a.os[i] = desc->o_strides[i];
        a.dos[i] = gs->do_strides[i];
        a.dqs[i] = gs->dq_strides[i];
        a.dks[i] = gs->dk_strides[i];
        a.dvs[i] = gs->dv_strides[i];
    }
    a.batch = desc->batch;
    a.hq = desc->n_q_heads;
    a.hkv = desc->n_kv_heads;
    a.d = desc->head_dim;
    a.P = desc->prompt_len;
    a.L = desc->resp_len;
    a.B = desc->block;
    a.N = (int)attn_N(desc);
    a.scale = eff_scale(desc->scale, desc->head_dim);
    return map_hip(mars::launch_attn_bwd_bf16(a, stream));
}

int mars_attn_tilelog_geometry(const mars_attn_desc* desc, int32_t* row_block, int32_t* key_block,
                               int64_t* rows_per_pair) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (desc->dtype != MARS_DTYPE_BF16) return MARS_EUNSUPPORTED;
    if (row_block) *row_block = mars::kAttnRowBlock;
    if (key_block) *key_block = mars::kAttnKeyBlock;
    if (rows_per_pair) *rows_per_pair = attn_N(desc) * (desc->n_q_heads / desc->n_kv_heads);
    return MARS_OK;
}

int mars_attn_fwd_tilelog(const mars_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                          float* lse, int8_t* tile_log, hipStream_t stream) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (desc->dtype != MARS_DTYPE_BF16) return MARS_EUNSUPPORTED;
    if (desc->batch == 0 || attn_N(desc) == 0) return MARS_OK;
    st = check_attn_tensors(desc, q, k, v, o, lse);
    if (st) return st;
    if (!tile_log) return MARS_EINVAL;
    const mars::AttnArgs a = make_attn_args(desc, q, k, v, o, lse, tile_log);
    return map_hip(mars::launch_attn_fwd_bf16(a, stream));
}

int mars_attn_work(const mars_attn_desc* desc, int32_t bm, int32_t bn, int64_t* nnz, int64_t* visible_elems) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (bm < 1 || bn < 1) return MARS_EINVAL;
    const int P = desc->prompt_len, L = desc->resp_len, B = desc->block;
    const int N = (int)attn_N(desc);
    if (nnz) {
        int64_t total = 0;
        for (int r = 0; r < N; ++r) {
            const mars::RowBounds rb = mars::row_bounds(r, P, L, B);
            total += rb.hi1 + std::max(0, r + 1 - rb.lo2);
        }
        *nnz = total;
    }
    if (visible_elems) {
        int64_t total = 0;
        for (int r0 = 0; r0 < N; r0 += bm) {
            const int r1 = std::min(N, r0 + bm);
            for (int c0 = 0; c0 < N; c0 += bn) {
                const int c1 = std::min(N, c0 + bn);
                bool any = false;
                for (int r = r0; r < r1 && !any; ++r) any = mars::range_any(r, c0, c1, mars::row_bounds(r, P, L, B));
                if (any) total += (int64_t)(r1 - r0) * (c1 - c0);
            }
        }
        *visible_elems = total;
    }
    return MARS_OK;
}

int mars_mask_materialize(const mars_attn_desc* desc, uint8_t* mask, hipStream_t stream) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (!mask) return MARS_EINVAL;
    const int64_t N = attn_N(desc);
    if (N > 65535) return MARS_EUNSUPPORTED;
    return map_hip(mars::launch_mask_materialize(desc->prompt_len, desc->resp_len, desc->block, mask, stream));
}

int mars_tile_map(const mars_attn_desc* desc, int32_t bm, int32_t bn, int8_t* map, hipStream_t stream) {
    int st = check_attn_desc(desc);
    if (st) return st;
    if (!map || bm < 1 || bn < 1 || bm > 1024 || bn > 1024) return MARS_EINVAL;
    const int64_t N = attn_N(desc);
    if ((N + bm - 1) / bm > 65535 || (N + bn - 1) / bn > (1 << 30)) return MARS_EUNSUPPORTED;
    return map_hip(mars::launch_tile_map(desc->prompt_len, desc->resp_len, desc->block, bm, bn, map, stream));
}

// ---------------------------------------------------------------------------------------

constexpr int64_t kMaxCachePosStride = int64_t(1) << 25;

static int check_decode_desc(const mars_decode_desc* d) {
    if (!d) return MARS_EINVAL;
    if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->window < 1 || d->cache_capacity < 0)
        return MARS_EINVAL;
    if (d->n_q_heads % d->n_kv_heads != 0) return MARS_EINVAL;
    if (!isfinite(d->scale) || d->scale < 0.f) return MARS_EINVAL;
    if (d->dtype != MARS_DTYPE_BF16) return d->dtype == MARS_DTYPE_FP32 ? MARS_EUNSUPPORTED : MARS_EINVAL;
    if (d->head_dim != 64 && d->head_dim != 128) return MARS_EUNSUPPORTED;
    if ((int64_t)(d->n_q_heads / d->n_kv_heads) * d->window > 64) return MARS_EUNSUPPORTED;
    if (d->batch > 65535 || d->n_kv_heads > 65535) return MARS_EUNSUPPORTED;
    if ((int64_t)d->batch * d->n_kv_heads > INT32_MAX) return MARS_EUNSUPPORTED;
    if (d->cache_capacity > mars::kDecodeMaxCapacity) return MARS_EUNSUPPORTED;
    return MARS_OK;
}

int mars_decode_workspace_bytes(const mars_decode_desc* desc, size_t* bytes) {
    int st = check_decode_desc(desc);
    if (st) return st;
    if (!bytes) return MARS_EINVAL;
    *bytes = mars::decode_workspace_bytes(desc->batch, desc->n_kv_heads, desc->n_q_heads / desc->n_kv_heads,
                                          desc->window, desc->head_dim, desc->cache_capacity);
    return MARS_OK;
}

static int check_decode_call(const mars_decode_desc* desc, const void* q_win, const void* k_win, const void* v_win,
                             const void* k_cache, const void* v_cache, const int32_t* cache_len, const void* o) {
    if (!q_win || !k_win || !v_win || !cache_len || !o) return MARS_EINVAL;
    if (desc->cache_capacity > 0 && (!k_cache || !v_cache)) return MARS_EINVAL;
    if (!aligned16(q_win) || !aligned16(k_win) || !aligned16(v_win) || !aligned16(o) || !aligned16(k_cache) ||
        !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(cache_len) & 3u))
        return MARS_EINVAL;
    if (!strides_ok(desc->qw_strides, 2) || !strides_ok(desc->kw_strides, 2) || !strides_ok(desc->vw_strides, 2) ||
        !strides_ok(desc->kc_strides, 2) || !strides_ok(desc->vc_strides, 2) || !strides_ok(desc->o_strides, 2))
        return MARS_EINVAL;
    // The cache copies address 32 positions from one base with 32-bit byte offsets.
    if (desc->kc_strides[2] > kMaxCachePosStride || desc->vc_strides[2] > kMaxCachePosStride)
        return MARS_EUNSUPPORTED;
    return MARS_OK;
}

static mars::DecodeArgs make_decode_args(const mars_decode_desc* desc, const void* q_win, const void* k_win,
                                         const void* v_win, const void* k_cache, const void* v_cache,
                                         const int32_t* cache_len, void* o, void* ws) {
    mars::DecodeArgs a;
    a.qw = q_win;
    a.kw = k_win;
    a.vw = v_win;
    a.kc = k_cache;
    a.vc = v_cache;
    a.cache_len = cache_len;
    a.o = o;
    a.ws = ws;
    for (int i = 0; i < 3; ++i) {
        a.qws[i] = desc->qw_strides[i];
        a.kws[i] = desc->kw_strides[i];
        a.vws[i] = desc->vw_strides[i];
        a.kcs[i] = desc->kc_strides[i];
        a.vcs[i] = desc->vc_strides[i];
        a.os[i] = desc->o_strides[i];
    }
    a.batch = desc->batch;
    a.hq = desc->n_q_heads;
    a.hkv = desc->n_kv_heads;
    a.d = desc->head_dim;
    a.W = desc->window;
    a.cap = desc->cache_capacity;
    a.scale = eff_scale(desc->scale, desc->head_dim);
    return a;
}

static size_t decode_need(const mars_decode_desc* desc) {
    return mars::decode_workspace_bytes(desc->batch, desc->n_kv_heads, desc->n_q_heads / desc->n_kv_heads,
                                        desc->window, desc->head_dim, desc->cache_capacity);
}

int mars_decode_step(const mars_decode_desc* desc, const void* q_win, const void* k_win, const void* v_win,
                     const void* k_cache, const void* v_cache, const int32_t* cache_len, void* o, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
    int st = check_decode_desc(desc);
    if (st) return st;
    if (desc->batch == 0) return MARS_OK;
    st = check_decode_call(desc, q_win, k_win, v_win, k_cache, v_cache, cache_len, o);
    if (st) return st;
    const size_t need = decode_need(desc);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MARS_EWORKSPACE;
    const mars::DecodeArgs a = make_decode_args(desc, q_win, k_win, v_win, k_cache, v_cache, cache_len, o, ws);
    return map_hip(mars::launch_decode(a, stream));
}

int mars_decode_step_noalloc(const mars_decode_desc* desc, const void* q_win, const void* k_win, const void* v_win,
                             const void* k_cache, const void* v_cache, const int32_t* cache_len, void* o,
                             hipStream_t stream) {
    int st = check_decode_desc(desc);
    if (st) return st;
    if (desc->batch == 0) return MARS_OK;
    st = check_decode_call(desc, q_win, k_win, v_win, k_cache, v_cache, cache_len, o);
    if (st) return st;
    if (decode_need(desc) > mars::kDecodeScratchBytes) return MARS_EWORKSPACE;
    const mars::DecodeArgs a = make_decode_args(desc, q_win, k_win, v_win, k_cache, v_cache, cache_len, o, nullptr);
    return map_hip(mars::launch_decode_noalloc(a, stream));
}

int mars_decode_scratch_bytes(size_t* bytes) {
    if (!bytes) return MARS_EINVAL;
    *bytes = mars::kDecodeScratchBytes;
    return MARS_OK;
}

// ---------------------------------------------------------------------------------------

static int check_accept_desc(const mars_accept_desc* d) {
    if (!d) return MARS_EINVAL;
    if (d->batch < 0 || d->window < 1 || d->vocab < 1) return MARS_EINVAL;
    if (d->window > 64) return MARS_EUNSUPPORTED;
    if (d->vocab > 65535 * 8192) return MARS_EUNSUPPORTED;
    if (d->dtype != MARS_DTYPE_BF16) return d->dtype == MARS_DTYPE_FP32 ? MARS_EUNSUPPORTED : MARS_EINVAL;
    if (!(d->tau > 0.f && d->tau <= 1.f)) return MARS_EINVAL;   // (0, 1]; NaN fails too
    if (d->min_accept != 1) return MARS_EINVAL;
    if (d->batch > 65535) return MARS_EUNSUPPORTED;
    return MARS_OK;
}

int mars_accept_workspace_bytes(const mars_accept_desc* desc, size_t* bytes) {
    int st = check_accept_desc(desc);
    if (st) return st;
    if (!bytes) return MARS_EINVAL;
    *bytes = mars::accept_workspace_bytes(desc->batch, desc->window, desc->vocab);
    return MARS_OK;
}

int mars_accept(const mars_accept_desc* desc, const void* logits, int32_t* tokens, float* pmax, int32_t* n_accept,
                void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_accept_desc(desc);
    if (st) return st;
    if (desc->batch == 0) return MARS_OK;
    if (!logits || !tokens || !pmax || !n_accept) return MARS_EINVAL;
    if (desc->batch_stride < 0 || desc->row_stride < 0 || desc->batch_stride % 8 || desc->row_stride % 8)
        return MARS_EINVAL;
    if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(tokens) & 3u) ||
        (reinterpret_cast<uintptr_t>(pmax) & 3u) || (reinterpret_cast<uintptr_t>(n_accept) & 3u))
        return MARS_EINVAL;
    const size_t need = mars::accept_workspace_bytes(desc->batch, desc->window, desc->vocab);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MARS_EWORKSPACE;
    mars::AcceptArgs a;
    a.logits = logits;
    a.tokens = tokens;
    a.pmax = pmax;
    a.margin = nullptr;
    a.n_accept = n_accept;
    a.ws = ws;
    a.batch_stride = desc->batch_stride;
    a.row_stride = desc->row_stride;
    a.batch = desc->batch;
    a.W = desc->window;
    a.V = desc->vocab;
    a.tau = desc->tau;
    return map_hip(mars::launch_accept(a, stream));
}

int mars_accept_margin(const mars_accept_desc* desc, const void* logits, int32_t* tokens, float* pmax,
                       float* margin, int32_t* n_accept, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_accept_desc(desc);
    if (st) return st;
    if (desc->batch == 0) return MARS_OK;
    if (!logits || !tokens || !margin || !n_accept) return MARS_EINVAL;
    if (desc->batch_stride < 0 || desc->row_stride < 0 || desc->batch_stride % 8 || desc->row_stride % 8)
        return MARS_EINVAL;
    if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(tokens) & 3u) ||
        (reinterpret_cast<uintptr_t>(pmax) & 3u) || (reinterpret_cast<uintptr_t>(margin) & 3u) ||
        (reinterpret_cast<uintptr_t>(n_accept) & 3u))
        return MARS_EINVAL;
    const size_t need = mars::accept_workspace_bytes(desc->batch, desc->window, desc->vocab);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MARS_EWORKSPACE;
    mars::AcceptArgs a;
    a.logits = logits;
    a.tokens = tokens;
    a.pmax = pmax;
    a.margin = margin;
    a.n_accept = n_accept;
    a.ws = ws;
    a.batch_stride = desc->batch_stride;
    a.row_stride = desc->row_stride;
    a.batch = desc->batch;
    a.W = desc->window;
    a.V = desc->vocab;
    a.tau = desc->tau;
    return map_hip(mars::launch_accept(a, stream));
}

int mars_kv_commit(const mars_decode_desc* desc, const void* k_win, const void* v_win, const int32_t* n_accept,
                   void* k_cache, void* v_cache, int32_t* cache_len, uint64_t* valid, int32_t* overflow,
                   int32_t policy, hipStream_t stream) {
    int st = check_decode_desc(desc);
    if (st) return st;
    if (policy != MARS_COMMIT_PER_SAMPLE && policy != MARS_COMMIT_BATCH_MIN) return MARS_EINVAL;
    if (desc->batch == 0) return MARS_OK;
    if (!k_win || !v_win || !n_accept || !cache_len) return MARS_EINVAL;
    if (desc->cache_capacity > 0 && (!k_cache || !v_cache)) return MARS_EINVAL;
    if (!aligned16(k_win) || !aligned16(v_win) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(n_accept) & 3u) || (reinterpret_cast<uintptr_t>(cache_len) & 3u) ||
        (reinterpret_cast<uintptr_t>(valid) & 7u) || (reinterpret_cast<uintptr_t>(overflow) & 3u))
        return MARS_EINVAL;
    if (!strides_ok(desc->kw_strides, 2) || !strides_ok(desc->vw_strides, 2) || !strides_ok(desc->kc_strides, 2) ||
        !strides_ok(desc->vc_strides, 2))
        return MARS_EINVAL;
    mars::CommitArgs a;
    a.kw = k_win;
    a.vw = v_win;
    a.n_accept = n_accept;
    a.kc = k_cache;
    a.vc = v_cache;
    a.cache_len = cache_len;
    a.valid = valid;
    a.overflow = overflow;
    for (int i = 0; i < 3; ++i) {
        a.kws[i] = desc->kw_strides[i];
        a.vws[i] = desc->vw_strides[i];
        a.kcs[i] = desc->kc_strides[i];
        a.vcs[i] = desc->vc_strides[i];
    }
    a.batch = desc->batch;
    a.hkv = desc->n_kv_heads;
    a.d = desc->head_dim;
    a.W = desc->window;
    a.cap = desc->cache_capacity;
    a.batch_min = policy == MARS_COMMIT_BATCH_MIN ? 1 : 0;
    return map_hip(mars::launch_kv_commit(a, stream));
}

static int check_ce_desc(const mars_ce_desc* d) {
    if (!d) return MARS_EINVAL;
    if (d->batch < 0 || d->prompt_len < 0 || d->resp_len < 0 || d->block < 1 || d->vocab < 1) return MARS_EINVAL;
    if (d->dtype != MARS_DTYPE_BF16) return d->dtype == MARS_DTYPE_FP32 ? MARS_EUNSUPPORTED : MARS_EINVAL;
    if (d->vocab % 8 != 0) return MARS_EUNSUPPORTED;
    if (d->batch > 65535) return MARS_EUNSUPPORTED;
    if ((int64_t)d->prompt_len + 2 * (int64_t)d->resp_len > (1 << 24)) return MARS_EUNSUPPORTED;
    return MARS_OK;
}

int mars_shifted_ce_workspace_bytes(const mars_ce_desc* desc, size_t* bytes) {
    const int st = check_ce_desc(desc);
    if (st) return st;
    if (!bytes) return MARS_EINVAL;
    *bytes = mars::shifted_ce_workspace_bytes(desc->batch, desc->prompt_len, desc->resp_len);
    return MARS_OK;
}

int mars_shifted_ce(const mars_ce_desc* desc, const void* logits, const int32_t* tokens, float* loss_mask,
                    float* loss_ar, void* dlogits, void* ws, size_t ws_bytes, hipStream_t stream) {
    const int st = check_ce_desc(desc);
    if (st) return st;
    if (desc->batch == 0) return MARS_OK;
    if (!loss_mask || !loss_ar) return MARS_EINVAL;
    const int64_t N = (int64_t)desc->prompt_len + 2 * (int64_t)desc->resp_len;
    if (N > 0 && (!logits || (desc->resp_len > 0 && !tokens))) return MARS_EINVAL;
    if (!aligned16(logits) || !aligned16(dlogits) || (reinterpret_cast<uintptr_t>(tokens) & 3u) ||
        (reinterpret_cast<uintptr_t>(loss_mask) & 3u) || (reinterpret_cast<uintptr_t>(loss_ar) & 3u))
        return MARS_EINVAL;
    for (int i = 0; i < 2; ++i) {
        if (desc->logits_strides[i] < 0 || desc->logits_strides[i] % 8) return MARS_EINVAL;
        if (dlogits && (desc->dlogits_strides[i] < 0 || desc->dlogits_strides[i] % 8)) return MARS_EINVAL;
    }
    if (desc->tokens_stride < 0) return MARS_EINVAL;
    const size_t need = mars::shifted_ce_workspace_bytes(desc->batch, desc->prompt_len, desc->resp_len);
    if (need > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 3u))) return MARS_EWORKSPACE;
    mars::CeArgs a;
    a.logits = logits;
    a.tokens = tokens;
    a.loss_mask = loss_mask;
    a.loss_ar = loss_ar;
    a.dlogits = dlogits;
    a.ws = ws;
    a.ls[0] = desc->logits_strides[0];
    a.ls[1] = desc->logits_strides[1];
    a.ds[0] = desc->dlogits_strides[0];
    a.ds[1] = desc->dlogits_strides[1];
    a.ts0 = desc->tokens_stride;
    a.batch = desc->batch;
    a.P = desc->prompt_len;
    a.L = desc->resp_len;
    a.B = desc->block;
    a.V = desc->vocab;
    return map_hip(mars::launch_shifted_ce(a, stream));
}

}  // extern "C"
