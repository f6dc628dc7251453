// Host-only driver of libmars's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host pass by tests/test_abi_sanitizers.py.  The process
// sees no GPU, so a call that passes validation stops at its launch with MARS_EHIP.
// Every entry point of include/mars.h is called with null, malformed, misaligned, too-small
// and NaN arguments; the host-side work counts run over many shapes.  Exit status 0 iff every
// returned code is the expected one and the sanitizers report nothing.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mars.h"

static int g_fail = 0;
#define EXPECT(call, code)                                                                   \
    do {                                                                                     \
        const int got_ = (call);                                                             \
        if (got_ != (code)) {                                                                \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (int)(code));                                                      \
            ++g_fail;                                                                        \
        }                                                                                    \
    } while (0)

static void* const FAKE = (void*)0x10000;       // aligned, never dereferenced
static void* const MIS = (void*)0x10002;        // misaligned

static mars_attn_desc attn(int b, int hq, int hkv, int d, int P, int L, int B, int dtype = MARS_DTYPE_BF16) {
    mars_attn_desc x;
    memset(&x, 0, sizeof x);
    x.batch = b; x.n_q_heads = hq; x.n_kv_heads = hkv; x.head_dim = d;
    x.prompt_len = P; x.resp_len = L; x.block = B; x.dtype = dtype;
    const int64_t N = (int64_t)P + 2 * L;
    x.q_strides[0] = N * hq * d; x.q_strides[1] = hq * d; x.q_strides[2] = d;
    x.k_strides[0] = N * hkv * d; x.k_strides[1] = hkv * d; x.k_strides[2] = d;
    memcpy(x.v_strides, x.k_strides, sizeof x.k_strides);
    memcpy(x.o_strides, x.q_strides, sizeof x.q_strides);
    return x;
}

static mars_decode_desc dec(int b, int hq, int hkv, int d, int W, int cap) {
    mars_decode_desc x;
    memset(&x, 0, sizeof x);
    x.batch = b; x.n_q_heads = hq; x.n_kv_heads = hkv; x.head_dim = d; x.window = W;
    x.cache_capacity = cap; x.dtype = MARS_DTYPE_BF16;
    x.qw_strides[0] = (int64_t)W * hq * d; x.qw_strides[1] = hq * d; x.qw_strides[2] = d;
    x.kw_strides[0] = (int64_t)W * hkv * d; x.kw_strides[1] = hkv * d; x.kw_strides[2] = d;
    memcpy(x.vw_strides, x.kw_strides, sizeof x.kw_strides);
    x.kc_strides[0] = (int64_t)hkv * cap * d; x.kc_strides[1] = (int64_t)cap * d; x.kc_strides[2] = d;
    memcpy(x.vc_strides, x.kc_strides, sizeof x.kc_strides);
    memcpy(x.o_strides, x.qw_strides, sizeof x.qw_strides);
    return x;
}

static mars_accept_desc acc(int b, int W, int V, float tau) {
    mars_accept_desc x;
    memset(&x, 0, sizeof x);
    x.batch = b; x.window = W; x.vocab = V; x.dtype = MARS_DTYPE_BF16;
    x.batch_stride = (int64_t)W * V; x.row_stride = V; x.tau = tau; x.min_accept = 1;
    return x;
}

static void attention() {
    EXPECT(mars_attn_fwd(nullptr, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    mars_attn_desc d = attn(2, 14, 2, 64, 10, 20, 4);
    mars_attn_desc x = d; x.n_q_heads = 15;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.head_dim = 96;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EUNSUPPORTED);
    x = d; x.scale = NAN;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.scale = INFINITY;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.scale = -1.f;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.reserved = 1;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.block = 0;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.dtype = 7;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.resp_len = 1 << 24;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EUNSUPPORTED);
    x = d; x.q_strides[1] = 7;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    x = d; x.k_strides[1] = (int64_t)1 << 26;
    EXPECT(mars_attn_fwd(&x, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EUNSUPPORTED);
    EXPECT(mars_attn_fwd(&d, MIS, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EINVAL);
    EXPECT(mars_attn_fwd(&d, FAKE, FAKE, FAKE, nullptr, nullptr, nullptr), MARS_EINVAL);
    EXPECT(mars_attn_fwd(&d, FAKE, FAKE, FAKE, FAKE, (float*)MIS, nullptr), MARS_EINVAL);
    x = d; x.batch = 0;
    EXPECT(mars_attn_fwd(&x, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), MARS_OK);
    // Valid descriptors reach the launcher's host code, which stops at the runtime (no GPU).
    EXPECT(mars_attn_fwd(&d, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EHIP);
    mars_attn_desc f = attn(1, 1, 1, 64, 16, 64, 4, MARS_DTYPE_FP32);
    EXPECT(mars_attn_fwd(&f, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr), MARS_EHIP);

    int8_t* log = (int8_t*)FAKE;
    EXPECT(mars_attn_fwd_tilelog(&d, FAKE, FAKE, FAKE, FAKE, nullptr, nullptr, nullptr), MARS_EINVAL);
    EXPECT(mars_attn_fwd_tilelog(&f, FAKE, FAKE, FAKE, FAKE, nullptr, log, nullptr), MARS_EUNSUPPORTED);
    int32_t rb = 0, kb = 0;
    int64_t rows = 0;
    EXPECT(mars_attn_tilelog_geometry(&d, &rb, &kb, &rows), MARS_OK);
    if (rows != (int64_t)(10 + 40) * 7) { fprintf(stderr, "tile log rows %lld\n", (long long)rows); ++g_fail; }
    EXPECT(mars_attn_tilelog_geometry(&f, &rb, &kb, &rows), MARS_EUNSUPPORTED);

    EXPECT(mars_mask_materialize(&d, nullptr, nullptr), MARS_EINVAL);
    x = attn(1, 1, 1, 64, 70000, 0, 1);
    EXPECT(mars_mask_materialize(&x, (uint8_t*)FAKE, nullptr), MARS_EUNSUPPORTED);
    EXPECT(mars_tile_map(&d, 0, 32, (int8_t*)FAKE, nullptr), MARS_EINVAL);
    EXPECT(mars_tile_map(&d, 32, 2048, (int8_t*)FAKE, nullptr), MARS_EINVAL);
    EXPECT(mars_tile_map(&d, 32, 32, nullptr, nullptr), MARS_EINVAL);

    // Host-side work counts over many shapes (integer loops: UBSan checks the arithmetic).
    for (int P = 0; P <= 9; P += 3)
        for (int L = 0; L <= 40; L += 7)
            for (int B = 1; B <= 12; B += 5) {
                if (P + 2 * L == 0) continue;
                mars_attn_desc w = attn(1, 1, 1, 64, P, L, B);
                int64_t nnz = -1, vis = -1;
                EXPECT(mars_attn_work(&w, 16, 48, &nnz, &vis), MARS_OK);
                if (nnz < P + 2 * L || vis < nnz) { fprintf(stderr, "work counts %d %d %d\n", P, L, B); ++g_fail; }
            }
    mars_attn_desc big = attn(1, 28, 4, 128, 1024, 7168, 32);
    int64_t nnz = 0;
    EXPECT(mars_attn_work(&big, 128, 128, &nnz, nullptr), MARS_OK);
    if (nnz != 66592256) { fprintf(stderr, "long layout nnz %lld\n", (long long)nnz); ++g_fail; }
    EXPECT(mars_attn_work(&big, 0, 128, &nnz, nullptr), MARS_EINVAL);

    // Backward.
    mars_attn_bwd_strides gs;
    memcpy(gs.do_strides, d.o_strides, sizeof gs.do_strides);
    memcpy(gs.dq_strides, d.q_strides, sizeof gs.dq_strides);
    memcpy(gs.dk_strides, d.k_strides, sizeof gs.dk_strides);
    memcpy(gs.dv_strides, d.v_strides, sizeof gs.dv_strides);
    size_t need = 0;
    EXPECT(mars_attn_bwd_workspace_bytes(&d, &need), MARS_OK);
    EXPECT(mars_attn_bwd_workspace_bytes(&f, &need), MARS_EUNSUPPORTED);
    EXPECT(mars_attn_bwd_workspace_bytes(&d, nullptr), MARS_EINVAL);
    {
        int32_t tc = 0, nch = 0, wl = 0;
        int64_t items = 0;
        EXPECT(mars_attn_bwd_plan(&d, &tc, &nch, &items, &wl), MARS_OK);
        EXPECT(mars_attn_bwd_plan(&d, nullptr, &nch, &items, &wl), MARS_EINVAL);
        EXPECT(mars_attn_bwd_plan(&d, &tc, &nch, nullptr, &wl), MARS_EINVAL);
        EXPECT(mars_attn_bwd_plan(&f, &tc, &nch, &items, &wl), MARS_EUNSUPPORTED);
        EXPECT(mars_attn_bwd_plan(nullptr, &tc, &nch, &items, &wl), MARS_EINVAL);
        // The largest layout the descriptor allows (2^24 positions, blocks of 1): the host's
        // chunk plan and workspace size in 64-bit arithmetic.
        mars_attn_desc big = d;
        big.prompt_len = (1 << 24) - 2 * 1000;
        big.resp_len = 1000;
        big.block = 1;
        size_t big_need = 0;
        EXPECT(mars_attn_bwd_plan(&big, &tc, &nch, &items, &wl), MARS_OK);
        EXPECT(mars_attn_bwd_workspace_bytes(&big, &big_need), MARS_OK);
        if (items < 1 || wl != (items <= 1024) || big_need < ((size_t)1 << 24) * 8) {
            fprintf(stderr, "implausible plan at 2^24 positions: items %lld, list %d, ws %zu\n", (long long)items,
                    (int)wl, big_need);
            ++g_fail;
        }
    }
    const float* lse = (const float*)FAKE;
    EXPECT(mars_attn_bwd(&d, nullptr, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, FAKE, 1u << 30, nullptr),
           MARS_EINVAL);
    EXPECT(mars_attn_bwd(&d, &gs, FAKE, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, FAKE, FAKE, FAKE, 1u << 30, nullptr),
           MARS_EINVAL);
    EXPECT(mars_attn_bwd(&d, &gs, FAKE, FAKE, FAKE, FAKE, lse, FAKE, MIS, FAKE, FAKE, FAKE, 1u << 30, nullptr),
           MARS_EINVAL);
    EXPECT(mars_attn_bwd(&d, &gs, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, nullptr),
           MARS_EWORKSPACE);
    EXPECT(mars_attn_bwd(&d, &gs, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, nullptr, need, nullptr),
           MARS_EWORKSPACE);
    mars_attn_bwd_strides g2 = gs;
    g2.dk_strides[2] = 3;
    EXPECT(mars_attn_bwd(&d, &g2, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, FAKE, need, nullptr),
           MARS_EINVAL);
    EXPECT(mars_attn_bwd(&f, &gs, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, FAKE, need, nullptr),
           MARS_EUNSUPPORTED);
    EXPECT(mars_attn_bwd(&d, &gs, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE, FAKE, FAKE, FAKE, need, nullptr), MARS_EHIP);
}

static void decode() {
    mars_decode_desc d = dec(32, 28, 4, 128, 4, 4096);
    size_t need = 0;
    EXPECT(mars_decode_workspace_bytes(&d, &need), MARS_OK);
    EXPECT(mars_decode_workspace_bytes(&d, nullptr), MARS_EINVAL);
    const int32_t* lens = (const int32_t*)FAKE;
    EXPECT(mars_decode_step(nullptr, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EINVAL);
    mars_decode_desc x = d;                         // G * W = 17 * 4 = 68 > 64 query rows
    x.n_q_heads = 4 * 17;
    EXPECT(mars_decode_step(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EUNSUPPORTED);
    x = d; x.scale = NAN;
    EXPECT(mars_decode_step(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EINVAL);
    x = d; x.dtype = MARS_DTYPE_FP32;
    EXPECT(mars_decode_step(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EUNSUPPORTED);
    x = d; x.cache_capacity = -1;
    EXPECT(mars_decode_step(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EINVAL);
    x = d; x.kc_strides[2] = (int64_t)1 << 26;
    EXPECT(mars_decode_step(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EUNSUPPORTED);
    EXPECT(mars_decode_step(&d, FAKE, FAKE, FAKE, FAKE, FAKE, (const int32_t*)MIS, FAKE, FAKE, need, nullptr),
           MARS_EINVAL);
    EXPECT(mars_decode_step(&d, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need - 1, nullptr), MARS_EWORKSPACE);
    EXPECT(mars_decode_step(&d, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, nullptr, need, nullptr), MARS_EWORKSPACE);
    x = d; x.batch = 0;
    EXPECT(mars_decode_step(&x, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           MARS_OK);
    EXPECT(mars_decode_step(&d, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, FAKE, need, nullptr), MARS_EHIP);

    size_t scratch = 0;
    EXPECT(mars_decode_scratch_bytes(nullptr), MARS_EINVAL);
    EXPECT(mars_decode_scratch_bytes(&scratch), MARS_OK);
    x = dec(32, 28, 4, 128, 4, 16384);              // partials beyond the scratch array
    EXPECT(mars_decode_step_noalloc(&x, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, nullptr), MARS_EWORKSPACE);
    EXPECT(mars_decode_step_noalloc(&d, FAKE, FAKE, FAKE, FAKE, FAKE, nullptr, FAKE, nullptr), MARS_EINVAL);
    x = d; x.batch = 0;
    EXPECT(mars_decode_step_noalloc(&x, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
           MARS_OK);
    EXPECT(mars_decode_step_noalloc(&d, FAKE, FAKE, FAKE, FAKE, FAKE, lens, FAKE, nullptr), MARS_EHIP);

    int32_t* cl = (int32_t*)FAKE;
    EXPECT(mars_kv_commit(&d, FAKE, FAKE, lens, FAKE, FAKE, cl, nullptr, nullptr, 2, nullptr), MARS_EINVAL);
    EXPECT(mars_kv_commit(&d, FAKE, FAKE, lens, FAKE, FAKE, cl, (uint64_t*)((char*)FAKE + 4), nullptr, 0, nullptr),
           MARS_EINVAL);
    EXPECT(mars_kv_commit(&d, FAKE, FAKE, nullptr, FAKE, FAKE, cl, nullptr, nullptr, 0, nullptr), MARS_EINVAL);
    EXPECT(mars_kv_commit(&d, FAKE, FAKE, lens, FAKE, FAKE, cl, nullptr, nullptr, 1, nullptr), MARS_EHIP);
}

static void accept() {
    mars_accept_desc d = acc(32, 4, 152064, 0.95f);
    size_t need = 0;
    EXPECT(mars_accept_workspace_bytes(&d, &need), MARS_OK);
    const float taus[] = {0.f, -0.5f, NAN, INFINITY, 1.0000002f, 2.f};
    for (float t : taus) {
        mars_accept_desc x = d;
        x.tau = t;
        EXPECT(mars_accept(&x, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr), MARS_EINVAL);
        EXPECT(mars_accept_margin(&x, FAKE, (int32_t*)FAKE, (float*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need,
                                  nullptr),
               MARS_EINVAL);
    }
    mars_accept_desc x = d; x.tau = 1.f;
    EXPECT(mars_accept(&x, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr), MARS_EHIP);
    x = d; x.window = 65;
    EXPECT(mars_accept(&x, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr),
           MARS_EUNSUPPORTED);
    x = d; x.row_stride = 152063;
    EXPECT(mars_accept(&x, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr), MARS_EINVAL);
    EXPECT(mars_accept(&d, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need - 1, nullptr),
           MARS_EWORKSPACE);
    EXPECT(mars_accept(&d, MIS, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr), MARS_EINVAL);
    EXPECT(mars_accept_margin(&d, FAKE, (int32_t*)FAKE, nullptr, nullptr, (int32_t*)FAKE, FAKE, need, nullptr),
           MARS_EINVAL);
    EXPECT(mars_accept(&d, FAKE, (int32_t*)FAKE, (float*)FAKE, (int32_t*)FAKE, FAKE, need, nullptr), MARS_EHIP);
}

static void loss() {
    mars_ce_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 8; d.prompt_len = 256; d.resp_len = 512; d.block = 4; d.vocab = 151936; d.dtype = MARS_DTYPE_BF16;
    d.logits_strides[0] = (int64_t)1280 * 151936; d.logits_strides[1] = 151936;
    memcpy(d.dlogits_strides, d.logits_strides, sizeof d.logits_strides);
    d.tokens_stride = 512;
    size_t need = 0;
    EXPECT(mars_shifted_ce_workspace_bytes(&d, &need), MARS_OK);
    const int32_t* tok = (const int32_t*)FAKE;
    float* fl = (float*)FAKE;
    mars_ce_desc x = d; x.vocab = 151937;
    EXPECT(mars_shifted_ce(&x, FAKE, tok, fl, fl, nullptr, FAKE, need, nullptr), MARS_EUNSUPPORTED);
    EXPECT(mars_shifted_ce(&d, FAKE, tok, nullptr, fl, nullptr, FAKE, need, nullptr), MARS_EINVAL);
    EXPECT(mars_shifted_ce(&d, FAKE, tok, fl, fl, nullptr, FAKE, need - 1, nullptr), MARS_EWORKSPACE);
    EXPECT(mars_shifted_ce(&d, FAKE, tok, fl, fl, MIS, FAKE, need, nullptr), MARS_EINVAL);
    EXPECT(mars_shifted_ce(&d, FAKE, tok, fl, fl, FAKE, FAKE, need, nullptr), MARS_EHIP);
}

int main() {
    if (mars_abi_version() != MARS_ABI_VERSION) ++g_fail;
    for (int c = -5; c <= 1; ++c)
        if (!mars_strerror(c)) ++g_fail;
    attention();
    decode();
    accept();
    loss();
    printf("abi validation: %d failure(s)\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}
