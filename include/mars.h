/*
 * mars.h - C ABI of libmars: MARS structured-mask attention on AMD Instinct MI355X (gfx950).
 *
 * The operations follow "MARS: Enabling Autoregressive Models Multi-Token Generation"
 * (arXiv 2604.07023):
 *   - mars_attn_fwd:    one forward of attention over [prompt ; x ; x~] with the
 *                       structured mask M of §3.2, Eq. 2 (training layout);
 *   - mars_attn_bwd:    its gradients dQ, dK, dV (training needs them for the losses of
 *                       §3.2-3.3, Eq. 3 and Eq. 5);
 *   - mars_decode_step: the sliding-window inference step of Fig. 2 (right): B appended
 *                       window rows attend to a per-sequence KV cache and, causally, to
 *                       the window itself;
 *   - mars_accept:      the confidence-threshold rule of the MARS author blog, section
 *                       "Inference: a knob, not a mode switch": commit window positions
 *                       left to right while the top-1 probability is >= tau, at least one;
 *   - mars_accept_margin: the same rule gated on the top-1 minus top-2 probability margin
 *                       (the blog's margin gate);
 *   - mars_kv_commit:   append the accepted window K/V to the caches and advance the
 *                       per-sequence cursors (or all at the batch minimum);
 *   - mars_shifted_ce:  the training loss L_mask + L_AR (§3.2 Eq. 3, §3.3 Eq. 5) over the
 *                       vocabulary, right-shifted logits, optional gradient.
 *
 * Conventions (all entry points):
 *   - Every call returns an int status: MARS_OK (0) or a negative MARS_E* code.
 *   - Descriptors live in host memory and are read during the call only.
 *   - Tensor pointers are device pointers owned by the caller. The library never
 *     allocates, frees or keeps them. Scratch memory comes in as a caller workspace, except
 *     for mars_decode_step_noalloc, which uses a fixed array of the library's own.
 *   - Validation is complete before any launch: on an error nothing is launched and
 *     nothing is written.
 *   - Work is enqueued on the caller's stream and the call returns without a host sync.
 *     A device fault surfaces at the caller's next synchronisation.
 *   - Calls are thread-safe. Two calls that share a workspace must not run concurrently.
 *     The library keeps two pieces of state between calls, both per device: the number of
 *     training-forward workgroups the GPU holds at once, queried from the runtime on the
 *     device's first mars_attn_fwd call and used only to order that kernel's work items
 *     (which items start first; every output is the same whatever the count), and the
 *     device address of mars_decode_step_noalloc's scratch array (see there).
 *   - Strides are in elements. The innermost dimension (head_dim or vocab) is contiguous.
 *     Tensor base pointers must be 16-byte aligned and every stride a multiple of
 *     16 bytes worth of elements (8 for bf16, 4 for fp32); MARS_EINVAL otherwise.
 *   - Outputs are fully overwritten.
 *   - A call with no work (batch == 0, or N == 0 for the forward) returns MARS_OK after
 *     validating the descriptor; its tensor pointers are not inspected and may be NULL.
 *   - bf16 means IEEE binary32 truncated to its top 16 bits (bfloat16); results are
 *     rounded to nearest even when stored as bf16.
 */
#ifndef MARS_H
#define MARS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MARS_ABI_VERSION 1

/* Status codes. */
#define MARS_OK 0
#define MARS_EINVAL (-1)       /* bad shape, enum, tau, null pointer, alignment or stride */
#define MARS_EUNSUPPORTED (-2) /* valid request the library does not implement (head_dim, dtype, window) */
#define MARS_EWORKSPACE (-3)   /* workspace null or smaller than the *_workspace_bytes figure */
#define MARS_EHIP (-4)         /* the HIP runtime reported an error at launch */

/* Element types. */
#define MARS_DTYPE_BF16 0
#define MARS_DTYPE_FP32 1

/* Returns MARS_ABI_VERSION of the loaded library. */
int mars_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* mars_strerror(int status);

/* ------------------------------------------------------------------------------------
 * Training-layout attention (MARS §3.2, Eq. 2; prompt as a causal prefix).
 *
 * Positions 0..N-1, N = prompt_len + 2*resp_len, hold [prompt ; x ; x~]:
 *   prompt  [0, P), clean stream x [P, P+L), noisy stream x~ [P+L, P+2L).
 * Row r sees key j when
 *   r < P + L (prompt or clean row):  j <= r                      (causal)
 *   r >= P + L (noisy row), t0 = r - P - L, k = t0 / block:
 *       j < P + k*block                 (the prompt and clean blocks before block k)
 *    or P + L + k*block <= j <= r        (its own block, causal and self-inclusive)
 * This is Eq. 2 with 1-indexed beta(t) = ceil(t/B) rewritten 0-indexed; a short last
 * block (L % block != 0) is allowed.  Every row sees at least itself.
 *
 * Computes O = softmax(scale * Q K^T + M) V per (batch, query head); query head h
 * reads KV head h / (n_q_heads / n_kv_heads) (grouped-query attention).
 * ------------------------------------------------------------------------------------ */
typedef struct mars_attn_desc {
    int32_t batch;       /* >= 0 (0: nothing to do) */
    int32_t n_q_heads;   /* >= 1, multiple of n_kv_heads */
    int32_t n_kv_heads;  /* >= 1 */
    int32_t head_dim;    /* 64 or 128 */
    int32_t prompt_len;  /* P >= 0 */
    int32_t resp_len;    /* L >= 0; N = P + 2L (N = 0: nothing to do) */
    int32_t block;       /* B >= 1 */
    int32_t dtype;       /* MARS_DTYPE_BF16 (MFMA path) or MARS_DTYPE_FP32 (fp32 vector path) */
    float scale;         /* softmax scale; 0 means 1/sqrt(head_dim); must be finite */
    int32_t reserved;    /* must be 0 */
    int64_t q_strides[3]; /* q [batch][N][n_q_heads][head_dim]: batch, position, head */
    int64_t k_strides[3]; /* k [batch][N][n_kv_heads][head_dim]; position stride (k and v)
                             <= 2^25 elements, else MARS_EUNSUPPORTED */
    int64_t v_strides[3]; /* v [batch][N][n_kv_heads][head_dim] */
    int64_t o_strides[3]; /* o [batch][N][n_q_heads][head_dim] */
} mars_attn_desc;

/*
 * q, k, v: inputs in desc->dtype.  o: output in desc->dtype (bf16 rounded to nearest
 * even).  lse (optional, may be NULL): fp32 [batch][n_q_heads][N], contiguous, the
 * natural-log log-sum-exp of each row's scaled, masked scores.  o must not alias q/k/v.
 */
int mars_attn_fwd(const mars_attn_desc* desc, const void* q, const void* k, const void* v,
                  void* o, float* lse, hipStream_t stream);

/*
 * Host-only work counts for one (batch, query head) of a forward:
 *   *nnz          = visible (query, key) pairs of the mask;
 *   *visible_elems = in-range elements of the bm x bn tiles that are not fully masked.
 * FLOPs of a forward = 4 * head_dim * count * batch * n_q_heads.  Either output may be NULL.
 */
int mars_attn_work(const mars_attn_desc* desc, int32_t bm, int32_t bn, int64_t* nnz,
                   int64_t* visible_elems);

/* Test support: the dense mask, uint8 [N][N] row-major (1 = visible), written on the
 * device by the same visibility predicate the attention kernels use. */
int mars_mask_materialize(const mars_attn_desc* desc, uint8_t* mask, hipStream_t stream);

/* Test support: class of each bm x bn tile of the mask, int8 [ceil(N/bm)][ceil(N/bn)]
 * row-major: 0 every in-range element masked, 2 every one visible, 1 mixed.
 * 1 <= bm, bn <= 1024. */
int mars_tile_map(const mars_attn_desc* desc, int32_t bm, int32_t bn, int8_t* map,
                  hipStream_t stream);

/*
 * Test support: geometry of the bf16 forward's tile log (see mars_attn_fwd_tilelog).
 * The bf16 kernel packs the G = n_q_heads/n_kv_heads query heads of a KV head as rows:
 * row u of a (batch, kv head) pair is position u / G, query head kvh*G + u % G.
 * It walks those rows in groups of *row_block and the keys in groups of *key_block.
 * *rows_per_pair = N * G.  Outputs may be NULL.  MARS_EUNSUPPORTED for fp32.
 */
int mars_attn_tilelog_geometry(const mars_attn_desc* desc, int32_t* row_block,
                               int32_t* key_block, int64_t* rows_per_pair);

/*
 * Test support: mars_attn_fwd (bf16 only) that also records, for every (batch, kv head,
 * row group, key group), how the kernel treated that tile:
 *   0 skipped, 1 computed with the element mask, 2 computed without it (all visible).
 * A key group that runs past position N - 1 is always computed with the mask.
 * tile_log: int8 [batch][n_kv_heads][ceil(N*G/row_block)][ceil(N/key_block)], device;
 * the caller zero-fills it (skipped tiles are not written).
 */
int mars_attn_fwd_tilelog(const mars_attn_desc* desc, const void* q, const void* k,
                          const void* v, void* o, float* lse, int8_t* tile_log,
                          hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Training backward: dQ, dK, dV of mars_attn_fwd (bf16 only).
 *
 * Training takes the losses of MARS §3.2-3.3 (Eq. 3, Eq. 5) through the Eq. 2 attention,
 * so it needs the gradients of that forward.  For one (batch, query head), with P the
 * forward's row probabilities (from the saved LSE), D_i = sum_d dO_id O_id and the chain
 * rule through the row softmax:
 *   dV = P^T dO,   dS = P o (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q;
 * dK and dV of KV head g sum the contributions of its query heads h (g = h / G).
 * Rows and keys outside the mask contribute nothing; skipped tiles are never computed.
 * Precision: bf16 MFMA operands, fp32 accumulation.  Scores are recomputed with one operand
 * times scale*log2(e) rounded to bf16: Q for dQ (as the forward rounds it), K for dK and dV.
 * P and dS enter their products in bf16; results are rounded to nearest even.
 * ------------------------------------------------------------------------------------ */
typedef struct mars_attn_bwd_strides {
    int64_t do_strides[3]; /* d_o [batch][N][n_q_heads][head_dim]: batch, position, head */
    int64_t dq_strides[3]; /* dq  [batch][N][n_q_heads][head_dim] */
    int64_t dk_strides[3]; /* dk  [batch][N][n_kv_heads][head_dim] */
    int64_t dv_strides[3]; /* dv  [batch][N][n_kv_heads][head_dim] */
} mars_attn_bwd_strides;

/* Workspace bytes of mars_attn_bwd for desc (bf16 only; MARS_EUNSUPPORTED for fp32). */
int mars_attn_bwd_workspace_bytes(const mars_attn_desc* desc, size_t* bytes);

/* Test support: the dK/dV schedule mars_attn_bwd launches for desc, computed on the host
 * (nothing is launched or read on the device).  A key block's walk over the position
 * tiles whose rows see its keys is split into at most 8 chunks of at most *chunk_tiles
 * tiles; *max_chunks is the largest chunk count over the key blocks, *items the number of
 * (key block, chunk) chunks that exist, and *work_list 1 when they are dispatched from the
 * host-built longest-first list (items <= 1024), 0 when the grid falls back to the
 * closed-form order (key blocks x max_chunks entries, the missing chunks exiting at once).
 * Errors as mars_attn_bwd_workspace_bytes; MARS_EINVAL for a null output pointer. */
int mars_attn_bwd_plan(const mars_attn_desc* desc, int32_t* chunk_tiles, int32_t* max_chunks, int64_t* items,
                       int32_t* work_list);

/*
 * desc: the forward's descriptor (q/k/v/o strides); dtype must be MARS_DTYPE_BF16.
 * gs:   strides of d_o, dq, dk, dv (same alignment rules as q/k/v/o).
 * q, k, v: the forward's inputs; o and lse: the forward's outputs (lse fp32
 *   [batch][n_q_heads][N], contiguous, as mars_attn_fwd writes it); d_o: dL/dO (bf16).
 * dq, dk, dv: outputs (bf16, rounded to nearest even), fully overwritten; they must not
 *   alias any input or each other.
 * ws: device workspace of at least mars_attn_bwd_workspace_bytes, 16-byte aligned; no
 *   initialisation needed (it holds two fp32 scalars per row, the dK/dV arrival counters,
 *   which the call zeroes itself, and the fp32 partial sums of key blocks whose walk is
 *   split); MARS_EWORKSPACE if null or too small.
 * Errors as mars_attn_fwd; key position strides (k, v) <= 2^25 elements and the q and d_o
 *   position strides <= 2^25 elements, else MARS_EUNSUPPORTED.
 */
int mars_attn_bwd(const mars_attn_desc* desc, const mars_attn_bwd_strides* gs, const void* q,
                  const void* k, const void* v, const void* o, const float* lse, const void* d_o,
                  void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Sliding-window decode step (MARS Fig. 2, right).
 *
 * For sequence b, window row i (0 <= i < window) and query head h (KV head
 * g = h / (n_q_heads / n_kv_heads)) the visible keys are, in order,
 *   cache positions [0, cache_len[b]) of k_cache/v_cache, then window rows 0..i of
 *   k_win/v_win (causal and self-inclusive, like a noisy block of Eq. 2).
 * o[b][i][h] = softmax(scale * q . keys) . values.  The cache is read only; committing
 * accepted window KV into it is the caller's business.
 * ------------------------------------------------------------------------------------ */
typedef struct mars_decode_desc {
    int32_t batch;          /* >= 0 */
    int32_t n_q_heads;      /* >= 1, multiple of n_kv_heads */
    int32_t n_kv_heads;     /* >= 1 */
    int32_t head_dim;       /* 128 or 64 */
    int32_t window;         /* 1 <= window; (n_q_heads/n_kv_heads) * window <= 64 */
    int32_t cache_capacity; /* 0 ..= 65535*512: positions allocated per (sequence, kv head) */
    int32_t dtype;          /* MARS_DTYPE_BF16 */
    float scale;            /* 0 means 1/sqrt(head_dim); must be finite */
    int64_t qw_strides[3];  /* q_win [batch][window][n_q_heads][head_dim]: batch, row, head */
    int64_t kw_strides[3];  /* k_win [batch][window][n_kv_heads][head_dim] */
    int64_t vw_strides[3];  /* v_win */
    int64_t kc_strides[3];  /* k_cache [batch][n_kv_heads][cache_capacity][head_dim]: batch, head, position
                               (position stride <= 2^25 elements, else MARS_EUNSUPPORTED) */
    int64_t vc_strides[3];  /* v_cache */
    int64_t o_strides[3];   /* o [batch][window][n_q_heads][head_dim] */
} mars_decode_desc;

/* Workspace the decode step needs, in bytes (fp32 partial results of the cache split). */
int mars_decode_workspace_bytes(const mars_decode_desc* desc, size_t* bytes);

/*
 * cache_len: int32 [batch] on the device; entries are clamped to [0, cache_capacity]
 * by the kernels (an out-of-range entry never causes an out-of-bounds read).
 * ws: device workspace of at least mars_decode_workspace_bytes; no initialisation needed.
 * o: bf16 output.
 */
int mars_decode_step(const mars_decode_desc* desc, const void* q_win, const void* k_win,
                     const void* v_win, const void* k_cache, const void* v_cache,
                     const int32_t* cache_len, void* o, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * mars_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same descriptor, inputs,
 * output and result as mars_decode_step, but the chunk partials live in a scratch array the
 * library holds on each device it runs on, from the device's first call until the process
 * ends; nothing is allocated or freed by the call.
 *   - The workspace mars_decode_workspace_bytes reports for desc must not exceed the
 *     array's size (mars_decode_scratch_bytes: 32 MiB; e.g. 32 sequences x 4 KV heads x
 *     28 query rows (7 heads x 4 window rows) of head_dim 128 fit up to a cache capacity of
 *     9216 positions), else MARS_EWORKSPACE and nothing is launched.
 *   - Every call on one device shares that device's array: calls that overlap on one GPU
 *     (other streams, other host threads) race and must be ordered by the caller.  The
 *     array needs no initialisation; a call overwrites what it reads.
 *   - The device's first call looks up the array's address (hipGetSymbolAddress); a
 *     runtime error there is MARS_EHIP.
 */
int mars_decode_step_noalloc(const mars_decode_desc* desc, const void* q_win, const void* k_win,
                             const void* v_win, const void* k_cache, const void* v_cache,
                             const int32_t* cache_len, void* o, hipStream_t stream);

/* Size in bytes of mars_decode_step_noalloc's per-device scratch array. */
int mars_decode_scratch_bytes(size_t* bytes);

/* ------------------------------------------------------------------------------------
 * Training loss over the vocabulary (MARS §3.2 Eq. 3 and §3.3 Eq. 5): L = L_mask + L_AR
 * on the logits of one forward over [prompt ; x ; x~] (N = P + 2L rows), right-shifted
 * as in AR training (the row of position p predicts the token at p + 1):
 *   L_AR   = sum over response tokens x_t of CE(row P - 1 + t, x_t)   (no term for t = 0
 *            when P = 0);
 *   L_mask = sum over x_t of CE(noisy row P + L + t - 1, x_t) inside a block, and, for the
 *            first token of each block (t % B == 0: its only fully clean context is the
 *            clean prefix, §3.3 and Eq. 4), CE(clean row P - 1 + t, x_t);
 *   CE(row, y) = logsumexp(row) - row[y]  (natural log).
 * Optionally also dL/dlogits = (w_AR + w_mask) * (softmax(row) - onehot(y)) per row, zero
 * rows where nothing is predicted.
 * ------------------------------------------------------------------------------------ */
typedef struct mars_ce_desc {
    int32_t batch;              /* >= 0, <= 65535 */
    int32_t prompt_len;         /* P >= 0 */
    int32_t resp_len;           /* L >= 0 */
    int32_t block;              /* B >= 1 */
    int32_t vocab;              /* >= 8, a multiple of 8 (16-byte rows), else MARS_EUNSUPPORTED */
    int32_t dtype;              /* MARS_DTYPE_BF16 */
    int64_t logits_strides[2];  /* logits [batch][N][vocab]: batch, position (vocab contiguous) */
    int64_t dlogits_strides[2]; /* dlogits, same shape (used only when dlogits is given) */
    int64_t tokens_stride;      /* tokens int32 [batch][resp_len]: batch stride (elements) */
} mars_ce_desc;

/* Workspace mars_shifted_ce needs, in bytes (one fp32 per (sequence, row)). */
int mars_shifted_ce_workspace_bytes(const mars_ce_desc* desc, size_t* bytes);

/*
 * logits: bf16, finite.  tokens: int32 response tokens x, each in [0, vocab) (a token
 * outside that range is never used as an index: its terms' CE is +inf and its rows'
 * gradient lacks the -w of the target entry).  Outputs on
 * the device: loss_mask, loss_ar fp32 [batch] (sums, summed in a fixed order); dlogits
 * (optional, may be NULL): bf16 gradient of loss_mask + loss_ar.  ws: device workspace of
 * at least mars_shifted_ce_workspace_bytes, no initialisation needed.
 */
int mars_shifted_ce(const mars_ce_desc* desc, const void* logits, const int32_t* tokens, float* loss_mask,
                    float* loss_ar, void* dlogits, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * KV commit and cursor advance (MARS author blog, "Batching is where methods like this
 * usually die": the block-level KV cache advancing at the batch-minimum acceptance, and
 * the deferred-KV sampler with per-sample cursors and a cache-validity bitmask).
 *
 * After acceptance, sequence b appends window rows 0..n_b-1 of k_win / v_win (the K and
 * V of its proposal forward) to k_cache / v_cache at positions cache_len[b] .. +n_b - 1
 * and advances cache_len[b] by n_b, where
 *   n_b = n_accept[b]                      (MARS_COMMIT_PER_SAMPLE: per-sample cursors)
 *   n_b = min over the batch of n_accept   (MARS_COMMIT_BATCH_MIN: the block cache)
 * clamped to [0, window].  If cache_len[b] + n_b > cache_capacity nothing is committed
 * for b (overflow[b] = 1).  valid (optional, uint64 [batch]): bit i set iff window row
 * i of b was committed.  overflow (optional, int32 [batch]).
 * desc: the decode step's descriptor (window, cache and window strides, head_dim); the q
 * and o strides and the scale are not used.  n_accept and cache_len are device int32
 * [batch] (cache_len is read, clamped to [0, cache_capacity], and rewritten).  The window
 * tensors must not overlap the caches.  One launch, no workspace.
 * ------------------------------------------------------------------------------------ */
#define MARS_COMMIT_PER_SAMPLE 0
#define MARS_COMMIT_BATCH_MIN 1
int mars_kv_commit(const mars_decode_desc* desc, const void* k_win, const void* v_win, const int32_t* n_accept,
                   void* k_cache, void* v_cache, int32_t* cache_len, uint64_t* valid, int32_t* overflow,
                   int32_t policy, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Confidence-threshold acceptance (MARS author blog, "Inference: a knob, not a mode
 * switch"; greedy decoding).
 *
 * Per window row (b, i): m = max_v logit, token = lowest v with logit == m,
 * pmax = 1 / sum_v exp(logit_v - m) (temperature-1 softmax over the full vocabulary).
 * Per sequence: n_accept[b] = length of the leading run of rows with pmax >= tau,
 * at least min_accept (= 1); tau = 1 gives exactly 1 (exact AR decoding, also where
 * finite precision rounds some pmax to 1).
 * ------------------------------------------------------------------------------------ */
typedef struct mars_accept_desc {
    int32_t batch;         /* >= 0 */
    int32_t window;        /* 1 <= window <= 64 */
    int32_t vocab;         /* >= 1 */
    int32_t dtype;         /* MARS_DTYPE_BF16 */
    int64_t batch_stride;  /* elements between sequences */
    int64_t row_stride;    /* elements between window rows */
    float tau;             /* 0 < tau <= 1, else MARS_EINVAL (tau == 1 means exact AR: one token) */
    int32_t min_accept;    /* must be 1 */
} mars_accept_desc;

/* Workspace mars_accept needs, in bytes. */
int mars_accept_workspace_bytes(const mars_accept_desc* desc, size_t* bytes);

/*
 * logits: bf16 [batch][window][vocab] (strided as in desc).  Outputs on the device:
 * tokens int32 [batch][window], pmax fp32 [batch][window], n_accept int32 [batch].
 * ws: device workspace of at least mars_accept_workspace_bytes; no initialisation needed.
 * Logits must be finite.
 */
int mars_accept(const mars_accept_desc* desc, const void* logits, int32_t* tokens, float* pmax,
                int32_t* n_accept, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Margin gate (MARS author blog, "Inference: a knob, not a mode switch", second finding:
 * gate on how far the top token is ahead rather than on how confident it is).  Per row,
 * with l1 >= l2 the two largest logits counted with multiplicity (a tied maximum gives
 * l2 = l1) and S = sum_v exp(l_v - l1):
 *   margin = top-1 minus top-2 probability = (1 - exp(l2 - l1)) / S   (in [0, 1)),
 * and n_accept[b] = the leading run of rows with margin >= desc->tau, at least one
 * (tau = 1: exactly one, exact AR decoding).  tokens as mars_accept; pmax (optional,
 * may be NULL) = 1 / S; margin fp32 [batch][window].  Same descriptor, workspace size and
 * errors as mars_accept.
 */
int mars_accept_margin(const mars_accept_desc* desc, const void* logits, int32_t* tokens, float* pmax,
                       float* margin, int32_t* n_accept, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MARS_H */
