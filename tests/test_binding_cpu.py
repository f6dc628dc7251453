"""CPU-only checks of the Python binding's argument validation: every wrapper rejects a wrong
dtype (TypeError), a wrong shape, a non-contiguous dense output, or a host tensor (ValueError)
before anything reaches the C ABI.  Host tensors stand in for device ones, so a call that got
past the checks would fail loudly here rather than run."""
import pytest
import torch

import structured_mask_attention_amd as M

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def t(shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_attn_fwd_arguments():
    q, k = t((1, 10, 4, 64)), t((1, 10, 2, 64))
    with pytest.raises(TypeError, match="q must have dtype"):
        M.mars_attn_fwd(q.half(), k, k, 2, 4, 2)
    with pytest.raises(TypeError, match="k must have dtype"):
        M.mars_attn_fwd(q, k.float(), k, 2, 4, 2)
    with pytest.raises(ValueError, match="v must have shape"):
        M.mars_attn_fwd(q, k, t((1, 10, 1, 64)), 2, 4, 2)
    with pytest.raises(ValueError, match="sequence length"):
        M.mars_attn_fwd(q, k, k, 2, 3, 2)
    with pytest.raises(ValueError, match="lse must have shape"):
        M.mars_attn_fwd(q, k, k, 2, 4, 2, lse=t((1, 10, 4), f32))
    with pytest.raises(TypeError, match="lse must have dtype"):
        M.mars_attn_fwd(q, k, k, 2, 4, 2, lse=t((1, 4, 10), bf))
    with pytest.raises(ValueError, match="lse must be contiguous"):
        M.mars_attn_fwd(q, k, k, 2, 4, 2, lse=t((1, 10, 4), f32).transpose(1, 2))
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_attn_fwd(q, k, k, 2, 4, 2)
    with pytest.raises(TypeError, match="q must have dtype"):
        M.mars_attn_fwd_tilelog(q.float(), k.float(), k.float(), 2, 4, 2)


def test_attn_bwd_arguments():
    q, k = t((1, 10, 4, 64)), t((1, 10, 2, 64))
    lse = t((1, 4, 10), f32)
    with pytest.raises(TypeError, match="q must have dtype"):
        M.mars_attn_bwd(q.float(), k.float(), k.float(), q.float(), lse, q.float(), 2, 4, 2)
    with pytest.raises(TypeError, match="dout must have dtype"):
        M.mars_attn_bwd(q, k, k, q, lse, q.float(), 2, 4, 2)
    with pytest.raises(ValueError, match="dk must have shape"):
        M.mars_attn_bwd(q, k, k, q, lse, q, 2, 4, 2, dk=t((1, 10, 4, 64)))
    with pytest.raises(ValueError, match="lse .* is required"):
        M.mars_attn_bwd(q, k, k, q, None, q, 2, 4, 2)
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_attn_bwd(q, k, k, q, lse, q, 2, 4, 2)


def test_decode_arguments():
    b, W, hq, hkv, d, cap = 2, 4, 28, 4, 128, 64
    qw, kw, kc = t((b, W, hq, d)), t((b, W, hkv, d)), t((b, hkv, cap, d))
    lens = t((b,), i32)
    with pytest.raises(TypeError, match="q_win must have dtype"):
        M.mars_decode_step(qw.float(), kw, kw, kc, kc, lens)
    with pytest.raises(TypeError, match="v_cache must have dtype"):
        M.mars_decode_step(qw, kw, kw, kc, kc.half(), lens)
    with pytest.raises(TypeError, match="cache_len must have dtype"):
        M.mars_decode_step(qw, kw, kw, kc, kc, lens.long())
    with pytest.raises(ValueError, match="cache_len must have shape"):
        M.mars_decode_step(qw, kw, kw, kc, kc, t((b + 1,), i32))
    with pytest.raises(ValueError, match="cache_len must be contiguous"):
        M.mars_decode_step(qw, kw, kw, kc, kc, t((2 * b,), i32)[::2])
    with pytest.raises(ValueError, match="k_win must have shape"):
        M.mars_decode_step(qw, t((b, W, hkv + 1, d)), kw, kc, kc, lens)
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_decode_step(qw, kw, kw, kc, kc, lens)


def test_accept_arguments():
    lg = t((2, 4, 1000))
    with pytest.raises(TypeError, match="logits must have dtype"):
        M.mars_accept(lg.float(), 0.9)
    with pytest.raises(TypeError, match="logits must have dtype"):
        M.mars_accept_margin(lg.half(), 0.9)
    with pytest.raises(ValueError, match="logits must be"):
        M.mars_accept(t((8, 1000)), 0.9)
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_accept(lg, 0.9)
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_accept_margin(lg, 0.9)


def test_kv_commit_arguments():
    b, W, hkv, d, cap = 2, 4, 4, 128, 64
    kw, kc, n, lens = t((b, W, hkv, d)), t((b, hkv, cap, d)), t((b,), i32), t((b,), i32)
    with pytest.raises(TypeError, match="n_accept must have dtype"):
        M.mars_kv_commit(kw, kw, n.long(), kc, kc, lens)
    with pytest.raises(ValueError, match="n_accept must have shape"):
        M.mars_kv_commit(kw, kw, t((b, 1), i32), kc, kc, lens)
    with pytest.raises(TypeError, match="cache_len must have dtype"):
        M.mars_kv_commit(kw, kw, n, kc, kc, lens.float())
    with pytest.raises(TypeError, match="k_cache must have dtype"):
        M.mars_kv_commit(kw, kw, n, kc.float(), kc, lens)
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_kv_commit(kw, kw, n, kc, kc, lens)


def test_shifted_ce_arguments():
    b, P, L, V = 2, 3, 5, 64
    lg, tok = t((b, P + 2 * L, V)), t((b, L), i32)
    with pytest.raises(TypeError, match="logits must have dtype"):
        M.mars_shifted_ce(lg.float(), tok, P, L, 2)
    with pytest.raises(TypeError, match="tokens must have dtype"):
        M.mars_shifted_ce(lg, tok.long(), P, L, 2)
    with pytest.raises(ValueError, match="tokens must have shape"):
        M.mars_shifted_ce(lg, t((b, L + 1), i32), P, L, 2)
    with pytest.raises(ValueError, match="logits rows"):
        M.mars_shifted_ce(lg, tok, P + 1, L, 2)
    with pytest.raises(TypeError, match="dlogits must have dtype"):
        M.mars_shifted_ce(lg, tok, P, L, 2, dlogits=lg.float())
    with pytest.raises(ValueError, match="must be a device"):
        M.mars_shifted_ce(lg, tok, P, L, 2)
