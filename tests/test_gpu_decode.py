"""GPU parity of mars_decode_step against the fp64 oracle (full outputs)."""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import check_close, dev, to_np64

pytestmark = pytest.mark.gpu


def decode_case(batch, hq, hkv, d, W, cap, lens, seed):
    print(f"decode b={batch} hq={hq} hkv={hkv} d={d} W={W} cap={cap} seed={seed}", flush=True)
    s = I.DecodeShape("adhoc", batch, hq, hkv, d, W, cap, 0, max(cap, 0), 8, 0.95, 0.5, seed)
    x = I.decode_inputs(s, with_logits=False)
    cache_len = torch.tensor(lens, dtype=torch.int32)
    out = M.mars_decode_step(x.q_win.to(dev()), x.k_win.to(dev()), x.v_win.to(dev()), x.k_cache.to(dev()),
                             x.v_cache.to(dev()), cache_len.to(dev()))
    torch.cuda.synchronize()
    clamped = np.clip(np.asarray(lens), 0, cap)
    ref = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache), to_np64(x.v_cache),
                   clamped)
    return to_np64(out), ref


@pytest.mark.parametrize("batch,hq,hkv,d,W,cap,lens", [
    (3, 28, 4, 128, 4, 700, [0, 1, 700]),            # empty cache, one key, full cache
    (4, 28, 4, 128, 4, 4096, [512, 4096, 2304, 33]),
    (2, 14, 2, 64, 4, 300, [257, 31]),               # head_dim 64, ragged chunk tails
    (2, 8, 1, 128, 8, 520, [519, 256]),              # G*W = 64 (two column blocks)
    (2, 4, 4, 128, 1, 100, [99, 64]),                # W = 1
    (2, 7, 1, 128, 9, 64, [-5, 1000]),               # out-of-range lengths are clamped
    (1, 2, 2, 64, 3, 0, [0]),                        # no cache at all
])
def test_decode_small(batch, hq, hkv, d, W, cap, lens):
    got, ref = decode_case(batch, hq, hkv, d, W, cap, lens, seed=batch * 100 + W)
    check_close(got, ref, f"decode b{batch} d{d} W{W} cap{cap}")


def test_decode_full_workload():
    s = I.DECODE7B
    x = I.decode_inputs(s, with_logits=False)
    out = M.mars_decode_step(x.q_win.to(dev()), x.k_win.to(dev()), x.v_win.to(dev()), x.k_cache.to(dev()),
                             x.v_cache.to(dev()), x.cache_len.to(dev()))
    torch.cuda.synchronize()
    ref = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache), to_np64(x.v_cache),
                   x.cache_len.numpy())
    check_close(to_np64(out), ref, "decode 7B b32 W4 full")


def test_decode_w1_equals_ar_step_of_training_kernel():
    """W = 1 (no mask slots): the decode row equals the last clean row of a causal forward."""
    b, hq, hkv, d, P, L = 2, 28, 4, 128, 30, 50
    q, k, v = (t.to(dev()) for t in I.small_train_inputs(b, hq, hkv, d, P, L, seed=3))
    o_train = M.mars_attn_fwd(q, k, v, P, L, 4)
    r = P + L - 1
    kc = k[:, :r].permute(0, 2, 1, 3).contiguous()
    vc = v[:, :r].permute(0, 2, 1, 3).contiguous()
    lens = torch.full((b,), r, dtype=torch.int32, device=dev())
    o_dec = M.mars_decode_step(q[:, r:r + 1].contiguous(), k[:, r:r + 1].contiguous(), v[:, r:r + 1].contiguous(),
                               kc, vc, lens)
    torch.cuda.synchronize()
    diff = (o_dec.float() - o_train[:, r:r + 1].float()).abs()
    assert float(diff.max()) <= 2e-2


def test_decode_deterministic():
    """The full 7B decode workload twice, the second time into a workspace filled with garbage
    first (only partials of chunks that exist are read, each written by the same call)."""
    s = I.DECODE7B
    x = I.decode_inputs(s, with_logits=False)
    args = [t.to(dev()) for t in (x.q_win, x.k_win, x.v_win, x.k_cache, x.v_cache, x.cache_len)]
    o1 = M.mars_decode_step(*args)
    ws = torch.full((M.mars_decode_workspace_bytes(s.batch, s.hq, s.hkv, s.d, s.W, s.cap),), 0xA5,
                    dtype=torch.uint8, device=dev())
    o2 = M.mars_decode_step(*args, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("q_gain", [24.0, -24.0])
def test_decode_large_scores_and_late_maxima(q_gain):
    """Scores in the hundreds (Q scaled up), and the largest scores in the last chunk of a
    long cache and in the window: the chunk and window merges must rescale by large
    amounts, and peaked softmax rows make the output follow one or two values."""
    batch, hq, hkv, d, W, cap = 2, 28, 4, 128, 4, 1500
    s = I.DecodeShape("adhoc", batch, hq, hkv, d, W, cap, 0, cap, 8, 0.95, 0.5, 91)
    x = I.decode_inputs(s, with_logits=False)
    q = (x.q_win.float() * q_gain).to(torch.bfloat16)
    kc = x.k_cache.float()
    kc[:, :, 1400:1450] *= 3.0                 # late keys with larger norms (last chunk of sequence 0)
    kc = kc.to(torch.bfloat16)
    kw = (x.k_win.float() * 2.0).to(torch.bfloat16)
    lens = torch.tensor([1500, 700], dtype=torch.int32)
    print(f"case decode large scores gain={q_gain}", flush=True)
    out = M.mars_decode_step(q.to(dev()), kw.to(dev()), x.v_win.to(dev()), kc.to(dev()), x.v_cache.to(dev()),
                             lens.to(dev()))
    torch.cuda.synchronize()
    ref = O.decode(to_np64(q), to_np64(kw), to_np64(x.v_win), to_np64(kc), to_np64(x.v_cache), lens.numpy())
    check_close(to_np64(out), ref, f"decode large scores gain {q_gain}")


def test_decode_strided_views():
    """Caches stored position-major ([b, cap, Hkv, D], the per-token layout, viewed as
    [b, Hkv, cap, D]: position stride Hkv*D, head stride D), window tensors and the output as
    views of larger buffers.  Bit-identical to the contiguous call, and against the oracle; the
    padding around the output view stays untouched."""
    batch, hq, hkv, d, W, cap = 3, 28, 4, 128, 4, 1100
    lens = [1100, 513, 2]
    print(f"case decode strided views cap={cap}", flush=True)
    s = I.DecodeShape("adhoc", batch, hq, hkv, d, W, cap, 0, cap, 8, 0.95, 0.5, 606)
    x = I.decode_inputs(s, with_logits=False)
    cache_len = torch.tensor(lens, dtype=torch.int32, device=dev())
    qw, kw, vw, kc, vc = (t.to(dev()) for t in (x.q_win, x.k_win, x.v_win, x.k_cache, x.v_cache))
    ref = M.mars_decode_step(qw, kw, vw, kc, vc, cache_len)

    def pos_major(c):
        return c.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    def padded_heads(t):
        big = torch.zeros((t.shape[0], t.shape[1], t.shape[2] + 3, d), dtype=t.dtype, device=t.device)
        big[:, :, :t.shape[2]] = t
        return big[:, :, :t.shape[2]]

    kcs, vcs = pos_major(kc), pos_major(vc)
    assert kcs.stride(2) == hkv * d and kcs.stride(1) == d
    obuf = torch.full((batch, W, hq + 3, d), 7.0, dtype=torch.bfloat16, device=dev())
    out = obuf[:, :, :hq]
    M.mars_decode_step(padded_heads(qw), padded_heads(kw), padded_heads(vw), kcs, vcs, cache_len, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.all(obuf[:, :, hq:] == 7.0)
    want = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache), to_np64(x.v_cache),
                    np.asarray(lens))
    check_close(to_np64(out), want, "decode strided views")
