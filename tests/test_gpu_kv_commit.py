"""GPU parity of mars_kv_commit against the oracle (bit for bit: a copy and integer
bookkeeping), and of a short decode loop (decode step -> accept -> commit, repeated)
against the oracle running the same loop."""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import PMAX_ABS, check_close, dev, to_np64

pytestmark = pytest.mark.gpu


def bf16(shape, rng, scale=0.5):
    return I.to_bf16(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


@pytest.mark.parametrize("batch_min", [False, True])
@pytest.mark.parametrize("b,hkv,d,W,cap", [(32, 4, 128, 4, 4096), (5, 2, 64, 7, 40), (3, 1, 128, 64, 200)])
def test_commit_matches_oracle(batch_min, b, hkv, d, W, cap):
    print(f"case commit b={b} hkv={hkv} d={d} W={W} cap={cap} batch_min={batch_min}", flush=True)
    rng = np.random.default_rng(b * 1000 + W + int(batch_min))
    kc, vc = bf16((b, hkv, cap, d), rng), bf16((b, hkv, cap, d), rng)
    kw, vw = bf16((b, W, hkv, d), rng), bf16((b, W, hkv, d), rng)
    lens = rng.integers(0, cap + 1, size=b).astype(np.int32)
    lens[0] = cap - 1                                 # overflow unless n = 1
    nacc = rng.integers(1, W + 1, size=b).astype(np.int32)
    kcd, vcd = kc.to(dev()), vc.to(dev())
    lend = torch.from_numpy(lens).to(dev())
    valid, over = M.mars_kv_commit(kw.to(dev()), vw.to(dev()), torch.from_numpy(nacc).to(dev()), kcd, vcd, lend,
                                   batch_min=batch_min)
    torch.cuda.synchronize()
    rk, rv, rl, rvalid, rover = O.kv_commit(to_np64(kc), to_np64(vc), lens, to_np64(kw), to_np64(vw), nacc,
                                           batch_min=batch_min)
    assert np.array_equal(lend.cpu().numpy(), rl)
    assert np.array_equal(valid.cpu().numpy().astype(np.uint64), rvalid)
    assert np.array_equal(over.cpu().numpy().astype(bool), rover)
    assert np.array_equal(to_np64(kcd), rk) and np.array_equal(to_np64(vcd), rv)


def test_commit_strided_caches_and_views():
    """Caches as head-padded views of larger buffers; the padding is never written."""
    rng = np.random.default_rng(5)
    b, hkv, d, W, cap = 4, 2, 128, 4, 64
    big_k = torch.full((b, hkv + 1, cap, d), 3.0, dtype=torch.bfloat16, device=dev())
    big_v = torch.full((b, hkv + 1, cap, d), 3.0, dtype=torch.bfloat16, device=dev())
    kc, vc = big_k[:, 1:], big_v[:, 1:]
    kw, vw = bf16((b, W, hkv, d), rng).to(dev()), bf16((b, W, hkv, d), rng).to(dev())
    lens = torch.tensor([0, 10, 60, 63], dtype=torch.int32, device=dev())
    nacc = torch.tensor([4, 2, 4, 1], dtype=torch.int32, device=dev())
    valid, over = M.mars_kv_commit(kw, vw, nacc, kc, vc, lens)
    torch.cuda.synchronize()
    assert lens.tolist() == [4, 12, 64, 64] and over.tolist() == [0, 0, 0, 0]
    assert torch.equal(kc[1, :, 10:12], kw[1, :2].permute(1, 0, 2))
    assert torch.all(big_k[:, 0] == 3.0) and torch.all(big_v[:, 0] == 3.0)


def test_decode_loop_matches_oracle():
    """Three rounds of decode step -> accept (tau = 0.3) -> commit on a small batch, fresh
    synthetic proposals each round; every round's outputs and the final caches match the
    oracle running the same loop."""
    rng = np.random.default_rng(11)
    b, hq, hkv, d, W, cap, V = 6, 8, 2, 128, 4, 96, 5000
    kc, vc = bf16((b, hkv, cap, d), rng), bf16((b, hkv, cap, d), rng)
    lens = rng.integers(0, 40, size=b).astype(np.int32)
    kcd, vcd, lend = kc.to(dev()), vc.to(dev()), torch.from_numpy(lens).to(dev())
    kc64, vc64, len64 = to_np64(kc), to_np64(vc), lens.copy()
    for rnd in range(3):
        print(f"case decode loop round {rnd}", flush=True)
        qw, kw, vw = bf16((b, W, hq, d), rng), bf16((b, W, hkv, d), rng), bf16((b, W, hkv, d), rng)
        logits = I.logits_inputs(b, W, V, seed=100 + rnd, spike_hi=20.0)
        o = M.mars_decode_step(qw.to(dev()), kw.to(dev()), vw.to(dev()), kcd, vcd, lend)
        tok, pmax, n = M.mars_accept(logits.to(dev()), 0.3)
        M.mars_kv_commit(kw.to(dev()), vw.to(dev()), n, kcd, vcd, lend)
        torch.cuda.synchronize()
        ro = O.decode(to_np64(qw), to_np64(kw), to_np64(vw), kc64, vc64, len64)
        check_close(to_np64(o), ro, f"loop round {rnd} decode")
        rtok, rpmax, rn = O.accept(to_np64(logits), 0.3)
        assert np.array_equal(tok.cpu().numpy(), rtok)
        assert np.abs(pmax.cpu().numpy() - rpmax).max() <= PMAX_ABS
        # the seeded logits keep every pmax away from tau, so n must agree exactly and the
        # oracle's own loop (driven by its own n) stays in step with the GPU's
        assert np.abs(rpmax - 0.3).min() > 1e-5
        assert np.array_equal(n.cpu().numpy(), rn)
        kc64, vc64, len64, _, _ = O.kv_commit(kc64, vc64, len64, to_np64(kw), to_np64(vw), rn)
        assert np.array_equal(lend.cpu().numpy(), len64)
    assert np.array_equal(to_np64(kcd), kc64) and np.array_equal(to_np64(vcd), vc64)
