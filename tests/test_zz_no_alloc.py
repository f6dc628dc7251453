"""The allocation-free decode step (mars_decode_step_noalloc, for callers that cannot allocate)
against mars_decode_step with a caller workspace: same kernels, so the outputs must agree bit
for bit, and both within the method's bar of the fp64 oracle (MARS Fig. 2 right).  Two calls
in a row on the shared scratch array, the second smaller; a call whose partials would not fit
the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import _lib as L
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import check_close, dev, to_np64

pytestmark = pytest.mark.gpu


def _case(shape, lens):
    x = I.decode_inputs(shape, with_logits=False)
    cl = torch.tensor(lens, dtype=torch.int32)
    t = [x.q_win.to(dev()), x.k_win.to(dev()), x.v_win.to(dev()), x.k_cache.to(dev()), x.v_cache.to(dev()),
         cl.to(dev())]
    return x, cl, t


def test_noalloc_decode_matches_workspace_entry_point():
    big = I.DECODE7B
    small = I.DecodeShape("noalloc_small", 3, 14, 2, 64, 4, 700, 0, 700, 8, 0.95, 0.5, 77)
    cases = [(big, None), (small, [0, 699, 513])]
    assert M.mars_decode_scratch_bytes() >= M.mars_decode_workspace_bytes(big.batch, big.hq, big.hkv, big.d, big.W,
                                                                          big.cap)
    for s, lens in cases:
        print(f"case noalloc decode {s.name} b={s.batch} hq={s.hq} hkv={s.hkv} d={s.d} W={s.W} cap={s.cap}",
              flush=True)
        x, cl, t = _case(s, lens if lens is not None else I.decode_inputs(s, with_logits=False).cache_len.tolist())
        out_na = torch.full_like(t[0], 7.0)
        M.mars_decode_step_noalloc(*t, out=out_na)
        out_ws = M.mars_decode_step(*t)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), f"{s.name}: outputs differ"
        ref = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache),
                       to_np64(x.v_cache), cl.numpy())
        check_close(to_np64(out_na), ref, f"noalloc decode {s.name}")


def test_noalloc_decode_rejects_partials_beyond_the_array():
    """A cache capacity whose chunk partials exceed the scratch array: MARS_EWORKSPACE, nothing
    launched, the output untouched."""
    b, hq, hkv, d, W = 32, 28, 4, 128, 4
    cap = 4096
    while M.mars_decode_workspace_bytes(b, hq, hkv, d, W, cap) <= M.mars_decode_scratch_bytes():
        cap *= 2
    desc = M.decode_desc(b, hq, hkv, d, W, cap)
    buf = torch.zeros(4096, dtype=torch.uint8, device=dev())
    p = buf.data_ptr()
    st = L.load().mars_decode_step_noalloc(ctypes.byref(desc), p, p, p, p, p, p, p, None)
    assert st == L.MARS_EWORKSPACE
    torch.cuda.synchronize()
    assert int(buf.sum()) == 0
