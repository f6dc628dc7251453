"""CPU-only checks of the C ABI: the library loads, exports every declared entry point,
validates arguments before launching anything, and its host-side work counts agree with
the oracle.  No call here reaches a kernel launch (no GPU is needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000           # aligned dummy device address (never dereferenced: validation fails first)
MISALIGNED = 0x10002


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mars.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mars_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = L.load()
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.exported_symbols()) == names
    assert M.mars_abi_version() == 1


def test_strerror_codes():
    for code in (0, -1, -2, -3, -4):
        assert M.mars_strerror(code) and M.mars_strerror(code) != "unknown status"
    assert M.mars_strerror(-99) == "unknown status"


@pytest.mark.parametrize("P,Lr,B", [(16, 64, 4), (256, 512, 4), (512, 1536, 8), (3, 37, 8), (0, 1, 1), (5, 0, 2)])
def test_attn_work_matches_oracle(P, Lr, B):
    nnz, vis = M.mars_attn_work(1, 1, 1, 64, P, Lr, B, 128, 128)
    assert nnz == O.mask_nnz(P, Lr, B)
    assert vis == O.visible_tile_elems(P, Lr, B, 128, 128)
    nnz2, vis2 = M.mars_attn_work(1, 1, 1, 64, P, Lr, B, 16, 48)
    assert vis2 == O.visible_tile_elems(P, Lr, B, 16, 48)


# Keys per dK/dV workgroup of the backward (192 at head_dim 128, 128 at head_dim 64) and the
# kernels' 32-position tiles: the geometry mars_attn_bwd_plan counts in.
BWD_KEYS_PER_WG = {64: 128, 128: 192}


@pytest.mark.parametrize("d,P,Lr,B", [(64, 40, 150, 4), (128, 33, 700, 8), (64, 130, 120, 4), (128, 0, 300, 1),
                                      (64, 1000, 3000, 16), (128, 5, 37, 64)])
def test_bwd_plan_items_brute_force(d, P, Lr, B):
    """The backward's dK/dV work items: for every key block, the 32-position tiles holding a row
    that sees one of its keys, counted on the oracle's dense mask (tile classes of 32 x keys-per-
    workgroup tiles), split into min(8, max(1, ceil(tiles / chunk_tiles))) chunks."""
    plan = M.mars_attn_bwd_plan(2, 4, 2, d, P, Lr, B)
    kpb = BWD_KEYS_PER_WG[d]
    tiles = (O.tile_map(O.mask_rules(P, Lr, B), 32, kpb) != 0).sum(axis=0)
    tc = plan["chunk_tiles"]
    assert tc >= 4
    chunks = np.minimum(8, np.maximum(1, -(-tiles // tc)))
    assert plan["items"] == int(chunks.sum())
    assert plan["max_chunks"] == int(chunks.max())
    assert plan["work_list"] == (plan["items"] <= 1024)


def test_bwd_plan_work_list_limit():
    """The two head_dim 64 layouts the GPU tests run on either side of the 1024-entry work
    list: N = 16512 has 129 key blocks x 8 chunks > 1024 but only 804 chunks that exist (list);
    N = 26128 has 1064 (closed-form order).  The bench's three training layouts use the list."""
    a = M.mars_attn_bwd_plan(1, 2, 1, 64, 16384, 64, 8)
    assert (a["max_chunks"], a["items"], a["work_list"]) == (8, 804, True)
    assert 129 * a["max_chunks"] > 1024
    b = M.mars_attn_bwd_plan(1, 2, 1, 64, 26000, 64, 8)
    assert (b["items"], b["work_list"]) == (1064, False)
    for bt, hq, hkv, d, P, Lr, B in [(1, 28, 4, 128, 1024, 7168, 32), (4, 28, 4, 128, 512, 1536, 8),
                                     (8, 14, 2, 64, 256, 512, 4)]:
        assert M.mars_attn_bwd_plan(bt, hq, hkv, d, P, Lr, B)["work_list"]
    with pytest.raises(M.MarsError):
        M.mars_attn_bwd_plan(1, 2, 1, 96, 16, 16, 4)


def _attn(desc, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None):
    return L.load().mars_attn_fwd(ctypes.byref(desc), q, k, v, o, lse, None)


def test_attn_validation_errors():
    lib = L.load()
    assert lib.mars_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None) == L.MARS_EINVAL
    good = lambda: M.attn_desc(2, 14, 2, 64, 10, 20, 4)
    d = good(); d.n_q_heads = 15
    assert _attn(d) == L.MARS_EINVAL                      # Hq % Hkv
    d = good(); d.head_dim = 96
    assert _attn(d) == L.MARS_EUNSUPPORTED
    d = good(); d.v_strides[1] = (1 << 25) + 8             # 32 positions overflow 32-bit offsets
    assert _attn(d) == L.MARS_EUNSUPPORTED
    d = good(); d.block = 0
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.resp_len = -1
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.dtype = 7
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.scale = float("nan")
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.scale = -1.0
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.reserved = 1
    assert _attn(d) == L.MARS_EINVAL
    assert _attn(good(), q=None) == L.MARS_EINVAL
    assert _attn(good(), o=MISALIGNED) == L.MARS_EINVAL
    d = good(); d.k_strides[1] = 2 * 64 + 4                # row start loses 16-byte alignment
    assert _attn(d) == L.MARS_EINVAL
    d = good(); d.q_strides[0] = -8
    assert _attn(d) == L.MARS_EINVAL
    assert _attn(good(), lse=FAKE + 2) == L.MARS_EINVAL
    # empty work: OK without touching pointers
    d = good(); d.batch = 0
    assert _attn(d, q=None, k=None, v=None, o=None) == L.MARS_OK
    d = good(); d.prompt_len = 0; d.resp_len = 0
    assert _attn(d, q=None, k=None, v=None, o=None) == L.MARS_OK
    # fp32 tile log unsupported; tile map bounds
    d = good(); d.dtype = L.MARS_DTYPE_FP32
    assert lib.mars_attn_fwd_tilelog(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == L.MARS_EUNSUPPORTED
    assert lib.mars_tile_map(ctypes.byref(good()), 0, 16, FAKE, None) == L.MARS_EINVAL
    assert lib.mars_tile_map(ctypes.byref(good()), 16, 2048, FAKE, None) == L.MARS_EINVAL
    assert lib.mars_tile_map(ctypes.byref(good()), 16, 16, None, None) == L.MARS_EINVAL
    assert lib.mars_mask_materialize(ctypes.byref(good()), None, None) == L.MARS_EINVAL


def _bwd(desc, gs, ws=FAKE, ws_bytes=1 << 30, lse=FAKE, dout=FAKE, dq=FAKE):
    return L.load().mars_attn_bwd(ctypes.byref(desc), ctypes.byref(gs) if gs is not None else None, FAKE, FAKE,
                                  FAKE, FAKE, lse, dout, dq, FAKE, FAKE, ws, ctypes.c_size_t(ws_bytes), None)


def test_attn_bwd_validation_errors():
    lib = L.load()
    good = lambda: M.attn_desc(2, 14, 2, 64, 10, 20, 4)

    def strides():
        gs = L.AttnBwdStrides()
        d = good()
        gs.do_strides, gs.dq_strides, gs.dk_strides, gs.dv_strides = d.o_strides, d.q_strides, d.k_strides, d.v_strides
        return gs
    n = ctypes.c_size_t()
    assert lib.mars_attn_bwd_workspace_bytes(ctypes.byref(good()), ctypes.byref(n)) == L.MARS_OK
    N, Np = 50, 64                                           # positions padded to a multiple of 32
    r256 = lambda x: (x + 255) // 256 * 256
    # -LSE2, -D, two counters (dV, dK) per (key block, pair, 32-key group); no partials
    # (one chunk per block)
    assert n.value == 2 * r256(2 * 14 * Np * 4) + r256(1 * 4 * 4 * 2 * 4)
    big = ctypes.c_size_t()
    assert lib.mars_attn_bwd_workspace_bytes(ctypes.byref(M.attn_desc(1, 2, 1, 64, 256, 512, 4)), ctypes.byref(big)) == 0
    Nb = 1280                                                # prompt keys walk all 40 tiles: 8 chunks
    assert big.value == (2 * r256(2 * Nb * 4) + r256(10 * 1 * 4 * 2 * 4)
                         + r256(8 * 10 * 1 * 128 * 2 * 64 * 4))
    assert lib.mars_attn_bwd_workspace_bytes(ctypes.byref(good()), None) == L.MARS_EINVAL
    d = good(); d.dtype = L.MARS_DTYPE_FP32
    assert lib.mars_attn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == L.MARS_EUNSUPPORTED
    assert _bwd(d, strides()) == L.MARS_EUNSUPPORTED
    assert _bwd(good(), None) == L.MARS_EINVAL
    assert _bwd(good(), strides(), lse=None) == L.MARS_EINVAL
    assert _bwd(good(), strides(), dout=None) == L.MARS_EINVAL
    assert _bwd(good(), strides(), dq=MISALIGNED) == L.MARS_EINVAL
    gs = strides(); gs.dk_strides[1] = 2 * 64 + 4
    assert _bwd(good(), gs) == L.MARS_EINVAL
    gs = strides(); gs.do_strides[1] = (1 << 25) + 8
    assert _bwd(good(), gs) == L.MARS_EUNSUPPORTED
    d = good(); d.q_strides[1] = (1 << 25) + 8             # the backward copies Q tiles too
    assert _bwd(d, strides()) == L.MARS_EUNSUPPORTED
    d = good(); d.head_dim = 96
    assert _bwd(d, strides()) == L.MARS_EUNSUPPORTED
    assert _bwd(good(), strides(), ws=None) == L.MARS_EWORKSPACE
    assert _bwd(good(), strides(), ws_bytes=n.value - 1 if n.value else 0) == L.MARS_EWORKSPACE
    assert _bwd(good(), strides(), ws=MISALIGNED) == L.MARS_EWORKSPACE
    d = good(); d.batch = 0
    assert L.load().mars_attn_bwd(ctypes.byref(d), ctypes.byref(strides()), None, None, None, None, None, None,
                                  None, None, None, None, ctypes.c_size_t(0), None) == L.MARS_OK


def test_decode_validation_errors():
    lib = L.load()
    good = lambda: M.decode_desc(4, 28, 4, 128, 4, 4096)

    def call(d, ws=FAKE, ws_bytes=1 << 40, ptr=FAKE, lens=FAKE):
        return lib.mars_decode_step(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, lens, ptr, ws, ws_bytes, None)

    d = good(); d.window = 0
    assert call(d) == L.MARS_EINVAL
    d = good(); d.window = 10                              # 7 * 10 rows > 64
    assert call(d) == L.MARS_EUNSUPPORTED
    d = good(); d.head_dim = 80
    assert call(d) == L.MARS_EUNSUPPORTED
    d = good(); d.dtype = L.MARS_DTYPE_FP32
    assert call(d) == L.MARS_EUNSUPPORTED
    assert call(good(), lens=None) == L.MARS_EINVAL
    d = good(); d.kc_strides[2] = 100                      # cache rows lose 16-byte alignment
    assert call(d) == L.MARS_EINVAL
    assert call(good(), ptr=MISALIGNED) == L.MARS_EINVAL
    need = M.mars_decode_workspace_bytes(4, 28, 4, 128, 4, 4096)
    assert need > 0
    assert call(good(), ws=None) == L.MARS_EWORKSPACE
    assert call(good(), ws_bytes=need - 1) == L.MARS_EWORKSPACE
    d = good(); d.cache_capacity = 65535 * 512 + 1        # chunk count beyond the grid's y limit
    assert call(d) == L.MARS_EUNSUPPORTED
    d = good(); d.kc_strides[2] = (1 << 25) + 8           # 32 positions overflow 32-bit offsets
    assert call(d) == L.MARS_EUNSUPPORTED
    d = good(); d.batch = 0
    assert call(d, ptr=None, lens=None, ws=None) == L.MARS_OK


def test_decode_noalloc_validation_errors():
    lib = L.load()
    n = ctypes.c_size_t()
    assert lib.mars_decode_scratch_bytes(None) == L.MARS_EINVAL
    assert lib.mars_decode_scratch_bytes(ctypes.byref(n)) == L.MARS_OK and n.value == 32 << 20

    def call(d, ptr=FAKE, lens=FAKE):
        return lib.mars_decode_step_noalloc(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, lens, ptr, None)

    assert call(M.decode_desc(32, 28, 4, 128, 4, 16384)) == L.MARS_EWORKSPACE     # partials beyond the array
    assert M.mars_decode_workspace_bytes(32, 28, 4, 128, 4, 4096) <= n.value     # the 7B decode workload fits
    assert call(M.decode_desc(32, 28, 4, 128, 4, 4096), lens=None) == L.MARS_EINVAL
    assert call(M.decode_desc(32, 28, 4, 128, 4, 4096), ptr=MISALIGNED) == L.MARS_EINVAL
    d = M.decode_desc(32, 28, 4, 96, 4, 4096)
    assert call(d) == L.MARS_EUNSUPPORTED
    d = M.decode_desc(32, 28, 4, 128, 4, 4096); d.batch = 0
    assert call(d, ptr=None, lens=None) == L.MARS_OK


def test_accept_validation_errors():
    lib = L.load()
    good = lambda: M.accept_desc(32, 4, 152064, 0.95)

    def call(d, ws=FAKE, ws_bytes=1 << 40, ptr=FAKE):
        return lib.mars_accept(ctypes.byref(d), ptr, ptr, ptr, ptr, ws, ws_bytes, None)

    for field, val, code in [("tau", 0.0, L.MARS_EINVAL), ("tau", -0.5, L.MARS_EINVAL),
                             ("tau", float("inf"), L.MARS_EINVAL), ("tau", 1.0000002, L.MARS_EINVAL),
                             ("tau", 2.0, L.MARS_EINVAL), ("tau", float("nan"), L.MARS_EINVAL),
                             ("min_accept", 2, L.MARS_EINVAL),
                             ("window", 65, L.MARS_EUNSUPPORTED), ("window", 0, L.MARS_EINVAL),
                             ("vocab", 0, L.MARS_EINVAL),
                             ("dtype", L.MARS_DTYPE_FP32, L.MARS_EUNSUPPORTED)]:
        d = good()
        setattr(d, field, val)
        assert call(d) == code, field
    d = good(); d.tau = 1.0                               # tau = 1 (exact AR) is inside the range
    n = ctypes.c_size_t()
    assert lib.mars_accept_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == L.MARS_OK
    d = good(); d.row_stride = 152063                     # rows lose 16-byte alignment
    assert call(d) == L.MARS_EINVAL
    assert call(good(), ptr=MISALIGNED) == L.MARS_EINVAL
    assert call(good(), ptr=None) == L.MARS_EINVAL
    need = M.mars_accept_workspace_bytes(32, 4, 152064)
    assert call(good(), ws_bytes=need - 1) == L.MARS_EWORKSPACE
    assert call(good(), ws=FAKE + 8) == L.MARS_EWORKSPACE
    d = good(); d.batch = 0
    assert call(d, ptr=None, ws=None) == L.MARS_OK


def test_accept_margin_validation_errors():
    lib = L.load()
    good = lambda: M.accept_desc(32, 4, 152064, 0.3)

    def call(d, ws=FAKE, ws_bytes=1 << 40, ptr=FAKE, pmax=FAKE, margin=FAKE):
        return lib.mars_accept_margin(ctypes.byref(d), ptr, ptr, pmax, margin, ptr, ws, ws_bytes, None)

    for field, val, code in [("tau", 0.0, L.MARS_EINVAL), ("tau", 1.5, L.MARS_EINVAL), ("min_accept", 2, L.MARS_EINVAL),
                             ("window", 65, L.MARS_EUNSUPPORTED), ("dtype", L.MARS_DTYPE_FP32, L.MARS_EUNSUPPORTED)]:
        d = good()
        setattr(d, field, val)
        assert call(d) == code, field
    assert call(good(), margin=None) == L.MARS_EINVAL          # margin output is required
    assert call(good(), margin=FAKE + 2) == L.MARS_EINVAL
    assert call(good(), pmax=FAKE + 2) == L.MARS_EINVAL
    assert call(good(), ptr=None) == L.MARS_EINVAL
    need = M.mars_accept_workspace_bytes(32, 4, 152064)
    assert call(good(), ws_bytes=need - 1) == L.MARS_EWORKSPACE
    d = good(); d.batch = 0
    assert call(d, ptr=None, ws=None, pmax=None, margin=None) == L.MARS_OK


def test_kv_commit_validation_errors():
    lib = L.load()
    good = lambda: M.decode_desc(4, 28, 4, 128, 4, 4096)

    def call(d, ptr=FAKE, valid=None, overflow=None, policy=0):
        return lib.mars_kv_commit(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, ptr, valid, overflow, policy, None)

    assert call(good(), policy=2) == L.MARS_EINVAL
    assert call(good(), policy=-1) == L.MARS_EINVAL
    assert call(good(), ptr=None) == L.MARS_EINVAL
    assert call(good(), ptr=MISALIGNED) == L.MARS_EINVAL
    assert call(good(), valid=FAKE + 4) == L.MARS_EINVAL          # uint64 alignment
    assert call(good(), overflow=FAKE + 2) == L.MARS_EINVAL
    d = good(); d.head_dim = 96
    assert call(d) == L.MARS_EUNSUPPORTED
    d = good(); d.kc_strides[2] = 100                              # cache rows lose 16-byte alignment
    assert call(d) == L.MARS_EINVAL
    d = good(); d.batch = 0
    assert call(d, ptr=None) == L.MARS_OK


def test_shifted_ce_validation_errors():
    lib = L.load()
    good = lambda: M.ce_desc(8, 256, 512, 4, 151936)

    def call(d, ptr=FAKE, lm=FAKE, la=FAKE, dl=None, ws=FAKE, ws_bytes=1 << 40):
        return lib.mars_shifted_ce(ctypes.byref(d), ptr, ptr, lm, la, dl, ws, ws_bytes, None)

    for field, val, code in [("vocab", 151937, L.MARS_EUNSUPPORTED), ("vocab", 0, L.MARS_EINVAL),
                             ("block", 0, L.MARS_EINVAL), ("resp_len", -1, L.MARS_EINVAL),
                             ("batch", 70000, L.MARS_EUNSUPPORTED), ("dtype", L.MARS_DTYPE_FP32, L.MARS_EUNSUPPORTED)]:
        d = good()
        setattr(d, field, val)
        assert call(d) == code, field
    assert call(good(), lm=None) == L.MARS_EINVAL
    assert call(good(), ptr=None) == L.MARS_EINVAL
    assert call(good(), ptr=MISALIGNED) == L.MARS_EINVAL
    assert call(good(), dl=MISALIGNED) == L.MARS_EINVAL
    assert call(good(), la=FAKE + 2) == L.MARS_EINVAL
    d = good(); d.logits_strides[1] = 151937                       # rows lose 16-byte alignment
    assert call(d) == L.MARS_EINVAL
    d = good(); d.dlogits_strides[0] = -8
    assert call(d, dl=FAKE) == L.MARS_EINVAL
    n = ctypes.c_size_t()
    assert lib.mars_shifted_ce_workspace_bytes(ctypes.byref(good()), ctypes.byref(n)) == L.MARS_OK
    assert n.value == 8 * (256 + 2 * 512) * 4
    assert call(good(), ws_bytes=n.value - 1) == L.MARS_EWORKSPACE
    assert call(good(), ws=None) == L.MARS_EWORKSPACE
    d = good(); d.batch = 0
    assert call(d, ptr=None, lm=None, la=None, ws=None) == L.MARS_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.load()
