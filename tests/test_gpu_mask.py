"""GPU: the device visibility predicate and tile map equal the oracle bit for bit."""
import numpy as np
import pytest

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

SHAPES = [(0, 8, 4), (16, 64, 4), (256, 512, 4), (3, 37, 8), (10, 5, 16), (0, 1, 1), (5, 0, 3), (7, 33, 1),
          (512, 1536, 8)]


@pytest.mark.parametrize("P,L,B", SHAPES)
def test_mask_bit_exact(P, L, B):
    m = M.mars_mask_materialize(P, L, B, dev()).cpu().numpy()
    ref = O.mask_rules(P, L, B).astype(np.uint8)
    assert np.array_equal(m, ref)


def test_fig2_mask():
    m = M.mars_mask_materialize(0, 8, 4, dev()).cpu().numpy()
    assert int(m.sum()) == 72 and np.array_equal(m, O.mask_rules_scalar(0, 8, 4))


@pytest.mark.parametrize("P,L,B,bm,bn", [
    (16, 64, 4, 128, 128), (256, 512, 4, 128, 128), (512, 1536, 8, 128, 128), (3, 37, 8, 16, 8),
    (256, 512, 4, 64, 32), (10, 5, 16, 7, 5), (1024, 7168, 32, 128, 128)])
def test_tile_map_bit_exact(P, L, B, bm, bn):
    tm = M.mars_tile_map(P, L, B, bm, bn, dev()).cpu().numpy()
    ref = O.tile_map_rules(P, L, B, bm, bn)
    assert np.array_equal(tm, ref)
