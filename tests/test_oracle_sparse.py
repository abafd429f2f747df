"""Pins for the tile geometry, block-map builder and block-sparse oracle."""

import os

import numpy as np
import pytest
import torch

import oracle
from workloads import video_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(777)


# --------------------------------------------------------------------------
# tile geometry
# --------------------------------------------------------------------------

def test_geometry_hand_example():
    with open(os.path.join(GOLDEN, "tile_geometry_3x2x5_t2x2x3.txt")) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    part = np.array(lines[0].split(), dtype=np.int64)
    sizes = np.array(lines[1].split(), dtype=np.int64)
    assert np.array_equal(oracle.tile_partition_indices((3, 2, 5), (2, 2, 3)), part)
    assert np.array_equal(oracle.variable_block_sizes((3, 2, 5), (2, 2, 3)), sizes)


@pytest.mark.parametrize("shape,tile", [((16, 32, 32), (4, 4, 4)), ((5, 7, 9), (4, 4, 4)), ((3, 2, 5), (2, 2, 3)),
                                        ((1, 1, 1), (4, 4, 4)), ((8, 8, 8), (4, 4, 4))])
def test_geometry_properties(shape, tile):
    part, sizes, non_pad, untile = oracle.tile_metadata(shape, tile, 64)
    n = int(np.prod(shape))
    assert np.array_equal(np.sort(part), np.arange(n))  # a permutation
    assert sizes.sum() == n and np.all(sizes >= 1) and np.all(sizes <= 64)
    assert non_pad.size == n and np.all(np.diff(non_pad) > 0)
    # each box's tokens fill its first sizes[c] rows, padding after them
    assert np.array_equal(non_pad, oracle.non_pad_index(sizes, 64))
    assert np.array_equal(np.sort(untile), non_pad)
    x = RNG.standard_normal((2, n, 3, 4))
    xt = oracle.to_tile_order(x, shape, tile)
    assert xt.shape == (2, sizes.size * 64, 3, 4)
    assert np.array_equal(oracle.from_tile_order(xt, shape, tile), x)
    pad = np.ones(xt.shape[1], dtype=bool)
    pad[non_pad] = False
    assert np.all(xt[:, pad] == 0)


def test_config5_geometry_is_256_full_tiles():
    _, sizes, _, _ = oracle.tile_metadata((16, 32, 32), (4, 4, 4), 64)
    assert sizes.size == 256 and np.all(sizes == 64)


# --------------------------------------------------------------------------
# block map builder
# --------------------------------------------------------------------------

def test_pool_hand_example():
    x = np.zeros((1, 128, 1, 2))
    x[0, 0:3, 0] = [[1.0, 10.0], [2.0, 20.0], [3.0, 60.0]]  # tile 0, 3 real rows
    x[0, 64:128, 0] = 5.0  # tile 1, full
    pooled = oracle.pool_tiles(x, [3, 64])
    assert np.allclose(pooled[0, 0, 0], [2.0, 30.0]) and np.allclose(pooled[0, 0, 1], [5.0, 5.0])
    # a zero-size tile divides by max(size, 1)
    assert np.all(oracle.pool_tiles(np.zeros((1, 64, 1, 2)), [0]) == 0.0)


def test_pooled_scores_hand_example():
    qp = np.array([[[[1.0, 2.0], [0.0, 1.0]]]])
    kp = np.array([[[[3.0, 1.0], [-1.0, 4.0]]]])
    s = oracle.pooled_scores(qp, kp, 0.5)
    assert np.allclose(s[0, 0], 0.5 * np.array([[5.0, 7.0], [1.0, 4.0]]))


def test_topk_map_properties():
    scores = RNG.standard_normal((2, 3, 20, 20))
    m = oracle.topk_block_map(scores, 6)
    assert np.all(m.sum(-1) == 6)
    kept_min = np.where(m, scores, np.inf).min(-1)
    dropped_max = np.where(~m, scores, -np.inf).max(-1)
    assert np.all(kept_min > dropped_max)
    assert np.all(oracle.topk_block_map(scores, 20)) and np.all(oracle.topk_block_map(scores, 99))


def test_topk_tie_break_lower_index():
    scores = np.array([[[[1.0, 3.0, 3.0, 3.0, 0.0]]]])
    m = oracle.topk_block_map(scores, 2)
    assert m[0, 0, 0].tolist() == [False, True, True, False, False]


def test_map_to_index_round_trip():
    m = RNG.random((2, 3, 17, 17)) < 0.3
    idx, num = oracle.map_to_index(m)
    for b in range(2):
        for h in range(3):
            for a in range(17):
                cols = np.nonzero(m[b, h, a])[0]
                assert num[b, h, a] == cols.size
                assert np.array_equal(idx[b, h, a, :cols.size], cols)
                assert np.all(idx[b, h, a, cols.size:] == -1)


# --------------------------------------------------------------------------
# block-sparse attention
# --------------------------------------------------------------------------

def _tiled_case(shape=(3, 5, 6), tile=(2, 2, 3), heads=2, hkv=2, d=8, seed=31):
    n = int(np.prod(shape))
    q = RNG.standard_normal((1, n, heads, d))
    k = RNG.standard_normal((1, n, hkv, d))
    v = RNG.standard_normal((1, n, hkv, d))
    part, sizes, non_pad, untile = oracle.tile_metadata(shape, tile, 64)
    to = lambda x: oracle.to_tile_order(x, shape, tile)  # noqa: E731
    return q, k, v, to(q), to(k), to(v), sizes, part, untile


def test_full_map_equals_dense():
    bsz, nt, h, d = 2, 3, 2, 16
    q = RNG.standard_normal((bsz, nt * 64, h, d))
    k = RNG.standard_normal((bsz, nt * 64, h, d))
    v = RNG.standard_normal((bsz, nt * 64, h, d))
    full = np.ones((bsz, h, nt, nt), dtype=bool)
    o, l_ = oracle.block_sparse_attention(q, k, v, full, [64] * nt, 0.25)
    od, ld = oracle.dense_attention(q, k, v, 0.25, False)
    assert np.allclose(o, od, atol=1e-13) and np.allclose(l_, ld, atol=1e-13)


def test_token_mask_equivalence_with_partial_tiles_and_gqa():
    q, k, v, qt, kt, vt, sizes, part, untile = _tiled_case(heads=4, hkv=2)
    nt = sizes.size
    bmap = RNG.random((1, 4, nt, nt)) < 0.5
    bmap[0, 1, 2] = False  # a query tile with no key tile at all
    o, l_ = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, 0.3)
    seq = nt * 64
    tile_of = np.arange(seq) // 64
    valid = (np.arange(seq) % 64) < sizes[tile_of]
    for h in range(4):
        mask = bmap[0, h][tile_of[:, None], tile_of[None, :]] & valid[None, :] & valid[:, None]
        qq = torch.from_numpy(qt[0, :, h])
        kk = torch.from_numpy(kt[0, :, h // 2])
        vv = torch.from_numpy(vt[0, :, h // 2])
        z = 0.3 * qq @ kk.T
        z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
        lse_ref = torch.logsumexp(z, dim=-1).numpy()
        w = torch.softmax(z, dim=-1).nan_to_num(0.0)
        o_ref = (w @ vv).numpy()
        rows = mask.any(axis=1)
        assert np.allclose(o[0, rows, h], o_ref[rows], atol=1e-12)
        assert np.allclose(l_[0, h, rows], lse_ref[rows], atol=1e-12)
        assert np.all(o[0, ~rows, h] == 0) and np.all(np.isneginf(l_[0, h, ~rows]))
    # pad rows: zero output, -inf lse
    assert np.all(o[0, ~valid] == 0) and np.all(np.isneginf(l_[0][:, ~valid]))


def test_raster_attention_equals_untiled_tile_attention():
    shape, tile = (3, 5, 6), (2, 2, 3)
    q, k, v, qt, kt, vt, sizes, part, untile = _tiled_case(shape, tile)
    nt = sizes.size
    bmap = RNG.random((1, 2, nt, nt)) < 0.6
    np.fill_diagonal(bmap[0, 0], True)
    np.fill_diagonal(bmap[0, 1], True)
    o, _ = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, 0.3)
    o_raster = oracle.from_tile_order(o, shape, tile)
    # token-level mask in raster order: tile of raster token n
    tile_of_raster = np.empty(part.size, dtype=np.int64)
    tile_of_raster[part] = np.repeat(np.arange(nt), sizes)
    for h in range(2):
        mask = bmap[0, h][tile_of_raster[:, None], tile_of_raster[None, :]]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, :, h]), torch.from_numpy(k[0, :, h]), torch.from_numpy(v[0, :, h]),
            attn_mask=torch.from_numpy(mask), scale=0.3)
        assert np.allclose(o_raster[0, :, h], ref.numpy(), atol=1e-12)


def test_config5_map_keeps_32_per_row():
    case = video_case((4, 8, 8), num_heads=2, head_dim=16, topk=4, seed=5)
    qt = oracle.to_tile_order(case.q.double().numpy(), case.video_shape, case.tile_shape)
    kt = oracle.to_tile_order(case.k.double().numpy(), case.video_shape, case.tile_shape)
    _, sizes, _, _ = oracle.tile_metadata(case.video_shape, case.tile_shape)
    s = oracle.pooled_scores(oracle.pool_tiles(qt, sizes), oracle.pool_tiles(kt, sizes), case.scale)
    m = oracle.topk_block_map(s, case.topk)
    assert m.shape == (1, 2, 4, 4) and np.all(m)  # topk == n_tiles keeps everything
    m2 = oracle.topk_block_map(s, 2)
    assert np.all(m2.sum(-1) == 2)
