"""Pins for the H3 geometry and block map oracles ([VSA] _get_h3_tile_metadata,
_build_h3_block_map): a geometry derived by hand from the page's rules, the
reduction to the plain video geometry and top-k map without a prefix,
permutation and round-trip properties, and a hand-scored map."""

import numpy as np

import oracle


def test_hand_derived_geometry():
    # prefix segments of 70 and 5 rows, then a (2, 5, 4) video in (4, 4, 4) boxes:
    # 70 = 64 + 6 and 5 give prefix chunks [64, 6, 5] (each segment cut on its
    # own); the video has one box along t (2 frames), two along h (4 + 1 rows)
    # and one along w (4): sizes 2*4*4 = 32 and 2*1*4 = 8
    part, sizes, non_pad, untile, n_pre, n_vid = oracle.h3_tile_metadata((70, 5), (2, 5, 4))
    assert sizes.tolist() == [64, 6, 5, 32, 8] and (n_pre, n_vid) == (3, 2)
    # padded rows: tile c starts at 64c
    assert non_pad.tolist() == (list(range(0, 64)) + list(range(64, 70)) + list(range(128, 133))
                                + list(range(192, 224)) + list(range(256, 264)))
    # prefix rows keep their order; video token (t, h, w) is 75 + 20t + 4h + w
    assert part[:75].tolist() == list(range(75))
    box0 = [75 + 20 * t + 4 * h + w for t in range(2) for h in range(4) for w in range(4)]
    box1 = [75 + 20 * t + 16 + w for t in range(2) for w in range(4)]
    assert part[75:].tolist() == box0 + box1
    # untile: raster row n sits at padded row untile[n]
    assert untile[74] == 132 and untile[75] == 192 and untile[75 + 16] == 256 and untile[75 + 20] == 208


def test_no_prefix_is_the_plain_video_geometry():
    for shape in [(5, 7, 9), (16, 32, 32), (1, 1, 3)]:
        a = oracle.h3_tile_metadata((), shape)
        b = oracle.tile_metadata(shape, (4, 4, 4), 64)
        for x, y in zip(a[:4], b):
            assert np.array_equal(x, y)
        assert a[4] == 0 and a[5] == b[1].size


def test_empty_segments_add_no_tile():
    a = oracle.h3_tile_metadata((0, 70, 0), (3, 4, 4))
    b = oracle.h3_tile_metadata((70,), (3, 4, 4))
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x), np.asarray(y))


def test_permutation_and_round_trip():
    segs, shape = (130, 64, 1), (5, 9, 7)
    part, sizes, non_pad, untile, n_pre, n_vid = oracle.h3_tile_metadata(segs, shape)
    total = sum(segs) + int(np.prod(shape))
    assert np.array_equal(np.sort(part), np.arange(total))
    assert sizes.sum() == total and n_pre == 3 + 1 + 1 and sizes[:n_pre].tolist() == [64, 64, 2, 64, 1]
    x = np.random.default_rng(5).standard_normal((2, total, 3))
    t = oracle.h3_to_tile_order(x, segs, shape)
    assert t.shape == (2, sizes.size * 64, 3)
    assert np.array_equal(oracle.h3_from_tile_order(t, segs, shape), x)
    pad = np.ones(sizes.size * 64, dtype=bool)
    pad[non_pad] = False
    assert np.all(t[:, pad] == 0.0)


def test_block_map_without_prefix_is_topk():
    s = np.random.default_rng(6).standard_normal((1, 2, 9, 9))
    for k in (1, 4, 9, 12):
        assert np.array_equal(oracle.h3_block_map(s, 0, 9, k), oracle.topk_block_map(s, k))


def test_block_map_hand_scored():
    # 2 prefix tiles, 4 video tiles, top-2 among the video columns
    s = np.zeros((1, 1, 6, 6))
    s[0, 0, 4] = [9, 8, 1, 5, 5, 3]   # a video query tile: video scores 1, 5, 5, 3
    s[0, 0, 5] = [0, 0, 7, 2, 7, 7]   # ties at 7: the two lowest video indices win
    m = oracle.h3_block_map(s, 2, 4, 2)[0, 0].astype(int)
    assert m[0].tolist() == [1] * 6 and m[1].tolist() == [1] * 6   # prefix query tiles: dense
    assert m[4].tolist() == [1, 1, 0, 1, 1, 0]
    assert m[5].tolist() == [1, 1, 1, 0, 1, 0]
    assert np.all(m[2:, :2] == 1)                                  # prefix keys: always kept
    assert np.all(m[2:, 2:].sum(1) == 2)
    assert np.all(oracle.h3_block_map(s, 2, 4, 4))                 # k covers every video tile
