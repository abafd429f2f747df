"""fp64/int statement of the video tile geometry ([VSA] page).

TEST INFRASTRUCTURE ONLY (see the package docstring).

A latent video of raster shape (T, H, W) is cut into boxes of (tt, th, tw)
tokens. Boxes are enumerated with the t-box index slowest, then h, then w; the
tokens of one box are listed in raster order; boxes at the far edge of an axis
are clipped to what is left ([VSA] _get_tile_partition_indices). A box's token
count is the product of its clipped extents ([VSA] _construct_variable_block_sizes).
In the padded tile-order layout each box owns ``block`` rows, the first
``size`` of them real ([VSA] _get_non_pad_index), and the inverse ("untile")
gather is ``non_pad[argsort(partition)]`` ([VSA] _get_tile_metadata).

Pinned: hand-computed small geometries, permutation and round-trip properties.
"""

from __future__ import annotations

import math

import numpy as np


def _boxes(shape, tile):
    """Yield the clipped (start, stop) ranges of each box in enumeration order."""
    nt = [math.ceil(s / t) for s, t in zip(shape, tile)]
    for bt in range(nt[0]):
        for bh in range(nt[1]):
            for bw in range(nt[2]):
                yield tuple(
                    (i * t, min((i + 1) * t, s)) for i, t, s in zip((bt, bh, bw), tile, shape)
                )


def tile_partition_indices(shape, tile) -> np.ndarray:
    """Raster token index of each position in tile order, int64 [T*H*W]."""
    t_len, h_len, w_len = shape
    raster = np.arange(t_len * h_len * w_len, dtype=np.int64).reshape(t_len, h_len, w_len)
    parts = [np.zeros(0, dtype=np.int64)]  # an empty video has no box
    for (t0, t1), (h0, h1), (w0, w1) in _boxes(shape, tile):
        parts.append(raster[t0:t1, h0:h1, w0:w1].reshape(-1))
    return np.concatenate(parts)


def variable_block_sizes(shape, tile) -> np.ndarray:
    """Real token count of every box, int32 [n_tiles]."""
    return np.asarray(
        [(t1 - t0) * (h1 - h0) * (w1 - w0) for (t0, t1), (h0, h1), (w0, w1) in _boxes(shape, tile)],
        dtype=np.int32,
    )


def non_pad_index(sizes, block: int = 64) -> np.ndarray:
    """Padded-layout row of every real token: tile c, row r < sizes[c] -> c*block + r."""
    sizes = np.asarray(sizes, dtype=np.int64)
    if np.any(sizes > block) or np.any(sizes < 0):
        raise ValueError("tile sizes must lie in [0, block]")
    return np.concatenate([np.zeros(0, dtype=np.int64)]
                          + [c * block + np.arange(s) for c, s in enumerate(sizes)]).astype(np.int64)


def untile_index(partition, non_pad) -> np.ndarray:
    """Padded-layout row that holds raster token n: non_pad[argsort(partition)]."""
    return np.asarray(non_pad)[np.argsort(np.asarray(partition), kind="stable")]


def tile_metadata(shape, tile, block: int = 64):
    """(partition, sizes, non_pad, untile) for one raster shape and box shape."""
    if math.prod(tile) > block:
        raise ValueError("a box must fit in one block")
    partition = tile_partition_indices(shape, tile)
    sizes = variable_block_sizes(shape, tile)
    non_pad = non_pad_index(sizes, block)
    return partition, sizes, non_pad, untile_index(partition, non_pad)


def to_tile_order(x, shape, tile, block: int = 64) -> np.ndarray:
    """Raster [B, N, H, D] -> padded tile order [B, n_tiles*block, H, D] (pad rows 0)."""
    xf = np.asarray(x)
    partition, sizes, non_pad, _ = tile_metadata(shape, tile, block)
    out = np.zeros((xf.shape[0], sizes.size * block) + xf.shape[2:], dtype=xf.dtype)
    out[:, non_pad] = xf[:, partition]
    return out


def from_tile_order(y, shape, tile, block: int = 64) -> np.ndarray:
    """Padded tile order [B, n_tiles*block, ...] -> raster [B, N, ...]."""
    _, _, _, untile = tile_metadata(shape, tile, block)
    return np.asarray(y)[:, untile]


def h3_tile_metadata(prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64):
    """[VSA] _get_h3_tile_metadata: the prefix rows (the segments before the
    target video, e.g. text and reference frames) come first, in their own
    order, each segment cut into chunks of ``block`` rows with its remainder as
    a last, partial chunk; the target video's boxes follow, with their raster
    token indices shifted past the prefix.

    Returns (partition, sizes, non_pad, untile, n_prefix_tiles, n_video_tiles).

    Pinned: a hand-computed geometry, no prefix = tile_metadata, permutation and
    round trip.
    """
    prefix_len = int(sum(int(s) for s in prefix_segments))
    prefix_sizes = []
    for seg in prefix_segments:
        full, rem = divmod(int(seg), block)
        prefix_sizes += [block] * full + ([rem] if rem else [])
    video_part = tile_partition_indices(video_shape, tile) + prefix_len
    video_sizes = variable_block_sizes(video_shape, tile)
    partition = np.concatenate([np.arange(prefix_len, dtype=np.int64), video_part])
    sizes = np.concatenate([np.asarray(prefix_sizes, dtype=np.int32), video_sizes])
    non_pad = non_pad_index(sizes, block)
    return partition, sizes, non_pad, untile_index(partition, non_pad), len(prefix_sizes), int(video_sizes.size)


def h3_to_tile_order(x, prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64) -> np.ndarray:
    """Raster [B, prefix + T*H*W, ...] -> padded H3 tile order (pad rows 0)."""
    xf = np.asarray(x)
    partition, sizes, non_pad, _, _, _ = h3_tile_metadata(prefix_segments, video_shape, tile, block)
    out = np.zeros((xf.shape[0], sizes.size * block) + xf.shape[2:], dtype=xf.dtype)
    out[:, non_pad] = xf[:, partition]
    return out


def h3_from_tile_order(y, prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64) -> np.ndarray:
    """Padded H3 tile order -> raster [B, prefix + T*H*W, ...]."""
    untile = h3_tile_metadata(prefix_segments, video_shape, tile, block)[3]
    return np.asarray(y)[:, untile]
