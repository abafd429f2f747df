"""Integer statement of the video tile geometry (vLLM-Omni fastvideo_vsa.py
page: _get_tile_partition_indices, _construct_variable_block_sizes,
_get_non_pad_index, _get_tile_metadata and _get_h3_tile_metadata).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition, as the page describes the layout. A latent video of raster shape
(T, H, W) is cut into boxes of (tt, th, tw) tokens. Boxes are numbered with the
t-box index slowest, then h, then w; a box at the far end of an axis is
clipped to the tokens left there, so its token count is the product of its
clipped extents. Inside a box the tokens keep raster order. In the padded
tile-order layout box c owns rows [c*block, (c+1)*block), its tokens first and
zero padding after them.

So each raster token (t, h, w) maps directly to a box and a row:
    box = (t // tt) * nH * nW + (h // th) * nW + (w // tw)
    row = (t % tt) * eh * ew + (h % th) * ew + (w % tw)
where (nH, nW) count the boxes along h and w and (eh, ew) are the clipped
h and w extents of that token's box. Everything else is derived from this
map: "untile" (padded row of each raster token) is box*block + row, the
tile-order token list ("partition") is its inverse, the real padded rows
("non_pad") are its image in increasing order.

The H3 layout puts prefix segments (text, reference frames) ahead of the
video: segment s is cut into consecutive chunks of block rows, its last chunk
holding the remainder, and each chunk is one tile, numbered after the chunks
of the segments before it; the video's boxes follow.

Pinned: hand-computed geometries (tests/golden/tile_geometry_3x2x5_t2x2x3.txt,
and the H3 case in the tests), permutation and round-trip properties.
"""

from __future__ import annotations

import math

import numpy as np


def _video_map(shape, tile, block: int):
    """(box, row) of every raster token (flattened raster order) and the token
    count of every box, straight from the definition."""
    t_len, h_len, w_len = (int(x) for x in shape)
    tt, th, tw = (int(x) for x in tile)
    n_t, n_h, n_w = math.ceil(t_len / tt), math.ceil(h_len / th), math.ceil(w_len / tw)
    t, h, w = np.meshgrid(np.arange(t_len), np.arange(h_len), np.arange(w_len), indexing="ij")
    t, h, w = t.reshape(-1), h.reshape(-1), w.reshape(-1)

    def extent(idx, step, length):
        # clipped extent along one axis of the box that holds index idx
        start = (idx // step) * step
        return np.minimum(start + step, length) - start

    box = (t // tt) * n_h * n_w + (h // th) * n_w + (w // tw)
    eh, ew = extent(h, th, h_len), extent(w, tw, w_len)
    row = (t % tt) * eh * ew + (h % th) * ew + (w % tw)
    bt, bh, bw = np.meshgrid(np.arange(n_t), np.arange(n_h), np.arange(n_w), indexing="ij")
    sizes = ((np.minimum((bt + 1) * tt, t_len) - bt * tt) * (np.minimum((bh + 1) * th, h_len) - bh * th)
             * (np.minimum((bw + 1) * tw, w_len) - bw * tw)).reshape(-1)
    return box.astype(np.int64), row.astype(np.int64), sizes.astype(np.int32)


def _layout(box, row, sizes, block: int):
    """(partition, sizes, non_pad, untile) from each token's (box, row)."""
    if sizes.size and (sizes.max() > block or sizes.min() < 0):
        raise ValueError("tile sizes must lie in [0, block]")
    untile = box * block + row  # padded row of raster token n
    order = np.argsort(untile, kind="stable")  # tile order: increasing padded row
    return order.astype(np.int64), sizes, untile[order], untile


def tile_partition_indices(shape, tile) -> np.ndarray:
    """Raster token index of each position in tile order, int64 [T*H*W]."""
    box, row, _ = _video_map(shape, tile, 64)
    return np.lexsort((row, box)).astype(np.int64)  # by box, then row within the box


def variable_block_sizes(shape, tile) -> np.ndarray:
    """Real token count of every box, int32 [n_tiles]."""
    return _video_map(shape, tile, 64)[2]


def non_pad_index(sizes, block: int = 64) -> np.ndarray:
    """Padded-layout row of every real token in tile order: tile c, row
    r < sizes[c] -> c*block + r."""
    sizes = np.asarray(sizes, dtype=np.int64)
    if np.any(sizes > block) or np.any(sizes < 0):
        raise ValueError("tile sizes must lie in [0, block]")
    box = np.repeat(np.arange(sizes.size, dtype=np.int64), sizes)
    start = np.concatenate([[0], np.cumsum(sizes)[:-1]]) if sizes.size else np.zeros(0, dtype=np.int64)
    row = np.arange(int(sizes.sum()), dtype=np.int64) - np.repeat(start, sizes)
    return box * block + row


def tile_metadata(shape, tile, block: int = 64):
    """(partition, sizes, non_pad, untile) for one raster shape and box shape."""
    if math.prod(tile) > block:
        raise ValueError("a box must fit in one block")
    box, row, sizes = _video_map(shape, tile, block)
    return _layout(box, row, sizes, block)


def to_tile_order(x, shape, tile, block: int = 64) -> np.ndarray:
    """Raster [B, N, H, D] -> padded tile order [B, n_tiles*block, H, D] (pad rows 0)."""
    xf = np.asarray(x)
    _, sizes, _, untile = tile_metadata(shape, tile, block)
    out = np.zeros((xf.shape[0], sizes.size * block) + xf.shape[2:], dtype=xf.dtype)
    out[:, untile] = xf
    return out


def from_tile_order(y, shape, tile, block: int = 64) -> np.ndarray:
    """Padded tile order [B, n_tiles*block, ...] -> raster [B, N, ...]."""
    untile = tile_metadata(shape, tile, block)[3]
    return np.asarray(y)[:, untile]


def h3_tile_metadata(prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64):
    """H3 layout: (partition, sizes, non_pad, untile, n_prefix_tiles,
    n_video_tiles) for prefix segments ahead of a video (see the module
    docstring). Raster order is the prefix rows, segment after segment, then
    the video in (t, h, w) raster order.

    Pinned: a hand-computed geometry, no prefix = tile_metadata, permutation and
    round trip.
    """
    segs = [int(s) for s in prefix_segments]
    if any(s < 0 for s in segs):
        raise ValueError("prefix segments must be >= 0")
    boxes, rows, prefix_sizes = [], [], []
    for seg in segs:
        offset = np.arange(seg, dtype=np.int64)
        boxes.append(len(prefix_sizes) + offset // block)  # this segment's chunks follow the earlier ones
        rows.append(offset % block)
        prefix_sizes += [min(block, seg - c * block) for c in range(math.ceil(seg / block))]
    n_pre = len(prefix_sizes)
    vbox, vrow, vsizes = _video_map(video_shape, tile, block)
    box = np.concatenate(boxes + [vbox + n_pre]) if boxes else vbox
    row = np.concatenate(rows + [vrow]) if rows else vrow
    sizes = np.concatenate([np.asarray(prefix_sizes, dtype=np.int32), vsizes])
    partition, sizes, non_pad, untile = _layout(box, row, sizes, block)
    return partition, sizes, non_pad, untile, n_pre, int(vsizes.size)


def h3_to_tile_order(x, prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64) -> np.ndarray:
    """Raster [B, prefix + T*H*W, ...] -> padded H3 tile order (pad rows 0)."""
    xf = np.asarray(x)
    _, sizes, _, untile, _, _ = h3_tile_metadata(prefix_segments, video_shape, tile, block)
    out = np.zeros((xf.shape[0], sizes.size * block) + xf.shape[2:], dtype=xf.dtype)
    out[:, untile] = xf
    return out


def h3_from_tile_order(y, prefix_segments, video_shape, tile=(4, 4, 4), block: int = 64) -> np.ndarray:
    """Padded H3 tile order -> raster [B, prefix + T*H*W, ...]."""
    untile = h3_tile_metadata(prefix_segments, video_shape, tile, block)[3]
    return np.asarray(y)[:, untile]
