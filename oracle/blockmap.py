"""fp64 statement of the block-map construction ([VSA] page).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[VSA] FastVideoVSAImpl._forward_h3 builds the per-query-tile key-tile map from
tile means: each tile's q and k rows are averaged over its real rows
(_pool_h3_tiles: sum over the tile's rows, pad rows being zero, divided by
max(size, 1)); the pooled scores are scale * q_pool k_pool^T; each query tile
keeps the ``topk`` key tiles of largest score, or every tile when topk reaches
the tile count (_build_h3_block_map). The Blackwell route turns the boolean map
into per-row ascending index lists plus counts (map_to_index).

Readings: the pages use torch.topk, whose tie order is unspecified; here the
lower key-tile index wins a tie. Pooling is done in float64 (the page sums in
float32). No prefix tiles (the H3 prefix-dense rows are a later extension).

Pinned: per-row counts, kept >= dropped scores, full-map case, index round trip,
hand-computed pooled means.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64


def pool_tiles(x_tiled, sizes, block: int = 64) -> np.ndarray:
    """Tile means. x_tiled [B, n_tiles*block, H, D] (pad rows zero) -> [B, H, n_tiles, D]."""
    xf = _f64(x_tiled)
    sizes = np.asarray(sizes, dtype=np.float64)
    bsz, seq, heads, dim = xf.shape
    n_tiles = seq // block
    sums = xf.reshape(bsz, n_tiles, block, heads, dim).sum(axis=2)
    means = sums / np.maximum(sizes, 1.0)[None, :, None, None]
    return means.transpose(0, 2, 1, 3)


def pooled_scores(q_pool, k_pool, scale: float) -> np.ndarray:
    """scale * q_pool k_pool^T -> [B, H, nQ, nK]."""
    return scale * (np.asarray(q_pool) @ np.swapaxes(np.asarray(k_pool), -1, -2))


def topk_block_map(scores, topk: int) -> np.ndarray:
    """Boolean [B, H, nQ, nK] keeping the min(topk, nK) largest scores per row."""
    s = np.asarray(scores)
    n_k = s.shape[-1]
    keep = min(int(topk), n_k)
    if keep == n_k:
        return np.ones(s.shape, dtype=bool)
    order = np.argsort(-s, axis=-1, kind="stable")  # ties: lower index first
    out = np.zeros(s.shape, dtype=bool)
    np.put_along_axis(out, order[..., :keep], True, axis=-1)
    return out


def h3_block_map(scores, n_prefix: int, n_video: int, topk: int) -> np.ndarray:
    """[VSA] _build_h3_block_map: prefix key tiles are kept for every query
    tile and prefix query tiles keep every key tile; a video query tile keeps
    the min(topk, n_video) best-scoring video key tiles (ties: lower index), on
    top of the prefix columns. When that is every video tile the map is all
    ones. scores [B, H, nT, nT] with nT = n_prefix + n_video.

    Pinned: no prefix = topk_block_map, hand example, forced rows and columns.
    """
    s = np.asarray(scores)
    if s.shape[-1] != n_prefix + n_video or s.shape[-2] != n_prefix + n_video:
        raise ValueError("scores must cover the prefix and video tiles")
    keep = min(int(topk), int(n_video))
    if keep == n_video:
        return np.ones(s.shape, dtype=bool)
    out = np.zeros(s.shape, dtype=bool)
    out[..., n_prefix:] = topk_block_map(s[..., n_prefix:], keep)
    out[..., :n_prefix] = True
    out[..., :n_prefix, :] = True
    return out


def map_to_index(block_map):
    """Ascending kept key-tile indices per row, int32 [..., nK] padded with -1,
    and the kept count per row, int32 [...] (any number of leading dims)."""
    m = np.asarray(block_map).astype(bool)
    num = m.sum(axis=-1).astype(np.int32)
    idx = np.full(m.shape, -1, dtype=np.int32)
    # stable sort of "not kept" puts kept columns first, in ascending order
    order = np.argsort(~m, axis=-1, kind="stable").astype(np.int32)
    pos = np.arange(m.shape[-1])
    valid = pos < num[..., None]
    idx[valid] = order[valid]
    return idx, num


def compressed_branch(q_tiled, k_tiled, v_tiled, sizes, scale: float, gate_tiled, out_tiled=None, block: int = 64):
    """[VSA] FastVideoVSAImpl._forward_h3, gate branch: with the tile means of
    q, k and v (pool_tiles) and the pooled scores S = scale * q_pool k_pool^T
    (the same scores the block map is built from), every query tile gets
    c = softmax(S, over all key tiles) @ v_pool; each of its rows then adds
    c * gate to the attention output: out + broadcast_rows(c) * gate, in tile
    order (the page's gate_tiled is zero on padding rows). With grouped heads
    query head h reads kv head h // (H / Hkv).

    q_tiled [B, T*block, H, D]; k/v_tiled [B, T*block, Hkv, D]; gate_tiled like
    q_tiled; out_tiled like q_tiled or None (zeros). Returns (out + c * gate,
    c [B, H, T, D]) in float64.

    Pinned: brute force on tiny inputs, uniform scores give the mean of the
    value means, a zero gate leaves the output, grouped = repeated heads.
    """
    qp = pool_tiles(q_tiled, sizes, block)
    kp = pool_tiles(k_tiled, sizes, block)
    vp = pool_tiles(v_tiled, sizes, block)
    group = qp.shape[1] // kp.shape[1]
    kp = np.repeat(kp, group, axis=1)
    vp = np.repeat(vp, group, axis=1)
    s = pooled_scores(qp, kp, scale)
    w = np.exp(s - s.max(axis=-1, keepdims=True))
    w /= w.sum(axis=-1, keepdims=True)
    comp = w @ vp  # [B, H, T, D]
    rows = np.repeat(comp.transpose(0, 2, 1, 3), block, axis=1)  # [B, T*block, H, D]
    base = np.zeros(rows.shape) if out_tiled is None else _f64(out_tiled)
    return base + rows * _f64(gate_tiled), comp
