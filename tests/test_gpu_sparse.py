"""GPU parity of attn_block_map_to_index (bit-exact) and attn_block_sparse_fwd
against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, dev, guard_intact, guarded_empty, host
from workloads import config5, randn_bf16, randn_bf16_on

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,density", [(48, 256, 0.125), (17, 17, 0.5), (9, 100, 0.0), (9, 130, 1.0),
                                               (3072, 256, 0.125)])
def test_map_to_index_bit_exact(rows, cols, density):
    rng = np.random.default_rng(rows + cols)
    m = rng.random((rows, cols)) < density
    if rows > 2:
        m[1] = False  # an empty row
        m[2] = True   # a full row
    announce("map_to_index", rows, cols, density)
    idx, num = sav.attn_block_map_to_index(dev(m.astype(np.uint8)))
    torch.cuda.synchronize()
    ref_idx, ref_num = oracle.map_to_index(m)
    num = num.cpu().numpy()
    idx = idx.cpu().numpy()
    assert np.array_equal(num, ref_num)
    for r in range(rows):
        assert np.array_equal(idx[r, :num[r]], ref_idx[r, :ref_num[r]])


def _tiled(shape, tile, b, hq, hkv, d, seed):
    n = int(np.prod(shape))
    part, sizes, non_pad, untile = oracle.tile_metadata(shape, tile, 64)
    nt = sizes.size
    raster = [randn_bf16((b, n, h, d), 1000 * seed + j) for j, h in enumerate((hq, hkv, hkv))]
    tiled = []
    for x in raster:
        t = torch.zeros((b, nt * 64) + tuple(x.shape[2:]), dtype=x.dtype)
        t[:, torch.from_numpy(non_pad)] = x[:, torch.from_numpy(part)]
        tiled.append(t)
    return tiled, sizes


def run(qt, kt, vt, bmap, sizes, scale, with_lse=True):
    res = sav.attn_block_sparse_fwd(dev(qt), dev(kt), dev(vt), dev(bmap.astype(np.uint8)),
                                    dev(sizes.astype(np.int32)), scale, return_lse=with_lse)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_partial_tiles_random_map(d, hq, hkv):
    shape, tile = (5, 7, 9), (4, 4, 4)  # 2x2x3 = 12 boxes, clipped edges of 16..64 tokens
    (qt, kt, vt), sizes = _tiled(shape, tile, 2, hq, hkv, d, seed=300 + d)
    nt = sizes.size
    rng = np.random.default_rng(d + hq)
    bmap = rng.random((2, hq, nt, nt)) < 0.4
    bmap[0, 0, 3] = False  # an empty row
    bmap[1, -1, 5] = True  # a full row
    scale = d ** -0.5
    announce("sparse", d, hq, hkv, sizes.tolist())
    out, lse = run(qt, kt, vt, bmap, sizes, scale)
    ref_o, ref_l = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, scale)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


@pytest.mark.parametrize("d", [128, 256])
def test_pipe_beyond_staged_list_capacity(d):
    # the pipelined kernel stages each query tile's kept-tile list in LDS for
    # up to 3072 tiles; a longer tile axis takes the general kernel
    b, nt, h = 1, 3100, 1
    q, k, v = (randn_bf16((b, nt * 64, h, d), 340 + j) for j in range(3))
    rng = np.random.default_rng(34)
    sizes = np.full(nt, 64, dtype=np.int32)
    sizes[rng.choice(nt, 40, replace=False)] = rng.integers(1, 64, 40)
    bmap = np.zeros((b, h, nt, nt), dtype=bool)
    for a in range(nt):
        bmap[0, 0, a, rng.choice(nt, 3, replace=False)] = True
    bmap[0, 0, nt - 1, rng.choice(nt, 200, replace=False)] = True  # one long kept list
    scale = d ** -0.5
    announce("sparse beyond list capacity", nt)
    out, lse = run(q, k, v, bmap, sizes, scale)
    sample = sorted({0, 1, 1500, 3071, 3072, 3073, nt - 2, nt - 1} | set(rng.choice(nt, 8, replace=False).tolist()))
    ref_o, ref_l = oracle.block_sparse_attention(q, k, v, bmap, sizes, scale, q_tiles=sample)
    rows = np.concatenate([np.arange(a * 64, a * 64 + 64) for a in sample])
    assert_close("out", host(out)[:, rows], ref_o[:, rows], OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse)[:, :, rows], ref_l[:, :, rows], LSE_TOL)


@pytest.mark.parametrize("density,d", [(0.45, 128), (0.9, 128), (0.9, 96), (0.45, 192), (0.9, 256)])
def test_pipe_long_kept_lists(density, d):
    """Kept lists longer than 64 tiles (the pipelined kernel reads its list
    through a 64-entry window that moves forward), with partial and empty tiles
    that are dropped from the lists, a row with every tile, one with none and
    one with 65."""
    b, nt, hq, hkv = 1, 150, 4, 2
    q = randn_bf16((b, nt * 64, hq, d), 350)
    k, v = (randn_bf16((b, nt * 64, hkv, d), 351 + j) for j in range(2))
    rng = np.random.default_rng(35 + int(density * 100) + (d - 128))
    sizes = np.full(nt, 64, dtype=np.int32)
    sizes[rng.choice(nt, 30, replace=False)] = rng.integers(0, 64, 30)  # some empty tiles
    bmap = rng.random((b, hq, nt, nt)) < density
    bmap[0, 0, 7] = True
    bmap[0, 1, 8] = False
    bmap[0, 2, 9] = False
    bmap[0, 2, 9, rng.choice(nt, 65, replace=False)] = True
    scale = d ** -0.5
    announce("sparse long kept lists", density, int(bmap.sum(-1).max()))
    out, lse = run(q, k, v, bmap, sizes, scale)
    sample = sorted({0, 7, 8, 9, nt - 1} | set(rng.choice(nt, 12, replace=False).tolist()))
    ref_o, ref_l = oracle.block_sparse_attention(q, k, v, bmap, sizes, scale, q_tiles=sample)
    rows = np.concatenate([np.arange(a * 64, a * 64 + 64) for a in sample])
    assert_close("out", host(out)[:, rows], ref_o[:, rows], OUT_TOL, bf16_output=True, few_keys=True)
    fin = np.isfinite(ref_l[:, :, rows])
    assert np.array_equal(fin, np.isfinite(host(lse)[:, :, rows]))
    assert_close("lse", host(lse)[:, :, rows][fin], ref_l[:, :, rows][fin], LSE_TOL)


@pytest.mark.parametrize("d", [128, 96, 256])
def test_full_map_matches_dense_oracle_and_is_deterministic(d):
    b, nt, h = 1, 5, 3
    q, k, v = (randn_bf16((b, nt * 64, h, d), 320 + j) for j in range(3))
    bmap = np.ones((b, h, nt, nt), dtype=bool)
    sizes = np.full(nt, 64, dtype=np.int32)
    announce("sparse full map")
    out, lse = run(q, k, v, bmap, sizes, d ** -0.5)
    out2, _ = run(q, k, v, bmap, sizes, d ** -0.5)
    ref_o, ref_l = oracle.dense_attention(q, k, v, d ** -0.5, False)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_item_order_longest_first_is_a_permutation():
    # The pipelined kernel runs the query tiles of each XCD chunk (8 equal
    # chunks of the (batch, head, tile) items) longest first. The order it
    # leaves in the workspace (after the index lists and their lengths) must
    # be a permutation of each chunk, non-increasing in the 16 count classes
    # and in item order within a class; the result must not depend on it.
    b, nt, h, d = 1, 40, 3, 128
    q, k, v = (randn_bf16((b, nt * 64, h, d), 350 + j) for j in range(3))
    rng = np.random.default_rng(35)
    bmap = rng.random((b, h, nt, nt)) < 0.1
    bmap[0, :, :4] = True      # dense rows at the start of every head
    bmap[0, 1, 20:23] = True   # and in the middle of one
    bmap[0, 2, 30] = False     # an empty row
    sizes = np.full(nt, 64, dtype=np.int32)
    ws = torch.empty(sav.attn_block_sparse_workspace_size(b, h, nt), dtype=torch.uint8, device="cuda")
    announce("sparse item order")
    out, lse = sav.attn_block_sparse_fwd(dev(q), dev(k), dev(v), dev(bmap.astype(np.uint8)), dev(sizes), d ** -0.5,
                                         return_lse=True, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.block_sparse_attention(q, k, v, bmap, sizes, d ** -0.5)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)
    rows = b * h * nt
    words = ws.view(torch.int32).cpu().numpy()
    counts = bmap.reshape(rows, nt).sum(1)
    assert np.array_equal(words[rows * nt:rows * nt + rows], counts)
    order = words[rows * nt + rows:rows * nt + 2 * rows]
    per = (rows + 7) // 8
    for x in range(8):
        lo, hi = x * per, min((x + 1) * per, rows)
        chunk = order[lo:hi]
        assert sorted(chunk.tolist()) == list(range(lo, hi))
        cls = 15 - (counts[chunk] * 16) // (counts[lo:hi].max() + 1)
        assert np.all(np.diff(cls) >= 0)
        for c in np.unique(cls):
            assert np.all(np.diff(chunk[cls == c]) > 0)
    assert order[0] < 4 and counts[order[0]] == nt


@pytest.mark.parametrize("b,nt,h", [(1, 1, 1), (1, 2, 1), (1, 3, 2), (1, 7, 1)])
def test_fewer_items_than_xcd_chunks(b, nt, h):
    # 1 to 7 (batch, head, tile) items: some XCD chunks of the item order are
    # empty or hold a single item
    q, k, v = (randn_bf16((b, nt * 64, h, 128), 370 + 10 * nt + j) for j in range(3))
    rng = np.random.default_rng(37 + nt)
    bmap = rng.random((b, h, nt, nt)) < 0.6
    bmap[..., 0, 0] = True
    sizes = np.full(nt, 64, dtype=np.int32)
    sizes[-1] = 41
    announce("sparse few items", b, nt, h)
    out, lse = run(q, k, v, bmap, sizes, 128 ** -0.5)
    ref_o, ref_l = oracle.block_sparse_attention(q, k, v, bmap, sizes, 128 ** -0.5)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def test_item_order_beyond_staged_counts():
    # 33600 items, 4200 per XCD chunk: the order kernel keeps the first 4096
    # counts of a chunk in LDS and re-reads the rest from memory. Every row
    # keeps one key tile; rows a % 97 == 0 keep 40 more (long items in every
    # chunk, also past position 4096 of a chunk).
    b, nt, hq, hkv, d = 1, 2800, 12, 1, 128
    rows = b * hq * nt
    q = randn_bf16_on((b, nt * 64, hq, d), 360, "cuda")
    k, v = (dev(randn_bf16((b, nt * 64, hkv, d), 361 + j)) for j in range(2))
    bmap = np.zeros((b, hq, nt, nt), dtype=np.uint8)
    a_idx, h_idx = np.arange(nt)[None, :], np.arange(hq)[:, None]
    bmap[0, h_idx, a_idx, (7 * a_idx + 13 * h_idx) % nt] = 1
    long_rows = np.arange(0, nt, 97)
    for j in range(40):
        bmap[0, :, long_rows, (3 * long_rows + 61 * j + 1) % nt] = 1
    sizes = np.full(nt, 64, dtype=np.int32)
    scale = d ** -0.5
    ws = torch.empty(sav.attn_block_sparse_workspace_size(b, hq, nt), dtype=torch.uint8, device="cuda")
    announce("sparse item order beyond staged counts", rows)
    out, lse = sav.attn_block_sparse_fwd(q, k, v, dev(bmap), dev(sizes), scale, return_lse=True, workspace=ws)
    torch.cuda.synchronize()
    words = ws.view(torch.int32)[rows * nt:rows * nt + 2 * rows].cpu().numpy()
    counts = bmap.reshape(rows, nt).sum(1, dtype=np.int64)
    assert np.array_equal(words[:rows], counts)
    order = words[rows:]
    per = (rows + 7) // 8
    assert per > 4096
    for x in range(8):
        lo, hi = x * per, min((x + 1) * per, rows)
        chunk = order[lo:hi]
        assert np.array_equal(np.sort(chunk), np.arange(lo, hi))
        cls = 15 - (counts[chunk] * 16) // (counts[lo:hi].max() + 1)
        assert np.all(np.diff(cls) >= 0)
        for c in np.unique(cls):
            assert np.all(np.diff(chunk[cls == c]) > 0)
    # sampled items (long and short, early and past position 4096 of a chunk)
    # against dense attention over their kept tiles
    kh, vh = k.cpu(), v.cpu()
    for item in [0, 97, 4200 * 3 + 4150, 4200 * 3 + 4151, 4200 * 7 + 4199 - 41, rows - 1,
                 2 * nt + 97 * 5, 5 * nt + 97 * 28]:
        h, a = divmod(item, nt)
        kept = np.nonzero(bmap[0, h, a])[0]
        sel = torch.from_numpy(np.concatenate([np.arange(c * 64, c * 64 + 64) for c in kept]))
        ref_o, ref_l = oracle.dense_attention(q[:, a * 64:a * 64 + 64, h:h + 1].cpu(), kh[:, sel], vh[:, sel], scale,
                                              False)
        assert_close("out", host(out[:, a * 64:a * 64 + 64, h:h + 1]), ref_o, OUT_TOL, bf16_output=True,
                     few_keys=True)
        assert_close("lse", host(lse[:, h:h + 1, a * 64:a * 64 + 64]), ref_l, LSE_TOL)


def test_guards_and_pad_rows_zero():
    shape, tile = (3, 5, 6), (2, 2, 3)
    (qt, kt, vt), sizes = _tiled(shape, tile, 1, 2, 2, 64, seed=330)
    nt = sizes.size
    bmap = np.random.default_rng(1).random((1, 2, nt, nt)) < 0.5
    announce("sparse guards")
    q, k, v = dev(qt), dev(kt), dev(vt)
    out, og = guarded_empty(q.shape, torch.bfloat16)
    lse, lg = guarded_empty((1, 2, nt * 64), torch.float32)
    sav.attn_block_sparse_fwd(q, k, v, dev(bmap.astype(np.uint8)), dev(sizes), 0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    assert guard_intact(og) and guard_intact(lg)
    pad = (np.arange(nt * 64) % 64) >= np.repeat(sizes, 64)
    assert torch.all(out[:, torch.from_numpy(pad)] == 0)
    assert torch.all(torch.isneginf(lse[:, :, torch.from_numpy(pad)]))


def test_kept_tile_probe_bit_exact():
    """K = 0 except one selected key per head with a logit 512 above the rest;
    every query tile whose map keeps the selected key's tile must return that
    key's V bit-exactly (V encodes tile and row)."""
    nt, h, d = 9, 3, 64
    q = torch.full((1, nt * 64, h, d), 8.0, dtype=torch.bfloat16)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    v[0, :, :, 0] = (torch.arange(nt * 64) // 64).view(-1, 1).to(torch.bfloat16)
    v[0, :, :, 1] = (torch.arange(nt * 64) % 64).view(-1, 1).to(torch.bfloat16)
    sel = [5 * 64 + 17, 0, nt * 64 - 1]
    for hh, j in enumerate(sel):
        k[0, j, hh] = 8.0
    rng = np.random.default_rng(5)
    bmap = rng.random((1, h, nt, nt)) < 0.5
    sizes = np.full(nt, 64, dtype=np.int32)
    announce("sparse probe")
    out = run(q, k, v, bmap, sizes, 0.125, with_lse=False).cpu()
    hits = 0
    for hh, j in enumerate(sel):
        for a in range(nt):
            if bmap[0, hh, a, j // 64]:
                assert torch.equal(out[0, a * 64:(a + 1) * 64, hh], v[0, j, hh].expand(64, d))
                hits += 1
    assert hits >= 6


def test_config5_full_size_with_oracle_map_every_tile():
    case = config5()
    part, sizes, non_pad, untile = oracle.tile_metadata(case.video_shape, case.tile_shape, 64)
    nt = sizes.size

    def tile_order(x):
        t = torch.zeros((x.shape[0], nt * 64) + tuple(x.shape[2:]), dtype=x.dtype)
        t[:, torch.from_numpy(non_pad)] = x[:, torch.from_numpy(part)]
        return t

    qt, kt, vt = tile_order(case.q), tile_order(case.k), tile_order(case.v)
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes), oracle.pool_tiles(kt, sizes), case.scale)
    bmap = oracle.topk_block_map(scores, case.topk)
    assert np.all(bmap.sum(-1) == 32)
    announce("sparse config5")
    out, lse = run(qt, kt, vt, bmap, sizes, case.scale)
    ref_o, ref_l = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, case.scale)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


# --------------------------------------------------------------------------
# tile geometry and block map built on the GPU
# --------------------------------------------------------------------------

def check_map_is_valid_topk(gpu_map, scores, topk, eps=1e-6):
    """Where the fp64 oracle's k-th and (k+1)-th scores of a row are apart by
    more than eps the kept set is unique and must match exactly; otherwise every
    kept score must be >= the k-th largest - eps and every dropped one <= it + eps."""
    s = np.asarray(scores, dtype=np.float64)
    g = np.asarray(gpu_map).astype(bool)
    n = s.shape[-1]
    keep = min(topk, n)
    assert np.all(g.sum(-1) == keep)
    if keep == n:
        return 0
    srt = -np.sort(-s, axis=-1)
    kth, nxt = srt[..., keep - 1], srt[..., keep]
    unique = (kth - nxt) > eps
    ref = oracle.topk_block_map(s, topk)
    assert np.array_equal(g[unique], ref[unique])
    kept_min = np.where(g, s, np.inf).min(-1)
    drop_max = np.where(~g, s, -np.inf).max(-1)
    assert np.all(kept_min >= kth - eps) and np.all(drop_max <= kth + eps)
    return int((~unique).sum())


@pytest.mark.parametrize("shape,tile", [((5, 7, 9), (4, 4, 4)), ((3, 2, 5), (2, 2, 3)), ((16, 32, 32), (4, 4, 4)),
                                        ((1, 1, 3), (4, 4, 4))])
def test_tile_gather_untile_bit_exact(shape, tile):
    n = int(np.prod(shape))
    x = randn_bf16((2, n, 3, 64), 77)
    announce("tile gather", shape, tile)
    xt, sizes = sav.attn_vsa_tile_gather(dev(x), shape, tile)
    back = sav.attn_vsa_untile(xt, shape, tile)
    torch.cuda.synchronize()
    part, ref_sizes, non_pad, untile = oracle.tile_metadata(shape, tile, 64)
    ref_t = oracle.to_tile_order(x.view(torch.int16).numpy(), shape, tile)  # integer view: exact bytes
    assert np.array_equal(sizes.cpu().numpy(), ref_sizes)
    assert np.array_equal(xt.cpu().view(torch.int16).numpy(), ref_t)
    assert torch.equal(back.cpu().view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("topk", [1, 4, 12, 20])
def test_block_map_matches_oracle_topk(topk):
    shape, tile = (5, 7, 9), (4, 4, 4)
    (qt, kt, vt), sizes = _tiled(shape, tile, 2, 4, 2, 128, seed=340)
    announce("vsa block map", topk)
    gmap = sav.attn_vsa_block_map(dev(qt), dev(kt), dev(sizes), 128 ** -0.5, topk)
    torch.cuda.synchronize()
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes),
                                  np.repeat(oracle.pool_tiles(kt, sizes), 2, axis=1), 128 ** -0.5)
    check_map_is_valid_topk(gmap.cpu().numpy(), scores, topk)


def test_raster_pipeline_end_to_end():
    """raster q/k/v -> tile order -> GPU block map -> block-sparse -> untile, against
    raster-order oracle attention with the same (GPU-built, validated) map."""
    shape, tile, hq, d, topk = (5, 7, 9), (4, 4, 4), 2, 64, 5
    n = int(np.prod(shape))
    q, k, v = (randn_bf16((1, n, hq, d), 350 + j) for j in range(3))
    announce("vsa pipeline")
    prep = sav.vsa_prepare(dev(q), dev(k), dev(v), shape, tile, topk, d ** -0.5)
    out_t = sav.attn_block_sparse_fwd(prep["q"], prep["k"], prep["v"], prep["block_map"], prep["tile_sizes"],
                                      d ** -0.5)
    out = sav.attn_vsa_untile(out_t, shape, tile)
    torch.cuda.synchronize()
    bmap = prep["block_map"].cpu().numpy().astype(bool)
    _, sizes, _, _ = oracle.tile_metadata(shape, tile, 64)
    qt = oracle.to_tile_order(q.double().numpy(), shape, tile)
    kt = oracle.to_tile_order(k.double().numpy(), shape, tile)
    vt = oracle.to_tile_order(v.double().numpy(), shape, tile)
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes), oracle.pool_tiles(kt, sizes), d ** -0.5)
    check_map_is_valid_topk(bmap, scores, topk)
    ref_t, _ = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, d ** -0.5)
    assert_close("out", host(out), oracle.from_tile_order(ref_t, shape, tile), OUT_TOL, bf16_output=True,
                 few_keys=True)


def test_config5_gpu_map_matches_oracle_map():
    case = config5()
    announce("config5 gpu map")
    prep = sav.vsa_prepare(dev(case.q), dev(case.k), dev(case.v), case.video_shape, case.tile_shape, case.topk,
                           case.scale)
    torch.cuda.synchronize()
    part, sizes, non_pad, _ = oracle.tile_metadata(case.video_shape, case.tile_shape, 64)
    nt = sizes.size
    qt = torch.zeros((1, nt * 64, 12, 128), dtype=torch.bfloat16)
    kt = torch.zeros_like(qt)
    qt[:, torch.from_numpy(non_pad)] = case.q[:, torch.from_numpy(part)]
    kt[:, torch.from_numpy(non_pad)] = case.k[:, torch.from_numpy(part)]
    assert torch.equal(prep["q"].cpu().view(torch.int16), qt.view(torch.int16))
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes), oracle.pool_tiles(kt, sizes), case.scale)
    near_ties = check_map_is_valid_topk(prep["block_map"].cpu().numpy(), scores, case.topk)
    print(f"[parity] config5 map: rows with a near-tie at the cut: {near_ties} of {scores.shape[2] * 12}")


def _gate_tiled(shape, tile, b, hq, d, seed):
    """A synthetic gate in tile order, zero on padding rows (as the page builds it)."""
    n = int(np.prod(shape))
    part, sizes, non_pad, _ = oracle.tile_metadata(shape, tile, 64)
    g = randn_bf16((b, n, hq, d), seed)
    t = torch.zeros((b, sizes.size * 64, hq, d), dtype=g.dtype)
    t[:, torch.from_numpy(non_pad)] = g[:, torch.from_numpy(part)]
    return t


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_compressed_branch_partial_tiles(d, hq, hkv):
    shape, tile = (5, 7, 9), (4, 4, 4)
    (qt, kt, vt), sizes = _tiled(shape, tile, 2, hq, hkv, d, seed=350 + d)
    gate = _gate_tiled(shape, tile, 2, hq, d, 360 + d)
    base = randn_bf16(qt.shape, 370 + d)
    scale = d ** -0.5
    announce("compressed branch", d, hq, hkv, sizes.tolist())
    out = dev(base)
    sav.attn_vsa_compressed_add(dev(qt), dev(kt), dev(vt), dev(sizes.astype(np.int32)), dev(gate), scale, out)
    torch.cuda.synchronize()
    ref, _ = oracle.compressed_branch(qt, kt, vt, sizes, scale, gate, base)
    assert_close("out", host(out), ref, OUT_TOL, bf16_output=True)


@pytest.mark.parametrize("shape", [(9, 7, 9), (20, 20, 21), (13, 4, 4)])
def test_compressed_branch_ragged_tile_counts(shape):
    # 18, 150 and 4 tiles: score rows that are not a multiple of 4 wide, GEMM
    # tiles cut by the tile count, and a single partial output tile
    tile = (4, 4, 4)
    (qt, kt, vt), sizes = _tiled(shape, tile, 1, 4, 2, 128, seed=385)
    gate = _gate_tiled(shape, tile, 1, 4, 128, 386)
    base = randn_bf16(qt.shape, 387)
    announce("compressed branch ragged", shape, sizes.size)
    out = dev(base)
    sav.attn_vsa_compressed_add(dev(qt), dev(kt), dev(vt), dev(sizes.astype(np.int32)), dev(gate), 128 ** -0.5, out)
    torch.cuda.synchronize()
    ref, _ = oracle.compressed_branch(qt, kt, vt, sizes, 128 ** -0.5, gate, base)
    assert_close("out", host(out), ref, OUT_TOL, bf16_output=True)


@pytest.mark.parametrize("shape,topk", [((9, 7, 9), 5), ((20, 20, 21), 17), ((12, 24, 28), 9), ((32, 28, 36), 40),
                                        ((32, 32, 36), 64), ((44, 44, 36), 50)])
def test_block_map_ragged_tile_counts(shape, topk):
    tile = (4, 4, 4)
    (qt, kt, vt), sizes = _tiled(shape, tile, 1, 4, 2, 128, seed=388)
    announce("vsa block map ragged", shape, sizes.size, topk)
    gmap = sav.attn_vsa_block_map(dev(qt), dev(kt), dev(sizes), 128 ** -0.5, topk)
    torch.cuda.synchronize()
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes),
                                  np.repeat(oracle.pool_tiles(kt, sizes), 2, axis=1), 128 ** -0.5)
    check_map_is_valid_topk(gmap.cpu().numpy(), scores, topk)


def test_block_map_exact_ties_lower_index_wins():
    # 64 full tiles whose keys are one of three exactly representable rows, and
    # one query row everywhere: every score is exact and ties are exact, so the
    # map must equal the oracle's (lower tile index first) bit for bit
    shape, tile, d = (16, 16, 16), (4, 4, 4), 128
    part, sizes, non_pad, _ = oracle.tile_metadata(shape, tile, 64)
    nt = sizes.size
    rng = np.random.default_rng(392)
    protos = torch.tensor(rng.integers(-4, 5, (3, d)) * 0.25, dtype=torch.bfloat16)
    which = rng.integers(0, 3, nt)
    kt = torch.zeros((1, nt * 64, 1, d), dtype=torch.bfloat16)
    for c in range(nt):
        kt[0, c * 64:(c + 1) * 64, 0] = protos[which[c]]
    qt = torch.zeros_like(kt)
    qt[0, :, 0] = torch.tensor(rng.integers(-4, 5, d) * 0.25, dtype=torch.bfloat16)
    scores = oracle.pooled_scores(oracle.pool_tiles(qt, sizes), oracle.pool_tiles(kt, sizes), 0.125)
    for topk in (1, 7, 21, 22, 40):
        gmap = sav.attn_vsa_block_map(dev(qt), dev(kt), dev(sizes), 0.125, topk)
        torch.cuda.synchronize()
        assert np.array_equal(gmap.cpu().numpy().astype(bool), oracle.topk_block_map(scores, topk)), topk


def test_compressed_branch_zero_gate_keeps_output():
    shape, tile = (4, 8, 8), (4, 4, 4)
    (qt, kt, vt), sizes = _tiled(shape, tile, 1, 3, 3, 128, seed=380)
    base = randn_bf16(qt.shape, 381)
    out = dev(base)
    sav.attn_vsa_compressed_add(dev(qt), dev(kt), dev(vt), dev(sizes.astype(np.int32)), dev(torch.zeros_like(qt)),
                                128 ** -0.5, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), base)


def test_compressed_branch_config5():
    case = config5()
    prep = sav.vsa_prepare(dev(case.q), dev(case.k), dev(case.v), case.video_shape, case.tile_shape, case.topk,
                           case.scale)
    qt, kt, vt, sizes = prep["q"], prep["k"], prep["v"], prep["tile_sizes"]
    gate = dev(_gate_tiled(case.video_shape, case.tile_shape, 1, case.num_heads, case.head_dim, 390))
    base = dev(randn_bf16(tuple(qt.shape), 391))
    out = base.clone()
    announce("compressed branch config5")
    sav.attn_vsa_compressed_add(qt, kt, vt, sizes, gate, case.scale, out)
    torch.cuda.synchronize()
    ref, _ = oracle.compressed_branch(qt.cpu(), kt.cpu(), vt.cpu(), sizes.cpu().numpy(), case.scale, gate.cpu(),
                                      base.cpu())
    assert_close("out", host(out), ref, OUT_TOL, bf16_output=True)


H3_CASES = [((70, 5), (2, 5, 4)), ((130, 64, 1), (5, 9, 7)), ((), (5, 7, 9)), ((300,), (0, 0, 0)),
            ((0, 512), (16, 32, 32))]


@pytest.mark.parametrize("segs,shape", H3_CASES)
def test_h3_tile_gather_untile_bit_exact(segs, shape):
    n = sum(segs) + int(np.prod(shape))
    x = randn_bf16((2, n, 3, 64), 395)
    announce("h3 tile gather", segs, shape)
    xt, sizes = sav.attn_vsa_h3_tile_gather(dev(x), segs, shape)
    back = sav.attn_vsa_h3_untile(xt, segs, shape)
    torch.cuda.synchronize()
    _, ref_sizes, _, _, n_pre, _ = oracle.h3_tile_metadata(segs, shape)
    ref_t = oracle.h3_to_tile_order(x.view(torch.int16).numpy(), segs, shape)
    assert np.array_equal(sizes.cpu().numpy(), ref_sizes)
    assert np.array_equal(xt.cpu().view(torch.int16).numpy(), ref_t)
    assert torch.equal(back.cpu().view(torch.int16), x.view(torch.int16))
    assert sav.attn_vsa_h3_num_tiles(segs, shape)[0] == n_pre


def _h3_scores(qt, kt, sizes, group, scale):
    return oracle.pooled_scores(oracle.pool_tiles(qt, sizes), np.repeat(oracle.pool_tiles(kt, sizes), group, axis=1),
                                scale)


def check_h3_map(gmap, scores, n_pre, topk):
    g = np.asarray(gmap).astype(bool)
    n_vid = g.shape[-1] - n_pre
    if min(topk, n_vid) == n_vid:
        assert g.all()
        return
    assert g[..., :n_pre, :].all() and g[..., :n_pre].all()  # prefix rows and columns kept
    check_map_is_valid_topk(g[..., n_pre:, n_pre:], np.asarray(scores)[..., n_pre:, n_pre:], topk)


@pytest.mark.parametrize("segs,shape,topk", [((70, 5), (8, 9, 10), 5), ((130, 64, 1), (5, 9, 7), 4),
                                             ((512,), (16, 16, 16), 20), ((70,), (4, 4, 8), 40),
                                             ((2000, 100), (20, 32, 32), 32)])
def test_h3_block_map(segs, shape, topk):
    n = sum(segs) + int(np.prod(shape))
    q, k = randn_bf16((1, n, 4, 128), 396), randn_bf16((1, n, 2, 128), 397)
    announce("h3 block map", segs, shape, topk)
    qt, sizes = sav.attn_vsa_h3_tile_gather(dev(q), segs, shape)
    kt, _ = sav.attn_vsa_h3_tile_gather(dev(k), segs, shape)
    n_pre, nt = sav.attn_vsa_h3_num_tiles(segs, shape)
    gmap = sav.attn_vsa_h3_block_map(qt, kt, sizes, n_pre, 128 ** -0.5, topk)
    torch.cuda.synchronize()
    scores = _h3_scores(qt.cpu(), kt.cpu(), sizes.cpu().numpy(), 2, 128 ** -0.5)
    check_h3_map(gmap.cpu().numpy(), scores, n_pre, topk)


def test_h3_raster_pipeline_end_to_end():
    """raster [prefix + video] q/k/v -> H3 tiles -> GPU H3 map -> block-sparse ->
    untile, against the oracle on the same (validated) map."""
    segs, shape, hq, d, topk = (90, 40), (5, 7, 9), 2, 128, 6
    n = sum(segs) + int(np.prod(shape))
    q, k, v = (randn_bf16((1, n, hq, d), 398 + j) for j in range(3))
    announce("h3 pipeline")
    prep = sav.vsa_h3_prepare(dev(q), dev(k), dev(v), segs, shape, topk, d ** -0.5)
    out_t = sav.attn_block_sparse_fwd(prep["q"], prep["k"], prep["v"], prep["block_map"], prep["tile_sizes"],
                                      d ** -0.5)
    out = sav.attn_vsa_h3_untile(out_t, segs, shape)
    torch.cuda.synchronize()
    bmap = prep["block_map"].cpu().numpy().astype(bool)
    _, sizes, _, _, n_pre, _ = oracle.h3_tile_metadata(segs, shape)
    qt, kt, vt = (oracle.h3_to_tile_order(x.double().numpy(), segs, shape) for x in (q, k, v))
    check_h3_map(bmap, _h3_scores(qt, kt, sizes, 1, d ** -0.5), n_pre, topk)
    ref_t, _ = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, d ** -0.5)
    assert_close("out", host(out), oracle.h3_from_tile_order(ref_t, segs, shape), OUT_TOL, bf16_output=True)


def test_h3_full_size_sampled_tiles():
    # workload 11: 512 prefix rows (8 dense tiles) ahead of the 16x32x32 video;
    # the GPU-built H3 map is checked against fp64 scores, then sampled prefix
    # and video query tiles against the oracle on that map
    from workloads import config11

    case = config11()
    segs = case.extra["prefix_segments"]
    announce("h3 full size")
    prep = sav.vsa_h3_prepare(dev(case.q), dev(case.k), dev(case.v), segs, case.video_shape, case.topk, case.scale)
    torch.cuda.synchronize()
    qt, kt, vt = prep["q"].cpu(), prep["k"].cpu(), prep["v"].cpu()
    sizes = prep["tile_sizes"].cpu().numpy()
    n_pre = prep["num_prefix_tiles"]
    bmap = prep["block_map"].cpu().numpy().astype(bool)
    assert n_pre == 8 and np.array_equal(sizes, oracle.h3_tile_metadata(segs, case.video_shape)[1])
    check_h3_map(bmap, _h3_scores(qt, kt, sizes, 1, case.scale), n_pre, case.topk)
    out, lse = run(qt, kt, vt, bmap.astype(np.uint8), sizes, case.scale)
    tiles = [0, 7, 8, 9, 100, 263]
    heads = [0, 11]
    ref_o, ref_l = oracle.block_sparse_attention(qt, kt, vt, bmap, sizes, case.scale, heads=heads, q_tiles=tiles)
    rows = np.concatenate([np.arange(a * 64, a * 64 + 64) for a in tiles])
    rt = torch.from_numpy(rows).cuda()
    assert_close("out", host(out.index_select(1, rt))[:, :, heads], ref_o[:, rows][:, :, heads], OUT_TOL,
                 bf16_output=True)
    assert_close("lse", host(lse.index_select(2, rt))[:, heads], ref_l[:, heads][:, :, rows], LSE_TOL)


@pytest.mark.parametrize("segs,shape,d,hq,hkv,topk", [((70, 5), (2, 5, 4), 64, 4, 2, 3),
                                                    ((130, 64, 1), (5, 9, 7), 128, 2, 2, 4),
                                                    ((), (5, 7, 9), 256, 3, 1, 5),
                                                    ((300,), (0, 0, 0), 128, 2, 1, 2),
                                                    ((), (16, 32, 32), 128, 12, 12, 32)])
def test_gather_block_map_equals_separate_calls(segs, shape, d, hq, hkv, topk):
    """The one-call gather + map gives the tile-order copies, sizes and map of the
    separate gather and map calls bit for bit (the tile means are summed in the
    same order), and its copies are the oracle's tile order."""
    n = sum(segs) + int(np.prod(shape))
    q, k = randn_bf16((2, n, hq, d), 399), randn_bf16((2, n, hkv, d), 400)
    announce("gather block map", segs, shape, d, hq, hkv, topk)
    scale = d ** -0.5
    qt, kt, sizes, gmap = sav.attn_vsa_h3_gather_block_map(dev(q), dev(k), segs, shape, scale, topk)
    rq, rsizes = sav.attn_vsa_h3_tile_gather(dev(q), segs, shape)
    rk, _ = sav.attn_vsa_h3_tile_gather(dev(k), segs, shape)
    n_pre, _ = sav.attn_vsa_h3_num_tiles(segs, shape)
    rmap = sav.attn_vsa_h3_block_map(rq, rk, rsizes, n_pre, scale, topk)
    torch.cuda.synchronize()
    assert torch.equal(qt.view(torch.int16), rq.view(torch.int16))
    assert torch.equal(kt.view(torch.int16), rk.view(torch.int16))
    assert torch.equal(sizes, rsizes)
    assert torch.equal(gmap, rmap)
    assert np.array_equal(qt.cpu().view(torch.int16).numpy(), oracle.h3_to_tile_order(q.view(torch.int16).numpy(),
                                                                                       segs, shape))
    if sizes.numel() <= 64:
        scores = _h3_scores(qt.cpu(), kt.cpu(), sizes.cpu().numpy(), hq // hkv, scale)
        check_h3_map(gmap.cpu().numpy(), scores, n_pre, topk)
