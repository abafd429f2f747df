"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that at least one pin fails for each. This shows the pins can tell a
wrong oracle from a right one."""

import numpy as np
import pytest

import oracle.attention as A
import oracle.blockmap as BM
import oracle.tiles as T
from tests import test_oracle_attention as ta
from tests import test_oracle_paged as tp
from tests import test_oracle_sparse as ts

_orig_attend = A._attend
_orig_causal = A._causal_allowed


def _attend_no_scale(q, k, v, scale, allowed):
    return _orig_attend(q, k, v, 1.0, allowed)


def _attend_neg_scale(q, k, v, scale, allowed):
    return _orig_attend(q, k, v, -scale, allowed)


def _attend_log2_lse(q, k, v, scale, allowed):
    o, l_ = _orig_attend(q, k, v, scale, allowed)
    return o, l_ / np.log(2.0)


def _attend_no_normalise(q, k, v, scale, allowed):
    o, l_ = _orig_attend(q, k, v, scale, allowed)
    return o * np.exp(l_ - l_.max() if np.isfinite(l_).any() else 0.0)[:, None] * 2.0, l_


def _causal_top_left(rows, lq, lk):
    return np.arange(lk)[None, :] <= rows[:, None]


def _causal_off_by_one(rows, lq, lk):
    return np.arange(lk)[None, :] < rows[:, None] + (lk - lq)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mutant", [_attend_no_scale, _attend_neg_scale, _attend_log2_lse, _attend_no_normalise])
def test_attend_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "_attend", mutant)
    caught = _fails(ta.test_closed_form_two_keys) or _fails(ta.test_closed_form_scale_and_sign)
    caught = caught or _fails(ta.test_torch_sdpa_fp64, False)
    assert caught


@pytest.mark.parametrize("mutant", [_causal_top_left, _causal_off_by_one])
def test_causal_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "_causal_allowed", mutant)
    assert _fails(ta.test_torch_sdpa_fp64, True) or _fails(ta.test_causal_row0_attends_only_itself)


def test_paged_wrong_offset_is_caught(monkeypatch):
    def paged_block_major(q, kv_cache, block_tables, context_lens, scale, seqs=None):
        # plant: read the slots of every block in reverse order
        cache = kv_cache.clone()
        cache = cache.flip(2)  # equivalent to reading the block's slots backwards
        return orig_paged(q, cache, block_tables, context_lens, scale, seqs)

    orig_paged = A.paged_decode_attention
    monkeypatch.setattr(tp.oracle, "paged_decode_attention", paged_block_major)
    assert _fails(tp.test_paged_equals_contiguous_gather)


def test_tile_order_mutant_is_caught(monkeypatch):
    orig_map = T._video_map

    def boxes_reversed(shape, tile, block):
        box, row, sizes = orig_map(shape, tile, block)
        return sizes.size - 1 - box, row, sizes[::-1].copy()

    monkeypatch.setattr(T, "_video_map", boxes_reversed)
    assert _fails(ts.test_geometry_hand_example)


def test_unclipped_box_rows_mutant_is_caught(monkeypatch):
    # rows numbered as if every box had its full (tt, th, tw) extent
    def rows_unclipped(shape, tile, block):
        box, _, sizes = orig_map(shape, tile, block)
        t, h, w = np.meshgrid(*(np.arange(int(s)) for s in shape), indexing="ij")
        tt, th, tw = tile
        row = (t % tt) * th * tw + (h % th) * tw + (w % tw)
        return box, row.reshape(-1).astype(np.int64), sizes

    orig_map = T._video_map
    monkeypatch.setattr(T, "_video_map", rows_unclipped)
    assert _fails(lambda: ts.test_geometry_properties((5, 7, 9), (4, 4, 4)))


def test_topk_smallest_mutant_is_caught(monkeypatch):
    orig = BM.topk_block_map

    def topk_smallest(scores, topk):
        return orig(-np.asarray(scores), topk)

    monkeypatch.setattr(ts.oracle, "topk_block_map", topk_smallest)
    assert _fails(ts.test_topk_map_properties)


def test_gqa_modulo_mutant_is_caught(monkeypatch):
    orig_varlen = A.varlen_attention

    def varlen_mod(q, k, v, cu_q, cu_k, scale, causal, rows=None):
        # plant: query head h reads kv head h % Hkv
        import torch

        hq, hkv = q.shape[1], k.shape[1]
        idx = torch.tensor([h % hkv for h in range(hq)])
        kk = (k if isinstance(k, torch.Tensor) else torch.from_numpy(k)).index_select(1, idx)
        vv = (v if isinstance(v, torch.Tensor) else torch.from_numpy(v)).index_select(1, idx)
        return orig_varlen(q, kk, vv, cu_q, cu_k, scale, causal, rows)

    monkeypatch.setattr(ta.oracle, "varlen_attention", varlen_mod)
    assert _fails(ta.test_torch_sdpa_fp64, False)


def test_paged_prefill_mutants_are_caught(monkeypatch):
    from tests import test_oracle_paged_prefill as tpp

    orig_gather = A._gather_paged

    def gather_reversed_slots(kv_cache, plane, blk, off):
        # plant: read each block's slots back to front
        return orig_gather(kv_cache, plane, blk, kv_cache.shape[2] - 1 - off)

    monkeypatch.setattr(A, "_gather_paged", gather_reversed_slots)
    assert _fails(tpp.test_brute_force_tiny)
    monkeypatch.setattr(A, "_gather_paged", orig_gather)

    # plant: top-left causal alignment (new queries treated as the first positions)
    monkeypatch.setattr(A, "_causal_allowed", _causal_top_left)
    assert _fails(tpp.test_brute_force_tiny)
    monkeypatch.setattr(A, "_causal_allowed", _orig_causal)

    orig_write = A.paged_kv_write

    def write_swapped(kv_cache, k, v, slot_mapping):
        # plant: K and V planes exchanged
        return orig_write(kv_cache, v, k, slot_mapping)

    monkeypatch.setattr(tpp.oracle, "paged_kv_write", write_swapped)
    assert _fails(tpp.test_kv_write_worked_example)


def test_compressed_branch_mutants_are_caught(monkeypatch):
    from tests import test_oracle_compressed as tc

    orig_pool = BM.pool_tiles

    def pool_sum_not_mean(x, sizes, block=64):
        # plant: tile sums instead of tile means
        return orig_pool(x, np.ones_like(np.asarray(sizes)), block)

    monkeypatch.setattr(BM, "pool_tiles", pool_sum_not_mean)
    assert _fails(tc.test_brute_force_tiny)
    monkeypatch.setattr(BM, "pool_tiles", orig_pool)

    orig_scores = BM.pooled_scores

    def scores_transposed(qp, kp, scale):
        # plant: key tiles scored against query tiles the other way round
        return np.swapaxes(orig_scores(qp, kp, scale), -1, -2)

    monkeypatch.setattr(BM, "pooled_scores", scores_transposed)
    assert _fails(tc.test_brute_force_tiny)


def test_variant_mutants_are_caught(monkeypatch):
    from tests import test_oracle_variants as tv

    orig_window = tv.oracle.sliding_window_decode_attention

    def window_one_short(q, kv_cache, block_tables, context_lens, scale, window, seqs=None):
        # plant: the window counts the query itself among its tokens
        return orig_window(q, kv_cache, block_tables, context_lens, scale, max(window - 1, 0), seqs)

    monkeypatch.setattr(tv.oracle, "sliding_window_decode_attention", window_one_short)
    assert _fails(tv.test_window_brute_force_tiny)
    monkeypatch.setattr(tv.oracle, "sliding_window_decode_attention", orig_window)

    orig_padded = tv.oracle.padded_prefix_attention

    def padded_key_lengths_for_queries(q, k, v, q_lens, k_lens, scale, causal):
        # plant: the query prefix taken from the key lengths
        return orig_padded(q, k, v, np.minimum(k_lens, q.shape[1]), k_lens, scale, causal)

    monkeypatch.setattr(tv.oracle, "padded_prefix_attention", padded_key_lengths_for_queries)
    assert _fails(tv.test_padded_prefix_equals_packed_varlen)
    monkeypatch.setattr(tv.oracle, "padded_prefix_attention", orig_padded)

    orig_masked = tv.oracle.masked_attention

    def masked_keeps_every_query(q, k, v, key_mask, scale, causal, mask_queries):
        # plant: self-attention keeps the padding tokens' query rows
        return orig_masked(q, k, v, key_mask, scale, causal, False)

    monkeypatch.setattr(tv.oracle, "masked_attention", masked_keeps_every_query)
    assert _fails(tv.test_self_mask_with_holes_brute_force_tiny)


def test_h3_mutants_are_caught(monkeypatch):
    from tests import test_oracle_h3 as th

    orig_meta = th.oracle.h3_tile_metadata

    def segments_merged(prefix_segments, video_shape, tile=(4, 4, 4), block=64):
        # plant: the prefix chunked as one run instead of segment by segment
        return orig_meta((sum(prefix_segments),), video_shape, tile, block)

    monkeypatch.setattr(th.oracle, "h3_tile_metadata", segments_merged)
    assert _fails(th.test_hand_derived_geometry)
    monkeypatch.setattr(th.oracle, "h3_tile_metadata", orig_meta)

    orig_map = th.oracle.h3_block_map

    def prefix_columns_ranked(scores, n_prefix, n_video, topk):
        # plant: the prefix columns compete in the top-k instead of being kept
        out = BM.topk_block_map(scores, min(topk, n_video))
        out[..., :n_prefix, :] = True
        return out

    monkeypatch.setattr(th.oracle, "h3_block_map", prefix_columns_ranked)
    assert _fails(th.test_block_map_hand_scored)
