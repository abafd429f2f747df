"""Pins for the paged-decode oracle: the pages' worked slot example, paged ==
contiguous gather (checked against the varlen oracle and torch SDPA), and
block-table indexing properties."""

import os

import numpy as np
import torch

import oracle
from workloads import paged_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slot_mapping_worked_example():
    rows = np.loadtxt(os.path.join(GOLDEN, "slot_mapping_worked_example.txt"), dtype=np.int64, comments="#")
    for slot, bs, blk, off in rows:
        b, o = oracle.slot_to_block_offset(np.array([slot]), int(bs))
        assert (int(b[0]), int(o[0])) == (blk, off)


def _small_case(seed=21, ctx=(1, 127, 128, 129, 300, 513)):
    return paged_case(list(ctx), num_heads=8, num_kv_heads=2, head_dim=32, seed=seed, block_size=128,
                      spare_blocks=3)


def _gather(case, b):
    length = int(case.context_lens[b])
    toks = []
    for t in range(length):  # token by token, the slot arithmetic spelled out
        blk = case.block_tables[b, t // case.block_size]
        toks.append((int(blk), t % case.block_size))
    k = torch.stack([case.kv_cache[0, blk, off] for blk, off in toks])
    v = torch.stack([case.kv_cache[1, blk, off] for blk, off in toks])
    return k, v


def test_paged_equals_contiguous_gather():
    case = _small_case()
    out, lse = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                             case.scale)
    for b in range(case.num_seqs):
        k, v = _gather(case, b)
        L = k.shape[0]
        # single query at the last position: bottom-right causal admits every key
        o2, l2 = oracle.varlen_attention(case.q[b:b + 1], k, v, [0, 1], [0, L], case.scale, True)
        assert np.allclose(out[b], o2[0], atol=1e-13) and np.allclose(lse[:, b], l2[:, 0], atol=1e-13)
        # torch SDPA in fp64 on the gathered keys
        qq = case.q[b].double()[:, None, :]  # [Hq, 1, D]
        kk = k.double().repeat_interleave(4, dim=1).transpose(0, 1)
        vv = v.double().repeat_interleave(4, dim=1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=case.scale)
        assert np.allclose(out[b], ref[:, 0].numpy(), atol=1e-12)


def test_table_tail_and_unused_blocks_never_read():
    case = _small_case(seed=22)
    out, lse = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                             case.scale)
    used = set()
    for b in range(case.num_seqs):
        n = -(-int(case.context_lens[b]) // case.block_size)
        used.update(int(x) for x in case.block_tables[b, :n])
        assert np.all(case.block_tables[b, n:] == -1)
    poisoned = case.kv_cache.clone()
    # poison every block that holds no live token, and the unused slots of each last block
    for blk in range(case.num_blocks):
        if blk not in used:
            poisoned[:, blk] = 1e4
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        n = -(-L // case.block_size)
        last = int(case.block_tables[b, n - 1])
        poisoned[:, last, L - (n - 1) * case.block_size:] = -1e4
    out2, lse2 = oracle.paged_decode_attention(case.q, poisoned, case.block_tables, case.context_lens, case.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_physical_block_relabelling_invariance():
    case = _small_case(seed=23)
    out, lse = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                             case.scale)
    rng = np.random.default_rng(0)
    relabel = rng.permutation(case.num_blocks)  # old block b moves to relabel[b]
    cache2 = torch.empty_like(case.kv_cache)
    cache2[:, torch.from_numpy(relabel)] = case.kv_cache
    tables2 = np.where(case.block_tables >= 0, relabel[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.paged_decode_attention(case.q, cache2, tables2, case.context_lens, case.scale)
    assert np.allclose(out, out2, atol=1e-15) and np.allclose(lse, lse2, atol=1e-15)


def test_seq_subset_matches_full():
    case = _small_case(seed=24)
    out, lse = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                             case.scale)
    sel = np.array([5, 0, 3])
    o2, l2 = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                           case.scale, seqs=sel)
    assert np.array_equal(o2, out[sel]) and np.array_equal(l2, lse[:, sel])
