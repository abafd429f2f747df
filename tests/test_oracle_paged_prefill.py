"""Pins for the paged KV write and multi-token paged attention oracles: the
pages' worked slot example, write-then-read round trips, brute force on tiny
inputs (pure Python, no shared helper), the contiguous-varlen and decode
equivalences, the chunk-split identity and physical block relabelling."""

import math
import os

import numpy as np
import torch

import oracle
from workloads import paged_prefill_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_write_worked_example():
    # [ASC] AscendMetadata.slot_mapping: slots [35, 2, 17] with block size 16
    rows = np.loadtxt(os.path.join(GOLDEN, "slot_mapping_worked_example.txt"), dtype=np.int64, comments="#")
    slots = rows[:, 0]
    bs = int(rows[0, 1])
    cache = np.zeros((2, 4, bs, 1, 2))
    k = np.array([[[1.0, 10.0]], [[2.0, 20.0]], [[3.0, 30.0]]])
    v = -k
    out = oracle.paged_kv_write(cache, k, v, slots)
    for i, (_, _, blk, off) in enumerate(rows):
        assert np.array_equal(out[0, blk, off], k[i]) and np.array_equal(out[1, blk, off], v[i])
    written = np.zeros(cache.shape[:3], dtype=bool)
    written[:, rows[:, 2], rows[:, 3]] = True
    assert np.all(out[~written] == 0.0)
    assert np.all(cache == 0.0)  # the input is left alone


def test_kv_write_round_trip_and_skipped_slots():
    rng = np.random.default_rng(61)
    nb, bs, hkv, d = 6, 128, 2, 8
    cache = torch.randn((2, nb, bs, hkv, d), generator=torch.Generator().manual_seed(61)).to(torch.bfloat16)
    n = 300
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int32)
    slots[[5, 77, 200]] = -1  # tokens that are not stored
    k = torch.randn((n, hkv, d), generator=torch.Generator().manual_seed(62)).to(torch.bfloat16)
    v = torch.randn((n, hkv, d), generator=torch.Generator().manual_seed(63)).to(torch.bfloat16)
    out = oracle.paged_kv_write(cache, k, v, slots)
    touched = np.zeros((nb, bs), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        touched[blk, off] = True
        assert torch.equal(out[0, blk, off], k[i]) and torch.equal(out[1, blk, off], v[i])
    t = torch.from_numpy(~touched)
    assert torch.equal(out[:, t], cache[:, t])


def _brute(case):
    """Pure-Python statement: softmax over the visible keys of each query, the
    cache row of key t looked up token by token."""
    q = case.q.double().numpy()
    kc = case.kv_cache.double().numpy()
    cu = case.cu_seqlens_q
    group = case.num_heads // case.num_kv_heads
    out = np.zeros(q.shape)
    lse = np.full((case.num_heads, q.shape[0]), -np.inf)
    for b in range(case.batch):
        lq = int(cu[b + 1] - cu[b])
        lk = int(case.context_lens[b])
        for i in range(lq):
            for h in range(case.num_heads):
                hk = h // group
                logits, vals = [], []
                for j in range(lk):
                    if j > i + (lk - lq):
                        continue
                    blk = int(case.block_tables[b, j // case.block_size])
                    off = j % case.block_size
                    dot = sum(q[cu[b] + i, h, d] * kc[0, blk, off, hk, d] for d in range(q.shape[2]))
                    logits.append(case.scale * dot)
                    vals.append(kc[1, blk, off, hk])
                if not logits:
                    continue
                w = [math.exp(z) for z in logits]
                tot = sum(w)
                out[cu[b] + i, h] = sum(wj * vj for wj, vj in zip(w, vals)) / tot
                lse[h, cu[b] + i] = math.log(tot)
    return out, lse


def test_brute_force_tiny():
    # small logits (D=4), so no max subtraction is needed in the brute force
    case = paged_prefill_case([3, 1, 5, 2], [3, 130, 9, 1], num_heads=4, num_kv_heads=2, head_dim=4, seed=64,
                              block_size=128, spare_blocks=2)
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    ref_o, ref_l = _brute(case)
    assert np.allclose(out, ref_o, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(ref_l))  # the last sequence's early queries see no key
    fin = np.isfinite(ref_l)
    assert np.allclose(lse[fin], ref_l[fin], atol=1e-12)


def _case(seed=65):
    return paged_prefill_case([5, 64, 1, 130, 17], [5, 300, 129, 513, 40], num_heads=8, num_kv_heads=2,
                              head_dim=32, seed=seed, spare_blocks=3)


def test_equals_contiguous_varlen():
    case = _case()
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    for b in range(case.batch):
        lk = int(case.context_lens[b])
        rows = [(int(case.block_tables[b, t // case.block_size]), t % case.block_size) for t in range(lk)]
        k = torch.stack([case.kv_cache[0, blk, off] for blk, off in rows])
        v = torch.stack([case.kv_cache[1, blk, off] for blk, off in rows])
        q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        o2, l2 = oracle.varlen_attention(case.q[q0:q1], k, v, [0, q1 - q0], [0, lk], case.scale, True)
        assert np.allclose(out[q0:q1], o2, atol=1e-13) and np.allclose(lse[:, q0:q1], l2, atol=1e-13)


def test_single_query_per_sequence_is_decode():
    case = paged_prefill_case([1] * 6, [1, 127, 128, 129, 300, 513], num_heads=8, num_kv_heads=2, head_dim=32,
                              seed=66, spare_blocks=3)
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    o2, l2 = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                           case.scale)
    assert np.allclose(out, o2, atol=1e-13) and np.allclose(lse, l2, atol=1e-13)


def test_chunk_split_identity():
    # serving the queries of a sequence in two chunks (the first chunk sees the
    # context as it was before the second chunk's tokens) gives the same rows
    case = _case(seed=67)
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    b = 3  # 130 queries over 513 keys
    q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
    lk = int(case.context_lens[b])
    a = 50
    for lo, hi, ctx in ((q0, q0 + a, lk - (q1 - q0 - a)), (q0 + a, q1, lk)):
        o2, l2 = oracle.paged_prefill_attention(case.q[lo:hi], case.kv_cache, case.block_tables[b:b + 1],
                                                [0, hi - lo], [ctx], case.scale)
        assert np.allclose(out[lo:hi], o2, atol=1e-13) and np.allclose(lse[:, lo:hi], l2, atol=1e-13)


def test_physical_block_relabelling_invariance():
    case = _case(seed=68)
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    perm = np.random.default_rng(68).permutation(case.num_blocks)  # new id of old block i is perm[i]
    cache2 = torch.empty_like(case.kv_cache)
    cache2[:, torch.from_numpy(perm)] = case.kv_cache
    tables2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    o2, l2 = oracle.paged_prefill_attention(case.q, cache2, tables2, case.cu_seqlens_q, case.context_lens,
                                            case.scale)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_row_subset_matches_full():
    case = _case(seed=69)
    out, lse = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                              case.context_lens, case.scale)
    rows = np.array([0, 4, 5, 70, 71, 100, 215])
    o2, l2 = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                            case.context_lens, case.scale, rows=rows)
    # the same rows, computed in a smaller product (BLAS may round differently)
    assert np.allclose(out[rows], o2, atol=1e-13) and np.allclose(lse[:, rows], l2, atol=1e-13)
