"""Pins for the boundary-variant oracles (sliding-window decode, padded
prefix, key-padding mask): reductions to the already pinned varlen, dense and
paged-decode statements, closed forms, poisoned padding, and brute force on
tiny inputs in pure Python (no shared helper)."""

import math

import numpy as np
import torch

import oracle
from workloads import paged_prefill_case, randn_bf16


# ---------------------------------------------------------------- sliding window
def _decode_case(seed=90, ctx=(1, 2, 127, 128, 129, 300, 513)):
    return paged_prefill_case([1] * len(ctx), list(ctx), num_heads=8, num_kv_heads=2, head_dim=16, seed=seed,
                              spare_blocks=2)


def test_window_covering_the_context_is_plain_decode():
    case = _decode_case()
    ref_o, ref_l = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                                 case.scale)
    for w in (512, 600, 10 ** 6):
        o, l_ = oracle.sliding_window_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                                       case.scale, w)
        assert np.array_equal(o, ref_o) and np.array_equal(l_, ref_l)


def test_window_zero_returns_the_last_value_row():
    case = _decode_case(seed=91)
    o, l_ = oracle.sliding_window_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                                   case.scale, 0)
    cache = case.kv_cache.double().numpy()
    q = case.q.double().numpy()
    group = case.num_heads // case.num_kv_heads
    for b, length in enumerate(case.context_lens):
        t = int(length) - 1
        blk, off = int(case.block_tables[b, t // 128]), t % 128
        for h in range(case.num_heads):
            assert np.array_equal(o[b, h], cache[1, blk, off, h // group])
            dot = float(np.dot(q[b, h], cache[0, blk, off, h // group]))
            assert abs(l_[h, b] - case.scale * dot) < 1e-12


def _brute_window(case, window):
    q = case.q.double().numpy()
    kc = case.kv_cache.double().numpy()
    group = case.num_heads // case.num_kv_heads
    out = np.zeros(q.shape)
    lse = np.zeros((case.num_heads, q.shape[0]))
    for b in range(q.shape[0]):
        length = int(case.context_lens[b])
        for h in range(case.num_heads):
            logits, vals = [], []
            for t in range(length):
                if length - 1 - t > window:  # more than `window` tokens before the query
                    continue
                blk, off = int(case.block_tables[b, t // 128]), t % 128
                logits.append(case.scale * sum(q[b, h, d] * kc[0, blk, off, h // group, d]
                                               for d in range(q.shape[2])))
                vals.append(kc[1, blk, off, h // group])
            w = [math.exp(z) for z in logits]
            out[b, h] = sum(wi * vi for wi, vi in zip(w, vals)) / sum(w)
            lse[h, b] = math.log(sum(w))
    return out, lse


def test_window_brute_force_tiny():
    case = paged_prefill_case([1] * 4, [1, 40, 129, 200], num_heads=2, num_kv_heads=1, head_dim=4, seed=92,
                              spare_blocks=1)
    for window in (1, 5, 127, 128):
        o, l_ = oracle.sliding_window_decode_attention(case.q, case.kv_cache, case.block_tables,
                                                       case.context_lens, case.scale, window)
        ref_o, ref_l = _brute_window(case, window)
        assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l_, ref_l, atol=1e-12)


# ---------------------------------------------------------------- padded prefix
def _padded(seed, b=3, sq=40, sk=40, hq=4, hkv=2, d=16):
    q = randn_bf16((b, sq, hq, d), seed)
    k = randn_bf16((b, sk, hkv, d), seed + 1)
    v = randn_bf16((b, sk, hkv, d), seed + 2)
    return q, k, v


def test_padded_prefix_equals_packed_varlen():
    q, k, v = _padded(93, sq=40, sk=33)
    ql, kl = np.array([40, 7, 0]), np.array([33, 20, 5])
    for causal in (False, True):
        out, lse = oracle.padded_prefix_attention(q, k, v, ql, kl, 0.25, causal)
        qp = torch.cat([q[b, :ql[b]] for b in range(3)])
        kp = torch.cat([k[b, :kl[b]] for b in range(3)])
        vp = torch.cat([v[b, :kl[b]] for b in range(3)])
        cu_q, cu_k = np.concatenate([[0], np.cumsum(ql)]), np.concatenate([[0], np.cumsum(kl)])
        o2, l2 = oracle.varlen_attention(qp, kp, vp, cu_q, cu_k, 0.25, causal)
        for b in range(3):
            rows = slice(cu_q[b], cu_q[b + 1])
            assert np.allclose(out[b, :ql[b]], o2[rows], atol=1e-13)
            assert np.allclose(lse[:, b * 40:b * 40 + ql[b]], l2[:, rows], atol=1e-13)
            assert np.all(out[b, ql[b]:] == 0.0) and np.all(lse[:, b * 40 + ql[b]:(b + 1) * 40] == -np.inf)


def test_padded_full_lengths_are_dense():
    q, k, v = _padded(94)
    for causal in (False, True):
        out, lse = oracle.padded_prefix_attention(q, k, v, [40] * 3, [40] * 3, 0.3, causal)
        o2, l2 = oracle.dense_attention(q, k, v, 0.3, causal)
        assert np.allclose(out, o2, atol=1e-13)
        assert np.allclose(lse, l2.transpose(1, 0, 2).reshape(4, -1), atol=1e-13)


def test_padded_pad_rows_never_matter():
    q, k, v = _padded(95)
    ql, kl = [30, 12, 1], [25, 40, 3]
    out, lse = oracle.padded_prefix_attention(q, k, v, ql, kl, 0.3, True)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for b in range(3):
        q2[b, ql[b]:] = 1e4
        k2[b, kl[b]:] = -3e3
        v2[b, kl[b]:] = float("nan")
    o2, l2 = oracle.padded_prefix_attention(q2, k2, v2, ql, kl, 0.3, True)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_padded_brute_force_tiny():
    q, k, v = _padded(96, b=2, sq=5, sk=6, hq=2, hkv=1, d=3)
    ql, kl = [4, 2], [6, 3]
    out, lse = oracle.padded_prefix_attention(q, k, v, ql, kl, 0.5, True)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for b in range(2):
        for i in range(5):
            for h in range(2):
                if i >= ql[b]:
                    assert np.all(out[b, i, h] == 0.0) and lse[h, b * 5 + i] == -np.inf
                    continue
                w, acc = [], np.zeros(3)
                for j in range(kl[b]):
                    if j > i + kl[b] - ql[b]:
                        continue
                    w.append(math.exp(0.5 * sum(qd[b, i, h, d] * kd[b, j, 0, d] for d in range(3))))
                    acc = acc + w[-1] * vd[b, j, 0]
                if not w:
                    assert np.all(out[b, i, h] == 0.0) and lse[h, b * 5 + i] == -np.inf
                    continue
                assert np.allclose(out[b, i, h], acc / sum(w), atol=1e-12)
                assert abs(lse[h, b * 5 + i] - math.log(sum(w))) < 1e-12


# ---------------------------------------------------------------- key-padding mask
def test_all_ones_mask_is_dense():
    q, k, v = _padded(97)
    mask = np.ones((3, 40), dtype=np.uint8)
    for causal in (False, True):
        out, lse = oracle.masked_attention(q, k, v, mask, 0.3, causal, mask_queries=True)
        o2, l2 = oracle.dense_attention(q, k, v, 0.3, causal)
        assert np.allclose(out, o2, atol=1e-13)
        assert np.allclose(lse, l2.transpose(1, 0, 2).reshape(4, -1), atol=1e-13)


def test_prefix_mask_is_padded_prefix():
    q, k, v = _padded(98)
    lens = [40, 13, 0]
    mask = np.zeros((3, 40), dtype=np.uint8)
    for b, n in enumerate(lens):
        mask[b, :n] = 1
    for causal in (False, True):
        out, lse = oracle.masked_attention(q, k, v, mask, 0.3, causal, mask_queries=True)
        o2, l2 = oracle.padded_prefix_attention(q, k, v, lens, lens, 0.3, causal)
        assert np.allclose(out, o2, atol=1e-13) and np.allclose(lse, l2, atol=1e-13)


def test_cross_mask_is_varlen_with_uniform_queries():
    q, k, v = _padded(99, sq=24, sk=40)
    rng = np.random.default_rng(99)
    mask = (rng.random((3, 40)) < 0.6).astype(np.uint8)
    mask[2] = 0  # an entry with no real key: its rows come back as zeros
    out, lse = oracle.masked_attention(q, k, v, mask, 0.3, False, mask_queries=False)
    kp = torch.cat([k[b, torch.from_numpy(np.nonzero(mask[b])[0])] for b in range(3)])
    vp = torch.cat([v[b, torch.from_numpy(np.nonzero(mask[b])[0])] for b in range(3)])
    cu_k = np.concatenate([[0], np.cumsum(mask.sum(1))])
    o2, l2 = oracle.varlen_attention(q.reshape(72, 4, 16), kp, vp, [0, 24, 48, 72], cu_k, 0.3, False)
    assert np.allclose(out.reshape(72, 4, 16), o2, atol=1e-13) and np.allclose(lse, l2, atol=1e-13)
    assert np.all(out[2] == 0.0) and np.all(lse[:, 48:] == -np.inf)


def test_self_mask_with_holes_brute_force_tiny():
    q, k, v = _padded(100, b=2, sq=6, sk=6, hq=2, hkv=1, d=3)
    mask = np.array([[1, 0, 1, 1, 0, 1], [0, 0, 1, 0, 0, 0]], dtype=np.uint8)
    out, lse = oracle.masked_attention(q, k, v, mask, 0.5, True, mask_queries=True)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for b in range(2):
        real = [j for j in range(6) if mask[b, j]]
        for i in range(6):
            for h in range(2):
                if i not in real:
                    assert np.all(out[b, i, h] == 0.0) and lse[h, b * 6 + i] == -np.inf
                    continue
                w, acc = [], np.zeros(3)
                for j in real:
                    if j > i:  # equal lengths: bottom-right = top-left on the real tokens
                        continue
                    w.append(math.exp(0.5 * sum(qd[b, i, h, d] * kd[b, j, 0, d] for d in range(3))))
                    acc = acc + w[-1] * vd[b, j, 0]
                assert np.allclose(out[b, i, h], acc / sum(w), atol=1e-12)
                assert abs(lse[h, b * 6 + i] - math.log(sum(w))) < 1e-12


def test_masked_positions_never_matter():
    q, k, v = _padded(101)
    rng = np.random.default_rng(101)
    mask = (rng.random((3, 40)) < 0.7).astype(np.uint8)
    out, lse = oracle.masked_attention(q, k, v, mask, 0.3, True, mask_queries=True)
    drop = torch.from_numpy(mask == 0)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[drop] = 7e3
    k2[drop] = -5e3
    v2[drop] = float("inf")
    o2, l2 = oracle.masked_attention(q2, k2, v2, mask, 0.3, True, mask_queries=True)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
