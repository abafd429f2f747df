"""Pins for the VSA compressed-branch oracle: pure-Python brute force on tiny
inputs, uniform scores, a zero gate, and grouped heads = repeated heads."""

import math

import numpy as np

import oracle


def _inputs(rng, b=1, t=3, block=4, h=2, hkv=2, d=3):
    q = rng.standard_normal((b, t * block, h, d))
    k = rng.standard_normal((b, t * block, hkv, d))
    v = rng.standard_normal((b, t * block, hkv, d))
    sizes = np.array([block, block - 1, 2][:t])
    for c, sz in enumerate(sizes):  # padding rows are zero in tile order
        q[:, c * block + sz:(c + 1) * block] = 0
        k[:, c * block + sz:(c + 1) * block] = 0
        v[:, c * block + sz:(c + 1) * block] = 0
    gate = rng.standard_normal(q.shape)
    out = rng.standard_normal(q.shape)
    return q, k, v, sizes, gate, out


def test_brute_force_tiny():
    rng = np.random.default_rng(91)
    block = 4
    q, k, v, sizes, gate, out = _inputs(rng, block=block)
    scale = 0.7
    got, comp = oracle.compressed_branch(q, k, v, sizes, scale, gate, out, block=block)
    b_, seq, h_, d_ = q.shape
    t_ = seq // block

    def mean(x, bb, c, hh, dd):
        return sum(x[bb, c * block + r, hh, dd] for r in range(sizes[c])) / max(sizes[c], 1)

    for bb in range(b_):
        for hh in range(h_):
            for a in range(t_):
                sc = [scale * sum(mean(q, bb, a, hh, dd) * mean(k, bb, c, hh, dd) for dd in range(d_))
                      for c in range(t_)]
                e = [math.exp(x) for x in sc]
                tot = sum(e)
                cvec = [sum(e[c] / tot * mean(v, bb, c, hh, dd) for c in range(t_)) for dd in range(d_)]
                assert np.allclose(comp[bb, hh, a], cvec, atol=1e-12)
                for r in range(block):
                    row = a * block + r
                    want = [out[bb, row, hh, dd] + cvec[dd] * gate[bb, row, hh, dd] for dd in range(d_)]
                    assert np.allclose(got[bb, row, hh], want, atol=1e-12)


def test_uniform_scores_give_mean_of_value_means():
    rng = np.random.default_rng(92)
    q, k, v, sizes, gate, _ = _inputs(rng, t=3)
    q[:] = 0.0  # every pooled score is 0: a uniform softmax over the 3 key tiles
    _, comp = oracle.compressed_branch(q, k, v, sizes, 0.5, gate, block=4)
    vp = oracle.pool_tiles(v, sizes, 4)  # [B, H, T, D]
    assert np.allclose(comp, vp.mean(axis=2, keepdims=True).repeat(3, axis=2), atol=1e-14)


def test_zero_gate_leaves_output():
    rng = np.random.default_rng(93)
    q, k, v, sizes, gate, out = _inputs(rng)
    got, _ = oracle.compressed_branch(q, k, v, sizes, 0.5, np.zeros_like(gate), out, block=4)
    assert np.array_equal(got, out)


def test_grouped_heads_equal_repeated_heads():
    rng = np.random.default_rng(94)
    q, k, v, sizes, gate, out = _inputs(rng, h=4, hkv=2)
    got, comp = oracle.compressed_branch(q, k, v, sizes, 0.5, gate, out, block=4)
    k2, v2 = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)
    got2, comp2 = oracle.compressed_branch(q, k2, v2, sizes, 0.5, gate, out, block=4)
    assert np.allclose(got, got2, atol=1e-14) and np.allclose(comp, comp2, atol=1e-14)
