"""Pins for the fp64 varlen/dense oracle: closed forms, brute force, a library
SDPA in float64, and invariants that the definition fixes.

Each check is something other than the oracle restated: a hand-solved value, a
pure-Python loop without max subtraction, torch's own SDPA with an explicit
mask, or a relation between two different calls.
"""

import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from workloads import cumulative, varlen_case

RNG = np.random.default_rng(12345)


def _rand(shape, rng=RNG):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_closed_form_two_keys():
    # scores z = scale*q.k = [0, ln 3] -> weights [1/4, 3/4]; O = 1/4*2 + 3/4*6 = 5; LSE = ln 4
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[1.0]]])
    v = np.array([[[2.0]], [[6.0]]])
    out, lse = oracle.varlen_attention(q, k, v, [0, 1], [0, 2], scale=math.log(3.0), causal=False)
    assert out[0, 0, 0] == pytest.approx(5.0, abs=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(4.0), abs=1e-14)


def test_closed_form_scale_and_sign():
    # z = scale * q.k with q.k = [-2, 1], scale 0.5: z = [-1, 0.5]
    # w = e^{-1}, e^{0.5}; O = (e^-1 * 10 + e^0.5 * -4) / (e^-1 + e^0.5)
    q = np.array([[[1.0, 2.0]]])
    k = np.array([[[0.0, -1.0]], [[1.0, 0.0]]])
    v = np.array([[[10.0, 0.0]], [[-4.0, 1.0]]])
    out, lse = oracle.varlen_attention(q, k, v, [0, 1], [0, 2], scale=0.5, causal=False)
    a, b = math.exp(-1.0), math.exp(0.5)
    assert out[0, 0, 0] == pytest.approx((10 * a - 4 * b) / (a + b), abs=1e-13)
    assert out[0, 0, 1] == pytest.approx(b / (a + b), abs=1e-13)
    assert lse[0, 0] == pytest.approx(math.log(a + b), abs=1e-13)


def test_constant_v_gives_v():
    case = varlen_case([37, 64], num_heads=4, num_kv_heads=2, head_dim=16, causal=True, seed=11)
    v = np.broadcast_to(np.linspace(-3, 3, 16), (case.v.shape[0], 2, 16)).copy()
    out, _ = oracle.varlen_attention(case.q, case.k, v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale, True)
    assert np.max(np.abs(out - np.linspace(-3, 3, 16))) <= 1e-12


def test_single_key_gives_its_value():
    q, k, v = _rand((1, 3, 8)), _rand((1, 3, 8)), _rand((1, 3, 8))
    out, lse = oracle.varlen_attention(q, k, v, [0, 1], [0, 1], scale=0.3, causal=False)
    assert np.allclose(out[0], v[0], atol=1e-15)
    assert np.allclose(lse[:, 0], 0.3 * np.einsum("hd,hd->h", q[0], k[0]), atol=1e-14)


def test_causal_row0_attends_only_itself():
    case = varlen_case([5, 9, 1], num_heads=2, num_kv_heads=1, head_dim=8, causal=True, seed=12)
    out, lse = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.scale, True)
    qf, kf, vf = (x.double().numpy() for x in (case.q, case.k, case.v))
    for b in range(case.batch):
        r = case.cu_seqlens_q[b]
        for h in range(2):
            assert np.allclose(out[r, h], vf[r, 0], atol=1e-14)
            assert lse[h, r] == pytest.approx(case.scale * qf[r, h] @ kf[r, 0], abs=1e-13)


def test_lse_bounds_and_convex_hull():
    case = varlen_case([23, 40], num_heads=3, num_kv_heads=3, head_dim=32, causal=False, seed=13)
    out, lse = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.scale, False)
    qf, kf, vf = (x.double().numpy() for x in (case.q, case.k, case.v))
    for b in range(2):
        q0, q1 = case.cu_seqlens_q[b:b + 2]
        for h in range(3):
            z = case.scale * qf[q0:q1, h] @ kf[q0:q1, h].T
            zmax = z.max(axis=1)
            n = q1 - q0
            assert np.all(lse[h, q0:q1] >= zmax - 1e-12)
            assert np.all(lse[h, q0:q1] <= zmax + math.log(n) + 1e-12)
            lo, hi = vf[q0:q1, h].min(axis=0), vf[q0:q1, h].max(axis=0)
            assert np.all(out[q0:q1, h] >= lo - 1e-12) and np.all(out[q0:q1, h] <= hi + 1e-12)


def test_fully_masked_row_reading():
    # bottom-right causal with Lq > Lk leaves the first Lq-Lk rows with no key
    q, k, v = _rand((5, 1, 4)), _rand((2, 1, 4)), _rand((2, 1, 4))
    out, lse = oracle.varlen_attention(q, k, v, [0, 5], [0, 2], scale=0.5, causal=True)
    assert np.all(out[:3] == 0.0) and np.all(np.isneginf(lse[0, :3]))
    assert np.all(np.isfinite(lse[0, 3:]))


# --------------------------------------------------------------------------
# brute force (pure-Python loops, no max subtraction) and torch SDPA in fp64
# --------------------------------------------------------------------------

def brute_force_varlen(q, k, v, cu_q, cu_k, scale, causal):
    tq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((tq, hq, v.shape[2]))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for h in range(hq):
            hk = h * hkv // hq
            for i in range(lq):
                num = [0.0] * v.shape[2]
                den = 0.0
                for j in range(lk):
                    if causal and j > i + lk - lq:
                        continue
                    s = 0.0
                    for c in range(d):
                        s += float(q[cu_q[b] + i, h, c]) * float(k[cu_k[b] + j, hk, c])
                    w = math.exp(scale * s)
                    den += w
                    for c in range(v.shape[2]):
                        num[c] += w * float(v[cu_k[b] + j, hk, c])
                if den > 0:
                    out[cu_q[b] + i, h] = [x / den for x in num]
                    lse[h, cu_q[b] + i] = math.log(den)
    return out, lse


@settings(max_examples=40, deadline=None)
@given(
    lens=st.lists(st.tuples(st.integers(0, 7), st.integers(0, 9)), min_size=1, max_size=3),
    group=st.sampled_from([1, 2, 3]),
    hkv=st.sampled_from([1, 2]),
    d=st.integers(1, 8),
    causal=st.booleans(),
    seed=st.integers(0, 2**31 - 1),
)
def test_brute_force_tiny(lens, group, hkv, d, causal, seed):
    rng = np.random.default_rng(seed)
    lq = [a for a, _ in lens]
    lk = [b for _, b in lens]
    cu_q, cu_k = cumulative(lq), cumulative(lk)
    hq = hkv * group
    q = rng.standard_normal((cu_q[-1], hq, d))
    k = rng.standard_normal((cu_k[-1], hkv, d))
    v = rng.standard_normal((cu_k[-1], hkv, d + 1))
    scale = float(rng.uniform(0.1, 1.0))
    out, lse = oracle.varlen_attention(q, k, v, cu_q, cu_k, scale, causal)
    ref_o, ref_l = brute_force_varlen(q, k, v, cu_q, cu_k, scale, causal)
    assert np.allclose(out, ref_o, atol=1e-12, rtol=1e-12)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], ref_l[fin], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa_fp64(causal):
    case = varlen_case([17, 64, 33], [17, 80, 33], num_heads=4, num_kv_heads=2, head_dim=24, causal=causal,
                       seed=14)
    out, lse = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.scale, causal)
    qd, kd, vd = (x.double() for x in (case.q, case.k, case.v))
    for b in range(case.batch):
        q0, q1 = case.cu_seqlens_q[b:b + 2]
        k0, k1 = case.cu_seqlens_k[b:b + 2]
        lq, lk = q1 - q0, k1 - k0
        mask = torch.ones(lq, lk, dtype=torch.bool)
        if causal:
            mask = torch.arange(lk)[None, :] <= torch.arange(lq)[:, None] + (lk - lq)
        qq = qd[q0:q1].transpose(0, 1)
        kk = kd[k0:k1].repeat_interleave(2, dim=1).transpose(0, 1)
        vv = vd[k0:k1].repeat_interleave(2, dim=1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=case.scale)
        assert np.allclose(out[q0:q1], ref.transpose(0, 1).numpy(), atol=1e-12)
        # LSE through torch.logsumexp of the explicitly masked scores
        z = case.scale * qq @ kk.transpose(-1, -2)
        z = z.masked_fill(~mask, float("-inf"))
        assert np.allclose(lse[:, q0:q1], torch.logsumexp(z, dim=-1).numpy(), atol=1e-12)


# --------------------------------------------------------------------------
# invariants between different calls
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_per_document_runs_and_ignores_other_docs(causal):
    case = varlen_case([31, 70, 5, 64], num_heads=4, num_kv_heads=2, head_dim=16, causal=causal, seed=15)
    out, lse = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.scale, causal)
    for b in range(case.batch):
        q0, q1 = case.cu_seqlens_q[b:b + 2]
        # poison every other document's K/V with huge values
        k = case.k.double().clone()
        v = case.v.double().clone()
        poison = torch.ones(k.shape[0], dtype=torch.bool)
        poison[q0:q1] = False
        k[poison] = 1e4
        v[poison] = -1e4
        o_b, l_b = oracle.varlen_attention(case.q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                           causal, rows=np.arange(q0, q1))
        assert np.allclose(o_b, out[q0:q1], atol=1e-12) and np.allclose(l_b, lse[:, q0:q1], atol=1e-12)
        # and a single-document call on the slice
        o_s, l_s = oracle.varlen_attention(case.q[q0:q1], case.k[q0:q1], case.v[q0:q1], [0, q1 - q0],
                                           [0, q1 - q0], case.scale, causal)
        assert np.allclose(o_s, out[q0:q1], atol=1e-12) and np.allclose(l_s, lse[:, q0:q1], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_equals_uniform_varlen(causal):
    bsz, s, h, d = 3, 19, 4, 8
    q, k, v = _rand((bsz, s, h, d)), _rand((bsz, s, 2, d)), _rand((bsz, s, 2, d))
    od, ld = oracle.dense_attention(q, k, v, 0.4, causal)
    cu = np.arange(0, (bsz + 1) * s, s)  # the page's arange-built cu_seqlens
    ov, lv = oracle.varlen_attention(q.reshape(-1, h, d), k.reshape(-1, 2, d), v.reshape(-1, 2, d), cu, cu, 0.4,
                                     causal)
    assert np.allclose(ov.reshape(bsz, s, h, d), od, atol=1e-13)
    assert np.allclose(lv.reshape(h, bsz, s).transpose(1, 0, 2), ld, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    case = varlen_case([40, 25], num_heads=6, num_kv_heads=2, head_dim=16, causal=True, seed=16)
    o_g, l_g = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.scale, True)
    k_rep = case.k.repeat_interleave(3, dim=1)
    v_rep = case.v.repeat_interleave(3, dim=1)
    o_m, l_m = oracle.varlen_attention(case.q, k_rep, v_rep, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                       True)
    assert np.allclose(o_g, o_m, atol=1e-14) and np.allclose(l_g, l_m, atol=1e-14)
    # and query head h really uses kv head h // 3, not h % 2
    k_bad = case.k.index_select(1, torch.tensor([0, 1, 0, 1, 0, 1]))
    v_bad = case.v.index_select(1, torch.tensor([0, 1, 0, 1, 0, 1]))
    o_b, _ = oracle.varlen_attention(case.q, k_bad, v_bad, case.cu_seqlens_q, case.cu_seqlens_k, case.scale, True)
    assert not np.allclose(o_g, o_b, atol=1e-3)


def test_split_merge_identity():
    q, k, v = _rand((12, 2, 8)), _rand((50, 2, 8)), _rand((50, 2, 8))
    full_o, full_l = oracle.varlen_attention(q, k, v, [0, 12], [0, 50], 0.35, False)
    parts = [(0, 7), (7, 30), (30, 30), (30, 50)]  # includes an empty part
    outs, lses = [], []
    for a, b in parts:
        o, l_ = oracle.varlen_attention(q, k[a:b], v[a:b], [0, 12], [0, b - a], 0.35, False)
        outs.append(o)
        lses.append(l_.T)
    mo, ml = oracle.merge_partials(outs, lses)
    assert np.allclose(mo, full_o, atol=1e-13) and np.allclose(ml.T, full_l, atol=1e-13)


@pytest.mark.parametrize("c", [2.0, 4.0])
def test_power_of_two_prescale_identity(c):
    # [FA] prefix-kv slice note: q,k,v / c, scale * c^2, output * c is the same attention
    case = varlen_case([33, 20], num_heads=2, num_kv_heads=2, head_dim=16, causal=True, seed=17)
    o, l_ = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                    True)
    qd, kd, vd = (x.double() / c for x in (case.q, case.k, case.v))
    o2, l2 = oracle.varlen_attention(qd, kd, vd, case.cu_seqlens_q, case.cu_seqlens_k, case.scale * c * c, True)
    assert np.allclose(o2 * c, o, atol=1e-13) and np.allclose(l2, l_, atol=1e-13)


def test_suffix_padding_slice_equals_mask():
    # [FA] prefix-kv slice note: a strict-suffix padding document dropped from K/V
    # gives the same rows as masking it out
    real, total = 45, 64
    q, k, v = _rand((total, 2, 8)), _rand((total, 2, 8)), _rand((total, 2, 8))
    o_slice, _ = oracle.varlen_attention(q[:real], k[:real], v[:real], [0, real], [0, real], 0.3, False)
    o_pack, _ = oracle.varlen_attention(q, k, v, [0, real, total], [0, real, total], 0.3, False)
    qt, kt, vt = (torch.from_numpy(x).transpose(0, 1) for x in (q, k, v))
    keep = torch.zeros(total, total, dtype=torch.bool)
    keep[:, :real] = True
    o_mask = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=keep, scale=0.3)
    assert np.allclose(o_slice, o_pack[:real], atol=1e-13)
    assert np.allclose(o_slice, o_mask.transpose(0, 1).numpy()[:real], atol=1e-12)


def test_key_permutation_invariance_noncausal():
    q, k, v = _rand((9, 2, 8)), _rand((30, 2, 8)), _rand((30, 2, 8))
    perm = RNG.permutation(30)
    o1, l1 = oracle.varlen_attention(q, k, v, [0, 9], [0, 30], 0.5, False)
    o2, l2 = oracle.varlen_attention(q, k[perm], v[perm], [0, 9], [0, 30], 0.5, False)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_rows_subset_matches_full():
    case = varlen_case([50, 77], num_heads=4, num_kv_heads=1, head_dim=16, causal=True, seed=18)
    o, l_ = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale, True)
    rows = np.array([126, 0, 49, 50, 90])
    o2, l2 = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                     True, rows=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(l2, l_[:, rows])
