"""GPU parity of attn_varlen_fwd against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import (LSE_TOL, OUT_TOL, announce, assert_close, dev, guard_intact, guarded_empty, host)
from workloads import config1, config2, config3, varlen_case

pytestmark = pytest.mark.gpu


def run_case(case, with_lse=True):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    cu_q, cu_k = dev(case.cu_seqlens_q), dev(case.cu_seqlens_k)
    res = sav.attn_varlen_fwd(q, k, v, cu_q, cu_k, case.max_seqlen_q, case.max_seqlen_k, case.scale, case.causal,
                              return_lse=with_lse)
    torch.cuda.synchronize()
    return res


def check_full(case, few_keys=False):
    announce("varlen", case.name, case.cu_seqlens_q.tolist()[:8], case.num_heads, case.num_kv_heads,
             case.head_dim, case.causal)
    out, lse = run_case(case)
    ref_o, ref_l = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                           case.causal)
    e_o = assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=few_keys)
    e_l = assert_close("lse", host(lse), ref_l, LSE_TOL)
    return e_o, e_l


def test_config1_tiny_full_parity():
    check_full(config1())


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
def test_sweep_ragged(d, causal, hq, hkv):
    # several 128-row query tiles and 64-key tiles, ragged tails, a 1-row doc
    lens = [1, 129, 300, 64, 190]
    case = varlen_case(lens, num_heads=hq, num_kv_heads=hkv, head_dim=d, causal=causal, seed=100 + d + hq + causal)
    check_full(case, few_keys=True)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_lengths_bottom_right(causal, d):
    # Lq != Lk per document, including Lq > Lk (rows with no key under causal)
    case = varlen_case([5, 200, 130, 70], [77, 150, 130, 1], num_heads=4, num_kv_heads=2, head_dim=d,
                       causal=causal, seed=41 + (d - 128))
    check_full(case, few_keys=True)


def test_empty_documents():
    case = varlen_case([0, 70, 0, 33], [0, 70, 5, 0], num_heads=2, num_kv_heads=2, head_dim=64, causal=False,
                       seed=42)
    check_full(case, few_keys=True)


@pytest.mark.parametrize("batch,d", [(511, 128), (512, 128), (700, 128), (300, 192), (300, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_many_documents(batch, causal, d):
    # hundreds of documents, most shorter than one 256-row query tile (many
    # empty workgroup slots), a few spanning several tiles, some empty
    rng = np.random.default_rng(batch + causal)
    lens = rng.integers(0, 96, batch)
    lens[rng.choice(batch, 5, replace=False)] = [257, 300, 513, 700, 1]
    lens[rng.choice(batch, 20, replace=False)] = 0
    case = varlen_case(lens.tolist(), num_heads=4, num_kv_heads=2, head_dim=d, causal=causal,
                       seed=44 + batch + (d - 128))
    check_full(case, few_keys=True)


def test_no_lse_and_determinism():
    case = varlen_case([300, 77], num_heads=4, num_kv_heads=2, head_dim=128, causal=True, seed=43)
    announce("varlen determinism")
    o1 = run_case(case, with_lse=False)
    o2 = run_case(case, with_lse=False)
    o3, l3 = run_case(case, with_lse=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_guard_canaries():
    case = varlen_case([130, 257], num_heads=4, num_kv_heads=4, head_dim=64, causal=False, seed=44)
    announce("varlen guards")
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    out, og = guarded_empty(q.shape, torch.bfloat16)
    lse, lg = guarded_empty((4, q.shape[0]), torch.float32)
    sav.attn_varlen_fwd(q, k, v, dev(case.cu_seqlens_q), dev(case.cu_seqlens_k), case.max_seqlen_q,
                        case.max_seqlen_k, case.scale, False, out=out, lse=lse)
    torch.cuda.synchronize()
    assert guard_intact(og) and guard_intact(lg)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_indexing_probe_bit_exact(causal, d):
    """K = 0 except one selected key per (doc, head) with a logit at least 512
    above the rest; every row that can see it must return that key's V
    bit-exactly, and V encodes (doc, token) and then the column index, so a
    wrong cu_seqlens offset or a misplaced 16-byte piece is visible. head_dims
    96 to 256 run the pipelined kernels (128-row items on split K/V rings;
    256-byte LDS rows at 96, padded, and 128; 512-byte rows at 192, padded,
    and 256)."""
    lens = [3, 129, 64, 250, 1, 385]
    hq = hkv = 3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = torch.full((T, hq, d), 8.0, dtype=torch.bfloat16)
    k = torch.zeros((T, hkv, d), dtype=torch.bfloat16)
    v = torch.zeros((T, hkv, d), dtype=torch.bfloat16)
    sel = {}
    for b, L in enumerate(lens):
        for h in range(hkv):
            j = [0, L - 1, L // 2][h]  # first, last, middle key of the document
            sel[(b, h)] = j
            k[cu[b] + j, h] = 8.0
        for t in range(L):
            v[cu[b] + t, :, 0] = b
            v[cu[b] + t, :, 1] = t % 128
            v[cu[b] + t, :, 2] = t // 128
            v[cu[b] + t, :, 3] = torch.arange(hkv)
            v[cu[b] + t, :, 4:] = (torch.arange(4, d) % 200).to(torch.bfloat16)
    announce("varlen probe", causal, d)
    out = sav.attn_varlen_fwd(dev(q), dev(k), dev(v), dev(cu), dev(cu), max(lens), max(lens), 0.125, causal)
    torch.cuda.synchronize()
    out = out.cpu()
    checked = 0
    for b, L in enumerate(lens):
        for h in range(hq):
            j = sel[(b, h)]
            for i in range(L):
                if causal and j > i:
                    continue
                assert torch.equal(out[cu[b] + i, h], v[cu[b] + j, h]), (b, h, i, j)
                checked += 1
    assert checked > 500


@pytest.mark.parametrize("seed", range(8))
def test_random_varlen_head_dim_128(seed):
    """Seeded random packings for the pipelined head_dim-128 kernels: 1-6
    documents of 1-700 query rows, key lengths equal or drawn separately
    (bottom-right causal then covers rows that see no key), grouped heads, causal
    or not, so ring wrap-around, partial tiles and diagonal positions vary."""
    rng = np.random.default_rng(7000 + seed)
    batch = int(rng.integers(1, 7))
    lq = rng.integers(1, 701, batch).tolist()
    lk = lq if rng.random() < 0.5 else rng.integers(1, 701, batch).tolist()
    group = int(rng.choice([1, 2, 4]))
    hkv = int(rng.integers(1, 3))
    causal = bool(rng.random() < 0.6)
    case = varlen_case(lq, lk, num_heads=hkv * group, num_kv_heads=hkv, head_dim=128, causal=causal,
                       seed=7000 + seed, name=f"random-{seed}")
    check_full(case, few_keys=True)


@pytest.mark.parametrize("d,causal", [(64, False), (96, False), (192, False), (256, False), (256, True)])
def test_head_dim_full_size_every_row(d, causal):
    """Head dims 64, 96, 192 and 256 on the shape their throughput is
    measured on (2 documents of 4096 rows, 24 heads, N(0,1) inputs), every row
    and head against the oracle: the pipelined kernel with padded LDS rows (64,
    96, 192), 512-byte rows (192, 256) and, at 192/256, its loads issued from
    inside the step."""
    case = varlen_case([4096, 4096], num_heads=24, num_kv_heads=24, head_dim=d, causal=causal, seed=7700 + d + causal,
                       name=f"dit-dense-b2-s4096-h24-d{d}" + ("-causal" if causal else ""))
    announce("varlen full-size", case.name)
    out, lse = run_case(case)
    ref_o, ref_l = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                           case.causal)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


@pytest.mark.parametrize("make", [config2, config3])
def test_full_size_config_every_row(make):
    """Configs 2 and 3 at full size, every row and head against the oracle."""
    case = make()
    announce("varlen full-size", case.name)
    out, lse = run_case(case)
    ref_o, ref_l = oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                           case.causal)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)
