"""GPU parity of attn_paged_kv_write (bit-exact) and attn_paged_prefill against
the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, dev, host
from workloads import paged_prefill_case, randn_bf16

pytestmark = pytest.mark.gpu


def run_prefill(case, q=None, with_lse=True):
    q = case.q if q is None else q
    res = sav.attn_paged_prefill(dev(q), dev(case.kv_cache), dev(case.block_tables), dev(case.cu_seqlens_q),
                                 dev(case.context_lens), case.max_seqlen_q, case.max_context_len, case.scale,
                                 return_lse=with_lse)
    torch.cuda.synchronize()
    return res


def check(case, rows=None, few_keys=True):
    announce("paged prefill", case.name, np.diff(case.cu_seqlens_q).tolist()[:8], case.context_lens.tolist()[:8],
             case.num_heads, case.num_kv_heads, case.head_dim)
    out, lse = run_prefill(case)
    ref_o, ref_l = oracle.paged_prefill_attention(case.q, case.kv_cache, case.block_tables, case.cu_seqlens_q,
                                                  case.context_lens, case.scale, rows=rows)
    if rows is not None:
        r = torch.from_numpy(np.asarray(rows)).cuda()
        out, lse = out.index_select(0, r), lse.index_select(1, r)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=few_keys)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def test_kv_write_bit_exact():
    rng = np.random.default_rng(71)
    nb, hkv, d, n = 9, 2, 128, 700
    cache = torch.randn((2, nb, 128, hkv, d), generator=torch.Generator().manual_seed(71)).to(torch.bfloat16)
    slots = rng.choice(nb * 128, n, replace=False).astype(np.int32)
    slots[[0, 13, 699]] = -1                  # padding tokens
    slots[[50]] = nb * 128 + 5                 # out of range: skipped as well
    k, v = randn_bf16((n, hkv, d), 72), randn_bf16((n, hkv, d), 73)
    announce("kv write", n, nb)
    got = sav.attn_paged_kv_write(dev(k), dev(v), dev(slots), dev(cache))
    torch.cuda.synchronize()
    ref_slots = slots.copy()
    ref_slots[50] = -1
    ref = oracle.paged_kv_write(cache, k, v, ref_slots)
    assert torch.equal(got.cpu(), ref)


PREFILL_CASES = {
    # chunked prefill / cache hit: several new tokens over longer contexts
    "chunked": ([5, 64, 1, 130, 17, 300], [5, 300, 129, 513, 40, 300]),
    # speculative decoding: up to 16 new tokens per sequence
    "spec": ([4, 4, 2, 16, 1, 8], [1000, 129, 64, 4097, 3, 256]),
    # fewer keys than queries: early queries see no key (O = 0, LSE = -inf)
    "short-ctx": ([9, 3], [4, 0]),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8)])
def test_paged_prefill_sweep(name, d, hq, hkv):
    ql, ctx = PREFILL_CASES[name]
    case = paged_prefill_case(ql, ctx, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=400 + d + hq + len(ql),
                              spare_blocks=3, name=f"{name}-d{d}-h{hq}kv{hkv}")
    check(case)


def test_write_then_attend():
    # store the new tokens with the write entry point, then attend over them
    rng = np.random.default_rng(75)
    ql, ctx = [7, 130, 1], [300, 130, 513]
    case = paged_prefill_case(ql, ctx, num_heads=8, num_kv_heads=2, head_dim=128, seed=75, spare_blocks=2)
    n = int(sum(ql))
    k_new, v_new = randn_bf16((n, 2, 128), 76), randn_bf16((n, 2, 128), 77)
    slots = []
    for b, (lq, lk) in enumerate(zip(ql, ctx)):
        for t in range(lk - lq, lk):  # the new tokens are the last lq positions
            slots.append(int(case.block_tables[b, t // 128]) * 128 + t % 128)
    slots = np.asarray(slots, dtype=np.int32)
    announce("write then attend", ql, ctx)
    cache_d = dev(case.kv_cache)
    sav.attn_paged_kv_write(dev(k_new), dev(v_new), dev(slots), cache_d)
    out, lse = sav.attn_paged_prefill(dev(case.q), cache_d, dev(case.block_tables), dev(case.cu_seqlens_q),
                                      dev(case.context_lens), case.max_seqlen_q, case.max_context_len, case.scale,
                                      return_lse=True)
    torch.cuda.synchronize()
    cache_ref = oracle.paged_kv_write(case.kv_cache, k_new, v_new, slots)
    assert torch.equal(cache_d.cpu(), cache_ref)
    ref_o, ref_l = oracle.paged_prefill_attention(case.q, cache_ref, case.block_tables, case.cu_seqlens_q,
                                                  case.context_lens, case.scale)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def test_single_token_rows_match_decode_entry_point():
    # Lq = 1 per sequence is the decode case: both entry points agree to fp32 rounding
    case = paged_prefill_case([1] * 5, [1, 127, 128, 129, 1000], num_heads=32, num_kv_heads=8, head_dim=128,
                              seed=78, spare_blocks=1)
    announce("paged prefill vs decode")
    out_p, lse_p = run_prefill(case)
    out_d, lse_d = sav.attn_paged_decode(dev(case.q), dev(case.kv_cache), dev(case.block_tables),
                                         dev(case.context_lens), case.max_context_len, case.scale, return_lse=True)
    torch.cuda.synchronize()
    assert (out_p.float() - out_d.float()).abs().max().item() <= 2 * 2.0 ** -8
    assert (lse_p - lse_d).abs().max().item() <= 1e-4


def test_determinism():
    case = paged_prefill_case([33, 250], [400, 260], num_heads=8, num_kv_heads=2, head_dim=128, seed=79)
    a, la = run_prefill(case)
    b, lb = run_prefill(case)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_chunked_prefill_full_size_every_row():
    # workload 6: 16 sequences, 256..1024 new tokens over 2k..16k contexts, 32/8 heads, D=128
    from workloads import config6

    check(config6(), few_keys=False)


def test_spec_decode_full_size_every_row():
    # workload 7: the decode workload's 64 contexts (1k..32k) with 4 new tokens
    # each: the streaming path, (token, head) columns, segments crossing sequences
    from workloads import config7

    check(config7(), few_keys=False)
