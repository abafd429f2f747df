"""GPU parity of attn_paged_decode against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, dev, guard_intact, guarded_empty, host
from workloads import config4, paged_case

pytestmark = pytest.mark.gpu


def run_case(case, with_lse=True, max_context_len=None):
    mcl = case.max_context_len if max_context_len is None else max_context_len
    res = sav.attn_paged_decode(dev(case.q), dev(case.kv_cache), dev(case.block_tables), dev(case.context_lens),
                                mcl, case.scale, return_lse=with_lse)
    torch.cuda.synchronize()
    return res


def check(case, seqs=None, few_keys=False):
    announce("paged", case.name, case.context_lens.tolist()[:10], case.num_heads, case.num_kv_heads, case.head_dim)
    out, lse = run_case(case)
    ref_o, ref_l = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                                 case.scale, seqs=seqs)
    if seqs is not None:
        s = torch.from_numpy(np.asarray(seqs)).cuda()
        out, lse = out.index_select(0, s), lse.index_select(1, s)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=few_keys)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


CTX_EDGE = [1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 1000, 4097]


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (16, 1), (40, 2)])
def test_sweep_edges(d, hq, hkv):
    case = paged_case(CTX_EDGE, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=200 + d + hq, spare_blocks=5,
                      max_blocks_per_seq=40, name=f"edges-d{d}-h{hq}kv{hkv}")
    check(case, few_keys=True)


def test_long_contexts_many_splits():
    ctx = [20000, 1, 32768, 9000, 128 * 70 + 5, 3]
    case = paged_case(ctx, num_heads=32, num_kv_heads=8, head_dim=128, seed=210, spare_blocks=2,
                      name="long-contexts")
    check(case, few_keys=True)


def test_zero_context_gives_zero_and_neg_inf():
    case = paged_case([0, 5, 0], num_heads=4, num_kv_heads=2, head_dim=64, seed=211, spare_blocks=1,
                      max_blocks_per_seq=2, name="zero-ctx")
    check(case, few_keys=True)


# head_dim 128 streams equal segments of the concatenated token stream (at
# least 256 positions each), so a segment can hold many sequences, start or end
# exactly on a sequence boundary, start inside a 32-token chunk, or cover one
# long sequence among many others
STREAM_CASES = {
    "zeros-between": [0, 5, 0, 300, 0, 0, 1, 0],
    "aligned-32s": [32] * 100,
    "ones-then-long": [1] * 50 + [257, 0, 513],
    "odd-mix": [7, 250, 3, 1000, 0, 33, 31, 129, 2, 600],
    "one-long": [40000],
}


@pytest.mark.parametrize("name", list(STREAM_CASES))
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 1), (40, 2)])
def test_stream_segments_d128(name, hq, hkv):
    ctx = STREAM_CASES[name]
    case = paged_case(ctx, num_heads=hq, num_kv_heads=hkv, head_dim=128, seed=230 + len(ctx) + hq, spare_blocks=3,
                      name=f"stream-{name}-h{hq}kv{hkv}")
    check(case, few_keys=True)


def test_host_max_context_len_larger_than_needed():
    # a generous host bound only changes the split plan, not the result
    case = paged_case([300, 2000, 17], num_heads=8, num_kv_heads=2, head_dim=128, seed=212, max_blocks_per_seq=64,
                      name="loose-bound")
    o1, l1 = run_case(case)
    o2, l2 = run_case(case, max_context_len=64 * 128)
    ref_o, ref_l = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens,
                                                 case.scale)
    assert_close("out", host(o2), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(l2), ref_l, LSE_TOL)
    assert_close("out-vs-tight", host(o1), host(o2), OUT_TOL)


def test_determinism_and_guards():
    case = paged_case([5000, 130, 20000], num_heads=32, num_kv_heads=8, head_dim=128, seed=213, name="det")
    announce("paged determinism")
    q, kv = dev(case.q), dev(case.kv_cache)
    bt, cl = dev(case.block_tables), dev(case.context_lens)
    outs = []
    for _ in range(2):
        out, og = guarded_empty(q.shape, torch.bfloat16)
        lse, lg = guarded_empty((32, 3), torch.float32)
        sav.attn_paged_decode(q, kv, bt, cl, case.max_context_len, case.scale, out=out, lse=lse)
        torch.cuda.synchronize()
        assert guard_intact(og) and guard_intact(lg)
        outs.append(out.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_block_table_probe_bit_exact():
    """K = 0 except one selected token per (sequence, kv head) whose logit is 512
    above the rest; V encodes (physical block, slot, kv head) as small integers.
    Every query head must return the selected token's V bit-exactly. Unused
    blocks and table tails (-1) are poisoned so any stray read shows up."""
    ctx = [1, 128, 129, 300, 777, 2048, 4100]
    hq, hkv, d = 8, 4, 64
    case = paged_case(ctx, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=214, spare_blocks=6,
                      max_blocks_per_seq=40, name="probe")
    kv = torch.zeros_like(case.kv_cache)
    nb = case.num_blocks
    # V plane: (block, slot, head) code everywhere; poisoned K in every block (cleared below for live tokens)
    kv[1, :, :, :, 0] = (torch.arange(nb) % 256).view(nb, 1, 1).to(torch.bfloat16)
    kv[1, :, :, :, 1] = (torch.arange(nb) // 256).view(nb, 1, 1).to(torch.bfloat16)
    kv[1, :, :, :, 2] = torch.arange(128).view(1, 128, 1).to(torch.bfloat16)
    kv[1, :, :, :, 3] = torch.arange(hkv).view(1, 1, hkv).to(torch.bfloat16)
    kv[0] = 8.0  # poison: a stray read of any non-live slot competes with the selected key
    sel = {}
    for b, L in enumerate(ctx):
        n = -(-L // 128)
        for t in range(L):  # live tokens: K = 0
            kv[0, case.block_tables[b, t // 128], t % 128] = 0.0
        for h in range(hkv):
            t = [L - 1, 0, L // 2, min(L - 1, 128)][h]
            sel[(b, h)] = t
            kv[0, case.block_tables[b, t // 128], t % 128, h] = 8.0
        assert np.all(case.block_tables[b, n:] == -1)
    q = torch.full_like(case.q, 8.0)
    announce("paged probe")
    out = sav.attn_paged_decode(dev(q), dev(kv), dev(case.block_tables), dev(case.context_lens), max(ctx), 0.125)
    torch.cuda.synchronize()
    out = out.cpu()
    for b, L in enumerate(ctx):
        for h in range(hq):
            hk = h // (hq // hkv)
            t = sel[(b, hk)]
            expect = kv[1, case.block_tables[b, t // 128], t % 128, hk]
            assert torch.equal(out[b, h], expect), (b, h, t)


def test_config4_full_size_every_sequence():
    check(config4())
