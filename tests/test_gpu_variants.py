"""GPU parity of the boundary variants against the fp64 oracle, through the C
ABI: sliding-window paged decode, attention over valid prefixes of a padded
batch, and key-padding-mask attention (self and cross)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, dev, host
from workloads import SLIDING_WINDOW, config8, config9, config10, padded_case, paged_prefill_case

pytestmark = pytest.mark.gpu

CTX = [1, 2, 31, 32, 33, 127, 128, 129, 500, 1000, 4097]


def check_window(case, window, seqs=None, few_keys=True):
    out, lse = sav.attn_paged_decode(dev(case.q), dev(case.kv_cache), dev(case.block_tables), dev(case.context_lens),
                                     int(case.context_lens.max()), case.scale, return_lse=True, window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sliding_window_decode_attention(case.q, case.kv_cache, case.block_tables,
                                                          case.context_lens, case.scale, window, seqs=seqs)
    if seqs is not None:
        s = torch.tensor(seqs).cuda()
        out, lse = out.index_select(0, s), lse.index_select(1, s)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=few_keys)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


@pytest.mark.parametrize("window", [0, 1, 31, 32, 33, 100, 127, 128, 1000, 4096, 5000])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8)])
def test_sliding_window_decode_d128(window, hq, hkv):
    case = paged_prefill_case([1] * len(CTX), CTX, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                              seed=500 + window % 97 + hq, spare_blocks=3)
    announce("swa decode d128", window, hq, hkv)
    check_window(case, window)


@pytest.mark.parametrize("d", [64, 96, 192, 256])
@pytest.mark.parametrize("window", [0, 33, 300])
def test_sliding_window_decode_other_dims(d, window):
    case = paged_prefill_case([1] * len(CTX), CTX, num_heads=16, num_kv_heads=4, head_dim=d, seed=520 + d + window,
                              spare_blocks=3)
    announce("swa decode", d, window)
    check_window(case, window)


def test_sliding_window_equals_plain_decode_when_it_covers_the_context():
    case = paged_prefill_case([1] * len(CTX), CTX, num_heads=8, num_kv_heads=2, head_dim=128, seed=530)
    announce("swa covers context")
    args = (dev(case.q), dev(case.kv_cache), dev(case.block_tables), dev(case.context_lens),
            int(case.context_lens.max()), case.scale)
    a, la = sav.attn_paged_decode(*args, return_lse=True)
    b, lb = sav.attn_paged_decode(*args, return_lse=True, window=int(case.context_lens.max()) - 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("d", [64, 96, 192, 256])
@pytest.mark.parametrize("ctx,window", [([8193, 5, 8000, 100], 8160), ([8193, 8193, 1, 4097], 8100),
                                        ([20000, 300, 16385, 9], 16000), ([700, 129, 640, 2], 600)])
def test_sliding_window_plan_fits_reported_workspace(d, ctx, window):
    """A windowed call gets exactly the workspace the size query reported for
    max_context_len, followed by a poisoned guard: the stream's prefix sums,
    window starts and partials stay inside it."""
    from tests._gpu_helpers import guard_intact, guarded_empty

    case = paged_prefill_case([1] * len(ctx), ctx, num_heads=32, num_kv_heads=8, head_dim=d, seed=540 + d,
                              spare_blocks=2)
    mcl = int(max(ctx))
    need = sav.attn_paged_decode_workspace_size(len(ctx), 32, 8, d, mcl)
    ws, guard = guarded_empty((need,), torch.uint8, guard=1 << 16, fill=171)
    announce("swa decode workspace", d, ctx, window, need)
    out, lse = sav.attn_paged_decode(dev(case.q), dev(case.kv_cache), dev(case.block_tables),
                                     dev(case.context_lens), mcl, case.scale, return_lse=True, window=window,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert guard_intact(guard, fill=171)
    ref_o, ref_l = oracle.sliding_window_decode_attention(case.q, case.kv_cache, case.block_tables,
                                                          case.context_lens, case.scale, window)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def test_sliding_window_decode_full_size_every_sequence():
    case = config8()
    announce("swa decode full size")
    check_window(case, SLIDING_WINDOW, few_keys=False)


def run_padded(case, with_lse=True):
    out, lse = sav.attn_padded_fwd(dev(case.q), dev(case.k), dev(case.v), dev(case.q_lens), dev(case.k_lens),
                                   case.scale, case.causal, return_lse=with_lse)
    torch.cuda.synchronize()
    return out, lse


PADDED = {
    "mixed": (3, 300, 260, [300, 17, 0], [260, 100, 5]),
    "one-row": (2, 64, 64, [1, 64], [64, 1]),
    "no-keys": (2, 70, 50, [70, 3], [0, 50]),
}


@pytest.mark.parametrize("name", list(PADDED))
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_prefix(name, d, causal):
    b, sq, sk, ql, kl = PADDED[name]
    case = padded_case(b, sq, sk, num_heads=8, num_kv_heads=2, head_dim=d, seed=540 + d, q_lens=ql, k_lens=kl,
                       causal=causal)
    announce("padded", name, d, causal)
    out, lse = run_padded(case)
    ref_o, ref_l = oracle.padded_prefix_attention(case.q, case.k, case.v, case.q_lens, case.k_lens, case.scale,
                                                  causal)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def test_padded_full_size():
    case = config10()
    announce("padded full size", case.q_lens.tolist())
    out, lse = run_padded(case)
    ref_o, ref_l = oracle.padded_prefix_attention(case.q, case.k, case.v, case.q_lens, case.k_lens, case.scale,
                                                  False)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def run_masked(case, mask_queries):
    out, lse = sav.attn_masked_fwd(dev(case.q), dev(case.k), dev(case.v), dev(case.key_mask), case.scale,
                                   case.causal, mask_queries=mask_queries, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def check_masked(case, mask_queries, few_keys=True):
    out, lse = run_masked(case, mask_queries)
    ref_o, ref_l = oracle.masked_attention(case.q, case.k, case.v, case.key_mask, case.scale, case.causal,
                                           mask_queries)
    assert_close("out", host(out), ref_o, OUT_TOL, bf16_output=True, few_keys=few_keys)
    assert_close("lse", host(lse), ref_l, LSE_TOL)


def _holes(b, s, p, seed):
    m = (np.random.default_rng(seed).random((b, s)) < p).astype(np.uint8)
    m[-1] = 0  # an entry with no real token
    return m


@pytest.mark.parametrize("d", [64, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])
def test_masked_self_with_holes(d, causal, hq, hkv):
    mask = _holes(3, 333, 0.7, 550 + d)
    case = padded_case(3, 333, 333, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=551 + d, key_mask=mask,
                       causal=causal)
    announce("masked self", d, causal, hq, hkv, mask.sum(1).tolist())
    check_masked(case, True)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_cross(d, causal):
    mask = _holes(3, 77, 0.5, 560 + d)
    case = padded_case(3, 300, 77, num_heads=8, num_kv_heads=4, head_dim=d, seed=561 + d, key_mask=mask,
                       causal=causal)
    announce("masked cross", d, causal, mask.sum(1).tolist())
    check_masked(case, False)


def test_masked_all_ones_equals_varlen_dense():
    case = padded_case(2, 500, 500, num_heads=8, num_kv_heads=8, head_dim=128, seed=570,
                       key_mask=np.ones((2, 500), dtype=np.uint8), causal=True)
    announce("masked all ones")
    out, lse = run_masked(case, True)
    cu = torch.tensor([0, 500, 1000], dtype=torch.int32)
    ref, lref = sav.attn_varlen_fwd(dev(case.q.reshape(1000, 8, 128)), dev(case.k.reshape(1000, 8, 128)),
                                    dev(case.v.reshape(1000, 8, 128)), dev(cu), dev(cu), 500, 500, case.scale, True,
                                    return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(1000, 8, 128), ref) and torch.equal(lse, lref)


def test_masked_cross_full_size():
    case = config9()
    announce("masked cross full size", case.k_lens.tolist())
    check_masked(case, False, few_keys=False)


def test_determinism():
    mask = _holes(2, 400, 0.6, 580)
    case = padded_case(2, 400, 400, num_heads=8, num_kv_heads=2, head_dim=128, seed=581, key_mask=mask, causal=True)
    a, la = run_masked(case, True)
    b, lb = run_masked(case, True)
    assert torch.equal(a, b) and torch.equal(la, lb)
