"""attn_paged_decode_scratch, the decode entry point that allocates nothing
(its prefix sums and partials live in the library's fixed per-GPU device array), against
attn_paged_decode with a caller workspace, through the C ABI: two calls in a
row on the same array, the second with a smaller input, each also against the
fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, dev, host
from workloads import paged_case

pytestmark = pytest.mark.gpu


def _cases(d):
    rng = np.random.default_rng(900 + d)
    big = rng.integers(1, 6001, 48).tolist() + [8192, 1, 129]
    small = rng.integers(1, 700, 5).tolist()
    return [paged_case(big, num_heads=32, num_kv_heads=8, head_dim=d, seed=901 + d, spare_blocks=3,
                       name=f"scratch-big-d{d}"),
            paged_case(small, num_heads=32, num_kv_heads=8, head_dim=d, seed=902 + d, spare_blocks=1,
                       name=f"scratch-small-d{d}")]


@pytest.mark.parametrize("d", [128, 64, 256, 192, 96])
def test_scratch_decode_matches_workspace_decode(d):
    for case in _cases(d):
        announce("decode scratch", case.name, case.num_seqs, case.max_context_len)
        args = (dev(case.q), dev(case.kv_cache), dev(case.block_tables), dev(case.context_lens),
                case.max_context_len, case.scale)
        ref_o, ref_l = sav.attn_paged_decode(*args, return_lse=True)
        out, lse = sav.attn_paged_decode_scratch(*args, return_lse=True)
        torch.cuda.synchronize()
        # same plan, same kernels: identical bits
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse, ref_l)
        exact_o, exact_l = oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables,
                                                         case.context_lens, case.scale)
        assert_close("out", host(out), exact_o, OUT_TOL, bf16_output=True, few_keys=True)
        assert_close("lse", host(lse), exact_l, LSE_TOL)
