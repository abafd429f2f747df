"""Graph capture: every entry point family recorded into a torch CUDA (HIP)
graph and replayed several times, with other eager work on the device between
replays, gives the eager result bit for bit on every replay. Outputs and
workspaces are allocated before capture; nothing in the captured calls
allocates or synchronises."""

import numpy as np
import pytest
import torch

import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import announce, dev
from workloads import paged_prefill_case, padded_case, randn_bf16, varlen_case

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first call outside the graph (library load, lazy module init)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_matches(g, outputs, expected, reset=None, other=None, times=3):
    for i in range(times):
        for o in outputs:
            o.fill_(0)  # a fill kernel, so a replay that skips a write is caught
        if reset is not None:
            reset()
        g.replay()
        if other is not None:
            other()  # unrelated eager work between replays
        torch.cuda.synchronize()
        for o, e in zip(outputs, expected):
            assert torch.equal(o, e), f"replay {i} differs"


def _other_work():
    a = torch.randn(1024, 1024, device="cuda")
    (a @ a).sum().item()


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_graph(d):
    case = varlen_case([300, 17, 700], num_heads=8, num_kv_heads=2, head_dim=d, causal=True, seed=600 + d)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    cu_q, cu_k = dev(case.cu_seqlens_q), dev(case.cu_seqlens_k)
    out = torch.empty_like(q)
    lse = torch.empty((8, q.shape[0]), dtype=torch.float32, device="cuda")
    fn = lambda: sav.attn_varlen_fwd(q, k, v, cu_q, cu_k, case.max_seqlen_q, case.max_seqlen_k, case.scale, True,  # noqa: E731
                                     out=out, lse=lse)
    announce("graph varlen", d)
    fn()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g = capture(fn)
    replay_matches(g, [out, lse], ref, other=_other_work)


@pytest.mark.parametrize("d,window", [(128, None), (128, 100), (64, None), (256, 33)])
def test_paged_decode_graph(d, window):
    case = paged_prefill_case([1] * 6, [1, 200, 129, 1000, 4097, 64], num_heads=16, num_kv_heads=4, head_dim=d,
                              seed=610 + d, spare_blocks=2)
    q, kv, bt, cl = dev(case.q), dev(case.kv_cache), dev(case.block_tables), dev(case.context_lens)
    mx = int(case.context_lens.max())
    out = torch.empty_like(q)
    lse = torch.empty((16, 6), dtype=torch.float32, device="cuda")
    ws = torch.empty(sav.attn_paged_decode_workspace_size(6, 16, 4, d, mx), dtype=torch.uint8, device="cuda")
    fn = lambda: sav.attn_paged_decode(q, kv, bt, cl, mx, case.scale, out=out, lse=lse, workspace=ws,  # noqa: E731
                                       window=window)
    announce("graph decode", d, window)
    fn()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g = capture(fn)
    replay_matches(g, [out, lse], ref, other=_other_work)


def test_paged_prefill_and_kv_write_graph():
    case = paged_prefill_case([4, 3, 16, 1], [300, 129, 2000, 64], num_heads=16, num_kv_heads=4, head_dim=128,
                              seed=620, spare_blocks=2)
    q, bt, cu, cl = dev(case.q), dev(case.block_tables), dev(case.cu_seqlens_q), dev(case.context_lens)
    base_cache = dev(case.kv_cache)
    kv = base_cache.clone()
    n = int(case.q.shape[0])
    k_new, v_new = dev(randn_bf16((n, 4, 128), 621)), dev(randn_bf16((n, 4, 128), 622))
    lq = np.diff(case.cu_seqlens_q)
    slots = np.concatenate([case.block_tables[b, t // 128].astype(np.int64) * 128 + t % 128
                            for b in range(4) for t in [np.arange(case.context_lens[b] - lq[b], case.context_lens[b])]])
    sl = dev(slots.astype(np.int32))
    out = torch.empty_like(q)
    lse = torch.empty((16, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(sav.attn_paged_prefill_workspace_size(4, 16, 4, 128, 16, 2000), dtype=torch.uint8,
                     device="cuda")

    def fn():
        sav.attn_paged_kv_write(k_new, v_new, sl, kv)
        sav.attn_paged_prefill(q, kv, bt, cu, cl, 16, 2000, case.scale, out=out, lse=lse, workspace=ws)

    announce("graph paged prefill")
    fn()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), kv.clone())
    g = capture(fn)
    replay_matches(g, [out, lse], ref[:2], reset=lambda: kv.copy_(base_cache), other=_other_work)
    assert torch.equal(kv, ref[2])


def test_block_sparse_and_vsa_graph():
    shape, tile = (5, 7, 9), (4, 4, 4)
    n = int(np.prod(shape))
    q, k, v = (dev(randn_bf16((1, n, 4, 128), 630 + j)) for j in range(3))
    prep = sav.vsa_prepare(q, k, v, shape, tile, 5, 128 ** -0.5)
    qt, kt, vt, sizes = prep["q"], prep["k"], prep["v"], prep["tile_sizes"]
    nt = sizes.numel()
    bmap = torch.empty((1, 4, nt, nt), dtype=torch.uint8, device="cuda")
    mws = torch.empty(sav.attn_vsa_block_map_workspace_size(1, 4, 4, nt, 128), dtype=torch.uint8, device="cuda")
    sws = torch.empty(sav.attn_block_sparse_workspace_size(1, 4, nt), dtype=torch.uint8, device="cuda")
    cws = torch.empty(sav.attn_vsa_compressed_workspace_size(1, 4, 4, nt, 128), dtype=torch.uint8, device="cuda")
    gate = dev(randn_bf16(tuple(qt.shape), 633))
    out = torch.empty_like(qt)
    lse = torch.empty((1, 4, qt.shape[1]), dtype=torch.float32, device="cuda")

    def fn():
        sav.attn_vsa_block_map(qt, kt, sizes, 128 ** -0.5, 5, block_map=bmap, workspace=mws)
        sav.attn_block_sparse_fwd(qt, kt, vt, bmap, sizes, 128 ** -0.5, out=out, lse=lse, workspace=sws)
        sav.attn_vsa_compressed_add(qt, kt, vt, sizes, gate, 128 ** -0.5, out, workspace=cws)

    announce("graph sparse + vsa")
    fn()
    torch.cuda.synchronize()
    ref = (bmap.clone(), out.clone(), lse.clone())
    g = capture(fn)
    replay_matches(g, [bmap, out, lse], ref, other=_other_work)


@pytest.mark.parametrize("masked", [True, False])
def test_padded_and_masked_graph(masked):
    mask = (np.random.default_rng(640).random((3, 200)) < 0.7).astype(np.uint8)
    case = padded_case(3, 200, 200, num_heads=8, num_kv_heads=2, head_dim=128, seed=641, q_lens=[200, 50, 0],
                       k_lens=[180, 200, 7], key_mask=mask, causal=True)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    out = torch.empty_like(q)
    lse = torch.empty((8, 600), dtype=torch.float32, device="cuda")
    if masked:
        m = dev(case.key_mask)
        ws = torch.empty(sav.attn_masked_fwd_workspace_size(3, 200, 200, 8, 2, 128, True), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: sav.attn_masked_fwd(q, k, v, m, case.scale, True, mask_queries=True, out=out, lse=lse,  # noqa: E731
                                         workspace=ws)
    else:
        ql, kl = dev(case.q_lens), dev(case.k_lens)
        ws = torch.empty(sav.attn_padded_fwd_workspace_size(3), dtype=torch.uint8, device="cuda")
        fn = lambda: sav.attn_padded_fwd(q, k, v, ql, kl, case.scale, True, out=out, lse=lse, workspace=ws)  # noqa: E731
    announce("graph padded", masked)
    fn()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g = capture(fn)
    replay_matches(g, [out, lse], ref, other=_other_work)
