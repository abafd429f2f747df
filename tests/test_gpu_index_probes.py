"""Bit-exact indexing probes through the kernels the full-size workloads run:
the streaming paged decode (plain at head_dims 96, 128, 192, sliding-window
and the speculative multi-token columns), the pipelined prefill kernel reading
keys from the paged cache (head_dims 96 to 256), and the pipelined
block-sparse kernel with its packed kept-tile lists (head_dims 96 to 256).

Construction, shared by every probe: one selected key per unit (sequence or
query tile, and head) scores thousands of logit units above every other key
the unit may see, so the exponent of the gap underflows to 0 in fp32 and the
output row must equal the selected key's value row bit for bit. Every key the
unit must NOT read (unused blocks and -1 table tails, the unused end of a
sequence's last block, keys before a sliding window, tile padding rows, tiles
the map drops) carries that same large score, so a stray read ties with the
selected key and moves the output. Value rows encode where they live (physical
block, slot, kv head; or tile, row, head) as small integers bf16 holds exactly.

Passages: the vLLM-Ascend attention_v1.py page (AscendMetadata.block_tables,
forward_paged_attention, _forward_fia_slidingwindow, _get_fia_params) and the
vLLM-Omni fastvideo_vsa.py page (_fastvideo_h3_vsa_bhsd_op with block_map and
variable_block_sizes)."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_varlen_amd as sav
from tests._gpu_helpers import OUT_TOL, announce, assert_close, dev, host
from workloads import cumulative, paged_case

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
# in-block slots the rounds cycle through: both ends of every 32-token chunk
SLOTS = [0, 31, 32, 33, 63, 64, 95, 96, 127, 1, 17, 100]


def _probe_cache(tables, ctx, lo, num_blocks, hkv, d):
    """[2, NB, 128, hkv, d] bf16 on the GPU: value rows hold (block % 256,
    block // 256, slot, head) and then column index % 200 (so a row read with
    its 16-byte pieces out of place differs); keys are 0 on the visible tokens
    [lo[b], ctx[b]) of every sequence and 8 (poison) on every other slot."""
    nb = num_blocks
    kv = torch.zeros((2, nb, 128, hkv, d), dtype=BF16)
    blk = torch.arange(nb)
    kv[1, :, :, :, 0] = (blk % 256).view(nb, 1, 1).to(BF16)
    kv[1, :, :, :, 1] = (blk // 256).view(nb, 1, 1).to(BF16)
    kv[1, :, :, :, 2] = torch.arange(128).view(1, 128, 1).to(BF16)
    kv[1, :, :, :, 3] = torch.arange(hkv).view(1, 1, hkv).to(BF16)
    kv[1, :, :, :, 4:] = (torch.arange(4, d) % 200).to(BF16)
    kv[0] = 8.0
    for b, L in enumerate(ctx):
        if L > lo[b]:
            t = torch.arange(int(lo[b]), int(L))
            kv[0, torch.from_numpy(tables[b]).long()[t // 128], t % 128] = 0.0
    return kv.cuda()


def _select(r, b, h, hkv, lo, L):
    """Token that kv head h of sequence b selects in round r: the rounds walk
    every block-table position that holds a visible token, each at a slot taken
    from SLOTS, clamped into [lo, L)."""
    first, last = lo // 128, (L - 1) // 128
    bi = first + (r * hkv + h) % (last - first + 1)
    t = bi * 128 + SLOTS[(r + h + b) % len(SLOTS)]
    return min(max(t, lo), L - 1)


def _rounds(ctx, lo, hkv):
    nblk = max(((L - 1) // 128 - l // 128 + 1) for L, l in zip(ctx, lo) if L > l)
    return -(-nblk // hkv)


class _Selection:
    """The selected tokens of one round, raised to the poison score on the GPU
    cache while the call runs."""

    def __init__(self, kv, tables, picks):
        self.picks = picks  # {(b, h): t}
        self.kv = kv
        rows = [(int(tables[b, t // 128]), t % 128, h) for (b, h), t in picks.items()]
        self.idx = torch.tensor(rows, dtype=torch.long, device=kv.device).t()

    def __enter__(self):
        self.kv[0, self.idx[0], self.idx[1], self.idx[2]] = 8.0
        return self

    def __exit__(self, *exc):
        self.kv[0, self.idx[0], self.idx[1], self.idx[2]] = 0.0

    def values(self):
        """Value row of each pick, in picks order, on the host."""
        return self.kv[1, self.idx[0], self.idx[1], self.idx[2]].cpu()


def _decode_probe(ctx, hq, hkv, d, seed, window=None):
    case = paged_case(ctx, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=seed, spare_blocks=7,
                      max_blocks_per_seq=-(-max(ctx) // 128) + 3, name=f"probe-{seed}")
    group = hq // hkv
    lo = [0 if window is None else max(0, L - 1 - window) for L in ctx]
    kv = _probe_cache(case.block_tables, ctx, lo, case.num_blocks, hkv, d)
    q = torch.full((len(ctx), hq, d), 8.0, dtype=BF16, device="cuda")
    bt, cl = dev(case.block_tables), dev(case.context_lens)
    checked = 0
    for r in range(_rounds(ctx, lo, hkv)):
        picks = {(b, h): _select(r, b, h, hkv, lo[b], L) for b, L in enumerate(ctx) if L > 0 for h in range(hkv)}
        with _Selection(kv, case.block_tables, picks) as sel:
            out = sav.attn_paged_decode(q, kv, bt, cl, max(ctx), 0.125, window=window)
            torch.cuda.synchronize()
            want = sel.values()
        out = out.cpu()
        for n, ((b, h), t) in enumerate(picks.items()):
            got = out[b, h * group:(h + 1) * group]
            assert torch.equal(got, want[n].expand(group, d)), (r, b, h, t, got[0, :4].tolist(), want[n, :4].tolist())
            checked += group
        for b, L in enumerate(ctx):
            if L == 0:
                assert torch.all(out[b] == 0)
    return checked


# contexts that end on, just before and just after 32-token chunk and 128-token
# block edges, short ones between long ones (the streaming kernel's equal
# segments of the concatenated token stream then start and end inside
# sequences, chunks and blocks), and an empty one
DECODE_CTX = [1, 31, 32, 33, 127, 128, 129, 0, 255, 257, 300, 777, 2048, 4100, 9000, 3]


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (40, 2, 128), (32, 8, 96), (32, 8, 192)])
def test_decode_stream_probe_every_block_position(hq, hkv, d):
    """head_dims 96 and 192 stream with token rows padded in LDS (256 and 512
    bytes); the probe's value rows encode every column, so a misplaced or
    padded piece shows."""
    announce("probe decode stream", hq, hkv, d)
    checked = _decode_probe(DECODE_CTX, hq, hkv, d, seed=240 + hq + (d - 128))
    assert checked >= 71 * hq


@pytest.mark.parametrize("window", [0, 31, 33, 300, 4096])
@pytest.mark.parametrize("d", [128, 64])
def test_sliding_window_decode_probe(window, d):
    """Keys before the window are live in the cache but poisoned, so the
    chunk-aligned start of the streamed range must mask them."""
    announce("probe swa decode", window, d)
    _decode_probe(DECODE_CTX, 32, 8, d, seed=260 + window % 89 + d, window=window)


def _paged_prefill_probe(ctx, qlens, hq, hkv, seed, d=128):
    case = paged_case(ctx, num_heads=hq, num_kv_heads=hkv, head_dim=d, seed=seed, spare_blocks=5,
                      max_blocks_per_seq=-(-max(ctx) // 128) + 2, name=f"probe-pp-{seed}")
    group = hq // hkv
    lo = [0] * len(ctx)
    kv = _probe_cache(case.block_tables, ctx, lo, case.num_blocks, hkv, d)
    cu = cumulative(qlens)
    tq = int(cu[-1])
    q_host = torch.full((tq, hq, d), 8.0, dtype=BF16)
    q = q_host.cuda()
    bt, cl, cuq = dev(case.block_tables), dev(case.context_lens), dev(cu)
    exact = 0
    for r in range(_rounds(ctx, lo, hkv)):
        picks = {(b, h): _select(r, b, h, hkv, 0, L) for b, L in enumerate(ctx) for h in range(hkv)}
        with _Selection(kv, case.block_tables, picks) as sel:
            out = sav.attn_paged_prefill(q, kv, bt, cuq, cl, max(qlens), max(ctx), 0.125)
            torch.cuda.synchronize()
            want = sel.values()
            kv_host = kv.cpu()
        out = out.cpu()
        # a query that sees its head's selected key returns that value row exactly
        seen = np.zeros((tq, hq), dtype=bool)
        for n, ((b, h), t) in enumerate(picks.items()):
            lq, lk = int(qlens[b]), int(ctx[b])
            for i in range(lq):
                if t <= i + lk - lq:
                    row = int(cu[b]) + i
                    got = out[row, h * group:(h + 1) * group]
                    assert torch.equal(got, want[n].expand(group, d)), (r, b, h, t, i)
                    seen[row, h * group:(h + 1) * group] = True
                    exact += group
        # the others see only zero keys: the mean of their visible value rows
        ref_o, _ = oracle.paged_prefill_attention(q_host, kv_host, case.block_tables, cu, case.context_lens, 0.125)
        if (~seen).any():
            assert_close("unseen rows", host(out)[~seen], ref_o[~seen], OUT_TOL, bf16_output=True)
    return exact


def test_speculative_columns_probe_every_block_position():
    """Short query runs (at most 16 tokens x a group of 4 heads) take the
    streaming decode kernel with (token, head) columns, each with its own
    bottom-right causal limit."""
    ctx = [16, 31, 129, 300, 777, 2048, 4100, 5, 9000]
    qlens = [16, 3, 16, 1, 7, 16, 12, 5, 2]
    announce("probe spec decode")
    exact = _paged_prefill_probe(ctx, qlens, 32, 8, seed=280)
    assert exact > 0


@pytest.mark.parametrize("d", [96, 128, 192, 256])
def test_paged_prefill_kernel_probe_every_block_position(d):
    """Long query runs take the pipelined prefill kernel with keys read
    through the block table (64-key tiles, one table lookup each): the 8-wave
    ring at head_dim 128, the 4-wave split rings with 512-byte LDS rows at 192
    (rows padded) and 256."""
    ctx = [300, 1000, 4100, 129, 2000, 64]
    qlens = [300, 17, 100, 129, 64, 1]
    announce("probe paged prefill", d)
    exact = _paged_prefill_probe(ctx, qlens, 8, 2, seed=290 + d, d=d)
    assert exact > 0


def _sparse_probe(nt, hq, hkv, seed, need_long=True, d=128):
    """Block-sparse probe. Query tile a of head h gets its own direction
    e = dir(h, a) (Q rows = 64 e). Real key rows of tile c hold 64 times the sum
    of the directions of every (head of the kv group, query tile) whose map
    drops c, and padding rows hold 64 times every direction: any read outside
    the kept tiles' real rows scores like the selected key. In each round every
    query tile picks one kept tile it has not yet picked and a free real row
    there, which is set to 64 e. Value rows encode (tile, row, kv head) and
    then the column index, so a misplaced 16-byte piece shows."""
    group = hq // hkv
    assert group * nt <= d
    rng = np.random.default_rng(seed)
    sizes = rng.integers(1, 65, nt).astype(np.int32)
    sizes[::9] = 64
    sizes[[4, 11]] = 0  # empty tiles: no rows, no keys
    sizes[7] = 1
    dens = rng.choice([0.0, 0.08, 0.4, 0.9, 1.0], size=(1, hq, nt))
    bmap = rng.random((1, hq, nt, nt)) < dens[..., None]
    bmap[0, :, 2] = False  # an empty map row
    bmap[0, 0, 5] = True  # a full one
    direction = lambda h, a: (h % group) * nt + a  # noqa: E731

    q = torch.zeros((1, nt * 64, hq, d), dtype=BF16)
    for h in range(hq):
        for a in range(nt):
            q[0, a * 64:(a + 1) * 64, h, direction(h, a)] = 64.0
    k = torch.zeros((1, nt * 64, hkv, d), dtype=BF16)
    for hk in range(hkv):
        for c in range(nt):
            poison = torch.zeros(d, dtype=BF16)
            for g in range(group):
                h = hk * group + g
                drop = np.nonzero(~bmap[0, h, :, c])[0]
                poison[[direction(h, a) for a in drop]] = 64.0
            k[0, c * 64:c * 64 + int(sizes[c]), hk] = poison
            everything = torch.zeros(d, dtype=BF16)
            everything[:group * nt] = 64.0
            k[0, c * 64 + int(sizes[c]):(c + 1) * 64, hk] = everything
    v = torch.zeros((1, nt * 64, hkv, d), dtype=BF16)
    v[0, :, :, 0] = (torch.arange(nt * 64) // 64).view(-1, 1).to(BF16)
    v[0, :, :, 1] = (torch.arange(nt * 64) % 64).view(-1, 1).to(BF16)
    v[0, :, :, 2] = torch.arange(hkv).view(1, hkv).to(BF16)
    v[0, :, :, 3:] = (torch.arange(3, d) % 200).to(BF16)

    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    md, sd = dev(bmap.astype(np.uint8)), dev(sizes)
    scale = d ** -0.5
    # kept tiles with real rows, per (head, query tile), that are still to be picked
    todo = {(h, a): [c for c in np.nonzero(bmap[0, h, a])[0].tolist() if sizes[c] > 0]
            for h in range(hq) for a in range(nt) if sizes[a] > 0}
    longest = max(len(x) for x in todo.values())
    if need_long:
        assert longest > 64, "the probe must cover kept lists longer than the 64-entry window"
    covered = 0
    rounds = 0
    while any(todo.values()):
        rounds += 1
        assert rounds <= 4 * longest, "probe rounds did not converge"
        taken = set()  # (kv head, key row)
        picks = {}
        for (h, a), lst in todo.items():
            hk = h // group
            for c in lst:
                free = [r for r in range(int(sizes[c])) if (hk, c * 64 + r) not in taken]
                if free:
                    row = c * 64 + free[(a * 7 + rounds * 13) % len(free)]
                    taken.add((hk, row))
                    picks[(h, a)] = (c, row)
                    lst.remove(c)
                    break
        rows = torch.tensor([row for (h, a), (c, row) in picks.items()], dtype=torch.long)
        heads = torch.tensor([h // group for (h, a) in picks], dtype=torch.long)
        vecs = torch.zeros((len(picks), d), dtype=BF16)
        for n, (h, a) in enumerate(picks):
            vecs[n, direction(h, a)] = 64.0
        saved = kd[0, rows.cuda(), heads.cuda()].clone()
        kd[0, rows.cuda(), heads.cuda()] = vecs.cuda()
        out = sav.attn_block_sparse_fwd(qd, kd, vd, md, sd, scale)
        torch.cuda.synchronize()
        kd[0, rows.cuda(), heads.cuda()] = saved
        out = out.cpu()
        for (h, a), (c, row) in picks.items():
            n = int(sizes[a])
            want = v[0, row, h // group]
            assert torch.equal(out[0, a * 64:a * 64 + n, h], want.expand(n, d)), (rounds, h, a, c, row)
            assert torch.all(out[0, a * 64 + n:(a + 1) * 64, h] == 0)
            covered += 1
        # rows whose query tile is empty, keeps nothing, or has no pick left
        for h in range(hq):
            for a in range(nt):
                if sizes[a] == 0 or not bmap[0, h, a][sizes > 0].any():
                    assert torch.all(out[0, a * 64:(a + 1) * 64, h] == 0), (h, a)
    return covered, longest


@pytest.mark.parametrize("d", [128, 96, 192, 256])
def test_sparse_pipe_kept_tile_probe_long_lists(d):
    """Up to 100 tiles, two heads: kept lists longer than 64 entries (the
    kernel holds 64 list entries in a register window at a time), partial,
    single-row and empty tiles, an empty map row; every kept tile of every
    (head, query tile) is selected in some round. head_dims 96 and 192 pad
    their LDS rows (256 and 512 bytes)."""
    nt = 100 if d >= 100 else 90
    announce("probe sparse long lists", d)
    covered, longest = _sparse_probe(nt, 2, 2, seed=300 + (d - 128), d=d)
    assert longest > 64 and covered > 900


@pytest.mark.parametrize("d", [128, 256])
def test_sparse_pipe_kept_tile_probe_grouped_heads(d):
    """Grouped heads (4 query heads on 2 kv heads, 60 tiles): query head h
    reads kv head h // 2."""
    announce("probe sparse gqa", d)
    covered, _ = _sparse_probe(60, 4, 2, seed=301 + (d - 128), need_long=False, d=d)
    assert covered > 1000
