"""The C-ABI library loads, exports every symbol the header declares, and its
host-side validation rejects bad arguments before any HIP call. No call here
reaches a kernel launch, so these run without a GPU."""

import ctypes
import os

import pytest

import softmax_attention_varlen_amd as sav

LIB = sav.LIB_PATH
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def lib():
    return sav.load_library()


def test_exports_every_declared_symbol():
    names = sav.exported_symbols()
    assert {"attn_varlen_fwd", "attn_paged_decode", "attn_block_sparse_fwd"} <= set(names)
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in the header but not exported"


def test_abi_version_and_status_strings():
    assert sav.attn_abi_version() == 1
    assert sav.attn_status_string(0) == "ok"
    assert sav.attn_status_string(1) == "invalid argument"
    assert sav.attn_status_string(3) == "workspace too small"
    assert sav.attn_status_string(99) == "unknown status"


def _varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cuq=FAKE, cuk=FAKE, batch=2, tq=256, tk=256, mq=156, mk=156, hq=4, hkv=4, d=64,
             scale=0.125, causal=0, out=FAKE, lse=None)
    a.update(kw)
    return lib().attn_varlen_fwd(a["q"], a["k"], a["v"], a["cuq"], a["cuk"], a["batch"], a["tq"], a["tk"], a["mq"],
                                 a["mk"], a["hq"], a["hkv"], a["d"], a["scale"], a["causal"], a["out"], a["lse"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), UNSUPPORTED), (dict(d=512), UNSUPPORTED), (dict(d=0), UNSUPPORTED),
    (dict(hq=6, hkv=4), UNSUPPORTED),
    (dict(hq=0), INVALID), (dict(hkv=0), INVALID), (dict(batch=-1), INVALID), (dict(tq=-5), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-0.1), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(causal=2), INVALID),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(cuq=None), INVALID), (dict(cuk=None), INVALID),
    (dict(k=None), INVALID), (dict(mq=300), INVALID), (dict(mk=300), INVALID), (dict(mq=0), INVALID),
])
def test_varlen_validation(kw, code):
    assert _varlen(**kw) == code


@pytest.mark.parametrize("kw", [dict(batch=0), dict(tq=0, mq=0)])
def test_varlen_empty_is_noop(kw):
    # nothing to do: returns before any HIP call, even with null buffers
    assert _varlen(q=None, out=None, **kw) == OK


def _decode(**kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, ctx=FAKE, nseq=4, nblocks=10, mbps=4, maxctx=500, hq=8, hkv=2, d=128,
             bs=128, scale=0.1, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib().attn_paged_decode(a["q"], a["kv"], a["bt"], a["ctx"], a["nseq"], a["nblocks"], a["mbps"],
                                   a["maxctx"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"], a["out"], a["lse"],
                                   a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=64), UNSUPPORTED), (dict(bs=16), UNSUPPORTED), (dict(d=100), UNSUPPORTED), (dict(hq=6, hkv=4), UNSUPPORTED),
    (dict(maxctx=513), INVALID), (dict(nseq=-1), INVALID), (dict(q=None), INVALID), (dict(kv=None), INVALID),
    (dict(bt=None), INVALID), (dict(ctx=None), INVALID), (dict(out=None), INVALID), (dict(scale=0.0), INVALID),
    (dict(wsb=0), WS_SMALL), (dict(ws=None), INVALID), (dict(nblocks=0), INVALID),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_is_noop():
    assert _decode(nseq=0, q=None, out=None, ws=None, wsb=0) == OK


def test_decode_workspace_query_covers_partials():
    # the plan does not depend on the context length
    small = sav.attn_paged_decode_workspace_size(64, 32, 8, 128, 1024)
    big = sav.attn_paged_decode_workspace_size(64, 32, 8, 128, 32768)
    assert 0 < small == big
    # fp32 partials (O and LSE) for num_seqs + n_seg slots of every head, and two
    # int32 arrays of num_seqs + 1; n_seg = 256 CUs x waves per CU / (kv heads x query chunks)
    for d, waves in ((64, 8), (96, 4), (128, 4), (192, 2), (256, 2)):
        n_seg = 256 * waves // 8
        want = (64 + n_seg) * 32 * (d + 1) * 4
        got = sav.attn_paged_decode_workspace_size(64, 32, 8, d, 4096)
        # plus the two int32 arrays and alignment to 256 bytes: at most 1 KiB here
        assert want <= got <= want + 1024, (d, got, want)
    with pytest.raises(sav.AttnError):
        sav.attn_paged_decode_workspace_size(64, 32, 8, 100, 1024)


def _sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, m=FAKE, ts=FAKE, b=1, nt=4, hq=2, hkv=2, d=128, scale=0.1, out=FAKE, lse=None,
             ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib().attn_block_sparse_fwd(a["q"], a["k"], a["v"], a["m"], a["ts"], a["b"], a["nt"], a["hq"], a["hkv"],
                                       a["d"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=32), UNSUPPORTED), (dict(hq=3, hkv=2), UNSUPPORTED), (dict(m=None), INVALID), (dict(ts=None), INVALID),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(wsb=10), WS_SMALL), (dict(ws=None), INVALID),
    (dict(scale=-1.0), INVALID), (dict(nt=-1), INVALID),
])
def test_sparse_validation(kw, code):
    assert _sparse(**kw) == code


def test_sparse_workspace_query():
    assert sav.attn_block_sparse_workspace_size(1, 12, 256) == 12 * 256 * 256 * 4 + 2 * 12 * 256 * 4


def test_map_to_index_validation():
    L = lib()
    assert L.attn_block_map_to_index(FAKE, 4, 0, FAKE, FAKE, None) == INVALID
    assert L.attn_block_map_to_index(None, 4, 8, FAKE, FAKE, None) == INVALID
    assert L.attn_block_map_to_index(None, 0, 8, None, None, None) == OK


def test_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        sav.attn_varlen_fwd(q, q, q, cu, cu, 4, 4, 0.125, False, out=torch.empty_like(q))


def _kv_write(**kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, n=16, hkv=2, d=128, nblocks=10, bs=128, cache=FAKE)
    a.update(kw)
    return lib().attn_paged_kv_write(a["k"], a["v"], a["slots"], a["n"], a["hkv"], a["d"], a["nblocks"], a["bs"],
                                     a["cache"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=64), UNSUPPORTED), (dict(d=100), UNSUPPORTED), (dict(n=-1), INVALID), (dict(hkv=0), INVALID),
    (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(slots=None), INVALID), (dict(cache=None), INVALID),
    (dict(nblocks=0), INVALID), (dict(nblocks=-3), INVALID),
])
def test_kv_write_validation(kw, code):
    assert _kv_write(**kw) == code


def test_kv_write_empty_is_noop():
    assert _kv_write(n=0, k=None, v=None, slots=None, cache=None) == OK


def _paged_prefill(**kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, cuq=FAKE, ctx=FAKE, batch=3, tq=300, mq=200, maxctx=500, nblocks=12, mbps=4,
             hq=8, hkv=2, d=128, bs=128, scale=0.1, out=FAKE, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib().attn_paged_prefill(a["q"], a["kv"], a["bt"], a["cuq"], a["ctx"], a["batch"], a["tq"], a["mq"],
                                    a["maxctx"], a["nblocks"], a["mbps"], a["hq"], a["hkv"], a["d"], a["bs"],
                                    a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=64), UNSUPPORTED), (dict(d=100), UNSUPPORTED), (dict(hq=6, hkv=4), UNSUPPORTED),
    (dict(maxctx=513), INVALID), (dict(mq=301), INVALID), (dict(mq=0), INVALID), (dict(batch=-1), INVALID),
    (dict(tq=-1), INVALID), (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(cuq=None), INVALID),
    (dict(ctx=None), INVALID), (dict(kv=None), INVALID), (dict(bt=None), INVALID), (dict(nblocks=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(hkv=0), INVALID),
    # 4 new tokens x group 4 = 16 columns: the streaming path, which needs a workspace
    (dict(mq=4, tq=12), WS_SMALL), (dict(mq=4, tq=12, wsb=1 << 30), INVALID),
])
def test_paged_prefill_validation(kw, code):
    assert _paged_prefill(**kw) == code


@pytest.mark.parametrize("kw", [dict(batch=0), dict(tq=0, mq=0)])
def test_paged_prefill_empty_is_noop(kw):
    assert _paged_prefill(q=None, out=None, **kw) == OK


def test_paged_prefill_workspace_query():
    # long query runs use the prefill kernels (no workspace); short ones stream like decode
    assert sav.attn_paged_prefill_workspace_size(16, 32, 8, 128, 1024, 16384) == 0
    # every head dim streams short runs
    for d in (64, 96, 192, 256):
        assert sav.attn_paged_prefill_workspace_size(16, 32, 8, d, 4, 16384) > 0
        assert sav.attn_paged_prefill_workspace_size(16, 32, 8, d, 1, 16384) == \
            sav.attn_paged_decode_workspace_size(16, 32, 8, d, 16384)
    n4 = sav.attn_paged_prefill_workspace_size(64, 32, 8, 128, 4, 32768)
    n1 = sav.attn_paged_prefill_workspace_size(64, 32, 8, 128, 1, 32768)
    assert n4 > n1 > 0
    assert n1 == sav.attn_paged_decode_workspace_size(64, 32, 8, 128, 32768)


def _window(**kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, ctx=FAKE, nseq=4, nblocks=10, mbps=4, maxctx=500, hq=8, hkv=2, d=128,
             bs=128, window=100, scale=0.1, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib().attn_paged_decode_sliding_window(a["q"], a["kv"], a["bt"], a["ctx"], a["nseq"], a["nblocks"],
                                                  a["mbps"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["bs"],
                                                  a["window"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"],
                                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), INVALID), (dict(bs=64), UNSUPPORTED), (dict(d=100), UNSUPPORTED), (dict(maxctx=513), INVALID),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(ctx=None), INVALID), (dict(wsb=0), WS_SMALL),
    (dict(scale=float("nan")), INVALID),
])
def test_sliding_window_validation(kw, code):
    assert _window(**kw) == code


def test_sliding_window_empty_is_noop():
    assert _window(nseq=0, q=None, out=None, ws=None, wsb=0) == OK


def _padded(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ql=FAKE, kl=FAKE, b=2, sq=100, sk=80, hq=8, hkv=2, d=128, scale=0.1, causal=0,
             out=FAKE, lse=None, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib().attn_padded_fwd(a["q"], a["k"], a["v"], a["ql"], a["kl"], a["b"], a["sq"], a["sk"], a["hq"],
                                 a["hkv"], a["d"], a["scale"], a["causal"], a["out"], a["lse"], a["ws"], a["wsb"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), UNSUPPORTED), (dict(hq=6, hkv=4), UNSUPPORTED), (dict(b=-1), INVALID), (dict(sq=-1), INVALID),
    (dict(sk=-2), INVALID), (dict(hq=0), INVALID), (dict(scale=0.0), INVALID), (dict(q=None), INVALID),
    (dict(out=None), INVALID), (dict(ql=None), INVALID), (dict(kl=None), INVALID), (dict(k=None), INVALID),
    (dict(wsb=0), WS_SMALL), (dict(ws=None), INVALID), (dict(b=70000, sq=70000), UNSUPPORTED),
])
def test_padded_validation(kw, code):
    assert _padded(**kw) == code


@pytest.mark.parametrize("kw", [dict(b=0), dict(sq=0)])
def test_padded_empty_is_noop(kw):
    assert _padded(q=None, out=None, ws=None, wsb=0, **kw) == OK


def _masked(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, mask=FAKE, b=2, sq=100, sk=100, hq=8, hkv=2, d=128, scale=0.1, causal=0, mq=1,
             out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib().attn_masked_fwd(a["q"], a["k"], a["v"], a["mask"], a["b"], a["sq"], a["sk"], a["hq"], a["hkv"],
                                 a["d"], a["scale"], a["causal"], a["mq"], a["out"], a["lse"], a["ws"], a["wsb"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(sk=90), INVALID), (dict(d=80), UNSUPPORTED), (dict(hq=6, hkv=4), UNSUPPORTED), (dict(b=-1), INVALID),
    (dict(scale=-1.0), INVALID), (dict(q=None), INVALID), (dict(mask=None), INVALID), (dict(v=None), INVALID),
    (dict(out=None), INVALID), (dict(wsb=0), WS_SMALL), (dict(ws=None), INVALID),
])
def test_masked_validation(kw, code):
    assert _masked(**kw) == code


def test_masked_empty_is_noop():
    assert _masked(b=0, q=None, out=None, ws=None, wsb=0) == OK
    assert _masked(sq=0, sk=0, q=None, out=None, ws=None, wsb=0) == OK


def test_padding_workspace_queries():
    assert sav.attn_padded_fwd_workspace_size(4) >= 2 * 5 * 4
    cross = sav.attn_masked_fwd_workspace_size(2, 4096, 512, 24, 24, 128, False)
    self_ = sav.attn_masked_fwd_workspace_size(2, 512, 512, 24, 24, 128, True)
    # packed k and v at least; self-attention also packs q and the output
    assert cross >= 2 * (2 * 512 * 24 * 128 * 2)
    assert self_ >= 4 * (2 * 512 * 24 * 128 * 2)
    with pytest.raises(sav.AttnError):
        sav.attn_padded_fwd_workspace_size(-1)


def test_h3_geometry_validation():
    segs = (ctypes.c_int32 * 17)(*([10] * 17))
    a, b = ctypes.c_int32(0), ctypes.c_int32(0)
    f = lib().attn_vsa_h3_num_tiles
    assert f(segs, 17, 4, 4, 4, 4, 4, 4, ctypes.byref(a), ctypes.byref(b)) == UNSUPPORTED
    neg = (ctypes.c_int32 * 2)(10, -1)
    assert f(neg, 2, 4, 4, 4, 4, 4, 4, ctypes.byref(a), ctypes.byref(b)) == INVALID
    assert f(None, 2, 4, 4, 4, 4, 4, 4, ctypes.byref(a), ctypes.byref(b)) == INVALID
    assert f(segs, 3, 4, 4, 4, 4, 4, 4, None, ctypes.byref(b)) == INVALID
    assert sav.attn_vsa_h3_num_tiles((70, 5), (2, 5, 4)) == (3, 5)
    assert sav.attn_vsa_h3_num_tiles((0, 130), (5, 9, 7)) == (3, 15)
    assert lib().attn_vsa_h3_tile_gather(FAKE, segs, 17, 1, 4, 4, 4, 4, 4, 4, 64, FAKE, None, None) == UNSUPPORTED
    assert lib().attn_vsa_h3_untile(FAKE, neg, 2, 1, 4, 4, 4, 4, 4, 4, 64, FAKE, None) == INVALID


def test_h3_block_map_validation():
    f = lib().attn_vsa_h3_block_map
    assert f(FAKE, FAKE, FAKE, 1, 10, 11, 4, 4, 128, 0.1, 4, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 1, 10, -1, 4, 4, 128, 0.1, 4, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 1, 10, 2, 4, 4, 128, 0.1, 0, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 1, 10, 2, 4, 4, 128, 0.1, 4, FAKE, FAKE, 0, None) == WS_SMALL


def test_h3_gather_block_map_validation():
    f = lib().attn_vsa_h3_gather_block_map
    segs = (ctypes.c_int32 * 2)(70, 5)
    many = (ctypes.c_int32 * 17)(*([10] * 17))
    neg = (ctypes.c_int32 * 2)(10, -1)

    def call(segments=segs, nseg=2, batch=1, shape=(2, 5, 4), tiles=(4, 4, 4), hq=4, hkv=2, d=128, scale=0.1,
             topk=4, q=FAKE, k=FAKE, qt=FAKE, kt=FAKE, sizes=None, bmap=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return f(q, k, segments, nseg, batch, *shape, *tiles, hq, hkv, d, scale, topk, qt, kt, sizes, bmap, ws,
                 ws_bytes, None)

    assert call(topk=0) == INVALID
    assert call(hq=0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(d=80) == UNSUPPORTED
    assert call(hq=6, hkv=4) == UNSUPPORTED
    assert call(segments=many, nseg=17) == UNSUPPORTED
    assert call(segments=neg) == INVALID
    assert call(segments=None) == INVALID
    assert call(tiles=(4, 4, 8)) == UNSUPPORTED  # a tile of more than 64 rows
    assert call(batch=-1) == INVALID
    assert call(q=None) == INVALID
    assert call(bmap=None) == INVALID
    assert call(ws_bytes=0) == WS_SMALL
    assert call(ws=None) == INVALID
    assert call(batch=0) == OK  # no-op
    assert call(segments=None, nseg=0, shape=(0, 0, 0)) == OK  # no tiles: no-op


def _decode_scratch(**kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, ctx=FAKE, nseq=4, nblocks=10, mbps=4, maxctx=500, hq=8, hkv=2, d=128,
             bs=128, scale=0.1, out=FAKE, lse=None)
    a.update(kw)
    return lib().attn_paged_decode_scratch(a["q"], a["kv"], a["bt"], a["ctx"], a["nseq"], a["nblocks"], a["mbps"],
                                           a["maxctx"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"], a["out"],
                                           a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=64), UNSUPPORTED), (dict(d=100), UNSUPPORTED), (dict(hq=6, hkv=4), UNSUPPORTED),
    (dict(maxctx=513), INVALID), (dict(nseq=-1), INVALID), (dict(q=None), INVALID), (dict(out=None), INVALID),
    (dict(scale=0.0), INVALID),
    # partials that do not fit the 32 MiB array: (128 + 4096) * 32 * 129 * 4 B at head_dim 128 and
    # (256 + 4096) * 32 * 65 * 4 B at head_dim 64
    (dict(nseq=4096, hq=32, hkv=8, d=128), WS_SMALL), (dict(nseq=4096, hq=32, hkv=8, d=64), WS_SMALL),
])
def test_decode_scratch_validation(kw, code):
    # every case is refused before the call looks up its device array
    assert _decode_scratch(**kw) == code


def test_decode_scratch_empty_is_noop():
    assert _decode_scratch(nseq=0, q=None, out=None) == OK
