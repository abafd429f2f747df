"""fp64 statement of the attention forward the pages dispatch to.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed everywhere (the pages call fused kernels with a softmax
scale, a causal flag or a mask and get back ``out`` or ``(out, lse)``; the
[FA] laser-attention note names the unscaled product S = Q K^T, and the [VSA]
compressed branch writes tile attention as softmax(scale * q k^T) v):

    z_ij   = scale * <q_i, k_j>             for allowed keys j of row i
    O_i    = sum_j exp(z_ij) v_j / sum_j exp(z_ij)
    LSE_i  = ln sum_j exp(z_ij)

A row with no allowed key has O_i = 0 and LSE_i = -inf (the pages leave this
case to the kernels' "invalid row" handling; no shipped workload reaches it).
Subtracting the row maximum before exp is an exact identity of the definition
and only keeps fp64 in range.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a (CPU) torch tensor of any float dtype."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    # torch tensor (bf16 has no numpy dtype; bf16 -> fp64 is exact)
    import torch

    return x.detach().to("cpu", torch.float64).numpy()


def _ints(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x.astype(np.int64, copy=False)
    if isinstance(x, (list, tuple)):
        return np.asarray(x, dtype=np.int64)
    return x.detach().to("cpu").numpy().astype(np.int64)


def _attend(qrows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float, allowed: np.ndarray):
    """softmax(scale * q k^T + mask) v for one head.

    qrows [M, D], keys [N, D], values [N, Dv], allowed bool [M, N].
    Returns (out [M, Dv], lse [M]).
    """
    m_rows = qrows.shape[0]
    dv = values.shape[1]
    if keys.shape[0] == 0 or m_rows == 0:
        return np.zeros((m_rows, dv)), np.full(m_rows, NEG_INF)
    z = scale * (qrows @ keys.T)
    z = np.where(allowed, z, NEG_INF)
    zmax = z.max(axis=1)
    has_key = np.isfinite(zmax)
    zmax_safe = np.where(has_key, zmax, 0.0)
    w = np.where(allowed, np.exp(z - zmax_safe[:, None]), 0.0)
    denom = w.sum(axis=1)
    out = np.zeros((m_rows, dv))
    out[has_key] = (w[has_key] @ values) / denom[has_key, None]
    lse = np.full(m_rows, NEG_INF)
    lse[has_key] = zmax_safe[has_key] + np.log(denom[has_key])
    return out, lse


def _causal_allowed(rows_local: np.ndarray, len_q: int, len_k: int) -> np.ndarray:
    """Bottom-right causal alignment, [FA] forward_fa_npu causal branch: key j is
    blocked for query i exactly when j > i + (len_k - len_q)."""
    j = np.arange(len_k)[None, :]
    return j <= rows_local[:, None] + (len_k - len_q)


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool, rows=None):
    """Packed variable-length attention ([FA] FlashAttentionImpl._forward_varlen_packed
    and _forward_varlen_dense: q/k/v are ``[total, heads, dim]`` with documents
    delimited by cumulative ``cu_seqlens``; a query attends only keys of its own
    document; grouped-query heads map query head h to kv head
    ``h // (num_heads // num_kv_heads)`` ([ASC] AscendAttentionBackendImpl keeps
    ``num_queries_per_kv = num_heads // num_kv_heads``).

    q [Tq, Hq, D], k [Tk, Hkv, D], v [Tk, Hkv, Dv].
    ``rows`` selects global query rows to compute (default: all).
    Returns out [R, Hq, Dv] and lse [Hq, R] in float64, R = number of rows.

    Pinned: closed forms, brute force, torch SDPA (fp64), packed == per-doc,
    GQA == repeated-KV MHA, dense == uniform varlen, split/merge, pre-scale.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    cu_q, cu_k = _ints(cu_seqlens_q), _ints(cu_seqlens_k)
    total_q, hq, _ = qf.shape
    hkv = kf.shape[1]
    if hq % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    rows = np.arange(total_q) if rows is None else _ints(rows)
    out = np.zeros((rows.size, hq, vf.shape[2]))
    lse = np.full((hq, rows.size), NEG_INF)
    # document of each requested row
    doc = np.searchsorted(cu_q, rows, side="right") - 1
    for b in np.unique(doc):
        sel = np.nonzero(doc == b)[0]
        q0, q1 = cu_q[b], cu_q[b + 1]
        k0, k1 = cu_k[b], cu_k[b + 1]
        len_q, len_k = q1 - q0, k1 - k0
        local = rows[sel] - q0
        if causal:
            allowed = _causal_allowed(local, len_q, len_k)
        else:
            allowed = np.ones((local.size, len_k), dtype=bool)
        for h in range(hq):
            hk = h // group
            o, l_ = _attend(qf[rows[sel], h], kf[k0:k1, hk], vf[k0:k1, hk], scale, allowed)
            out[sel, h] = o
            lse[h, sel] = l_
    return out, lse


def dense_attention(q, k, v, scale: float, causal: bool):
    """Batched ``[B, S, H, D]`` attention ([FA] FlashAttentionImpl.forward_cuda dense
    branch, flash_attn_func). Written per (batch, head) directly, independently of
    the varlen indexing, so that dense == varlen(uniform cu_seqlens) is a real check.

    Returns out [B, Sq, Hq, Dv], lse [B, Hq, Sq].
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    bsz, sq, hq, _ = qf.shape
    sk, hkv = kf.shape[1], kf.shape[2]
    group = hq // hkv
    out = np.zeros((bsz, sq, hq, vf.shape[3]))
    lse = np.full((bsz, hq, sq), NEG_INF)
    if causal:
        allowed = _causal_allowed(np.arange(sq), sq, sk)
    else:
        allowed = np.ones((sq, sk), dtype=bool)
    for b in range(bsz):
        for h in range(hq):
            o, l_ = _attend(qf[b, :, h], kf[b, :, h // group], vf[b, :, h // group], scale, allowed)
            out[b, :, h] = o
            lse[b, h] = l_
    return out, lse


def slot_to_block_offset(slot, block_size: int):
    """[ASC] AscendMetadata.slot_mapping: a flat cache slot addresses
    (physical block, offset in block) = (slot // block_size, slot % block_size),
    offsets counted from 0. Pinned by the page's worked example."""
    s = _ints(slot)
    return s // block_size, s % block_size


def paged_decode_attention(q, kv_cache, block_tables, context_lens, scale: float, seqs=None):
    """Single-token decode over a paged KV cache ([ASC] get_kv_cache_shape:
    cache ``(2, num_blocks, block_size, num_kv_heads, head_size)`` with index 0 = K
    and 1 = V; forward_paged_attention passes ``block_table`` and
    ``context_lens``; AscendMetadata.block_tables maps a sequence to its physical
    blocks). Token t < context_lens[b] of sequence b lives in block
    ``block_tables[b, t // block_size]`` at offset ``t % block_size``. The cache is
    written before attention ([ASC] forward calls reshape_and_cache first), so the
    one query token is the last position and bottom-right causal admits every one
    of the context_lens[b] keys.

    q [S, Hq, D]; kv_cache [2, NB, BS, Hkv, D] (torch or numpy); block_tables [S, MB].
    Returns out [R, Hq, D], lse [Hq, R] in float64 for the selected sequences.

    Pinned: paged == contiguous gather (against varlen), slot worked example.
    """
    qf = _f64(q)
    bt = _ints(block_tables)
    ctx = _ints(context_lens)
    nseq, hq, _ = qf.shape
    block_size = kv_cache.shape[2]
    hkv = kv_cache.shape[3]
    group = hq // hkv
    seqs = np.arange(nseq) if seqs is None else _ints(seqs)
    dv = kv_cache.shape[4]
    out = np.zeros((seqs.size, hq, dv))
    lse = np.full((hq, seqs.size), NEG_INF)
    for r, b in enumerate(seqs):
        length = int(ctx[b])
        t = np.arange(length)
        blk = bt[b, t // block_size]
        off = t % block_size
        if isinstance(kv_cache, np.ndarray):
            keys = kv_cache[0][blk, off]
            vals = kv_cache[1][blk, off]
        else:  # torch: index on the host tensor, then upcast only what is used
            import torch

            bi = torch.from_numpy(blk)
            oi = torch.from_numpy(off)
            keys = kv_cache[0][bi, oi]
            vals = kv_cache[1][bi, oi]
        keys, vals = _f64(keys), _f64(vals)  # [L, Hkv, D]
        allowed = np.ones((1, length), dtype=bool)
        for h in range(hq):
            o, l_ = _attend(qf[b, h][None, :], keys[:, h // group], vals[:, h // group], scale, allowed)
            out[r, h] = o[0]
            lse[h, r] = l_[0]
    return out, lse


def block_sparse_attention(q, k, v, block_map, tile_sizes, scale: float, tile: int = 64, heads=None, q_tiles=None):
    """Tile-granular block-sparse attention ([VSA] fastvideo_h3_vsa_bhsd op and
    FastVideoVSAImpl._forward_h3: q/k/v are in tile order with ``tile`` rows per
    tile, of which the first ``tile_sizes[c]`` are real; ``block_map[b, h, a, c]``
    says whether query tile a attends key tile c). Query row i of tile a is valid
    iff i % tile < tile_sizes[a]; invalid rows give O = 0, LSE = -inf (the op
    zero-pads rows outside the logical blocks). Keys allowed for a valid row of
    tile a: the valid rows of every key tile c with block_map[b, h, a, c].

    q [B, S, H, D], k/v [B, S, Hkv, D] with S = n_tiles * tile.
    ``heads`` / ``q_tiles`` restrict the computed (head, query tile) pairs;
    rows outside them are left at O = 0, LSE = -inf.
    Returns out [B, S, H, D] and lse [B, H, S] in float64.

    Pinned: full map == dense, brute force, token-mask equivalence.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    bmap = block_map if isinstance(block_map, np.ndarray) else block_map.detach().cpu().numpy()
    bmap = bmap.astype(bool)
    sizes = _ints(tile_sizes)
    bsz, seq, hq, _ = qf.shape
    hkv = kf.shape[2]
    group = hq // hkv
    n_tiles = sizes.size
    if seq != n_tiles * tile:
        raise ValueError("sequence length must equal n_tiles * tile")
    row_valid = (np.arange(seq) % tile) < np.repeat(sizes, tile)
    out = np.zeros((bsz, seq, hq, vf.shape[3]))
    lse = np.full((bsz, hq, seq), NEG_INF)
    heads = range(hq) if heads is None else heads
    for b in range(bsz):
        for h in heads:
            hk = h // group
            for a in (range(n_tiles) if q_tiles is None else q_tiles):
                qrows = np.arange(a * tile, a * tile + sizes[a])
                if qrows.size == 0:
                    continue
                key_tiles = np.nonzero(bmap[b, h, a])[0]
                keys = np.concatenate([np.arange(c * tile, (c + 1) * tile) for c in key_tiles]) if key_tiles.size else np.zeros(0, dtype=np.int64)
                keys = keys[row_valid[keys]]
                allowed = np.ones((qrows.size, keys.size), dtype=bool)
                o, l_ = _attend(qf[b, qrows, h], kf[b, keys, hk], vf[b, keys, hk], scale, allowed)
                out[b, qrows, h] = o
                lse[b, h, qrows] = l_
    return out, lse


def _gather_paged(kv_cache, plane: int, blk: np.ndarray, off: np.ndarray) -> np.ndarray:
    """Rows (blk[i], off[i]) of one cache plane as float64 [N, Hkv, D]."""
    if isinstance(kv_cache, np.ndarray):
        return kv_cache[plane][blk, off].astype(np.float64)
    import torch

    return kv_cache[plane][torch.from_numpy(blk), torch.from_numpy(off)].to(torch.float64).numpy()


def paged_kv_write(kv_cache, k, v, slot_mapping):
    """[ASC] AscendAttentionImpl.reshape_and_cache with AscendMetadata.slot_mapping:
    new token i's K and V rows go to the cache slot slot_mapping[i], i.e. block
    slot // block_size at offset slot % block_size (slot_to_block_offset).
    Reading: a negative slot marks a token that is not stored (padding).

    kv_cache [2, NB, BS, Hkv, D]; k, v [N, Hkv, D]. Returns a new cache (same
    dtype and container type); the input is not modified.

    Pinned: worked slot example, write-then-gather round trip, untouched slots.
    """
    slots = _ints(slot_mapping)
    bs = kv_cache.shape[2]
    keep = np.nonzero(slots >= 0)[0]
    blk, off = slot_to_block_offset(slots[keep], bs)
    if isinstance(kv_cache, np.ndarray):
        cache = kv_cache.copy()
        cache[0][blk, off] = np.asarray(k)[keep]
        cache[1][blk, off] = np.asarray(v)[keep]
        return cache
    import torch

    cache = kv_cache.clone()
    ki, bi, oi = torch.from_numpy(keep), torch.from_numpy(blk), torch.from_numpy(off)
    cache[0][bi, oi] = k[ki].to(cache.dtype)
    cache[1][bi, oi] = v[ki].to(cache.dtype)
    return cache


def paged_prefill_attention(q, kv_cache, block_tables, cu_seqlens_q, context_lens, scale: float, rows=None):
    """Multi-token attention over a paged cache ([ASC] _get_fia_params for
    PrefillCacheHit / ChunkedPrefill / SpecDecoding: keys and values come from
    the paged cache through ``block_table`` with ``actual_seq_lengths_kv`` =
    seq_lens, the queries are packed by cumulative query lengths). The cache
    already holds the sequence's new tokens (reshape_and_cache runs first), so
    sequence b has Lk = context_lens[b] keys, its Lq = cu_q[b+1] - cu_q[b]
    queries are the last Lq positions, and bottom-right causal applies: key j
    is visible to query i iff j <= i + (Lk - Lq). Key t of sequence b is cache
    row (block_tables[b, t // BS], t % BS).

    q [Tq, Hq, D]; kv_cache [2, NB, BS, Hkv, D]. Returns out [R, Hq, D] and
    lse [Hq, R] (float64) for the selected packed rows (all by default).

    Pinned: contiguous varlen equivalence, decode (Lq = 1) equivalence, chunk
    split identity, physical block relabelling.
    """
    qf = _f64(q)
    bt = _ints(block_tables)
    cu = _ints(cu_seqlens_q)
    ctx = _ints(context_lens)
    total_q, hq, _ = qf.shape
    bs = kv_cache.shape[2]
    hkv = kv_cache.shape[3]
    group = hq // hkv
    sel = np.arange(total_q) if rows is None else _ints(rows)
    out = np.zeros((sel.size, hq, kv_cache.shape[4]))
    lse = np.full((hq, sel.size), NEG_INF)
    for b in range(cu.size - 1):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        pick = np.nonzero((sel >= q0) & (sel < q1))[0]
        if pick.size == 0:
            continue
        lk = int(ctx[b])
        t = np.arange(lk)
        keys = _gather_paged(kv_cache, 0, bt[b, t // bs], t % bs)
        vals = _gather_paged(kv_cache, 1, bt[b, t // bs], t % bs)
        local = sel[pick] - q0
        allowed = _causal_allowed(local, q1 - q0, lk)
        for h in range(hq):
            o, l_ = _attend(qf[sel[pick], h], keys[:, h // group], vals[:, h // group], scale, allowed)
            out[pick, h] = o
            lse[h, pick] = l_
    return out, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint key subsets into the result over
    their union (the definition split over keys: each part carries its normalised
    output O_s and LSE_s; then LSE = ln sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s). Parts with LSE_s = -inf carry no keys.

    outs [P, ..., Dv], lses [P, ...]. Returns (out [..., Dv], lse [...]).
    Pinned: split/merge identity against the unsplit definition.
    """
    o = np.asarray(outs, dtype=np.float64)
    s = np.asarray(lses, dtype=np.float64)
    smax = s.max(axis=0)
    finite = np.isfinite(smax)
    smax_safe = np.where(finite, smax, 0.0)
    w = np.where(np.isfinite(s), np.exp(s - smax_safe[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, smax_safe + np.log(np.where(finite, tot, 1.0)), NEG_INF)
    coef = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    out = (coef[..., None] * o).sum(axis=0)
    return out, lse
