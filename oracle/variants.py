"""fp64 statement of the boundary variants of the attention forward: the
sliding-window decode, attention over a valid prefix of a padded batch
("packed padding") and attention under a key-padding mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each function states its rows and keys in the padded layout the caller holds
and reuses the plain softmax of one head (``attention._attend``); none of them
unpads, gathers or scans the way the kernels do.
"""

from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _attend, _causal_allowed, _f64, _ints


def sliding_window_decode_attention(q, kv_cache, block_tables, context_lens, scale: float, window: int, seqs=None):
    """Single-token decode with a sliding window ([ASC]
    AscendAttentionBackendImpl._forward_fia_slidingwindow: the decode-only
    branch passes the layer's sliding window as the fused kernel's
    ``pre_tokens`` with one query token per sequence and ``seq_lens`` keys).
    Reading: ``pre_tokens`` counts the tokens before the query that it may
    still see, so the query at position L - 1 attends keys
    ``max(0, L - 1 - window) <= t <= L - 1`` (window + 1 keys when the context
    is long enough). Cache addressing as in paged decode.

    q [S, Hq, D]; kv_cache [2, NB, BS, Hkv, D]; block_tables [S, MB].
    Returns out [R, Hq, D], lse [Hq, R] in float64.

    Pinned: window >= L - 1 is plain decode; window = 0 returns the last value
    row with LSE = scale * q.k_last; brute force on tiny inputs.
    """
    if window < 0:
        raise ValueError("window must be >= 0")
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
        first = max(0, length - 1 - int(window))
        t = np.arange(first, length)
        blk = bt[b, t // block_size]
        off = t % block_size
        if isinstance(kv_cache, np.ndarray):
            keys, vals = kv_cache[0][blk, off], kv_cache[1][blk, off]
        else:
            import torch

            bi, oi = torch.from_numpy(blk), torch.from_numpy(off)
            keys, vals = kv_cache[0][bi, oi], kv_cache[1][bi, oi]
        keys, vals = _f64(keys), _f64(vals)
        allowed = np.ones((1, t.size), dtype=bool)
        for h in range(hq):
            o, l_ = _attend(qf[b, h][None, :], keys[:, h // group], vals[:, h // group], scale, allowed)
            out[r, h] = o[0]
            lse[h, r] = l_[0]
    return out, lse


def padded_prefix_attention(q, k, v, q_lens, k_lens, scale: float, causal: bool):
    """Attention over the valid prefix of each batch entry of a padded batch
    ([VSA] FastVideoVSAImpl._fallback and forward_cuda with
    ``packed_padding``: the first ``q_length`` query rows and ``kv_length`` key
    rows are real; attention runs on those prefixes and the output rows past
    ``q_length`` are zero). Causal masking, when asked for, is bottom-right on
    the prefix lengths, as for varlen.

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D]; q_lens, k_lens [B] with
    0 <= q_lens[b] <= Sq, 0 <= k_lens[b] <= Sk.
    Returns out [B, Sq, Hq, D] and lse [Hq, B * Sq] (padded row order, -inf on
    pad rows) in float64.

    Pinned: equals packed varlen on the prefixes; full lengths equal dense
    attention; pad-row contents never matter; brute force on tiny inputs.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    ql, kl = _ints(q_lens), _ints(k_lens)
    bsz, sq, hq, _ = qf.shape
    hkv = kf.shape[2]
    group = hq // hkv
    out = np.zeros((bsz, sq, hq, vf.shape[3]))
    lse = np.full((hq, bsz * sq), NEG_INF)
    for b in range(bsz):
        lq, lk = int(ql[b]), int(kl[b])
        if not (0 <= lq <= sq and 0 <= lk <= kf.shape[1]):
            raise ValueError("prefix lengths out of range")
        if causal:
            allowed = _causal_allowed(np.arange(lq), lq, lk)
        else:
            allowed = np.ones((lq, lk), dtype=bool)
        for h in range(hq):
            o, l_ = _attend(qf[b, :lq, h], kf[b, :lk, h // group], vf[b, :lk, h // group], scale, allowed)
            out[b, :lq, h] = o
            lse[h, b * sq:b * sq + lq] = l_
    return out, lse


def masked_attention(q, k, v, key_mask, scale: float, causal: bool, mask_queries: bool):
    """Attention under a 2-D key-padding mask ([FA]
    FlashAttentionImpl._forward_varlen_masked: ``attention_mask`` is
    ``(batch, seq_len)`` with nonzero = real token).

    * ``mask_queries`` (self-attention with equal query and key lengths): the
      mask also selects the query rows. The real tokens of each batch entry,
      in their original order, form one document; its query rows attend its
      keys, and the rows of padding tokens come back as zeros.
    * otherwise (cross-attention): the mask covers keys only and every query
      row attends the real keys of its batch entry.

    Causal masking, when asked for, is bottom-right on the real-token counts
    (counted among real tokens only), as for varlen.

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D], key_mask [B, Sk].
    Returns out [B, Sq, Hq, D] and lse [Hq, B * Sq] (-inf on dropped rows).

    Pinned: an all-ones mask is dense attention; a prefix mask is the padded
    prefix attention; brute force with holes on tiny inputs; cross-attention
    equals packed varlen with uniform query documents.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    mask = np.asarray(key_mask).astype(bool)
    bsz, sq, hq, _ = qf.shape
    sk, hkv = kf.shape[1], kf.shape[2]
    if mask.shape != (bsz, sk):
        raise ValueError("key_mask must be [batch, seq_len_k]")
    if mask_queries and sq != sk:
        raise ValueError("a mask over the queries needs equal query and key lengths")
    group = hq // hkv
    out = np.zeros((bsz, sq, hq, vf.shape[3]))
    lse = np.full((hq, bsz * sq), NEG_INF)
    for b in range(bsz):
        keys = np.nonzero(mask[b])[0]
        rows = keys if mask_queries else np.arange(sq)
        lq, lk = rows.size, keys.size
        if causal:
            allowed = _causal_allowed(np.arange(lq), lq, lk)
        else:
            allowed = np.ones((lq, lk), dtype=bool)
        for h in range(hq):
            o, l_ = _attend(qf[b, rows, h], kf[b, keys, h // group], vf[b, keys, h // group], scale, allowed)
            out[b, rows, h] = o
            lse[h, b * sq + rows] = l_
    return out, lse
