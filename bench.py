"""Attention forward throughput on one MI355X.

Default run (no flags): the DiT-style dense self-attention workload (batch 2 x
seq 4096 packed as uniform varlen, 24 heads, head_dim 128, non-causal, fp32 LSE)
is the headline line (TFLOP/s). The causal GQA varlen prefill, paged decode
and video block-sparse workloads are timed too and reported under "secondary".
Inputs are seeded synthetic bf16 tensors already resident in HBM when the
timed region starts; each step is one call of the entry point (every kernel it
launches). Timing uses HIP events on the stream the kernels run on.

Prints ONE JSON line. `--gpus N` with N > 1 is refused: this library runs on
one GPU and nothing here shards across devices.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import softmax_attention_varlen_amd as sav  # noqa: E402
import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E

# HBM traffic of each workload's main kernel, per launch: rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one pass each), scaled by what
# the same counters read for a plain 1 GiB device copy (bench.py --only copy):
# FETCH_SIZE reports half the bytes read, WRITE_SIZE all the bytes written.
# A record holds only while the kernel sources it was taken from are unchanged:
# the sha256 of their code (comments and blank lines stripped) is stored with
# it and a mismatch reports null.
FETCH_SCALE = 2.0
WRITE_SCALE = 1.0
CSRC = os.path.join(ROOT, "softmax_attention_varlen_amd", "csrc")
_PREFILL_SRC = ["prefill_pipe.hip", "pipe.hpp", "attn_common.hpp", "key_rows.hpp"]
_DECODE_SRC = ["paged_decode_stream.hip", "attn_common.hpp"]
_SPARSE_SRC = ["block_sparse_pipe.hip", "pipe.hpp", "attn_common.hpp"]
_VARLEN_SRC = ["varlen_fwd.hip", "attn_common.hpp", "key_rows.hpp"]
_SPARSE_GEN_SRC = ["block_sparse.hip", "attn_common.hpp"]
TRAFFIC = {
    "tiny": {"kernel": "prefill_pipe_kernel<64,false,false,4,true>", "fetch_kib": 289.4, "write_kib": 132.1,
             "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "dense_d64": {"kernel": "prefill_pipe_kernel<64,false,false,4,true>", "fetch_kib": 36967.4, "write_kib": 25344.0,
                  "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "dense_d96": {"kernel": "prefill_pipe_kernel<96,false,false,4,true>", "fetch_kib": 73826.7, "write_kib": 37663.8,
                  "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "dense_d192": {"kernel": "prefill_pipe_kernel<192,false,false,4,true>", "fetch_kib": 110841.0,
                   "write_kib": 74496.2, "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "dense_d256": {"kernel": "prefill_pipe_kernel<256,false,false,4,true>", "fetch_kib": 149700.3,
                   "write_kib": 116571.4, "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "sparse_d64": {"kernel": "block_sparse_fwd_kernel<64>", "fetch_kib": 322495.8, "write_kib": 24576.7,
                   "sources": _SPARSE_GEN_SRC, "sha256": "44f3ef3fc81f11ed"},
    "sparse_d96": {"kernel": "block_sparse_pipe_kernel<96>", "fetch_kib": 263609.2, "write_kib": 36864.7,
                   "sources": _SPARSE_SRC, "sha256": "de8b74545248f2d3"},
    "sparse_d192": {"kernel": "block_sparse_pipe_kernel<192>", "fetch_kib": 651084.4, "write_kib": 73728.0,
                    "sources": _SPARSE_SRC, "sha256": "de8b74545248f2d3"},
    "sparse_d256": {"kernel": "block_sparse_pipe_kernel<256>", "fetch_kib": 969442.6, "write_kib": 98304.1,
                    "sources": _SPARSE_SRC, "sha256": "de8b74545248f2d3"},
    "decode_d96": {"kernel": "paged_decode_stream_kernel<96>", "fetch_kib": 1962417.4, "write_kib": 2285.3,
                   "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "decode_d192": {"kernel": "paged_decode_stream_kernel<192>", "fetch_kib": 3658877.8, "write_kib": 2901.3,
                    "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "decode_d64": {"kernel": "paged_decode_stream_kernel<64>", "fetch_kib": 1226021.6, "write_kib": 2602.2,
                   "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "decode_d256": {"kernel": "paged_decode_stream_kernel<256>", "fetch_kib": 4878550.5, "write_kib": 3862.3,
                    "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "dense": {"kernel": "prefill_pipe_kernel<128,false,false,4,true>", "fetch_kib": 73859.3, "write_kib": 49939.0,
              "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "causal": {"kernel": "prefill_pipe_kernel<128,true,false,4,true>", "fetch_kib": 111911.1, "write_kib": 142486.2,
               "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "paged": {"kernel": "paged_decode_stream_kernel<128>", "fetch_kib": 2443505.8, "write_kib": 3042.5,
              "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "sparse": {"kernel": "block_sparse_pipe_kernel<128>", "fetch_kib": 259852.9, "write_kib": 49920.8,
               "sources": _SPARSE_SRC, "sha256": "de8b74545248f2d3"},
    "paged_prefill": {"kernel": "prefill_pipe_kernel<128,true,true,8,false>", "fetch_kib": 708951.2,
                      "write_kib": 87202.2, "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "spec": {"kernel": "paged_decode_stream_kernel<128>", "fetch_kib": 2445743.6, "write_kib": 12164.9,
             "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "h3": {"kernel": "block_sparse_pipe_kernel<128>", "fetch_kib": 477754.3, "write_kib": 51488.2,
           "sources": _SPARSE_SRC, "sha256": "de8b74545248f2d3"},
    "swa": {"kernel": "paged_decode_stream_kernel<128>", "fetch_kib": 531385.8, "write_kib": 3081.3,
            "sources": _DECODE_SRC, "sha256": "867349d6b3aa0d47"},
    "masked": {"kernel": "prefill_pipe_kernel<128,false,false,4,true>", "fetch_kib": 28947.8, "write_kib": 50085.1,
               "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
    "padded": {"kernel": "prefill_pipe_kernel<128,false,false,4,true>", "fetch_kib": 107215.3, "write_kib": 66236.4,
               "sources": _PREFILL_SRC, "sha256": "0fdaca010aad7acb"},
}


def code_only(text: str) -> str:
    """C/C++ source without comments and blank lines (string literals kept), so
    that editing a comment does not void a measurement of the code."""
    out, i, n, in_str = [], 0, len(text), False
    while i < n:
        ch = text[i]
        if in_str:
            out.append(ch)
            if ch == "\\" and i + 1 < n:
                out.append(text[i + 1])
                i += 2
                continue
            if ch == '"':
                in_str = False
            i += 1
        elif ch == '"':
            in_str = True
            out.append(ch)
            i += 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def sources_sha256(files) -> str:
    import hashlib
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            m.update(code_only(fh.read()).encode())
    return m.hexdigest()[:16]


def traffic_bytes(workload: str):
    """Measured HBM bytes per launch of the workload's main kernel, or None when
    none was measured or the kernel sources changed since the counters were taken."""
    rec = TRAFFIC.get(workload)
    if rec is None or "fetch_kib" not in rec:
        return None
    if sources_sha256(rec["sources"]) != rec["sha256"]:
        return None
    return int(round((rec["fetch_kib"] * FETCH_SCALE + rec["write_kib"] * WRITE_SCALE) * 1024))


def roofline(workload: str, bound: str, achieved: float, work: float):
    """Roofline object: achieved rate of the step against the MI355X peak."""
    peak, unit = (PEAK_BF16_TFLOPS, "TFLOP/s") if bound == "mfma" else (PEAK_HBM_GBPS, "GB/s")
    rec = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": traffic_bytes(workload),
           "kernel": TRAFFIC[workload]["kernel"]}
    rec["algorithmic_gflop_per_launch" if bound == "mfma" else "algorithmic_gb_per_launch"] = round(work / 1e9, 4)
    return rec


# ----------------------------------------------------------------------------
# algorithmic work (only what the method must do)
# ----------------------------------------------------------------------------

def varlen_flops(case) -> float:
    """4 * D flops per allowed (query, key) pair and query head (QK^T and PV)."""
    lq = np.diff(case.cu_seqlens_q).astype(np.int64)
    lk = np.diff(case.cu_seqlens_k).astype(np.int64)
    pairs = 0
    for a, b in zip(lq, lk):
        if case.causal:
            i = np.arange(a)
            pairs += int(np.clip(i + (b - a) + 1, 0, b).sum())
        else:
            pairs += int(a * b)
    return 4.0 * case.head_dim * case.num_heads * pairs


def paged_bytes(case) -> float:
    """K and V bytes of every context token, plus Q, O, block tables and lengths."""
    kv = float(case.context_lens.astype(np.int64).sum()) * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2.0 * case.num_seqs * case.num_heads * case.head_dim * 2
    return kv + qo + case.block_tables.nbytes + case.context_lens.nbytes


def window_bytes(case, window: int) -> float:
    """K and V bytes of the keys inside each sequence's window, plus Q, O,
    block tables and lengths."""
    keys = np.minimum(case.context_lens.astype(np.int64), window + 1).sum()
    kv = float(keys) * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2.0 * case.num_seqs * case.num_heads * case.head_dim * 2
    return kv + qo + case.block_tables.nbytes + case.context_lens.nbytes


def padded_flops(case, q_rows, k_rows) -> float:
    """4 * D flops per visible (query, key) pair and query head: q_rows[b]
    real query rows attend k_rows[b] real keys (non-causal)."""
    pairs = float((np.asarray(q_rows, dtype=np.int64) * np.asarray(k_rows, dtype=np.int64)).sum())
    return 4.0 * case.head_dim * case.num_heads * pairs


def paged_prefill_flops(case) -> float:
    """4 * D flops per visible (query, key) pair and query head, bottom-right causal."""
    lq = np.diff(case.cu_seqlens_q).astype(np.int64)
    lk = case.context_lens.astype(np.int64)
    pairs = 0
    for a, b in zip(lq, lk):
        i = np.arange(a)
        pairs += int(np.clip(i + (b - a) + 1, 0, b).sum())
    return 4.0 * case.head_dim * case.num_heads * pairs


def paged_prefill_bytes(case) -> float:
    """K and V bytes of every context token, plus Q, O, tables and lengths."""
    kv = float(case.context_lens.astype(np.int64).sum()) * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2.0 * case.q.shape[0] * case.num_heads * case.head_dim * 2
    return kv + qo + case.block_tables.nbytes + case.context_lens.nbytes + case.cu_seqlens_q.nbytes


def sparse_flops(bmap: np.ndarray, sizes: np.ndarray, head_dim: int) -> float:
    """4 * D flops per (valid query row, valid key row) pair of every kept tile pair."""
    sz = sizes.astype(np.float64)
    per_pair = np.outer(sz, sz)  # [nQ, nK] valid row pairs
    return 4.0 * head_dim * float((bmap.astype(np.float64) * per_pair[None, None]).sum())


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------

CLOCK_WARMUP_MS = 200.0  # set from --clock-warmup-ms


class StepTime:
    """Milliseconds per step: the mean over the timed window and the median and
    minimum of the individual steps (one HIP event between consecutive steps)."""

    def __init__(self, per_step, mean):
        self.mean = mean
        self.median = float(np.median(per_step))
        self.min = float(np.min(per_step))

    def stats(self):
        return {"ms_median": round(self.median, 5), "ms_min": round(self.min, 5)}


def time_steps(step, steps: int, warmup: int) -> StepTime:
    """Milliseconds per step over `steps` timed steps (HIP events on the stream
    the kernels run on).

    Before the `warmup` untimed steps, the step is repeated for CLOCK_WARMUP_MS
    of wall time: under sustained load the GPU's clocks ramp for tens of
    milliseconds (the first 20-step window after 5 warm-up steps runs 15-17 %
    slower than the steady state), and the steady state is what a serving or
    training loop sees."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < CLOCK_WARMUP_MS:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return StepTime(per_step, ev[0].elapsed_time(ev[-1]) / steps)


def bench_varlen(case, steps, warmup, with_lse=True, operands="randn"):
    """operands: "randn" (the workload's seeded inputs) or "ones" / "zeros"
    (the same shapes filled with one constant, for the power measurement of
    --only dense_const: the kernel runs the same instructions either way)."""
    dev = torch.device("cuda")
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    if operands != "randn":
        fill = torch.ones_like if operands == "ones" else torch.zeros_like
        q, k, v = fill(q), fill(k), fill(v)
    cu_q = torch.from_numpy(case.cu_seqlens_q).to(dev)
    cu_k = torch.from_numpy(case.cu_seqlens_k).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.num_heads, q.shape[0]), dtype=torch.float32, device=dev) if with_lse else None

    def step():
        sav.attn_varlen_fwd(q, k, v, cu_q, cu_k, case.max_seqlen_q, case.max_seqlen_k, case.scale, case.causal,
                            out=out, lse=lse)

    ms = time_steps(step, steps, warmup)
    return ms, varlen_flops(case)


def bench_paged(case, steps, warmup, window=None):
    dev = torch.device("cuda")
    q, kv = case.q.to(dev), case.kv_cache.to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.num_heads, case.num_seqs), dtype=torch.float32, device=dev)
    ws = torch.empty(sav.attn_paged_decode_workspace_size(case.num_seqs, case.num_heads, case.num_kv_heads,
                                                          case.head_dim, case.max_context_len),
                     dtype=torch.uint8, device=dev)

    def step():
        sav.attn_paged_decode(q, kv, bt, cl, case.max_context_len, case.scale, out=out, lse=lse, workspace=ws,
                              window=window)

    ms = time_steps(step, steps, warmup)
    del kv
    return ms, (paged_bytes(case) if window is None else window_bytes(case, window))


def bench_padded(case, steps, warmup, masked: bool):
    """attn_masked_fwd (key mask, cross-attention) or attn_padded_fwd (valid
    prefixes): the whole entry call, its gathers and fills included."""
    dev = torch.device("cuda")
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.num_heads, q.shape[0] * q.shape[1]), dtype=torch.float32, device=dev)
    if masked:
        mask = torch.from_numpy(case.key_mask).to(dev)
        ws = torch.empty(sav.attn_masked_fwd_workspace_size(q.shape[0], q.shape[1], k.shape[1], case.num_heads,
                                                            case.num_kv_heads, case.head_dim, False),
                         dtype=torch.uint8, device=dev)

        def step():
            sav.attn_masked_fwd(q, k, v, mask, case.scale, case.causal, mask_queries=False, out=out, lse=lse,
                                workspace=ws)

        flops = padded_flops(case, np.full(q.shape[0], q.shape[1]), case.key_mask.sum(1))
    else:
        ql = torch.from_numpy(case.q_lens).to(dev)
        kl = torch.from_numpy(case.k_lens).to(dev)
        ws = torch.empty(sav.attn_padded_fwd_workspace_size(q.shape[0]), dtype=torch.uint8, device=dev)

        def step():
            sav.attn_padded_fwd(q, k, v, ql, kl, case.scale, case.causal, out=out, lse=lse, workspace=ws)

        flops = padded_flops(case, case.q_lens, case.k_lens)
    return time_steps(step, steps, warmup), flops


def bench_paged_prefill(case, steps, warmup):
    dev = torch.device("cuda")
    q, kv = case.q.to(dev), case.kv_cache.to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cu = torch.from_numpy(case.cu_seqlens_q).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.num_heads, q.shape[0]), dtype=torch.float32, device=dev)

    def step():
        sav.attn_paged_prefill(q, kv, bt, cu, cl, case.max_seqlen_q, case.max_context_len, case.scale, out=out,
                               lse=lse)

    ms = time_steps(step, steps, warmup)
    del kv
    return ms


def bench_kv_write(case, steps, warmup):
    """Store every sequence's new tokens (the last Lq positions) into the cache."""
    dev = torch.device("cuda")
    kv = case.kv_cache.to(dev)
    n = case.q.shape[0]
    k_new = workloads.randn_bf16((n, case.num_kv_heads, case.head_dim), 1000 * case.seed + 4).to(dev)
    v_new = workloads.randn_bf16((n, case.num_kv_heads, case.head_dim), 1000 * case.seed + 5).to(dev)
    lq = np.diff(case.cu_seqlens_q)
    slots = np.concatenate([case.block_tables[b, t // 128].astype(np.int64) * 128 + t % 128
                            for b in range(case.batch)
                            for t in [np.arange(case.context_lens[b] - lq[b], case.context_lens[b])]])
    sl = torch.from_numpy(slots.astype(np.int32)).to(dev)
    ms = time_steps(lambda: sav.attn_paged_kv_write(k_new, v_new, sl, kv), steps, warmup).mean
    del kv
    # bf16 K and V rows read once and written once, plus the int32 slot of each token
    return ms, 2 * 2 * 2.0 * n * case.num_kv_heads * case.head_dim + 4 * n


def bench_h3(case, steps, warmup):
    """H3 layout: prefix + video tiles and the H3 map built in the library's
    kernels; the block-sparse call is the timed step, the map build is reported."""
    dev = torch.device("cuda")
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    segs = case.extra["prefix_segments"]
    prep = sav.vsa_h3_prepare(q, k, v, segs, case.video_shape, case.topk, case.scale)
    qt, kt, vt, bmap, sizes = prep["q"], prep["k"], prep["v"], prep["block_map"], prep["tile_sizes"]
    out = torch.empty_like(qt)
    lse = torch.empty((qt.shape[0], case.num_heads, qt.shape[1]), dtype=torch.float32, device=dev)
    ws = torch.empty(sav.attn_block_sparse_workspace_size(qt.shape[0], case.num_heads, sizes.numel()),
                     dtype=torch.uint8, device=dev)

    def step():
        sav.attn_block_sparse_fwd(qt, kt, vt, bmap, sizes, case.scale, out=out, lse=lse, workspace=ws)

    ms = time_steps(step, steps, warmup)
    flops = sparse_flops(bmap.cpu().numpy(), sizes.cpu().numpy(), case.head_dim)
    prep_ms = time_steps(lambda: sav.vsa_h3_prepare(q, k, v, segs, case.video_shape, case.topk, case.scale), steps,
                         warmup).mean
    return ms, flops, prep_ms


def bench_sparse(case, steps, warmup):
    """Tile order, pooled-score top-k map and the block-sparse call all run in the
    library's kernels; only the block-sparse call is in the timed step."""
    dev = torch.device("cuda")
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)  # raster inputs, resident before any timing
    prep = sav.vsa_prepare(q, k, v, case.video_shape, case.tile_shape, case.topk, case.scale)
    qt, kt, vt, bmap, sizes = prep["q"], prep["k"], prep["v"], prep["block_map"], prep["tile_sizes"]
    out = torch.empty_like(qt)
    lse = torch.empty((qt.shape[0], case.num_heads, qt.shape[1]), dtype=torch.float32, device=dev)
    ws = torch.empty(sav.attn_block_sparse_workspace_size(qt.shape[0], case.num_heads, sizes.numel()),
                     dtype=torch.uint8, device=dev)

    def step():
        sav.attn_block_sparse_fwd(qt, kt, vt, bmap, sizes, case.scale, out=out, lse=lse, workspace=ws)

    ms = time_steps(step, steps, warmup)
    flops = sparse_flops(bmap.cpu().numpy(), sizes.cpu().numpy(), case.head_dim)
    prep_ms = time_steps(lambda: sav.vsa_prepare(q, k, v, case.video_shape, case.tile_shape, case.topk, case.scale),
                         steps, warmup).mean
    # the gate branch on the same tiles, with a synthetic gate (a trained one
    # comes from a checkpoint's projection)
    gate = workloads.randn_bf16(tuple(qt.shape), 1000 * case.seed + 6).to(dev)
    cws = torch.empty(sav.attn_vsa_compressed_workspace_size(qt.shape[0], case.num_heads, kt.shape[2],
                                                             sizes.numel(), case.head_dim), dtype=torch.uint8,
                      device=dev)
    comp_ms = time_steps(lambda: sav.attn_vsa_compressed_add(qt, kt, vt, sizes, gate, case.scale, out, workspace=cws),
                         steps, warmup).mean
    host = {"q": qt.cpu(), "k": kt.cpu(), "v": vt.cpu(), "block_map": bmap.cpu().numpy(),
            "tile_sizes": sizes.cpu().numpy()}
    return ms, flops, prep_ms, comp_ms, host


def bench_head_dims(steps, warmup):
    """The head dims other than 128 that the pages list (D = 64, 96, 192,
    256): dense non-causal prefill of 2 x 4096 rows with 24 heads, decode over
    workload 4's 64 contexts (32 query / 8 kv heads, a random permutation of
    cache blocks), and block-sparse attention on workload 5's tile grid with
    seeded random top-32 maps; inputs drawn on the device. Returns (workload
    name, kind, StepTime, algorithmic work, bound) per line."""
    dev = torch.device("cuda")
    rows = []
    for d in (64, 96, 192, 256):
        n, h = 2 * 4096, 24
        q, k, v = (workloads.randn_bf16_on((n, h, d), 7700 + 10 * d + j, dev) for j in range(3))
        cu = torch.tensor([0, 4096, 8192], dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((h, n), dtype=torch.float32, device=dev)
        t = time_steps(lambda: sav.attn_varlen_fwd(q, k, v, cu, cu, 4096, 4096, d ** -0.5, False, out=out, lse=lse),
                       steps, warmup)
        rows.append((f"dit-dense-b2-s4096-h24-d{d}", f"dense_d{d}", t, 4.0 * 2 * h * d * 4096 * 4096, "mfma"))
        del q, k, v, out
    ctx = workloads.config4_lengths()
    nblk = [(int(c) + 127) // 128 for c in ctx]
    perm = np.random.default_rng(4).permutation(sum(nblk))
    tables = np.full((len(ctx), max(nblk)), -1, dtype=np.int32)
    o = 0
    for i, nb in enumerate(nblk):
        tables[i, :nb] = perm[o:o + nb]
        o += nb
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(dev)
    for d in (64, 96, 192, 256):
        cache = workloads.randn_bf16_on((2, sum(nblk), 128, 8, d), 7800 + d, dev)
        q = workloads.randn_bf16_on((len(ctx), 32, d), 7801 + d, dev)
        out = torch.empty_like(q)
        ws = torch.empty(max(sav.attn_paged_decode_workspace_size(len(ctx), 32, 8, d, int(max(ctx))), 1),
                         dtype=torch.uint8, device=dev)
        t = time_steps(lambda: sav.attn_paged_decode(q, cache, bt, cl, int(max(ctx)), d ** -0.5, out=out,
                                                     workspace=ws), steps, warmup)
        # K and V of every context token, plus Q, O, tables and lengths
        nbytes = float(sum(int(c) for c in ctx)) * 8 * d * 2 * 2 + 2.0 * len(ctx) * 32 * d * 2 + tables.nbytes + 256
        rows.append((f"paged-decode-64seq-ctx1k-32k-h32kv8-d{d}", f"decode_d{d}", t, nbytes, "hbm"))
        del cache, q, out, ws
        torch.cuda.empty_cache()
    # block-sparse on workload 5's tile grid (256 full tiles, 12 heads), each
    # query tile keeping 32 key tiles drawn at random (seeded)
    nt, h = 256, 12
    rng = np.random.default_rng(5)
    kept = np.zeros((1, h, nt, nt), dtype=np.uint8)
    for hh in range(h):
        for a in range(nt):
            kept[0, hh, a, rng.choice(nt, 32, replace=False)] = 1
    bmap = torch.from_numpy(kept).to(dev)
    sizes = torch.full((nt,), 64, dtype=torch.int32, device=dev)
    ws = torch.empty(sav.attn_block_sparse_workspace_size(1, h, nt), dtype=torch.uint8, device=dev)
    for d in (64, 96, 192, 256):
        q, k, v = (workloads.randn_bf16_on((1, nt * 64, h, d), 7900 + 10 * d + j, dev) for j in range(3))
        out = torch.empty_like(q)
        t = time_steps(lambda: sav.attn_block_sparse_fwd(q, k, v, bmap, sizes, d ** -0.5, out=out, workspace=ws),
                       steps, warmup)
        flops = sparse_flops(kept, sizes.cpu().numpy(), d)
        rows.append((f"block-sparse-256tiles-h12-top32-d{d}", f"sparse_d{d}", t, flops, "mfma"))
        del q, k, v, out
    return rows


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle timed on a bounded sample of each workload
# ----------------------------------------------------------------------------

def _oracle_threads():
    from threadpoolctl import threadpool_info

    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def _growing_sample(run, start, limit, budget_s):
    """Double the sample size n (from start, at most limit) until run(n) takes
    budget_s; returns (n, seconds of the last run)."""
    n = start
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= limit:
            return n, dt
        n = min(2 * n, limit)


def gemm_reference(steps, warmup, n=8192, kinds=("randn", "constant")):
    """Context for the MFMA roofline: the vendor's bf16 GEMM (torch.mm, which
    runs hipBLASLt) on square n^3 products, timed like the workloads. On
    seeded N(0,1) operands (the workloads' value distribution) and on constant
    operands: the two run the same instructions, and the gap between them is
    the clock the chip gives up for operand bit toggling. Not part of any
    workload's step."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(8192)
    out = {"kind": "torch.mm bf16 (hipBLASLt), m = n = k = %d" % n, "unit": "TFLOP/s"}
    makers = {"randn": lambda: torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g),
              "constant": lambda: torch.ones(n, n, device=dev, dtype=torch.bfloat16)}
    for name in kinds:
        a, b = makers[name](), makers[name]()
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        t = time_steps(lambda: torch.mm(a, b, out=c), steps, warmup)
        out[name] = round(2.0 * n ** 3 / (t.mean * 1e-3) / 1e12, 1)
        del a, b, c
    if "randn" in out:
        out["randn_frac_of_peak"] = round(out["randn"] / PEAK_BF16_TFLOPS, 4)
    torch.cuda.empty_cache()
    return out


def mfma_stream_reference(steps, warmup, iters=4096, kinds=("randn", "constant")):
    """The sustained rate of the attention kernels' MFMA (32x32x16 bf16) in a
    plain stream on operands held in registers (the calibration kernel in
    softmax_attention_varlen_amd/calib), two 4-wave workgroups per CU, on
    seeded N(0,1) operands and on constant ones. None when that library is not
    built."""
    import ctypes

    path = os.path.join(ROOT, "softmax_attention_varlen_amd", "libattn_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.attn_calib_mfma_stream
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    dev = torch.device("cuda")
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    threads = wgs * 256
    flops = float(wgs) * 4 * iters * 8 * 32768  # 4 waves, iters x 8 MFMAs each
    sink = torch.empty(threads, device=dev, dtype=torch.float32)
    g = torch.Generator(device=dev)
    g.manual_seed(32)
    out = {"kind": "v_mfma_f32_32x32x16_bf16 stream, operands in registers, %d workgroups of 4 waves" % wgs,
           "unit": "TFLOP/s"}
    for name in kinds:
        shape = (16 * threads * 8,)
        ops = (torch.randn(shape, device=dev, dtype=torch.bfloat16, generator=g) if name == "randn"
               else torch.ones(shape, device=dev, dtype=torch.bfloat16))
        stream = torch.cuda.current_stream().cuda_stream

        def step():
            rc = fn(ops.data_ptr(), sink.data_ptr(), wgs, iters, stream)
            if rc != 0:
                raise RuntimeError(f"calibration kernel launch failed ({rc})")

        t = time_steps(step, steps, warmup)
        out[name] = round(flops / (t.mean * 1e-3) / 1e12, 1)
        del ops
    if "randn" in out:
        out["randn_frac_of_peak"] = round(out["randn"] / PEAK_BF16_TFLOPS, 4)
    return out


def cpu_baseline_varlen(case, budget_s):
    """The first n query rows of every document (all heads), n doubling until the
    oracle takes budget_s; rate in the GPU line's unit (algorithmic flops of the
    sampled rows: under the causal mask only their visible keys count)."""
    import oracle  # test infrastructure: used only for this reported baseline

    lq = np.diff(case.cu_seqlens_q).astype(np.int64)
    lk = np.diff(case.cu_seqlens_k).astype(np.int64)

    def local_rows(n, b):
        # n rows spread evenly over the document, so that under the causal
        # mask the sample sees the workload's mix of short and long rows
        return np.unique(np.linspace(0, lq[b] - 1, min(n, lq[b])).round().astype(np.int64)) if lq[b] else \
            np.zeros(0, dtype=np.int64)

    def run(n):
        rows = np.concatenate([case.cu_seqlens_q[b] + local_rows(n, b) for b in range(case.batch)])
        oracle.varlen_attention(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k, case.scale,
                                case.causal, rows=rows)

    n, dt = _growing_sample(run, 64, int(lq.max()), budget_s)
    whole = n >= int(lq.max())
    reps = 1
    if whole and dt < 0.25 * budget_s:  # a small workload: repeat it for a measurable time
        reps = max(1, int(0.25 * budget_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(n)
        dt = (time.perf_counter() - t0) / reps
    pairs = 0
    for b in range(case.batch):
        i = local_rows(n, b)
        pairs += int(np.clip(i + (lk[b] - lq[b]) + 1, 0, lk[b]).sum()) if case.causal else int(i.size * lk[b])
    flops = 4.0 * case.head_dim * case.num_heads * pairs
    sample = ("the whole workload" + (f" (mean of {reps} runs)" if reps > 1 else "") if whole
              else f"{n} query rows spread over each of the {case.batch} documents") + \
        f", all {case.num_heads} heads, fp64 numpy ({dt:.2f} s)"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def cpu_baseline_paged(case, budget_s):
    """Whole sequences, one at a time in order, until the oracle takes budget_s;
    rate in GB/s of the same algorithmic bytes the GPU line counts."""
    import oracle  # test infrastructure: used only for this reported baseline

    t0 = time.perf_counter()
    done = 0
    while done < case.num_seqs and time.perf_counter() - t0 < budget_s:
        oracle.paged_decode_attention(case.q, case.kv_cache, case.block_tables, case.context_lens, case.scale,
                                      seqs=[done])
        done += 1
    dt = time.perf_counter() - t0
    ctx = case.context_lens[:done].astype(np.int64)
    nbytes = float(ctx.sum()) * case.num_kv_heads * case.head_dim * 2 * 2 + \
        2.0 * done * case.num_heads * case.head_dim * 2 + 4.0 * done * (case.block_tables.shape[1] + 1)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"the first {done} of {case.num_seqs} sequences ({int(ctx.sum())} context tokens), one at a "
                      f"time, all {case.num_heads} heads, fp64 numpy ({dt:.1f} s)",
            "seconds": round(dt, 2)}


def cpu_baseline_sparse(case, host, budget_s):
    """The first n query tiles of every head (the GPU's own tile-order inputs
    and map), n doubling until the oracle takes budget_s; rate in TFLOP/s of
    the kept tile pairs of those tiles."""
    import oracle  # test infrastructure: used only for this reported baseline

    sizes, bmap = host["tile_sizes"], host["block_map"]
    nt = sizes.size

    def run(n):
        oracle.block_sparse_attention(host["q"], host["k"], host["v"], bmap, sizes, case.scale,
                                      q_tiles=list(range(n)))

    n, dt = _growing_sample(run, 4, nt, budget_s)
    sz = sizes.astype(np.float64)
    flops = 4.0 * case.head_dim * float((bmap[:, :, :n].astype(np.float64) * np.outer(sz[:n], sz)[None, None]).sum())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"the first {n} of {nt} query tiles of all {case.num_heads} heads with their kept key tiles, "
                      f"fp64 numpy ({dt:.1f} s)",
            "seconds": round(dt, 2)}


def main():
    global CLOCK_WARMUP_MS
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["dense", "tiny", "causal", "paged", "sparse", "h3", "paged_prefill", "spec", "swa",
                                       "masked", "padded", "copy", "head_dims", "gemm_ref", "gemm_ref_const",
                                       "mfma_stream", "mfma_stream_const", "dense_const", "causal_const",
                                       "sparse_const"],
                    default=None,
                    help="time one workload only (for profiling runs); 'copy' times a plain 1 GiB device "
                         "copy, the reference that scales the HBM byte counters; 'head_dims' times the head "
                         "dims other than 128; 'gemm_ref' / 'gemm_ref_const' time the vendor bf16 GEMM on "
                         "N(0,1) / constant operands; 'mfma_stream' / 'mfma_stream_const' the MFMA "
                         "calibration kernel on the same two; 'dense_const' / 'causal_const' / 'sparse_const' "
                         "workloads 2, 3 and 5 on constant inputs")
    ap.add_argument("--clock-warmup-ms", type=float, default=CLOCK_WARMUP_MS,
                    help="repeat each workload's step for this long before its warm-up steps (0: off)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip timing the vendor bf16 GEMM that puts the MFMA roofline in context")
    ap.add_argument("--cpu-budget-s", type=float, default=4.0,
                    help="seconds of fp64 oracle work per workload for the cpu baselines (workloads 1-5)")
    args = ap.parse_args()
    CLOCK_WARMUP_MS = max(0.0, args.clock_warmup_ms)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path exists)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    sav.load_library()
    torch.cuda.set_device(0)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        ms = time_steps(lambda: dst.copy_(src), args.steps, args.warmup).mean
        print(json.dumps({"metric": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "ms": round(ms, 5), "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}))
        return
    if args.only in ("gemm_ref", "gemm_ref_const"):
        ref = gemm_reference(args.steps, args.warmup, kinds=("randn",) if args.only == "gemm_ref" else ("constant",))
        print(json.dumps({"metric": "vendor bf16 GEMM", **ref}))
        return
    if args.only in ("dense_const", "causal_const"):
        # workload 2 (or 3) with all-ones, then all-zero Q, K and V: the same
        # instructions as on N(0,1) inputs, less operand bit toggling
        case = workloads.config2() if args.only == "dense_const" else workloads.config3()
        rec = {"metric": "attention on constant inputs", "workload": case.name, "unit": "TFLOP/s"}
        for operands in ("ones", "zeros"):
            t, flops = bench_varlen(case, args.steps, args.warmup, operands=operands)
            rec[operands] = round(flops / (t.mean * 1e-3) / 1e12, 1)
            rec[operands + "_ms"] = round(t.mean, 5)
        print(json.dumps(rec))
        return
    if args.only == "sparse_const":
        # workload 5's block-sparse call with the map built from its N(0,1)
        # inputs, then run on all-ones tile-order Q, K and V (same items, same
        # kept tiles, same instructions)
        case = workloads.config5()
        dev = torch.device("cuda")
        prep = sav.vsa_prepare(case.q.to(dev), case.k.to(dev), case.v.to(dev), case.video_shape, case.tile_shape,
                               case.topk, case.scale)
        bmap, sizes = prep["block_map"], prep["tile_sizes"]
        qt, kt, vt = (torch.ones_like(prep[n]) for n in ("q", "k", "v"))
        out = torch.empty_like(qt)
        ws = torch.empty(sav.attn_block_sparse_workspace_size(qt.shape[0], case.num_heads, sizes.numel()),
                         dtype=torch.uint8, device=dev)
        t = time_steps(lambda: sav.attn_block_sparse_fwd(qt, kt, vt, bmap, sizes, case.scale, out=out, workspace=ws),
                       args.steps, args.warmup)
        flops = sparse_flops(bmap.cpu().numpy(), sizes.cpu().numpy(), case.head_dim)
        print(json.dumps({"metric": "attention on constant inputs", "workload": case.name, "unit": "TFLOP/s",
                          "ones": round(flops / (t.mean * 1e-3) / 1e12, 1), "ones_ms": round(t.mean, 5)}))
        return
    if args.only in ("mfma_stream", "mfma_stream_const"):
        kinds = ("randn",) if args.only == "mfma_stream" else ("constant",)
        print(json.dumps({"metric": "MFMA stream", **(mfma_stream_reference(args.steps, args.warmup, kinds=kinds) or {})}))
        return

    secondary = []
    head = None
    want = lambda name: args.only == name or (args.only is None and not args.no_secondary)  # noqa: E731
    cpu = not args.no_cpu_baseline
    budget = args.cpu_budget_s

    def line_for(name, t, work, bound, extra=None):
        """One secondary line: throughput over the mean step, median and min step."""
        rate = work / (t.mean * 1e-3) / (1e12 if bound == "mfma" else 1e9)
        unit = "TFLOP/s" if bound == "mfma" else "GB/s"
        rec = {"workload": name, "value": round(rate, 2), "unit": unit, "ms": round(t.mean, 5), **t.stats(),
               "roofline": roofline(KIND[name], bound, rate, work)}
        rec.update(extra or {})
        secondary.append(rec)
        log(f"{name}: {t.mean * 1e3:.1f} us/step (median {t.median * 1e3:.1f}, min {t.min * 1e3:.1f}), "
            f"{rate:.1f} {unit}")
        return rec

    KIND = {}
    if args.only in (None, "dense"):
        case = workloads.config2()
        t, flops = bench_varlen(case, args.steps, args.warmup)
        tf = flops / (t.mean * 1e-3) / 1e12
        log(f"{case.name}: {t.mean * 1e3:.1f} us/step (median {t.median * 1e3:.1f}, min {t.min * 1e3:.1f}), "
            f"{tf:.1f} TFLOP/s")
        head = (case, t, flops, tf)
    if want("tiny"):
        case = workloads.config1()
        KIND[case.name] = "tiny"
        t, flops = bench_varlen(case, args.steps, args.warmup)
        rec = line_for(case.name, t, flops, "mfma", {"note": "latency-bound: 35 MFLOP in one launch of 8 workgroups"})
        if cpu:
            rec["cpu_baseline"] = cpu_baseline_varlen(case, budget)
    if want("causal"):
        case = workloads.config3()
        KIND[case.name] = "causal"
        t, flops = bench_varlen(case, args.steps, args.warmup)
        rec = line_for(case.name, t, flops, "mfma")
        if cpu:
            rec["cpu_baseline"] = cpu_baseline_varlen(case, budget)
    decode_case = None  # workload 4's cache (10 GB of bf16) serves the windowed decode line too
    if want("paged"):
        decode_case = workloads.config4()
        KIND[decode_case.name] = "paged"
        t, nbytes = bench_paged(decode_case, args.steps, args.warmup)
        rec = line_for(decode_case.name, t, nbytes, "hbm")
        if cpu:
            rec["cpu_baseline"] = cpu_baseline_paged(decode_case, budget)
        torch.cuda.empty_cache()
    if want("sparse"):
        case = workloads.config5()
        KIND[case.name] = "sparse"
        t, flops, prep_ms, comp_ms, host = bench_sparse(case, args.steps, args.warmup)
        rec = line_for(case.name, t, flops, "mfma", {"tile_prep_and_map_ms": round(prep_ms, 4),
                                                    "compressed_branch_ms": round(comp_ms, 4)})
        log(f"  map build {prep_ms * 1e3:.0f} us, compressed branch {comp_ms * 1e3:.0f} us")
        if cpu:
            rec["cpu_baseline"] = cpu_baseline_sparse(case, host, budget)
        del host
    if want("h3"):
        case = workloads.config11()
        KIND[case.name] = "h3"
        t, flops, prep_ms = bench_h3(case, args.steps, args.warmup)
        line_for(case.name, t, flops, "mfma", {"tile_prep_and_map_ms": round(prep_ms, 4)})
        log(f"  H3 map build {prep_ms * 1e3:.0f} us")
    if want("paged_prefill"):
        case = workloads.config6()
        KIND[case.name] = "paged_prefill"
        t = bench_paged_prefill(case, args.steps, args.warmup)
        wms, wbytes = bench_kv_write(case, args.steps, args.warmup)
        line_for(case.name, t, paged_prefill_flops(case), "mfma",
                 {"kv_write": {"ms": round(wms, 5), "GB/s": round(wbytes / (wms * 1e-3) / 1e9, 1),
                               "tokens": int(case.q.shape[0])}})
        log(f"  kv write {wms * 1e3:.1f} us")
        del case
        torch.cuda.empty_cache()
    if want("spec"):
        case = workloads.config7()
        KIND[case.name] = "spec"
        t = bench_paged_prefill(case, args.steps, args.warmup)
        line_for(case.name, t, paged_prefill_bytes(case), "hbm")
        del case
        torch.cuda.empty_cache()
    if want("swa"):
        case = workloads.config8(decode_case)  # the same cache, tables and queries as workload 4
        KIND[case.name] = "swa"
        t, nbytes = bench_paged(case, args.steps, args.warmup, window=workloads.SLIDING_WINDOW)
        line_for(case.name, t, nbytes, "hbm")
        del case
    del decode_case
    torch.cuda.empty_cache()
    if want("head_dims"):
        for name, kind, t, work, bound in bench_head_dims(args.steps, args.warmup):
            KIND[name] = kind
            line_for(name, t, work, bound)
    for name, cfg, masked in (("masked", workloads.config9, True), ("padded", workloads.config10, False)):
        if want(name):
            case = cfg()
            KIND[case.name] = name
            t, flops = bench_padded(case, args.steps, args.warmup, masked)
            line_for(case.name, t, flops, "mfma")
            del case
            torch.cuda.empty_cache()

    if head is None:  # a single secondary workload was asked for
        print(json.dumps({"metric": "attention throughput", "secondary": secondary}))
        return
    case, t, flops, tf = head
    line = {
        "metric": "attention TFLOP/s (prefill, sparse) and HBM GB/s (paged decode), 1 MI355X",
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t.mean, 5),
        **t.stats(),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, resident in HBM)",
        "clock_warmup_ms": CLOCK_WARMUP_MS,
        "config": {"workload": case.name, "batch": 2, "seq_len": 4096, "num_heads": case.num_heads,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "causal": case.causal,
                   "layout": "packed varlen [total, heads, dim], cu_seqlens [0, 4096, 8192]", "lse": "fp32"},
        "roofline": roofline("dense", "mfma", tf, flops),
        "secondary": secondary,
    }
    if not args.no_gemm_reference:
        ref = gemm_reference(args.steps, args.warmup)
        ref["headline_over_randn"] = round(tf / ref["randn"], 4)
        log(f"vendor bf16 GEMM: {ref['randn']} TFLOP/s on N(0,1) operands, {ref['constant']} on constant ones")
        stream_ref = mfma_stream_reference(args.steps, args.warmup)
        if stream_ref is not None:
            stream_ref["headline_over_randn"] = round(tf / stream_ref["randn"], 4)
            log(f"MFMA stream: {stream_ref['randn']} TFLOP/s on N(0,1) operands, {stream_ref['constant']} on "
                f"constant ones")
        ref["mfma_stream"] = stream_ref
        line["mfma_reference"] = ref
    if cpu:
        log("timing the fp64 oracle on a sample (cpu baseline)")
        line["cpu_baseline"] = cpu_baseline_varlen(case, budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
