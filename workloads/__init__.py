"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark. This module holds no attention arithmetic: it only draws
lengths, permutations and N(0, 1) tensors.

Recipe (same for every case):
* integer structure (lengths, block permutation) comes from
  ``numpy.random.default_rng(seed)``: lengths first, then the permutation;
* float tensors are ``torch.randn(..., float32)`` from a CPU generator seeded
  ``1000 * seed + j`` (j = 0 for Q, 1 for K, 2 for V or the KV cache), rounded
  to bf16 on the host (round-to-nearest-even);
* the five named workloads follow the shapes of the pages' use cases: a tiny
  two-document varlen prefill, DiT-style dense self-attention, causal GQA
  varlen prefill, paged-KV decode with a shuffled block pool, and 3-D video
  block-sparse attention with 64-token (4, 4, 4) tiles.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = torch.bfloat16


def randn_bf16(shape, seed: int) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randn(tuple(shape), dtype=torch.float32, generator=g).to(BF16)


def randn_bf16_on(shape, seed: int, device) -> torch.Tensor:
    """N(0, 1) bf16 drawn on ``device`` by a seeded generator of that device,
    for inputs too large to draw on the host (the oracle reads slices of the
    same tensor)."""
    g = torch.Generator(device).manual_seed(int(seed))
    return torch.randn(tuple(shape), dtype=torch.float32, generator=g, device=device).to(BF16)


def cumulative(lengths) -> np.ndarray:
    """[0, l0, l0+l1, ...] as int32 (the cu_seqlens layout)."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out.astype(np.int32)


@dataclass
class VarlenCase:
    name: str
    q: torch.Tensor  # [Tq, Hq, D] bf16
    k: torch.Tensor  # [Tk, Hkv, D]
    v: torch.Tensor  # [Tk, Hkv, D]
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    cu_seqlens_k: np.ndarray
    num_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    scale: float
    seed: int

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens_q) - 1

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if self.batch else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(np.diff(self.cu_seqlens_k).max()) if self.batch else 0


def varlen_case(lengths_q, lengths_k=None, *, num_heads, num_kv_heads, head_dim, causal, seed,
                scale=None, name="varlen") -> VarlenCase:
    lengths_k = lengths_q if lengths_k is None else lengths_k
    cu_q, cu_k = cumulative(lengths_q), cumulative(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    return VarlenCase(
        name=name,
        q=randn_bf16((tq, num_heads, head_dim), 1000 * seed + 0),
        k=randn_bf16((tk, num_kv_heads, head_dim), 1000 * seed + 1),
        v=randn_bf16((tk, num_kv_heads, head_dim), 1000 * seed + 2),
        cu_seqlens_q=cu_q,
        cu_seqlens_k=cu_k,
        num_heads=num_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        causal=causal,
        scale=float(scale) if scale is not None else head_dim ** -0.5,
        seed=seed,
    )


def config1() -> VarlenCase:
    """Tiny varlen prefill: cu_seqlens [0, 100, 256], 4 heads, D 64, non-causal."""
    return varlen_case([100, 156], num_heads=4, num_kv_heads=4, head_dim=64, causal=False, seed=1,
                       scale=1.0 / 8.0, name="tiny-varlen-2doc-h4-d64")


def config2() -> VarlenCase:
    """DiT-style dense self-attention: batch 2 x seq 4096 as uniform varlen, 24 heads, D 128."""
    return varlen_case([4096, 4096], num_heads=24, num_kv_heads=24, head_dim=128, causal=False, seed=2,
                       name="dit-dense-b2-s4096-h24-d128")


def config3_lengths() -> np.ndarray:
    return np.random.default_rng(3).integers(512, 4097, 8)


def config3() -> VarlenCase:
    """Causal GQA varlen prefill: 8 docs, lengths uniform in [512, 4096], 32/8 heads, D 128."""
    return varlen_case(config3_lengths().tolist(), num_heads=32, num_kv_heads=8, head_dim=128, causal=True,
                       seed=3, name="causal-gqa-varlen-8doc-h32kv8-d128")


@dataclass
class PagedCase:
    name: str
    q: torch.Tensor  # [S, Hq, D] bf16
    kv_cache: torch.Tensor  # [2, NB, BS, Hkv, D] bf16
    block_tables: np.ndarray  # int32 [S, MB], unused tail = -1
    context_lens: np.ndarray  # int32 [S]
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    seed: int

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


def paged_case(context_lens, *, num_heads, num_kv_heads, head_dim, seed, block_size=128,
               max_blocks_per_seq=None, spare_blocks=0, rng=None, scale=None, name="paged",
               chunk_blocks=512) -> PagedCase:
    """Blocks of a shuffled pool are dealt to sequences in order; table tails are -1.

    ``rng`` continues the integer stream that drew ``context_lens`` (the block
    permutation is drawn after the lengths)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    need = [math.ceil(c / block_size) for c in ctx]
    num_blocks = int(sum(need)) + int(spare_blocks)
    rng = np.random.default_rng(seed) if rng is None else rng
    perm = rng.permutation(num_blocks)
    mb = max(need) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    mb = max(mb, 1)
    tables = np.full((len(ctx), mb), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    cache = torch.empty((2, num_blocks, block_size, num_kv_heads, head_dim), dtype=BF16)
    g = torch.Generator("cpu").manual_seed(1000 * seed + 2)
    for b0 in range(0, num_blocks, chunk_blocks):
        b1 = min(num_blocks, b0 + chunk_blocks)
        cache[:, b0:b1] = torch.randn((2, b1 - b0, block_size, num_kv_heads, head_dim), dtype=torch.float32,
                                      generator=g).to(BF16)
    return PagedCase(
        name=name,
        q=randn_bf16((len(ctx), num_heads, head_dim), 1000 * seed + 0),
        kv_cache=cache,
        block_tables=tables,
        context_lens=ctx.astype(np.int32),
        num_heads=num_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        scale=float(scale) if scale is not None else head_dim ** -0.5,
        seed=seed,
    )


@dataclass
class PagedPrefillCase:
    name: str
    q: torch.Tensor  # packed [Tq, Hq, D] bf16
    cu_seqlens_q: np.ndarray  # int32 [B + 1]
    kv_cache: torch.Tensor  # [2, NB, BS, Hkv, D] bf16 (already holds every sequence's new tokens)
    block_tables: np.ndarray  # int32 [B, MB], unused tail = -1
    context_lens: np.ndarray  # int32 [B]: keys per sequence, new tokens included
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    seed: int

    @property
    def batch(self) -> int:
        return int(self.context_lens.size)

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if self.batch else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[1])


def paged_prefill_case(q_lens, context_lens, *, num_heads, num_kv_heads, head_dim, seed, block_size=128,
                       max_blocks_per_seq=None, spare_blocks=0, rng=None, scale=None,
                       name="paged-prefill") -> PagedPrefillCase:
    """Multi-token queries over a paged cache: cache and tables as in paged_case
    (same seed, same streams), queries drawn with generator seed 1000*seed + 3."""
    base = paged_case(context_lens, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, seed=seed,
                      block_size=block_size, max_blocks_per_seq=max_blocks_per_seq, spare_blocks=spare_blocks,
                      rng=rng, scale=scale, name=name)
    ql = np.asarray(q_lens, dtype=np.int64)
    return PagedPrefillCase(
        name=name,
        q=randn_bf16((int(ql.sum()), num_heads, head_dim), 1000 * seed + 3),
        cu_seqlens_q=cumulative(ql),
        kv_cache=base.kv_cache,
        block_tables=base.block_tables,
        context_lens=base.context_lens,
        num_heads=num_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        scale=base.scale,
        seed=seed,
    )


def config4_lengths(rng=None) -> np.ndarray:
    rng = np.random.default_rng(4) if rng is None else rng
    return rng.integers(1024, 32769, 64)


def config4() -> PagedCase:
    """Paged decode: 64 seqs, contexts uniform in [1024, 32768], cache (2, NB, 128, 8, 128), 32 q heads."""
    rng = np.random.default_rng(4)
    ctx = config4_lengths(rng)
    return paged_case(ctx, num_heads=32, num_kv_heads=8, head_dim=128, seed=4, block_size=128,
                      max_blocks_per_seq=256, rng=rng, name="paged-decode-64seq-ctx1k-32k-h32kv8-d128")


def config6() -> PagedPrefillCase:
    """Chunked / cache-hit prefill over a paged cache: 16 sequences, 256..1024 new
    tokens each over contexts of 2048..16384 keys (new tokens included), 32/8 heads, D=128."""
    rng = np.random.default_rng(6)
    ql = rng.integers(256, 1025, 16)
    ctx = rng.integers(2048, 16385, 16)
    return paged_prefill_case(ql, ctx, num_heads=32, num_kv_heads=8, head_dim=128, seed=6, rng=rng,
                              name="paged-prefill-16seq-q256-1k-ctx2k-16k-h32kv8-d128")


def config7() -> PagedPrefillCase:
    """Speculative decoding over a paged cache: the 64 contexts of the decode
    workload, each with 4 new query tokens (the last 4 positions), 32/8 heads, D=128."""
    rng = np.random.default_rng(4)
    ctx = config4_lengths(rng)
    return paged_prefill_case(np.full(ctx.size, 4), ctx, num_heads=32, num_kv_heads=8, head_dim=128, seed=7,
                              max_blocks_per_seq=256, name="spec-decode-64seq-q4-ctx1k-32k-h32kv8-d128")


@dataclass
class VideoCase:
    name: str
    q: torch.Tensor  # raster [B, N, H, D] bf16
    k: torch.Tensor
    v: torch.Tensor
    video_shape: tuple = (16, 32, 32)
    tile_shape: tuple = (4, 4, 4)
    block: int = 64
    topk: int = 32
    num_heads: int = 12
    head_dim: int = 128
    scale: float = 128 ** -0.5
    seed: int = 5
    extra: dict = field(default_factory=dict)

    @property
    def num_tiles(self) -> int:
        return math.prod(math.ceil(s / t) for s, t in zip(self.video_shape, self.tile_shape))


def video_case(video_shape, *, num_heads, head_dim, topk, seed, tile_shape=(4, 4, 4), batch=1,
               name="video") -> VideoCase:
    n = math.prod(video_shape)
    return VideoCase(
        name=name,
        q=randn_bf16((batch, n, num_heads, head_dim), 1000 * seed + 0),
        k=randn_bf16((batch, n, num_heads, head_dim), 1000 * seed + 1),
        v=randn_bf16((batch, n, num_heads, head_dim), 1000 * seed + 2),
        video_shape=tuple(video_shape),
        tile_shape=tuple(tile_shape),
        topk=topk,
        num_heads=num_heads,
        head_dim=head_dim,
        scale=head_dim ** -0.5,
        seed=seed,
    )


def config5() -> VideoCase:
    """Video block-sparse: 16x32x32 latent, (4,4,4) tiles (256 tiles of 64), 12 heads, D 128, top-32."""
    return video_case((16, 32, 32), num_heads=12, head_dim=128, topk=32, seed=5,
                      name="video-block-sparse-16x32x32-t444-h12-d128-top32")


SLIDING_WINDOW = 4096  # tokens before the query that stay visible


def config8(decode_case: PagedCase | None = None) -> PagedCase:
    """Sliding-window decode: the decode workload (64 contexts of 1k..32k over
    a shuffled block pool, 32/8 heads, D=128) with a window of 4096 preceding
    tokens (the window length of common sliding-window decoders). An already
    built workload 4 may be passed in to share its cache."""
    import dataclasses

    base = config4() if decode_case is None else decode_case
    return dataclasses.replace(base, name="swa-decode-64seq-ctx1k-32k-w4096-h32kv8-d128")


@dataclass
class PaddedCase:
    name: str
    q: torch.Tensor  # [B, Sq, Hq, D] bf16
    k: torch.Tensor  # [B, Sk, Hkv, D]
    v: torch.Tensor  # [B, Sk, Hkv, D]
    q_lens: np.ndarray  # int32 [B] valid prefix lengths (padded batch)
    k_lens: np.ndarray
    key_mask: np.ndarray  # uint8 [B, Sk] (key-padding mask)
    num_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    scale: float
    seed: int


def padded_case(batch, seqlen_q, seqlen_k, *, num_heads, num_kv_heads, head_dim, seed, q_lens=None, k_lens=None,
                key_mask=None, causal=False, name="padded") -> PaddedCase:
    """A padded batch with N(0, 1) rows everywhere (padding rows included, so a
    kernel that reads them is caught). Valid lengths default to full; the key
    mask defaults to the key prefixes."""
    ql = np.full(batch, seqlen_q) if q_lens is None else np.asarray(q_lens)
    kl = np.full(batch, seqlen_k) if k_lens is None else np.asarray(k_lens)
    if key_mask is None:
        key_mask = (np.arange(seqlen_k)[None, :] < kl[:, None]).astype(np.uint8)
    return PaddedCase(
        name=name,
        q=randn_bf16((batch, seqlen_q, num_heads, head_dim), 1000 * seed + 0),
        k=randn_bf16((batch, seqlen_k, num_kv_heads, head_dim), 1000 * seed + 1),
        v=randn_bf16((batch, seqlen_k, num_kv_heads, head_dim), 1000 * seed + 2),
        q_lens=ql.astype(np.int32),
        k_lens=kl.astype(np.int32),
        key_mask=np.asarray(key_mask, dtype=np.uint8),
        num_heads=num_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        causal=causal,
        scale=1.0 / math.sqrt(head_dim),
        seed=seed,
    )


def config9() -> PaddedCase:
    """Cross-attention under a text padding mask (DiT text conditioning): 2
    latent sequences of 4096 query tokens attend 512 text tokens whose real
    count is uniform in [64, 512] (the rest are padding), 24 heads, D=128."""
    rng = np.random.default_rng(9)
    kl = rng.integers(64, 513, 2)
    return padded_case(2, 4096, 512, num_heads=24, num_kv_heads=24, head_dim=128, seed=9, k_lens=kl,
                       name="masked-cross-b2-q4096-k512-h24-d128")


def config10() -> PaddedCase:
    """Padded batch (packed padding): 4 sequences padded to 4096 tokens with
    valid lengths uniform in [1024, 4096], non-causal self-attention, 24 heads,
    D=128."""
    rng = np.random.default_rng(10)
    ln = rng.integers(1024, 4097, 4)
    return padded_case(4, 4096, 4096, num_heads=24, num_kv_heads=24, head_dim=128, seed=10, q_lens=ln, k_lens=ln,
                       name="padded-b4-s4096-valid1k-4k-h24-d128")


def config11() -> VideoCase:
    """H3 layout: workload 5's 16x32x32 video behind a 512-row text prefix (one
    segment: 8 dense prefix tiles ahead of 256 video tiles), 12 heads, D=128,
    top-32 among the video tiles."""
    segs = (512,)
    n = sum(segs) + 16 * 32 * 32
    seed = 11
    return VideoCase(
        name="h3-prefix512-video-16x32x32-t444-h12-d128-top32",
        q=randn_bf16((1, n, 12, 128), 1000 * seed + 0),
        k=randn_bf16((1, n, 12, 128), 1000 * seed + 1),
        v=randn_bf16((1, n, 12, 128), 1000 * seed + 2),
        topk=32,
        seed=seed,
        extra={"prefix_segments": segs},
    )
