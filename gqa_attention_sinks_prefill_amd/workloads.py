"""Seeded synthetic workloads for sink-attention prefill and split-KV decode.

This module only draws inputs; it holds none of the attention arithmetic and
is the one piece that the tests, the benchmark and the oracle checks share.

The pages' workloads are trained GPT-OSS / Qwen3 models on live traffic
("GPT-OSS on day 0": sections "Attention: GQA with attention sinks" and "Cost
and performance", decode at sequence lengths 8192 and 32768; "Hosting Qwen on
Blackwell": sections "Prefillers" and "Decoders", about 6000-token inputs and
only 4 KV heads for Qwen3 235B).  Neither weights nor traffic are available,
so every tensor is drawn from a seeded ``torch.Generator('cpu')`` with the
shapes of those workloads:

* draw order: lengths, then Q, then K, then V, then sinks;
* Q/K/V: ``randn`` in fp32 rounded to bf16 (round-to-nearest-even);
* sinks: fp32 ``uniform_(lo, hi)``; edge heads are then overwritten;
* variable lengths: ``randint(lo, hi + 1)``.

Layouts: prefill Q and O are ``[T, Hq, D]`` over the packed tokens of all
sequences (``cu_seqlens`` marks the boundaries); prefill K/V are HND
``[Hkv, T, D]``.  Decode Q is ``[B, Hq, D]`` and the KV cache is HND per
request, ``[B, Hkv, max_ctx, D]``; cache slots at or beyond a request's
length are filled with NaN so that any read of them shows up in the output.
Multi-token decode Q is ``[B, q_len, Hq, D]``: the q_len new tokens are the
last q_len cached tokens of each request.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    seqlens: tuple | None          # fixed lengths, or None to draw them
    num_seqs: int
    len_range: tuple | None        # (lo, hi) inclusive when drawn
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sink_range: tuple
    seed: int
    causal: bool = True
    edge_sinks: dict = field(default_factory=dict)   # head -> value

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    ctx: int | None                # fixed context, or None to draw it
    ctx_range: tuple | None        # (lo, hi) inclusive when drawn
    max_ctx: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sink_range: tuple
    split_size: int
    seed: int
    edge_sinks: dict = field(default_factory=dict)
    q_len: int = 1                 # new tokens per request (speculative / MTP verification)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def num_splits(self) -> int:
        return -(-self.max_ctx // self.split_size)


# Tiny causal prefill: one 256-token sequence, GQA 4:1, head_dim 64, seed 0.
TINY_PREFILL = PrefillConfig("tiny_prefill_b1_s256_h4kv1_d64", (256,), 1, None,
                             4, 1, 64, (-2.0, 2.0), seed=0)
# GPT-OSS-shaped causal prefill: one 8192-token sequence, 64 q / 8 KV heads, d 64.
GPTOSS_PREFILL = PrefillConfig("gptoss_prefill_b1_s8192_h64kv8_d64", (8192,), 1, None,
                               64, 8, 64, (-4.0, 4.0), seed=1)
# Split-KV decode: 64 requests x 8192 cached tokens, 64 q / 8 KV heads, 1024-token chunks.
SPLIT_DECODE = DecodeConfig("decode_b64_ctx8192_h64kv8_d64_split1024", 64, 8192, None, 8192,
                            64, 8, 64, (-4.0, 4.0), split_size=1024, seed=2)
# Wide-GQA varlen prefill: 16 sequences of U[512, 6000] tokens, 64 q / 4 KV heads, d 128;
# head 5 (inside the first GQA group) gets sink -inf, i.e. plain attention.
VARLEN_PREFILL = PrefillConfig("varlen_prefill_16seq_512to6000_h64kv4_d128", None, 16,
                               (512, 6000), 64, 4, 128, (-4.0, 4.0), seed=4,
                               edge_sinks={5: float("-inf")})


# Chunked prefill: 4 sequences of 8192 tokens whose last 2048 are the new chunk
# (the earlier 6144 are cached), GPT-OSS heads; use chunked_prefill_inputs(cfg, 2048).
CHUNKED_PREFILL = PrefillConfig("chunked_prefill_4seq_8192_chunk2048_h64kv8_d64", (8192,) * 4, 4,
                                None, 64, 8, 64, (-4.0, 4.0), seed=6)
CHUNK_LEN = 2048

# Multi-token decode (speculative / MTP verification): the split-decode shape with 4
# new tokens per request, the last 4 of its 8192 cached tokens.
MTP_DECODE = DecodeConfig("mtp_decode_b64_q4_ctx8192_h64kv8_d64_split1024", 64, 8192, None,
                          8192, 64, 8, 64, (-4.0, 4.0), split_size=1024, seed=5, q_len=4)


def ragged_decode(batch: int) -> DecodeConfig:
    """Long-context ragged decode: contexts U[1024, 32768], 64 q / 8 KV heads, d 64
    (1024-token chunks unless a caller picks another split size).

    Head 0 gets sink -inf (plain attention) and head 63 (another GQA group)
    gets sink +20 (the sink dominates the softmax).
    """
    return DecodeConfig(f"ragged_decode_b{batch}_ctx1024to32768_h64kv8_d64",
                        batch, None, (1024, 32768), 32768, 64, 8, 64, (-4.0, 4.0),
                        split_size=1024, seed=3,
                        edge_sinks={0: float("-inf"), 63: 20.0})


RAGGED_BATCHES = (1, 8, 32, 128)


def _sinks(g, n, rng, edges):
    s = torch.empty(n, dtype=torch.float32).uniform_(rng[0], rng[1], generator=g)
    for h, val in edges.items():
        s[h] = val
    return s


def prefill_inputs(cfg: PrefillConfig) -> dict:
    """CPU tensors for a prefill workload (see the module docstring for the recipe)."""
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    if cfg.seqlens is not None:
        lens = torch.tensor(cfg.seqlens, dtype=torch.int32)
    else:
        lo, hi = cfg.len_range
        lens = torch.randint(lo, hi + 1, (cfg.num_seqs,), generator=g, dtype=torch.int64)
        lens = lens.to(torch.int32)
    cu = torch.zeros(cfg.num_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    T = int(cu[-1])
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    q = torch.randn(T, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(Hkv, T, D, generator=g).to(torch.bfloat16)
    v = torch.randn(Hkv, T, D, generator=g).to(torch.bfloat16)
    sinks = _sinks(g, Hq, cfg.sink_range, cfg.edge_sinks)
    return dict(q=q, k=k, v=v, sinks=sinks, cu_seqlens=cu, seqlens=lens,
                max_seqlen=int(lens.max()) if cfg.num_seqs else 0, total_tokens=T)


def chunked_prefill_inputs(cfg: PrefillConfig, chunk: int) -> dict:
    """CPU tensors for chunked prefill: each sequence of the config (its full
    length is the key count) gets a query chunk of its last min(chunk, length)
    tokens.  Q is ``[Tq, Hq, D]`` over the chunks (``cu_seqlens_q``), K/V are
    HND ``[Hkv, Tk, D]`` over the whole sequences (``cu_seqlens_k``)."""
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    if cfg.seqlens is not None:
        lens_k = torch.tensor(cfg.seqlens, dtype=torch.int32)
    else:
        lo, hi = cfg.len_range
        lens_k = torch.randint(lo, hi + 1, (cfg.num_seqs,), generator=g,
                               dtype=torch.int64).to(torch.int32)
    lens_q = torch.clamp(lens_k, max=chunk)
    cu_q = torch.zeros(cfg.num_seqs + 1, dtype=torch.int32)
    cu_q[1:] = torch.cumsum(lens_q, 0).to(torch.int32)
    cu_k = torch.zeros(cfg.num_seqs + 1, dtype=torch.int32)
    cu_k[1:] = torch.cumsum(lens_k, 0).to(torch.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    q = torch.randn(Tq, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(Hkv, Tk, D, generator=g).to(torch.bfloat16)
    v = torch.randn(Hkv, Tk, D, generator=g).to(torch.bfloat16)
    sinks = _sinks(g, Hq, cfg.sink_range, cfg.edge_sinks)
    return dict(q=q, k=k, v=v, sinks=sinks, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                seqlens_q=lens_q, seqlens_k=lens_k,
                max_seqlen_q=int(lens_q.max()) if cfg.num_seqs else 0)


def decode_inputs(cfg: DecodeConfig, poison: float = float("nan"), lens=None) -> dict:
    """CPU tensors for a decode workload; unused cache slots hold ``poison``.
    ``lens`` (one length per request) overrides the configured lengths."""
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    B, Hq, Hkv, D = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    if lens is not None:
        lens = torch.tensor(list(lens), dtype=torch.int32)
        if lens.numel() != B or int(lens.max()) > cfg.max_ctx:
            raise ValueError("lens must give one length <= max_ctx per request")
    elif cfg.ctx is not None:
        lens = torch.full((B,), cfg.ctx, dtype=torch.int32)
    else:
        lo, hi = cfg.ctx_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    qshape = (B, Hq, D) if cfg.q_len == 1 else (B, cfg.q_len, Hq, D)
    q = torch.randn(*qshape, generator=g).to(torch.bfloat16)
    caches = []
    for _ in range(2):                                   # K first, then V
        c = torch.empty(B, Hkv, cfg.max_ctx, D, dtype=torch.bfloat16)
        for b in range(B):
            L = int(lens[b])
            c[b, :, :L] = torch.randn(Hkv, L, D, generator=g).to(torch.bfloat16)
            c[b, :, L:] = poison
        caches.append(c)
    sinks = _sinks(g, Hq, cfg.sink_range, cfg.edge_sinks)
    return dict(q=q, k_cache=caches[0], v_cache=caches[1], seq_lens=lens, sinks=sinks)


# KV-cache append: 64 requests each append 1024 new tokens (8 KV heads, d 64,
# token-major rows as a QKV projection writes them) to HND caches of 8192 slots.
KV_APPEND = dict(name="kv_append_b64_new1024_kv8_d64_ctx8192", batch=64, new=1024,
                 num_kv_heads=8, head_dim=64, max_ctx=8192, seed=7)


def kv_append_inputs(counts, max_ctx: int, num_kv_heads: int, head_dim: int, seed: int,
                     pos=None) -> dict:
    """New K/V rows ``[T, Hkv, D]`` (token-major, packed by ``cu_seqlens_new``)
    and a first cache slot per request (drawn so the rows fit when ``pos`` is
    None).  Draw order: positions, K rows, V rows."""
    g = torch.Generator("cpu").manual_seed(seed)
    counts = torch.tensor(list(counts), dtype=torch.int32)
    cu = torch.zeros(counts.numel() + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(counts, 0).to(torch.int32)
    if pos is None:
        room = torch.clamp(max_ctx - counts, min=0).to(torch.int64)
        pos = (torch.rand(counts.numel(), generator=g) * (room + 1).double()).floor().to(torch.int32)
    else:
        pos = torch.tensor(list(pos), dtype=torch.int32)
    T = int(cu[-1])
    k = torch.randn(T, num_kv_heads, head_dim, generator=g).to(torch.bfloat16)
    v = torch.randn(T, num_kv_heads, head_dim, generator=g).to(torch.bfloat16)
    return dict(k_new=k, v_new=v, cu_seqlens_new=cu, cache_pos=pos, counts=counts)


def prefill_flops(seqlens, num_q_heads: int, head_dim: int, causal: bool = True) -> float:
    """Algorithmic flops: 4*D per visible (query, key) pair (2*D for QK^T, 2*D for PV)."""
    pairs = sum(int(n) * (int(n) + 1) // 2 if causal else int(n) * int(n) for n in seqlens)
    return 4.0 * head_dim * num_q_heads * pairs


def chunked_prefill_flops(seqlens_q, seqlens_k, num_q_heads: int, head_dim: int) -> float:
    """Algorithmic flops of causal chunked prefill: query i of a chunk of lq at the
    end of lk keys sees lk - lq + i + 1 keys; 4*D flops per visible pair."""
    pairs = sum(int(lq) * (int(lk) - int(lq)) + int(lq) * (int(lq) + 1) // 2
                for lq, lk in zip(seqlens_q, seqlens_k))
    return 4.0 * head_dim * num_q_heads * pairs


def decode_kv_bytes(seq_lens, num_kv_heads: int, head_dim: int) -> float:
    """Algorithmic bytes: K and V of every cached token read once per KV head (bf16)."""
    return float(sum(int(n) for n in seq_lens)) * num_kv_heads * head_dim * 2 * 2


# FP8 KV cache: the split-decode shape (64 requests x 8192 tokens, 64 q / 8 KV
# heads, d 64) over E4M3 caches.  Codes are drawn uniformly from the 254
# finite E4M3 codes (no quantizer runs here); per-KV-head scales U[0.005, 0.015]
# put the dequantized values in about [-6.7, 6.7].
FP8_DECODE = DecodeConfig("fp8_decode_b64_ctx8192_h64kv8_d64_split1024", 64, 8192, None, 8192,
                          64, 8, 64, (-4.0, 4.0), split_size=1024, seed=8)
FP8_SCALE_RANGE = (0.005, 0.015)


def fp8_decode_inputs(cfg: DecodeConfig, lens=None) -> dict:
    """CPU tensors for decode over FP8 caches: q (as decode_inputs), uint8 code
    caches ``[B, Hkv, max_ctx, D]``, ``k_scale`` / ``v_scale`` ``[Hkv]`` fp32.
    Draw order: lengths, Q, K codes, V codes, sinks, K scales, V scales; slots
    at or beyond a request's length hold the NaN code 0x7F."""
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    B, Hq, Hkv, D = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    if lens is not None:
        lens = torch.tensor(list(lens), dtype=torch.int32)
    elif cfg.ctx is not None:
        lens = torch.full((B,), cfg.ctx, dtype=torch.int32)
    else:
        lo, hi = cfg.ctx_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    qshape = (B, Hq, D) if cfg.q_len == 1 else (B, cfg.q_len, Hq, D)
    q = torch.randn(qshape, generator=g).to(torch.bfloat16)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    shape = (B, Hkv, cfg.max_ctx, D)
    kc = finite[torch.randint(0, finite.numel(), shape, generator=g)]
    vc = finite[torch.randint(0, finite.numel(), shape, generator=g)]
    slot = torch.arange(cfg.max_ctx).view(1, 1, -1, 1)
    unused = slot >= lens.view(-1, 1, 1, 1).to(torch.int64)
    kc = kc.masked_fill(unused, 0x7F)
    vc = vc.masked_fill(unused, 0x7F)
    sinks = _sinks(g, Hq, cfg.sink_range, cfg.edge_sinks)
    ks = torch.empty(Hkv, dtype=torch.float32).uniform_(*FP8_SCALE_RANGE, generator=g)
    vs = torch.empty(Hkv, dtype=torch.float32).uniform_(*FP8_SCALE_RANGE, generator=g)
    return dict(q=q, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs, seq_lens=lens, sinks=sinks)


def decode_kv_bytes_fp8(seq_lens, num_kv_heads: int, head_dim: int) -> float:
    """Algorithmic bytes of decode over FP8 caches: K and V codes of every
    cached token read once per KV head, one byte each."""
    return float(sum(int(n) for n in seq_lens)) * num_kv_heads * head_dim * 2
