"""CPU oracle for GQA attention with a learned per-head sink logit.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``gqa_attention_sinks_prefill_amd``) never does, and the two share no code.

The arithmetic lives in ``sink_oracle.c`` (fp64, OpenMP, two-pass softmax over
``[sink_h, scale * q.k_j]`` followed by a weighted sum of V; the sink has no
value row).  Its header cites the passages of "GPT-OSS on day 0" (section
"Kernels for GPT-OSS / Sink-Attention") and "Hosting Qwen on Blackwell"
(section "Deployment on GB200 NVL72", HND cache order) that it follows.  This
module only builds the shared object with gcc, marshals torch CPU tensors into
pointers and strides, and returns numpy float64 arrays.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sink_oracle.c")
_LIB = os.path.join(_HERE, "libsinkoracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_F64 = ctypes.c_double


def build(verbose: bool = False) -> str:
    """Compile sink_oracle.c into libsinkoracle.so (gcc, -O2, OpenMP, no fast-math)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_prefill.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                   _P, _P, _I32, _I32, _I32, _I32, _F64, _I32,
                                   _P, _I64, _I32, _P, _P, _P]
    lib.oracle_prefill.restype = _I32
    lib.oracle_prefill_chunked.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                           _P, _P, _P, _I32, _I32, _I32, _I32, _F64, _I32,
                                           _P, _I64, _I32, _P, _P, _P]
    lib.oracle_prefill_chunked.restype = _I32
    lib.oracle_decode.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _I64,
                                  _P, _I32, _P, _I32, _I32, _I32, _F64,
                                  _P, _I64, _I32, _P, _P, _P]
    lib.oracle_decode.restype = _I32
    lib.oracle_decode_multi.argtypes = [_P, _I64, _I64, _I64, _P, _P, _I64, _I64, _I64,
                                        _P, _I32, _I32, _P, _I32, _I32, _I32, _F64,
                                        _P, _I64, _I32, _P, _P, _P]
    lib.oracle_decode_multi.restype = _I32
    lib.oracle_chunk_states.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _I64,
                                        _P, _I32, _P, _I32, _I32, _I32, _F64,
                                        _I32, _I32, _I32, _P, _I64, _I32, _P, _P, _P]
    lib.oracle_chunk_states.restype = _I32
    lib.oracle_merge_states.argtypes = [_P, _P, _P, _I64, _I32, _I32, _P, _P]
    lib.oracle_merge_states.restype = _I32
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads the oracle uses: the process's CPU affinity, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _bf16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.bfloat16 or t.device.type != "cpu":
        raise TypeError("oracle inputs must be bfloat16 CPU tensors")
    if t.stride(-1) != 1:
        raise ValueError("oracle inputs need unit stride along head_dim")
    return t


def _rows(rows, n_default):
    if rows is None:
        return None, n_default
    arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    return arr, arr.shape[0]


def _ptr(a) -> int | None:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def prefill(q, k, v, sinks, cu_seqlens, *, causal=True, scale=None, rows=None,
            kv_layout="hnd", threads=None):
    """Sink attention over packed sequences.

    q: [T, Hq, D] bf16; k, v: bf16, [Hkv, T, D] for kv_layout="hnd" (heads
    leading, tokens contiguous) or [T, Hkv, D] for "nhd"; any strides with
    unit stride along D.  sinks: [Hq] fp32; cu_seqlens: [S+1] int32.
    rows: optional iterable of (token, head) pairs; default all, token-major.
    Returns (o [n, D], lse [n], sink_share [n]) as float64 numpy arrays.
    """
    q, k, v = _bf16(q), _bf16(k), _bf16(v)
    T, Hq, D = q.shape
    k_st, k_sh, Hkv = _kv_strides(k, kv_layout)
    v_st, v_sh, _ = _kv_strides(v, kv_layout)
    sinks = sinks.to(torch.float32).contiguous()
    cu = cu_seqlens.to(torch.int32).contiguous()
    rows_arr, n = _rows(rows, T * Hq)
    o = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    share = np.zeros(n, np.float64)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_prefill(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k_st, k_sh,
        v.data_ptr(), v_st, v_sh, sinks.data_ptr(), cu.data_ptr(), cu.numel() - 1,
        Hq, Hkv, D, scale, int(bool(causal)), _ptr(rows_arr), n,
        threads or default_threads(), o.ctypes.data, lse.ctypes.data, share.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return o, lse, share


def prefill_chunked(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, *, causal=True, scale=None,
                    rows=None, kv_layout="hnd", threads=None):
    """Chunked prefill: per sequence, len_q new queries (packed by cu_seqlens_q)
    against len_k >= len_q keys (packed by cu_seqlens_k), the queries being the
    sequence's last len_q tokens.  Layouts and return values as prefill()."""
    q, k, v = _bf16(q), _bf16(k), _bf16(v)
    Tq, Hq, D = q.shape
    k_st, k_sh, Hkv = _kv_strides(k, kv_layout)
    v_st, v_sh, _ = _kv_strides(v, kv_layout)
    sinks = sinks.to(torch.float32).contiguous()
    cq = cu_seqlens_q.to(torch.int32).contiguous()
    ck = cu_seqlens_k.to(torch.int32).contiguous()
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    rows_arr, n = _rows(rows, Tq * Hq)
    o = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    share = np.zeros(n, np.float64)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_prefill_chunked(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k_st, k_sh,
        v.data_ptr(), v_st, v_sh, sinks.data_ptr(), cq.data_ptr(), ck.data_ptr(),
        cq.numel() - 1, Hq, Hkv, D, scale, int(bool(causal)), _ptr(rows_arr), n,
        threads or default_threads(), o.ctypes.data, lse.ctypes.data, share.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_prefill_chunked rejected its arguments")
    return o, lse, share


def _kv_strides(t: torch.Tensor, layout: str):
    """(token stride, head stride, Hkv) of a 3-D K/V tensor in HND or NHD order."""
    if t.dim() != 3:
        raise ValueError("K/V must be 3-D")
    if layout == "hnd":
        return t.stride(1), t.stride(0), t.shape[0]      # [Hkv, T, D]
    if layout == "nhd":
        return t.stride(0), t.stride(1), t.shape[1]      # [T, Hkv, D]
    raise ValueError("kv_layout must be 'hnd' or 'nhd'")


def decode(q, k_cache, v_cache, seq_lens, sinks, *, scale=None, rows=None, threads=None):
    """Sink attention of one query token per request over an HND cache.

    q: [B, Hq, D] bf16; k_cache, v_cache: [B, Hkv, max_ctx, D] bf16 (any
    strides with unit d-stride, both caches sharing them); seq_lens: [B] int32.
    Returns (o [n, D], lse [n], sink_share [n]) float64, rows (b, h) b-major.
    """
    q, k_cache, v_cache = _bf16(q), _bf16(k_cache), _bf16(v_cache)
    if k_cache.stride() != v_cache.stride():
        raise ValueError("K and V caches must share strides")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    sinks = sinks.to(torch.float32).contiguous()
    lens = seq_lens.to(torch.int32).contiguous()
    rows_arr, n = _rows(rows, B * Hq)
    o = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    share = np.zeros(n, np.float64)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_decode(
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), lens.data_ptr(), B,
        sinks.data_ptr(), Hq, Hkv, D, scale, _ptr(rows_arr), n,
        threads or default_threads(), o.ctypes.data, lse.ctypes.data, share.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o, lse, share


def decode_multi(q, k_cache, v_cache, seq_lens, sinks, *, scale=None, rows=None, threads=None):
    """Multi-token decode: q_len new tokens per request, at the end of its cache.

    q: [B, q_len, Hq, D] bf16; new token t of request b sees cached tokens
    0 .. seq_lens[b] - q_len + t.  Caches as in decode().  rows: (b, t, h)
    triples, default all in (b, t, h) order.  Returns (o [n, D], lse [n],
    sink_share [n]) float64.
    """
    q, k_cache, v_cache = _bf16(q), _bf16(k_cache), _bf16(v_cache)
    if k_cache.stride() != v_cache.stride():
        raise ValueError("K and V caches must share strides")
    B, q_len, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    sinks = sinks.to(torch.float32).contiguous()
    lens = seq_lens.to(torch.int32).contiguous()
    if rows is None:
        rows_arr, n = None, B * q_len * Hq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows_arr.shape[0]
    o = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    share = np.zeros(n, np.float64)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_decode_multi(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        lens.data_ptr(), B, q_len, sinks.data_ptr(), Hq, Hkv, D, scale, _ptr(rows_arr), n,
        threads or default_threads(), o.ctypes.data, lse.ctypes.data, share.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_decode_multi rejected its arguments")
    return o, lse, share


def chunk_states(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits, *,
                 sink_chunk=0, scale=None, rows=None, threads=None):
    """Per-chunk (o, m, d) states of decode rows; m in natural-log units.

    Returns o [n, num_splits, D], m [n, num_splits], d [n, num_splits].
    sink_chunk selects which chunk carries the sink (-1: all of them, wrong
    on purpose, used only as a negative control).
    """
    q, k_cache, v_cache = _bf16(q), _bf16(k_cache), _bf16(v_cache)
    if k_cache.stride() != v_cache.stride():
        raise ValueError("K and V caches must share strides")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    sinks = sinks.to(torch.float32).contiguous()
    lens = seq_lens.to(torch.int32).contiguous()
    rows_arr, n = _rows(rows, B * Hq)
    o = np.zeros((n, num_splits, D), np.float64)
    m = np.zeros((n, num_splits), np.float64)
    d = np.zeros((n, num_splits), np.float64)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_chunk_states(
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), lens.data_ptr(), B,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits),
        int(sink_chunk), _ptr(rows_arr), n, threads or default_threads(),
        o.ctypes.data, m.ctypes.data, d.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_chunk_states rejected its arguments")
    return o, m, d


def merge_states(o_parts, m_parts, d_parts):
    """Merge chunk states: o [n, S, D], m/d [n, S] float64 -> (o [n, D], lse [n])."""
    o_parts = np.ascontiguousarray(o_parts, np.float64)
    m_parts = np.ascontiguousarray(m_parts, np.float64)
    d_parts = np.ascontiguousarray(d_parts, np.float64)
    n, S, D = o_parts.shape
    o = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    rc = _load().oracle_merge_states(o_parts.ctypes.data, m_parts.ctypes.data,
                                     d_parts.ctypes.data, n, S, D, o.ctypes.data,
                                     lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_merge_states rejected its arguments")
    return o, lse


def kv_append(k_new, v_new, cu_seqlens_new, cache_pos, k_cache, v_cache):
    """Write new tokens' K/V rows into HND caches, the definition written out.

    "Hosting Qwen on Blackwell", section "Deployment on GB200 NVL72": caches
    are HND; new rows arrive token-major.  For request b and new token t of
    its n_b (packed by cu_seqlens_new), slot cache_pos[b] + t of every KV head
    receives the row; slots outside [0, max_ctx) are not written.
    k_new, v_new: [T, Hkv, D] bf16 (CPU); caches [B, Hkv, max_ctx, D] bf16.
    Returns new (k_cache, v_cache) tensors; the inputs are not modified.
    """
    kc, vc = k_cache.clone(), v_cache.clone()
    cu = [int(x) for x in cu_seqlens_new]
    pos = [int(x) for x in cache_pos]
    max_ctx = kc.shape[2]
    for b in range(len(cu) - 1):
        for t in range(cu[b + 1] - cu[b]):
            slot = pos[b] + t
            if 0 <= slot < max_ctx:
                kc[b, :, slot, :] = k_new[cu[b] + t]
                vc[b, :, slot, :] = v_new[cu[b] + t]
    return kc, vc


# ----------------------------------------------------------- FP8 KV cache --
# The pages name FP8 only for weights; an FP8 KV cache is a plain extension
# (the decode step is memory-bound, "Hosting Qwen on Blackwell", section
# "Decoders").  Reading taken: the cache holds OCP FP8 E4M3 codes (1 sign,
# 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
# subnormal; S.1111.111 is NaN; no infinities; largest finite 448), with one
# fp32 scale per KV head: value = e4m3(code) * scale[g].  Attention is then
# the same definition, evaluated on the dequantized values in float64.

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> E4M3 codes: round to nearest, ties to the even
    mantissa, magnitudes past 448 saturated to +-448, NaN -> 0x7F.

    By brute force against the table of finite codes: the nearest value;
    among equally near codes the one with an even mantissa, and between +0
    and -0 the one with the sign of x.
    """
    x = np.asarray(x, np.float32).astype(np.float64)
    codes = np.array([c for c in range(256) if not math.isnan(E4M3_TABLE[c])])
    vals = E4M3_TABLE[codes]
    odd = (codes & 1).astype(np.int64)
    neg = (codes >> 7).astype(np.int64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    for s in range(0, flat.size, 1 << 15):
        v = flat[s:s + (1 << 15)]
        nan = np.isnan(v)
        vc = np.clip(np.where(nan, 0.0, v), -E4M3_MAX, E4M3_MAX)
        dist = np.abs(vals[None, :] - vc[:, None])
        tie = dist == dist.min(axis=1, keepdims=True)
        sign_x = np.signbit(vc).astype(np.int64)
        rank = np.where(tie, 2 * odd[None, :] + (neg[None, :] != sign_x[:, None]), 99)
        c = codes[np.argmin(rank, axis=1)]
        out[s:s + v.size] = np.where(nan, 0x7F, c)
    return out.reshape(x.shape)


def fp8_quantize(x, scale) -> np.ndarray:
    """Quantize values for a cache with dequantization scale `scale` (any
    shape broadcasting against x): code = e4m3_encode(fp32(x) * fp32(1 / scale)),
    the reciprocal and the product each rounded to float32 (the form a kernel
    evaluates)."""
    inv = np.float32(1.0) / np.asarray(scale, np.float32)
    return e4m3_encode(np.asarray(x, np.float32) * inv)


def kv_append_fp8(k_new, v_new, cu_seqlens_new, cache_pos, k_cache, v_cache, k_scale, v_scale):
    """kv_append into FP8 caches: the row of KV head g is quantized with that
    head's scale (fp8_quantize) and written to its slot; slots outside
    [0, max_ctx) are not written.  k_new, v_new: [T, Hkv, D] bf16; caches
    [B, Hkv, max_ctx, D] uint8 codes; scales [Hkv] float32.
    Returns new (k_cache, v_cache) uint8 tensors."""
    kc, vc = k_cache.clone(), v_cache.clone()
    cu = [int(x) for x in cu_seqlens_new]
    pos = [int(x) for x in cache_pos]
    ks = np.asarray(k_scale, np.float32)[None, :, None]
    vs = np.asarray(v_scale, np.float32)[None, :, None]
    kq = torch.from_numpy(fp8_quantize(k_new.float().numpy(), ks))    # [T, Hkv, D]
    vq = torch.from_numpy(fp8_quantize(v_new.float().numpy(), vs))
    max_ctx = kc.shape[2]
    for b in range(len(cu) - 1):
        for t in range(cu[b + 1] - cu[b]):
            slot = pos[b] + t
            if 0 <= slot < max_ctx:
                kc[b, :, slot, :] = kq[cu[b] + t]
                vc[b, :, slot, :] = vq[cu[b] + t]
    return kc, vc


def dequantize_fp8(codes, scales) -> np.ndarray:
    """[B, Hkv, L, D] uint8 codes, [Hkv] scales -> float64 values."""
    c = np.asarray(codes.numpy() if isinstance(codes, torch.Tensor) else codes, np.uint8)
    s = np.asarray(scales, np.float32).astype(np.float64)
    return E4M3_TABLE[c] * s[None, :, None, None]


def decode_multi_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens, sinks, *, scale=None,
                     rows=None):
    """Multi-token decode over FP8 caches (q_len >= 1 new tokens per request,
    at the end of the cache; new token t sees tokens 0 .. len_b - q_len + t),
    evaluated on the dequantized cache in float64, two passes per row:
        x_j = scale * q . k_j,  M = max(s_h, max x),  Z = exp(s_h - M) + sum exp(x_j - M),
        o = sum exp(x_j - M) v_j / Z,  lse = M + ln Z.
    q: [B, q_len, Hq, D] bf16; codes [B, Hkv, max_ctx, D] uint8; scales [Hkv].
    rows: (b, t, h) triples, default all in (b, t, h) order.
    Returns (o [n, D], lse [n], sink_share [n]) float64.
    """
    qf = q.float().numpy().astype(np.float64)
    B, q_len, Hq, D = qf.shape
    Hkv = k_codes.shape[1]
    r = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    sk = sinks.to(torch.float32).numpy().astype(np.float64)
    lens = [int(x) for x in seq_lens]
    if rows is None:
        rows = [(b, t, h) for b in range(B) for t in range(q_len) for h in range(Hq)]
    kc = np.asarray(k_codes.numpy(), np.uint8)
    vc = np.asarray(v_codes.numpy(), np.uint8)
    ks = np.asarray(k_scale, np.float32).astype(np.float64)
    vs = np.asarray(v_scale, np.float32).astype(np.float64)
    o = np.zeros((len(rows), D), np.float64)
    lse = np.zeros(len(rows), np.float64)
    share = np.zeros(len(rows), np.float64)
    by_bg = {}
    for i, (b, t, h) in enumerate(rows):
        by_bg.setdefault((b, h // r), []).append(i)
    for (b, g), idx in by_bg.items():
        n_max = max(0, lens[b])
        K = E4M3_TABLE[kc[b, g, :n_max]] * ks[g]
        V = E4M3_TABLE[vc[b, g, :n_max]] * vs[g]
        for i in idx:
            _, t, h = rows[i]
            n = max(0, lens[b] - q_len + t + 1)
            x = scale * (K[:n] @ qf[b, t, h])
            s = sk[h]
            M = max([s] + ([x.max()] if n else []))
            if M == -math.inf:
                lse[i] = -math.inf
                continue
            es = math.exp(s - M) if s != -math.inf else 0.0
            e = np.exp(x - M)
            Z = es + e.sum()
            o[i] = (e @ V[:n]) / Z
            lse[i] = M + math.log(Z)
            share[i] = es / Z
    return o, lse, share


# --------------------------------------------------------- paged KV cache --
# The pages keep caches in HND order per request; a paged (block-table) cache
# is the serving-engine form of the same data and is a plain extension (not on
# the pages).  Reading taken: physical pages [num_pages, Hkv, page_size, D]
# (HND inside a page); request b's logical token j lives in page
# block_tables[b, j // page_size], slot j % page_size.  Attention over it is the
# definition above on the logical cache; the oracle gathers that cache with
# plain indexing and evaluates the existing definitions.

def gather_pages(pages, block_tables, page_size, length):
    """Logical caches [B, Hkv, length, D] from pages [num_pages, Hkv, P, D] and
    block_tables [B, >= ceil(length / P)] (int); a copy, dtype preserved."""
    B = block_tables.shape[0]
    num_pages, Hkv, P, D = pages.shape
    if P != page_size:
        raise ValueError("pages' third dimension must be page_size")
    out = torch.empty((B, Hkv, length, D), dtype=pages.dtype)
    for b in range(B):
        for j in range(length):
            out[b, :, j] = pages[int(block_tables[b, j // P]), :, j % P]
    return out


def decode_multi_paged(q, k_pages, v_pages, block_tables, page_size, seq_lens, sinks, *,
                       k_scale=None, v_scale=None, scale=None, rows=None):
    """Multi-token decode over a paged cache (bf16 pages, or FP8 E4M3 code pages
    when k_scale / v_scale are given): gather each request's logical cache,
    then decode_multi / decode_multi_fp8.  q: [B, q_len, Hq, D]."""
    L = max([int(x) for x in seq_lens] + [1])
    kc = gather_pages(k_pages, block_tables, page_size, L)
    vc = gather_pages(v_pages, block_tables, page_size, L)
    if k_scale is None:
        return decode_multi(q, kc, vc, seq_lens, sinks, scale=scale, rows=rows)
    return decode_multi_fp8(q, kc, vc, k_scale, v_scale, seq_lens, sinks, scale=scale, rows=rows)


def kv_append_paged(k_new, v_new, cu_seqlens_new, cache_pos, k_pages, v_pages, block_tables,
                    page_size, *, k_scale=None, v_scale=None):
    """Append into a paged cache: new token t of request b goes to logical slot
    cache_pos[b] + t, i.e. page block_tables[b, slot // P], slot % P; slots
    at or past (table width) * P are dropped.  bf16 rows are copied, or
    quantized (fp8_quantize, per KV head) when k_scale / v_scale are given.
    Returns new (k_pages, v_pages)."""
    kp, vp = k_pages.clone(), v_pages.clone()
    cu = [int(x) for x in cu_seqlens_new]
    pos = [int(x) for x in cache_pos]
    width = block_tables.shape[1]
    if k_scale is not None:
        kq = torch.from_numpy(fp8_quantize(k_new.float().numpy(),
                                           np.asarray(k_scale, np.float32)[None, :, None]))
        vq = torch.from_numpy(fp8_quantize(v_new.float().numpy(),
                                           np.asarray(v_scale, np.float32)[None, :, None]))
    else:
        kq, vq = k_new, v_new
    for b in range(len(cu) - 1):
        for t in range(cu[b + 1] - cu[b]):
            slot = pos[b] + t
            if 0 <= slot < width * page_size:
                page = int(block_tables[b, slot // page_size])
                kp[page, :, slot % page_size] = kq[cu[b] + t]
                vp[page, :, slot % page_size] = vq[cu[b] + t]
    return kp, vp
