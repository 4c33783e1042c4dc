"""GQA attention with learned per-head sinks on MI355X (gfx950).

Thin ctypes binding over ``libsinkattn.so`` (declared in ``include/sinkattn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor dtypes/devices, passes device pointers, element strides and
the current HIP stream, and turns a non-zero return code into an exception.
PyTorch is used for device memory and streams only.

Entry points (same names as the C ABI):
  prefill      sink_attn_prefill (causal / non-causal varlen),
               sink_attn_prefill_chunked (queries at the end of a longer key range)
  decode       sink_attn_decode_split (chunk states), sink_attn_merge_states,
               sink_attn_decode_multi_split (q_len new tokens per request),
               sink_attn_decode_multi_split_fp8 (FP8 E4M3 caches),
               sink_attn_decode_paged_split (block-table pages, bf16 or FP8),
               sink_attn_decode_fused (split and merge in one launch; counters from
               decode_counters), sink_attn_decode_merged (split and a merge over
               the chunks that hold keys; for ragged batches)
               sink_attn_decode_merged_noalloc (the same with the chunk states in
               the library's device scratch array: no buffers beyond in- and outputs),
               sink_attn_decode_split_size (the library's chunk size for a shape)
  KV cache     sink_attn_kv_append, sink_attn_kv_append_fp8, sink_attn_kv_append_paged
and the wrappers sink_attn_decode, sink_attn_decode_multi, sink_attn_decode_fp8 and
sink_attn_decode_paged (split + merge on one stream).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["sink_attn_prefill", "sink_attn_prefill_chunked", "sink_attn_decode_split", "sink_attn_decode_multi_split",
           "sink_attn_merge_states", "sink_attn_decode", "sink_attn_decode_multi",
           "sink_attn_kv_append", "sink_attn_decode_multi_split_fp8", "sink_attn_decode_fp8",
           "sink_attn_kv_append_fp8", "sink_attn_decode_paged_split", "sink_attn_decode_paged",
           "sink_attn_kv_append_paged", "sink_attn_decode_fused", "sink_attn_decode_merged", "decode_counters",
           "sink_attn_decode_split_size", "sink_attn_decode_merged_noalloc",
           "SinkAttnError", "library_path", "load_library", "EXPORTED_SYMBOLS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsinkattn.so")
_lib = None

EXPORTED_SYMBOLS = ("sink_attn_prefill", "sink_attn_prefill_chunked", "sink_attn_decode_split", "sink_attn_decode_multi_split",
                    "sink_attn_decode_multi_split_fp8", "sink_attn_decode_paged_split",
                    "sink_attn_decode_fused", "sink_attn_decode_merged",
                    "sink_attn_merge_states", "sink_attn_kv_append", "sink_attn_kv_append_fp8",
                    "sink_attn_kv_append_paged", "sink_attn_decode_split_size",
                    "sink_attn_decode_merged_noalloc", "sink_attn_last_error")


class SinkAttnError(RuntimeError):
    """A libsinkattn call returned a non-zero status."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsinkattn.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m gqa_attention_sinks_prefill_amd.build_native` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.sink_attn_prefill.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, P, I32, I32,
                                      I32, I32, I32, F32, I32, P, I64, I64, P, P]
    lib.sink_attn_prefill.restype = ctypes.c_int
    lib.sink_attn_prefill_chunked.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, P, P,
                                              I32, I32, I32, I32, I32, F32, I32, P, I64, I64,
                                              P, P]
    lib.sink_attn_prefill_chunked.restype = ctypes.c_int
    lib.sink_attn_decode_split.argtypes = [P, I64, I64, P, P, I64, I64, I64, P, I32, I32, P,
                                           I32, I32, I32, F32, I32, I32, P, P, P, P]
    lib.sink_attn_decode_split.restype = ctypes.c_int
    lib.sink_attn_decode_multi_split.argtypes = [P, I64, I64, I64, I32, P, P, I64, I64, I64, P,
                                                 I32, I32, P, I32, I32, I32, F32, I32, I32,
                                                 P, P, P, P]
    lib.sink_attn_decode_multi_split.restype = ctypes.c_int
    lib.sink_attn_merge_states.argtypes = [P, P, P, I32, I32, I32, I32, P, I64, I64, P, P]
    lib.sink_attn_merge_states.restype = ctypes.c_int
    lib.sink_attn_kv_append.argtypes = [P, P, I64, I64, P, P, I32, I32, P, P, I64, I64, I64,
                                        I32, I32, I32, P]
    lib.sink_attn_kv_append.restype = ctypes.c_int
    lib.sink_attn_decode_multi_split_fp8.argtypes = [P, I64, I64, I64, I32, P, P, I64, I64, I64,
                                                     P, P, P, I32, I32, P, I32, I32, I32, F32,
                                                     I32, I32, P, P, P, P]
    lib.sink_attn_decode_multi_split_fp8.restype = ctypes.c_int
    lib.sink_attn_kv_append_fp8.argtypes = [P, P, I64, I64, P, P, I32, I32, P, P, I64, I64, I64,
                                            P, P, I32, I32, I32, P]
    lib.sink_attn_kv_append_fp8.restype = ctypes.c_int
    lib.sink_attn_decode_paged_split.argtypes = [P, I64, I64, I64, I32, P, P, I64, I64, I64, I32,
                                                 P, I64, I32, P, P, P, I32, P, I32, I32, I32, F32,
                                                 I32, I32, P, P, P, P]
    lib.sink_attn_decode_paged_split.restype = ctypes.c_int
    lib.sink_attn_kv_append_paged.argtypes = [P, P, I64, I64, P, P, I32, I32, P, P, I64, I64, I64,
                                              I32, P, I64, I32, P, P, I32, I32, P]
    lib.sink_attn_kv_append_paged.restype = ctypes.c_int
    lib.sink_attn_decode_fused.argtypes = [P, I64, I64, I64, I32, P, P, I64, I64, I64, P, P, P,
                                           I32, I32, P, I32, I32, I32, F32, I32, I32, P, P, P, P,
                                           P, I64, I64, I64, P, P]
    lib.sink_attn_decode_fused.restype = ctypes.c_int
    # the same arguments without the counters
    fused = list(lib.sink_attn_decode_fused.argtypes)
    lib.sink_attn_decode_merged.argtypes = fused[:25] + fused[26:]
    lib.sink_attn_decode_merged.restype = ctypes.c_int
    # ... and without the partial buffers either
    lib.sink_attn_decode_merged_noalloc.argtypes = fused[:22] + fused[26:]
    lib.sink_attn_decode_merged_noalloc.restype = ctypes.c_int
    lib.sink_attn_decode_split_size.argtypes = [I32, I32, I32, I32, I32, I32, P]
    lib.sink_attn_decode_split_size.restype = ctypes.c_int32
    lib.sink_attn_last_error.argtypes = []
    lib.sink_attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        msg = load_library().sink_attn_last_error().decode(errors="replace")
        raise SinkAttnError(fn, rc, msg)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, dim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    return t


def _prefill_args(q, k, v, sinks, kv_layout, out, lse):
    _dev(q, "q", torch.bfloat16, 3)
    _dev(k, "k", torch.bfloat16, 3)
    _dev(v, "v", torch.bfloat16, 3)
    _dev(sinks, "sinks", torch.float32, 1)
    T, Hq, D = q.shape
    if kv_layout == "hnd":
        Hkv = k.shape[0]
        (k_sh, k_st), (v_sh, v_st) = k.stride()[:2], v.stride()[:2]
    elif kv_layout == "nhd":
        Hkv = k.shape[1]
        (k_st, k_sh), (v_st, v_sh) = k.stride()[:2], v.stride()[:2]
    else:
        raise ValueError("kv_layout must be 'hnd' or 'nhd'")
    if q.stride(2) != 1 or k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("q, k, v need unit stride along head_dim")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _dev(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _dev(lse, "lse", torch.float32, 2)
        if not lse.is_contiguous() or tuple(lse.shape) != (T, Hq):
            raise ValueError("lse must be a contiguous [T, Hq] fp32 tensor")
    return T, Hq, Hkv, D, (k_st, k_sh), (v_st, v_sh), out


def sink_attn_prefill(q, k, v, sinks, cu_seqlens, max_seqlen, *, causal=True, scale=None,
                      kv_layout="hnd", out=None, lse=None, stream=None):
    """Sink-attention prefill over packed sequences.

    q: [T, Hq, D] bf16.  k, v: bf16 [Hkv, T, D] for kv_layout="hnd" (default)
    or [T, Hkv, D] for "nhd"; any strides with unit stride along D.
    sinks: [Hq] fp32.  cu_seqlens: [S+1] int32 on the GPU.  max_seqlen: int.
    Returns out [T, Hq, D] bf16 (allocated if not given); fills lse [T, Hq]
    fp32 when passed.
    """
    _dev(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, Hq, Hkv, D, (k_st, k_sh), (v_st, v_sh), out = _prefill_args(q, k, v, sinks, kv_layout,
                                                                    out, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_prefill(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k_st, k_sh,
        v.data_ptr(), v_st, v_sh, sinks.data_ptr(), cu_seqlens.data_ptr(),
        cu_seqlens.numel() - 1, int(max_seqlen), Hq, Hkv, D, scale, int(bool(causal)),
        out.data_ptr(), out.stride(0), out.stride(1),
        lse.data_ptr() if lse is not None else None, _stream(stream))
    _check("sink_attn_prefill", rc)
    return out


def sink_attn_prefill_chunked(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, *,
                              causal=True, scale=None, kv_layout="hnd", out=None, lse=None,
                              stream=None):
    """Chunked prefill: per sequence, the queries packed by cu_seqlens_q are the
    last tokens of a sequence whose keys are packed by cu_seqlens_k (same
    count of sequences, every chunk no longer than its keys).  Layouts as
    sink_attn_prefill, with q / out over the query tokens and k / v over the
    key tokens.
    """
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    T, Hq, Hkv, D, (k_st, k_sh), (v_st, v_sh), out = _prefill_args(q, k, v, sinks, kv_layout,
                                                                    out, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_prefill_chunked(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k_st, k_sh,
        v.data_ptr(), v_st, v_sh, sinks.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, int(max_seqlen_q), Hq, Hkv, D, scale,
        int(bool(causal)), out.data_ptr(), out.stride(0), out.stride(1),
        lse.data_ptr() if lse is not None else None, _stream(stream))
    _check("sink_attn_prefill_chunked", rc)
    return out


def sink_attn_decode_split(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits=None,
                           *, max_ctx=None, scale=None, part_o=None, part_m=None, part_d=None,
                           stream=None):
    """Per-chunk decode states over an HND cache [B, Hkv, max_ctx, D].

    Returns (part_o [B, Hq, S, D], part_m [B, Hq, S], part_d [B, Hq, S]) fp32.
    """
    _dev(q, "q", torch.bfloat16, 3)
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q.stride(2) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    shape = (B, Hq, num_splits)
    if part_o is None:
        part_o = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        part_m = torch.empty(shape, dtype=torch.float32, device=q.device)
        part_d = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((part_o, "part_o", shape + (D,)), (part_m, "part_m", shape),
                       (part_d, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be contiguous with shape {shp}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_split(
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), seq_lens.data_ptr(), B,
        max_ctx, sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits),
        part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(), _stream(stream))
    _check("sink_attn_decode_split", rc)
    return part_o, part_m, part_d


def sink_attn_decode_multi_split(q, k_cache, v_cache, seq_lens, sinks, split_size,
                                 num_splits=None, *, max_ctx=None, scale=None, part_o=None,
                                 part_m=None, part_d=None, stream=None):
    """Per-chunk states of multi-token decode: q [B, q_len, Hq, D], the q_len new
    tokens being the last of each request's cache [B, Hkv, max_ctx, D].

    Returns (part_o [B, q_len, Hq, S, D], part_m [B, q_len, Hq, S],
    part_d [B, q_len, Hq, S]) fp32.
    """
    _dev(q, "q", torch.bfloat16, 4)
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, q_len, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    shape = (B, q_len, Hq, num_splits)
    if part_o is None:
        part_o = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        part_m = torch.empty(shape, dtype=torch.float32, device=q.device)
        part_d = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((part_o, "part_o", shape + (D,)), (part_m, "part_m", shape),
                       (part_d, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be contiguous with shape {shp}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_multi_split(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), q_len, k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        seq_lens.data_ptr(), B, max_ctx, sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size),
        int(num_splits), part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(),
        _stream(stream))
    _check("sink_attn_decode_multi_split", rc)
    return part_o, part_m, part_d


def sink_attn_merge_states(part_o, part_m, part_d, *, out=None, lse=None, stream=None):
    """Merge chunk states [B, Hq, S, D] into out [B, Hq, D] bf16 (and lse [B, Hq])."""
    _dev(part_o, "part_o", torch.float32, 4)
    _dev(part_m, "part_m", torch.float32, 3)
    _dev(part_d, "part_d", torch.float32, 3)
    B, Hq, S, D = part_o.shape
    for t, nm in ((part_o, "part_o"), (part_m, "part_m"), (part_d, "part_d")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if tuple(part_m.shape) != (B, Hq, S) or tuple(part_d.shape) != (B, Hq, S):
        raise ValueError("part_m / part_d must be [B, Hq, S]")
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=part_o.device)
    _dev(out, "out", torch.bfloat16, 3)
    if out.stride(2) != 1:
        raise ValueError("out needs unit stride along head_dim")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if not lse.is_contiguous() or lse.numel() != B * Hq:
            raise ValueError("lse must be a contiguous [B, Hq] fp32 tensor")
    rc = load_library().sink_attn_merge_states(
        part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(), B, Hq, S, D,
        out.data_ptr(), out.stride(0), out.stride(1),
        lse.data_ptr() if lse is not None else None, _stream(stream))
    _check("sink_attn_merge_states", rc)
    return out


def sink_attn_decode(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits=None, *,
                     max_ctx=None, scale=None, out=None, lse=None, partials=None, stream=None):
    """Split-KV decode: sink_attn_decode_split then sink_attn_merge_states, same stream."""
    po, pm, pd = partials if partials is not None else (None, None, None)
    po, pm, pd = sink_attn_decode_split(q, k_cache, v_cache, seq_lens, sinks, split_size,
                                        num_splits, max_ctx=max_ctx, scale=scale, part_o=po,
                                        part_m=pm, part_d=pd, stream=stream)
    return sink_attn_merge_states(po, pm, pd, out=out, lse=lse, stream=stream)


def sink_attn_decode_multi(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits=None, *,
                           max_ctx=None, scale=None, out=None, lse=None, partials=None,
                           stream=None):
    """Multi-token decode (speculative / MTP verification): split then merge.

    q [B, q_len, Hq, D]; returns out [B, q_len, Hq, D] bf16 (lse, if given,
    [B, q_len, Hq] fp32 contiguous).
    """
    B, q_len, Hq, D = q.shape
    po, pm, pd = partials if partials is not None else (None, None, None)
    po, pm, pd = sink_attn_decode_multi_split(q, k_cache, v_cache, seq_lens, sinks, split_size,
                                              num_splits, max_ctx=max_ctx, scale=scale,
                                              part_o=po, part_m=pm, part_d=pd, stream=stream)
    S = po.shape[3]
    if out is None:
        out = torch.empty(B, q_len, Hq, D, dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.bfloat16, 4)
    if out.stride(3) != 1 or out.stride(0) != q_len * out.stride(1):
        raise ValueError("out needs unit d-stride and (request, token) dims that flatten")
    rows = out.as_strided((B * q_len, Hq, D), (out.stride(1), out.stride(2), 1))
    sink_attn_merge_states(po.view(B * q_len, Hq, S, D), pm.view(B * q_len, Hq, S),
                           pd.view(B * q_len, Hq, S), out=rows, lse=lse, stream=stream)
    return out


def sink_attn_kv_append(k_new, v_new, cu_seqlens_new, cache_pos, k_cache, v_cache, *,
                        max_new=None, stream=None):
    """Write new tokens' K and V ([T, Hkv, D] token-major, packed by
    cu_seqlens_new) into the HND caches [B, Hkv, max_ctx, D] at slots
    cache_pos[b] .. cache_pos[b] + n_b - 1 (in place; returns the caches)."""
    _dev(k_new, "k_new", torch.bfloat16, 3)
    _dev(v_new, "v_new", torch.bfloat16, 3)
    _dev(cu_seqlens_new, "cu_seqlens_new", torch.int32, 1)
    _dev(cache_pos, "cache_pos", torch.int32, 1)
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    if k_new.stride() != v_new.stride() or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must share shape and strides")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_new.stride(2) != 1 or k_cache.stride(3) != 1:
        raise ValueError("the new rows and the caches need unit stride along head_dim")
    B, Hkv, max_ctx, D = k_cache.shape
    S = cu_seqlens_new.numel() - 1
    if cache_pos.numel() != S or k_new.shape[1] != Hkv or k_new.shape[2] != D:
        raise ValueError("shapes of the new rows, cu_seqlens_new, cache_pos and caches disagree")
    if S > B:
        raise ValueError("more sequences than cache rows")
    if max_new is None:
        max_new = k_new.shape[0]
    rc = load_library().sink_attn_kv_append(
        k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_new.stride(1),
        cu_seqlens_new.data_ptr(), cache_pos.data_ptr(), S, int(max_new), k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), max_ctx,
        Hkv, D, _stream(stream))
    _check("sink_attn_kv_append", rc)
    return k_cache, v_cache


# ------------------------------------------------------------- FP8 caches --
def _fp8_scales(k_scale, v_scale, Hkv):
    for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, nm, torch.float32, 1)
        if t.numel() != Hkv or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous fp32 tensor of num_kv_heads ({Hkv}) scales")


def sink_attn_decode_multi_split_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, sinks,
                                     split_size, num_splits=None, *, max_ctx=None, scale=None,
                                     part_o=None, part_m=None, part_d=None, stream=None):
    """sink_attn_decode_multi_split over FP8 E4M3 caches (uint8 codes
    [B, Hkv, max_ctx, D]) with per-KV-head scales k_scale, v_scale [Hkv] fp32.
    q: [B, q_len, Hq, D] bf16.  Returns the chunk states, as the bf16 form."""
    _dev(q, "q", torch.bfloat16, 4)
    _dev(k_cache, "k_cache", torch.uint8, 4)
    _dev(v_cache, "v_cache", torch.uint8, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, q_len, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    _fp8_scales(k_scale, v_scale, Hkv)
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    shape = (B, q_len, Hq, num_splits)
    if part_o is None:
        part_o = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        part_m = torch.empty(shape, dtype=torch.float32, device=q.device)
        part_d = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((part_o, "part_o", shape + (D,)), (part_m, "part_m", shape),
                       (part_d, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be contiguous with shape {shp}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_multi_split_fp8(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), q_len, k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        k_scale.data_ptr(), v_scale.data_ptr(), seq_lens.data_ptr(), B, max_ctx,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits),
        part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(), _stream(stream))
    _check("sink_attn_decode_multi_split_fp8", rc)
    return part_o, part_m, part_d


def sink_attn_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, sinks, split_size,
                         num_splits=None, *, max_ctx=None, scale=None, out=None, lse=None,
                         partials=None, stream=None):
    """Decode over FP8 caches: q [B, Hq, D] (one new token) or [B, q_len, Hq, D];
    sink_attn_decode_multi_split_fp8 then sink_attn_merge_states on one stream.
    Returns out shaped like q (bf16)."""
    q4 = q.unsqueeze(1) if q.dim() == 3 else q
    B, q_len, Hq, D = q4.shape
    po, pm, pd = partials if partials is not None else (None, None, None)
    po, pm, pd = sink_attn_decode_multi_split_fp8(
        q4, k_cache, v_cache, k_scale, v_scale, seq_lens, sinks, split_size, num_splits,
        max_ctx=max_ctx, scale=scale, part_o=po, part_m=pm, part_d=pd, stream=stream)
    S = po.shape[3]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    out4 = out.unsqueeze(1) if out.dim() == 3 else out
    if tuple(out4.shape) != (B, q_len, Hq, D) or out4.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride along head_dim")
    if q_len == 1:
        merged = out4[:, 0]
    else:
        if not out4.is_contiguous():
            raise ValueError("out must be contiguous when q_len > 1")
        merged = out4.view(B * q_len, Hq, D)
    sink_attn_merge_states(po.view(B * q_len, Hq, S, D), pm.view(B * q_len, Hq, S),
                           pd.view(B * q_len, Hq, S), out=merged, lse=lse, stream=stream)
    return out


def sink_attn_kv_append_fp8(k_new, v_new, cu_seqlens_new, cache_pos, k_cache, v_cache, k_scale,
                            v_scale, *, max_new=None, stream=None):
    """sink_attn_kv_append into FP8 E4M3 caches (uint8 [B, Hkv, max_ctx, D]):
    each bf16 row of KV head g is quantized with 1 / k_scale[g] (v_scale[g])."""
    _dev(k_new, "k_new", torch.bfloat16, 3)
    _dev(v_new, "v_new", torch.bfloat16, 3)
    _dev(cu_seqlens_new, "cu_seqlens_new", torch.int32, 1)
    _dev(cache_pos, "cache_pos", torch.int32, 1)
    _dev(k_cache, "k_cache", torch.uint8, 4)
    _dev(v_cache, "v_cache", torch.uint8, 4)
    if k_new.stride() != v_new.stride() or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must share shape and strides")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_new.stride(2) != 1 or k_cache.stride(3) != 1:
        raise ValueError("the new rows and the caches need unit stride along head_dim")
    B, Hkv, max_ctx, D = k_cache.shape
    _fp8_scales(k_scale, v_scale, Hkv)
    S = cu_seqlens_new.numel() - 1
    if cache_pos.numel() != S or k_new.shape[1] != Hkv or k_new.shape[2] != D:
        raise ValueError("shapes of the new rows, cu_seqlens_new, cache_pos and caches disagree")
    if S > B:
        raise ValueError("more sequences than cache rows")
    if max_new is None:
        max_new = k_new.shape[0]
    rc = load_library().sink_attn_kv_append_fp8(
        k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_new.stride(1),
        cu_seqlens_new.data_ptr(), cache_pos.data_ptr(), S, int(max_new), k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        k_scale.data_ptr(), v_scale.data_ptr(), max_ctx, Hkv, D, _stream(stream))
    _check("sink_attn_kv_append_fp8", rc)
    return k_cache, v_cache


# ------------------------------------------------------------ paged caches --
def _paged_common(k_pages, v_pages, block_tables, k_scale, v_scale):
    dtype = torch.bfloat16 if k_scale is None else torch.uint8
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale (FP8 pages) or neither (bf16 pages)")
    _dev(k_pages, "k_pages", dtype, 4)
    _dev(v_pages, "v_pages", dtype, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    if k_pages.stride() != v_pages.stride() or k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages must share shape and strides")
    if k_pages.stride(3) != 1 or block_tables.stride(1) != 1:
        raise ValueError("pages need unit stride along head_dim, block_tables along its rows")
    if k_scale is not None:
        _fp8_scales(k_scale, v_scale, k_pages.shape[1])


def sink_attn_decode_paged_split(q, k_pages, v_pages, block_tables, seq_lens, sinks, split_size,
                                 num_splits=None, *, k_scale=None, v_scale=None, scale=None,
                                 part_o=None, part_m=None, part_d=None, stream=None):
    """Chunk states of (multi-token) decode over a paged cache: pages
    [num_pages, Hkv, page_size, D] (bf16, or FP8 E4M3 codes with k_scale /
    v_scale), block_tables [B, pages_per_seq] int32; q [B, q_len, Hq, D]."""
    _dev(q, "q", torch.bfloat16, 4)
    _paged_common(k_pages, v_pages, block_tables, k_scale, v_scale)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if q.stride(3) != 1:
        raise ValueError("q needs unit stride along head_dim")
    B, q_len, Hq, D = q.shape
    _, Hkv, P, _ = k_pages.shape
    pages_per_seq = block_tables.shape[1]
    if block_tables.shape[0] < B:
        raise ValueError("block_tables needs a row per request")
    if num_splits is None:
        num_splits = -(-(pages_per_seq * P) // split_size)
    shape = (B, q_len, Hq, num_splits)
    if part_o is None:
        part_o = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        part_m = torch.empty(shape, dtype=torch.float32, device=q.device)
        part_d = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((part_o, "part_o", shape + (D,)), (part_m, "part_m", shape),
                       (part_d, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be contiguous with shape {shp}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_paged_split(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), q_len, k_pages.data_ptr(),
        v_pages.data_ptr(), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2), P,
        block_tables.data_ptr(), block_tables.stride(0), pages_per_seq,
        None if k_scale is None else k_scale.data_ptr(),
        None if v_scale is None else v_scale.data_ptr(), seq_lens.data_ptr(), B,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits),
        part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(), _stream(stream))
    _check("sink_attn_decode_paged_split", rc)
    return part_o, part_m, part_d


def sink_attn_decode_paged(q, k_pages, v_pages, block_tables, seq_lens, sinks, split_size,
                           num_splits=None, *, k_scale=None, v_scale=None, scale=None, out=None,
                           lse=None, partials=None, stream=None):
    """Decode over a paged cache: sink_attn_decode_paged_split then
    sink_attn_merge_states on one stream.  q [B, Hq, D] or [B, q_len, Hq, D];
    returns out shaped like q (bf16)."""
    q4 = q.unsqueeze(1) if q.dim() == 3 else q
    B, q_len, Hq, D = q4.shape
    po, pm, pd = partials if partials is not None else (None, None, None)
    po, pm, pd = sink_attn_decode_paged_split(
        q4, k_pages, v_pages, block_tables, seq_lens, sinks, split_size, num_splits,
        k_scale=k_scale, v_scale=v_scale, scale=scale, part_o=po, part_m=pm, part_d=pd,
        stream=stream)
    S = po.shape[3]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    out4 = out.unsqueeze(1) if out.dim() == 3 else out
    if tuple(out4.shape) != (B, q_len, Hq, D) or out4.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride along head_dim")
    if q_len == 1:
        merged = out4[:, 0]
    else:
        if not out4.is_contiguous():
            raise ValueError("out must be contiguous when q_len > 1")
        merged = out4.view(B * q_len, Hq, D)
    sink_attn_merge_states(po.view(B * q_len, Hq, S, D), pm.view(B * q_len, Hq, S),
                           pd.view(B * q_len, Hq, S), out=merged, lse=lse, stream=stream)
    return out


def sink_attn_kv_append_paged(k_new, v_new, cu_seqlens_new, cache_pos, k_pages, v_pages,
                              block_tables, *, k_scale=None, v_scale=None, max_new=None,
                              stream=None):
    """Append new tokens' K/V rows [T, Hkv, D] into a paged cache through its
    block table (a copy into bf16 pages, or quantizing into FP8 pages)."""
    _dev(k_new, "k_new", torch.bfloat16, 3)
    _dev(v_new, "v_new", torch.bfloat16, 3)
    _dev(cu_seqlens_new, "cu_seqlens_new", torch.int32, 1)
    _dev(cache_pos, "cache_pos", torch.int32, 1)
    _paged_common(k_pages, v_pages, block_tables, k_scale, v_scale)
    if k_new.stride() != v_new.stride() or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must share shape and strides")
    if k_new.stride(2) != 1:
        raise ValueError("the new rows need unit stride along head_dim")
    _, Hkv, P, D = k_pages.shape
    S = cu_seqlens_new.numel() - 1
    if cache_pos.numel() != S or k_new.shape[1] != Hkv or k_new.shape[2] != D:
        raise ValueError("shapes of the new rows, cu_seqlens_new, cache_pos and pages disagree")
    if block_tables.shape[0] < S:
        raise ValueError("block_tables needs a row per request")
    if max_new is None:
        max_new = k_new.shape[0]
    rc = load_library().sink_attn_kv_append_paged(
        k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_new.stride(1),
        cu_seqlens_new.data_ptr(), cache_pos.data_ptr(), S, int(max_new), k_pages.data_ptr(),
        v_pages.data_ptr(), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2), P,
        block_tables.data_ptr(), block_tables.stride(0), block_tables.shape[1],
        None if k_scale is None else k_scale.data_ptr(),
        None if v_scale is None else v_scale.data_ptr(), Hkv, D, _stream(stream))
    _check("sink_attn_kv_append_paged", rc)
    return k_pages, v_pages


def sink_attn_decode_split_size(batch, max_ctx, num_q_heads, num_kv_heads, head_dim, q_len=1,
                                seq_lens=None):
    """Tokens per chunk for split-KV decode of this launch shape (the library's
    choice).  seq_lens: the request lengths on the host (list, array or CPU
    tensor) when the caller has them -- equal lengths get long chunks -- else
    None (treated as ragged)."""
    ptr, keep = None, None
    if seq_lens is not None:
        keep = torch.as_tensor(seq_lens, dtype=torch.int32).cpu().contiguous()
        if keep.numel() != int(batch):
            raise ValueError("seq_lens needs one length per request")
        ptr = keep.data_ptr()
    rc = load_library().sink_attn_decode_split_size(int(batch), int(max_ctx), int(q_len),
                                                    int(num_q_heads), int(num_kv_heads),
                                                    int(head_dim), ptr)
    if rc <= 0:
        _check("sink_attn_decode_split_size", rc if rc != 0 else -1)
    return int(rc)


# ------------------------------------------------------- one-launch decode --
def decode_counters(batch, num_q_heads, num_kv_heads, q_len=1, device="cuda"):
    """Zeroed arrival counters for sink_attn_decode_fused, sized for the shape
    (each call leaves them zero again, so one buffer serves every call)."""
    n = batch * num_kv_heads * -(-(q_len * (num_q_heads // num_kv_heads)) // 16)
    return torch.zeros(max(n, 1), dtype=torch.int32, device=device)


def sink_attn_decode_fused(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits=None, *,
                           k_scale=None, v_scale=None, counters=None, max_ctx=None, scale=None,
                           out=None, lse=None, partials=None, stream=None):
    """Split decode and merge in one launch (bf16 caches, or FP8 E4M3 code
    caches with k_scale / v_scale).  q [B, Hq, D] or [B, q_len, Hq, D];
    returns out shaped like q (bf16)."""
    q4 = q.unsqueeze(1) if q.dim() == 3 else q
    _dev(q4, "q", torch.bfloat16, 4)
    f8 = k_scale is not None
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale (FP8 caches) or neither (bf16 caches)")
    _dev(k_cache, "k_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q4.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, q_len, Hq, D = q4.shape
    Hkv = k_cache.shape[1]
    if f8:
        _fp8_scales(k_scale, v_scale, Hkv)
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    shape = (B, q_len, Hq, num_splits)
    po, pm, pd = partials if partials is not None else (None, None, None)
    if po is None:
        po = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        pm = torch.empty(shape, dtype=torch.float32, device=q.device)
        pd = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((po, "part_o", shape + (D,)), (pm, "part_m", shape), (pd, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or t.numel() != math.prod(shp):
            raise ValueError(f"{nm} must be contiguous with {math.prod(shp)} elements")
    if counters is None:
        counters = decode_counters(B, Hq, Hkv, q_len, q.device)
    _dev(counters, "counters", torch.int32, 1)
    if counters.numel() < B * Hkv * -(-(q_len * (Hq // Hkv)) // 16):
        raise ValueError("counters is too small for this shape")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    out4 = out.unsqueeze(1) if out.dim() == 3 else out
    _dev(out4, "out", torch.bfloat16, 4)
    if tuple(out4.shape) != (B, q_len, Hq, D) or out4.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride along head_dim")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if not lse.is_contiguous() or lse.numel() != B * q_len * Hq:
            raise ValueError("lse must be a contiguous fp32 tensor of B * q_len * Hq rows")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_fused(
        q4.data_ptr(), q4.stride(0), q4.stride(1), q4.stride(2), q_len, k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        None if k_scale is None else k_scale.data_ptr(),
        None if v_scale is None else v_scale.data_ptr(), seq_lens.data_ptr(), B, max_ctx,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits), po.data_ptr(),
        pm.data_ptr(), pd.data_ptr(), counters.data_ptr(), out4.data_ptr(), out4.stride(0),
        out4.stride(1), out4.stride(2), lse.data_ptr() if lse is not None else None,
        _stream(stream))
    _check("sink_attn_decode_fused", rc)
    return out


def sink_attn_decode_merged(q, k_cache, v_cache, seq_lens, sinks, split_size, num_splits=None, *,
                            k_scale=None, v_scale=None, max_ctx=None, scale=None, out=None,
                            lse=None, partials=None, stream=None):
    """Split decode and a merge that stops at each request's last chunk with
    keys (two launches; chunks past a request's end write no state).  bf16
    caches, or FP8 E4M3 code caches with k_scale / v_scale.  q [B, Hq, D] or
    [B, q_len, Hq, D]; returns out shaped like q (bf16), bitwise the output of
    split decode + sink_attn_merge_states."""
    q4 = q.unsqueeze(1) if q.dim() == 3 else q
    _dev(q4, "q", torch.bfloat16, 4)
    f8 = k_scale is not None
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale (FP8 caches) or neither (bf16 caches)")
    _dev(k_cache, "k_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q4.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, q_len, Hq, D = q4.shape
    Hkv = k_cache.shape[1]
    if f8:
        _fp8_scales(k_scale, v_scale, Hkv)
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    shape = (B, q_len, Hq, num_splits)
    po, pm, pd = partials if partials is not None else (None, None, None)
    if po is None:
        po = torch.empty(*shape, D, dtype=torch.float32, device=q.device)
        pm = torch.empty(shape, dtype=torch.float32, device=q.device)
        pd = torch.empty(shape, dtype=torch.float32, device=q.device)
    for t, nm, shp in ((po, "part_o", shape + (D,)), (pm, "part_m", shape), (pd, "part_d", shape)):
        _dev(t, nm, torch.float32)
        if not t.is_contiguous() or t.numel() != math.prod(shp):
            raise ValueError(f"{nm} must be contiguous with {math.prod(shp)} elements")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    out4 = out.unsqueeze(1) if out.dim() == 3 else out
    _dev(out4, "out", torch.bfloat16, 4)
    if tuple(out4.shape) != (B, q_len, Hq, D) or out4.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride along head_dim")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if not lse.is_contiguous() or lse.numel() != B * q_len * Hq:
            raise ValueError("lse must be a contiguous fp32 tensor of B * q_len * Hq rows")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_merged(
        q4.data_ptr(), q4.stride(0), q4.stride(1), q4.stride(2), q_len, k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        None if k_scale is None else k_scale.data_ptr(),
        None if v_scale is None else v_scale.data_ptr(), seq_lens.data_ptr(), B, max_ctx,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits), po.data_ptr(),
        pm.data_ptr(), pd.data_ptr(), out4.data_ptr(), out4.stride(0),
        out4.stride(1), out4.stride(2), lse.data_ptr() if lse is not None else None,
        _stream(stream))
    _check("sink_attn_decode_merged", rc)
    return out


def sink_attn_decode_merged_noalloc(q, k_cache, v_cache, seq_lens, sinks, split_size,
                                    num_splits=None, *, k_scale=None, v_scale=None, max_ctx=None,
                                    scale=None, out=None, lse=None, stream=None):
    """sink_attn_decode_merged with its chunk states in the library's device
    scratch array (128 MiB per GPU): the call allocates nothing, for callers
    that cannot (graph capture, serving loops).  Pass `out` (and `lse`) to keep
    this wrapper from allocating them.  Calls that overlap on one GPU race."""
    q4 = q.unsqueeze(1) if q.dim() == 3 else q
    _dev(q4, "q", torch.bfloat16, 4)
    f8 = k_scale is not None
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale (FP8 caches) or neither (bf16 caches)")
    _dev(k_cache, "k_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.uint8 if f8 else torch.bfloat16, 4)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if q4.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches need unit stride along head_dim")
    B, q_len, Hq, D = q4.shape
    Hkv = k_cache.shape[1]
    if f8:
        _fp8_scales(k_scale, v_scale, Hkv)
    max_ctx = k_cache.shape[2] if max_ctx is None else int(max_ctx)
    if num_splits is None:
        num_splits = -(-max_ctx // split_size)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    out4 = out.unsqueeze(1) if out.dim() == 3 else out
    _dev(out4, "out", torch.bfloat16, 4)
    if tuple(out4.shape) != (B, q_len, Hq, D) or out4.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride along head_dim")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if not lse.is_contiguous() or lse.numel() != B * q_len * Hq:
            raise ValueError("lse must be a contiguous fp32 tensor of B * q_len * Hq rows")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().sink_attn_decode_merged_noalloc(
        q4.data_ptr(), q4.stride(0), q4.stride(1), q4.stride(2), q_len, k_cache.data_ptr(),
        v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        None if k_scale is None else k_scale.data_ptr(),
        None if v_scale is None else v_scale.data_ptr(), seq_lens.data_ptr(), B, max_ctx,
        sinks.data_ptr(), Hq, Hkv, D, scale, int(split_size), int(num_splits), out4.data_ptr(),
        out4.stride(0), out4.stride(1), out4.stride(2),
        lse.data_ptr() if lse is not None else None, _stream(stream))
    _check("sink_attn_decode_merged_noalloc", rc)
    return out
