"""CPU-side checks of the C ABI: the library loads, exports every symbol that
include/sinkattn.h declares, and rejects bad arguments on the host before any
HIP call (so these run without a GPU; no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import gqa_attention_sinks_prefill_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sa.library_path()),
                                reason="libsinkattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sink_attn_\w+)\s*\(", text)))


def test_header_declares_the_exported_api():
    assert declared_functions() == sorted(sa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = sa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _prefill(**kw):
    args = dict(q=16, q_st=512, q_sh=64, k=16, k_st=64, k_sh=64 * 256, v=16, v_st=64,
                v_sh=64 * 256, sinks=4, cu=4, num_seqs=1, max_seqlen=256, hq=8, hkv=2, d=64,
                scale=0.125, causal=1, o=16, o_st=512, o_sh=64, lse=None)
    args.update(kw)
    a = args
    lib = sa.load_library()
    rc = lib.sink_attn_prefill(a["q"], a["q_st"], a["q_sh"], a["k"], a["k_st"], a["k_sh"],
                               a["v"], a["v_st"], a["v_sh"], a["sinks"], a["cu"], a["num_seqs"],
                               a["max_seqlen"], a["hq"], a["hkv"], a["d"], a["scale"],
                               a["causal"], a["o"], a["o_st"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


# Fake, never-dereferenced "device" addresses: every case below must fail in
# validation, before anything touches them.
@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), -1, "null"),
    (dict(o=None), -1, "null"),
    (dict(cu=None), -1, "null"),
    (dict(hq=6, hkv=4), -1, "multiple"),
    (dict(hkv=0), -1, "positive"),
    (dict(d=96), -2, "head_dim"),
    (dict(d=256), -2, "head_dim"),
    (dict(q=24), -1, "aligned"),
    (dict(sinks=6), -1, "aligned"),
    (dict(k_st=60), -1, "multiples of 8"),
    (dict(o_sh=-8), -1, "multiples of 8"),
    (dict(num_seqs=-1), -1, ">= 0"),
    (dict(causal=2), -1, "causal"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
])
def test_prefill_rejects_bad_arguments(kw, code, needle):
    rc, msg = _prefill(**kw)
    assert rc == code
    assert needle in msg


def test_prefill_empty_work_is_a_noop():
    assert _prefill(num_seqs=0, q=None, o=None)[0] == 0
    assert _prefill(max_seqlen=0)[0] == 0


def _prefill_chunked(**kw):
    a = dict(q=16, q_st=512, q_sh=64, k=16, k_st=64, k_sh=64 * 256, v=16, v_st=64,
             v_sh=64 * 256, sinks=4, cuq=4, cuk=4, num_seqs=1, max_seqlen=256, hq=8, hkv=2,
             d=64, scale=0.125, causal=1, o=16, o_st=512, o_sh=64, lse=None)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_prefill_chunked(a["q"], a["q_st"], a["q_sh"], a["k"], a["k_st"],
                                       a["k_sh"], a["v"], a["v_st"], a["v_sh"], a["sinks"],
                                       a["cuq"], a["cuk"], a["num_seqs"], a["max_seqlen"],
                                       a["hq"], a["hkv"], a["d"], a["scale"], a["causal"],
                                       a["o"], a["o_st"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(cuk=None), -1, "null"),
    (dict(cuq=None), -1, "null"),
    (dict(cuk=6), -1, "aligned"),
    (dict(d=32), -2, "head_dim"),
    (dict(causal=-1), -1, "causal"),
])
def test_prefill_chunked_rejects_bad_arguments(kw, code, needle):
    rc, msg = _prefill_chunked(**kw)
    assert rc == code
    assert needle in msg


def test_prefill_chunked_empty_work_is_a_noop():
    assert _prefill_chunked(num_seqs=0, q=None, cuk=None)[0] == 0


def _decode(**kw):
    a = dict(q=16, q_sb=4096, q_sh=64, k=16, v=16, kv_sb=8 * 1024 * 64, kv_sh=1024 * 64,
             kv_st=64, lens=4, batch=4, max_ctx=1024, sinks=4, hq=64, hkv=8, d=64,
             scale=0.125, split=256, nsplit=4, po=4, pm=4, pd=4)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_split(a["q"], a["q_sb"], a["q_sh"], a["k"], a["v"], a["kv_sb"],
                                    a["kv_sh"], a["kv_st"], a["lens"], a["batch"], a["max_ctx"],
                                    a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"],
                                    a["split"], a["nsplit"], a["po"], a["pm"], a["pd"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(k=None), -1, "null"),
    (dict(pd=None), -1, "null"),
    (dict(split=100), -1, "split_size"),
    (dict(split=0), -1, "split_size"),
    (dict(nsplit=3), -1, "cover"),
    (dict(nsplit=0), -1, "num_splits"),
    (dict(hq=12), -1, "multiple"),
    (dict(d=80), -2, "head_dim"),
    (dict(v=8), -1, "aligned"),
    (dict(kv_st=66), -1, "multiples of 8"),
    (dict(batch=-2), -1, ">= 0"),
])
def test_decode_split_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode(**kw)
    assert rc == code
    assert needle in msg


def test_decode_split_empty_batch_is_a_noop():
    assert _decode(batch=0, q=None)[0] == 0


def _decode_multi(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=4, k=16, v=16,
             kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, lens=4, batch=4, max_ctx=1024,
             sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4, po=4, pm=4, pd=4)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_multi_split(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["kv_sb"],
        a["kv_sh"], a["kv_st"], a["lens"], a["batch"], a["max_ctx"], a["sinks"], a["hq"],
        a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"], a["po"], a["pm"], a["pd"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q_len=0), -1, "q_len"),
    (dict(q_len=-3), -1, "q_len"),
    (dict(q_st=100), -1, "multiples of 8"),
    (dict(q_st=-8), -1, "multiples of 8"),
    (dict(q=None), -1, "null"),
    (dict(split=96), -1, "split_size"),
    (dict(nsplit=2), -1, "cover"),
    (dict(hq=60), -1, "multiple"),
    (dict(d=32), -2, "head_dim"),
    (dict(k=40), -1, "aligned"),
])
def test_decode_multi_split_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode_multi(**kw)
    assert rc == code
    assert needle in msg


def test_decode_multi_split_empty_batch_is_a_noop():
    assert _decode_multi(batch=0, q=None)[0] == 0


def _kv_append(**kw):
    a = dict(kn=16, vn=32, n_st=512, n_sh=64, cu=4, pos=8, num_seqs=2, max_new=100, kc=48,
             vc=64, kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, max_ctx=1024, hkv=8, d=64)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_kv_append(a["kn"], a["vn"], a["n_st"], a["n_sh"], a["cu"], a["pos"],
                                 a["num_seqs"], a["max_new"], a["kc"], a["vc"], a["kv_sb"],
                                 a["kv_sh"], a["kv_st"], a["max_ctx"], a["hkv"], a["d"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(kn=None), -1, "null"),
    (dict(pos=None), -1, "null"),
    (dict(kc=40), -1, "aligned"),
    (dict(cu=6), -1, "aligned"),
    (dict(n_st=100), -1, "multiples of 8"),
    (dict(hkv=0), -1, "positive"),
    (dict(d=96), -2, "head_dim"),
    (dict(max_new=-1), -1, ">= 0"),
    (dict(vc=48), -1, "alias"),
])
def test_kv_append_rejects_bad_arguments(kw, code, needle):
    rc, msg = _kv_append(**kw)
    assert rc == code
    assert needle in msg


def test_kv_append_empty_work_is_a_noop():
    assert _kv_append(num_seqs=0, kn=None)[0] == 0
    assert _kv_append(max_new=0)[0] == 0


def _decode_multi_fp8(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=4, k=16, v=16,
             kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, ks=4, vs=8, lens=4, batch=4,
             max_ctx=1024, sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4, po=4,
             pm=4, pd=4)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_multi_split_fp8(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["kv_sb"],
        a["kv_sh"], a["kv_st"], a["ks"], a["vs"], a["lens"], a["batch"], a["max_ctx"],
        a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"], a["po"],
        a["pm"], a["pd"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=None), -1, "k_scale"),
    (dict(vs=None), -1, "k_scale"),
    (dict(ks=6), -1, "aligned"),
    (dict(kv_st=72), -1, "multiples of 16"),
    (dict(kv_sh=1024 * 64 + 8), -1, "multiples of 16"),
    (dict(kv_st=1 << 22, split=1024), -2, "2 GiB"),
    (dict(q_len=0), -1, "q_len"),
    (dict(q_st=100), -1, "multiples of 8"),
    (dict(q=None), -1, "null"),
    (dict(split=96), -1, "split_size"),
    (dict(nsplit=2), -1, "cover"),
    (dict(d=32), -2, "head_dim"),
    (dict(k=40), -1, "aligned"),
])
def test_decode_multi_split_fp8_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode_multi_fp8(**kw)
    assert rc == code
    assert needle in msg


def test_decode_multi_split_fp8_empty_batch_is_a_noop():
    assert _decode_multi_fp8(batch=0, q=None)[0] == 0


def _decode_fused(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=4, k=16, v=16,
             kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, ks=None, vs=None, lens=4, batch=4,
             max_ctx=1024, sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4, po=4,
             pm=4, pd=4, cnt=4, o=32, o_sb=4 * 4096, o_st=4096, o_sh=64, lse=None)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_fused(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["kv_sb"],
        a["kv_sh"], a["kv_st"], a["ks"], a["vs"], a["lens"], a["batch"], a["max_ctx"],
        a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"], a["po"],
        a["pm"], a["pd"], a["cnt"], a["o"], a["o_sb"], a["o_st"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=4), -1, "both"),
    (dict(vs=4), -1, "both"),
    (dict(cnt=None), -1, "null"),
    (dict(o=None), -1, "null"),
    (dict(cnt=6), -1, "aligned"),
    (dict(o=40), -1, "aligned"),
    (dict(lse=6), -1, "aligned"),
    (dict(o_st=100), -1, "multiples of 8"),
    (dict(o_sh=-8), -1, "multiples of 8"),
    (dict(ks=4, vs=8, kv_st=72), -1, "multiples of 16"),
    (dict(q_len=0), -1, "q_len"),
    (dict(nsplit=2), -1, "cover"),
    (dict(d=32), -2, "head_dim"),
])
def test_decode_fused_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode_fused(**kw)
    assert rc == code
    assert needle in msg


def test_decode_fused_empty_batch_is_a_noop():
    assert _decode_fused(batch=0, q=None, cnt=None, o=None)[0] == 0


def test_prefill_sequence_span_must_fit_32_bits():
    lib = sa.load_library()
    # NHD keys with a 1M-element token stride: 4096 tokens span 8 GiB
    rc = lib.sink_attn_prefill(16, 512, 64, 16, 1 << 20, 64, 16, 1 << 20, 64, 4, 4, 1, 4096, 8,
                               8, 64, 0.125, 1, 16, 512, 64, None, None)
    assert rc == -2 and "2 GiB" in lib.sink_attn_last_error().decode()


def test_decode_split_size_times_stride_must_fit_32_bits():
    rc, msg = _decode_multi(kv_st=1 << 21, split=1024)
    assert rc == -2 and "2 GiB" in msg


def _kv_append_fp8(**kw):
    a = dict(kn=16, vn=32, n_st=512, n_sh=64, cu=4, pos=8, num_seqs=2, max_new=100, kc=48,
             vc=64, kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, ks=4, vs=8, max_ctx=1024,
             hkv=8, d=64)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_kv_append_fp8(a["kn"], a["vn"], a["n_st"], a["n_sh"], a["cu"], a["pos"],
                                     a["num_seqs"], a["max_new"], a["kc"], a["vc"], a["kv_sb"],
                                     a["kv_sh"], a["kv_st"], a["ks"], a["vs"], a["max_ctx"],
                                     a["hkv"], a["d"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=None), -1, "k_scale"),
    (dict(vs=None), -1, "k_scale"),
    (dict(vs=6), -1, "aligned"),
    (dict(kn=None), -1, "null"),
    (dict(kc=40), -1, "aligned"),
    (dict(d=96), -2, "head_dim"),
    (dict(vc=48), -1, "alias"),
])
def test_kv_append_fp8_rejects_bad_arguments(kw, code, needle):
    rc, msg = _kv_append_fp8(**kw)
    assert rc == code
    assert needle in msg


def test_kv_append_fp8_empty_work_is_a_noop():
    assert _kv_append_fp8(num_seqs=0, kn=None)[0] == 0


def _decode_paged(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=1, k=16, v=16, sp=8 * 16 * 64,
             kv_sh=16 * 64, kv_st=64, ps=16, bt=4, bt_st=64, pps=64, ks=None, vs=None, lens=4,
             batch=4, sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4, po=4, pm=4,
             pd=4)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_paged_split(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["sp"], a["kv_sh"],
        a["kv_st"], a["ps"], a["bt"], a["bt_st"], a["pps"], a["ks"], a["vs"], a["lens"],
        a["batch"], a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"],
        a["po"], a["pm"], a["pd"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ps=24), -1, "power of two"),
    (dict(ps=8), -1, "power of two"),
    (dict(ps=0), -1, "power of two"),
    (dict(bt=None), -1, "null"),
    (dict(bt=6), -1, "aligned"),
    (dict(bt_st=-1), -1, ">= 0"),
    (dict(pps=-1), -1, ">= 0"),
    (dict(pps=1 << 27, ps=32), -2, "2^31"),
    (dict(ks=4), -1, "both"),
    (dict(split=8192, nsplit=1, ps=16), -2, "255 pages"),
    (dict(nsplit=2), -1, "cover"),
    (dict(kv_st=68), -1, "multiples of 8"),
    (dict(ks=4, vs=8, kv_st=72), -1, "multiples of 16"),
    (dict(d=32), -2, "head_dim"),
])
def test_decode_paged_split_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode_paged(**kw)
    assert rc == code
    assert needle in msg


def test_decode_paged_split_empty_batch_is_a_noop():
    assert _decode_paged(batch=0, q=None)[0] == 0


def _kv_append_paged(**kw):
    a = dict(kn=16, vn=32, n_st=512, n_sh=64, cu=4, pos=8, num_seqs=2, max_new=100, kc=48,
             vc=64, sp=8 * 16 * 64, kv_sh=16 * 64, kv_st=64, ps=16, bt=4, bt_st=64, pps=64,
             ks=None, vs=None, hkv=8, d=64)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_kv_append_paged(a["kn"], a["vn"], a["n_st"], a["n_sh"], a["cu"], a["pos"],
                                       a["num_seqs"], a["max_new"], a["kc"], a["vc"], a["sp"],
                                       a["kv_sh"], a["kv_st"], a["ps"], a["bt"], a["bt_st"],
                                       a["pps"], a["ks"], a["vs"], a["hkv"], a["d"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ps=48), -1, "power of two"),
    (dict(bt=None), -1, "null"),
    (dict(bt=2), -1, "aligned"),
    (dict(vs=8), -1, "both"),
    (dict(kn=None), -1, "null"),
    (dict(d=96), -2, "head_dim"),
])
def test_kv_append_paged_rejects_bad_arguments(kw, code, needle):
    rc, msg = _kv_append_paged(**kw)
    assert rc == code
    assert needle in msg


def test_kv_append_paged_empty_work_is_a_noop():
    assert _kv_append_paged(num_seqs=0, kn=None)[0] == 0
    assert _kv_append_paged(pps=0)[0] == 0


def _merge(**kw):
    a = dict(po=4, pm=4, pd=4, batch=2, hq=8, ns=4, d=64, o=16, o_sb=512, o_sh=64, lse=None)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_merge_states(a["po"], a["pm"], a["pd"], a["batch"], a["hq"], a["ns"],
                                    a["d"], a["o"], a["o_sb"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(po=None), -1, "null"),
    (dict(o=None), -1, "null"),
    (dict(ns=0), -1, "num_splits"),
    (dict(hq=0), -1, "num_q_heads"),
    (dict(d=32), -2, "head_dim"),
    (dict(o=18), -1, "aligned"),
    (dict(lse=6), -1, "aligned"),
    (dict(o_sh=3), -1, "multiples of 8"),
])
def test_merge_rejects_bad_arguments(kw, code, needle):
    rc, msg = _merge(**kw)
    assert rc == code
    assert needle in msg


def test_error_message_clears_on_success():
    _merge(po=None)
    assert sa.load_library().sink_attn_last_error() != b""
    assert _merge(batch=0)[0] == 0
    assert sa.load_library().sink_attn_last_error() == b""


def test_python_binding_requires_gpu_tensors():
    import torch
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sa.sink_attn_prefill(q, q, q, torch.zeros(2), torch.zeros(2, dtype=torch.int32), 4)


def _decode_merged(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=4, k=16, v=16,
             kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, ks=None, vs=None, lens=4, batch=4,
             max_ctx=1024, sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4, po=4,
             pm=4, pd=4, o=32, o_sb=4 * 4096, o_st=4096, o_sh=64, lse=None)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_merged(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["kv_sb"],
        a["kv_sh"], a["kv_st"], a["ks"], a["vs"], a["lens"], a["batch"], a["max_ctx"],
        a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"], a["po"],
        a["pm"], a["pd"], a["o"], a["o_sb"], a["o_st"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=4), -1, "both"),
    (dict(o=None), -1, "null"),
    (dict(o=40), -1, "aligned"),
    (dict(lse=6), -1, "aligned"),
    (dict(o_st=100), -1, "multiples of 8"),
    (dict(q_len=0), -1, "q_len"),
    (dict(nsplit=2), -1, "cover"),
    (dict(d=32), -2, "head_dim"),
])
def test_decode_merged_rejects_bad_arguments(kw, code, needle):
    rc, msg = _decode_merged(**kw)
    assert rc == code and needle in msg, (rc, msg)


def test_decode_merged_empty_batch_is_a_noop():
    rc, msg = _decode_merged(batch=0, q=None, k=None, v=None, lens=None, sinks=None, po=None,
                             pm=None, pd=None, o=None)
    assert rc == 0, msg


@pytest.mark.parametrize("kw,code,needle", [
    (dict(batch=-1), -1, ">= 0"),
    (dict(max_ctx=-5), -1, ">= 0"),
    (dict(q_len=0), -1, "q_len"),
    (dict(hq=6, hkv=4), -1, "multiple"),
    (dict(d=96), -2, "head_dim"),
    (dict(lens=[100] * 7 + [40000]), -1, "outside"),
    (dict(lens=[100] * 7 + [-1]), -1, "outside"),
])
def test_decode_split_size_rejects_bad_arguments(kw, code, needle):
    a = dict(batch=8, max_ctx=32768, q_len=1, hq=64, hkv=8, d=64, lens=None)
    a.update(kw)
    lib = sa.load_library()
    lens = None if a["lens"] is None else (ctypes.c_int32 * len(a["lens"]))(*a["lens"])
    rc = lib.sink_attn_decode_split_size(a["batch"], a["max_ctx"], a["q_len"], a["hq"], a["hkv"],
                                         a["d"], lens)
    assert rc == code and needle in lib.sink_attn_last_error().decode()


def test_decode_split_size_follows_the_launch_shape():
    # host only: no device work is enqueued (without a GPU the CU count
    # falls back to the MI355X's 256)
    for batch in (0, 1, 2, 8, 64, 1024):
        for max_ctx in (0, 1, 1000, 8192, 32768, 1 << 20):
            for q_len, hq, hkv, d in ((1, 64, 8, 64), (4, 64, 8, 64), (1, 64, 4, 128)):
                for lens in (None, [max_ctx] * batch, [max_ctx // (b + 1) for b in range(batch)]):
                    s = sa.sink_attn_decode_split_size(batch, max_ctx, hq, hkv, d, q_len, lens)
                    assert s in (1024, 2048, 4096, 8192) or (s % 128 == 0 and 128 <= s < 1024)
    split = sa.sink_attn_decode_split_size
    # ragged or unknown lengths: 1024, or 2048 for many long requests
    assert split(64, 8192, 64, 8, 64) == 1024
    assert split(1, 32768, 64, 8, 64) == 1024
    assert split(8, 32768, 64, 8, 64) == 1024
    assert split(32, 32768, 64, 8, 64) == 2048
    assert split(128, 32768, 64, 8, 64) == 2048
    ragged = [1024 + (31744 * b) // 31 for b in range(32)]
    assert split(32, 32768, 64, 8, 64, seq_lens=ragged) == 2048
    assert split(8, 32768, 64, 8, 64, seq_lens=ragged[::4]) == 1024
    # equal lengths: the longest chunk that covers a request and leaves a unit
    # for every fourth SIMD
    assert split(64, 8192, 64, 8, 64, seq_lens=[8192] * 64) == 8192
    assert split(64, 8192, 64, 8, 64, q_len=4, seq_lens=[8192] * 64) == 8192
    assert split(16, 32768, 64, 8, 64, seq_lens=[32768] * 16) == 8192
    assert split(256, 2048, 64, 8, 64, seq_lens=[2048] * 256) == 2048
    assert split(1, 32768, 64, 8, 64, seq_lens=[32768]) == 1024
    assert split(4, 32768, 64, 8, 64, seq_lens=[32768] * 4) == 4096
    assert split(64, 8192, 64, 8, 64, seq_lens=[5000] * 64) == 8192
    assert split(64, 8192, 64, 8, 64, seq_lens=[3000] * 64) == 4096
    # a few equal requests that leave CUs idle at 1024: the shortest multiple of
    # 128 giving at most one (request, KV head, chunk) unit per CU
    assert split(1, 32768, 64, 8, 64, seq_lens=[22656]) == 768      # 30 chunks x 8 heads
    assert split(1, 16384, 64, 8, 64, seq_lens=[16384]) == 512      # 32 x 8 = 256
    assert split(1, 16384, 64, 8, 64, seq_lens=[16000]) == 512
    assert split(1, 8192, 64, 8, 64, seq_lens=[8192]) == 256        # 32 x 8 = 256
    assert split(1, 1000, 64, 8, 64, seq_lens=[1000]) == 128
    assert split(1, 4096, 64, 8, 64, seq_lens=[4096]) == 128        # 32 x 8
    assert split(2, 16384, 64, 8, 64, seq_lens=[16384] * 2) == 1024  # 1024 already fills the CUs
    assert split(1, 16384, 64, 4, 128, seq_lens=[16384]) == 256      # 4 KV heads: 64 x 4
    assert split(1, 32768, 64, 8, 64) == 1024                        # lengths unknown: ragged rule

def _noalloc(**kw):
    a = dict(q=16, q_sb=4 * 4096, q_st=4096, q_sh=64, q_len=4, k=16, v=16,
             kv_sb=8 * 1024 * 64, kv_sh=1024 * 64, kv_st=64, ks=None, vs=None, lens=4, batch=4,
             max_ctx=1024, sinks=4, hq=64, hkv=8, d=64, scale=0.125, split=256, nsplit=4,
             o=32, o_sb=4 * 4096, o_st=4096, o_sh=64, lse=None)
    a.update(kw)
    lib = sa.load_library()
    rc = lib.sink_attn_decode_merged_noalloc(
        a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["q_len"], a["k"], a["v"], a["kv_sb"],
        a["kv_sh"], a["kv_st"], a["ks"], a["vs"], a["lens"], a["batch"], a["max_ctx"],
        a["sinks"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["nsplit"], a["o"],
        a["o_sb"], a["o_st"], a["o_sh"], a["lse"], None)
    return rc, lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=4), -1, "both"),
    (dict(o=None), -1, "null"),
    (dict(q=None), -1, "null"),
    (dict(o=40), -1, "aligned"),
    (dict(o_st=100), -1, "multiples of 8"),
    (dict(q_len=0), -1, "q_len"),
    (dict(nsplit=2), -1, "cover"),
    (dict(d=32), -2, "head_dim"),
    # 4 * 4 * 64 * 2048 * 66 fp32 of chunk states: past the 2^25 of the scratch
    (dict(nsplit=2048), -1, "scratch"),
    (dict(batch=1 << 16, nsplit=4), -1, "scratch"),
])
def test_decode_merged_noalloc_rejects_bad_arguments(kw, code, needle):
    # every case fails on the host, before the scratch address is looked up
    rc, msg = _noalloc(**kw)
    assert rc == code and needle in msg, (rc, msg)


def test_decode_merged_noalloc_empty_batch_is_a_noop():
    rc, msg = _noalloc(batch=0, q=None, k=None, v=None, lens=None, sinks=None, o=None)
    assert rc == 0, msg
