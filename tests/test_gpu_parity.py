"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Bar: max-abs <= 2e-2 and mean-abs <= 2e-3 over the compared output elements
(bf16 inputs, fp32 accumulation).  Every output buffer is pre-filled with NaN,
so an element the kernels fail to write fails the test.  Full-size workloads
are checked on sampled rows (each computed one by one by the oracle) plus
properties that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import gqa_attention_sinks_prefill_amd as sa
import oracle
from gqa_attention_sinks_prefill_amd import workloads as wl
from parity_utils import (LSE_ABS, MAX_ABS, MEAN_ABS, assert_close, assert_lse_close, gather_rows,
                          sample_prefill_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _prefill_gpu(inp, *, causal=True, kv_layout="hnd", with_lse=True):
    q = inp["q"].to(DEV)
    k, v = inp["k"].to(DEV), inp["v"].to(DEV)
    if kv_layout == "nhd":
        k, v = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()
    T, Hq, D = q.shape
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    sa.sink_attn_prefill(q, k, v, inp["sinks"].to(DEV), inp["cu_seqlens"].to(DEV),
                         inp["max_seqlen"], causal=causal, kv_layout=kv_layout, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _prefill_case(lens, Hq, Hkv, D, seed, sink_range=(-4.0, 4.0), edges=None):
    cfg = wl.PrefillConfig("case", tuple(lens), len(lens), None, Hq, Hkv, D, sink_range,
                           seed=seed, edge_sinks=edges or {})
    return wl.prefill_inputs(cfg)


# ------------------------------------------------------------------ prefill --
def test_prefill_tiny_all_rows():
    inp = wl.prefill_inputs(wl.TINY_PREFILL)
    out, lse = _prefill_gpu(inp)
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=True, scale=wl.TINY_PREFILL.scale)
    assert_close(out.reshape(-1, 64), o_ref, what="tiny prefill O")
    assert_lse_close(lse.reshape(-1), lse_ref, what="tiny prefill lse")


def test_prefill_tiny_is_deterministic():
    inp = wl.prefill_inputs(wl.TINY_PREFILL)
    a, la = _prefill_gpu(inp)
    b, lb = _prefill_gpu(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def _all_rows_stats(inp, out, lse, cfg, chunk_rows=1 << 17):
    """Every (token, head) row of a prefill against the oracle, in chunks of
    rows (the oracle evaluates each row on its own): max-abs and mean-abs over
    all output elements, and the largest lse error."""
    T, Hq, D = inp["q"].shape
    out_c, lse_c = out.detach().cpu(), lse.detach().cpu()
    mx, total, lse_mx = 0.0, 0.0, 0.0
    for r0 in range(0, T * Hq, chunk_rows):
        flat = np.arange(r0, min(T * Hq, r0 + chunk_rows))
        rows = np.stack([flat // Hq, flat % Hq], 1)
        o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                           inp["cu_seqlens"], causal=True, scale=cfg.scale,
                                           rows=rows)
        t, h = torch.from_numpy(rows[:, 0]), torch.from_numpy(rows[:, 1])
        got = out_c[t, h].double().numpy()
        assert np.all(np.isfinite(got)), "non-finite values in the GPU output"
        err = np.abs(got - o_ref)
        mx, total = max(mx, float(err.max())), total + float(err.sum())
        g_lse = lse_c[t, h].double().numpy()
        assert np.array_equal(np.isneginf(g_lse), np.isneginf(lse_ref)), "lse -inf pattern differs"
        fin = ~np.isneginf(lse_ref)
        if fin.any():
            lse_mx = max(lse_mx, float(np.abs(g_lse[fin] - lse_ref[fin]).max()))
    return mx, total / (T * Hq * D), lse_mx


@pytest.mark.timeout(300)
def test_prefill_gptoss_shape_all_rows():
    """The GPT-OSS-shaped prefill (8192 tokens, 64 / 8 heads, d 64) in the
    launch configuration the benchmark times, every one of its 524 288
    (token, head) rows against the oracle."""
    cfg = wl.GPTOSS_PREFILL
    inp = wl.prefill_inputs(cfg)
    out, lse = _prefill_gpu(inp)
    mx, mean, lse_mx = _all_rows_stats(inp, out, lse, cfg)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"gpt-oss prefill: max-abs {mx:.3e}, mean-abs {mean:.3e}"
    assert lse_mx <= LSE_ABS, f"gpt-oss prefill lse max-abs {lse_mx:.3e}"


@pytest.mark.parametrize("n,Hq,Hkv,D", [(32768, 16, 2, 64), (20000, 16, 1, 128)])
def test_prefill_long_sequence_sampled_rows(n, Hq, Hkv, D):
    """One sequence four times (D 64) and 2.4 times (D 128) longer than the
    benchmark shapes: row tiles, key offsets and the per-row key loop far past
    them, checked on sampled rows (the oracle computes just those)."""
    cfg = wl.PrefillConfig("long", (n,), 1, None, Hq, Hkv, D, (-4.0, 4.0), seed=230 + D,
                           edge_sinks={0: float("-inf"), Hq - 1: 20.0})
    inp = wl.prefill_inputs(cfg)
    out, lse = _prefill_gpu(inp)
    assert not torch.isnan(out).any().item(), "unwritten or non-finite outputs"
    rows = sample_prefill_rows(inp["cu_seqlens"], Hq, n_random=150, seed=230 + D,
                               all_heads_positions=1)
    rows = sorted(set(rows) | {(n - 1, h) for h in range(Hq)})
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=True, scale=cfg.scale, rows=rows)
    assert_close(gather_rows(out, rows), o_ref, what=f"long prefill n={n} D={D}")
    idx = torch.tensor(rows)
    assert_lse_close(lse.cpu()[idx[:, 0], idx[:, 1]], lse_ref, what=f"long prefill lse D={D}")


@pytest.mark.timeout(600)
def test_prefill_varlen_wide_gqa_d128_all_rows():
    """The wide-GQA varlen prefill (16 packed sequences of U[512, 6000] tokens,
    64 / 4 heads, d 128, head 5 with sink -inf) as the benchmark launches it:
    every (token, head) row against the oracle -- max-abs and mean-abs over
    all 3.8 M rows' elements (the oracle needs about a minute on 16 threads)."""
    cfg = wl.VARLEN_PREFILL
    inp = wl.prefill_inputs(cfg)
    out, lse = _prefill_gpu(inp)
    mx, mean, lse_mx = _all_rows_stats(inp, out, lse, cfg)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"varlen d128 prefill: max-abs {mx:.3e}, mean-abs {mean:.3e}"
    assert lse_mx <= LSE_ABS, f"varlen d128 prefill lse max-abs {lse_mx:.3e}"


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 8), (4, 2), (32, 1)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged_edges_all_rows(Hq, Hkv, D, causal):
    """Lengths around tile edges, a zero-length sequence, GQA groups of 1, 2, 4, 32."""
    lens = [1, 31, 33, 0, 64, 65, 127, 200]
    inp = _prefill_case(lens, Hq, Hkv, D, seed=100 + Hq + D + causal,
                        edges={0: float("-inf"), Hq - 1: 20.0})
    out, lse = _prefill_gpu(inp, causal=causal)
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=causal, scale=1 / math.sqrt(D))
    assert_close(out.reshape(-1, D), o_ref, what=f"ragged prefill Hq={Hq} Hkv={Hkv} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="ragged prefill lse")


@pytest.mark.parametrize("Hq,Hkv", [(12, 4), (12, 2), (24, 2), (40, 8)])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_odd_gqa_groups_all_rows(Hq, Hkv, D):
    """GQA groups of 3, 6, 12 and 5: one, two or four heads per workgroup, and
    head-group counts on either side of a multiple of the 8 XCDs."""
    lens = [40, 0, 97, 130]
    inp = _prefill_case(lens, Hq, Hkv, D, seed=300 + Hq + Hkv + D,
                        edges={1: float("-inf"), Hq - 1: 20.0})
    out, lse = _prefill_gpu(inp, causal=True)
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=True, scale=1 / math.sqrt(D))
    assert_close(out.reshape(-1, D), o_ref, what=f"prefill Hq={Hq} Hkv={Hkv} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"prefill lse Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_growing_logits_all_rows(D, causal):
    """Key j of a sequence scaled by 1 + j/8, so the logits' spread grows along
    the sequence by far more than the sink: the running maximum (the kernel's
    stabiliser) has to move on many tiles after O already holds partial sums."""
    lens = [300, 129, 64]
    inp = _prefill_case(lens, 8, 2, D, seed=11 + D + causal, sink_range=(-1.0, 1.0))
    pos = torch.cat([torch.arange(n, dtype=torch.float32) for n in lens])
    k = (inp["k"].float() * (1.0 + pos / 8.0)[None, :, None]).to(torch.bfloat16)
    inp = dict(inp, k=k)
    out, lse = _prefill_gpu(inp, causal=causal)
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=causal, scale=1 / math.sqrt(D))
    assert_close(out.reshape(-1, D), o_ref, what=f"growing-logit prefill D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="growing-logit prefill lse")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_nhd_kv_layout(D):
    inp = _prefill_case([150, 77], 8, 2, D, seed=7)
    out, _ = _prefill_gpu(inp, kv_layout="nhd", with_lse=False)
    o_ref, _, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                 causal=True, scale=1 / math.sqrt(D))
    assert_close(out.reshape(-1, D), o_ref, what="nhd prefill O")


def test_prefill_empty_batches_leave_outputs_untouched():
    inp = _prefill_case([0, 0], 4, 1, 64, seed=3)
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 7.0)
    sa.sink_attn_prefill(q, q[:, :1].transpose(0, 1), q[:, :1].transpose(0, 1),
                         inp["sinks"].to(DEV), inp["cu_seqlens"].to(DEV), 0, out=out)
    cu0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    sa.sink_attn_prefill(q, q[:, :1].transpose(0, 1), q[:, :1].transpose(0, 1),
                         inp["sinks"].to(DEV), cu0, 16, out=out)
    # a real launch whose every workgroup finds an empty sequence
    sa.sink_attn_prefill(q, q[:, :1].transpose(0, 1), q[:, :1].transpose(0, 1),
                         inp["sinks"].to(DEV), inp["cu_seqlens"].to(DEV), 16, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ------------------------------------------------------------------- decode --
def _decode_gpu(inp, split_size, num_splits=None, *, max_ctx=None):
    q = inp["q"].to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    B, Hq, D = q.shape
    max_ctx = kc.shape[2] if max_ctx is None else max_ctx
    ns = -(-max_ctx // split_size) if num_splits is None else num_splits
    po = torch.full((B, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq), float("nan"), device=DEV)
    lens, sinks = inp["seq_lens"].to(DEV), inp["sinks"].to(DEV)
    sa.sink_attn_decode_split(q, kc, vc, lens, sinks, split_size, ns, max_ctx=max_ctx,
                              part_o=po, part_m=pm, part_d=pd)
    sa.sink_attn_merge_states(po, pm, pd, out=out, lse=lse)
    torch.cuda.synchronize()
    del kc, vc
    return out, lse, (po, pm, pd)


def _check_decode(inp, out, lse, what):
    o_ref, lse_ref, _ = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"],
                                      inp["seq_lens"], inp["sinks"])
    D = inp["q"].shape[-1]
    assert_close(out.reshape(-1, D), o_ref, what=f"{what} O")
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"{what} lse")


def test_decode_split_kv_full_config():
    cfg = wl.SPLIT_DECODE
    inp = wl.decode_inputs(cfg)
    out, lse, (po, pm, pd) = _decode_gpu(inp, cfg.split_size)
    _check_decode(inp, out, lse, "split decode")
    # chunk states against the oracle's own chunk states on sampled rows
    rng = np.random.default_rng(2)
    rows = sorted({(int(rng.integers(cfg.batch)), int(rng.integers(cfg.num_q_heads)))
                   for _ in range(64)} | {(0, 0), (cfg.batch - 1, cfg.num_q_heads - 1)})
    o_c, m_c, d_c = oracle.chunk_states(inp["q"], inp["k_cache"], inp["v_cache"],
                                        inp["seq_lens"], inp["sinks"], cfg.split_size,
                                        cfg.num_splits, rows=rows)
    idx = torch.tensor(rows)
    g_o = po.cpu()[idx[:, 0], idx[:, 1]]
    g_m = pm.cpu()[idx[:, 0], idx[:, 1]].double().numpy()
    g_d = pd.cpu()[idx[:, 0], idx[:, 1]].double().numpy()
    assert_close(g_o, o_c, what="split decode chunk o")
    np.testing.assert_allclose(g_m, m_c, rtol=0, atol=2e-3)
    np.testing.assert_allclose(g_d, d_c, rtol=2e-3)


def test_decode_split_kv_shape_library_chunk_size():
    """The split-KV decode shape (64 x 8192) through sink_attn_decode_merged with
    the chunk size the library picks for these equal lengths (8192: one chunk
    per request): every row against the oracle, and bitwise equal to split
    decode + sink_attn_merge_states at the same chunk size."""
    cfg = wl.SPLIT_DECODE
    inp = wl.decode_inputs(cfg)
    split = sa.sink_attn_decode_split_size(cfg.batch, cfg.max_ctx, cfg.num_q_heads,
                                           cfg.num_kv_heads, cfg.head_dim, seq_lens=inp["seq_lens"])
    assert split == 8192
    out_m, lse_m, _ = _merged_gpu(inp, split)
    _check_decode(inp, out_m[:, 0], lse_m[:, 0], f"split-KV shape, split {split}")
    out_s, lse_s, _ = _decode_gpu(inp, split)
    assert _bitwise(out_m[:, 0], out_s) and torch.equal(lse_m[:, 0], lse_s)


def test_decode_is_deterministic():
    cfg = wl.DecodeConfig("det", 8, None, (1, 5000), 5000, 64, 8, 64, (-4.0, 4.0),
                          split_size=1024, seed=5)
    inp = wl.decode_inputs(cfg)
    a, la, _ = _decode_gpu(inp, 1024)
    b, lb, _ = _decode_gpu(inp, 1024)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@pytest.mark.parametrize("batch", wl.RAGGED_BATCHES)
def test_decode_ragged_long_context(batch):
    """The ragged long-context decode at each batch size, every row against the
    oracle, through split + merge and through sink_attn_decode_merged (the
    entry point the benchmark times for these rows, with the split size the
    benchmark uses): its output and lse bitwise those of split + merge, and the
    states of chunks past each request's end never written."""
    cfg = wl.ragged_decode(batch)
    inp = wl.decode_inputs(cfg)     # slots past each length hold NaN
    out, lse, _ = _decode_gpu(inp, cfg.split_size)
    _check_decode(inp, out, lse, f"ragged decode B={batch}")
    # head 0 (sink -inf) is plain attention: sink share 0; head 63 (sink +20)
    # is dominated by the sink: its output is tiny.
    assert out[:, 63].abs().max().item() < 5e-3
    chosen = sa.sink_attn_decode_split_size(batch, cfg.max_ctx, cfg.num_q_heads, cfg.num_kv_heads,
                                            cfg.head_dim, seq_lens=inp["seq_lens"])
    for split in sorted({cfg.split_size, chosen}):
        out_m, lse_m, (po, pm, pd) = _merged_gpu(inp, split)
        ref_o, ref_lse = (out, lse) if split == cfg.split_size else _decode_gpu(inp, split)[:2]
        assert _bitwise(out_m[:, 0], ref_o), f"merged output differs from split+merge, split {split}"
        assert torch.equal(lse_m[:, 0], ref_lse), f"merged lse differs from split+merge, split {split}"
        if split != cfg.split_size:
            _check_decode(inp, ref_o, ref_lse, f"ragged decode B={batch} split {split}")
        ns = pm.shape[-1]
        for b, L in enumerate(inp["seq_lens"].tolist()):
            live = max(1, min(ns, -(-L // split)))
            assert torch.isnan(pm[b, ..., live:]).all() and not torch.isnan(pm[b, ..., :live]).any()
        del po, pm, pd


@pytest.mark.parametrize("L", [1, 64, 1000, 4096, 8192, 16000, 22656, 32768])
def test_decode_single_request_library_split(L):
    """One request at the chunk size the library picks for it (below 1024 tokens
    when 1024 would leave CUs without a unit): sink_attn_decode_merged bitwise
    equal to split + merge, and every row against the oracle."""
    cfg = wl.DecodeConfig("single", 1, L, None, L, 64, 8, 64, (-4.0, 4.0), split_size=1024,
                          seed=60 + L % 97, edge_sinks={0: float("-inf"), 63: 20.0})
    inp = wl.decode_inputs(cfg)
    split = sa.sink_attn_decode_split_size(1, L, 64, 8, 64, seq_lens=inp["seq_lens"])
    assert split % 128 == 0 and 128 <= split <= 8192
    out, lse, _ = _decode_gpu(inp, split)
    out_m, lse_m, _ = _merged_gpu(inp, split)
    assert _bitwise(out_m[:, 0], out) and torch.equal(lse_m[:, 0], lse), f"L={L} split {split}"
    _check_decode(inp, out, lse, f"single request L={L} split {split}")


@pytest.mark.parametrize("split", [64, 256, 1024, 4096, 8192])
def test_decode_split_size_invariance(split):
    cfg = wl.DecodeConfig("splits", 6, None, (1, 3000), 3000, 16, 2, 64, (-4.0, 4.0),
                          split_size=split, seed=9, edge_sinks={1: float("-inf"), 2: 20.0})
    inp = wl.decode_inputs(cfg)
    out, lse, _ = _decode_gpu(inp, split, -(-3000 // split) + 2)     # + 2 empty chunks
    _check_decode(inp, out, lse, f"split {split}")


@pytest.mark.parametrize("D,split", [(64, 4096), (128, 2048)])
def test_decode_very_long_context(D, split):
    """Contexts of 100k-131k tokens (4x the ragged benchmark's longest): cache
    offsets far past the benchmark shapes, 32-64 chunks per request; split +
    merge and the one-launch call both against the oracle on every row."""
    cfg = wl.DecodeConfig("long", 2, None, (100000, 131072), 131072, 16, 2, D, (-4.0, 4.0),
                          split_size=split, seed=231 + D, edge_sinks={3: float("-inf")})
    inp = wl.decode_inputs(cfg)
    out, lse, _ = _decode_gpu(inp, split)
    _check_decode(inp, out, lse, f"131k-token decode D={D}")
    out_f, lse_f, _ = _fused_gpu(inp, split)
    assert torch.equal(out_f[:, 0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse_f[:, 0], lse)


def test_decode_edge_lengths():
    lens = [0, 1, 63, 64, 65, 255, 256, 257, 1024, 1025, 0]
    B, Hq, Hkv, D, max_ctx = len(lens), 8, 2, 64, 1280
    g = torch.Generator().manual_seed(31)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.full((B, Hkv, max_ctx, D), float("nan"), dtype=torch.bfloat16)
    vc = torch.full((B, Hkv, max_ctx, D), float("nan"), dtype=torch.bfloat16)
    for b, L in enumerate(lens):
        kc[b, :, :L] = torch.randn(Hkv, L, D, generator=g).to(torch.bfloat16)
        vc[b, :, :L] = torch.randn(Hkv, L, D, generator=g).to(torch.bfloat16)
    sinks = torch.tensor([float("-inf"), 0.0, 1.0, -2.0, 20.0, float("-inf"), 3.0, -4.0])
    inp = dict(q=q, k_cache=kc, v_cache=vc, seq_lens=torch.tensor(lens, dtype=torch.int32),
               sinks=sinks)
    out, lse, _ = _decode_gpu(inp, 256)
    _check_decode(inp, out, lse, "edge lengths")
    assert torch.all(out[0] == 0) and torch.all(out[-1] == 0)


@pytest.mark.parametrize("Hq,Hkv,D", [(64, 2, 128), (8, 8, 128), (32, 1, 64)])
def test_decode_head_dims_and_groups(Hq, Hkv, D):
    cfg = wl.DecodeConfig("groups", 5, None, (1, 2500), 2500, Hq, Hkv, D, (-4.0, 4.0),
                          split_size=512, seed=Hq + D, edge_sinks={0: float("-inf")})
    inp = wl.decode_inputs(cfg)
    out, lse, _ = _decode_gpu(inp, 512)
    _check_decode(inp, out, lse, f"decode Hq={Hq} Hkv={Hkv} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_decode_nhd_cache_layout(D):
    """Token-major caches [B, max_ctx, Hkv, D] passed as strided [B, Hkv,
    max_ctx, D] views (token stride Hkv * D, head stride D): split + merge
    against the oracle, the one-launch call bitwise against it."""
    cfg = wl.DecodeConfig("nhd", 4, None, (1, 1500), 1536, 16, 4, D, (-4.0, 4.0),
                          split_size=512, seed=320 + D, edge_sinks={2: float("-inf")})
    inp = wl.decode_inputs(cfg)
    nhd = lambda t: t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    kn, vn = nhd(inp["k_cache"]), nhd(inp["v_cache"])
    assert kn.stride(2) == 4 * D and kn.stride(1) == D
    out, lse, _ = _decode_gpu(dict(inp, k_cache=kn, v_cache=vn), 512)
    _check_decode(inp, out, lse, f"NHD-cache decode D={D}")
    out_f, lse_f, _ = _fused_gpu(dict(inp, k_cache=kn, v_cache=vn), 512)
    assert torch.equal(out_f[:, 0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse_f[:, 0], lse)


def test_decode_strided_query_and_output():
    """Non-contiguous q / out views with head stride != D."""
    cfg = wl.DecodeConfig("strided", 3, None, (100, 900), 1024, 8, 2, 64, (-4.0, 4.0),
                          split_size=256, seed=12)
    inp = wl.decode_inputs(cfg)
    qbig = torch.zeros(3, 8, 128, dtype=torch.bfloat16)
    qbig[:, :, 32:96] = inp["q"]
    q = qbig.to(DEV)[:, :, 32:96]
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    po, pm, pd = sa.sink_attn_decode_split(q, kc, vc, inp["seq_lens"].to(DEV),
                                           inp["sinks"].to(DEV), 256)
    obig = torch.full((3, 8, 192), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = obig[:, :, 64:128]
    sa.sink_attn_merge_states(po, pm, pd, out=out)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                inp["sinks"])
    assert_close(out.reshape(-1, 64), o_ref, what="strided decode O")
    assert torch.isnan(obig[:, :, :64]).all() and torch.isnan(obig[:, :, 128:]).all()


# ------------------------------------------------------- multi-token decode --
def _decode_multi_gpu(inp, split_size, *, lens=None):
    q = inp["q"].to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    B, q_len, Hq, D = q.shape
    ns = -(-kc.shape[2] // split_size)
    po = torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    lens = (inp["seq_lens"] if lens is None else lens).to(DEV)
    sa.sink_attn_decode_multi(q, kc, vc, lens, inp["sinks"].to(DEV), split_size, ns, out=out,
                              lse=lse, partials=(po, pm, pd))
    torch.cuda.synchronize()
    return out, lse


def _multi_cfg(lens, q_len, Hq, Hkv, D, seed, split, max_ctx=None, edges=None):
    cfg = wl.DecodeConfig("multi", len(lens), None, (1, 1), max_ctx or max(lens), Hq, Hkv, D,
                          (-4.0, 4.0), split_size=split, seed=seed, edge_sinks=edges or {},
                          q_len=q_len)
    return wl.decode_inputs(cfg, lens=lens)


@pytest.mark.parametrize("q_len", [2, 3, 4])
@pytest.mark.parametrize("Hq,Hkv,D", [(64, 8, 64), (64, 4, 64), (64, 4, 128), (8, 8, 64)])
def test_decode_multi_all_rows(q_len, Hq, Hkv, D):
    """q_len new tokens per request against the oracle on every row: lengths
    equal to q_len (only new tokens), around 64-key sub-tiles and chunk edges;
    (token, head) columns per KV head from 2 to 64 (one to four 16-column
    blocks per workgroup, one or two workgroups per chunk)."""
    lens = [q_len, 5, 64, 65, 257, 1000]
    inp = _multi_cfg(lens, q_len, Hq, Hkv, D, seed=60 + q_len + Hq + D, split=256,
                     edges={0: float("-inf"), Hq - 1: 20.0})
    out, lse = _decode_multi_gpu(inp, 256)
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, D), o_ref, what=f"multi decode q_len={q_len} Hq={Hq} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="multi decode lse")


@pytest.mark.parametrize("Hq,Hkv,q_len", [(12, 4, 1), (12, 4, 3), (40, 8, 2), (24, 4, 5)])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_odd_gqa_groups_all_rows(Hq, Hkv, q_len, D):
    """GQA groups of 3, 5 and 6 with 1-5 new tokens: 3 to 30 (token, head)
    columns per KV head, partly filled 16-column blocks."""
    lens = [0, 1, q_len, 300, 1100]
    inp = _multi_cfg(lens, q_len, Hq, Hkv, D, seed=330 + Hq + q_len + D, split=256,
                     edges={0: float("-inf"), Hq - 1: 20.0})
    inp = dict(inp, q=_q4(inp["q"]))        # [B, q_len, Hq, D] also for q_len = 1
    out, lse = _decode_multi_gpu(inp, 256)
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, D), o_ref, what=f"decode Hq={Hq} Hkv={Hkv} q_len={q_len} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="odd-group decode lse")


@pytest.mark.parametrize("q_len", [8, 16])
def test_decode_multi_long_drafts(q_len):
    """Longer draft runs: 64 and 128 columns per KV head."""
    lens = [q_len, 130, 700]
    inp = _multi_cfg(lens, q_len, 64, 8, 64, seed=80 + q_len, split=512)
    out, lse = _decode_multi_gpu(inp, 512)
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, 64), o_ref, what=f"multi decode q_len={q_len}")
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"multi decode q_len={q_len} lse")


def test_decode_multi_rows_that_see_no_token():
    """Requests shorter than q_len: the leading new tokens see only the sink."""
    lens = [1, 2, 3]
    inp = _multi_cfg(lens, 4, 8, 2, 64, seed=70, split=64, max_ctx=64,
                     edges={1: float("-inf")})
    out, lse = _decode_multi_gpu(inp, 64)
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, 64), o_ref, what="multi decode, short requests")
    assert_lse_close(lse.reshape(-1), lse_ref, what="multi decode lse, short requests")


def test_decode_multi_single_token_matches_decode_split():
    """q_len = 1 through the multi-token entry point is bitwise plain decode."""
    cfg = wl.DecodeConfig("one", 6, None, (1, 3000), 3000, 64, 8, 64, (-4.0, 4.0),
                          split_size=512, seed=71)
    inp = wl.decode_inputs(cfg)
    out_d, lse_d, _ = _decode_gpu(inp, 512)
    multi = dict(inp, q=inp["q"].unsqueeze(1))
    out_m, lse_m = _decode_multi_gpu(multi, 512)
    assert torch.equal(out_m[:, 0].view(torch.int16), out_d.view(torch.int16))
    assert torch.equal(lse_m[:, 0], lse_d)


def test_decode_multi_full_config_all_rows():
    """64 requests x 8192 tokens, 4 new tokens each (the bench's multi-token
    line): every (request, new token, head) row against the oracle, with
    1024-token chunks and with the library's chunk size for these equal lengths."""
    cfg = wl.MTP_DECODE
    inp = wl.decode_inputs(cfg)
    B, q_len, Hq, D = inp["q"].shape
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    chosen = sa.sink_attn_decode_split_size(B, cfg.max_ctx, Hq, cfg.num_kv_heads, D, q_len,
                                            seq_lens=inp["seq_lens"])
    for split in sorted({cfg.split_size, chosen}):
        out, lse = _decode_multi_gpu(inp, split)
        assert_close(out.reshape(-1, D), o_ref, what=f"multi decode full config, split {split}")
        assert_lse_close(lse.reshape(-1), lse_ref, what=f"multi decode full config lse, split {split}")


_EDGE_LENS = [0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 447, 448, 511, 512]


@pytest.mark.parametrize("B,Hkv,D,q_len,split", [
    (128, 8, 64, 1, 64),      # one column block: four waves per chunk
    (128, 8, 64, 3, 64),      # 24 columns (two blocks), 8192 chunks: a wave per chunk
    (24, 8, 64, 3, 128),      # two blocks, 768 chunks: two waves per chunk
    (32, 8, 64, 8, 128),      # 64 columns (four blocks), 1024 chunks: a wave per chunk
    (64, 8, 128, 1, 128),     # head_dim 128, 2048 chunks: a wave per chunk
    (1040, 8, 64, 1, 64),     # over a thousand requests, 66560 units, most chunks empty
])
def test_decode_work_splits_edge_lengths(B, Hkv, D, q_len, split):
    """Each way a chunk is shared by waves (one, two or four per chunk), at
    launches big enough to pick it, with lengths on and around sub-tile and
    chunk edges, zero included; every chunk state is checked (empty chunks
    exactly (0, -inf, 0)), not only the merged output."""
    lens = [_EDGE_LENS[(7 * i) % len(_EDGE_LENS)] for i in range(B)]
    inp = _multi_cfg(lens, q_len, 64, Hkv, D, seed=90 + q_len + D + split, split=split,
                     max_ctx=512, edges={0: float("-inf"), 63: 20.0})
    if inp["q"].dim() == 3:
        inp = dict(inp, q=inp["q"].unsqueeze(1))
    q = inp["q"].to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    ns = 512 // split
    po = torch.full((B, q_len, 64, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, 64, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, 64, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, 64, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, 64), float("nan"), device=DEV)
    sa.sink_attn_decode_multi(q, kc, vc, inp["seq_lens"].to(DEV), inp["sinks"].to(DEV), split,
                              ns, out=out, lse=lse, partials=(po, pm, pd))
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    what = f"decode B={B} D={D} q_len={q_len} split={split}"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"{what} lse")
    # the chunk states themselves (empty chunks exactly (0, -inf, 0))
    po, pm, pd = po.cpu(), pm.cpu(), pd.cpu()
    assert not torch.isnan(po).any() and not torch.isnan(pm).any() and not torch.isnan(pd).any()
    for b, L in enumerate(lens):
        first_empty = max(-(-L // split), 1)
        assert torch.all(po[b, :, :, first_empty:] == 0)
        assert torch.all(pm[b, :, :, first_empty:] == float("-inf"))
        assert torch.all(pd[b, :, :, first_empty:] == 0)
    if q_len == 1:
        rows = [(b, h) for b in range(0, B, 5) for h in (0, 17, 63)]
        o_c, m_c, d_c = oracle.chunk_states(inp["q"][:, 0], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"], split, ns, rows=rows)
        idx = torch.tensor(rows)
        assert_close(po[idx[:, 0], 0, idx[:, 1]], o_c, what=f"{what} chunk o")
        g_m = pm[idx[:, 0], 0, idx[:, 1]].double().numpy()
        g_d = pd[idx[:, 0], 0, idx[:, 1]].double().numpy()
        np.testing.assert_allclose(g_m, m_c, rtol=0, atol=2e-3)
        np.testing.assert_allclose(g_d, d_c, rtol=2e-3)


# ------------------------------------------------------------ chunked prefill --
def _chunked_gpu(inp, *, causal=True):
    q = inp["q"].to(DEV)
    k, v = inp["k"].to(DEV), inp["v"].to(DEV)
    Tq, Hq, D = q.shape
    out = torch.full((Tq, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((Tq, Hq), float("nan"), dtype=torch.float32, device=DEV)
    sa.sink_attn_prefill_chunked(q, k, v, inp["sinks"].to(DEV), inp["cu_seqlens_q"].to(DEV),
                                 inp["cu_seqlens_k"].to(DEV), inp["max_seqlen_q"],
                                 causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("Hq,Hkv", [(64, 8), (8, 8), (16, 1)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_chunked_all_rows(Hq, Hkv, D, causal):
    """Chunks of up to 100 new queries at the end of sequences of 1..700 keys:
    chunk and prefix lengths around 32/64-key tiles, a chunk that is the whole
    sequence, one-query chunks."""
    lens = (1, 33, 64, 100, 131, 700)
    cfg = wl.PrefillConfig("chunked", lens, len(lens), None, Hq, Hkv, D, (-4.0, 4.0),
                           seed=90 + Hq + D + causal, edge_sinks={0: float("-inf"), Hq - 1: 20.0})
    inp = wl.chunked_prefill_inputs(cfg, 100)
    out, lse = _chunked_gpu(inp, causal=causal)
    o_ref, lse_ref, _ = oracle.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                               inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                               causal=causal, scale=1 / math.sqrt(D))
    assert_close(out.reshape(-1, D), o_ref, what=f"chunked prefill Hq={Hq} Hkv={Hkv} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="chunked prefill lse")


def test_prefill_chunked_full_config_sampled_rows():
    """4 sequences of 8192 tokens whose last 2048 are the new chunk (the bench line)."""
    cfg = wl.CHUNKED_PREFILL
    inp = wl.chunked_prefill_inputs(cfg, wl.CHUNK_LEN)
    out, lse = _chunked_gpu(inp)
    assert not torch.isnan(out).any().item()
    rows = sample_prefill_rows(inp["cu_seqlens_q"], cfg.num_q_heads, n_random=400, seed=6)
    o_ref, lse_ref, _ = oracle.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                               inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                               scale=cfg.scale, rows=rows)
    assert_close(gather_rows(out, rows), o_ref, what="chunked prefill full config (sampled rows)")
    idx = torch.tensor(rows)
    assert_lse_close(lse.cpu()[idx[:, 0], idx[:, 1]], lse_ref, what="chunked prefill lse")


def test_prefill_chunked_with_equal_boundaries_is_bitwise_prefill():
    inp = _prefill_case([150, 77, 64], 8, 2, 64, seed=91)
    out_p, lse_p = _prefill_gpu(inp)
    chunk = dict(inp, cu_seqlens_q=inp["cu_seqlens"], cu_seqlens_k=inp["cu_seqlens"],
                 max_seqlen_q=inp["max_seqlen"])
    out_c, lse_c = _chunked_gpu(chunk)
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(lse_c, lse_p)


# ------------------------------------------------------------- KV-cache append --
def _random_bits_cache(B, Hkv, max_ctx, D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-32768, 32768, (B, Hkv, max_ctx, D), generator=g,
                         dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


@pytest.mark.parametrize("Hkv,D", [(8, 64), (4, 128), (1, 64)])
def test_kv_append_bitwise(Hkv, D):
    """Counts around the kernel's token blocks (0 .. 1000), positions at the
    cache start, in the middle and at its end (the overflow is dropped); the
    caches start as random bits and every slot is compared bit for bit."""
    counts = [0, 1, 31, 32, 33, 200, 1000, 70]
    max_ctx = 1100
    pos = [5, 0, 1000, 17, 1067, 300, 100, 1090]      # request 7: 10 of 70 fit
    inp = wl.kv_append_inputs(counts, max_ctx, Hkv, D, seed=100 + Hkv + D, pos=pos)
    kc = _random_bits_cache(len(counts), Hkv, max_ctx, D, seed=1)
    vc = _random_bits_cache(len(counts), Hkv, max_ctx, D, seed=2)
    k_ref, v_ref = oracle.kv_append(inp["k_new"], inp["v_new"], inp["cu_seqlens_new"],
                                    inp["cache_pos"], kc, vc)
    kd, vd = kc.to(DEV), vc.to(DEV)
    sa.sink_attn_kv_append(inp["k_new"].to(DEV), inp["v_new"].to(DEV),
                           inp["cu_seqlens_new"].to(DEV), inp["cache_pos"].to(DEV), kd, vd,
                           max_new=max(counts))
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu().view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(vd.cpu().view(torch.int16), v_ref.view(torch.int16))


def test_kv_append_from_a_fused_qkv_row():
    """New rows read straight out of a fused [T, Hq + 2 Hkv, D] QKV tensor
    (token stride (Hq + 2 Hkv) * D), into caches that are a slice of a larger
    allocation (strided requests)."""
    Hq, Hkv, D, max_ctx = 16, 4, 64, 300
    counts = [40, 129, 7]
    inp = wl.kv_append_inputs(counts, max_ctx, Hkv, D, seed=120)
    T = sum(counts)
    g = torch.Generator().manual_seed(121)
    qkv = torch.randn(T, Hq + 2 * Hkv, D, generator=g).to(torch.bfloat16)
    qkv[:, Hq:Hq + Hkv] = inp["k_new"]
    qkv[:, Hq + Hkv:] = inp["v_new"]
    big_k = _random_bits_cache(6, Hkv, max_ctx, D, seed=3)
    big_v = _random_bits_cache(6, Hkv, max_ctx, D, seed=4)
    kc, vc = big_k[::2], big_v[::2]                     # requests 2 cache rows apart
    k_ref, v_ref = oracle.kv_append(inp["k_new"], inp["v_new"], inp["cu_seqlens_new"],
                                    inp["cache_pos"], kc, vc)
    qd, bkd, bvd = qkv.to(DEV), big_k.to(DEV), big_v.to(DEV)
    sa.sink_attn_kv_append(qd[:, Hq:Hq + Hkv], qd[:, Hq + Hkv:], inp["cu_seqlens_new"].to(DEV),
                           inp["cache_pos"].to(DEV), bkd[::2], bvd[::2], max_new=max(counts))
    torch.cuda.synchronize()
    assert torch.equal(bkd.cpu()[::2].view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(bvd.cpu()[::2].view(torch.int16), v_ref.view(torch.int16))
    assert torch.equal(bkd.cpu()[1::2].view(torch.int16), big_k[1::2].view(torch.int16))


# ------------------------------------------------------------ FP8 KV caches --
def _fp8_cfg(lens, q_len, Hq, Hkv, D, seed, split, max_ctx=None, edges=None):
    cfg = wl.DecodeConfig("fp8", len(lens), None, (1, 1), max_ctx or max(max(lens), 1), Hq, Hkv,
                          D, (-4.0, 4.0), split_size=split, seed=seed, edge_sinks=edges or {},
                          q_len=q_len)
    return wl.fp8_decode_inputs(cfg, lens=lens)


def _q4(q):
    return q.unsqueeze(1) if q.dim() == 3 else q


def _fp8_gpu(inp, split, ns=None):
    q = _q4(inp["q"]).to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    B, q_len, Hq, D = q.shape
    ns = -(-kc.shape[2] // split) if ns is None else ns
    po = torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    sa.sink_attn_decode_fp8(q, kc, vc, inp["k_scale"].to(DEV), inp["v_scale"].to(DEV),
                            inp["seq_lens"].to(DEV), inp["sinks"].to(DEV), split, ns, out=out,
                            lse=lse, partials=(po, pm, pd))
    torch.cuda.synchronize()
    return out, lse, (po, pm, pd)


def _fp8_ref(inp, rows=None):
    return oracle.decode_multi_fp8(_q4(inp["q"]), inp["k_cache"], inp["v_cache"],
                                   inp["k_scale"].numpy(), inp["v_scale"].numpy(),
                                   inp["seq_lens"], inp["sinks"], rows=rows)


@pytest.mark.parametrize("q_len,Hq,Hkv,D", [(1, 64, 8, 64), (1, 64, 4, 128), (3, 64, 8, 64),
                                             (2, 64, 4, 128), (8, 64, 8, 64), (1, 8, 8, 64)])
def test_decode_fp8_all_rows(q_len, Hq, Hkv, D):
    """FP8 caches against the oracle on every row: lengths 0, around 64-key
    sub-tiles and chunk edges; unused slots hold the NaN code."""
    lens = [0, q_len, 5, 64, 65, 257, 1000]
    inp = _fp8_cfg(lens, q_len, Hq, Hkv, D, seed=100 + q_len + D, split=256,
                   edges={0: float("-inf"), Hq - 1: 20.0})
    out, lse, _ = _fp8_gpu(inp, 256)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    assert_close(out.reshape(-1, D), o_ref, what=f"fp8 decode q_len={q_len} Hq={Hq} D={D}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="fp8 decode lse")


def test_decode_fp8_over_a_quantized_normal_cache():
    """Caches made by quantizing normal bf16 K/V with the oracle's quantizer."""
    g = torch.Generator().manual_seed(101)
    lens, Hq, Hkv, D, max_ctx = [1, 200, 300], 32, 4, 64, 320
    B = len(lens)
    k = torch.randn(B, Hkv, max_ctx, D, generator=g)
    v = torch.randn(B, Hkv, max_ctx, D, generator=g)
    ks = np.float32([0.004 * (1 + h) for h in range(Hkv)])
    vs = np.float32([0.02 / (1 + h) for h in range(Hkv)])
    kc = torch.from_numpy(oracle.fp8_quantize(k.numpy(), ks[None, :, None, None]))
    vc = torch.from_numpy(oracle.fp8_quantize(v.numpy(), vs[None, :, None, None]))
    inp = dict(q=torch.randn(B, Hq, D, generator=g).to(torch.bfloat16), k_cache=kc, v_cache=vc,
               k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs),
               seq_lens=torch.tensor(lens, dtype=torch.int32),
               sinks=torch.empty(Hq).uniform_(-4, 4, generator=g))
    out, lse, _ = _fp8_gpu(inp, 128)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    assert_close(out.reshape(-1, D), o_ref, what="fp8 decode, quantized normal cache")
    assert_lse_close(lse.reshape(-1), lse_ref, what="fp8 decode lse, quantized normal cache")


@pytest.mark.parametrize("B,Hkv,D,q_len,split", [
    (128, 8, 64, 1, 64),      # one column block: four waves per chunk
    (128, 8, 64, 3, 64),      # two blocks, 8192 chunks: a wave per chunk
    (24, 8, 64, 3, 128),      # two blocks, 768 chunks: two waves per chunk
    (32, 8, 64, 8, 128),      # four blocks: a wave per chunk
    (64, 8, 128, 1, 128),     # head_dim 128: a wave per chunk
])
def test_decode_fp8_work_splits_edge_lengths(B, Hkv, D, q_len, split):
    """Each way waves share a chunk, FP8 caches, edge lengths (zero included),
    every chunk state checked (empty chunks exactly (0, -inf, 0))."""
    lens = [_EDGE_LENS[(5 * i) % len(_EDGE_LENS)] for i in range(B)]
    inp = _fp8_cfg(lens, q_len, 64, Hkv, D, seed=110 + q_len + D + split, split=split,
                   max_ctx=512, edges={0: float("-inf"), 63: 20.0})
    ns = 512 // split
    out, lse, (po, pm, pd) = _fp8_gpu(inp, split, ns)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    what = f"fp8 decode B={B} D={D} q_len={q_len} split={split}"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"{what} lse")
    po, pm, pd = po.cpu(), pm.cpu(), pd.cpu()
    assert not torch.isnan(po).any() and not torch.isnan(pm).any() and not torch.isnan(pd).any()
    for b, L in enumerate(lens):
        first_empty = max(-(-L // split), 1)
        assert torch.all(po[b, :, :, first_empty:] == 0)
        assert torch.all(pm[b, :, :, first_empty:] == float("-inf"))
        assert torch.all(pd[b, :, :, first_empty:] == 0)


def test_decode_fp8_full_config_all_rows():
    """64 requests x 8192 tokens over FP8 caches (the bench's FP8 decode line):
    every row against the oracle, with 1024-token chunks and with the library's
    chunk size for these equal lengths."""
    cfg = wl.FP8_DECODE
    inp = wl.fp8_decode_inputs(cfg)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    chosen = sa.sink_attn_decode_split_size(cfg.batch, cfg.max_ctx, cfg.num_q_heads,
                                            cfg.num_kv_heads, cfg.head_dim, seq_lens=inp["seq_lens"])
    for split in sorted({cfg.split_size, chosen}):
        out, lse, _ = _fp8_gpu(inp, split)
        assert_close(out.reshape(-1, cfg.head_dim), o_ref, what=f"fp8 decode full config, split {split}")
        assert_lse_close(lse.reshape(-1), lse_ref, what=f"fp8 decode full config lse, split {split}")


@pytest.mark.parametrize("Hkv,D", [(8, 64), (4, 128), (1, 64)])
def test_kv_append_fp8_bitwise(Hkv, D):
    """Quantizing append against the oracle, code for code; slots outside the
    cache are dropped and untouched slots keep their codes."""
    counts, max_ctx = [3, 0, 130, 64, 200], 256
    d = wl.kv_append_inputs(counts, max_ctx, Hkv, D, seed=120 + D, pos=[0, 5, 100, 192, 250])
    g = torch.Generator().manual_seed(121)
    B = len(counts)
    kc = torch.randint(0, 256, (B, Hkv, max_ctx, D), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, Hkv, max_ctx, D), generator=g, dtype=torch.uint8)
    ks = torch.empty(Hkv).uniform_(0.002, 0.02, generator=g)
    vs = torch.empty(Hkv).uniform_(0.002, 0.02, generator=g)
    kn = (d["k_new"].float() * 3).to(torch.bfloat16)      # some values saturate at +-448
    vn = d["v_new"]
    ko, vo = oracle.kv_append_fp8(kn, vn, d["cu_seqlens_new"], d["cache_pos"], kc, vc,
                                  ks.numpy(), vs.numpy())
    kg, vg = kc.to(DEV), vc.to(DEV)
    sa.sink_attn_kv_append_fp8(kn.to(DEV), vn.to(DEV), d["cu_seqlens_new"].to(DEV),
                               d["cache_pos"].to(DEV), kg, vg, ks.to(DEV), vs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kg.cpu(), ko) and torch.equal(vg.cpu(), vo)


def test_kv_append_fp8_then_decode():
    """Append bf16 rows into empty FP8 caches on the GPU, then decode over them:
    equal to the oracle decode over the oracle's own quantized caches."""
    g = torch.Generator().manual_seed(122)
    counts, Hq, Hkv, D, max_ctx = [37, 300, 129], 64, 8, 64, 320
    d = wl.kv_append_inputs(counts, max_ctx, Hkv, D, seed=123, pos=[0, 0, 0])
    ks = torch.empty(Hkv).uniform_(0.005, 0.02, generator=g)
    vs = torch.empty(Hkv).uniform_(0.005, 0.02, generator=g)
    B = len(counts)
    zero = torch.zeros(B, Hkv, max_ctx, D, dtype=torch.uint8)
    ko, vo = oracle.kv_append_fp8(d["k_new"], d["v_new"], d["cu_seqlens_new"], d["cache_pos"],
                                  zero, zero, ks.numpy(), vs.numpy())
    kg, vg = zero.to(DEV), zero.clone().to(DEV)
    sa.sink_attn_kv_append_fp8(d["k_new"].to(DEV), d["v_new"].to(DEV),
                               d["cu_seqlens_new"].to(DEV), d["cache_pos"].to(DEV), kg, vg,
                               ks.to(DEV), vs.to(DEV))
    inp = dict(q=torch.randn(B, Hq, D, generator=g).to(torch.bfloat16), k_cache=kg.cpu(),
               v_cache=vg.cpu(), k_scale=ks, v_scale=vs,
               seq_lens=torch.tensor(counts, dtype=torch.int32),
               sinks=torch.empty(Hq).uniform_(-4, 4, generator=g))
    assert torch.equal(inp["k_cache"], ko) and torch.equal(inp["v_cache"], vo)
    out, lse, _ = _fp8_gpu(inp, 64)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    assert_close(out.reshape(-1, D), o_ref, what="fp8 append then decode")
    assert_lse_close(lse.reshape(-1), lse_ref, what="fp8 append then decode lse")


# ------------------------------------------------------------- paged caches --
def _to_pages(logical, P, g, extra_pages=7, poison=None):
    """Scatter logical caches [B, Hkv, L, D] into pages [num_pages, Hkv, P, D]
    under a random permutation; unreferenced pages and the tail of the last
    page of each request hold `poison`.  Returns (pages, block_tables [B, L/P])."""
    B, Hkv, L, D = logical.shape
    per = -(-L // P)
    num_pages = B * per + extra_pages
    perm = torch.randperm(num_pages, generator=g)[:B * per].view(B, per).to(torch.int32)
    pages = torch.full((num_pages, Hkv, P, D), poison, dtype=logical.dtype) if poison is not None \
        else torch.zeros((num_pages, Hkv, P, D), dtype=logical.dtype)
    for b in range(B):
        for p in range(per):
            blk = logical[b, :, p * P:(p + 1) * P]
            pages[int(perm[b, p]), :, :blk.shape[1]] = blk
    return pages, perm


def _paged_case(lens, q_len, Hq, Hkv, D, P, fp8, seed, max_ctx):
    if fp8:
        cfg = wl.DecodeConfig("pg8", len(lens), None, (1, 1), max_ctx, Hq, Hkv, D, (-4.0, 4.0),
                              split_size=64, seed=seed, edge_sinks={0: float("-inf"), Hq - 1: 20.0},
                              q_len=q_len)
        inp = wl.fp8_decode_inputs(cfg, lens=lens)
        poison = 0x7F
    else:
        cfg = wl.DecodeConfig("pg", len(lens), None, (1, 1), max_ctx, Hq, Hkv, D, (-4.0, 4.0),
                              split_size=64, seed=seed, edge_sinks={0: float("-inf"), Hq - 1: 20.0},
                              q_len=q_len)
        inp = wl.decode_inputs(cfg, lens=lens)
        poison = float("nan")
    g = torch.Generator().manual_seed(seed)
    kp, bt = _to_pages(inp["k_cache"], P, g, poison=poison)
    vp = torch.full_like(kp, poison) if fp8 else torch.full_like(kp, float("nan"))
    for b in range(bt.shape[0]):
        for p in range(bt.shape[1]):
            blk = inp["v_cache"][b, :, p * P:(p + 1) * P]
            vp[int(bt[b, p]), :, :blk.shape[1]] = blk
    return inp, kp, vp, bt


def _paged_gpu(inp, kp, vp, bt, split, fp8):
    q = _q4(inp["q"]).to(DEV)
    B, q_len, Hq, D = q.shape
    ns = -(-bt.shape[1] * kp.shape[2] // split)
    po = torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    sc = dict(k_scale=inp["k_scale"].to(DEV), v_scale=inp["v_scale"].to(DEV)) if fp8 else {}
    sa.sink_attn_decode_paged(q, kp.to(DEV), vp.to(DEV), bt.to(DEV), inp["seq_lens"].to(DEV),
                              inp["sinks"].to(DEV), split, ns, out=out, lse=lse,
                              partials=(po, pm, pd), **sc)
    torch.cuda.synchronize()
    return out, lse, (po, pm, pd)


def _paged_ref(inp, kp, vp, bt, P, fp8, rows=None):
    sc = dict(k_scale=inp["k_scale"].numpy(), v_scale=inp["v_scale"].numpy()) if fp8 else {}
    return oracle.decode_multi_paged(_q4(inp["q"]), kp, vp, bt, P, inp["seq_lens"],
                                     inp["sinks"], rows=rows, **sc)


@pytest.mark.parametrize("Hq,Hkv,q_len,D", [(12, 4, 1, 64), (12, 4, 3, 128), (40, 8, 2, 64)])
def test_decode_fp8_odd_gqa_groups_all_rows(Hq, Hkv, q_len, D):
    """FP8 caches with GQA groups of 3 and 5 (partly filled column blocks)."""
    lens = [0, q_len, 70, 300, 1100]
    inp = _fp8_cfg(lens, q_len, Hq, Hkv, D, seed=340 + Hq + q_len + D, split=256,
                   edges={0: float("-inf"), Hq - 1: 20.0})
    out, lse, _ = _fp8_gpu(inp, 256)
    o_ref, lse_ref, _ = _fp8_ref(inp)
    assert_close(out.reshape(-1, D), o_ref, what=f"fp8 decode Hq={Hq} Hkv={Hkv} q_len={q_len}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="fp8 odd-group decode lse")


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_paged_odd_gqa_group_all_rows(fp8):
    """Pages of 16 tokens with a GQA group of 3 and 2 new tokens."""
    lens = [2, 33, 200, 0]
    inp, kp, vp, bt = _paged_case(lens, 2, 12, 4, 64, 16, fp8, seed=350 + fp8, max_ctx=256)
    out, lse, _ = _paged_gpu(inp, kp, vp, bt, 64, fp8)
    o_ref, lse_ref, _ = _paged_ref(inp, kp, vp, bt, 16, fp8)
    assert_close(out.reshape(-1, 64), o_ref, what=f"paged decode group 3 fp8={fp8}")
    assert_lse_close(lse.reshape(-1), lse_ref, what="paged odd-group decode lse")


@pytest.mark.parametrize("P,fp8,q_len,D", [(16, False, 1, 64), (16, True, 1, 64),
                                           (64, False, 3, 64), (256, True, 2, 64),
                                           (16, False, 1, 128), (32, True, 4, 128)])
def test_decode_paged_all_rows(P, fp8, q_len, D):
    """Pages under a random table against the oracle on every row; lengths on
    page, sub-tile and chunk edges; unreferenced pages and page tails hold NaN
    (bf16) or the NaN code (FP8)."""
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700]
    max_ctx = -(-704 // P) * P
    inp, kp, vp, bt = _paged_case(lens, q_len, 64, 8, D, P, fp8, 130 + P + q_len + D, max_ctx)
    out, lse, _ = _paged_gpu(inp, kp, vp, bt, 256, fp8)
    o_ref, lse_ref, _ = _paged_ref(inp, kp, vp, bt, P, fp8)
    what = f"paged decode P={P} fp8={fp8} q_len={q_len} D={D}"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"{what} lse")


@pytest.mark.parametrize("P,split,fp8,D", [(256, 384, False, 64), (256, 384, True, 64),
                                            (128, 640, False, 128), (512, 896, True, 64)])
def test_decode_paged_chunks_straddle_pages_all_rows(P, split, fp8, D):
    """Chunk sizes that are not multiples of the page size (the chunk-size rule
    picks multiples of 128 below 1024 tokens for a few requests): chunks begin
    and end inside pages; every row against the oracle."""
    lens = [0, 1, 383, 384, 385, 511, 512, 513, 767, 768, 1000, 1900]
    max_ctx = -(-1904 // P) * P
    inp, kp, vp, bt = _paged_case(lens, 1, 16, 2, D, P, fp8, 170 + P + split + D, max_ctx)
    out, lse, _ = _paged_gpu(inp, kp, vp, bt, split, fp8)
    o_ref, lse_ref, _ = _paged_ref(inp, kp, vp, bt, P, fp8)
    what = f"paged decode P={P} split={split} fp8={fp8} D={D}"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"{what} lse")


@pytest.mark.parametrize("B,q_len,fp8", [(128, 1, False), (128, 3, True), (24, 3, False)])
def test_decode_paged_work_splits(B, q_len, fp8):
    """Each way waves share a chunk (four, one, two) over 16-token pages."""
    lens = [_EDGE_LENS[(3 * i) % len(_EDGE_LENS)] for i in range(B)]
    inp, kp, vp, bt = _paged_case(lens, q_len, 64, 8, 64, 16, fp8, 140 + B + q_len, 512)
    out, lse, (po, pm, pd) = _paged_gpu(inp, kp, vp, bt, 64, fp8)
    o_ref, lse_ref, _ = _paged_ref(inp, kp, vp, bt, 16, fp8)
    assert_close(out.reshape(-1, 64), o_ref, what=f"paged decode B={B} q_len={q_len}")
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"paged decode B={B} lse")
    assert not torch.isnan(po).any() and not torch.isnan(pm).any()


def test_decode_paged_full_config_all_rows():
    """64 requests x 8192 tokens in 16-token pages under a random table: every
    row against the oracle, with 1024-token chunks and with the 2048-token
    chunks the bench uses (the library's choice capped at 254 pages a chunk)."""
    cfg = wl.SPLIT_DECODE
    inp = wl.decode_inputs(cfg)
    g = torch.Generator().manual_seed(150)
    kp, bt = _to_pages(inp["k_cache"], 16, g, extra_pages=0)
    vp = torch.empty_like(kp)
    for b in range(bt.shape[0]):
        for p in range(bt.shape[1]):
            vp[int(bt[b, p])] = inp["v_cache"][b, :, p * 16:(p + 1) * 16]
    o_ref, lse_ref, _ = oracle.decode_multi(_q4(inp["q"]), inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    for split in (1024, 2048):
        out, lse, _ = _paged_gpu(inp, kp, vp, bt, split, False)
        assert_close(out.reshape(-1, cfg.head_dim), o_ref, what=f"paged decode full config, split {split}")
        assert_lse_close(lse.reshape(-1), lse_ref, what=f"paged decode full config lse, split {split}")


@pytest.mark.parametrize("fp8,P,D", [(False, 16, 64), (True, 16, 64), (False, 64, 128), (True, 32, 128)])
def test_kv_append_paged_bitwise(fp8, P, D):
    """Append through a random block table against the oracle, element for
    element (codes for FP8); slots past the table's capacity are dropped."""
    counts, Hkv, width = [3, 0, 130, 64, 90], 4, 8          # capacity 8 pages per request
    d = wl.kv_append_inputs(counts, width * P, Hkv, D, seed=160 + P + D,
                            pos=[0, 5, P + 3, width * P - 64, width * P - 50])
    g = torch.Generator().manual_seed(161)
    B = len(counts)
    num_pages = B * width + 3
    bt = torch.randperm(num_pages, generator=g)[:B * width].view(B, width).to(torch.int32)
    if fp8:
        kp = torch.randint(0, 256, (num_pages, Hkv, P, D), generator=g, dtype=torch.uint8)
        vp = torch.randint(0, 256, (num_pages, Hkv, P, D), generator=g, dtype=torch.uint8)
        ks = torch.empty(Hkv).uniform_(0.002, 0.02, generator=g)
        vs = torch.empty(Hkv).uniform_(0.002, 0.02, generator=g)
        sc = dict(k_scale=ks.numpy(), v_scale=vs.numpy())
        sg = dict(k_scale=ks.to(DEV), v_scale=vs.to(DEV))
    else:
        kp = torch.randn(num_pages, Hkv, P, D, generator=g).to(torch.bfloat16)
        vp = torch.randn(num_pages, Hkv, P, D, generator=g).to(torch.bfloat16)
        sc, sg = {}, {}
    ko, vo = oracle.kv_append_paged(d["k_new"], d["v_new"], d["cu_seqlens_new"], d["cache_pos"],
                                    kp, vp, bt, P, **sc)
    kg, vg = kp.to(DEV), vp.to(DEV)
    sa.sink_attn_kv_append_paged(d["k_new"].to(DEV), d["v_new"].to(DEV),
                                 d["cu_seqlens_new"].to(DEV), d["cache_pos"].to(DEV), kg, vg,
                                 bt.to(DEV), **sg)
    torch.cuda.synchronize()
    view = (lambda t: t) if fp8 else (lambda t: t.view(torch.int16))
    assert torch.equal(view(kg.cpu()), view(ko)) and torch.equal(view(vg.cpu()), view(vo))


# ---------------------------------------------------- one-launch decode --
def _fused_gpu(inp, split, *, fp8=False, counters=None):
    q = _q4(inp["q"]).to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    B, q_len, Hq, D = q.shape
    ns = -(-kc.shape[2] // split)
    po = torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    if counters is None:
        counters = sa.decode_counters(B, Hq, kc.shape[1], q_len, DEV)
    kw = dict(k_scale=inp["k_scale"].to(DEV), v_scale=inp["v_scale"].to(DEV)) if fp8 else {}
    sa.sink_attn_decode_fused(q, kc, vc, inp["seq_lens"].to(DEV), inp["sinks"].to(DEV), split,
                              ns, counters=counters, out=out, lse=lse, partials=(po, pm, pd),
                              **kw)
    torch.cuda.synchronize()
    return out, lse, counters


def _split_merge_gpu(inp, split, fp8):
    if fp8:
        out, lse, _ = _fp8_gpu(inp, split)
        return out, lse
    return _decode_multi_gpu(dict(inp, q=_q4(inp["q"])), split)


def _bitwise(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# (lens, q_len, Hq, Hkv, D, split): the waves each chunk gets (1, 2 or 4) and
# the column blocks per workgroup follow from the shape, so these cover all of
# them -- head_dim 64 with one 16-column block (4 waves), head_dim 128 with
# 1024 chunks (1 wave) and 512 chunks (2 waves), few chunks (4 waves), two
# column blocks at 1024 chunks, and 128 columns per KV head (two slices).
_FUSED_CASES = [
    ([0, 1, 65, 257, 1000, 3000], 1, 64, 8, 64, 256),
    ([5, 700, 8192, 8192], 1, 64, 8, 128, 256),
    ([5, 700, 4096, 4096], 1, 64, 8, 128, 256),
    ([3, 64, 1000], 2, 64, 4, 128, 256),
    ([4, 129, 8192, 8000], 4, 64, 8, 64, 256),
    ([16, 130, 700], 16, 64, 8, 64, 512),
]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("case", range(len(_FUSED_CASES)))
def test_decode_fused_is_bitwise_split_then_merge(case, fp8):
    """The one-launch call gives bitwise the output and lse of the two-call
    path (the merge is the same per-row code), and leaves its counters zero."""
    lens, q_len, Hq, Hkv, D, split = _FUSED_CASES[case]
    mk = _fp8_cfg if fp8 else _multi_cfg
    inp = mk(lens, q_len, Hq, Hkv, D, seed=190 + case, split=split,
             edges={0: float("-inf"), Hq - 1: 20.0})
    out_f, lse_f, cnt = _fused_gpu(inp, split, fp8=fp8)
    out_s, lse_s = _split_merge_gpu(inp, split, fp8)
    assert _bitwise(out_f, out_s), f"fused output differs from split+merge, case {case}"
    assert torch.equal(lse_f, lse_s), f"fused lse differs from split+merge, case {case}"
    assert int(cnt.abs().sum()) == 0


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_fused_all_rows_against_the_oracle(fp8):
    """Ragged lengths (0, shorter than q_len, chunk edges) on every row."""
    lens, q_len, Hq, Hkv, D = [0, 2, 3, 64, 257, 513, 1000], 3, 32, 4, 64
    mk = _fp8_cfg if fp8 else _multi_cfg
    inp = mk(lens, q_len, Hq, Hkv, D, seed=200, split=256, edges={1: float("-inf"), 5: 20.0})
    out, lse, _ = _fused_gpu(inp, 256, fp8=fp8)
    if fp8:
        o_ref, lse_ref, _ = _fp8_ref(inp)
    else:
        o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                                inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, D), o_ref, what=f"fused decode fp8={fp8}")
    assert_lse_close(lse.reshape(-1), lse_ref, what=f"fused decode lse fp8={fp8}")


def test_decode_fused_reuses_its_counters_across_shapes():
    """One counter buffer serves calls of different shapes back to back (the
    last arrival of every slice resets its counter)."""
    big = _multi_cfg([7, 3000, 2048, 90], 4, 64, 8, 64, seed=210, split=256)
    small = _multi_cfg([1, 500], 1, 64, 8, 64, seed=211, split=256)
    cnt = sa.decode_counters(4, 64, 8, 4, DEV)
    for inp in (big, small, big):
        out_f, lse_f, _ = _fused_gpu(inp, 256, counters=cnt)
        out_s, lse_s = _split_merge_gpu(inp, 256, False)
        assert _bitwise(out_f, out_s) and torch.equal(lse_f, lse_s)
        assert int(cnt.abs().sum()) == 0


def test_decode_fused_strided_output():
    """Output rows inside a wider buffer: only the addressed elements change."""
    inp = _multi_cfg([50, 600], 2, 16, 2, 128, seed=220, split=256)
    q = inp["q"].to(DEV)
    big = torch.full((2, 3, 16, 144), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = big[:, 1:, :, 8:136]
    sa.sink_attn_decode_fused(q, inp["k_cache"].to(DEV), inp["v_cache"].to(DEV),
                              inp["seq_lens"].to(DEV), inp["sinks"].to(DEV), 256, out=out)
    torch.cuda.synchronize()
    ref, _ = _split_merge_gpu(inp, 256, False)
    assert _bitwise(out.contiguous(), ref)
    rest = big.clone()
    rest[:, 1:, :, 8:136] = 0
    assert torch.isnan(rest[:, :1].float()).all() and torch.isnan(rest[..., :8].float()).all()
    assert torch.isnan(rest[..., 136:].float()).all()


# ----------------------------------------------------------- graph capture --
def test_decode_and_prefill_replay_from_a_captured_graph():
    """The calls only enqueue kernels on the caller's stream (no allocation,
    no synchronisation, no memset), so they can be captured in a HIP graph.
    Capture prefill + split decode + merge + one-launch decode once, then replay with new inputs
    copied into the captured buffers, eager work and a synchronisation between
    replays, and check every replay against an eager run."""
    g = torch.Generator().manual_seed(170)
    pre = _prefill_case([300, 77], 16, 2, 64, seed=171)
    dcfg = wl.DecodeConfig("graph", 4, None, (100, 2000), 2048, 16, 2, 64, (-4.0, 4.0),
                           split_size=512, seed=172)
    dec = wl.decode_inputs(dcfg, poison=0.0)
    q_p, k_p, v_p = pre["q"].to(DEV), pre["k"].to(DEV), pre["v"].to(DEV)
    s_p, cu = pre["sinks"].to(DEV), pre["cu_seqlens"].to(DEV)
    q_d, kc, vc = dec["q"].to(DEV), dec["k_cache"].to(DEV), dec["v_cache"].to(DEV)
    lens, s_d = dec["seq_lens"].to(DEV), dec["sinks"].to(DEV)
    o_p = torch.empty_like(q_p)
    ns = 4
    po = torch.empty(4, 16, ns, 64, device=DEV)
    pm = torch.empty(4, 16, ns, device=DEV)
    pd = torch.empty(4, 16, ns, device=DEV)
    o_d = torch.empty(4, 16, 64, dtype=torch.bfloat16, device=DEV)
    o_f = torch.empty_like(o_d)
    cnt = sa.decode_counters(4, 16, 2, 1, DEV)
    fpart = (torch.empty_like(po), torch.empty_like(pm), torch.empty_like(pd))

    def step():
        sa.sink_attn_prefill(q_p, k_p, v_p, s_p, cu, pre["max_seqlen"], out=o_p)
        sa.sink_attn_decode(q_d, kc, vc, lens, s_d, 512, ns, out=o_d, partials=(po, pm, pd))
        sa.sink_attn_decode_fused(q_d, kc, vc, lens, s_d, 512, ns, counters=cnt, out=o_f,
                                  partials=fpart)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        q_p.copy_(torch.randn(q_p.shape, generator=g).to(torch.bfloat16))
        q_d.copy_(torch.randn(q_d.shape, generator=g).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_p, got_d, got_f = o_p.clone(), o_d.clone(), o_f.clone()
        scratch = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        step()                                   # eager reference on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_p.view(torch.int16), o_p.view(torch.int16)), f"prefill replay {rep}"
        assert torch.equal(got_d.view(torch.int16), o_d.view(torch.int16)), f"decode replay {rep}"
        assert torch.equal(got_f.view(torch.int16), o_d.view(torch.int16)), f"fused replay {rep}"
        assert int(cnt.abs().sum()) == 0
        assert torch.isfinite(scratch)
    # and the replayed decode is right, not merely repeatable
    o_ref, _, _ = oracle.decode(q_d.cpu(), dec["k_cache"], dec["v_cache"], dec["seq_lens"],
                                dec["sinks"])
    assert_close(o_d.cpu().reshape(-1, 64), o_ref, what="decode after graph replays")


def _merge_inputs(B, Hq, ns, D, seed):
    """Chunk states with the cases a merge meets: chunks with m = -inf and d = 0
    (past a request's end), rows with no weight at all, a wide spread of m and
    chunks with d = 0 but a finite m."""
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(B, Hq, ns, D, generator=g)
    pm = torch.randn(B, Hq, ns, generator=g) * 8
    pd = torch.rand(B, Hq, ns, generator=g) * 50
    empty = torch.rand(B, Hq, ns, generator=g) < 0.4
    pm[empty], pd[empty], po[empty] = float("-inf"), 0.0, 0.0
    pm[0, 0], pd[0, 0], po[0, 0] = float("-inf"), 0.0, 0.0          # a row with no weight
    pd[0, 1, 0] = 0.0                                                 # d = 0, finite m
    return po, pm, pd


@pytest.mark.parametrize("ns", [1, 7, 16, 17, 40, 100])
@pytest.mark.parametrize("D", [64, 128])
def test_merge_states_against_the_oracle(ns, D):
    """sink_attn_merge_states on adversarial chunk states (up to 16 chunks and
    past it) against the oracle's fp64 merge; and, from a part_o that is only
    4-byte aligned, the same bits."""
    B, Hq = 3, 40
    po, pm, pd = _merge_inputs(B, Hq, ns, D, seed=500 + ns + D)
    o_ref, lse_ref = oracle.merge_states(po.reshape(-1, ns, D).double().numpy(),
                                         pm.reshape(-1, ns).double().numpy(),
                                         pd.reshape(-1, ns).double().numpy())
    g_po, g_pm, g_pd = po.to(DEV), pm.to(DEV), pd.to(DEV)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq), float("nan"), device=DEV)
    sa.sink_attn_merge_states(g_po, g_pm, g_pd, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_close(out.reshape(-1, D), o_ref, what=f"merge ns={ns} D={D}")
    lse_h = lse.reshape(-1).cpu()
    assert torch.isneginf(lse_h[0]) and torch.all(out[0, 0].float() == 0)
    assert_lse_close(lse_h, lse_ref, what=f"merge ns={ns} D={D} lse")
    # part_o one float past a 16-byte boundary
    buf = torch.empty(po.numel() + 1, device=DEV)
    g_po2 = buf[1:].view(po.shape)
    g_po2.copy_(g_po)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    sa.sink_attn_merge_states(g_po2, g_pm, g_pd, out=out2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse2, lse)


# ------------------------------------------ split + length-aware merge --
def _merged_gpu(inp, split, *, fp8=False):
    q = _q4(inp["q"]).to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    B, q_len, Hq, D = q.shape
    ns = -(-kc.shape[2] // split)
    po = torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV)
    pm = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    pd = torch.full((B, q_len, Hq, ns), float("nan"), device=DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    kw = dict(k_scale=inp["k_scale"].to(DEV), v_scale=inp["v_scale"].to(DEV)) if fp8 else {}
    sa.sink_attn_decode_merged(q, kc, vc, inp["seq_lens"].to(DEV), inp["sinks"].to(DEV), split,
                               ns, out=out, lse=lse, partials=(po, pm, pd), **kw)
    torch.cuda.synchronize()
    return out, lse, (po, pm, pd)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("case", range(len(_FUSED_CASES)))
def test_decode_merged_is_bitwise_split_then_merge(case, fp8):
    """Split decode whose chunks past a request's end write nothing, merged
    over the chunks that hold keys: bitwise the output and lse of split decode
    + sink_attn_merge_states (the partials start as NaN, so a chunk state the
    merge read without it being written would show); every wave split."""
    lens, q_len, Hq, Hkv, D, split = _FUSED_CASES[case]
    mk = _fp8_cfg if fp8 else _multi_cfg
    inp = mk(lens, q_len, Hq, Hkv, D, seed=290 + case, split=split,
             edges={0: float("-inf"), Hq - 1: 20.0})
    out_m, lse_m, (po, pm, pd) = _merged_gpu(inp, split, fp8=fp8)
    out_s, lse_s = _split_merge_gpu(inp, split, fp8)
    assert _bitwise(out_m, out_s), f"merged output differs from split+merge, case {case}"
    assert torch.equal(lse_m, lse_s), f"merged lse differs from split+merge, case {case}"
    # chunks past each request's end were left untouched (still NaN)
    ns = pm.shape[-1]
    for b, L in enumerate(lens):
        live = max(1, min(ns, -(-L // split)))
        assert torch.isnan(pm[b, ..., live:]).all() and not torch.isnan(pm[b, ..., :live]).any()


def test_decode_merged_ragged_against_the_oracle():
    """Every row of a ragged batch with most chunks past the ends (lengths 0,
    shorter than q_len, chunk edges; 40 chunks of 64 keys) against the oracle."""
    lens, q_len, Hq, Hkv, D = [0, 2, 3, 64, 65, 257, 513, 1000, 2560], 3, 32, 4, 64
    inp = _multi_cfg(lens, q_len, Hq, Hkv, D, seed=300, split=64, max_ctx=2560,
                     edges={1: float("-inf"), 5: 20.0})
    out, lse, _ = _merged_gpu(inp, 64)
    o_ref, lse_ref, _ = oracle.decode_multi(inp["q"], inp["k_cache"], inp["v_cache"],
                                            inp["seq_lens"], inp["sinks"])
    assert_close(out.reshape(-1, D), o_ref, what="merged decode")
    assert_lse_close(lse.reshape(-1), lse_ref, what="merged decode lse")
