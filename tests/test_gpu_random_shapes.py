"""GPU parity over seeded random shapes: prefill (plain and chunked) and decode
(split + merge, length-aware merge, FP8 and paged caches) against the fp64
oracle on every row, with the shape of each case -- lengths, GQA group, head
dim, causal flag, sink edge values, chunk size, new tokens per request, page
size -- drawn from a seeded generator.  The case number names the draw.
"""
import random

import pytest
import torch

import gqa_attention_sinks_prefill_amd as sa
import oracle
from gqa_attention_sinks_prefill_amd import workloads as wl
from parity_utils import assert_close, assert_lse_close

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
N_PREFILL, N_CHUNKED, N_DECODE = 64, 24, 64


def _heads(r):
    Hkv = r.choice([1, 2, 4, 8])
    group = r.choice([1, 2, 3, 4, 5, 6, 8, 16])
    return Hkv * group, Hkv


def _edges(r, Hq):
    """Up to two heads with an edge sink: -inf (plain attention) or +20 (the sink dominates)."""
    e = {}
    for _ in range(r.randint(0, 2)):
        e[r.randrange(Hq)] = r.choice([float("-inf"), 20.0])
    return e


def _length(r, hi):
    """A length in [0, hi]: often near a 32 / 64-token tile edge, sometimes 0-4."""
    if r.random() < 0.12:
        return r.randint(0, 4)
    if r.random() < 0.4:
        return max(0, min(hi, r.choice([32, 64, 128, 256, 512]) * r.randint(1, 4) + r.randint(-1, 1)))
    return r.randint(0, hi)


def _prefill_draw(case):
    r = random.Random(1000 + case)
    Hq, Hkv = _heads(r)
    D = r.choice([64, 128])
    lens = [_length(r, 700) for _ in range(r.randint(1, 4))]
    if max(lens) == 0:
        lens[0] = 1
    return dict(lens=lens, Hq=Hq, Hkv=Hkv, D=D, causal=r.random() < 0.7,
                nhd=r.random() < 0.25, edges=_edges(r, Hq), seed=2000 + case)


@pytest.mark.parametrize("case", range(N_PREFILL))
def test_random_prefill_all_rows(case):
    p = _prefill_draw(case)
    cfg = wl.PrefillConfig("random", tuple(p["lens"]), len(p["lens"]), None, p["Hq"], p["Hkv"],
                           p["D"], (-4.0, 4.0), seed=p["seed"], edge_sinks=p["edges"])
    inp = wl.prefill_inputs(cfg)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    layout = "nhd" if p["nhd"] else "hnd"
    if p["nhd"]:
        k, v = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()
    T = q.shape[0]
    out = torch.full((T, p["Hq"], p["D"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, p["Hq"]), float("nan"), device=DEV)
    sa.sink_attn_prefill(q, k, v, inp["sinks"].to(DEV), inp["cu_seqlens"].to(DEV),
                         inp["max_seqlen"], causal=p["causal"], kv_layout=layout, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                       inp["cu_seqlens"], causal=p["causal"], scale=cfg.scale)
    what = f"random prefill case {case} {p}"
    assert_close(out.reshape(-1, p["D"]), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=what)


@pytest.mark.parametrize("case", range(N_CHUNKED))
def test_random_chunked_prefill_all_rows(case):
    r = random.Random(3000 + case)
    Hq, Hkv = _heads(r)
    D = r.choice([64, 128])
    lens = [max(1, _length(r, 900)) for _ in range(r.randint(1, 4))]
    chunk = r.choice([1, 17, 64, 100, 256, 512])
    causal = r.random() < 0.7
    cfg = wl.PrefillConfig("random_chunked", tuple(lens), len(lens), None, Hq, Hkv, D,
                           (-4.0, 4.0), seed=4000 + case, edge_sinks=_edges(r, Hq))
    inp = wl.chunked_prefill_inputs(cfg, chunk)
    q = inp["q"].to(DEV)
    Tq = q.shape[0]
    out = torch.full((Tq, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((Tq, Hq), float("nan"), device=DEV)
    sa.sink_attn_prefill_chunked(q, inp["k"].to(DEV), inp["v"].to(DEV), inp["sinks"].to(DEV),
                                 inp["cu_seqlens_q"].to(DEV), inp["cu_seqlens_k"].to(DEV),
                                 inp["max_seqlen_q"], causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                               inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                               causal=causal, scale=cfg.scale)
    what = f"random chunked prefill case {case} (lens {lens}, chunk {chunk}, Hq {Hq}, Hkv {Hkv}, D {D})"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=what)


def _decode_draw(case):
    r = random.Random(5000 + case)
    Hq, Hkv = _heads(r)
    D = r.choice([64, 128])
    q_len = r.choice([1, 1, 1, 2, 3, 4])
    lens = [_length(r, 3000) for _ in range(r.randint(1, 5))]
    max_ctx = max(max(lens), 1) + r.choice([0, 0, 37, 300])
    split = 64 * r.randint(1, 32)
    path = r.choice(["split_merge", "merged", "fp8", "paged", "paged_fp8"])
    page = r.choice([16, 32, 64])
    return dict(Hq=Hq, Hkv=Hkv, D=D, q_len=q_len, lens=lens, max_ctx=max_ctx, split=split,
                path=path, page=page, edges=_edges(r, Hq), seed=6000 + case)


def _partials(B, q_len, Hq, ns, D):
    return (torch.full((B, q_len, Hq, ns, D), float("nan"), device=DEV),
            torch.full((B, q_len, Hq, ns), float("nan"), device=DEV),
            torch.full((B, q_len, Hq, ns), float("nan"), device=DEV))


@pytest.mark.parametrize("case", range(N_DECODE))
def test_random_decode_all_rows(case):
    p = _decode_draw(case)
    fp8 = p["path"] in ("fp8", "paged_fp8")
    cfg = wl.DecodeConfig("random_decode", len(p["lens"]), None, (1, 1), p["max_ctx"], p["Hq"],
                          p["Hkv"], p["D"], (-4.0, 4.0), split_size=p["split"], seed=p["seed"],
                          edge_sinks=p["edges"], q_len=p["q_len"])
    inp = (wl.fp8_decode_inputs if fp8 else wl.decode_inputs)(cfg, lens=p["lens"])
    q = inp["q"]
    q4 = (q.unsqueeze(1) if q.dim() == 3 else q).to(DEV)
    B, q_len, Hq, D = q4.shape
    split = p["split"]
    lens, sinks = inp["seq_lens"].to(DEV), inp["sinks"].to(DEV)
    out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    sc = dict(k_scale=inp["k_scale"].to(DEV), v_scale=inp["v_scale"].to(DEV)) if fp8 else {}
    if p["path"].startswith("paged"):
        P = p["page"]
        g = torch.Generator().manual_seed(p["seed"])
        L = inp["k_cache"].shape[2]
        per = -(-L // P)
        perm = torch.randperm(B * per + 3, generator=g)[:B * per].view(B, per).to(torch.int32)
        poison = 0x7F if fp8 else float("nan")
        shape = (B * per + 3, p["Hkv"], P, D)
        kp = torch.full(shape, poison, dtype=inp["k_cache"].dtype)
        vp = torch.full(shape, poison, dtype=inp["v_cache"].dtype)
        for b in range(B):
            for j in range(per):
                kb = inp["k_cache"][b, :, j * P:(j + 1) * P]
                kp[int(perm[b, j]), :, :kb.shape[1]] = kb
                vp[int(perm[b, j]), :, :kb.shape[1]] = inp["v_cache"][b, :, j * P:(j + 1) * P]
        ns = -(-per * P // split)
        sa.sink_attn_decode_paged(q4, kp.to(DEV), vp.to(DEV), perm.to(DEV), lens, sinks, split, ns,
                                  out=out, lse=lse, partials=_partials(B, q_len, Hq, ns, D), **sc)
        torch.cuda.synchronize()
        ref_kw = dict(k_scale=inp["k_scale"].numpy(), v_scale=inp["v_scale"].numpy()) if fp8 else {}
        o_ref, lse_ref, _ = oracle.decode_multi_paged(q4.cpu(), kp, vp, perm, P, inp["seq_lens"],
                                                      inp["sinks"], **ref_kw)
    else:
        kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
        ns = -(-kc.shape[2] // split)
        part = _partials(B, q_len, Hq, ns, D)
        if p["path"] == "merged":
            sa.sink_attn_decode_merged(q4, kc, vc, lens, sinks, split, ns, out=out, lse=lse,
                                       partials=part)
        elif fp8:
            sa.sink_attn_decode_fp8(q4, kc, vc, sc["k_scale"], sc["v_scale"], lens, sinks, split,
                                    ns, out=out, lse=lse, partials=part)
        else:
            sa.sink_attn_decode_multi(q4, kc, vc, lens, sinks, split, ns, out=out, lse=lse,
                                      partials=part)
        torch.cuda.synchronize()
        if fp8:
            o_ref, lse_ref, _ = oracle.decode_multi_fp8(q4.cpu(), inp["k_cache"], inp["v_cache"],
                                                        inp["k_scale"].numpy(),
                                                        inp["v_scale"].numpy(), inp["seq_lens"],
                                                        inp["sinks"])
        else:
            o_ref, lse_ref, _ = oracle.decode_multi(q4.cpu(), inp["k_cache"], inp["v_cache"],
                                                    inp["seq_lens"], inp["sinks"])
    what = f"random decode case {case} {p}"
    assert_close(out.reshape(-1, D), o_ref, what=what)
    assert_lse_close(lse.reshape(-1), lse_ref, what=what)
