"""sink_attn_decode_merged_noalloc (chunk states in the library's device scratch
array) against sink_attn_decode_merged (caller-owned partials): called through
the C ABI, bitwise equal output and lse on two calls in a row, the second with
a smaller input, and within the parity bar of the oracle."""
import ctypes

import pytest
import torch

import gqa_attention_sinks_prefill_amd as sa
import oracle
from gqa_attention_sinks_prefill_amd import workloads as wl
from parity_utils import assert_close, assert_lse_close

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _case(lens, q_len, Hq, Hkv, D, split, seed, max_ctx):
    cfg = wl.DecodeConfig("noalloc", len(lens), None, (1, 1), max_ctx, Hq, Hkv, D, (-4.0, 4.0),
                          split_size=split, seed=seed, q_len=q_len,
                          edge_sinks={0: float("-inf"), Hq - 1: 20.0})
    return cfg, wl.decode_inputs(cfg, lens=lens)


def _noalloc_abi(q4, kc, vc, lens, sinks, split, ns, out, lse):
    """The entry point called through ctypes with raw device pointers."""
    lib = sa.load_library()
    B, q_len, Hq, D = q4.shape
    rc = lib.sink_attn_decode_merged_noalloc(
        q4.data_ptr(), q4.stride(0), q4.stride(1), q4.stride(2), q_len, kc.data_ptr(),
        vc.data_ptr(), kc.stride(0), kc.stride(1), kc.stride(2), None, None, lens.data_ptr(), B,
        kc.shape[2], sinks.data_ptr(), Hq, kc.shape[1], D, ctypes.c_float(1.0 / D ** 0.5),
        split, ns, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.sink_attn_last_error().decode()


def _run_pair(lens, q_len, Hq, Hkv, D, split, seed, max_ctx):
    cfg, inp = _case(lens, q_len, Hq, Hkv, D, split, seed, max_ctx)
    q = inp["q"] if q_len > 1 else inp["q"].unsqueeze(1)
    q4 = q.to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    lens_d, sinks = inp["seq_lens"].to(DEV), inp["sinks"].to(DEV)
    B = len(lens)
    ns = -(-max_ctx // split)
    out_n = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse_n = torch.full((B, q_len, Hq), float("nan"), device=DEV)
    _noalloc_abi(q4, kc, vc, lens_d, sinks, split, ns, out_n, lse_n)
    out_r = torch.full_like(out_n, float("nan"))
    lse_r = torch.full_like(lse_n, float("nan"))
    sa.sink_attn_decode_merged(q4, kc, vc, lens_d, sinks, split, ns, out=out_r, lse=lse_r)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16), out_r.view(torch.int16)), "output differs"
    assert torch.equal(lse_n, lse_r), "lse differs"
    o_ref, lse_ref, _ = oracle.decode_multi(q, inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                            inp["sinks"])
    assert_close(out_n.reshape(-1, D), o_ref, what="no-alloc decode")
    assert_lse_close(lse_n.reshape(-1), lse_ref, what="no-alloc decode lse")


def test_decode_merged_noalloc_matches_the_allocating_call_twice():
    # first call: 16 requests of up to 9000 tokens, 1024-token chunks (4.4 M fp32 of states)
    lens = [0, 1, 63, 64, 1025, 4096, 9000, 8191, 3000, 700, 5, 2048, 6000, 7777, 100, 8999]
    _run_pair(lens, 1, 64, 8, 64, 1024, seed=401, max_ctx=9000)
    # second call, smaller: 3 requests, 3 new tokens each, head_dim 128, 256-token chunks;
    # the scratch still holds the first call's states past this call's rows
    _run_pair([2, 700, 1500], 3, 32, 4, 128, 256, seed=402, max_ctx=1500)


def test_decode_merged_noalloc_rejects_states_past_its_scratch():
    q = torch.zeros(1, 64, 64, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, 8, 64, 64, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(1, dtype=torch.int32, device=DEV)
    with pytest.raises(sa.SinkAttnError, match="scratch"):
        sa.sink_attn_decode_merged_noalloc(q, kc, kc, lens, torch.zeros(64, device=DEV), 64,
                                           num_splits=1 << 14)
