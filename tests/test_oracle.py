"""Pins for the CPU oracle: each test ties it to something other than itself.

Sources of truth, none of which is the oracle's own formula typed again:
* a library routine: torch's scaled_dot_product_attention in float64 on CPU
  (a -inf sink must reduce sink attention to it exactly; a finite sink must
  equal it over one extra all-zero key whose column carries the sink as an
  additive mask);
* closed forms (identical keys; a single visible key; the sink share);
* invariants (split-then-merge equals unsplit for every chunk size, with a
  negative control; GQA equals MHA over repeated K/V; key permutation).

A plausible slip in the oracle -- a dropped sink term, the sink scaled by the
softmax scale, j < i instead of j <= i, the wrong GQA grouping, the sink in
every chunk -- fails at least one test here.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _bf16_randn(g, *shape, scale=1.0):
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _sdpa(q, k, v, *, causal, scale, mask=None):
    """float64 SDPA; q [H, L, D], k/v [H, S, D] (already expanded over GQA)."""
    return F.scaled_dot_product_attention(
        q.double().unsqueeze(0), k.double().unsqueeze(0), v.double().unsqueeze(0),
        attn_mask=None if mask is None else mask.unsqueeze(0), is_causal=causal,
        scale=scale).squeeze(0)


def _packed_prefill(g, lens, Hq, Hkv, D):
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens), 0)
    T = int(cu[-1])
    q = _bf16_randn(g, T, Hq, D)
    k = _bf16_randn(g, Hkv, T, D)
    v = _bf16_randn(g, Hkv, T, D)
    return q, k, v, cu


# ---------------------------------------------------------------- P1 ------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 8), (6, 2, 4), (8, 8, 64), (8, 2, 64)])
def test_neg_inf_sink_is_standard_attention_prefill(causal, Hq, Hkv, D):
    g = torch.Generator().manual_seed(11 + Hq + D)
    lens = [1, 5, 17, 33]
    q, k, v, cu = _packed_prefill(g, lens, Hq, Hkv, D)
    sinks = torch.full((Hq,), float("-inf"))
    scale = 1.0 / math.sqrt(D)
    o, _, share = oracle.prefill(q, k, v, sinks, cu, causal=causal, scale=scale)
    o = o.reshape(-1, Hq, D)
    r = Hq // Hkv
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        qs = q[a:b].transpose(0, 1)                              # [Hq, L, D]
        ks = k[:, a:b].repeat_interleave(r, dim=0)               # contiguous groups
        vs = v[:, a:b].repeat_interleave(r, dim=0)
        ref = _sdpa(qs, ks, vs, causal=causal, scale=scale).transpose(0, 1)
        np.testing.assert_allclose(o[a:b], ref.numpy(), rtol=0, atol=1e-12)
    assert np.all(share == 0.0)


def test_neg_inf_sink_is_standard_attention_decode():
    g = torch.Generator().manual_seed(5)
    B, Hq, Hkv, D, max_ctx = 3, 8, 2, 16, 40
    lens = torch.tensor([40, 1, 23], dtype=torch.int32)
    q = _bf16_randn(g, B, Hq, D)
    kc = _bf16_randn(g, B, Hkv, max_ctx, D)
    vc = _bf16_randn(g, B, Hkv, max_ctx, D)
    sinks = torch.full((Hq,), float("-inf"))
    o, _, _ = oracle.decode(q, kc, vc, lens, sinks)
    o = o.reshape(B, Hq, D)
    for b in range(B):
        L = int(lens[b])
        ks = kc[b, :, :L].repeat_interleave(Hq // Hkv, dim=0)
        vs = vc[b, :, :L].repeat_interleave(Hq // Hkv, dim=0)
        ref = _sdpa(q[b].unsqueeze(1), ks, vs, causal=False, scale=1 / math.sqrt(D))
        np.testing.assert_allclose(o[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P5 ------
@pytest.mark.parametrize("causal", [True, False])
def test_sink_is_an_extra_zero_key_with_additive_mask(causal):
    """A finite sink equals SDPA over n+1 keys: an all-zero key (logit 0) with
    a zero value row, whose column gets the raw sink as an additive mask."""
    g = torch.Generator().manual_seed(7)
    Hq, Hkv, D, L = 8, 2, 32, 29
    q, k, v, cu = _packed_prefill(g, [L], Hq, Hkv, D)
    sinks = torch.empty(Hq).uniform_(-4, 4, generator=g)
    sinks[3] = 20.0
    scale = 1.0 / math.sqrt(D)
    o, _, _ = oracle.prefill(q, k, v, sinks, cu, causal=causal, scale=scale)
    o = o.reshape(L, Hq, D)
    r = Hq // Hkv
    qs = q.transpose(0, 1)
    ks = torch.cat([torch.zeros(Hkv, 1, D, dtype=k.dtype), k], 1).repeat_interleave(r, 0)
    vs = torch.cat([torch.zeros(Hkv, 1, D, dtype=v.dtype), v], 1).repeat_interleave(r, 0)
    mask = torch.zeros(Hq, L, L + 1, dtype=torch.float64)
    mask[:, :, 0] = sinks.double()[:, None]
    if causal:   # key j+1 of the extended set is visible to row i iff j <= i
        mask[:, :, 1:] = torch.triu(torch.full((L, L), float("-inf"), dtype=torch.float64), 1)
    ref = _sdpa(qs, ks, vs, causal=False, scale=scale, mask=mask).transpose(0, 1)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P2 ------
@pytest.mark.parametrize("n", [1, 2, 7, 64])
@pytest.mark.parametrize("sink", [-3.0, 0.0, 1.5, 20.0])
def test_identical_keys_closed_form(n, sink):
    """n copies of one key/value: o = n e^x / (n e^x + e^s) * v with x = scale q.k."""
    D = 8
    qv = torch.tensor([1.0, -0.5, 0.25, 2.0, 0.0, 1.0, -1.0, 0.5])
    kv = torch.tensor([0.5, 1.0, -2.0, 0.75, 3.0, -0.25, 0.5, 1.0])
    vv = torch.tensor([1.0, 2.0, -3.0, 0.5, 0.0, -1.25, 4.0, 0.125])
    q = qv.to(torch.bfloat16).reshape(1, 1, D)
    kc = kv.to(torch.bfloat16).reshape(1, 1, 1, D).expand(1, 1, n, D).contiguous()
    vc = vv.to(torch.bfloat16).reshape(1, 1, 1, D).expand(1, 1, n, D).contiguous()
    scale = 0.5
    o, lse, share = oracle.decode(q, kc, vc, torch.tensor([n], dtype=torch.int32),
                                  torch.tensor([sink]), scale=scale)
    x = scale * float(np.dot(qv.numpy().astype(np.float64), kv.numpy().astype(np.float64)))
    w = n * math.exp(x) / (n * math.exp(x) + math.exp(sink))
    np.testing.assert_allclose(o[0], w * vv.numpy().astype(np.float64), rtol=1e-13, atol=1e-300)
    assert lse[0] == pytest.approx(math.log(n * math.exp(x) + math.exp(sink)), rel=1e-13)
    assert share[0] == pytest.approx(1.0 - w, rel=1e-12, abs=1e-15)


def test_first_causal_row_sees_only_key_zero():
    """Row 0 of a causal prefill sees key 0 alone: o = e^x0/(e^x0+e^s) v0."""
    g = torch.Generator().manual_seed(3)
    q, k, v, cu = _packed_prefill(g, [9, 6], 2, 1, 16)
    sinks = torch.tensor([0.7, -1.1])
    o, _, _ = oracle.prefill(q, k, v, sinks, cu, causal=True, scale=0.25,
                             rows=[(0, 0), (0, 1), (9, 1)])
    for i, (t, h) in enumerate([(0, 0), (0, 1), (9, 1)]):
        x0 = 0.25 * float(q[t, h].double() @ k[0, t].double())
        p = math.exp(x0) / (math.exp(x0) + math.exp(float(sinks[h])))
        np.testing.assert_allclose(o[i], p * v[0, t].double().numpy(), rtol=1e-13, atol=1e-300)


# ---------------------------------------------------------------- P3 ------
def test_sink_share_matches_logaddexp():
    g = torch.Generator().manual_seed(9)
    B, Hq, Hkv, D, L = 2, 4, 1, 64, 50
    q = _bf16_randn(g, B, Hq, D)
    kc = _bf16_randn(g, B, Hkv, L, D, scale=2.0)
    vc = _bf16_randn(g, B, Hkv, L, D)
    sinks = torch.tensor([-2.0, 0.0, 3.0, 20.0])
    lens = torch.tensor([L, 13], dtype=torch.int32)
    o_nos, lse_nos, _ = oracle.decode(q, kc, vc, lens, torch.full((Hq,), float("-inf")))
    o, lse, share = oracle.decode(q, kc, vc, lens, sinks)
    s = np.tile(sinks.double().numpy(), B)
    # share = e^s / (e^s + sum e^x) = exp(s - logaddexp(s, lse_std))
    np.testing.assert_allclose(share, np.exp(s - np.logaddexp(s, lse_nos)), rtol=1e-12)
    np.testing.assert_allclose(lse, np.logaddexp(s, lse_nos), rtol=1e-13)
    # ---------------------------------------------------------- P6 ------
    # o_sink = sigmoid(lse_std - s) * o_std, row by row
    sig = 1.0 / (1.0 + np.exp(s - lse_nos))
    np.testing.assert_allclose(o, sig[:, None] * o_nos, rtol=0, atol=1e-13)
    # the weights of the keys and the sink sum to one: sum_j p_j = 1 - share
    rows = [(0, 1)]
    o1, _, sh1 = oracle.decode(q, kc, torch.ones_like(vc), lens, sinks, rows=rows)
    np.testing.assert_allclose(o1[0], np.full(D, 1.0 - sh1[0]), rtol=1e-13)


# ---------------------------------------------------------------- P4 ------
def _decode_case(seed=21, n=37, D=8):
    g = torch.Generator().manual_seed(seed)
    q = _bf16_randn(g, 1, 2, D)
    kc = _bf16_randn(g, 1, 1, n, D, scale=1.5)
    vc = _bf16_randn(g, 1, 1, n, D)
    sinks = torch.tensor([1.25, -0.5])
    return q, kc, vc, torch.tensor([n], dtype=torch.int32), sinks


def test_split_then_merge_equals_unsplit_every_chunk_size():
    q, kc, vc, lens, sinks = _decode_case()
    n = int(lens[0])
    o_ref, lse_ref, _ = oracle.decode(q, kc, vc, lens, sinks)
    for S in range(1, n + 1):
        for extra in (0, 2):                     # trailing empty chunks too
            ns = -(-n // S) + extra
            o_p, m_p, d_p = oracle.chunk_states(q, kc, vc, lens, sinks, S, ns)
            o, lse = oracle.merge_states(o_p, m_p, d_p)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12, err_msg=f"S={S}")
            np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, err_msg=f"S={S}")
            if extra:
                assert np.all(np.isneginf(m_p[:, -1])) and np.all(d_p[:, -1] == 0)


def test_sink_in_any_single_chunk_is_equivalent():
    q, kc, vc, lens, sinks = _decode_case(seed=4)
    o_ref, _, _ = oracle.decode(q, kc, vc, lens, sinks)
    for c in range(5):
        o, _ = oracle.merge_states(*oracle.chunk_states(q, kc, vc, lens, sinks, 8, 5,
                                                        sink_chunk=c))
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)


def test_sink_in_every_chunk_is_wrong_negative_control():
    """Seeding every chunk counts the sink k times: equal to sink + ln k, not sink."""
    q, kc, vc, lens, sinks = _decode_case(seed=8)
    o_ref, _, _ = oracle.decode(q, kc, vc, lens, sinks)
    for k in (2, 3, 5):
        S = -(-int(lens[0]) // k)
        o_all, _ = oracle.merge_states(*oracle.chunk_states(q, kc, vc, lens, sinks, S, k,
                                                            sink_chunk=-1))
        o_shift, _, _ = oracle.decode(q, kc, vc, lens, sinks + math.log(k))
        # sinks are fp32, so s + ln k is rounded to ~1e-7 relative before use
        np.testing.assert_allclose(o_all, o_shift, rtol=0, atol=1e-8)
        assert np.max(np.abs(o_all - o_ref)) > 1e-3


def test_empty_request_and_empty_chunk_states():
    q, kc, vc, _, _ = _decode_case(seed=2)
    lens = torch.tensor([0], dtype=torch.int32)
    sinks = torch.tensor([0.75, float("-inf")])
    o, lse, share = oracle.decode(q, kc, vc, lens, sinks)
    assert np.all(o == 0)
    assert lse[0] == pytest.approx(0.75) and share[0] == 1.0
    assert np.isneginf(lse[1]) and share[1] == 0.0
    o_p, m_p, d_p = oracle.chunk_states(q, kc, vc, lens, sinks, 4, 3)
    assert m_p[0, 0] == pytest.approx(0.75) and d_p[0, 0] == 1.0
    assert np.all(np.isneginf(m_p[0, 1:])) and np.all(np.isneginf(m_p[1]))
    o_m, lse_m = oracle.merge_states(o_p, m_p, d_p)
    assert np.all(o_m == 0) and lse_m[0] == pytest.approx(0.75) and np.isneginf(lse_m[1])


# ---------------------------------------------------------------- P7 ------
def test_gqa_equals_mha_with_repeated_kv():
    g = torch.Generator().manual_seed(13)
    Hq, Hkv, D = 8, 2, 16
    q, k, v, cu = _packed_prefill(g, [12, 30], Hq, Hkv, D)
    sinks = torch.empty(Hq).uniform_(-4, 4, generator=g)
    o_gqa, lse_gqa, _ = oracle.prefill(q, k, v, sinks, cu)
    k_rep = k.repeat_interleave(Hq // Hkv, 0).contiguous()
    v_rep = v.repeat_interleave(Hq // Hkv, 0).contiguous()
    o_mha, lse_mha, _ = oracle.prefill(q, k_rep, v_rep, sinks, cu)
    assert np.array_equal(o_gqa, o_mha) and np.array_equal(lse_gqa, lse_mha)


# ---------------------------------------------------------------- P8 ------
def test_decode_is_invariant_to_key_order():
    g = torch.Generator().manual_seed(17)
    B, Hq, Hkv, D, L = 1, 4, 2, 32, 45
    q = _bf16_randn(g, B, Hq, D)
    kc = _bf16_randn(g, B, Hkv, L, D)
    vc = _bf16_randn(g, B, Hkv, L, D)
    sinks = torch.tensor([0.5, -1.0, 3.0, -3.5])
    lens = torch.tensor([L], dtype=torch.int32)
    perm = torch.randperm(L, generator=g)
    o, lse, _ = oracle.decode(q, kc, vc, lens, sinks)
    o_p, lse_p, _ = oracle.decode(q, kc[:, :, perm].contiguous(), vc[:, :, perm].contiguous(),
                                  lens, sinks)
    np.testing.assert_allclose(o_p, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, rtol=1e-14)


def test_prefill_and_decode_agree_on_the_last_row():
    """Decode over a cache equals the last causal row of the same prefill,
    whether the prefill K/V is HND or NHD."""
    g = torch.Generator().manual_seed(23)
    Hq, Hkv, D, L = 4, 2, 64, 40
    q, k, v, cu = _packed_prefill(g, [L], Hq, Hkv, D)
    sinks = torch.tensor([-1.0, 0.0, 2.0, float("-inf")])
    rows = [(L - 1, h) for h in range(Hq)]
    o_p, lse_p, _ = oracle.prefill(q, k, v, sinks, cu, rows=rows)
    o_n, lse_n, _ = oracle.prefill(q, k.transpose(0, 1).contiguous(),
                                   v.transpose(0, 1).contiguous(), sinks, cu, rows=rows,
                                   kv_layout="nhd")
    o_d, lse_d, _ = oracle.decode(q[L - 1:L], k.unsqueeze(0), v.unsqueeze(0),
                                  torch.tensor([L], dtype=torch.int32), sinks)
    assert np.array_equal(o_p, o_d) and np.array_equal(lse_p, lse_d)
    assert np.array_equal(o_p, o_n)


def test_rejects_bad_rows():
    g = torch.Generator().manual_seed(1)
    q, k, v, cu = _packed_prefill(g, [4], 2, 1, 4)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, torch.zeros(2), cu, rows=[(4, 0)])
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, torch.zeros(2), cu, rows=[(0, 2)])


# ------------------------------------------------------- multi-token decode --
def _multi_case(g, lens, q_len, Hq, Hkv, D, max_ctx=None):
    max_ctx = max_ctx or max(lens)
    B = len(lens)
    q = _bf16_randn(g, B, q_len, Hq, D)
    kc = _bf16_randn(g, B, Hkv, max_ctx, D)
    vc = _bf16_randn(g, B, Hkv, max_ctx, D)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("q_len", [2, 3, 4])
def test_multi_token_decode_matches_sdpa_bottom_right_mask(q_len):
    """New token t of a request with L cached tokens (the q_len new ones last)
    equals SDPA over [zero key with the sink as additive mask] + keys
    0..L-q_len+t, the rest masked out."""
    g = torch.Generator().manual_seed(40 + q_len)
    Hq, Hkv, D = 8, 2, 32
    lens = [q_len, 9, 23]
    q, kc, vc, sl = _multi_case(g, lens, q_len, Hq, Hkv, D)
    sinks = torch.empty(Hq).uniform_(-3, 3, generator=g)
    sinks[5] = 20.0
    scale = 1.0 / math.sqrt(D)
    o, _, _ = oracle.decode_multi(q, kc, vc, sl, sinks, scale=scale)
    o = o.reshape(len(lens), q_len, Hq, D)
    r = Hq // Hkv
    for b, L in enumerate(lens):
        ks = torch.cat([torch.zeros(Hkv, 1, D, dtype=kc.dtype), kc[b, :, :L]], 1).repeat_interleave(r, 0)
        vs = torch.cat([torch.zeros(Hkv, 1, D, dtype=vc.dtype), vc[b, :, :L]], 1).repeat_interleave(r, 0)
        mask = torch.zeros(Hq, q_len, L + 1, dtype=torch.float64)
        mask[:, :, 0] = sinks.double()[:, None]
        for t in range(q_len):
            mask[:, t, 1 + (L - q_len + t) + 1:] = float("-inf")
        ref = _sdpa(q[b].transpose(0, 1), ks, vs, causal=False, scale=scale, mask=mask)
        np.testing.assert_allclose(o[b], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def test_multi_token_decode_of_a_whole_sequence_is_causal_prefill():
    """With every cached token new (q_len = L) the rows are those of causal prefill."""
    g = torch.Generator().manual_seed(44)
    Hq, Hkv, D, L = 4, 1, 64, 12
    q, kc, vc, sl = _multi_case(g, [L], L, Hq, Hkv, D)
    sinks = torch.tensor([-2.0, 0.5, float("-inf"), 3.0])
    o_m, lse_m, sh_m = oracle.decode_multi(q, kc, vc, sl, sinks)
    cu = torch.tensor([0, L], dtype=torch.int32)
    o_p, lse_p, sh_p = oracle.prefill(q[0], kc[0], vc[0], sinks, cu, causal=True)
    np.testing.assert_allclose(o_m, o_p, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_m, lse_p, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sh_m, sh_p, rtol=0, atol=1e-13)


def test_multi_token_decode_single_token_is_decode():
    g = torch.Generator().manual_seed(45)
    q, kc, vc, sl = _multi_case(g, [1, 17, 40], 1, 8, 8, 16)
    sinks = torch.empty(8).uniform_(-2, 2, generator=g)
    o_m, lse_m, _ = oracle.decode_multi(q, kc, vc, sl, sinks)
    o_d, lse_d, _ = oracle.decode(q[:, 0], kc, vc, sl, sinks)
    assert np.array_equal(o_m, o_d) and np.array_equal(lse_m, lse_d)


def test_multi_token_decode_ignores_tokens_after_its_position():
    """Changing cached tokens past a new token's position leaves that token's
    output unchanged; changing its own position changes it."""
    g = torch.Generator().manual_seed(46)
    q_len, L = 3, 20
    q, kc, vc, sl = _multi_case(g, [L], q_len, 4, 2, 16, max_ctx=L + 5)
    sinks = torch.zeros(4)
    o0, _, _ = oracle.decode_multi(q, kc, vc, sl, sinks)
    o0 = o0.reshape(q_len, 4, 16)
    for t in range(q_len):
        last = L - q_len + t
        k2, v2 = kc.clone(), vc.clone()
        k2[:, :, last + 1:] = _bf16_randn(g, *k2[:, :, last + 1:].shape)
        v2[:, :, last + 1:] = _bf16_randn(g, *v2[:, :, last + 1:].shape)
        o1, _, _ = oracle.decode_multi(q, k2, v2, sl, sinks)
        assert np.array_equal(o1.reshape(q_len, 4, 16)[t], o0[t])
        k3 = kc.clone()
        k3[:, :, last] = _bf16_randn(g, *k3[:, :, last].shape)
        o3, _, _ = oracle.decode_multi(q, k3, vc, sl, sinks)
        assert not np.allclose(o3.reshape(q_len, 4, 16)[t], o0[t])


def test_multi_token_rows_that_see_no_token_see_only_the_sink():
    g = torch.Generator().manual_seed(47)
    q_len = 4
    q, kc, vc, sl = _multi_case(g, [2], q_len, 2, 1, 8, max_ctx=4)
    sinks = torch.tensor([1.25, float("-inf")])
    o, lse, share = oracle.decode_multi(q, kc, vc, sl, sinks)
    o, lse, share = o.reshape(q_len, 2, 8), lse.reshape(q_len, 2), share.reshape(q_len, 2)
    # tokens t = 0, 1 see 2 - 4 + t + 1 <= 0 cached tokens
    assert np.all(o[:2] == 0.0)
    assert np.all(lse[:2, 0] == 1.25) and np.all(share[:2, 0] == 1.0)
    assert np.all(lse[:2, 1] == -np.inf) and np.all(share[:2, 1] == 0.0)
    assert np.all(np.isfinite(o[2:])) and np.all(share[2:, 0] < 1.0)


# ------------------------------------------------------------ chunked prefill --
def _chunked_case(g, lens_q, lens_k, Hq, Hkv, D):
    cq = torch.zeros(len(lens_q) + 1, dtype=torch.int32)
    cq[1:] = torch.cumsum(torch.tensor(lens_q), 0)
    ck = torch.zeros(len(lens_k) + 1, dtype=torch.int32)
    ck[1:] = torch.cumsum(torch.tensor(lens_k), 0)
    q = _bf16_randn(g, int(cq[-1]), Hq, D)
    k = _bf16_randn(g, Hkv, int(ck[-1]), D)
    v = _bf16_randn(g, Hkv, int(ck[-1]), D)
    return q, k, v, cq, ck


@pytest.mark.parametrize("causal", [True, False])
def test_chunked_prefill_matches_sdpa_bottom_right_mask(causal):
    """Query i of a len_q chunk at the end of len_k keys equals SDPA over
    [zero key with the sink as additive mask] + keys 0..len_k-len_q+i."""
    g = torch.Generator().manual_seed(50 + causal)
    Hq, Hkv, D = 8, 2, 32
    lens_q, lens_k = [5, 1, 17], [5, 40, 33]
    q, k, v, cq, ck = _chunked_case(g, lens_q, lens_k, Hq, Hkv, D)
    sinks = torch.empty(Hq).uniform_(-3, 3, generator=g)
    sinks[2] = 20.0
    scale = 1.0 / math.sqrt(D)
    o, _, _ = oracle.prefill_chunked(q, k, v, sinks, cq, ck, causal=causal, scale=scale)
    o = o.reshape(-1, Hq, D)
    r = Hq // Hkv
    for s_, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        qs = q[int(cq[s_]):int(cq[s_ + 1])].transpose(0, 1)
        kk, vv = k[:, int(ck[s_]):int(ck[s_ + 1])], v[:, int(ck[s_]):int(ck[s_ + 1])]
        ks = torch.cat([torch.zeros(Hkv, 1, D, dtype=k.dtype), kk], 1).repeat_interleave(r, 0)
        vs = torch.cat([torch.zeros(Hkv, 1, D, dtype=v.dtype), vv], 1).repeat_interleave(r, 0)
        mask = torch.zeros(Hq, lq, lk + 1, dtype=torch.float64)
        mask[:, :, 0] = sinks.double()[:, None]
        if causal:
            for i in range(lq):
                mask[:, i, 1 + (lk - lq + i) + 1:] = float("-inf")
        ref = _sdpa(qs, ks, vs, causal=False, scale=scale, mask=mask).transpose(0, 1)
        np.testing.assert_allclose(o[int(cq[s_]):int(cq[s_ + 1])], ref.numpy(), rtol=0, atol=1e-12)


def test_chunked_prefill_of_a_split_sequence_equals_one_prefill():
    """Prefill of a sequence cut into chunks (each chunk against all keys up to
    its end) gives exactly the rows of one causal prefill of the whole."""
    g = torch.Generator().manual_seed(52)
    Hq, Hkv, D, L = 4, 2, 64, 50
    q, k, v, cu = _packed_prefill(g, [L], Hq, Hkv, D)
    sinks = torch.tensor([0.5, -1.0, float("-inf"), 3.0])
    o_full, lse_full, _ = oracle.prefill(q, k, v, sinks, cu)
    cuts = [0, 13, 14, 37, L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        cq = torch.tensor([0, b - a], dtype=torch.int32)
        ck = torch.tensor([0, b], dtype=torch.int32)
        o_c, lse_c, _ = oracle.prefill_chunked(q[a:b], k[:, :b], v[:, :b], sinks, cq, ck)
        assert np.array_equal(o_c, o_full[a * Hq:b * Hq]) and np.array_equal(lse_c, lse_full[a * Hq:b * Hq])


def test_chunked_prefill_with_equal_lengths_is_prefill_and_single_query_is_decode():
    g = torch.Generator().manual_seed(53)
    Hq, Hkv, D = 8, 8, 16
    q, k, v, cq, ck = _chunked_case(g, [7, 12], [7, 12], Hq, Hkv, D)
    sinks = torch.empty(Hq).uniform_(-2, 2, generator=g)
    for causal in (True, False):
        o_c, lse_c, _ = oracle.prefill_chunked(q, k, v, sinks, cq, ck, causal=causal)
        o_p, lse_p, _ = oracle.prefill(q, k, v, sinks, cq, causal=causal)
        assert np.array_equal(o_c, o_p) and np.array_equal(lse_c, lse_p)
    # one query at the end of 30 keys: the decode of that query over the 30 keys
    q1, k1, v1, cq1, ck1 = _chunked_case(g, [1], [30], Hq, Hkv, D)
    o_c, lse_c, _ = oracle.prefill_chunked(q1, k1, v1, sinks, cq1, ck1)
    o_d, lse_d, _ = oracle.decode(q1, k1.unsqueeze(0), v1.unsqueeze(0),
                                  torch.tensor([30], dtype=torch.int32), sinks)
    np.testing.assert_allclose(o_c, o_d, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse_c, lse_d, rtol=0, atol=1e-14)


def test_chunked_prefill_rejects_a_chunk_longer_than_its_keys():
    g = torch.Generator().manual_seed(54)
    q, k, v, cq, ck = _chunked_case(g, [6], [5], 2, 1, 8)
    with pytest.raises(ValueError):
        oracle.prefill_chunked(q, k, v, torch.zeros(2), cq, ck)


# ------------------------------------------------------------- KV-cache append --
def _append_case(g, counts, pos, B, Hkv, D, max_ctx):
    cu = torch.zeros(len(counts) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(counts), 0)
    T = int(cu[-1])
    kn, vn = _bf16_randn(g, T, Hkv, D), _bf16_randn(g, T, Hkv, D)
    kc, vc = _bf16_randn(g, B, Hkv, max_ctx, D), _bf16_randn(g, B, Hkv, max_ctx, D)
    return kn, vn, cu, torch.tensor(pos, dtype=torch.int32), kc, vc


def test_kv_append_element_by_element():
    """Against a loop over every element, and every unwritten slot unchanged;
    tokens that would land past the cache end are dropped."""
    g = torch.Generator().manual_seed(60)
    B, Hkv, D, max_ctx = 3, 2, 8, 12
    counts, pos = [3, 0, 5], [0, 4, 9]          # request 2: slots 9..13, the last two dropped
    kn, vn, cu, cp, kc, vc = _append_case(g, counts, pos, B, Hkv, D, max_ctx)
    ko, vo = oracle.kv_append(kn, vn, cu, cp, kc, vc)
    written = set()
    for b in range(B):
        for t in range(counts[b]):
            j = pos[b] + t
            if j >= max_ctx:
                continue
            written.add((b, j))
            for h in range(Hkv):
                for d in range(D):
                    assert ko[b, h, j, d].item() == kn[int(cu[b]) + t, h, d].item()
                    assert vo[b, h, j, d].item() == vn[int(cu[b]) + t, h, d].item()
    for b in range(B):
        for j in range(max_ctx):
            if (b, j) not in written:
                assert torch.equal(ko[b, :, j].view(torch.int16), kc[b, :, j].view(torch.int16))
                assert torch.equal(vo[b, :, j].view(torch.int16), vc[b, :, j].view(torch.int16))


def test_kv_append_then_decode_equals_prefill_last_row():
    """Prefill K/V appended in two pieces into an empty cache: decode over that
    cache equals the last causal prefill row."""
    g = torch.Generator().manual_seed(61)
    Hq, Hkv, D, L = 4, 2, 32, 21
    q, k, v, cu = _packed_prefill(g, [L], Hq, Hkv, D)
    sinks = torch.tensor([0.3, -1.0, 2.0, float("-inf")])
    kc = torch.zeros(1, Hkv, 32, D, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kn, vn = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()   # token-major
    kc, vc = oracle.kv_append(kn[:13], vn[:13], torch.tensor([0, 13], dtype=torch.int32),
                              torch.tensor([0], dtype=torch.int32), kc, vc)
    kc, vc = oracle.kv_append(kn[13:], vn[13:], torch.tensor([0, L - 13], dtype=torch.int32),
                              torch.tensor([13], dtype=torch.int32), kc, vc)
    o_d, lse_d, _ = oracle.decode(q[L - 1:L], kc, vc, torch.tensor([L], dtype=torch.int32), sinks)
    o_p, lse_p, _ = oracle.prefill(q, k, v, sinks, cu, rows=[(L - 1, h) for h in range(Hq)])
    assert np.array_equal(o_d, o_p) and np.array_equal(lse_d, lse_p)


# ------------------------------------------------------------ FP8 KV cache --
# Pins for the FP8 cache extension: the E4M3 table against torch's
# float8_e4m3fn (a library routine) and against values fixed by the format;
# the encoder's rounding, ties and saturation; the quantizer against torch's
# conversion of the float32 product; the FP8 decode against the (separately
# pinned) bf16 oracle where the dequantized cache is exact in bf16.

def test_e4m3_table_matches_torch_float8_e4m3fn():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.E4M3_TABLE
    assert np.array_equal(np.isnan(t), np.isnan(ours))
    fin = ~np.isnan(t)
    assert np.array_equal(t[fin], ours[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(ours[fin]))


def test_e4m3_values_fixed_by_the_format():
    v = oracle.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0           # largest finite
    assert v(0x08) == 2.0 ** -6                             # smallest normal
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals
    assert v(0x38) == 1.0 and v(0x39) == 1.125 and v(0xC0) == -2.0
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert not any(math.isinf(v(c)) for c in range(256))


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    back = oracle.e4m3_encode(oracle.E4M3_TABLE[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def test_e4m3_encode_rounding_ties_and_saturation():
    cases = {
        1.0625: 0x38,              # halfway 1.0 | 1.125: even mantissa (1.0)
        1.1875: 0x3A,              # halfway 1.125 | 1.25: even mantissa (1.25)
        1.05: 0x38, 1.1: 0x39,     # nearest
        2.0 ** -10: 0x00,          # halfway 0 | 2^-9: to +0
        -(2.0 ** -10): 0x80,       # ... to -0
        3 * 2.0 ** -10: 0x02,      # halfway 2^-9 | 2^-8: even (2^-8)
        2.0 ** -12: 0x00,
        440.0: 0x7E, 449.0: 0x7E, 464.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE,   # saturate
        float("inf"): 0x7E, float("-inf"): 0xFE,
    }
    got = oracle.e4m3_encode(np.array(list(cases), np.float32))
    assert [int(c) for c in got] == list(cases.values())
    assert int(oracle.e4m3_encode([float("nan")])[0]) == 0x7F


def test_e4m3_encode_matches_torch_on_in_range_values():
    rng = np.random.default_rng(70)
    x = np.concatenate([rng.normal(0, 30, 20000), rng.normal(0, 0.01, 5000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_quantize_is_the_float32_product_with_the_reciprocal():
    rng = np.random.default_rng(71)
    x = (rng.normal(0, 1, 20000) * rng.choice([0.1, 1, 10], 20000)).astype(np.float32)
    for s in (0.0123, 1.0 / 3.0, 0.5, 2.5e-3):
        inv = np.float32(1.0) / np.float32(s)
        prod = torch.from_numpy(x * inv).clamp(-448, 448)
        ref = prod.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.fp8_quantize(x, s), ref)


def test_kv_append_fp8_places_quantized_rows():
    g = torch.Generator().manual_seed(72)
    B, Hkv, D, max_ctx = 3, 2, 16, 12
    counts, pos = [3, 0, 5], [0, 4, 9]
    kn, vn, cu, cp, _, _ = _append_case(g, counts, pos, B, Hkv, D, max_ctx)
    kc = torch.randint(0, 256, (B, Hkv, max_ctx, D), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, Hkv, max_ctx, D), generator=g, dtype=torch.uint8)
    ks, vs = np.float32([0.01, 0.003]), np.float32([0.02, 0.5])
    ko, vo = oracle.kv_append_fp8(kn, vn, cu, cp, kc, vc, ks, vs)
    written = set()
    for b in range(B):
        for t in range(counts[b]):
            j = pos[b] + t
            if j >= max_ctx:
                continue
            written.add((b, j))
            for h in range(Hkv):
                row_k = kn[int(cu[b]) + t, h].float().numpy()
                row_v = vn[int(cu[b]) + t, h].float().numpy()
                ref_k = torch.from_numpy((row_k * (np.float32(1) / ks[h])).clip(-448, 448))
                ref_v = torch.from_numpy((row_v * (np.float32(1) / vs[h])).clip(-448, 448))
                assert torch.equal(ko[b, h, j], ref_k.to(torch.float8_e4m3fn).view(torch.uint8))
                assert torch.equal(vo[b, h, j], ref_v.to(torch.float8_e4m3fn).view(torch.uint8))
    for b in range(B):
        for j in range(max_ctx):
            if (b, j) not in written:
                assert torch.equal(ko[b, :, j], kc[b, :, j]) and torch.equal(vo[b, :, j], vc[b, :, j])


def _fp8_decode_case(g, lens, q_len, Hq, Hkv, D, max_ctx):
    B = len(lens)
    q = _bf16_randn(g, B, q_len, Hq, D)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    kc = finite[torch.randint(0, 254, (B, Hkv, max_ctx, D), generator=g)]
    vc = finite[torch.randint(0, 254, (B, Hkv, max_ctx, D), generator=g)]
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32)


def test_decode_fp8_equals_bf16_oracle_for_power_of_two_scales():
    """With power-of-two scales every dequantized value is exact in bf16, so
    the FP8 decode must equal the bf16 oracle run on that cache."""
    g = torch.Generator().manual_seed(73)
    lens, q_len, Hq, Hkv, D, max_ctx = [0, 1, 5, 40, 70], 3, 8, 2, 16, 72
    q, kc, vc, sl = _fp8_decode_case(g, lens, q_len, Hq, Hkv, D, max_ctx)
    ks, vs = np.float32([2.0 ** -7, 2.0 ** -5]), np.float32([2.0 ** -6, 2.0 ** -8])
    sinks = torch.tensor([0.5, float("-inf"), 2.0, -1.0, 20.0, 0.0, 1.0, -3.0])
    kd, vd = oracle.dequantize_fp8(kc, ks), oracle.dequantize_fp8(vc, vs)
    kb, vb = torch.from_numpy(kd).to(torch.bfloat16), torch.from_numpy(vd).to(torch.bfloat16)
    assert np.array_equal(kb.double().numpy(), kd) and np.array_equal(vb.double().numpy(), vd)
    o8, l8, s8 = oracle.decode_multi_fp8(q, kc, vc, ks, vs, sl, sinks)
    ob, lb, sb = oracle.decode_multi(q, kb, vb, sl, sinks)
    np.testing.assert_allclose(o8, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l8, lb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s8, sb, rtol=1e-12, atol=1e-12)


def test_decode_fp8_scales_act_as_factors():
    """k_scale multiplies every logit (the same as scaling the softmax scale);
    v_scale multiplies the output."""
    g = torch.Generator().manual_seed(74)
    lens, Hq, Hkv, D = [9, 33], 4, 2, 16
    q, kc, vc, sl = _fp8_decode_case(g, lens, 1, Hq, Hkv, D, 40)
    sinks = torch.tensor([0.3, -1.0, 4.0, float("-inf")])
    ks, vs = np.float32([0.01, 0.02]), np.float32([0.1, 0.3])
    o1, l1, _ = oracle.decode_multi_fp8(q, kc, vc, ks, vs, sl, sinks, scale=0.25)
    o2, l2, _ = oracle.decode_multi_fp8(q, kc, vc, ks * 2, vs, sl, sinks, scale=0.125)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
    o3, _, _ = oracle.decode_multi_fp8(q, kc, vc, ks, vs * 4, sl, sinks, scale=0.25)
    np.testing.assert_allclose(o3, 4 * o1, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- paged KV cache --
# Pins for the paged cache: pages scattered by a hand-written loop under a
# random table and gathered back must give the logical cache bit for bit, and
# every paged function must equal its (separately pinned) contiguous form.

def _scatter_pages(logical, P, num_pages, g):
    """Scatter logical caches [B, Hkv, L, D] into num_pages pages of P slots by
    a random permutation; returns (pages, block_tables)."""
    B, Hkv, L, D = logical.shape
    per = -(-L // P)
    perm = torch.randperm(num_pages, generator=g)[:B * per].view(B, per).to(torch.int32)
    pages = torch.zeros((num_pages, Hkv, P, D), dtype=logical.dtype)
    for b in range(B):
        for j in range(L):
            pages[int(perm[b, j // P]), :, j % P] = logical[b, :, j]
    return pages, perm


def test_gather_pages_inverts_a_random_scatter():
    g = torch.Generator().manual_seed(80)
    logical = _bf16_randn(g, 3, 2, 45, 8)
    for P in (1, 4, 16, 64):
        pages, bt = _scatter_pages(logical, P, 3 * (-(-45 // P)) + 5, g)
        back = oracle.gather_pages(pages, bt, P, 45)
        assert torch.equal(back.view(torch.int16), logical.view(torch.int16))


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_paged_equals_contiguous(fp8):
    g = torch.Generator().manual_seed(81 + fp8)
    lens, q_len, Hq, Hkv, D, L = [0, 1, 15, 16, 17, 40], 2, 8, 2, 16, 48
    B = len(lens)
    q = _bf16_randn(g, B, q_len, Hq, D)
    if fp8:
        finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
        kl = finite[torch.randint(0, 254, (B, Hkv, L, D), generator=g)]
        vl = finite[torch.randint(0, 254, (B, Hkv, L, D), generator=g)]
        scales = dict(k_scale=np.float32([0.01, 0.02]), v_scale=np.float32([0.03, 0.005]))
    else:
        kl, vl = _bf16_randn(g, B, Hkv, L, D), _bf16_randn(g, B, Hkv, L, D)
        scales = {}
    sinks = torch.tensor([0.5, float("-inf"), 2.0, -1.0, 20.0, 0.0, 1.0, -3.0])
    sl = torch.tensor(lens, dtype=torch.int32)
    P = 16
    kp, bt = _scatter_pages(kl, P, 40, g)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for j in range(L):
            vp[int(bt[b, j // P]), :, j % P] = vl[b, :, j]
    o_p, l_p, _ = oracle.decode_multi_paged(q, kp, vp, bt, P, sl, sinks, **scales)
    if fp8:
        o_c, l_c, _ = oracle.decode_multi_fp8(q, kl, vl, scales["k_scale"], scales["v_scale"], sl, sinks)
    else:
        o_c, l_c, _ = oracle.decode_multi(q, kl, vl, sl, sinks)
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


def test_decode_paged_with_shared_prefix_pages():
    """Two requests whose tables share their first page (a shared prefix) equal
    contiguous caches holding copies of it."""
    g = torch.Generator().manual_seed(83)
    Hq, Hkv, D, P = 4, 1, 8, 4
    pages = _bf16_randn(g, 6, Hkv, P, D)
    bt = torch.tensor([[0, 1, 2], [0, 3, 4]], dtype=torch.int32)
    sl = torch.tensor([10, 12], dtype=torch.int32)
    logical = torch.stack([torch.cat([pages[int(p)] for p in bt[b]], dim=1) for b in range(2)])
    q = _bf16_randn(g, 2, 1, Hq, D)
    sinks = torch.tensor([0.0, 1.0, -1.0, float("-inf")])
    o_p, _, _ = oracle.decode_multi_paged(q, pages, pages, bt, P, sl, sinks)
    o_c, _, _ = oracle.decode_multi(q, logical, logical, sl, sinks)
    assert np.array_equal(o_p, o_c)


@pytest.mark.parametrize("fp8", [False, True])
def test_kv_append_paged_equals_contiguous_append(fp8):
    """Append into pages then gather equals the contiguous append into the
    logical cache; slots past the table's capacity are dropped."""
    g = torch.Generator().manual_seed(84 + fp8)
    B, Hkv, D, P, width = 3, 2, 16, 8, 3           # capacity 24 slots per request
    counts, pos = [5, 0, 9], [3, 7, 20]            # request 2: slots 20..28, 24.. dropped
    kn, vn, cu, cp, _, _ = _append_case(g, counts, pos, B, Hkv, D, width * P)
    num_pages = 12
    bt = torch.randperm(num_pages, generator=g)[:B * width].view(B, width).to(torch.int32)
    if fp8:
        kp = torch.randint(0, 256, (num_pages, Hkv, P, D), generator=g, dtype=torch.uint8)
        vp = torch.randint(0, 256, (num_pages, Hkv, P, D), generator=g, dtype=torch.uint8)
        ks, vs = np.float32([0.01, 0.03]), np.float32([0.02, 0.004])
        kp2, vp2 = oracle.kv_append_paged(kn, vn, cu, cp, kp, vp, bt, P, k_scale=ks, v_scale=vs)
    else:
        kp, vp = _bf16_randn(g, num_pages, Hkv, P, D), _bf16_randn(g, num_pages, Hkv, P, D)
        kp2, vp2 = oracle.kv_append_paged(kn, vn, cu, cp, kp, vp, bt, P)
    kl = oracle.gather_pages(kp, bt, P, width * P)
    vl = oracle.gather_pages(vp, bt, P, width * P)
    if fp8:
        kl2, vl2 = oracle.kv_append_fp8(kn, vn, cu, cp, kl, vl, ks, vs)
    else:
        kl2, vl2 = oracle.kv_append(kn, vn, cu, cp, kl, vl)
    same = (lambda a, b: torch.equal(a, b)) if fp8 else \
        (lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16)))
    assert same(oracle.gather_pages(kp2, bt, P, width * P), kl2)
    assert same(oracle.gather_pages(vp2, bt, P, width * P), vl2)
    used = set(int(x) for x in bt.flatten())
    for p in range(num_pages):                     # pages outside every table: untouched
        if p not in used:
            assert same(kp2[p], kp[p]) and same(vp2[p], vp[p])
