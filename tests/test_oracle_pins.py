"""Pins of the fp64 CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against mathematics or the pages:

* central finite differences of l = sum(dO * O) (backward vs forward),
* an independent library routine (torch CPU scaled_dot_product_attention in
  float64, the routine [TE-3333]'s and [TE-3216]'s references call; for the
  bottom-right causal triangle, with torch's own lower-right causal bias),
* hand-derived closed forms (one key, two keys, identical keys, causal row 0),
* invariants (softmax rows sum to one, GQA == summed MHA over repeated KV,
  padding rows inert and exactly zero),
* values printed on the pages (golden fixtures under tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import workloads
from oracle import attn_bwd, attn_fwd, attn_fwd_seq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(t):
    return t.to(torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def run_case(c, mode="definition"):
    args = (c.cu_seqlens_q, c.cu_seqlens_kv, c.cu_seqlens_q_padded, c.cu_seqlens_kv_padded)
    o, l = attn_fwd(f64(c.q), f64(c.k), f64(c.v), *args, scale=c.scale, causal=c.causal)
    g = attn_bwd(f64(c.q), f64(c.k), f64(c.v), f64(c.dout), *args, scale=c.scale,
                 causal=c.causal, out=o, lse=l, mode=mode)
    return o, l, g


def small_case(rng, lq, lk, pq, pk, hq, hkv, d, causal, scale=None):
    """Random fp64 case with padding rows (filled with noise)."""
    Tq, Tk = sum(pq), sum(pk)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    return dict(q=rng.standard_normal((Tq, hq, d)), k=rng.standard_normal((Tk, hkv, d)),
                v=rng.standard_normal((Tk, hkv, d)), dout=rng.standard_normal((Tq, hq, d)),
                cu_q=cu(lq), cu_kv=cu(lk), cu_qp=cu(pq), cu_kp=cu(pk),
                scale=scale if scale is not None else 1 / math.sqrt(d), causal=causal)


def fwd_of(c, q=None, k=None, v=None):
    return attn_fwd(c["q"] if q is None else q, c["k"] if k is None else k,
                    c["v"] if v is None else v, c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"],
                    scale=c["scale"], causal=c["causal"])


def bwd_of(c):
    return attn_bwd(c["q"], c["k"], c["v"], c["dout"], c["cu_q"], c["cu_kv"], c["cu_qp"],
                    c["cu_kp"], scale=c["scale"], causal=c["causal"])


# ---------------------------------------------------------------- finite differences
def _fd_check(c, eps=1e-6):
    """Analytic gradient vs central differences of l = sum(dO*O), every element."""
    grads = dict(zip("qkv", bwd_of(c)))
    for name in "qkv":
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            lp = np.sum(c["dout"] * fwd_of(c, **{name: xp})[0])
            lm = np.sum(c["dout"] * fwd_of(c, **{name: xm})[0])
            num[idx] = (lp - lm) / (2 * eps)
        an = grads[name]
        err = np.linalg.norm(an - num) / max(np.linalg.norm(num), 1e-30)
        assert err <= 1e-7, (name, err)
        # padding rows: perturbing them changes l by exactly zero
        zero_rows = np.all(num == 0.0, axis=(1, 2))
        assert np.all(an[zero_rows] == 0.0)


@pytest.mark.parametrize("call", [0, 1])
def test_finite_differences_tiny_gqa_calls(call):
    """The TE-2448 two-call shapes (T=12, hq=2, hkv=1, d=8, padding mask, scale 0.1)."""
    case = workloads.tiny_gqa_two_calls()[call]
    c = dict(q=f64(case.q), k=f64(case.k), v=f64(case.v), dout=f64(case.dout),
             cu_q=case.cu_seqlens_q, cu_kv=case.cu_seqlens_kv, cu_qp=case.cu_seqlens_q_padded,
             cu_kp=case.cu_seqlens_kv_padded, scale=case.scale, causal=case.causal)
    _fd_check(c)


def test_finite_differences_causal_gqa_with_padding():
    rng = np.random.default_rng(7)
    c = small_case(rng, lq=[3, 5], lk=[3, 5], pq=[4, 6], pk=[4, 6], hq=4, hkv=2, d=8, causal=True)
    _fd_check(c)


def test_finite_differences_causal_lq_ne_lk():
    """Top-left causal with Lq != Lk (a reading; the pages only use Lq == Lk with causal)."""
    rng = np.random.default_rng(8)
    c = small_case(rng, lq=[2, 4], lk=[5, 3], pq=[3, 4], pk=[6, 4], hq=2, hkv=1, d=8, causal=True)
    _fd_check(c)


# ---------------------------------------------------------------- library cross-check
def _sdpa_ref(c):
    """torch CPU fp64 SDPA per sequence (+ autograd), placed in the padded layout."""
    q = torch.tensor(c["q"], requires_grad=True)
    k = torch.tensor(c["k"], requires_grad=True)
    v = torch.tensor(c["v"], requires_grad=True)
    out = torch.zeros_like(q)
    outs = []
    for b in range(len(c["cu_q"]) - 1):
        oq, lq = int(c["cu_qp"][b]), int(c["cu_q"][b + 1] - c["cu_q"][b])
        ok, lk = int(c["cu_kp"][b]), int(c["cu_kv"][b + 1] - c["cu_kv"][b])
        if lq == 0 or lk == 0:
            continue
        qi = q[oq:oq + lq].transpose(0, 1)[None]
        ki = k[ok:ok + lk].transpose(0, 1)[None]
        vi = v[ok:ok + lk].transpose(0, 1)[None]
        if c["causal"] == "bottom_right":
            kw = dict(attn_mask=causal_lower_right(lq, lk))
        else:
            kw = dict(is_causal=bool(c["causal"]))
        o = F.scaled_dot_product_attention(qi, ki, vi, scale=c["scale"], enable_gqa=True, **kw)
        outs.append((oq, lq, o[0].transpose(0, 1)))
    for oq, lq, o in outs:
        out = out.index_put((torch.arange(oq, oq + lq),), o)
    (out * torch.tensor(c["dout"])).sum().backward()
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(lq=[5, 0, 7], lk=[6, 4, 7], pq=[8, 2, 8], pk=[8, 4, 9], hq=6, hkv=2, d=16),
    dict(lq=[17], lk=[17], pq=[20], pk=[20], hq=4, hkv=4, d=32),
    dict(lq=[9, 12], lk=[4, 12], pq=[9, 16], pk=[4, 13], hq=8, hkv=1, d=8),
])
def test_matches_torch_sdpa_fp64(shape, causal):
    rng = np.random.default_rng(11)
    c = small_case(rng, causal=causal, **shape)
    o, l = fwd_of(c)
    dq, dk, dv = bwd_of(c)
    ro, rdq, rdk, rdv = _sdpa_ref(c)
    for a, b in [(o, ro), (dq, rdq), (dk, rdk), (dv, rdv)]:
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


BR_SHAPES = [
    dict(lq=[5, 0, 3], lk=[6, 4, 7], pq=[8, 2, 3], pk=[8, 4, 9], hq=6, hkv=2, d=16),
    dict(lq=[17, 1], lk=[17, 9], pq=[20, 1], pk=[20, 9], hq=4, hkv=4, d=32),
]


@pytest.mark.parametrize("shape", BR_SHAPES)
def test_bottom_right_matches_torch_lower_right_bias(shape):
    """Bottom-right causal (Lq <= Lk) against torch's lower-right causal bias."""
    rng = np.random.default_rng(12)
    c = small_case(rng, causal="bottom_right", **shape)
    o, l = fwd_of(c)
    dq, dk, dv = bwd_of(c)
    ro, rdq, rdk, rdv = _sdpa_ref(c)
    for a, b in [(o, ro), (dq, rdq), (dk, rdk), (dv, rdv)]:
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_bottom_right_equals_top_left_when_lengths_match():
    rng = np.random.default_rng(13)
    c = small_case(rng, lq=[6, 9, 1], lk=[6, 9, 1], pq=[7, 9, 2], pk=[7, 9, 2], hq=4, hkv=2,
                   d=8, causal=True)
    br = dict(c, causal="bottom_right")
    for a, b in zip(fwd_of(c) + bwd_of(c), fwd_of(br) + bwd_of(br)):
        np.testing.assert_array_equal(a, b)


def test_bottom_right_short_queries_are_the_tail_of_a_square_problem():
    """Lq < Lk: the Lq queries behave as the last Lq rows of a top-left causal
    problem over all Lk keys (the earlier rows given dO = 0 add nothing to dK, dV)."""
    rng = np.random.default_rng(14)
    lq, lk, hq, hkv, d = 4, 11, 4, 2, 8
    q, dout = rng.standard_normal((lq, hq, d)), rng.standard_normal((lq, hq, d))
    k, v = rng.standard_normal((lk, hkv, d)), rng.standard_normal((lk, hkv, d))
    qs = np.concatenate([rng.standard_normal((lk - lq, hq, d)), q])
    dos = np.concatenate([np.zeros((lk - lq, hq, d)), dout])
    cq, ck = np.array([0, lq], np.int32), np.array([0, lk], np.int32)
    o, l = attn_fwd(q, k, v, cq, ck, scale=0.4, causal="bottom_right")
    g = attn_bwd(q, k, v, dout, cq, ck, scale=0.4, causal="bottom_right")
    o2, l2 = attn_fwd(qs, k, v, ck, ck, scale=0.4, causal=True)
    g2 = attn_bwd(qs, k, v, dos, ck, ck, scale=0.4, causal=True)
    np.testing.assert_allclose(o, o2[lk - lq:], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l, l2[lk - lq:], rtol=1e-13)
    np.testing.assert_allclose(g[0], g2[0][lk - lq:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[1], g2[1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[2], g2[2], rtol=1e-12, atol=1e-14)


def test_bottom_right_long_queries_lead_with_empty_rows():
    """Lq > Lk: the first Lq - Lk queries see no key (O = 0, LSE = -inf, dQ = 0);
    the last Lk queries form a top-left causal problem over the Lk keys."""
    rng = np.random.default_rng(15)
    lq, lk, hq, hkv, d = 10, 4, 2, 1, 8
    q, dout = rng.standard_normal((lq, hq, d)), rng.standard_normal((lq, hq, d))
    k, v = rng.standard_normal((lk, hkv, d)), rng.standard_normal((lk, hkv, d))
    cq, ck = np.array([0, lq], np.int32), np.array([0, lk], np.int32)
    o, l = attn_fwd(q, k, v, cq, ck, scale=0.4, causal="bottom_right")
    dq, dk, dv = attn_bwd(q, k, v, dout, cq, ck, scale=0.4, causal="bottom_right")
    e = lq - lk
    assert np.all(o[:e] == 0) and np.all(np.isneginf(l[:e])) and np.all(dq[:e] == 0)
    o2, l2 = attn_fwd(q[e:], k, v, ck, ck, scale=0.4, causal=True)
    dq2, dk2, dv2 = attn_bwd(q[e:], k, v, dout[e:], ck, ck, scale=0.4, causal=True)
    np.testing.assert_allclose(o[e:], o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l[e:], l2, rtol=1e-13)
    for a, b in [(dq[e:], dq2), (dk, dk2), (dv, dv2)]:
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # the formula mode (saved statistics with -inf rows) agrees with the definition
    gf = attn_bwd(q, k, v, dout, cq, ck, scale=0.4, causal="bottom_right", out=o, lse=l,
                  mode="formula")
    for a, b in zip((dq, dk, dv), gf):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_finite_differences_bottom_right_both_directions():
    rng = np.random.default_rng(16)
    c = small_case(rng, lq=[2, 5], lk=[5, 3], pq=[3, 5], pk=[6, 4], hq=2, hkv=1, d=8,
                   causal="bottom_right")
    _fd_check(c)


def test_unknown_alignment_is_rejected():
    with pytest.raises(ValueError):
        attn_fwd_seq(np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), 1.0,
                     "top_right")


# ---------------------------------------------------------------- closed forms
def test_single_token_sequence():
    """Lq = Lk = 1: O = v, LSE = scale*q.k, dQ = dK = 0, dV = dO."""
    rng = np.random.default_rng(1)
    c = small_case(rng, lq=[1], lk=[1], pq=[1], pk=[1], hq=2, hkv=1, d=8, causal=False, scale=0.37)
    o, l = fwd_of(c)
    dq, dk, dv = bwd_of(c)
    for h in range(2):
        np.testing.assert_array_equal(o[0, h], c["v"][0, 0])
        assert l[0, h] == pytest.approx(0.37 * c["q"][0, h] @ c["k"][0, 0], rel=1e-15)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0], c["dout"][0, 0] + c["dout"][0, 1], rtol=1e-15)


def test_two_keys_closed_form():
    """One query, two keys: O = s*v0 + (1-s)*v1 with s = sigmoid(scale*q.(k0-k1)).

    Gradients by hand: with w = s(1-s) dO.(v0-v1),
    dq = scale*w*(k0-k1), dk0 = scale*w*q = -dk1, dv0 = s*dO, dv1 = (1-s)*dO.
    """
    rng = np.random.default_rng(2)
    d, sc = 8, 0.7
    c = small_case(rng, lq=[1], lk=[2], pq=[1], pk=[2], hq=1, hkv=1, d=d, causal=False, scale=sc)
    q, k0, k1 = c["q"][0, 0], c["k"][0, 0], c["k"][1, 0]
    v0, v1, do = c["v"][0, 0], c["v"][1, 0], c["dout"][0, 0]
    a = sc * q @ (k0 - k1)
    s = 1 / (1 + math.exp(-a))
    o, l = fwd_of(c)
    np.testing.assert_allclose(o[0, 0], s * v0 + (1 - s) * v1, rtol=1e-13)
    np.testing.assert_allclose(l[0, 0], math.log(math.exp(sc * q @ k0) + math.exp(sc * q @ k1)),
                               rtol=1e-13)
    dq, dk, dv = bwd_of(c)
    w = s * (1 - s) * do @ (v0 - v1)
    np.testing.assert_allclose(dq[0, 0], sc * w * (k0 - k1), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], sc * w * q, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[1, 0], -sc * w * q, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], s * do, rtol=1e-13)
    np.testing.assert_allclose(dv[1, 0], (1 - s) * do, rtol=1e-13)


def test_identical_keys_give_mean_of_values():
    """All keys equal: P is uniform over the allowed keys, O = their mean,
    LSE = scale*q.k + ln(#allowed)."""
    rng = np.random.default_rng(3)
    L, d = 6, 8
    q = rng.standard_normal((L, 1, d))
    krow = rng.standard_normal(d)
    k = np.tile(krow, (L, 1, 1))
    v = rng.standard_normal((L, 1, d))
    for causal in (False, True):
        o, l = attn_fwd_seq(q, k, v, 0.5, causal)
        for i in range(L):
            n = i + 1 if causal else L
            np.testing.assert_allclose(o[i, 0], v[:n, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
            assert l[i, 0] == pytest.approx(0.5 * q[i, 0] @ krow + math.log(n), rel=1e-12)


def test_causal_first_row_sees_only_first_key():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((5, 2, 8)) for _ in range(3))
    o, l = attn_fwd_seq(q, k, v, 0.3, True)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(l[0], 0.3 * np.sum(q[0] * k[0], axis=-1), rtol=1e-15)


def test_softmax_rows_sum_to_one():
    """With one-hot value rows, O_i is row i of P: it sums to 1 and is 0 off the allowed set."""
    rng = np.random.default_rng(5)
    L = 7
    q = rng.standard_normal((L, 1, L))
    k = rng.standard_normal((L, 1, L))
    v = np.eye(L)[:, None, :]
    for causal in (False, True):
        p, _ = attn_fwd_seq(q, k, v, 1.3, causal)
        p = p[:, 0, :]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        if causal:
            assert np.all(p[np.triu_indices(L, 1)] == 0.0)
        assert np.all(p >= 0)


# ---------------------------------------------------------------- invariants
def test_gqa_equals_summed_mha_over_repeated_kv():
    """[TE-3216] repeat_interleave: GQA dK/dV of a group == sum over its heads of MHA."""
    rng = np.random.default_rng(6)
    c = small_case(rng, lq=[6, 9], lk=[6, 9], pq=[7, 9], pk=[7, 9], hq=6, hkv=2, d=8, causal=True)
    G = 3
    o, l = fwd_of(c)
    dq, dk, dv = bwd_of(c)
    kr, vr = np.repeat(c["k"], G, axis=1), np.repeat(c["v"], G, axis=1)
    o2, l2 = fwd_of(c, k=kr, v=vr)
    c2 = dict(c, k=kr, v=vr)
    dq2, dk2, dv2 = bwd_of(c2)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk, dk2.reshape(dk2.shape[0], 2, G, -1).sum(axis=2), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(dv2.shape[0], 2, G, -1).sum(axis=2), rtol=1e-12,
                               atol=1e-14)


def test_padding_rows_exact_zero_and_inert():
    """Rows outside the real ranges are exactly 0 (lse -inf); redrawing them changes nothing."""
    rng = np.random.default_rng(9)
    c = small_case(rng, lq=[3, 0, 5], lk=[4, 2, 5], pq=[5, 3, 8], pk=[6, 2, 7], hq=4, hkv=2, d=8,
                   causal=False)
    o, l = fwd_of(c)
    dq, dk, dv = bwd_of(c)
    real_q = np.zeros(o.shape[0], bool)
    real_k = np.zeros(dk.shape[0], bool)
    for b in range(3):
        real_q[c["cu_qp"][b]:c["cu_qp"][b] + c["cu_q"][b + 1] - c["cu_q"][b]] = True
        if c["cu_q"][b + 1] > c["cu_q"][b]:
            real_k[c["cu_kp"][b]:c["cu_kp"][b] + c["cu_kv"][b + 1] - c["cu_kv"][b]] = True
    assert np.all(o[~real_q] == 0) and np.all(np.isneginf(l[~real_q]))
    assert np.all(dq[~real_q] == 0)
    assert np.all(dk[~real_k] == 0) and np.all(dv[~real_k] == 0)
    # redraw all padding rows with noise (and NaN in one of them): nothing moves
    c2 = dict(c)
    for name, mask in (("q", real_q), ("dout", real_q), ("k", real_k), ("v", real_k)):
        x = c[name].copy()
        x[~mask] = rng.standard_normal(x[~mask].shape) * 100
        c2[name] = x
    o2, l2 = fwd_of(c2)
    g2 = bwd_of(c2)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    for a, b in zip((dq, dk, dv), g2):
        np.testing.assert_array_equal(a, b)


def test_formula_mode_equals_definition_with_own_stats():
    rng = np.random.default_rng(10)
    c = small_case(rng, lq=[5, 8], lk=[5, 8], pq=[6, 8], pk=[6, 8], hq=4, hkv=1, d=16, causal=True)
    o, l = fwd_of(c)
    a = bwd_of(c)
    b = attn_bwd(c["q"], c["k"], c["v"], c["dout"], c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"],
                 scale=c["scale"], causal=True, out=o, lse=l, mode="formula")
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- values from the pages
def test_te2448_second_call_first_four_kv_rows_zero():
    gold = json.load(open(os.path.join(GOLDEN, "te2448_second_call_zero_rows.json")))
    case = workloads.tiny_gqa_two_calls()[1]
    assert list(case.cu_seqlens_q) == gold["cu_seqlens_q"]
    assert list(case.cu_seqlens_kv) == gold["cu_seqlens_kv"]
    assert list(case.cu_seqlens_q_padded) == gold["cu_seqlens_padded"]
    _, _, (dq, dk, dv) = run_case(case)
    rows = gold["zero_rows_dk_dv"]
    assert np.all(dk[rows] == 0) and np.all(dv[rows] == 0)
    # the second sequence does have gradient, so the zeros are not vacuous
    assert np.abs(dk[4:10]).max() > 0 and np.abs(dv[4:10]).max() > 0


@pytest.mark.parametrize("lengths", workloads.MHA_CAUSAL_LENGTH_SETS)
def test_te3333_query_gradient_norms(lengths):
    gold = json.load(open(os.path.join(GOLDEN, "te3333_qgrad_norms.json")))
    ref = gold["ref_norms"][",".join(map(str, lengths))]
    case = workloads.mha_causal_lengths(list(lengths))
    _, _, (dq, _, _) = run_case(case)
    nrm = float(np.linalg.norm(dq))
    assert abs(nrm - ref) <= gold["rel_tol"] * ref, (lengths, nrm, ref)


def test_te2448_comment_dk_max_magnitude():
    gold = json.load(open(os.path.join(GOLDEN, "te2448_dk_max.json")))
    rng = np.random.default_rng(0)
    T, hq, hkv, d = 128, 4, 1, 256
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    q = bf(rng.standard_normal((T, hq, d), dtype=np.float32))
    k = bf(rng.standard_normal((T, hkv, d), dtype=np.float32))
    v = bf(rng.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.array([0, 64, 128], np.int32)
    dq, dk, dv = attn_bwd(q, k, v, np.ones((T, hq, d)), cu, cu, cu, cu, scale=d ** -0.5,
                          causal=True)
    m = float(np.abs(dk).max())
    lo, hi = gold["range"]
    assert lo <= m <= hi, m


# ---------------------------------------------------------------- chunked (context-parallel) form
from oracle import merge_partials  # noqa: E402


def _chunk_rows(lengths, cuts):
    """Per sequence, the [start, end) of each chunk given interior cut points."""
    return [list(zip([0] + c, c + [L])) for L, c in zip(lengths, cuts)]


def _gather(x, offs, ranges):
    """Rows of chunk `ranges[b]` of every sequence b, packed (THD, no padding)."""
    return np.concatenate([x[o + a:o + b] for o, (a, b) in zip(offs, ranges)], axis=0)


def _cu_of(ranges):
    return np.concatenate([[0], np.cumsum([b - a for a, b in ranges])]).astype(np.int32)


def test_chunked_causal_forward_merge_and_backward_equal_the_whole():
    """Queries and keys of every sequence cut into uneven chunks at sequence
    positions q0/k0: the causal rule on positions per chunk pair, partial (O, LSE)
    merged over key chunks, equals attention over the whole sequences; the
    backward of every chunk pair with the whole O and LSE sums to the whole
    gradients (dQ over key chunks, dK/dV over query chunks)."""
    rng = np.random.default_rng(17)
    L = [13, 7, 20]
    hq, hkv, d, sc = 4, 2, 8, 0.35
    T = sum(L)
    offs = np.concatenate([[0], np.cumsum(L)])[:-1]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    q, dout = rng.standard_normal((T, hq, d)), rng.standard_normal((T, hq, d))
    k, v = rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hkv, d))
    o_full, l_full = attn_fwd(q, k, v, cu, cu, scale=sc, causal=True)
    g_full = attn_bwd(q, k, v, dout, cu, cu, scale=sc, causal=True)
    qch = _chunk_rows(L, [[5], [3], [8, 9]])            # 2, 2, 3 query chunks
    kch = _chunk_rows(L, [[4, 11], [6], [2, 15]])        # 3, 2, 3 key chunks
    nq = max(len(c) for c in qch)
    nk = max(len(c) for c in kch)
    pick = lambda ch, i: [c[i] if i < len(c) else (c[-1][1], c[-1][1]) for c in ch]
    dq = np.zeros_like(q)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for iq in range(nq):
        qr = pick(qch, iq)
        qq, qdo = _gather(q, offs, qr), _gather(dout, offs, qr)
        cq = _cu_of(qr)
        o_glob, l_glob = _gather(o_full, offs, qr), _gather(l_full, offs, qr)
        acc_o, acc_l = None, None
        for ik in range(nk):
            kr = pick(kch, ik)
            kk, vv, ck = _gather(k, offs, kr), _gather(v, offs, kr), _cu_of(kr)
            pos = dict(q_pos0=[a for a, _ in qr], kv_pos0=[a for a, _ in kr])
            o_p, l_p = attn_fwd(qq, kk, vv, cq, ck, scale=sc, causal=True, **pos)
            acc_o, acc_l = (o_p, l_p) if acc_o is None else merge_partials(acc_o, acc_l, o_p, l_p)
            gq, gk, gv = attn_bwd(qq, kk, vv, qdo, cq, ck, scale=sc, causal=True, out=o_glob,
                                  lse=l_glob, mode="formula", **pos)
            for b, ((qa, qb), (ka, kb)) in enumerate(zip(qr, kr)):
                dq[offs[b] + qa:offs[b] + qb] += gq[cq[b]:cq[b + 1]]
                dk[offs[b] + ka:offs[b] + kb] += gk[ck[b]:ck[b + 1]]
                dv[offs[b] + ka:offs[b] + kb] += gv[ck[b]:ck[b + 1]]
        np.testing.assert_allclose(acc_o, o_glob, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(acc_l, l_glob, rtol=1e-13)
    for a, b in zip((dq, dk, dv), g_full):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_position_shift_reproduces_both_alignments():
    rng = np.random.default_rng(18)
    q, k, v = rng.standard_normal((5, 2, 8)), rng.standard_normal((9, 1, 8)), rng.standard_normal((9, 1, 8))
    np.testing.assert_array_equal(attn_fwd_seq(q, k, v, 0.5, True, shift=0)[0],
                                  attn_fwd_seq(q, k, v, 0.5, True)[0])
    np.testing.assert_array_equal(attn_fwd_seq(q, k, v, 0.5, True, shift=4)[0],
                                  attn_fwd_seq(q, k, v, 0.5, "bottom_right")[0])
    # a key chunk entirely after every query: nothing visible
    o, l = attn_fwd_seq(q, k, v, 0.5, True, shift=-5)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_merge_partials_closed_forms():
    rng = np.random.default_rng(19)
    oa, ob = rng.standard_normal((6, 3, 4)), rng.standard_normal((6, 3, 4))
    la, lb = rng.standard_normal((6, 3)), rng.standard_normal((6, 3))
    ninf = np.full((6, 3), -np.inf)
    # an empty side leaves the other unchanged, exactly
    o, l = merge_partials(oa, la, ob, ninf)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    # both empty: zero output, -inf statistic
    o, l = merge_partials(oa, ninf, ob, ninf)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # two equal halves: same output, statistic + ln 2
    o, l = merge_partials(oa, la, oa, la)
    np.testing.assert_allclose(o, oa, rtol=1e-15)
    np.testing.assert_allclose(l, la + math.log(2), rtol=1e-15)
    # symmetric, and the weights are the two softmax masses
    o1, l1 = merge_partials(oa, la, ob, lb)
    o2, l2 = merge_partials(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    w = 1.0 / (1.0 + np.exp(lb - la))
    np.testing.assert_allclose(o1, w[..., None] * oa + (1 - w)[..., None] * ob, rtol=1e-12)


# ---------------------------------------------------------------- dropout (counter-based mask)
from oracle.philox import dropout_threshold, keep_mask, philox4x32_10  # noqa: E402


@pytest.mark.parametrize("ctr,key,want", [
    # known-answer vectors published with the Philox generator (Salmon et al.,
    # "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11; Random123's
    # philox4x32, 10 rounds): zero, all-ones, and digits-of-pi inputs
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, want):
    got = philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
    assert [int(x) for x in got] == want


def test_keep_mask_rate_and_determinism():
    t = dropout_threshold(0.1)
    assert t == 26
    m = keep_mask(700, 900, 3, 5, 8, seed=2024, offset=7, t=t)
    rate, want = m.mean(), 1 - t / 256
    assert abs(rate - want) <= 5 * math.sqrt(want * (1 - want) / m.size)
    assert np.array_equal(m, keep_mask(700, 900, 3, 5, 8, seed=2024, offset=7, t=t))
    # other sequence, head, offset or seed: another mask (about p(1-p)*2 of entries differ)
    for other in (dict(b=4, h=5, offset=7, seed=2024), dict(b=3, h=6, offset=7, seed=2024),
                  dict(b=3, h=5, offset=8, seed=2024), dict(b=3, h=5, offset=7, seed=2025)):
        o = keep_mask(700, 900, other["b"], other["h"], 8, seed=other["seed"],
                      offset=other["offset"], t=t)
        assert 0.12 < np.mean(o != m) < 0.24
    assert keep_mask(5, 7, 0, 0, 1, seed=1, offset=0, t=0).all()


def _philox_scalar(ctr, key):
    """Philox4x32-10 on Python integers, one counter at a time, written from the
    generator's description (Salmon et al., SC'11, "Philox"): per round, the
    64-bit products of words 0 and 2 with the two multipliers; new words =
    (hi(w2 product) ^ w1 ^ k0, lo(w2 product), hi(w0 product) ^ w3 ^ k1,
    lo(w0 product)); the key is bumped by the two Weyl constants between rounds."""
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    M = 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + 0x9E3779B9) & M, (k1 + 0xBB67AE85) & M
        p0, p1 = 0xD2511F53 * c0, 0xCD9E8D57 * c2
        c0, c1, c2, c3 = (p1 >> 32) ^ c1 ^ k0, p1 & M, (p0 >> 32) ^ c3 ^ k1, p0 & M
    return [c0, c1, c2, c3]


def test_philox_scalar_matches_known_answers():
    assert _philox_scalar([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert _philox_scalar([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                          [0xA4093822, 0x299F31D0]) == [0xD16CFE09, 0x94FDCCEB, 0x5001E420,
                                                        0x24126EA1]


# (query i, key j, sequence b, head h, hq, seed, offset): i and j differ in both
# their quad (>> 2) and their position in it (& 3), so a transposed counter or
# a word / byte mix-up picks another byte
KEEP_POINTS = [(6, 13, 0, 0, 1, 1, 0), (13, 6, 2, 3, 8, 0xDEADBEEF12345678, 5),
               (1, 10, 5, 7, 8, 2024, 7), (250, 97, 1, 2, 4, 0x5EED, 0),
               (33, 70, 15, 63, 64, 0xC0FFEE, 3)]


def _keep_byte(i, j, b, h, hq, seed, offset, word_of=lambda i, j: i & 3,
               byte_of=lambda i, j: j & 3, ctr_of=lambda i, j: (j >> 2, i >> 2)):
    c0, c1 = ctr_of(i, j)
    words = _philox_scalar([c0, c1, b, (offset * hq + h) & 0xFFFFFFFF],
                           [seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF])
    return (words[word_of(i, j)] >> (8 * byte_of(i, j))) & 0xFF


def test_keep_mask_layout_by_hand():
    """Element (i, j) of keep_mask is decided by byte (j & 3) of word (i & 3) of
    the Philox call with counter (j >> 2, i >> 2, b, offset * hq + h) and key
    (seed_lo, seed_hi): thresholds t = byte and t = byte + 1 straddle it, so the
    mask pins the byte exactly at every point."""
    for i, j, b, h, hq, seed, offset in KEEP_POINTS:
        byte = _keep_byte(i, j, b, h, hq, seed, offset)
        for t, want in ((byte, True), (byte + 1, False)):
            if t > 255:
                continue
            m = keep_mask(i + 1, j + 1, b, h, hq, seed=seed, offset=offset, t=t)
            assert bool(m[i, j]) is want, (i, j, b, h, t)
    # the points tell the plausible mistakes apart
    swaps = [dict(ctr_of=lambda i, j: (i >> 2, j >> 2)),
             dict(word_of=lambda i, j: j & 3, byte_of=lambda i, j: i & 3)]
    for sw in swaps:
        assert any(_keep_byte(*pt, **sw) != _keep_byte(*pt) for pt in KEEP_POINTS)


def _dropout_case(seed=21, causal=True):
    rng = np.random.default_rng(seed)
    return small_case(rng, lq=[5, 9], lk=[7, 9], pq=[6, 10], pk=[8, 9], hq=4, hkv=2, d=8,
                      causal=causal)


def test_dropout_zero_is_no_dropout():
    c = _dropout_case()
    args = (c["q"], c["k"], c["v"], c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"])
    a = attn_fwd(*args, scale=c["scale"], causal=True)
    b = attn_fwd(*args, scale=c["scale"], causal=True, dropout=(0.0, 5, 0))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_dropout_finite_differences():
    """Gradients with a fixed keep mask (same seed) against central differences."""
    c = _dropout_case(seed=22)
    drop = (0.3, 99, 3)
    args = lambda q, k, v: (q, k, v, c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"])
    grads = attn_bwd(c["q"], c["k"], c["v"], c["dout"], c["cu_q"], c["cu_kv"], c["cu_qp"],
                     c["cu_kp"], scale=c["scale"], causal=True, dropout=drop)
    eps = 1e-6
    for gi, name in enumerate("qkv"):
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xs = []
            for sgn in (1, -1):
                xp = x.copy()
                xp[idx] += sgn * eps
                kw = dict(q=c["q"], k=c["k"], v=c["v"])
                kw[name] = xp
                o, _ = attn_fwd(*args(kw["q"], kw["k"], kw["v"]), scale=c["scale"], causal=True,
                                dropout=drop)
                xs.append(np.sum(c["dout"] * o))
            num[idx] = (xs[0] - xs[1]) / (2 * eps)
        err = np.linalg.norm(grads[gi] - num) / np.linalg.norm(num)
        assert err <= 1e-7, (name, err)


def test_dropout_formula_mode_matches_definition():
    c = _dropout_case(seed=23)
    drop = (0.25, 11, 0)
    a = (c["q"], c["k"], c["v"], c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"])
    o, l = attn_fwd(*a, scale=c["scale"], causal=True, dropout=drop)
    g1 = attn_bwd(c["q"], c["k"], c["v"], c["dout"], *a[3:], scale=c["scale"], causal=True,
                  dropout=drop)
    g2 = attn_bwd(c["q"], c["k"], c["v"], c["dout"], *a[3:], scale=c["scale"], causal=True,
                  dropout=drop, out=o, lse=l, mode="formula")
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-13)
    # LSE is the softmax's own: unchanged by dropout
    _, l0 = attn_fwd(*a, scale=c["scale"], causal=True)
    np.testing.assert_array_equal(l, l0)


def test_dropout_is_unbiased_over_seeds():
    """E over masks of O equals the output without dropout (inverted dropout)."""
    c = _dropout_case(seed=24, causal=False)
    a = (c["q"], c["k"], c["v"], c["cu_q"], c["cu_kv"], c["cu_qp"], c["cu_kp"])
    o0, _ = attn_fwd(*a, scale=c["scale"])
    n = 600
    acc = np.zeros_like(o0)
    sq = np.zeros_like(o0)
    for s in range(n):
        o, _ = attn_fwd(*a, scale=c["scale"], dropout=(0.5, 1000 + s, 0))
        acc += o
        sq += o * o
    mean = acc / n
    sd = np.sqrt(np.maximum(sq / n - mean ** 2, 0) / n)
    rows = np.abs(o0).sum(axis=(1, 2)) > 0
    z = np.abs(mean - o0)[rows] / (sd[rows] + 1e-12)
    assert np.max(z) < 6.0


# ---------------------------------------------------------------- FP8 inputs
from oracle.fp8 import attn_bwd_fp8, attn_fwd_fp8, decode_e4m3  # noqa: E402


def test_e4m3_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9


def test_fp8_forward_folds_descales_into_the_bf16_definition():
    """FP8 codes with descales equal the plain forward on the scaled values; scaling
    q by 2 and its descale by 1/2 (exact in E4M3 away from the range ends) changes nothing."""
    rng = np.random.default_rng(30)
    T, hq, hkv, d = 20, 4, 2, 16
    qn = rng.standard_normal((T, hq, d), dtype=np.float32) * 2
    qn = np.sign(qn) * np.maximum(np.abs(qn), 0.1)    # normal E4M3 values: doubling is exact
    q = torch.from_numpy(qn.astype(np.float32))
    k = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32))
    v = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32))
    f8 = lambda t: t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    cu = np.array([0, 7, 20], np.int32)
    o, l = attn_fwd_fp8(f8(q), f8(k), f8(v), 0.5, 0.25, 3.0, cu, cu, causal=True)
    back = lambda t: t.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    o2, l2 = attn_fwd(back(q) * 0.5, back(k) * 0.25, back(v) * 3.0, cu, cu, causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    o3, l3 = attn_fwd_fp8(f8(q * 2), f8(k), f8(v), 0.25, 0.25, 3.0, cu, cu, causal=True)
    np.testing.assert_allclose(o3, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3, l, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
def test_fp8_backward_chain_rule_through_the_descales(causal):
    """With the codes fixed, L = sum(dO o O) is a function of the three descales and
    dL/ds_q = sum(dQ o Q8), dL/ds_k = sum(dK o K8), dL/ds_v = sum(dV o V8), where
    dQ, dK, dV are the gradients with respect to the real-valued inputs.  Central
    differences of the forward pin the backward, the descale placement included."""
    rng = np.random.default_rng(33)
    lq, lk, pq, pk = [5, 9], [7, 9], [8, 9], [8, 10]
    hq, hkv, d = 4, 2, 8
    Tq, Tk = sum(pq), sum(pk)
    f8 = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32) * 8).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    q8, k8, v8 = f8(Tq, hq, d), f8(Tk, hkv, d), f8(Tk, hkv, d)
    do = rng.standard_normal((Tq, hq, d))
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    args = (cu(lq), cu(lk), cu(pq), cu(pk))
    s = np.array([0.07, 0.11, 0.3])

    def loss(sv):
        o, _ = attn_fwd_fp8(q8, k8, v8, *sv, *args, causal=causal)
        return float(np.sum(do * o))

    dq, dk, dv = attn_bwd_fp8(q8, k8, v8, *s, do, *args, causal=causal)
    codes = (decode_e4m3(q8), decode_e4m3(k8), decode_e4m3(v8))
    for i, (g, c) in enumerate(zip((dq, dk, dv), codes)):
        h = 1e-6 * s[i]
        e = np.zeros(3)
        e[i] = h
        fd = (loss(s + e) - loss(s - e)) / (2 * h)
        an = float(np.sum(g * c))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)
