"""fp64 CPU oracle for scaled-dot-product attention over packed THD sequences.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

It is the plain definition, written for a reader to check by eye:
one sequence and one query head at a time, full Lq x Lk matrices, numpy
float64, no tiling, no online softmax, no fusion.  Inputs are the exact
storage-dtype values widened to float64.

Sources (web pages, cited by title and section):

* [TE-2448] TransformerEngine issue "Inconsistent fused_attn_bwd results of
  dk, dv under THD layout + GQA on multiple calls": THD tensors
  ``(seqlen, heads, d)``, ``cu_seqlens_*`` next to ``cu_seqlens_*_padded``,
  ``attn_scale``, the ``padding`` mask, GQA with hq=2/hkv=1 ("Steps/Code to
  reproduce bug"); padded KV slots of a sequence without valid queries must
  get all-zero dK/dV ("Expected behavior").
* [TE-3333] "FusedAttention (cuDNN) THD backward produces wrong gradients on
  sm_120 ...": the reference is a loop over sequences of full causal SDPA,
  concatenated ("Reproduction").
* [TE-3216] "flash-attn-4 4.0.0b11: DotProductAttention batched backward
  returns wrong dQ/dK/dV at head_dim=256": the fp32 reference repeats each
  KV head over its group of query heads (``repeat_interleave``), scales by
  ``1/sqrt(d)`` and masks the strict upper triangle for causal
  ("Reproduce", the fp32_reference function).
* [TE-2892] "SIGSEGV in fused_attn_fwd when cu_seqlens_q !=
  cu_seqlens_q_padded": real boundaries mask, padded boundaries index, the
  output keeps the padded layout ("Expected Behavior").

Readings taken where the pages are silent:

* real tokens of sequence b occupy rows ``[cu_pad[b], cu_pad[b] + L_b)``,
  the rest of the slot is padding;
* causal is top-left aligned: query i may see key j iff j <= i (the pages
  only use causal with Lq == Lk, where every alignment agrees); the
  bottom-right variant, which the pages do not name, aligns the ends:
  j <= i + (Lk - Lq);
* LSE is the natural-log log-sum-exp of the scaled scores, fp32 ``[T, hq]``;
* a query row with no allowed key (and every padding row) has O = 0 and
  LSE = -inf; every gradient row outside the real ranges is +0.0;
* query head h reads KV head ``h // (hq // hkv)``;
* dropout (absent from the pages, which set ``dropout=0.0``): inverted
  dropout on the softmax probabilities with the counter-based keep mask of
  ``oracle.philox``; LSE is that of the softmax before dropout.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["sequence_slots", "attn_fwd", "attn_bwd", "attn_fwd_seq", "attn_bwd_seq",
           "allowed_mask", "merge_partials"]


def sequence_slots(cu_seqlens: np.ndarray, cu_seqlens_padded: Optional[np.ndarray]):
    """Per sequence: (memory offset, real length).

    [TE-2892] "Expected Behavior": ``cu_seqlens`` gives the real token counts
    (used for masking), ``cu_seqlens_padded`` the memory layout (used for
    indexing).  A missing padded array means the layout has no padding.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cup = cu if cu_seqlens_padded is None else np.asarray(cu_seqlens_padded, dtype=np.int64)
    lengths = cu[1:] - cu[:-1]
    offsets = cup[:-1]
    slots = cup[1:] - cup[:-1]
    if np.any(lengths < 0) or np.any(lengths > slots):
        raise ValueError("real length must be in [0, padded slot length]")
    return [(int(o), int(L)) for o, L in zip(offsets, lengths)]


def allowed_mask(lq: int, lk: int, causal, shift: Optional[int] = None) -> np.ndarray:
    """Boolean [lq, lk]: key j is visible to query i.

    ``padding`` (causal False): all real keys of the sequence ([TE-2448],
    attn_mask_type "padding").  ``padding_causal`` (causal True or
    "top_left"): additionally j <= i -- the complement of the strict upper
    triangle masked in [TE-3216]'s fp32_reference.  "bottom_right": the same
    triangle aligned to the last query and key, j <= i + (lk - lq); with
    lq == lk both alignments agree (the pages use causal only there, and do
    not name the bottom-right variant: its definition here is the plain
    reading of aligning the two sequences at their ends).

    ``shift`` (causal True only) gives the diagonal directly: j <= i + shift.
    A chunk of queries at sequence positions q0 + i and a chunk of keys at
    k0 + j see each other iff k0 + j <= q0 + i, i.e. shift = q0 - k0 (the
    causal rule of the whole sequence restricted to the two chunks).
    """
    m = np.ones((lq, lk), dtype=bool)
    if causal:
        if causal not in (True, "top_left", "bottom_right"):
            raise ValueError(f"causal must be False, True, 'top_left' or 'bottom_right', not {causal!r}")
        if shift is None:
            shift = (lk - lq) if causal == "bottom_right" else 0
        elif causal == "bottom_right":
            raise ValueError("an explicit shift goes with causal=True")
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        m &= j <= i + shift
    return m


def _softmax_rows(s: np.ndarray, allowed: np.ndarray):
    """Row softmax restricted to ``allowed``; returns (P, LSE).

    Rows with no allowed entry get P = 0 and LSE = -inf (ln of an empty sum).
    """
    lse = np.full(s.shape[0], -np.inf)
    p = np.zeros_like(s)
    rows = allowed.any(axis=1)
    if rows.any():
        sm = np.where(allowed, s, -np.inf)[rows]
        mx = sm.max(axis=1, keepdims=True)
        e = np.exp(sm - mx)                      # exp(-inf) = 0 off the allowed set
        tot = e.sum(axis=1, keepdims=True)
        p[rows] = e / tot
        lse[rows] = (mx + np.log(tot))[:, 0]
    return p, lse


def attn_fwd_seq(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal,
                 shift: Optional[int] = None, keep=None, keep_scale: float = 1.0):
    """Forward of one sequence, all heads: O = softmax(scale * Q K^T + mask) V.

    q: [Lq, hq, d]; k, v: [Lk, hkv, d] (real rows only, float64).
    Returns O [Lq, hq, d] and LSE [Lq, hq].
    [TE-3333] "Reproduction" (per-sequence SDPA); [TE-3216] "Reproduce" (GQA
    by repeating KV heads over contiguous groups, explicit scale).

    Dropout (``keep``: bool [hq, Lq, Lk]): the probabilities are multiplied by
    keep * keep_scale before the product with V; LSE stays that of the
    softmax itself.
    """
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    G = hq // hkv
    out = np.zeros((lq, hq, d))
    lse = np.full((lq, hq), -np.inf)
    allowed = allowed_mask(lq, lk, causal, shift)
    for h in range(hq):
        g = h // G
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        p, l = _softmax_rows(s, allowed)
        if keep is not None:
            p = p * keep[h] * keep_scale
        out[:, h, :] = p @ v[:, g, :]
        lse[:, h] = l
    return out, lse


def attn_bwd_seq(q, k, v, dout, scale: float, causal, out=None, lse=None,
                 mode: str = "definition", shift: Optional[int] = None, keep=None,
                 keep_scale: float = 1.0):
    """Backward of one sequence, all heads: dQ, dK, dV of l = sum(dO * O).

    ``definition`` (default): the exact gradient, with P recomputed from q,k
    in float64 and Delta_i = sum_j P_ij dP_ij; the given out/lse are ignored.

    ``formula``: what a fused backward evaluates from its saved statistics,
    P_ij = exp(scale*q_i.k_j - LSE_i) on the allowed set and
    Delta_i = sum_c dO_ic O_ic, with the caller's ``out`` and ``lse``.

    dK and dV of a KV head sum the contributions of every query head in its
    group ([TE-3216] repeat_interleave; its transpose is a sum).

    With dropout (``keep``, as in ``attn_fwd_seq``) the output is
    O = (P o D) V with D = keep * keep_scale, so dV = (P o D)^T dO and the
    gradient reaching P is dP = D o (dO V^T); Delta = sum_j P_ij dP_ij, which
    equals rowsum(dO o O) (the formula mode's form).
    """
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    G = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    allowed = allowed_mask(lq, lk, causal, shift)
    for h in range(hq):
        g = h // G
        Q, K, V, dO = q[:, h, :], k[:, g, :], v[:, g, :], dout[:, h, :]
        s = scale * (Q @ K.T)
        D = 1.0 if keep is None else keep[h] * keep_scale
        if mode == "definition":
            p, _ = _softmax_rows(s, allowed)
            dp = D * (dO @ V.T)
            delta = np.sum(p * dp, axis=1)
        elif mode == "formula":
            L = lse[:, h]
            use = allowed & np.isfinite(L)[:, None]
            p = np.zeros_like(s)
            p[use] = np.exp((s - L[:, None])[use])
            dp = D * (dO @ V.T)
            delta = np.sum(dO * out[:, h, :], axis=1)
        else:
            raise ValueError(mode)
        ds = p * (dp - delta[:, None])
        dq[:, h, :] = scale * (ds @ K)
        dk[:, g, :] += scale * (ds.T @ Q)
        dv[:, g, :] += (p * D).T @ dO
    return dq, dk, dv


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _dropout_masks(dropout, b, lq, lk, hq):
    """(keep [hq, lq, lk], keep_scale) of sequence b for dropout = (p, seed, offset)."""
    if dropout is None or dropout[0] == 0.0:
        return None, 1.0
    from .philox import dropout_threshold, keep_mask
    p, seed, offset = dropout
    t = dropout_threshold(p)
    keep = np.stack([keep_mask(lq, lk, b, h, hq, seed, offset, t) for h in range(hq)])
    return keep, 256.0 / (256.0 - t)


def _shifts(q_pos0, kv_pos0, n):
    """Per-sequence diagonal shift q_pos0[b] - kv_pos0[b] (None: derived from the mask)."""
    if q_pos0 is None and kv_pos0 is None:
        return [None] * n
    qp = np.zeros(n, np.int64) if q_pos0 is None else np.asarray(q_pos0, np.int64)
    kp = np.zeros(n, np.int64) if kv_pos0 is None else np.asarray(kv_pos0, np.int64)
    return [int(a - b) for a, b in zip(qp, kp)]


def attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded=None,
             cu_seqlens_kv_padded=None, scale: float = None, causal=False,
             q_pos0=None, kv_pos0=None, dropout=None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward over the packed THD tensors.

    q: [Tq, hq, d], k, v: [Tkv, hkv, d].  Returns out [Tq, hq, d] (float64)
    and lse [Tq, hq] (float64).  Every row outside the real ranges has
    out = 0 and lse = -inf; the output keeps the padded layout ([TE-2892]
    "Expected Behavior", item 3).  ``scale`` defaults to 1/sqrt(d)
    ([TE-3216] fp32_reference, [TE-2448] comment's softmax_scale).

    ``q_pos0`` / ``kv_pos0`` (per sequence, with causal True): the slots hold
    chunks of longer sequences whose first real tokens sit at these positions;
    the causal rule is applied to the positions (see ``allowed_mask``).

    ``dropout`` = (p, seed, offset): the keep mask of ``oracle.philox`` for
    every sequence b (its index in the batch) and query head.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, hq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if hq % k.shape[1]:
        raise ValueError("hkv must divide hq")
    out = np.zeros_like(q)
    lse = np.full((Tq, hq), -np.inf)
    qs = sequence_slots(cu_seqlens_q, cu_seqlens_q_padded)
    ks = sequence_slots(cu_seqlens_kv, cu_seqlens_kv_padded)
    shifts = _shifts(q_pos0, kv_pos0, len(qs))
    for b, ((oq, lq), (ok, lk), sh) in enumerate(zip(qs, ks, shifts)):
        if lq == 0:
            continue
        keep, ks_ = _dropout_masks(dropout, b, lq, lk, hq)
        o_b, l_b = attn_fwd_seq(q[oq:oq + lq], k[ok:ok + lk], v[ok:ok + lk], scale, causal, sh,
                                keep, ks_)
        out[oq:oq + lq] = o_b
        lse[oq:oq + lq] = l_b
    return out, lse


def attn_bwd(q, k, v, dout, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded=None,
             cu_seqlens_kv_padded=None, scale: float = None, causal=False,
             out=None, lse=None, mode: str = "definition", q_pos0=None, kv_pos0=None,
             dropout=None):
    """Backward over the packed THD tensors: (dq, dk, dv), float64, padded layout.

    Rows outside the real ranges are exactly 0; so is every KV row of a
    sequence with no valid query ([TE-2448] "Expected behavior": the first
    4 tokens of dk and dv of the second call are all zeros).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, hq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if mode == "formula":
        out, lse = _f64(out), _f64(lse)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    qs = sequence_slots(cu_seqlens_q, cu_seqlens_q_padded)
    ks = sequence_slots(cu_seqlens_kv, cu_seqlens_kv_padded)
    shifts = _shifts(q_pos0, kv_pos0, len(qs))
    for b, ((oq, lq), (ok, lk), sh) in enumerate(zip(qs, ks, shifts)):
        if lq == 0 or lk == 0:
            continue
        sq, sk = slice(oq, oq + lq), slice(ok, ok + lk)
        keep, ks_ = _dropout_masks(dropout, b, lq, lk, hq)
        r = attn_bwd_seq(q[sq], k[sk], v[sk], dout[sq], scale, causal,
                         None if out is None else out[sq], None if lse is None else lse[sq], mode,
                         sh, keep, ks_)
        dq[sq], dk[sk], dv[sk] = r
    return dq, dk, dv


def merge_partials(out_a, lse_a, out_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax over the union of two disjoint key sets from the two partial results.

    With P_a = exp(S - LSE_a) over set A (so that O_a = P_a V_A) and likewise
    for B, the softmax over A u B has LSE = ln(exp(LSE_a) + exp(LSE_b)) and
    O = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.  A side with LSE = -inf
    (no key) has weight 0; if both do, O = 0 and LSE = -inf.
    out_*: [T, h, d], lse_*: [T, h] (float64).
    """
    la, lb = _f64(lse_a), _f64(lse_b)
    oa, ob = _f64(out_a), _f64(out_b)
    lse = np.logaddexp(la, lb)                 # -inf when both are -inf
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    wa = np.where(fin, np.exp(la - safe), 0.0)  # exp(-inf) = 0 for an empty side
    wb = np.where(fin, np.exp(lb - safe), 0.0)
    out = wa[..., None] * oa + wb[..., None] * ob
    return out, lse
