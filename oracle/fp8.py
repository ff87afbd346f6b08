"""FP8 E4M3 decoding and the FP8-input attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E4M3 as in the OCP 8-bit floating point specification (the format of
``torch.float8_e4m3fn``): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 encodes subnormals m * 2^-9; the codes S.1111.111 are
NaN; there is no infinity (largest finite 448).

The pages run FP8 attention only through TransformerEngine's recipes
(TE-2892 "Reproduction": the blockwise recipe on THD with cu_seqlens_q !=
cu_seqlens_q_padded, where the forward crashes) and never spell out the
arithmetic; the forward specified here takes Q, K, V as E4M3 codes with one
float32 descale factor per tensor:

    O = softmax(scale * s_q * s_k * Q8 K8^T + mask) (s_v * V8),

LSE that of the scaled scores, with the THD boundaries and masks of the bf16
path (``attention.attn_fwd``).  Its backward is the gradient with respect to
the real-valued inputs s_q Q8, s_k K8, s_v V8 (the plain reading: the codes
and descales define the values, the gradient is that of the attention over
them), i.e. ``attention.attn_bwd`` on those values.
"""
from __future__ import annotations

import numpy as np

from .attention import attn_bwd, attn_fwd

__all__ = ["decode_e4m3", "attn_fwd_fp8", "attn_bwd_fp8"]


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def attn_fwd_fp8(q8, k8, v8, s_q: float, s_k: float, s_v: float, cu_seqlens_q, cu_seqlens_kv,
                 cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None, scale: float = None,
                 causal=False):
    """Forward from E4M3 codes (uint8 [T, h, d]) and per-tensor descales; float64 out, lse."""
    q, k, v = decode_e4m3(q8), decode_e4m3(k8), decode_e4m3(v8)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return attn_fwd(q * s_q, k * s_k, v * s_v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                    cu_seqlens_kv_padded, scale=scale, causal=causal)


def attn_bwd_fp8(q8, k8, v8, s_q: float, s_k: float, s_v: float, dout, cu_seqlens_q,
                 cu_seqlens_kv, cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None,
                 scale: float = None, causal=False):
    """Backward of ``attn_fwd_fp8``: float64 (dq, dk, dv) with respect to s_q Q8, s_k K8,
    s_v V8, for the output gradient dout."""
    q, k, v = decode_e4m3(q8), decode_e4m3(k8), decode_e4m3(v8)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return attn_bwd(q * s_q, k * s_k, v * s_v, np.asarray(dout, dtype=np.float64), cu_seqlens_q,
                    cu_seqlens_kv, cu_seqlens_q_padded, cu_seqlens_kv_padded, scale=scale,
                    causal=causal)
