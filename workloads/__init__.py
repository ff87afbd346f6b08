"""Seeded synthetic inputs for packed variable-length (THD) attention.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It only draws random numbers, rounds them to the storage dtype and
builds the ``cu_seqlens`` boundary arrays; it holds none of the attention
arithmetic.  Every draw uses ``numpy.random.default_rng(seed)`` so the values
are identical on every machine.

Workloads (each named by what it is, with its sizes):

* ``tiny_gqa_two_calls``  -- TE issue 2448 "Inconsistent fused_attn_bwd
  results of dk, dv under THD layout + GQA on multiple calls", section
  "Steps/Code to reproduce bug": T=12 tokens in two padded slots
  ``[0,4,12]``, hq=2, hkv=1, d=8, fp16, scale 0.1, ``padding`` mask; call 1
  has ``cu_seqlens_q=[0,1,3]``, call 2 ``[0,0,3]``, both
  ``cu_seqlens_kv=[0,3,9]``.  As in the page's loop, each call draws its
  own tensors from one stream seeded once with 42.
* ``mha_causal_lengths``  -- TE issue 3333 "FusedAttention (cuDNN) THD
  backward produces wrong gradients on sm_120", section "Reproduction":
  H=8, d=128, bf16, ``padding_causal``, default scale, independent N(0,1)
  q/k/v after one seed (42), dout = ones (the gradient of ``out.sum()``),
  cu_seqlens == cu_seqlens_padded, length sets [128], [128,96], [128,128],
  [256,256].
* ``real_vs_padded``      -- TE issue 2892 "SIGSEGV in fused_attn_fwd when
  cu_seqlens_q != cu_seqlens_q_padded with FP8 blockwise", section
  "Reproduction": real lengths [100,150,120,130] in padded slots
  [112,160,128,144], 32 heads, d=48, bf16; every row (padding rows too)
  is N(0,1) so that any leak of padding rows shows.
* ``gqa_d256_batched``    -- TE issue 3216 "flash-attn-4 4.0.0b11 ...
  wrong dQ/dK/dV at head_dim=256", sections "Conditions"/"Reproduce": two
  sequences of 384 tokens (sbhd [384,2,16,256] re-expressed as THD), hq=16,
  hkv=2, d=256, bf16, causal, scale 1/16; optional variant with a few
  8-sigma outlier channels per KV head (the page's captured activations are
  not available, so seeded outliers stand in for them).
* ``throughput_65k``      -- 65536 packed tokens, lengths uniform in
  [256, 8192] padded to multiples of 64, hq=64, hkv=8, d=128, bf16,
  ``padding_causal``.
* ``d64_65k``, ``d256_65k`` -- the throughput_65k sequences at head dims 64
  and 256 (hq=64, hkv=8, bf16, causal); ``mqa_65k`` with one KV head.
* ``large_offsets``       -- 266304 tokens (260 slots of 1024, 64 trailing
  rows), hq=64, hkv=8, d=128, bf16, ``padding_causal``: the query-side
  tensors pass 2^31 elements and 2^32 bytes.  The one workload drawn on the
  GPU (torch's seeded generator): numpy would spend about a minute on its
  4.4e9 draws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Union

import numpy as np
import torch

BF16 = "bf16"
FP16 = "fp16"

_TORCH_DTYPE = {BF16: torch.bfloat16, FP16: torch.float16}


@dataclass
class Case:
    """One attention call's inputs (tensors in the storage dtype, on the CPU
    except where a workload says otherwise)."""

    name: str
    q: torch.Tensor            # [total_q, hq, d]
    k: torch.Tensor            # [total_kv, hkv, d]
    v: torch.Tensor            # [total_kv, hkv, d]
    dout: torch.Tensor         # [total_q, hq, d]
    cu_seqlens_q: np.ndarray   # int32 [B+1], real token boundaries
    cu_seqlens_kv: np.ndarray
    cu_seqlens_q_padded: np.ndarray  # int32 [B+1], memory layout boundaries
    cu_seqlens_kv_padded: np.ndarray
    scale: float
    causal: Union[bool, str]   # False, True (top-left triangle) or "bottom_right"
    dtype: str
    max_seqlen_q: int = 0
    max_seqlen_kv: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.cu_seqlens_q) - 1)

    @property
    def hq(self) -> int:
        return int(self.q.shape[1])

    @property
    def hkv(self) -> int:
        return int(self.k.shape[1])

    @property
    def d(self) -> int:
        return int(self.q.shape[2])

    @property
    def mask_type(self) -> str:
        if self.causal == "bottom_right":
            return "padding_causal_bottom_right"
        return "padding_causal" if self.causal else "padding"


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) draw in fp32, rounded (RNE) to the storage dtype."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(_TORCH_DTYPE[dtype])


def _cu(lengths: List[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def tiny_gqa_two_calls() -> List[Case]:
    """The two fused_attn_bwd calls of the TE 2448 reproduction (T=12, hq=2, hkv=1, d=8)."""
    rng = np.random.default_rng(42)
    cu_pad = np.array([0, 4, 12], dtype=np.int32)
    cu_q_calls = [np.array([0, 1, 3], dtype=np.int32), np.array([0, 0, 3], dtype=np.int32)]
    cu_kv_calls = [np.array([0, 3, 9], dtype=np.int32), np.array([0, 3, 9], dtype=np.int32)]
    T, hq, hkv, d = 12, 2, 1, 8
    cases = []
    for i in range(2):
        q = _normal(rng, (T, hq, d), FP16)
        k = _normal(rng, (T, hkv, d), FP16)
        v = _normal(rng, (T, hkv, d), FP16)
        # the page also draws random out and lse; they are kept as extras
        out_rand = _normal(rng, (T, hq, d), FP16)
        dout = _normal(rng, (T, hq, d), FP16)
        lse_rand = _normal(rng, (T, hq), FP16).to(torch.float32)
        cases.append(Case(
            name=f"tiny_gqa_call{i + 1}", q=q, k=k, v=v, dout=dout,
            cu_seqlens_q=cu_q_calls[i], cu_seqlens_kv=cu_kv_calls[i],
            cu_seqlens_q_padded=cu_pad.copy(), cu_seqlens_kv_padded=cu_pad.copy(),
            scale=0.1, causal=False, dtype=FP16, max_seqlen_q=8, max_seqlen_kv=8,
            extra={"out_random": out_rand, "lse_random": lse_rand}))
    return cases


MHA_CAUSAL_LENGTH_SETS = ([128], [128, 96], [128, 128], [256, 256])


def mha_causal_lengths(lengths: List[int], seed: int = 42, shared_qkv: bool = False) -> Case:
    """TE 3333 reproduction: MHA H=8 d=128 bf16 causal, dout = ones.

    ``shared_qkv`` gives the literal q = k = v variant (one draw used three times).
    """
    rng = np.random.default_rng(seed)
    T, H, d = int(sum(lengths)), 8, 128
    q = _normal(rng, (T, H, d), BF16)
    if shared_qkv:
        k, v = q.clone(), q.clone()
    else:
        k = _normal(rng, (T, H, d), BF16)
        v = _normal(rng, (T, H, d), BF16)
    dout = torch.ones((T, H, d), dtype=torch.bfloat16)
    cu = _cu(lengths)
    return Case(name=f"mha_causal_{'_'.join(map(str, lengths))}", q=q, k=k, v=v, dout=dout,
                cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(), cu_seqlens_q_padded=cu.copy(),
                cu_seqlens_kv_padded=cu.copy(), scale=1.0 / math.sqrt(d), causal=True,
                dtype=BF16, max_seqlen_q=max(lengths), max_seqlen_kv=max(lengths))


REAL_LENGTHS = [100, 150, 120, 130]
PADDED_LENGTHS = [112, 160, 128, 144]


def real_vs_padded(total: int = 544, causal: bool = False, seed: int = 0) -> Case:
    """TE 2892 reproduction: real [100,150,120,130] inside padded [112,160,128,144].

    ``total`` = 544 is the sum of the padded slots; 576 adds 32 trailing rows
    that belong to no sequence.
    """
    assert total >= sum(PADDED_LENGTHS)
    rng = np.random.default_rng(seed)
    H, d = 32, 48
    q = _normal(rng, (total, H, d), BF16)
    k = _normal(rng, (total, H, d), BF16)
    v = _normal(rng, (total, H, d), BF16)
    dout = _normal(rng, (total, H, d), BF16)
    cu, cu_pad = _cu(REAL_LENGTHS), _cu(PADDED_LENGTHS)
    return Case(name=f"real_vs_padded_T{total}{'_causal' if causal else ''}", q=q, k=k, v=v,
                dout=dout, cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(), cu_seqlens_q_padded=cu_pad,
                cu_seqlens_kv_padded=cu_pad.copy(), scale=1.0 / math.sqrt(d), causal=causal,
                dtype=BF16, max_seqlen_q=max(REAL_LENGTHS), max_seqlen_kv=max(REAL_LENGTHS))


def gqa_d256_batched(outliers: bool = False, seed: int = 0) -> Case:
    """TE 3216 shape: sbhd [384,2,16,256] as THD [768,16,256], hkv=2, causal, scale 1/16."""
    rng = np.random.default_rng(seed)
    S, Bt, hq, hkv, d = 384, 2, 16, 2, 256
    T = S * Bt
    qf = rng.standard_normal(size=(T, hq, d), dtype=np.float32)
    kf = rng.standard_normal(size=(T, hkv, d), dtype=np.float32)
    vf = rng.standard_normal(size=(T, hkv, d), dtype=np.float32)
    dof = rng.standard_normal(size=(T, hq, d), dtype=np.float32)
    if outliers:
        G = hq // hkv
        for g in range(hkv):
            chans = rng.choice(d, size=4, replace=False)
            for c in chans:
                sign_q = rng.choice([-1.0, 1.0], size=(T, G)).astype(np.float32)
                sign_k = rng.choice([-1.0, 1.0], size=T).astype(np.float32)
                sign_v = rng.choice([-1.0, 1.0], size=T).astype(np.float32)
                qf[:, g * G:(g + 1) * G, c] = 8.0 * sign_q
                kf[:, g, c] = 8.0 * sign_k
                vf[:, g, c] = 8.0 * sign_v
    cast = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    cu = _cu([S] * Bt)
    return Case(name=f"gqa_d256{'_outliers' if outliers else ''}", q=cast(qf), k=cast(kf),
                v=cast(vf), dout=cast(dof), cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(),
                cu_seqlens_q_padded=cu.copy(), cu_seqlens_kv_padded=cu.copy(), scale=1.0 / 16.0,
                causal=True, dtype=BF16, max_seqlen_q=S, max_seqlen_kv=S)


def throughput_lengths(seed: int = 0, total: int = 65536, lo: int = 256, hi: int = 8192,
                       align: int = 64):
    """Real and padded lengths of the 65536-token throughput workload.

    Lengths are uniform in [lo, hi]; each slot is padded to a multiple of
    ``align``; the last slot takes whatever budget is left.
    """
    rng = np.random.default_rng(seed)
    real, padded, used = [], [], 0
    while used < total:
        L = int(rng.integers(lo, hi, endpoint=True))
        P = int(math.ceil(L / align) * align)
        if P > total - used:
            P = total - used
            L = min(L, P)
        real.append(L)
        padded.append(P)
        used += P
    return real, padded, rng


def throughput_65k(seed: int = 0, hq: int = 64, hkv: int = 8, d: int = 128,
                   heads_subset: Optional[int] = None) -> Case:
    """65536 packed tokens, seq lengths U[256,8192] padded to 64, hq=64 hkv=8 d=128 causal.

    ``heads_subset`` (a number of KV groups) draws only that many groups, for
    quick tests with the same length mix.
    """
    real, padded, rng = throughput_lengths(seed)
    T = sum(padded)
    if heads_subset is not None:
        hq, hkv = hq // hkv * heads_subset, heads_subset
    q = _normal(rng, (T, hq, d), BF16)
    k = _normal(rng, (T, hkv, d), BF16)
    v = _normal(rng, (T, hkv, d), BF16)
    dout = _normal(rng, (T, hq, d), BF16)
    cu, cu_pad = _cu(real), _cu(padded)
    return Case(name="throughput_65k" + (f"_g{heads_subset}" if heads_subset else ""),
                q=q, k=k, v=v, dout=dout, cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(),
                cu_seqlens_q_padded=cu_pad, cu_seqlens_kv_padded=cu_pad.copy(),
                scale=1.0 / math.sqrt(d), causal=True, dtype=BF16, max_seqlen_q=max(real),
                max_seqlen_kv=max(real))


def d64_65k(seed: int = 0) -> Case:
    """The throughput_65k sequences at head dim 64 (hq=64, hkv=8, bf16, causal)."""
    c = throughput_65k(seed, d=64)
    c.name = "d64_65k"
    return c


def d256_65k(seed: int = 0) -> Case:
    """The throughput_65k sequences at head dim 256 (hq=64, hkv=8, bf16, causal)."""
    c = throughput_65k(seed, d=256)
    c.name = "d256_65k"
    return c


def mqa_65k(seed: int = 0) -> Case:
    """The throughput_65k sequences with one KV head for 64 query heads (d=128,
    bf16, causal)."""
    c = throughput_65k(seed, hkv=1)
    c.name = "mqa_65k"
    return c


def large_offsets(seed: int = 0, device: str = "cuda") -> Case:
    """Tensors whose rows run past element 2^31: 260 slots of 1024 tokens (the
    last holding 1000 real tokens, 24 padding rows) and 64 trailing rows after
    the last slot, T = 266304, hq=64, hkv=8, d=128, bf16, ``padding_causal``,
    scale 1/sqrt(d).  q, dout (and the out / dq the call writes) hold 2.18e9
    elements, 4.36 GB each; every row from token 262144 on lies past element
    2^31 and byte 2^32 of them.

    The tensors are drawn on ``device`` with ``torch.Generator`` seeded with
    ``seed`` (N(0,1) in bf16; padding and trailing rows too, so a leak of them
    shows); callers copy the rows the oracle needs to the host.
    """
    slots, slot, last_real, trailing = 260, 1024, 1000, 64
    real = [slot] * (slots - 1) + [last_real]
    padded = [slot] * slots
    T = slots * slot + trailing
    hq, hkv, d = 64, 8, 128
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    draw = lambda *shape: torch.randn(shape, generator=gen, device=device, dtype=torch.bfloat16)
    q, k, v, dout = draw(T, hq, d), draw(T, hkv, d), draw(T, hkv, d), draw(T, hq, d)
    cu, cu_pad = _cu(real), _cu(padded)
    return Case(name="large_offsets", q=q, k=k, v=v, dout=dout, cu_seqlens_q=cu,
                cu_seqlens_kv=cu.copy(), cu_seqlens_q_padded=cu_pad,
                cu_seqlens_kv_padded=cu_pad.copy(), scale=1.0 / math.sqrt(d), causal=True,
                dtype=BF16, max_seqlen_q=slot, max_seqlen_kv=slot)


def sbhd_65k(seed: int = 0, S: int = 4096, B: int = 16, hq: int = 64, hkv: int = 8,
             d: int = 128) -> Case:
    """16 full sequences of 4096 tokens (65536 tokens), hq=64 hkv=8 d=128, bf16,
    padding_causal, in THD form (token i of sequence b is row b*S + i); the
    benchmark lays it out as sbhd [S, B, h, d] on the device."""
    rng = np.random.default_rng(seed)
    T = S * B
    q = _normal(rng, (T, hq, d), BF16)
    k = _normal(rng, (T, hkv, d), BF16)
    v = _normal(rng, (T, hkv, d), BF16)
    dout = _normal(rng, (T, hq, d), BF16)
    cu = _cu([S] * B)
    return Case(name="sbhd_65k", q=q, k=k, v=v, dout=dout, cu_seqlens_q=cu,
                cu_seqlens_kv=cu.copy(), cu_seqlens_q_padded=cu.copy(),
                cu_seqlens_kv_padded=cu.copy(), scale=1.0 / math.sqrt(d), causal=True,
                dtype=BF16, max_seqlen_q=S, max_seqlen_kv=S)


def chunked_bottom_right(seed: int = 0, chunk: int = 2048, total_kv: int = 65536,
                         lo: int = 2048, hi: int = 8192, hq: int = 64, hkv: int = 8,
                         d: int = 128) -> Case:
    """Query chunks against longer contexts, bottom-right causal: context
    lengths U[lo, hi] (seed) padded to 64 until total_kv tokens; each
    sequence's queries are its last min(chunk, Lk) tokens.  bf16, hq=64 hkv=8
    d=128."""
    real_k, pad_k, rng = throughput_lengths(seed, total=total_kv, lo=lo, hi=hi)
    real_q = [min(chunk, L) for L in real_k]
    pad_q = [int(math.ceil(L / 64) * 64) for L in real_q]
    Tq, Tk = sum(pad_q), sum(pad_k)
    q = _normal(rng, (Tq, hq, d), BF16)
    k = _normal(rng, (Tk, hkv, d), BF16)
    v = _normal(rng, (Tk, hkv, d), BF16)
    dout = _normal(rng, (Tq, hq, d), BF16)
    return Case(name="chunked_bottom_right", q=q, k=k, v=v, dout=dout,
                cu_seqlens_q=_cu(real_q), cu_seqlens_kv=_cu(real_k),
                cu_seqlens_q_padded=_cu(pad_q), cu_seqlens_kv_padded=_cu(pad_k),
                scale=1.0 / math.sqrt(d), causal="bottom_right", dtype=BF16,
                max_seqlen_q=max(real_q), max_seqlen_kv=max(real_k))


def causal_flops(cu_q: np.ndarray, cu_kv: np.ndarray, hq: int, d: int, causal: bool):
    """FLOP model of the headline metric: 4*d*hq*sum(Lq*Lkv), halved when causal.

    Returns (fwd, bwd = 2.5 * fwd).
    """
    lq = np.diff(np.asarray(cu_q, dtype=np.int64))
    lk = np.diff(np.asarray(cu_kv, dtype=np.int64))
    f = 4.0 * d * hq * float(np.sum(lq * lk))
    if causal:
        f *= 0.5
    return f, 2.5 * f
