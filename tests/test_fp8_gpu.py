"""GPU parity of the FP8-input forward (attn_fwd_thd_fp8).

The E4M3 decode is exact (every code is a bf16 / fp16 value): with one query
and one key the output is the value row itself, so O must equal the decoded
codes bit for bit for all 256 of them.  The forward on the FP8 page's THD
shape (TE-2892 "Reproduction": real [100,150,120,130] in padded
[112,160,128,144], 32 heads, d = 48, real != padded) and on a GQA d = 128 case
is compared with the oracle at the bar of the 16-bit output dtype.  The
backward from the same inputs (gradients with respect to the descaled values)
is compared with the oracle's on those shapes, and with power-of-two descales,
where every folded factor is an exact scaling, with the 16-bit backward on the
decoded values bit for bit.
"""
import numpy as np
import pytest
import torch

from helpers import assert_close, assert_lse_close, cu_dev, f64, real_rows
from oracle.fp8 import attn_bwd_fp8, attn_fwd_fp8, decode_e4m3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_decode_exact_for_every_code(out_dtype):
    import bwd_thd_varlen_amd as A
    d = 256
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(1, 1, d)
    q8 = torch.full((1, 1, d), 0x38, dtype=torch.uint8)     # 1.0
    cu = cu_dev([0, 1])
    o, l = A.fwd_fp8(q8.cuda(), q8.cuda(), codes.cuda(), 1.0, 1.0, 1.0, cu, cu,
                     out_dtype=out_dtype)
    want = decode_e4m3(codes.numpy())[0, 0]
    got = o.float().cpu().numpy()[0, 0]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # one key: LSE = its scaled score
    assert abs(float(l[0, 0]) - float(np.dot(np.ones(d), np.ones(d))) / np.sqrt(d)) < 1e-3


def _quantize(x: torch.Tensor):
    """Per-tensor E4M3 codes and descale (amax maps to 448)."""
    s = float(x.abs().max()) / 448.0
    return (x / s).to(torch.float8_e4m3fn).view(torch.uint8), s


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_fp8_real_vs_padded_te2892_shape(causal, out_dtype):
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(90)
    real, padded = [100, 150, 120, 130], [112, 160, 128, 144]
    T, H, d = sum(padded) + 32, 32, 48                     # 32 rows past every slot
    x = lambda: torch.from_numpy(rng.standard_normal((T, H, d), dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(x()), _quantize(x()), _quantize(x())
    cu = np.concatenate([[0], np.cumsum(real)]).astype(np.int32)
    cp = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    mask = "padding_causal" if causal else "padding"
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, cu_dev(cu), cu_dev(cu),
                     cu_dev(cp), cu_dev(cp), attn_mask_type=mask, out_dtype=out_dtype)
    ro, rl = attn_fwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, cu, cu, cp, cp,
                          causal=causal)
    rows = real_rows(cu, cp, T)
    dt = "bf16" if out_dtype == torch.bfloat16 else "fp16"
    assert_close("out", o, ro, dt, rows)
    assert_lse_close(l, rl, rows)
    assert int(torch.count_nonzero(o[torch.as_tensor(~rows, device="cuda")].float())) == 0
    assert bool(torch.all(torch.isneginf(l[torch.as_tensor(~rows, device="cuda")])))


def test_fp8_gqa_d128_bottom_right():
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(91)
    lq, lk = [64, 200, 33], [130, 200, 9]
    pq, pk = [64, 208, 40], [136, 200, 16]
    Tq, Tk = sum(pq), sum(pk)
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(g(Tq, 8, 128)), _quantize(g(Tk, 2, 128)), \
        _quantize(g(Tk, 2, 128))
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, cu_dev(cu(lq)), cu_dev(cu(lk)),
                     cu_dev(cu(pq)), cu_dev(cu(pk)), attn_mask_type="padding_causal_bottom_right")
    ro, rl = attn_fwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, cu(lq), cu(lk),
                          cu(pq), cu(pk), causal="bottom_right")
    rows = real_rows(cu(lq), cu(pq), Tq, cu(lk))
    assert_close("out", o, ro, "bf16", rows)
    assert_lse_close(l, rl, rows)


@pytest.mark.parametrize("d,causal", [(48, True), (64, False), (80, True), (96, False),
                                      (128, True), (176, False), (256, True)])
def test_fp8_scores_on_8bit_products(d, causal):
    """Head dims 48..256 (multiples of 16) take the scores on the E4M3 MFMA, in
    64-code chunks of the head dim (48, 80, 176: the last chunk part zeros)."""
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(92 + d)
    L, P = [1, 77, 300, 129], [8, 80, 300, 136]
    T = sum(P)
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(g(T, 8, d)), _quantize(g(T, 2, d)), \
        _quantize(g(T, 2, d))
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cp = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    mask = "padding_causal" if causal else "padding"
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, cu_dev(cu), cu_dev(cu),
                     cu_dev(cp), cu_dev(cp), attn_mask_type=mask)
    ro, rl = attn_fwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, cu, cu, cp, cp,
                          causal=causal)
    rows = real_rows(cu, cp, T)
    assert_close("out", o, ro, "bf16", rows)
    assert_lse_close(l, rl, rows)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_paths_agree(d):
    """The 8-bit-product path and the decode path (taken when the codes are only
    8-byte aligned) compute the same scores up to summation order."""
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(99 + d)
    L = [200, 57]
    T = sum(L)
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(g(T, 4, d)), _quantize(g(T, 4, d)), \
        _quantize(g(T, 4, d))
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]))
    o1, l1 = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, cu, cu,
                       attn_mask_type="padding_causal")
    buf = torch.zeros(q8.numel() + 16, dtype=torch.uint8, device="cuda")
    q8m = buf[8:8 + q8.numel()].view(q8.shape)          # 8-byte aligned only
    q8m.copy_(q8.cuda())
    o2, l2 = A.fwd_fp8(q8m, k8.cuda(), v8.cuda(), sq, sk, sv, cu, cu,
                       attn_mask_type="padding_causal")
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2 * o2.float().abs().max().item()
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("d,causal", [(16, True), (40, False), (136, True), (248, True)])
def test_fp8_decode_path_head_dims(d, causal):
    """Head dims up to 32, and those that are not multiples of 16, decode q, k,
    v exactly and run the 16-bit forward: parity at the bar of the output dtype."""
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(200 + d)
    L, P = [3, 90, 200], [8, 96, 200]
    T = sum(P)
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(g(T, 4, d)), _quantize(g(T, 2, d)), \
        _quantize(g(T, 2, d))
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cp = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    mask = "padding_causal" if causal else "padding"
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, cu_dev(cu), cu_dev(cu),
                     cu_dev(cp), cu_dev(cp), attn_mask_type=mask)
    ro, rl = attn_fwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, cu, cu, cp, cp,
                          causal=causal)
    rows = real_rows(cu, cp, T)
    assert_close("out", o, ro, "bf16", rows)
    assert_lse_close(l, rl, rows)
    assert int(torch.count_nonzero(o[torch.as_tensor(~rows, device="cuda")].float())) == 0


# ---------------------------------------------------------------- backward
def _bwd_case(rng, lq, lk, pq, pk, hq, hkv, d, extra=0):
    Tq, Tk = sum(pq) + extra, sum(pk) + extra
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    (q8, sq), (k8, sk), (v8, sv) = _quantize(g(Tq, hq, d)), _quantize(g(Tk, hkv, d)), \
        _quantize(g(Tk, hkv, d))
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    return q8, k8, v8, sq, sk, sv, g(Tq, hq, d), (cu(lq), cu(lk), cu(pq), cu(pk)), (Tq, Tk)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [48, 128])
def test_fp8_backward_te2892_shape(causal, out_dtype, d):
    """The TE-2892 lengths (real != padded, 32 rows past every slot) at its head
    dim 48 and at 128 (8 heads), with and without the causal mask."""
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(95 + d)
    real, padded = [100, 150, 120, 130], [112, 160, 128, 144]
    h = 32 if d == 48 else 8
    q8, k8, v8, sq, sk, sv, do, cus, (Tq, Tk) = _bwd_case(rng, real, real, padded, padded, h,
                                                          h, d, extra=32)
    mask = "padding_causal" if causal else "padding"
    print(f"[fp8 bwd] te2892 shape causal={causal} {out_dtype} d={d}", flush=True)
    dev = [cu_dev(c) for c in cus]
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, *dev, attn_mask_type=mask,
                     out_dtype=out_dtype)
    dout = do.to(out_dtype)
    dq, dk, dv = A.bwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, o, dout.cuda(), l, *dev,
                           attn_mask_type=mask)
    rdq, rdk, rdv = attn_bwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, f64(dout), *cus,
                                 causal=causal)
    dt = "bf16" if out_dtype == torch.bfloat16 else "fp16"
    rq, rk = real_rows(cus[0], cus[2], Tq), real_rows(cus[1], cus[3], Tk)
    assert_close("dq", dq, rdq, dt, rq)
    assert_close("dk", dk, rdk, dt, rk)
    assert_close("dv", dv, rdv, dt, rk)
    for t, rows in ((dq, rq), (dk, rk), (dv, rk)):
        assert int(torch.count_nonzero(t[torch.as_tensor(~rows, device="cuda")].float())) == 0


def test_fp8_backward_gqa_d128_bottom_right():
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(96)
    q8, k8, v8, sq, sk, sv, do, cus, (Tq, Tk) = _bwd_case(
        rng, [64, 200, 33, 0], [130, 200, 9, 5], [64, 208, 40, 8], [136, 200, 16, 8], 8, 2, 128)
    print("[fp8 bwd] gqa d128 bottom_right", flush=True)
    dev = [cu_dev(c) for c in cus]
    mask = "padding_causal_bottom_right"
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, *dev, attn_mask_type=mask)
    dout = do.to(torch.bfloat16)
    dq, dk, dv = A.bwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, o, dout.cuda(), l, *dev,
                           attn_mask_type=mask)
    rdq, rdk, rdv = attn_bwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, f64(dout), *cus,
                                 causal="bottom_right")
    rq, rk = real_rows(cus[0], cus[2], Tq, cus[1]), real_rows(cus[1], cus[3], Tk, cus[0])
    assert_close("dq", dq, rdq, "bf16", rq)
    assert_close("dk", dk, rdk, "bf16", rk)
    assert_close("dv", dv, rdv, "bf16", rk)
    # the sequence with no queries: its key rows get zero gradients
    assert int(torch.count_nonzero(dk[~torch.as_tensor(rk, device="cuda")].float())) == 0


@pytest.mark.parametrize("dtype,sv", [(torch.bfloat16, 2.0 ** -5), (torch.float16, 1.0)])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_backward_bitwise_16bit_with_power_of_two_descales(dtype, sv, d):
    """Power-of-two descales make every folded factor an exact scaling, so the FP8
    backward equals the 16-bit backward on the decoded, descaled values bit for bit
    (fp16 keeps descale_v = 1: scaling dS there would move values across fp16's
    subnormal boundary)."""
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(97 + d)
    L, P = [1, 77, 300, 129], [8, 80, 300, 136]
    T = sum(P)
    sq, sk = 2.0 ** -4, 2.0 ** -3
    g = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
    f8 = lambda x, s_: (x / s_).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    q8, k8, v8 = f8(g(T, 8, d), sq), f8(g(T, 2, d), sk), f8(g(T, 2, d) * 4, sv)
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cp = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    dev = [cu_dev(cu), cu_dev(cu), cu_dev(cp), cu_dev(cp)]
    print(f"[fp8 bwd] bitwise {dtype} d={d}", flush=True)
    o, l = A.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, *dev,
                     attn_mask_type="padding_causal", out_dtype=dtype)
    dout = g(T, 8, d).to(dtype).cuda()
    got = A.bwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, o, dout, l, *dev,
                    attn_mask_type="padding_causal")
    dec = lambda c, s_: (c.view(torch.float8_e4m3fn).to(torch.float32) * s_).to(dtype).cuda()
    want = A.bwd(dec(q8, sq), dec(k8, sk), dec(v8, sv), o, dout, l, *dev[:2],
                 cu_seqlens_q_padded=dev[2], cu_seqlens_kv_padded=dev[3],
                 attn_mask_type="padding_causal")
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(a, b), name
