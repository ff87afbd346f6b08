"""The forward and backward kernels are instantiated per product extent (the
head dim rounded up to 16, inside tiles 32, 64, 128, 192 or 256 columns
wide; the split kernels above 128 and, for dQ, above 192).  The plain path
is compared with the oracle at every head dim in tests/test_parity_gpu.py;
here the other kernel variants -- dropout, the GQA group spread over several
dK/dV workgroups (fp32 partial planes and their sum) and the accumulating
chunked backward -- are compared at head dims on both sides of each tile
width, each case run once through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

from helpers import (assert_close, assert_exact_zero_rows, assert_lse_close, check_case, f64,
                     oracle_run, real_rows)
from test_chunk_gpu import _run_chunked
from test_dropout_gpu import _case as drop_case, _gpu as drop_gpu, _oracle as drop_oracle
from test_split_group_gpu import _case as group_case, split_of

pytestmark = pytest.mark.gpu

# one past / at the end of each tile width and of the 16-column extents
DROP_DIMS = [56, 72, 104, 136, 168, 184, 200, 232, 248]


@pytest.mark.parametrize("d", DROP_DIMS)
def test_dropout_across_head_dims(d):
    causal = DROP_DIMS.index(d) % 2 == 0   # both masks across the tile widths
    dtype = "fp16" if d % 32 == 24 else "bf16"
    lq = [5, 130, 64, 0, 200]
    lk = lq if causal else [9, 70, 64, 12, 150]
    pq = [8, 130, 70, 4, 208]
    pk = [9, 133, 70, 12, 208]
    case = drop_case(lq, lk, pq, pk, hq=4, hkv=2, d=d, causal=causal, dtype=dtype, seed=300 + d)
    print(f"[headdim] dropout d={d} {dtype} causal={causal}", flush=True)
    drop = (0.15, 7 + d, 1)
    res, ref = drop_gpu(case, drop), drop_oracle(case, drop)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert_close("out", res[0], ref[0], dtype, qrows)
    assert_lse_close(res[1], ref[1], qrows)
    # gradients from the GPU forward's own O and LSE: the formula the kernels
    # evaluate (the exact-gradient comparison of dropout is in
    # tests/test_dropout_gpu.py)
    form = drop_oracle(case, drop, out=f64(res[0]), lse=f64(res[1]), mode="formula")
    assert_close("dq", res[2], form[2], dtype, qrows)
    assert_close("dk", res[3], form[3], dtype, krows)
    assert_close("dv", res[4], form[4], dtype, krows)
    for name, t, rows in (("out", res[0], ~qrows), ("dq", res[2], ~qrows),
                          ("dk", res[3], ~krows), ("dv", res[4], ~krows)):
        assert_exact_zero_rows(name, t, rows)


GROUP_DIMS = [72, 104, 136, 168, 200, 232]


@pytest.mark.parametrize("d", GROUP_DIMS)
def test_split_group_across_head_dims(d):
    causal = [True, False, "bottom_right"][GROUP_DIMS.index(d) % 3]
    dtype = "bf16" if d % 64 == 8 else "fp16"
    lq = [200, 0, 129, 64, 333]
    lk = [200, 40, 129, 64, 333] if causal is True else [150, 40, 200, 1, 300]
    pq = [208, 8, 136, 64, 340]
    pk = [208, 40, 136, 64, 333] if causal is True else [160, 40, 200, 8, 300]
    case = group_case(lq, lk, pq, pk, 16, 2, d, causal, dtype, seed=500 + d)
    split = split_of(case.batch, case.q.shape[0], case.k.shape[0], 16, 2, d)
    print(f"[headdim] split group d={d} {dtype} causal={causal} split={split}", flush=True)
    assert split > 1, split
    check_case(case)


CHUNK_DIMS = [(88, 4, 2), (152, 4, 2), (184, 16, 2), (216, 4, 2), (248, 16, 2)]


@pytest.mark.parametrize("d,hq,hkv", CHUNK_DIMS)
def test_accumulating_chunks_across_head_dims(d, hq, hkv):
    """Chunk pairs whose backward adds into dq / dk / dv; groups of 8 query
    heads also take the partial planes."""
    dtype = "bf16" if CHUNK_DIMS.index((d, hq, hkv)) % 2 == 0 else "fp16"
    print(f"[headdim] chunks d={d} hq={hq} hkv={hkv} {dtype}", flush=True)
    L = [300, 77, 513, 1]
    qcuts = [[128, 200], [40], [100, 256, 400], []]
    kcuts = [[64, 150, 299], [5], [256], []]
    case, res = _run_chunked(L, qcuts, kcuts, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=900 + d)
    o, l, dq, dk, dv = res
    ref_o, ref_l, *_ = oracle_run(case)
    rows = np.ones(case.q.shape[0], bool)
    assert_close("out", o, ref_o, dtype, rows)
    assert_lse_close(l, ref_l, rows)
    _, _, rdq, rdk, rdv = oracle_run(case, mode="formula", out=f64(o), lse=f64(l))
    assert_close("dq", dq, rdq, dtype, rows)
    assert_close("dk", dk, rdk, dtype, rows)
    assert_close("dv", dv, rdv, dtype, rows)
