"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad host arguments before
launching anything (no GPU is touched on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_thd.h")


@pytest.fixture(scope="module")
def A():
    import bwd_thd_varlen_amd as A
    A.lib()
    return A


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd_thd", "attn_bwd_thd", "attn_thd_workspace_size", "attn_thd_status_string",
              "attn_thd_read_device_status"):
        assert n in names


def test_library_exports_every_declared_symbol(A):
    lib = A.lib()
    for n in declared_functions():
        assert hasattr(lib, n), f"missing export {n}"


def test_status_strings(A):
    for code in range(5):
        assert A.status_string(code)
    assert A.status_string(99) == "unknown status"


def test_workspace_size(A):
    ws = A.workspace_size(16, 65536, 65536, 64, 8, 128)
    # Delta alone is total_q * hq * 4 bytes
    assert ws >= 65536 * 64 * 4
    assert ws % 256 == 0
    assert A.workspace_size(-1, 10, 10, 1, 1, 8) == 0
    assert A.workspace_size(0, 0, 0, 1, 1, 8) > 0


FAKE = 1 << 20   # never dereferenced: every call below fails validation first


def fwd_call(A, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, cu_seqlens_q=FAKE,
                cu_seqlens_kv=FAKE, cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None, batch=2,
                total_q=16, total_kv=16, max_seqlen_q=8, max_seqlen_kv=8, hq=4, hkv=2, d=64,
                scale=0.125, mask_type=0, dtype=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return A.attn_fwd_thd(**args)


@pytest.mark.parametrize("over,code", [
    (dict(hq=4, hkv=3), 1),                 # hkv does not divide hq
    (dict(hq=0), 1),
    (dict(batch=-1), 1),
    (dict(total_q=-5), 1),
    (dict(d=12), 2),                        # not a multiple of 8
    (dict(d=264), 2),                       # above 256
    (dict(dtype=7), 2),
    (dict(mask_type=3), 2),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(cu_seqlens_q=None), 1),
    (dict(q=None), 1),
    (dict(workspace=None), 3),              # every other argument fine
    (dict(workspace=FAKE, workspace_bytes=16), 3),
    (dict(workspace=FAKE + 8, workspace_bytes=1 << 30), 3),   # misaligned
])
def test_fwd_rejects_bad_host_arguments(A, over, code):
    assert fwd_call(A, **over) == code


def test_bwd_rejects_bad_host_arguments(A):
    base = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                cu_seqlens_q=FAKE, cu_seqlens_kv=FAKE, cu_seqlens_q_padded=None,
                cu_seqlens_kv_padded=None, batch=2, total_q=16, total_kv=16, max_seqlen_q=8,
                max_seqlen_kv=8, hq=4, hkv=2, d=64, scale=0.125, mask_type=1, dtype=1,
                workspace=None, workspace_bytes=0, stream=None)
    assert A.attn_bwd_thd(**dict(base, hkv=3)) == 1
    assert A.attn_bwd_thd(**dict(base, d=4)) == 2
    assert A.attn_bwd_thd(**base) == 3
    assert A.attn_bwd_thd(**dict(base, dk=None, workspace=FAKE, workspace_bytes=1 << 30)) == 1
    assert A.attn_bwd_thd(**dict(base, dout=None, workspace=FAKE, workspace_bytes=1 << 30)) == 1


def test_product_has_no_cpu_fallback():
    """The binding loads only the HIP library; it never imports the oracle."""
    src = open(os.path.join(ROOT, "bwd_thd_varlen_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("the CPU oracle", "")
    for f in os.listdir(os.path.join(ROOT, "bwd_thd_varlen_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "bwd_thd_varlen_amd", "csrc", f)).read()


def test_bottom_right_mask_is_accepted(A):
    # mask_type 2 passes validation: the call fails only at the missing workspace
    assert fwd_call(A, mask_type=2) == 3


def batched_fwd_call(A, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, cu_seqlens_q=None,
                cu_seqlens_kv=None, layout=2, batch=2, seqlen_q=8, seqlen_kv=8, hq=4, hkv=2,
                d=64, scale=0.125, mask_type=1, dtype=0, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(over)
    return A.attn_fwd_batched(**args)


@pytest.mark.parametrize("over,code", [
    (dict(), 3),                                # NULL real lengths are fine (full slots)
    (dict(layout=1), 3),
    (dict(layout=0), 2),                        # THD goes through attn_fwd_thd
    (dict(layout=3), 2),
    (dict(seqlen_q=-1), 1),
    (dict(batch=1 << 16, seqlen_q=1 << 16), 1),  # batch * seqlen above INT32_MAX
    (dict(batch=1 << 15, hq=64, hkv=8, d=128), 1),  # a strided 256-token tile spans > 2 GiB
    (dict(hq=4, hkv=3), 1),
    (dict(d=12), 2),
])
def test_batched_rejects_bad_host_arguments(A, over, code):
    assert batched_fwd_call(A, **over) == code


def test_batched_bwd_rejects_bad_host_arguments(A):
    base = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                cu_seqlens_q=None, cu_seqlens_kv=None, layout=1, batch=2, seqlen_q=8,
                seqlen_kv=8, hq=4, hkv=2, d=64, scale=0.125, mask_type=0, dtype=1,
                workspace=None, workspace_bytes=0, stream=None)
    assert A.attn_bwd_batched(**base) == 3
    assert A.attn_bwd_batched(**dict(base, layout=5)) == 2
    assert A.attn_bwd_batched(**dict(base, dq=None, workspace=FAKE, workspace_bytes=1 << 30)) == 1


def test_chunk_entry_points_reject_bad_host_arguments(A):
    base = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, cu_q=FAKE, cu_kv=FAKE, cu_qp=None,
                cu_kp=None, q_pos0=FAKE, kv_pos0=None, batch=2, total_q=16, total_kv=16, hq=4,
                hkv=2, d=64, scale=0.125, mask=1, dtype=0, ws=None, wsb=0, stream=None,
                events=None, n_events=0)
    call = lambda **o: A.attn_fwd_thd_chunk(*dict(base, **o).values())
    assert call() == 3                        # positions with the causal mask: fine
    assert call(mask=0) == 1                  # positions need the causal mask
    assert call(mask=2) == 1
    assert call(q_pos0=None, mask=2) == 3     # no positions: any mask
    bb = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
              cu_q=FAKE, cu_kv=FAKE, cu_qp=None, cu_kp=None, q_pos0=None, kv_pos0=FAKE, batch=2,
              total_q=16, total_kv=16, hq=4, hkv=2, d=64, scale=0.125, mask=1, acc=1, dtype=0,
              ws=None, wsb=0, stream=None, events=None, n_events=0)
    bcall = lambda **o: A.attn_bwd_thd_chunk(*dict(bb, **o).values())
    assert bcall() == 3
    assert bcall(acc=2) == 3
    assert bcall(acc=3) == 3
    assert bcall(acc=4) == 1
    assert bcall(mask=0) == 1


@pytest.mark.parametrize("over,code", [
    (dict(total_q=-1), 1), (dict(hq=0), 1), (dict(d=12), 2), (dict(d=512), 2),
    (dict(dtype=5), 2), (dict(out=None), 1), (dict(lse_part=FAKE + 2), 1),
    (dict(out_part=FAKE + 8), 1), (dict(total_q=1 << 20, hq=4096), 1),
])
def test_merge_rejects_bad_host_arguments(A, over, code):
    args = dict(out=FAKE, lse=FAKE, out_part=FAKE, lse_part=FAKE, total_q=16, hq=4, d=64, dtype=0,
                stream=None)
    args.update(over)
    assert A.attn_merge_thd(**args) == code


@pytest.mark.parametrize("p,code", [(0.1, 3), (0.0, 3), (0.99, 3), (-0.1, 1), (1.0, 1),
                                    (float("nan"), 1), (0.999, 1)])
def test_dropout_probability_range(A, p, code):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 2, 16, 16, 4, 2, 64, 0.125, 1,
            p, 1234, 0, 0, None, 0, None, None, 0]
    assert A.attn_fwd_thd_dropout(*args) == code
    bargs = [FAKE] * 9 + [FAKE, FAKE, None, None, 2, 16, 16, 4, 2, 64, 0.125, 1, p, 1234, 0, 0,
                          None, 0, None, None, 0]
    assert A.attn_bwd_thd_dropout(*bargs) == code


@pytest.mark.parametrize("over,code", [
    (dict(), 3), (dict(sq=0.0), 1), (dict(sv=float("inf")), 1), (dict(sk=-1.0), 1),
    (dict(q8=FAKE + 4), 1), (dict(d=12), 2), (dict(out_dtype=9), 2), (dict(mask=4), 2),
    (dict(hq=4, hkv=3), 1),
])
def test_fp8_forward_rejects_bad_host_arguments(A, over, code):
    args = dict(q8=FAKE, k8=FAKE, v8=FAKE, sq=0.5, sk=0.5, sv=2.0, out=FAKE, lse=FAKE,
                cu_q=FAKE, cu_kv=FAKE, cu_qp=None, cu_kp=None, batch=2, total_q=16, total_kv=16,
                hq=4, hkv=2, d=64, scale=0.125, mask=1, out_dtype=0, ws=None, wsb=0, stream=None,
                events=None, n_events=0)
    args.update(over)
    assert A.attn_fwd_thd_fp8(*args.values()) == code


@pytest.mark.parametrize("over,code", [
    (dict(), 3), (dict(sq=0.0), 1), (dict(sv=float("nan")), 1), (dict(sk=-1.0), 1),
    (dict(sv=1e-39), 1), (dict(sq=1e30, sv=1e30), 1), (dict(v8=FAKE + 2), 1), (dict(d=12), 2),
    (dict(dtype=9), 2), (dict(mask=4), 2), (dict(hq=4, hkv=3), 1), (dict(dq=FAKE + 8), 1),
    (dict(dout=None), 1), (dict(n_events=6), 1), (dict(n_events=7), 3),
])
def test_fp8_backward_rejects_bad_host_arguments(A, over, code):
    """Host-checkable errors return before anything is enqueued (no GPU is touched).
    With no workspace the size check answers first; with the plain backward's
    workspace (smaller than the FP8 one) the pointer and event checks are reached."""
    ev = (ctypes.c_void_p * 7)()
    args = dict(q8=FAKE, k8=FAKE, v8=FAKE, sq=0.5, sk=0.5, sv=2.0, out=FAKE, dout=FAKE, lse=FAKE,
                dq=FAKE, dk=FAKE, dv=FAKE, cu_q=FAKE, cu_kv=FAKE, cu_qp=None, cu_kp=None, batch=2,
                total_q=16, total_kv=16, hq=4, hkv=2, d=64, scale=0.125, mask=1, dtype=0,
                ws=None, wsb=0, stream=None, events=None, n_events=0)
    args.update(over)
    if "dq" in over or "dout" in over or "n_events" in over:
        args["ws"], args["wsb"] = FAKE, A.workspace_size(2, 16, 16, 4, 2, 64)
    if "n_events" in over:
        args["events"] = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    assert A.attn_bwd_thd_fp8(*args.values()) == code


def test_fp8_workspace_is_larger(A):
    assert A.fp8_workspace_size(2, 100, 80, 8, 2, 64) >= \
        A.workspace_size(2, 100, 80, 8, 2, 64) + (100 * 8 + 2 * 80 * 2) * 64 * 2


def test_output_shape_checked_before_anything_else(A):
    """Outputs reach the kernels as raw pointers, so the binding checks their
    shapes first: an undersized out / lse / dq / dk / dv must raise, not be
    written past its end."""
    import torch
    t = torch.empty((10, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(A.AttnError, match="shape"):
        A._need(t, "out", torch.bfloat16, None, (12, 4, 64))
    with pytest.raises(A.AttnError, match="shape"):
        A._need(torch.empty((10, 3), dtype=torch.float32), "lse", torch.float32, None, (10, 4))
    # the right shape gets past the shape check (and stops at the device check on the CPU)
    with pytest.raises(A.AttnError, match="GPU"):
        A._need(t, "out", torch.bfloat16, None, (10, 4, 64))


def test_noalloc_rejects_oversized_and_invalid_problems(A):
    """attn_bwd_thd_noalloc refuses, before any HIP call, a problem whose
    workspace exceeds its static scratch (ATTN_THD_ESCRATCH) and invalid sizes."""
    args = lambda **o: [dict(FAKE_ARGS, **o)[n] for n in NOALLOC_ORDER]
    big_tq, hq = 1 << 20, 16    # Delta and LSE rows alone: 2 x 4 B x 2^24 = 128 MiB
    assert A.workspace_size(1, big_tq, big_tq, hq, 1, 64) > A.NOALLOC_SCRATCH_BYTES
    assert A.attn_bwd_thd_noalloc(*args(total_q=big_tq, total_kv=big_tq, hq=hq)) == 5
    assert A.attn_bwd_thd_noalloc(*args(hq=0)) == 1
    assert A.attn_bwd_thd_noalloc(*args(batch=-1)) == 1
    assert A.status_string(5).startswith("problem exceeds")


NOALLOC_ORDER = ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "cu_q", "cu_kv", "cu_qp",
                 "cu_kp", "batch", "total_q", "total_kv", "max_q", "max_kv", "hq", "hkv", "d",
                 "scale", "mask", "dtype", "stream"]
FAKE_ARGS = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                 cu_q=FAKE, cu_kv=FAKE, cu_qp=None, cu_kp=None, batch=1, total_q=16, total_kv=16,
                 max_q=0, max_kv=0, hq=1, hkv=1, d=64, scale=0.125, mask=0, dtype=0, stream=None)


def test_split_group_workspace_rule(A):
    """Groups of 8 or more query heads with few key tiles get fp32 partial
    dK / dV planes (2 x split x total_kv x hkv x d) in the workspace: split
    doubles while it divides the group, leaves every workgroup at least 2 of
    its heads, and the dK/dV workgroups (key tiles of 128 plus one per
    sequence, times hkv) stay below 4096.  Read off the size's growth with d,
    the only term that depends on it."""
    def split(batch, t, hq, hkv, d=128):
        grow = A.workspace_size(batch, t, t, hq, hkv, d) - A.workspace_size(batch, t, t, hq, hkv, d - 8)
        return round(grow / (2 * t * hkv * 8 * 4))
    assert split(16, 65536, 64, 1) == 8      # 528 workgroups -> 4224
    assert split(16, 65536, 64, 2) == 4      # 1056 -> 4224
    assert split(16, 65536, 64, 4) == 2      # 2112 -> 4224
    assert split(16, 65536, 64, 8) == 0      # 4224 workgroups already: no partial planes
    assert split(8, 16384, 64, 1) == 32      # 136 -> 4352, below the group of 64
    assert split(4, 1000, 4, 1) == 0         # a group of 4: never split
    assert split(4, 1000, 24, 1) == 8        # 24 = 8 x 3: doubling stops where 2 split no longer divides
    assert split(4, 1000, 8, 1) == 4         # a group of 8: 2 heads per workgroup at most split
    assert split(4, 1000, 16, 1) == 8
