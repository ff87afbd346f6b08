"""MI355X (gfx950) fused attention over packed variable-length THD sequences.

A thin ctypes binding of ``libattn_thd.so`` (C ABI in ``include/attn_thd.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments: PyTorch supplies device memory (outputs and the
workspace are ``torch.empty``) and the current stream.  There is no fallback:
if the library is missing or fails to load, every call raises.

Names follow TransformerEngine's ``DotProductAttention`` / ``fused_attn_bwd``
arguments (``cu_seqlens_q``, ``cu_seqlens_kv``, ``cu_seqlens_q_padded``,
``cu_seqlens_kv_padded``, ``max_seqlen_q``, ``max_seqlen_kv``,
``attn_mask_type`` in {"padding", "padding_causal",
"padding_causal_bottom_right"}: the causal triangle top-left aligned, key
j <= query i, or aligned at the sequence ends, j <= i + Lk - Lq).
``fwd_batched`` / ``bwd_batched`` read bshd ``[b, s, h, d]`` and sbhd
``[s, b, h, d]`` tensors in place through the same kernels; ``attention_thd``
is the forward and backward as one ``torch.autograd`` op.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["lib", "lib_path", "workspace_size", "attn_fwd_thd", "attn_bwd_thd",
           "attn_fwd_thd_timed", "attn_bwd_thd_timed", "fwd", "bwd", "status_string",
           "read_device_status", "AttnError", "STATUS", "DEV_BAD_SEQLENS", "StageEvents",
           "FWD_STAGES", "BWD_STAGES", "attn_fwd_batched", "attn_bwd_batched", "fwd_batched",
           "bwd_batched", "LAYOUTS", "attn_fwd_thd_chunk", "attn_bwd_thd_chunk",
           "attn_merge_thd", "fwd_chunk", "bwd_chunk", "merge", "attn_fwd_thd_dropout",
           "attn_bwd_thd_dropout", "attention_thd", "attn_fwd_thd_fp8", "fwd_fp8",
           "fp8_workspace_size", "attn_bwd_thd_fp8", "bwd_fp8", "attn_bwd_thd_noalloc",
           "bwd_noalloc", "NOALLOC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_THD_LIB: another build of the same library (e.g. for A/B timing runs)
_LIB_PATH = os.environ.get("ATTN_THD_LIB") or os.path.join(_HERE, "libattn_thd.so")
_LIB = None

STATUS = {0: "ATTN_THD_OK", 1: "ATTN_THD_EINVAL", 2: "ATTN_THD_EUNSUPPORTED",
          3: "ATTN_THD_EWORKSPACE", 4: "ATTN_THD_ELAUNCH", 5: "ATTN_THD_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20    # ATTN_THD_NOALLOC_SCRATCH_BYTES
DEV_BAD_SEQLENS = 1
_DTYPE = {torch.bfloat16: 0, torch.float16: 1}
_MASK = {"padding": 0, "padding_causal": 1, "padding_causal_bottom_right": 2}
LAYOUTS = {"bshd": 1, "sbhd": 2}
ACC_DQ, ACC_DKDV = 1, 2     # accumulate bits of attn_bwd_thd_chunk

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
_FWD_ARGS = [_P, _P, _P, _P, _P,          # q k v out lse
             _P, _P, _P, _P,              # cu_q cu_kv cu_q_pad cu_kv_pad
             _I, _I, _I, _I, _I,          # batch total_q total_kv max_q max_kv
             _I, _I, _I, _F, _I, _I,      # hq hkv d scale mask dtype
             _P, _S, _P]                  # workspace bytes stream
FWD_STAGES = ("sched", "fwd", "zero_fill_q")
BWD_STAGES = ("sched", "dq", "dkdv", "zero_fill_q", "zero_fill_kv")
FP8_FWD_STAGES = ("decode",) + FWD_STAGES
FP8_BWD_STAGES = ("decode",) + BWD_STAGES
_BWD_ARGS = [_P, _P, _P, _P, _P, _P,      # q k v out dout lse
             _P, _P, _P,                  # dq dk dv
             _P, _P, _P, _P,
             _I, _I, _I, _I, _I,
             _I, _I, _I, _F, _I, _I,
             _P, _S, _P]


_BFWD_ARGS = [_P, _P, _P, _P, _P,         # q k v out lse
              _P, _P, _I,                 # cu_q cu_kv layout
              _I, _I, _I,                 # batch seqlen_q seqlen_kv
              _I, _I, _I, _F, _I, _I,     # hq hkv d scale mask dtype
              _P, _S, _P]                 # workspace bytes stream
_BBWD_ARGS = [_P, _P, _P, _P, _P, _P,     # q k v out dout lse
              _P, _P, _P,                 # dq dk dv
              _P, _P, _I,
              _I, _I, _I,
              _I, _I, _I, _F, _I, _I,
              _P, _S, _P]


_CFWD_ARGS = [_P, _P, _P, _P, _P,         # q k v out lse
              _P, _P, _P, _P, _P, _P,     # cu_q cu_kv cu_q_pad cu_kv_pad q_pos0 kv_pos0
              _I, _I, _I,                 # batch total_q total_kv
              _I, _I, _I, _F, _I, _I,     # hq hkv d scale mask dtype
              _P, _S, _P, ctypes.POINTER(_P), _I]   # workspace bytes stream events n_events
_CBWD_ARGS = [_P, _P, _P, _P, _P, _P,     # q k v out dout lse
              _P, _P, _P,                 # dq dk dv
              _P, _P, _P, _P, _P, _P,
              _I, _I, _I,
              _I, _I, _I, _F, _I, _I, _I,  # hq hkv d scale mask accumulate dtype
              _P, _S, _P, ctypes.POINTER(_P), _I]


_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32
_DFWD_ARGS = [_P, _P, _P, _P, _P,         # q k v out lse
              _P, _P, _P, _P,             # cu_q cu_kv cu_q_pad cu_kv_pad
              _I, _I, _I,                 # batch total_q total_kv
              _I, _I, _I, _F, _I,         # hq hkv d scale mask
              _F, _U64, _U32, _I,         # dropout_p seed offset dtype
              _P, _S, _P, ctypes.POINTER(_P), _I]
_DBWD_ARGS = [_P, _P, _P, _P, _P, _P,     # q k v out dout lse
              _P, _P, _P,                 # dq dk dv
              _P, _P, _P, _P,
              _I, _I, _I,
              _I, _I, _I, _F, _I,
              _F, _U64, _U32, _I,
              _P, _S, _P, ctypes.POINTER(_P), _I]


class AttnError(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Loads libattn_thd.so (built in-tree by ``python -m bwd_thd_varlen_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise AttnError(f"{_LIB_PATH} is not built: run `python -m bwd_thd_varlen_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.attn_thd_workspace_size.argtypes = [_I] * 6
        L.attn_thd_workspace_size.restype = _S
        L.attn_fwd_thd.argtypes = _FWD_ARGS
        L.attn_fwd_thd.restype = ctypes.c_int
        L.attn_bwd_thd.argtypes = _BWD_ARGS
        L.attn_bwd_thd.restype = ctypes.c_int
        L.attn_fwd_thd_timed.argtypes = _FWD_ARGS + [ctypes.POINTER(_P), _I]
        L.attn_fwd_thd_timed.restype = ctypes.c_int
        L.attn_bwd_thd_timed.argtypes = _BWD_ARGS + [ctypes.POINTER(_P), _I]
        L.attn_bwd_thd_timed.restype = ctypes.c_int
        L.attn_fwd_batched.argtypes = _BFWD_ARGS
        L.attn_fwd_batched.restype = ctypes.c_int
        L.attn_bwd_batched.argtypes = _BBWD_ARGS
        L.attn_bwd_batched.restype = ctypes.c_int
        L.attn_fwd_batched_timed.argtypes = _BFWD_ARGS + [ctypes.POINTER(_P), _I]
        L.attn_fwd_batched_timed.restype = ctypes.c_int
        L.attn_bwd_batched_timed.argtypes = _BBWD_ARGS + [ctypes.POINTER(_P), _I]
        L.attn_bwd_batched_timed.restype = ctypes.c_int
        L.attn_fwd_thd_chunk.argtypes = _CFWD_ARGS
        L.attn_fwd_thd_chunk.restype = ctypes.c_int
        L.attn_bwd_thd_chunk.argtypes = _CBWD_ARGS
        L.attn_bwd_thd_chunk.restype = ctypes.c_int
        L.attn_merge_thd.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P]
        L.attn_merge_thd.restype = ctypes.c_int
        L.attn_thd_fp8_workspace_size.argtypes = [_I] * 6
        L.attn_thd_fp8_workspace_size.restype = _S
        L.attn_fwd_thd_fp8.argtypes = [_P, _P, _P, _F, _F, _F, _P, _P, _P, _P, _P, _P,
                                       _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P,
                                       ctypes.POINTER(_P), _I]
        L.attn_fwd_thd_fp8.restype = ctypes.c_int
        L.attn_bwd_thd_fp8.argtypes = [_P, _P, _P, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P,
                                       ctypes.POINTER(_P), _I]
        L.attn_bwd_thd_fp8.restype = ctypes.c_int
        L.attn_fwd_thd_dropout.argtypes = _DFWD_ARGS
        L.attn_fwd_thd_dropout.restype = ctypes.c_int
        L.attn_bwd_thd_dropout.argtypes = _DBWD_ARGS
        L.attn_bwd_thd_dropout.restype = ctypes.c_int
        L.attn_bwd_thd_noalloc.argtypes = _BWD_ARGS[:-3] + [_P]   # no workspace arguments
        L.attn_bwd_thd_noalloc.restype = ctypes.c_int
        L.attn_thd_status_string.argtypes = [_I]
        L.attn_thd_status_string.restype = ctypes.c_char_p
        L.attn_thd_read_device_status.argtypes = [_P, _P, ctypes.POINTER(_I)]
        L.attn_thd_read_device_status.restype = ctypes.c_int
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().attn_thd_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise AttnError(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


# ----------------------------------------------------------------- raw C-ABI mirrors
def workspace_size(batch: int, total_q: int, total_kv: int, hq: int, hkv: int, d: int) -> int:
    return int(lib().attn_thd_workspace_size(batch, total_q, total_kv, hq, hkv, d))


def attn_fwd_thd(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                 cu_seqlens_kv_padded, batch, total_q, total_kv, max_seqlen_q, max_seqlen_kv,
                 hq, hkv, d, scale, mask_type, dtype, workspace, workspace_bytes, stream) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_fwd_thd(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv,
                                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q,
                                  total_kv, max_seqlen_q, max_seqlen_kv, hq, hkv, d, scale,
                                  mask_type, dtype, workspace, workspace_bytes, stream))


def attn_bwd_thd(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                 cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv,
                 max_seqlen_q, max_seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                 workspace_bytes, stream) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_bwd_thd(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q,
                                  cu_seqlens_kv, cu_seqlens_q_padded, cu_seqlens_kv_padded, batch,
                                  total_q, total_kv, max_seqlen_q, max_seqlen_kv, hq, hkv, d,
                                  scale, mask_type, dtype, workspace, workspace_bytes, stream))


def attn_fwd_batched(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, layout, batch, seqlen_q,
                     seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace, workspace_bytes,
                     stream) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_fwd_batched(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, layout,
                                      batch, seqlen_q, seqlen_kv, hq, hkv, d, scale, mask_type,
                                      dtype, workspace, workspace_bytes, stream))


def attn_bwd_batched(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv, layout,
                     batch, seqlen_q, seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                     workspace_bytes, stream) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_bwd_batched(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q,
                                      cu_seqlens_kv, layout, batch, seqlen_q, seqlen_kv, hq, hkv,
                                      d, scale, mask_type, dtype, workspace, workspace_bytes,
                                      stream))


def attn_fwd_batched_timed(*args, events, n_events) -> int:
    """attn_fwd_batched plus per-stage HIP events (see StageEvents)."""
    return int(lib().attn_fwd_batched_timed(*args, events, n_events))


def attn_bwd_batched_timed(*args, events, n_events) -> int:
    """attn_bwd_batched plus per-stage HIP events (see StageEvents)."""
    return int(lib().attn_bwd_batched_timed(*args, events, n_events))


def attn_fwd_thd_fp8(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_fwd_thd_fp8(*args))


def attn_bwd_thd_fp8(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_bwd_thd_fp8(*args))


def fp8_workspace_size(batch: int, total_q: int, total_kv: int, hq: int, hkv: int,
                       d: int) -> int:
    return int(lib().attn_thd_fp8_workspace_size(batch, total_q, total_kv, hq, hkv, d))


def attn_fwd_thd_dropout(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_fwd_thd_dropout(*args))


def attn_bwd_thd_dropout(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_bwd_thd_dropout(*args))


def attn_fwd_thd_chunk(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_fwd_thd_chunk(*args))


def attn_bwd_thd_chunk(*args) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_bwd_thd_chunk(*args))


def attn_merge_thd(out, lse, out_part, lse_part, total_q, hq, d, dtype, stream) -> int:
    """Same arguments as the C function (pointers as ints); returns the status code."""
    return int(lib().attn_merge_thd(out, lse, out_part, lse_part, total_q, hq, d, dtype, stream))


def attn_bwd_thd_noalloc(*args) -> int:
    """C ABI attn_bwd_thd_noalloc: attn_bwd_thd's arguments without the workspace pair."""
    return lib().attn_bwd_thd_noalloc(*args)


def attn_fwd_thd_timed(*args, events, n_events) -> int:
    """attn_fwd_thd plus per-stage HIP events (see StageEvents)."""
    return int(lib().attn_fwd_thd_timed(*args, events, n_events))


def attn_bwd_thd_timed(*args, events, n_events) -> int:
    """attn_bwd_thd plus per-stage HIP events (see StageEvents)."""
    return int(lib().attn_bwd_thd_timed(*args, events, n_events))


class StageEvents:
    """n HIP events (created with the HIP runtime torch loaded) to hand to the
    instrumented entry points; ``stage_ms()`` reads the stage durations.

    ``only=i`` creates just the two events around stage i (the other slots
    stay NULL, so the call records nothing else); ``stage_ms()`` then gives
    None for the stages it did not time."""

    def __init__(self, n: int, only: Optional[int] = None):
        self.n = n
        self._hip = _hip_runtime()
        self._arr = (_P * n)()
        self._made = [i for i in range(n) if only is None or i in (only, only + 1)]
        for i in self._made:
            ev = _P()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise AttnError("hipEventCreate failed")
            self._arr[i] = ev
        self.ptr = ctypes.cast(self._arr, ctypes.POINTER(_P))

    def stage_ms(self):
        self._hip.hipEventSynchronize(self._arr[self._made[-1]])
        out = []
        for i in range(self.n - 1):
            if not (self._arr[i] and self._arr[i + 1]):
                out.append(None)
                continue
            ms = ctypes.c_float(0.0)
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self._arr[i], self._arr[i + 1]) != 0:
                raise AttnError("hipEventElapsedTime failed")
            out.append(float(ms.value))
        return out

    def __del__(self):
        try:
            for i in self._made:
                self._hip.hipEventDestroy(self._arr[i])
        except Exception:
            pass


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already mapped into this process (the one torch loaded)."""
    torch.cuda.init()
    for line in open("/proc/self/maps"):
        path = line.split()[-1] if len(line.split()) >= 6 else ""
        if os.path.basename(path).startswith("libamdhip64.so"):
            h = ctypes.CDLL(path)
            h.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
            h.hipEventSynchronize.argtypes = [_P]
            h.hipEventDestroy.argtypes = [_P]
            return h
    raise AttnError("HIP runtime not loaded")


def read_device_status(workspace: torch.Tensor) -> int:
    """Synchronises the current stream and returns the device status word of the last call."""
    st = _I(0)
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    _check(lib().attn_thd_read_device_status(workspace.data_ptr(), stream, ctypes.byref(st)),
           "attn_thd_read_device_status")
    return int(st.value)


# ----------------------------------------------------------------- tensor wrappers
def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, dev=None, shape=None) -> None:
    """Checks a tensor argument; `shape` (checked first) guards the outputs,
    which the kernels write through raw pointers: an undersized tensor would
    be written past its end."""
    if not isinstance(t, torch.Tensor):
        raise AttnError(f"{name} must be a tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise AttnError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise AttnError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise AttnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise AttnError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise AttnError(f"{name} must be on {dev}")


def _cu(t, name, dev):
    if t is None:
        return None
    _need(t, name, torch.int32, dev)
    return t


def _workspace(ws, batch, tq, tk, hq, hkv, d, dev):
    """The caller's workspace, or a new one of workspace_size bytes.  A
    caller's workspace below workspace_size is passed on as it is: the library
    accepts any that holds the layout without partial dK/dV planes (the
    backward then spreads a GQA group over fewer workgroups) and answers
    ATTN_THD_EWORKSPACE below that."""
    if ws is None:
        ws = torch.empty(max(workspace_size(batch, tq, tk, hq, hkv, d), 256), dtype=torch.uint8,
                         device=dev)
    return ws


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
        cu_seqlens_kv: torch.Tensor, cu_seqlens_q_padded: Optional[torch.Tensor] = None,
        cu_seqlens_kv_padded: Optional[torch.Tensor] = None, max_seqlen_q: int = 0,
        max_seqlen_kv: int = 0, attn_mask_type: str = "padding",
        softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
        events: Optional["StageEvents"] = None, dropout_p: float = 0.0, rng_seed: int = 0,
        rng_offset: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward: returns (out [Tq,hq,d] in q's dtype, lse [Tq,hq] float32).

    dropout_p > 0: dropout on the probabilities with the Philox keep mask of
    (rng_seed, rng_offset); the backward must get the same three values."""
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    tq, hq, d = q.shape
    tk, hkv, dk_ = k.shape
    if v.shape != k.shape or dk_ != d:
        raise AttnError("k and v must be [total_kv, hkv, d] with q's d")
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    cqp = _cu(cu_seqlens_q_padded, "cu_seqlens_q_padded", dev)
    ckp = _cu(cu_seqlens_kv_padded, "cu_seqlens_kv_padded", dev)
    batch = cq.numel() - 1
    if ck.numel() != batch + 1 or any(c is not None and c.numel() != batch + 1 for c in (cqp, ckp)):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    _need(out, "out", q.dtype, dev, q.shape)
    _need(lse, "lse", torch.float32, dev, (tq, hq))
    ws = _workspace(workspace, batch, tq, tk, hq, hkv, d, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if dropout_p:
        st = attn_fwd_thd_dropout(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            cq.data_ptr(), ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk, hq, hkv, d, scale,
            _MASK[attn_mask_type], float(dropout_p), int(rng_seed) & (2 ** 64 - 1),
            int(rng_offset) & 0xFFFFFFFF, _DTYPE[q.dtype], ws.data_ptr(),
            ws.numel() * ws.element_size(), stream, None if events is None else events.ptr,
            0 if events is None else events.n)
        _check(st, "attn_fwd_thd_dropout")
        return out, lse
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            cq.data_ptr(), ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk,
            int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, d, scale, _MASK[attn_mask_type],
            _DTYPE[q.dtype], ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if events is None:
        st = attn_fwd_thd(*args)
    else:
        st = attn_fwd_thd_timed(*args, events=events.ptr, n_events=events.n)
    _check(st, "attn_fwd_thd")
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
        dout: torch.Tensor, lse: torch.Tensor, cu_seqlens_q: torch.Tensor,
        cu_seqlens_kv: torch.Tensor, cu_seqlens_q_padded: Optional[torch.Tensor] = None,
        cu_seqlens_kv_padded: Optional[torch.Tensor] = None, max_seqlen_q: int = 0,
        max_seqlen_kv: int = 0, attn_mask_type: str = "padding",
        softmax_scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, events: Optional["StageEvents"] = None,
        dropout_p: float = 0.0, rng_seed: int = 0, rng_offset: int = 0
        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward: returns (dq, dk, dv) in q's dtype (dropout arguments as ``fwd``)."""
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    for t, n in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if out.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or k.shape[2] != d:
        raise AttnError("shape mismatch among q, k, v, out, dout")
    if tuple(lse.shape) != (tq, hq):
        raise AttnError("lse must be [total_q, hq]")
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    cqp = _cu(cu_seqlens_q_padded, "cu_seqlens_q_padded", dev)
    ckp = _cu(cu_seqlens_kv_padded, "cu_seqlens_kv_padded", dev)
    batch = cq.numel() - 1
    if ck.numel() != batch + 1 or any(c is not None and c.numel() != batch + 1 for c in (cqp, ckp)):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, dev, q.shape)
    _need(dk, "dk", q.dtype, dev, k.shape)
    _need(dv, "dv", q.dtype, dev, k.shape)
    ws = _workspace(workspace, batch, tq, tk, hq, hkv, d, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if dropout_p:
        st = attn_bwd_thd_dropout(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cq.data_ptr(),
            ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk, hq, hkv, d, scale,
            _MASK[attn_mask_type], float(dropout_p), int(rng_seed) & (2 ** 64 - 1),
            int(rng_offset) & 0xFFFFFFFF, _DTYPE[q.dtype], ws.data_ptr(),
            ws.numel() * ws.element_size(), stream, None if events is None else events.ptr,
            0 if events is None else events.n)
        _check(st, "attn_bwd_thd_dropout")
        return dq, dk, dv
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cq.data_ptr(),
            ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk, int(max_seqlen_q),
            int(max_seqlen_kv), hq, hkv, d, scale, _MASK[attn_mask_type], _DTYPE[q.dtype],
            ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if events is None:
        st = attn_bwd_thd(*args)
    else:
        st = attn_bwd_thd_timed(*args, events=events.ptr, n_events=events.n)
    _check(st, "attn_bwd_thd")
    return dq, dk, dv


def bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                dout: torch.Tensor, lse: torch.Tensor, cu_seqlens_q: torch.Tensor,
                cu_seqlens_kv: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
                dv: torch.Tensor, cu_seqlens_q_padded: Optional[torch.Tensor] = None,
                cu_seqlens_kv_padded: Optional[torch.Tensor] = None, max_seqlen_q: int = 0,
                max_seqlen_kv: int = 0, attn_mask_type: str = "padding",
                softmax_scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """``bwd`` through attn_bwd_thd_noalloc: the caller passes every output, and
    neither this wrapper nor the library allocates device memory (the scratch
    is the library's static per-GPU array; calls that overlap on one GPU race)."""
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    for t, n in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if out.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or k.shape[2] != d:
        raise AttnError("shape mismatch among q, k, v, out, dout")
    _need(lse, "lse", torch.float32, dev, (tq, hq))
    _need(dq, "dq", q.dtype, dev, q.shape)
    _need(dk, "dk", q.dtype, dev, k.shape)
    _need(dv, "dv", q.dtype, dev, k.shape)
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    cqp = _cu(cu_seqlens_q_padded, "cu_seqlens_q_padded", dev)
    ckp = _cu(cu_seqlens_kv_padded, "cu_seqlens_kv_padded", dev)
    batch = cq.numel() - 1
    if ck.numel() != batch + 1 or any(c is not None and c.numel() != batch + 1 for c in (cqp, ckp)):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = attn_bwd_thd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cq.data_ptr(), ck.data_ptr(),
        _ptr(cqp), _ptr(ckp), batch, tq, tk, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, d,
        scale, _MASK[attn_mask_type], _DTYPE[q.dtype], torch.cuda.current_stream(dev).cuda_stream)
    _check(st, "attn_bwd_thd_noalloc")
    return dq, dk, dv


# ----------------------------------------------------------------- batched layouts
def _batched_dims(q, k, layout):
    if layout not in LAYOUTS:
        raise AttnError(f"layout must be one of {sorted(LAYOUTS)}")
    if q.dim() != 4 or k.dim() != 4:
        raise AttnError("batched q and k must be 4-d ([b,s,h,d] or [s,b,h,d])")
    if layout == "bshd":
        (b, sq, hq, d), (bk, skv, hkv, dk_) = q.shape, k.shape
    else:
        (sq, b, hq, d), (skv, bk, hkv, dk_) = q.shape, k.shape
    if bk != b or dk_ != d:
        raise AttnError("q and k disagree on batch or head dim")
    return b, sq, skv, hq, hkv, d


def _lse_shape(layout, b, sq, hq):
    return (b, sq, hq) if layout == "bshd" else (sq, b, hq)


def fwd_batched(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "sbhd",
                cu_seqlens_q: Optional[torch.Tensor] = None,
                cu_seqlens_kv: Optional[torch.Tensor] = None, attn_mask_type: str = "padding",
                softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                events: Optional["StageEvents"] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward on bshd ``[b, s, h, d]`` or sbhd ``[s, b, h, d]`` tensors, read in place.

    cu_seqlens_* (int32 [b+1]) give real lengths within the slots (None: full).
    Returns out (q's layout and dtype) and lse float32 ([b, s, hq] or [s, b, hq]).
    """
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    if v.shape != k.shape:
        raise AttnError("k and v must have the same shape")
    b, sq, skv, hq, hkv, d = _batched_dims(q, k, layout)
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    if any(c is not None and c.numel() != b + 1 for c in (cq, ck)):
        raise AttnError("cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(_lse_shape(layout, b, sq, hq), dtype=torch.float32, device=dev) \
        if lse is None else lse
    _need(out, "out", q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    if out.shape != q.shape or tuple(lse.shape) != _lse_shape(layout, b, sq, hq):
        raise AttnError("out or lse has the wrong shape")
    ws = _workspace(workspace, b, b * sq, b * skv, hq, hkv, d, dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), _ptr(cq),
            _ptr(ck), LAYOUTS[layout], b, sq, skv, hq, hkv, d, scale, _MASK[attn_mask_type],
            _DTYPE[q.dtype], ws.data_ptr(), ws.numel() * ws.element_size(),
            torch.cuda.current_stream(dev).cuda_stream)
    if events is None:
        st = attn_fwd_batched(*args)
    else:
        st = attn_fwd_batched_timed(*args, events=events.ptr, n_events=events.n)
    _check(st, "attn_fwd_batched")
    return out, lse


def bwd_batched(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                dout: torch.Tensor, lse: torch.Tensor, layout: str = "sbhd",
                cu_seqlens_q: Optional[torch.Tensor] = None,
                cu_seqlens_kv: Optional[torch.Tensor] = None, attn_mask_type: str = "padding",
                softmax_scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
                dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, events: Optional["StageEvents"] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward on bshd / sbhd tensors (arguments as ``fwd_batched``); returns (dq, dk, dv)."""
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    for t, n in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    b, sq, skv, hq, hkv, d = _batched_dims(q, k, layout)
    if out.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise AttnError("shape mismatch among q, k, v, out, dout")
    if tuple(lse.shape) != _lse_shape(layout, b, sq, hq):
        raise AttnError("lse has the wrong shape")
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    if any(c is not None and c.numel() != b + 1 for c in (cq, ck)):
        raise AttnError("cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, dev, q.shape)
    _need(dk, "dk", q.dtype, dev, k.shape)
    _need(dv, "dv", q.dtype, dev, k.shape)
    ws = _workspace(workspace, b, b * sq, b * skv, hq, hkv, d, dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(cq), _ptr(ck),
            LAYOUTS[layout], b, sq, skv, hq, hkv, d, scale, _MASK[attn_mask_type],
            _DTYPE[q.dtype], ws.data_ptr(), ws.numel() * ws.element_size(),
            torch.cuda.current_stream(dev).cuda_stream)
    if events is None:
        st = attn_bwd_batched(*args)
    else:
        st = attn_bwd_batched_timed(*args, events=events.ptr, n_events=events.n)
    _check(st, "attn_bwd_batched")
    return dq, dk, dv


# ----------------------------------------------------------------- chunked form
def _thd_common(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded, cu_seqlens_kv_padded,
                q_pos0, kv_pos0, attn_mask_type):
    dev = q.device
    _need(q, "q", None, dev)
    if q.dtype not in _DTYPE:
        raise AttnError(f"q must be bf16 or fp16, got {q.dtype}")
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    if v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise AttnError("k and v must be [total_kv, hkv, d] with q's d")
    cs = [_cu(t, n, dev) for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_kv, "cu_seqlens_kv"),
                                      (cu_seqlens_q_padded, "cu_seqlens_q_padded"),
                                      (cu_seqlens_kv_padded, "cu_seqlens_kv_padded"))]
    batch = cs[0].numel() - 1
    if any(c is not None and c.numel() != batch + 1 for c in cs):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    ps = [_cu(t, n, dev) for t, n in ((q_pos0, "q_pos0"), (kv_pos0, "kv_pos0"))]
    if any(t is not None and t.numel() != batch for t in ps):
        raise AttnError("q_pos0 / kv_pos0 need batch entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    return dev, cs, ps, batch


def fwd_chunk(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded=None,
              cu_seqlens_kv_padded=None, q_pos0=None, kv_pos0=None,
              attn_mask_type: str = "padding_causal", softmax_scale: Optional[float] = None,
              out=None, lse=None, workspace=None, events: Optional["StageEvents"] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Partial forward over a key chunk: (out, lse) of the chunk's visible keys,
    the causal rule applied to positions q_pos0[b] + i and kv_pos0[b] + j."""
    dev, cs, ps, batch = _thd_common(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                                     cu_seqlens_kv_padded, q_pos0, kv_pos0, attn_mask_type)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((tq, hq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", q.dtype, dev, q.shape)
    _need(lse, "lse", torch.float32, dev, (tq, hq))
    ws = _workspace(workspace, batch, tq, tk, hq, hkv, d, dev)
    st = attn_fwd_thd_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), *[_ptr(c) for c in cs], *[_ptr(t) for t in ps], batch,
                            tq, tk, hq, hkv, d, scale, _MASK[attn_mask_type], _DTYPE[q.dtype],
                            ws.data_ptr(), ws.numel() * ws.element_size(),
                            torch.cuda.current_stream(dev).cuda_stream,
                            None if events is None else events.ptr,
                            0 if events is None else events.n)
    _check(st, "attn_fwd_thd_chunk")
    return out, lse


def bwd_chunk(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded=None,
              cu_seqlens_kv_padded=None, q_pos0=None, kv_pos0=None,
              attn_mask_type: str = "padding_causal", softmax_scale: Optional[float] = None,
              dq=None, dk=None, dv=None, accumulate=False, workspace=None,
              events: Optional["StageEvents"] = None
              ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of one (query chunk, key chunk) pair from the whole out / lse.

    accumulate: False, True (add into dq, dk and dv), or a set of names among
    {"dq", "dkdv"}; the accumulated outputs must be given."""
    dev, cs, ps, batch = _thd_common(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                                     cu_seqlens_kv_padded, q_pos0, kv_pos0, attn_mask_type)
    for t, n in ((out, "out"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if out.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (tq, hq):
        raise AttnError("shape mismatch among q, out, dout, lse")
    if isinstance(accumulate, bool):
        acc = ACC_DQ | ACC_DKDV if accumulate else 0
    else:
        if not set(accumulate) <= {"dq", "dkdv"}:
            raise AttnError("accumulate names are 'dq' and 'dkdv'")
        acc = (ACC_DQ if "dq" in accumulate else 0) | (ACC_DKDV if "dkdv" in accumulate else 0)
    if (acc & ACC_DQ and dq is None) or (acc & ACC_DKDV and (dk is None or dv is None)):
        raise AttnError("an accumulated output must be given")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, dev, q.shape)
    _need(dk, "dk", q.dtype, dev, k.shape)
    _need(dv, "dv", q.dtype, dev, k.shape)
    ws = _workspace(workspace, batch, tq, tk, hq, hkv, d, dev)
    st = attn_bwd_thd_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), *[_ptr(c) for c in cs], *[_ptr(t) for t in ps], batch,
                            tq, tk, hq, hkv, d, scale, _MASK[attn_mask_type], acc,
                            _DTYPE[q.dtype], ws.data_ptr(), ws.numel() * ws.element_size(),
                            torch.cuda.current_stream(dev).cuda_stream,
                            None if events is None else events.ptr,
                            0 if events is None else events.n)
    _check(st, "attn_bwd_thd_chunk")
    return dq, dk, dv


def merge(out: torch.Tensor, lse: torch.Tensor, out_part: torch.Tensor,
          lse_part: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Combines two partials over disjoint key sets, in place on (out, lse)."""
    dev = out.device
    _need(out, "out", None, dev)
    if out.dtype not in _DTYPE:
        raise AttnError(f"out must be bf16 or fp16, got {out.dtype}")
    _need(out_part, "out_part", out.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    _need(lse_part, "lse_part", torch.float32, dev)
    tq, hq, d = out.shape
    if out_part.shape != out.shape or lse.shape != (tq, hq) or lse_part.shape != (tq, hq):
        raise AttnError("merge: shape mismatch")
    _check(attn_merge_thd(out.data_ptr(), lse.data_ptr(), out_part.data_ptr(), lse_part.data_ptr(),
                          tq, hq, d, _DTYPE[out.dtype], torch.cuda.current_stream(dev).cuda_stream),
           "attn_merge_thd")
    return out, lse


# ----------------------------------------------------------------- autograd
class _AttentionTHD(torch.autograd.Function):
    """The forward and backward entry points as one differentiable op (the
    backward gets the forward's own out and lse, as TE-style callers pass them)."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                cu_seqlens_kv_padded, attn_mask_type, softmax_scale, dropout_p, rng_seed,
                rng_offset):
        kw = dict(cu_seqlens_q_padded=cu_seqlens_q_padded,
                  cu_seqlens_kv_padded=cu_seqlens_kv_padded, attn_mask_type=attn_mask_type,
                  softmax_scale=softmax_scale, dropout_p=dropout_p, rng_seed=rng_seed,
                  rng_offset=rng_offset)
        out, lse = fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, **kw)
        ctx.save_for_backward(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv)
        ctx.kw = kw
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse, cq, ck = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, out, dout.contiguous(), lse, cq, ck, **ctx.kw)
        return dq, dk, dv, None, None, None, None, None, None, None, None, None


def attention_thd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor,
                  cu_seqlens_q_padded: Optional[torch.Tensor] = None,
                  cu_seqlens_kv_padded: Optional[torch.Tensor] = None,
                  attn_mask_type: str = "padding_causal", softmax_scale: Optional[float] = None,
                  dropout_p: float = 0.0, rng_seed: int = 0, rng_offset: int = 0,
                  return_lse: bool = False):
    """Differentiable THD attention: out (and lse if asked); gradients flow to q, k, v."""
    out, lse = _AttentionTHD.apply(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                                   cu_seqlens_kv_padded, attn_mask_type, softmax_scale,
                                   dropout_p, rng_seed, rng_offset)
    return (out, lse) if return_lse else out


# ----------------------------------------------------------------- FP8 inputs
def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, descale_q: float,
            descale_k: float, descale_v: float, cu_seqlens_q: torch.Tensor,
            cu_seqlens_kv: torch.Tensor, cu_seqlens_q_padded: Optional[torch.Tensor] = None,
            cu_seqlens_kv_padded: Optional[torch.Tensor] = None,
            attn_mask_type: str = "padding", softmax_scale: Optional[float] = None,
            out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            events: Optional["StageEvents"] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward from E4M3 inputs (torch.float8_e4m3fn or uint8 codes) with per-tensor
    descales: (out [Tq,hq,d] in out_dtype, lse [Tq,hq] float32)."""
    dev = q8.device
    codes = lambda t, n: _fp8_codes(t, n, dev)
    q8, k8, v8 = codes(q8, "q8"), codes(k8, "k8"), codes(v8, "v8")
    tq, hq, d = q8.shape
    tk, hkv, dk_ = k8.shape
    if v8.shape != k8.shape or dk_ != d:
        raise AttnError("k8 and v8 must be [total_kv, hkv, d] with q8's d")
    if out_dtype not in _DTYPE:
        raise AttnError("out_dtype must be bf16 or fp16")
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    cqp = _cu(cu_seqlens_q_padded, "cu_seqlens_q_padded", dev)
    ckp = _cu(cu_seqlens_kv_padded, "cu_seqlens_kv_padded", dev)
    batch = cq.numel() - 1
    if ck.numel() != batch + 1 or any(c is not None and c.numel() != batch + 1 for c in (cqp, ckp)):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty((tq, hq, d), dtype=out_dtype, device=dev) if out is None else out
    lse = torch.empty((tq, hq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", out_dtype, dev, (tq, hq, d))
    _need(lse, "lse", torch.float32, dev, (tq, hq))
    need = fp8_workspace_size(batch, tq, tk, hq, hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = attn_fwd_thd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(descale_q),
                          float(descale_k), float(descale_v), out.data_ptr(), lse.data_ptr(),
                          cq.data_ptr(), ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk, hq,
                          hkv, d, scale, _MASK[attn_mask_type], _DTYPE[out_dtype],
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          torch.cuda.current_stream(dev).cuda_stream,
                          None if events is None else events.ptr,
                          0 if events is None else events.n)
    _check(st, "attn_fwd_thd_fp8")
    return out, lse


def bwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, descale_q: float,
            descale_k: float, descale_v: float, out: torch.Tensor, dout: torch.Tensor,
            lse: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor,
            cu_seqlens_q_padded: Optional[torch.Tensor] = None,
            cu_seqlens_kv_padded: Optional[torch.Tensor] = None,
            attn_mask_type: str = "padding", softmax_scale: Optional[float] = None,
            dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
            dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            events: Optional["StageEvents"] = None
            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of ``fwd_fp8``: gradients (dq, dk, dv), in out's dtype, with respect to
    the real-valued inputs descale_q * q8, descale_k * k8, descale_v * v8."""
    dev = q8.device
    codes = lambda t, n: _fp8_codes(t, n, dev)
    q8, k8, v8 = codes(q8, "q8"), codes(k8, "k8"), codes(v8, "v8")
    tq, hq, d = q8.shape
    tk, hkv, dk_ = k8.shape
    if v8.shape != k8.shape or dk_ != d:
        raise AttnError("k8 and v8 must be [total_kv, hkv, d] with q8's d")
    if out.dtype not in _DTYPE:
        raise AttnError("out must be bf16 or fp16")
    _need(out, "out", out.dtype, dev)
    _need(dout, "dout", out.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (tq, hq, d) or dout.shape != out.shape or tuple(lse.shape) != (tq, hq):
        raise AttnError("out and dout must be [total_q, hq, d], lse [total_q, hq]")
    cq = _cu(cu_seqlens_q, "cu_seqlens_q", dev)
    ck = _cu(cu_seqlens_kv, "cu_seqlens_kv", dev)
    cqp = _cu(cu_seqlens_q_padded, "cu_seqlens_q_padded", dev)
    ckp = _cu(cu_seqlens_kv_padded, "cu_seqlens_kv_padded", dev)
    batch = cq.numel() - 1
    if ck.numel() != batch + 1 or any(c is not None and c.numel() != batch + 1 for c in (cqp, ckp)):
        raise AttnError("all cu_seqlens arrays need batch + 1 entries")
    if attn_mask_type not in _MASK:
        raise AttnError(f"attn_mask_type must be one of {sorted(_MASK)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty((tq, hq, d), dtype=out.dtype, device=dev) if dq is None else dq
    dk = torch.empty((tk, hkv, d), dtype=out.dtype, device=dev) if dk is None else dk
    dv = torch.empty((tk, hkv, d), dtype=out.dtype, device=dev) if dv is None else dv
    for t, n, shp in ((dq, "dq", (tq, hq, d)), (dk, "dk", (tk, hkv, d)), (dv, "dv", (tk, hkv, d))):
        _need(t, n, out.dtype, dev, shp)
    need = fp8_workspace_size(batch, tq, tk, hq, hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = attn_bwd_thd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(descale_q),
                          float(descale_k), float(descale_v), out.data_ptr(), dout.data_ptr(),
                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          cq.data_ptr(), ck.data_ptr(), _ptr(cqp), _ptr(ckp), batch, tq, tk, hq,
                          hkv, d, scale, _MASK[attn_mask_type], _DTYPE[out.dtype],
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          torch.cuda.current_stream(dev).cuda_stream,
                          None if events is None else events.ptr,
                          0 if events is None else events.n)
    _check(st, "attn_bwd_thd_fp8")
    return dq, dk, dv


def _fp8_codes(t: torch.Tensor, name: str, dev) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _need(t, name, torch.uint8, dev)
    return t
