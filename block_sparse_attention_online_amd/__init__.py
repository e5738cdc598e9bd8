"""Skip-softmax (BLASST) attention for AMD MI355X: Python binding of libssattn.so.

The functions here carry the C entry points' names (include/ss_attn.h) and do
argument marshalling only: they check device, dtype, contiguity and shapes of
torch tensors, allocate outputs when asked to, and pass raw device pointers
and the current HIP stream to the library.  Every step of the attention runs
in the library's gfx950 kernels; there is no CPU or PyTorch fallback, and
importing a function that needs the library raises if it was not built.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "ss_attn_prefill", "ss_attn_prefill_f32", "ss_attn_prefill_ex", "ss_attn_decode",
    "ss_attn_decode_ex", "ss_attn_decode_partial", "ss_attn_decode_combine", "SPLIT_MODES",
    "ss_attn_decode_workspace_bytes", "ss_decode_num_splits", "ss_factor", "ss_threshold",
    "ss_gate_enabled", "ss_resolve_threshold", "ss_last_error", "ss_version", "library_path",
    "SSError", "TILE", "ORDERS", "mask_shape_prefill", "mask_shape_decode",
    "ss_attn_decode_paged", "GRANULARITIES", "row_mask_shape_prefill", "row_mask_shape_decode",
    "ss_attn_prefill_backward", "ss_attn_prefill_backward_workspace_bytes",
    "ss_attn_decode_lookback_timeouts", "ss_attn_decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES",
]

TILE = 128
DECODE_NOALLOC_SCRATCH_BYTES = 48 << 20  # SS_DECODE_NOALLOC_SCRATCH_BYTES in ss_attn.h
ORDERS = {"ascending": 0, "diag_first": 1}
SS_FACTOR_DIRECT, SS_FACTOR_CALIBRATED = 0, 1
_DTYPE = {torch.bfloat16: 0, torch.float32: 1}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libssattn.so")


class SSError(RuntimeError):
    """A non-zero ss_status from the library."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"ssattn error {code}: {msg}")
        self.code = code


class _PrefillParams(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("B", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("Lq", ctypes.c_int), ("Lk", ctypes.c_int),
                ("D", ctypes.c_int), ("Dv", ctypes.c_int), ("scale", ctypes.c_float),
                ("threshold", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("order", ctypes.c_int), ("skip_mask_out", ctypes.c_void_p),
                ("granularity", ctypes.c_int), ("row_mask_out", ctypes.c_void_p),
                ("lse_out", ctypes.c_void_p)]


class _DecodeParams(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("B", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("Lk", ctypes.c_int), ("D", ctypes.c_int),
                ("Dv", ctypes.c_int), ("scale", ctypes.c_float), ("threshold", ctypes.c_float),
                ("num_splits", ctypes.c_int), ("split_mode", ctypes.c_int),
                ("skip_mask_out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("granularity", ctypes.c_int),
                ("row_mask_out", ctypes.c_void_p)]


class _DecodePagedParams(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("thresholds", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("B", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("D", ctypes.c_int), ("Dv", ctypes.c_int),
                ("block_size", ctypes.c_int), ("max_blocks_per_seq", ctypes.c_int),
                ("num_blocks", ctypes.c_int), ("max_seq_len", ctypes.c_int),
                ("scale", ctypes.c_float), ("factor", ctypes.c_float),
                ("num_splits", ctypes.c_int), ("skip_mask_out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class _PrefillBwdParams(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("skip_mask", ctypes.c_void_p), ("dq", ctypes.c_void_p),
                ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("B", ctypes.c_int),
                ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("Lq", ctypes.c_int),
                ("Lk", ctypes.c_int), ("D", ctypes.c_int), ("Dv", ctypes.c_int),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


SPLIT_MODES = {"chained": 0, "independent": 1}
# who takes a skip decision: the whole row block of a tile, or every row alone
GRANULARITIES = {"tile": 0, "row": 1}

_LIB = None

_P, _I, _F, _D, _SZ, _I64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double,
                             ctypes.c_size_t, ctypes.c_int64)
_SIGNATURES = {
    "ss_attn_prefill": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _F, _P, _P]),
    "ss_attn_prefill_f32": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _F, _P, _P]),
    "ss_attn_prefill_ex": (_I, [ctypes.POINTER(_PrefillParams), _P]),
    "ss_attn_prefill_backward": (_I, [ctypes.POINTER(_PrefillBwdParams), _P]),
    "ss_attn_prefill_backward_workspace_bytes": (_SZ, [_I, _I, _I]),
    "ss_attn_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _P, _SZ, _P]),
    "ss_attn_decode_ex": (_I, [ctypes.POINTER(_DecodeParams), _P]),
    "ss_attn_decode_paged": (_I, [ctypes.POINTER(_DecodePagedParams), _P]),
    "ss_attn_decode_partial": (_I, [ctypes.POINTER(_DecodeParams), _P]),
    "ss_attn_decode_combine": (_I, [ctypes.POINTER(_DecodeParams), _P]),
    "ss_attn_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _P]),
    "ss_attn_decode_lookback_timeouts": (_I, [ctypes.POINTER(_DecodeParams),
                                              ctypes.POINTER(ctypes.c_uint), _I, _P]),
    "ss_attn_decode_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "ss_decode_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "ss_factor": (_I, [_I, _D, _D, _D, _D, _I64, ctypes.POINTER(_D)]),
    "ss_threshold": (_I, [_D, _I64, ctypes.POINTER(_D)]),
    "ss_gate_enabled": (_I, [_I, _D, _I, _D]),
    "ss_resolve_threshold": (_I, [_I, _D, _D, _D, _D, _I64, _I, _D, _I, _D,
                                  ctypes.POINTER(_F)]),
    "ss_last_error": (ctypes.c_char_p, []),
    "ss_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load libssattn.so (built in-tree by build.py); raise if it is missing."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m block_sparse_attention_online_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def ss_last_error() -> str:
    return lib().ss_last_error().decode()


def ss_version() -> str:
    return lib().ss_version().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise SSError(rc, ss_last_error())


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def mask_shape_prefill(B, Hq, Lq, Lk):
    return (B, Hq, -(-Lq // TILE), -(-Lk // TILE))


def mask_shape_decode(B, Hkv, Lk):
    return (B, Hkv, -(-Lk // TILE))


def row_mask_shape_prefill(B, Hq, Lq, Lk):
    return (B, Hq, Lq, -(-Lk // TILE))


def row_mask_shape_decode(B, Hq, Lk):
    return (B, Hq, -(-Lk // TILE))


def _granularity(granularity, row_mask, shape):
    if granularity not in GRANULARITIES:
        raise ValueError(f"granularity must be one of {sorted(GRANULARITIES)}")
    if row_mask is None:
        return GRANULARITIES[granularity], None
    if granularity != "row":
        raise ValueError("row_mask needs granularity='row'")
    if tuple(row_mask.shape) != shape:
        raise ValueError(f"row_mask must be {shape}")
    return GRANULARITIES[granularity], _dev(row_mask, "row_mask", torch.uint8)


# --------------------------------------------------------------------------- prefill

def ss_attn_prefill_ex(q, k, v, out=None, *, scale=None, causal=False, threshold=0.0,
                       skip_mask=None, order="ascending", granularity="tile", row_mask=None,
                       lse=None, stream=None):
    """Skip-softmax prefill: q[B,Hq,Lq,D], k[B,Hkv,Lk,D], v[B,Hkv,Lk,Dv] on the GPU
    (all bf16 or all fp32).  Returns ``out`` [B,Hq,Lq,Dv]; fills ``skip_mask``
    (u8 [B,Hq,ceil(Lq/128),ceil(Lk/128)]) when given.  ``granularity="row"``
    lets every query row decide alone; ``row_mask`` (u8
    [B,Hq,Lq,ceil(Lk/128)]) then receives the per-row decisions.  ``lse``
    (fp32 [B,Hq,Lq]) receives each row's log-sum-exp over its kept keys.
    Asynchronous on ``stream`` (default: the current stream)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, D]")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape[:3]) != (B, Hkv, Lk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    Dv = v.shape[3]
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dt = q.dtype
    if out is None:
        out = torch.empty((B, Hq, Lq, Dv), dtype=dt, device=q.device)
    elif tuple(out.shape) != (B, Hq, Lq, Dv):
        raise ValueError(f"out must be {(B, Hq, Lq, Dv)}")
    mptr = None
    if skip_mask is not None:
        if tuple(skip_mask.shape) != mask_shape_prefill(B, Hq, Lq, Lk):
            raise ValueError(f"skip_mask must be {mask_shape_prefill(B, Hq, Lq, Lk)}")
        mptr = _dev(skip_mask, "skip_mask", torch.uint8)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if order not in ORDERS:
        raise ValueError(f"order must be one of {sorted(ORDERS)}")
    gran, rptr = _granularity(granularity, row_mask, row_mask_shape_prefill(B, Hq, Lq, Lk))
    lptr = None
    if lse is not None:
        if tuple(lse.shape) != (B, Hq, Lq):
            raise ValueError(f"lse must be {(B, Hq, Lq)}")
        lptr = _dev(lse, "lse", torch.float32)
    p = _PrefillParams(_dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt), _dev(out, "out", dt),
                       B, Hq, Hkv, Lq, Lk, D, Dv, float(scale), float(threshold), int(bool(causal)),
                       _DTYPE[dt], ORDERS[order], mptr, gran, rptr, lptr)
    _check(lib().ss_attn_prefill_ex(ctypes.byref(p), _stream(stream, q.device)))
    return out


def ss_attn_prefill(q, k, v, out=None, *, scale=None, causal=False, threshold=0.0,
                    skip_mask=None, stream=None):
    """bf16 skip-softmax prefill in ascending key-tile order (see ss_attn_prefill_ex)."""
    if q.dtype != torch.bfloat16:
        raise TypeError("ss_attn_prefill takes bf16 tensors")
    return ss_attn_prefill_ex(q, k, v, out, scale=scale, causal=causal, threshold=threshold,
                              skip_mask=skip_mask, stream=stream)


def ss_attn_prefill_f32(q, k, v, out=None, *, scale=None, causal=False, threshold=0.0,
                        skip_mask=None, stream=None):
    """fp32 debug path of the skip-softmax prefill (see ss_attn_prefill_ex)."""
    if q.dtype != torch.float32:
        raise TypeError("ss_attn_prefill_f32 takes fp32 tensors")
    return ss_attn_prefill_ex(q, k, v, out, scale=scale, causal=causal, threshold=threshold,
                              skip_mask=skip_mask, stream=stream)


def ss_attn_prefill_backward_workspace_bytes(B, Hq, Lq) -> int:
    return int(lib().ss_attn_prefill_backward_workspace_bytes(B, Hq, Lq))


def ss_attn_prefill_backward(q, k, v, out, dout, lse, skip_mask=None, *, scale=None,
                             causal=False, dq=None, dk=None, dv=None, workspace=None,
                             stream=None):
    """Skip-aware backward of the bf16 prefill: gradients of ``out`` with the
    forward's skip decisions held fixed.  ``out`` and ``lse`` (fp32 [B,Hq,Lq])
    come from the forward call (``ss_attn_prefill_ex(..., lse=...)``), ``dout``
    is dL/dout, ``skip_mask`` the forward's tile mask (None: dense attention).
    ``scale`` and ``causal`` must be the forward's.  Returns ``(dq, dk, dv)``
    (bf16, allocated when not given).  Asynchronous on ``stream``."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, D]")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    Dv = v.shape[3]
    if (Bk, Dk) != (B, D) or tuple(v.shape[:3]) != (B, Hkv, Lk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for name, t in (("out", out), ("dout", dout)):
        if tuple(t.shape) != (B, Hq, Lq, Dv):
            raise ValueError(f"{name} must be {(B, Hq, Lq, Dv)}")
    if tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError(f"lse must be {(B, Hq, Lq)}")
    dt = torch.bfloat16
    if q.dtype != dt:
        raise TypeError("ss_attn_prefill_backward takes bf16 tensors")
    mptr = None
    if skip_mask is not None:
        if tuple(skip_mask.shape) != mask_shape_prefill(B, Hq, Lq, Lk):
            raise ValueError(f"skip_mask must be {mask_shape_prefill(B, Hq, Lq, Lk)}")
        mptr = _dev(skip_mask, "skip_mask", torch.uint8)
    if dq is None:
        dq = torch.empty((B, Hq, Lq, D), dtype=dt, device=q.device)
    if dk is None:
        dk = torch.empty((B, Hkv, Lk, D), dtype=dt, device=q.device)
    if dv is None:
        dv = torch.empty((B, Hkv, Lk, Dv), dtype=dt, device=q.device)
    for name, t, shp in (("dq", dq, (B, Hq, Lq, D)), ("dk", dk, (B, Hkv, Lk, D)),
                         ("dv", dv, (B, Hkv, Lk, Dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {shp}")
    if workspace is None:
        need = ss_attn_prefill_backward_workspace_bytes(B, Hq, Lq)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    p = _PrefillBwdParams(_dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
                          _dev(out, "out", dt), _dev(dout, "dout", dt),
                          _dev(lse, "lse", torch.float32), mptr, _dev(dq, "dq", dt),
                          _dev(dk, "dk", dt), _dev(dv, "dv", dt), B, Hq, Hkv, Lq, Lk, D, Dv,
                          float(scale), int(bool(causal)), _DTYPE[dt], _dev(workspace, "workspace"),
                          workspace.numel() * workspace.element_size())
    _check(lib().ss_attn_prefill_backward(ctypes.byref(p), _stream(stream, q.device)))
    return dq, dk, dv


# --------------------------------------------------------------------------- decode

def ss_decode_num_splits(B, Hq, Hkv, Lk, D, Dv) -> int:
    return int(lib().ss_decode_num_splits(B, Hq, Hkv, Lk, D, Dv))


def ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, num_splits=0) -> int:
    return int(lib().ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, num_splits))


def _decode_params(q, k, v, out, dv, scale, threshold, num_splits, split_mode, skip_mask,
                   workspace, granularity="tile", row_mask=None, alloc_workspace=True):
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and k [B, Hkv, Lk, D]")
    B, Hq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    dt = torch.bfloat16
    if v is None:
        if dv is None:
            raise ValueError("v=None needs dv (value columns of the latent row)")
        Dv, vptr = int(dv), None
    else:
        if v.dim() != 4 or tuple(v.shape[:3]) != (B, Hkv, Lk):
            raise ValueError(f"v must be [B, Hkv, Lk, Dv] (got {tuple(v.shape)})")
        Dv, vptr = v.shape[3], _dev(v, "v", dt)
    if out is not None and tuple(out.shape) != (B, Hq, Dv):
        raise ValueError(f"out must be {(B, Hq, Dv)}")
    mptr = None
    if skip_mask is not None:
        if tuple(skip_mask.shape) != mask_shape_decode(B, Hkv, Lk):
            raise ValueError(f"skip_mask must be {mask_shape_decode(B, Hkv, Lk)}")
        mptr = _dev(skip_mask, "skip_mask", torch.uint8)
    if split_mode not in SPLIT_MODES:
        raise ValueError(f"split_mode must be one of {sorted(SPLIT_MODES)}")
    if workspace is None and alloc_workspace:  # zeroed: the give-up counter starts at 0
        need = ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, num_splits)
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    gran, rptr = _granularity(granularity, row_mask, row_mask_shape_decode(B, Hq, Lk))
    p = _DecodeParams(_dev(q, "q", dt), _dev(k, "k", dt), vptr,
                      None if out is None else _dev(out, "out", dt), B, Hq, Hkv, Lk, D, Dv,
                      float(scale), float(threshold), int(num_splits), SPLIT_MODES[split_mode],
                      mptr, None if workspace is None else _dev(workspace, "workspace"),
                      0 if workspace is None else workspace.numel() * workspace.element_size(),
                      gran, rptr)
    return p, workspace, (B, Hq, Dv)


def ss_attn_decode_partial(q, k, v=None, *, dv=None, scale=None, threshold=0.0, num_splits=0,
                           split_mode="chained", skip_mask=None, workspace=None,
                           granularity="tile", row_mask=None, stream=None):
    """First stage of the decode: run every split into ``workspace`` (returned)."""
    p, ws, _ = _decode_params(q, k, v, None, dv, scale, threshold, num_splits, split_mode,
                              skip_mask, workspace, granularity, row_mask)
    _check(lib().ss_attn_decode_partial(ctypes.byref(p), _stream(stream, q.device)))
    return ws


def ss_attn_decode_combine(q, k, workspace, out, *, v=None, dv=None, num_splits=0,
                           split_mode="chained", stream=None):
    """Second stage: log-sum-exp merge of the split partials into ``out``.
    ``q``, ``k`` (and ``v`` or ``dv``) only give the sizes; they are not read."""
    p, _, _ = _decode_params(q, k, v, out, dv, 1.0, 0.0, num_splits, split_mode, None, workspace)
    _check(lib().ss_attn_decode_combine(ctypes.byref(p), _stream(stream, out.device)))
    return out


def ss_attn_decode_noalloc(q, k, v=None, out=None, *, dv=None, scale=None, threshold=0.0,
                           num_splits=0, skip_mask=None, stream=None):
    """ss_attn_decode (chained splits) with the split workspace taken from the
    library's fixed per-GPU array (DECODE_NOALLOC_SCRATCH_BYTES): the library
    allocates nothing.  ``out`` is allocated here only when None.  Calls that
    overlap in time on one GPU race (they share the array)."""
    if out is None:
        Dv = int(dv) if v is None else v.shape[3]
        out = torch.empty((q.shape[0], q.shape[1], Dv), dtype=torch.bfloat16, device=q.device)
    p, _, _ = _decode_params(q, k, v, out, dv, scale, threshold, num_splits, "chained",
                             skip_mask, None, alloc_workspace=False)
    _check(lib().ss_attn_decode_noalloc(p.q, p.k, p.v, p.out, p.B, p.Hq, p.Hkv, p.Lk, p.D, p.Dv,
                                        p.scale, p.threshold, p.num_splits, p.skip_mask_out,
                                        _stream(stream, q.device)))
    return out


def ss_attn_decode_lookback_timeouts(q, k, workspace, *, v=None, dv=None, num_splits=0,
                                     split_mode="chained", reset=False, stream=None) -> int:
    """Look-back waits that gave up, counted in ``workspace`` by the decode
    calls that used it (cumulative; ``reset=True`` clears it after reading).
    ``q``, ``k`` (and ``v`` or ``dv``), ``num_splits`` and ``split_mode`` must
    be those of the calls; only their sizes are used.  Synchronizes the
    stream."""
    p, _, _ = _decode_params(q, k, v, None, dv, 1.0, 0.0, num_splits, split_mode, None, workspace)
    n = ctypes.c_uint()
    _check(lib().ss_attn_decode_lookback_timeouts(ctypes.byref(p), ctypes.byref(n), int(bool(reset)),
                                                  _stream(stream, q.device)))
    return int(n.value)


def ss_attn_decode_ex(q, k, v=None, out=None, *, dv=None, scale=None, threshold=0.0,
                      num_splits=0, split_mode="chained", skip_mask=None, workspace=None,
                      granularity="tile", row_mask=None, stream=None):
    """Split-KV skip-softmax decode: q[B,Hq,D], k[B,Hkv,Lk,D], v[B,Hkv,Lk,Dv] bf16,
    or ``v=None`` with ``dv`` for a latent cache whose value rows are the first
    ``dv`` columns of each key row.  Returns ``out`` [B,Hq,Dv]; fills
    ``skip_mask`` (u8 [B,Hkv,ceil(Lk/128)]) when given.  ``split_mode``:
    "chained" (decisions of one streaming pass) or "independent" (each split
    restarts the running max).  ``workspace``: a uint8 GPU tensor of at least
    ss_attn_decode_workspace_bytes() bytes (allocated here when None).
    ``granularity="row"`` lets every query head decide alone (separate V only);
    ``row_mask`` (u8 [B,Hq,ceil(Lk/128)]) then receives the per-row decisions."""
    if out is None:
        Dv = int(dv) if v is None else v.shape[3]
        out = torch.empty((q.shape[0], q.shape[1], Dv), dtype=torch.bfloat16, device=q.device)
    p, _, _ = _decode_params(q, k, v, out, dv, scale, threshold, num_splits, split_mode,
                             skip_mask, workspace, granularity, row_mask)
    _check(lib().ss_attn_decode_ex(ctypes.byref(p), _stream(stream, q.device)))
    return out


def ss_attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len,
                         out=None, dv=None, scale=None, factor=0.0, thresholds=None,
                         num_splits=0, skip_mask=None, workspace=None, stream=None):
    """Skip-softmax decode over a block-paged cache with per-sequence lengths.

    q [B,Hq,D] bf16; k_cache [num_blocks,Hkv,block_size,D] bf16; v_cache the
    same shape with Dv columns, or None for a latent cache whose value rows are
    the first ``dv`` columns of the key rows; block_table int32
    [B,max_blocks]; seq_lens int32 [B] (all GPU tensors).  Sequence b uses
    ``thresholds[b]`` (fp32 GPU tensor) when given, else
    ``factor / seq_lens[b]``.  Returns ``out`` [B,Hq,Dv]; fills ``skip_mask``
    (u8 [B,Hkv,ceil(max_seq_len/128)], 2 past a sequence's end) when given."""
    if q.dim() != 3 or k_cache.dim() != 4 or (v_cache is not None and v_cache.dim() != 4):
        raise ValueError("q must be [B, Hq, D] and the caches [num_blocks, Hkv, block_size, D]")
    B, Hq, D = q.shape
    nblk, Hkv, bs, Dk = k_cache.shape
    if v_cache is None:
        if dv is None:
            raise ValueError("a latent cache (v_cache=None) needs dv")
        Dv = int(dv)
    else:
        if tuple(v_cache.shape[:3]) != (nblk, Hkv, bs):
            raise ValueError(f"cache shapes k{tuple(k_cache.shape)} v{tuple(v_cache.shape)}")
        Dv = v_cache.shape[3]
    if Dk != D:
        raise ValueError(f"cache shape k{tuple(k_cache.shape)} vs q{tuple(q.shape)}")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    dt = torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=dt, device=q.device)
    mptr = None
    if skip_mask is not None:
        if tuple(skip_mask.shape) != mask_shape_decode(B, Hkv, max_seq_len):
            raise ValueError(f"skip_mask must be {mask_shape_decode(B, Hkv, max_seq_len)}")
        mptr = _dev(skip_mask, "skip_mask", torch.uint8)
    if workspace is None:
        need = ss_attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, D, Dv, num_splits)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    tptr = None if thresholds is None else _dev(thresholds, "thresholds", torch.float32)
    vptr = None if v_cache is None else _dev(v_cache, "v_cache", dt)
    p = _DecodePagedParams(_dev(q, "q", dt), _dev(k_cache, "k_cache", dt),
                           vptr, _dev(block_table, "block_table", torch.int32),
                           _dev(seq_lens, "seq_lens", torch.int32), tptr, _dev(out, "out", dt),
                           B, Hq, Hkv, D, Dv, bs, block_table.shape[1], nblk, int(max_seq_len),
                           float(scale), float(factor), int(num_splits), mptr,
                           _dev(workspace, "workspace"),
                           workspace.numel() * workspace.element_size())
    _check(lib().ss_attn_decode_paged(ctypes.byref(p), _stream(stream, q.device)))
    return out


def ss_attn_decode(q, k, v=None, out=None, *, dv=None, scale=None, threshold=0.0, num_splits=0,
                   skip_mask=None, workspace=None, stream=None):
    """Split-KV skip-softmax decode with chained splits (see ss_attn_decode_ex)."""
    return ss_attn_decode_ex(q, k, v, out, dv=dv, scale=scale, threshold=threshold,
                             num_splits=num_splits, split_mode="chained", skip_mask=skip_mask,
                             workspace=workspace, stream=stream)


# --------------------------------------------------------------------------- host helpers

def ss_factor(mode, a=0.0, b=0.0, target_sparsity=0.0, threshold=0.0, seqlen=1) -> float:
    """Calibrated factor a*exp(b*target_sparsity) or direct factor threshold*seqlen."""
    m = {"direct": SS_FACTOR_DIRECT, "calibrated": SS_FACTOR_CALIBRATED}.get(mode, mode)
    out = ctypes.c_double()
    _check(lib().ss_factor(int(m), a, b, target_sparsity, threshold, int(seqlen),
                           ctypes.byref(out)))
    return out.value


def ss_threshold(factor, seqlen) -> float:
    out = ctypes.c_double()
    _check(lib().ss_threshold(float(factor), int(seqlen), ctypes.byref(out)))
    return out.value


def ss_gate_enabled(timestep=None, disabled_until=None) -> bool:
    return bool(lib().ss_gate_enabled(timestep is not None, 0.0 if timestep is None else timestep,
                                      disabled_until is not None,
                                      0.0 if disabled_until is None else disabled_until))


def ss_resolve_threshold(mode, *, a=0.0, b=0.0, target_sparsity=0.0, threshold=0.0, seqlen=1,
                         timestep=None, disabled_until=None) -> float:
    """The fp32 threshold a kernel call receives: 0 (dense) when gated off."""
    m = {"direct": SS_FACTOR_DIRECT, "calibrated": SS_FACTOR_CALIBRATED}.get(mode, mode)
    out = ctypes.c_float()
    _check(lib().ss_resolve_threshold(int(m), a, b, target_sparsity, threshold, int(seqlen),
                                      timestep is not None, 0.0 if timestep is None else timestep,
                                      disabled_until is not None,
                                      0.0 if disabled_until is None else disabled_until,
                                      ctypes.byref(out)))
    return out.value
