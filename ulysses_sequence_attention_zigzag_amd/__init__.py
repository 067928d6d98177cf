"""Python binding of libusp: ring / zigzag / striped / Ulysses-hybrid attention on gfx950.

Argument marshalling only: every step runs in the HIP kernels of libusp.so,
which must be built (``python -m ulysses_sequence_attention_zigzag_amd.build``).
Calls raise ``UspError`` on any non-OK status and ``RuntimeError`` when the
library is missing -- there is no fallback path.  torch supplies device
memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# USP_LIBRARY names an alternative build of libusp.so (e.g. a tuning variant);
# by default the in-tree build is loaded.
LIB_PATH = os.environ.get("USP_LIBRARY") or os.path.join(_PKG, "libusp.so")

IMPL = {"basic": 0, "zigzag": 1, "stripe": 2}
MASK = {"empty": 0, "full": 1, "causal": 2, "causal_strict": 3, "positional": 4}
DT = {torch.bfloat16: 0, torch.float32: 1}
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class UspError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"usp error {STATUS.get(status, status)}: {msg}")
        self.status = status


class PosMap(ctypes.Structure):
    _fields_ = [("impl", ctypes.c_int32), ("ring_degree", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("stripe_block", ctypes.c_int32), ("S_global", ctypes.c_int64)]


class RingArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("Hq", ctypes.c_int64),
                ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("window", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("cu_seqlens_dev", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
                ("nseq", ctypes.c_int32), ("impl", ctypes.c_int32), ("ring_degree", ctypes.c_int32),
                ("ulysses_degree", ctypes.c_int32), ("stripe_block", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("ulysses_rank", ctypes.c_int32),
                ("input_order", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("merge_mode", ctypes.c_int32), ("qkv_packed", ctypes.c_int32),
                ("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p),
                ("out_layout", ctypes.c_int32)]


class RingBwdArgs(ctypes.Structure):
    _fields_ = [("fwd", RingArgs), ("dout", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p),
                ("dv", ctypes.c_void_p)]


_lib = None

_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_PM = ctypes.POINTER(PosMap)
_SIGS = {
    "usp_last_error": ([], ctypes.c_char_p),
    "usp_version": ([], ctypes.c_char_p),
    "usp_permute": ([_P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P], _I32),
    "usp_ulysses_relayout": ([_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P], _I32),
    "usp_block_attn_fwd_workspace_size": ([_I64, _I64, _I32, _PM, _PM, _I32, _I32, _I32, _P, _I32], _SZ),
    "usp_block_attn_fwd": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_float, _I32,
                            _PM, _PM, _I32, _I32, _I32, _P, _P, _I32,
                            _I32, _I32, ctypes.c_float, _P, _P, _SZ, _P], _I32),
    "usp_lse_merge": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P], _I32),
    "usp_ring_fwd_workspace_size": ([ctypes.POINTER(RingArgs)], ctypes.c_size_t),
    "usp_ring_fwd": ([ctypes.POINTER(RingArgs), _P, ctypes.c_size_t, _P], _I32),
    "usp_ring_stage": ([ctypes.POINTER(RingArgs), _P, _P, _P, _P], _I32),
    "usp_ring_fwd_noalloc": ([ctypes.POINTER(RingArgs), _P], _I32),
    "usp_ring_bwd_workspace_size": ([ctypes.POINTER(RingBwdArgs)], ctypes.c_size_t),
    "usp_ring_bwd": ([ctypes.POINTER(RingBwdArgs), _P, ctypes.c_size_t, _P], _I32),
    "usp_plan_block": ([_I64, _I64, _I64, _I32, ctypes.POINTER(PosMap), ctypes.POINTER(PosMap), _I32, _I32,
                        _I32, _P, _I32, _I32, _P, _I64, _P, _I64, ctypes.POINTER(_I64),
                        ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_int32),
                        ctypes.POINTER(ctypes.c_int32)], _I32),
    "usp_plan_block_kv": ([_I64, _I64, _I64, _I32, ctypes.POINTER(PosMap), ctypes.POINTER(PosMap), _I32, _I32,
                           _I32, _P, _I32, _P, _I64, _P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                           ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)], _I32),
    "usp_attn_bwd_preprocess": ([_P, _I32, _P, _P, _I64, _I64, _I64, _I64, _P], _I32),
    "usp_block_attn_bwd_workspace_size": ([_I64, _I64, _I32, _PM, _PM, _I32, _I32, _I32, _P, _I32], _SZ),
    "usp_block_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                            ctypes.c_float, _I32, _PM, _PM, _I32, _I32,
                            _I32, _P, _P, _I32, ctypes.c_float, _P, _P, _SZ, _P], _I32),
    "usp_plan_block_device": ([_I64, _I64, _I32, _PM, _PM, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _SZ,
                               ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(_SZ), _P],
                              _I32),
    "usp_decode_split_fwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_float,
                              _I32, _I32, ctypes.c_float, _P, _P], _I32),
    "usp_decode_merge": ([_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _I32, _P, _P], _I32),
    "usp_timing_enable": ([_I32], _I32),
    "usp_timing_reset": ([], _I32),
    "usp_timing_read": ([_I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)], _I32),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded libusp.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m ulysses_sequence_attention_zigzag_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise UspError(status, lib().usp_last_error().decode())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _resolve(stream=None):
    """The torch stream a call is enqueued on (the current one by default)."""
    return stream if stream is not None else torch.cuda.current_stream()


def _on_stream(t: torch.Tensor, s) -> None:
    """Keeps a temporary device tensor from being reused before the work
    enqueued on stream ``s`` has run (no host synchronisation)."""
    if t is not None and t.is_cuda:
        t.record_stream(s)


def _host_to_device_on(values, dtype, device, s) -> torch.Tensor:
    """A small host list copied to the device in stream order on ``s``."""
    host = torch.tensor(list(values), dtype=dtype)
    with torch.cuda.stream(s):
        dev = host.to(device)
    _on_stream(dev, s)
    return dev


def _workspace(nbytes: int, device, s) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _on_stream(ws, s)
    return ws


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t: torch.Tensor, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def posmap(impl: str, ring_degree: int, rank: int, S_global: int, stripe_block: int = 1) -> PosMap:
    return PosMap(IMPL[impl], ring_degree, rank, stripe_block, S_global)


# ---------------------------------------------------------------- permute
def permute(x: torch.Tensor, impl: str, ring_degree: int, *, ulysses_degree: int = 1, stripe_block: int = 1,
            rank: int = -1, inverse: bool = False, dim: int = 1, S_global: Optional[int] = None,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Token reorder along ``dim`` (see usp_permute).  rank >= 0 extracts
    (or, with inverse, scatters back) global USP rank ``rank``'s shard."""
    dim = dim % x.dim()
    outer = 1
    for s in x.shape[:dim]:
        outer *= s
    inner = 1
    for s in x.shape[dim + 1:]:
        inner *= s
    if rank >= 0 and inverse:
        S = S_global
        if S is None:
            raise ValueError("inverse extract needs S_global")
    else:
        S = x.shape[dim]
    if out is None:
        shape = list(x.shape)
        if rank >= 0:
            shape[dim] = S if inverse else S // ring_degree // ulysses_degree
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _check(lib().usp_permute(_dev(x, name="in"), _dev(out, x.dtype, "out"), outer, S, inner, DT[x.dtype],
                             IMPL[impl], ring_degree, ulysses_degree, stripe_block, rank, int(inverse),
                             _stream(stream)))
    return out


def ulysses_relayout(shards: Sequence[torch.Tensor], local: torch.Tensor, ulysses_rank: int, direction: int,
                     stream=None) -> None:
    """seq -> head (direction 0: shards -> local) or head -> seq (1)."""
    ud = len(shards)
    B, Ls, H, D = shards[0].shape
    arr = (ctypes.c_void_p * ud)(*[_dev(s, local.dtype, "shard").value for s in shards])
    _check(lib().usp_ulysses_relayout(ctypes.cast(arr, ctypes.c_void_p), _dev(local, name="local"), B, Ls, H, D,
                                      DT[local.dtype], ud, ulysses_rank, direction, _stream(stream)))


# ---------------------------------------------------------------- attention
def _cu(cu_seqlens, device, s=None):
    """(device copy, host copy, nseq) of cu_seqlens; the device copy is made in
    stream order on ``s`` and kept alive for the work enqueued there."""
    if cu_seqlens is None:
        return None, None, 0
    vals = list(cu_seqlens) if not torch.is_tensor(cu_seqlens) else cu_seqlens.tolist()
    host = torch.tensor(vals, dtype=torch.int32)
    dev = _host_to_device_on(vals, torch.int32, device, s if s is not None else torch.cuda.current_stream())
    return dev, host, host.numel() - 1


def _slopes(alibi_slopes: Optional[torch.Tensor], H: int):
    """Device pointer of an [H] f32 slope vector (None when not given)."""
    if alibi_slopes is None:
        return None
    if tuple(alibi_slopes.shape) != (H,):
        raise ValueError(f"alibi_slopes must be [{H}]")
    return _dev(alibi_slopes, torch.float32, "alibi_slopes")


def block_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, mask: str = "positional",
                   qmap: Optional[PosMap] = None, kmap: Optional[PosMap] = None, causal: bool = False,
                   window: int = 0, n_sink: int = 0, cu_seqlens=None, softmax_scale: float = 0.0,
                   out_dtype=torch.float32, accumulate: bool = False, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, softcap: float = 0.0,
                   alibi_slopes: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One ring step (usp_block_attn_fwd).  q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] bf16; alibi_slopes [Hq] f32 on
    the device."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty((B, Lq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    s = _resolve(stream)
    cu_dev, cu_host, nseq = _cu(cu_seqlens, q.device, s)
    qm = ctypes.byref(qmap) if qmap else None
    km = ctypes.byref(kmap) if kmap else None
    nbytes = lib().usp_block_attn_fwd_workspace_size(Lq, Lk, MASK[mask], qm, km, int(causal), int(window),
                                                     int(n_sink), _ptr(cu_host), nseq)
    ws = _workspace(nbytes, q.device, s)
    _check(lib().usp_block_attn_fwd(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(out, out_dtype, "out"), _dev(lse, torch.float32, "lse"), B, Lq, Lk, Hq, Hkv, D,
        float(softmax_scale), MASK[mask], qm, km, int(causal), int(window), int(n_sink),
        _ptr(cu_dev), _ptr(cu_host), nseq,
        DT[out.dtype], int(accumulate), float(softcap), _slopes(alibi_slopes, Hq), _ptr(ws), nbytes,
        ctypes.c_void_p(s.cuda_stream)))
    return out, lse


def attn_bwd_preprocess(out: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """delta [B,H,L] f32 = rowsum(dout * out) (usp_attn_bwd_preprocess); out [B,L,H,D] bf16 or f32,
    dout [B,L,H,D] bf16."""
    B, L, H, D = out.shape
    if tuple(dout.shape) != (B, L, H, D):
        raise ValueError("dout must have the shape of out")
    if delta is None:
        delta = torch.empty((B, H, L), dtype=torch.float32, device=out.device)
    _check(lib().usp_attn_bwd_preprocess(_dev(out, None, "out"), DT[out.dtype], _dev(dout, torch.bfloat16, "dout"),
                                         _dev(delta, torch.float32, "delta"), B, L, H, D, _stream(stream)))
    return delta


def block_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                   delta: torch.Tensor, *, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                   dv: Optional[torch.Tensor] = None, mask: str = "positional", qmap: Optional[PosMap] = None,
                   kmap: Optional[PosMap] = None, causal: bool = False, window: int = 0, n_sink: int = 0,
                   cu_seqlens=None, softmax_scale: float = 0.0, softcap: float = 0.0,
                   alibi_slopes: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """One ring step's gradient terms (usp_block_attn_bwd), ADDED into f32 dq [B,Lq,Hq,D] and dk, dv
    [B,Lk,Hkv,D] (zero-initialised here when not given).  q, dout [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] bf16;
    lse, delta [B,Hq,Lq] f32 of the final forward."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if tuple(dout.shape) != (B, Lq, Hq, D):
        raise ValueError("dout must have the shape of q")
    for name, t in (("lse", lse), ("delta", delta)):
        if tuple(t.shape) != (B, Hq, Lq):
            raise ValueError(f"{name} must be [B,Hq,Lq]")
    if dq is None:
        dq = torch.zeros((B, Lq, Hq, D), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.zeros((B, Lk, Hkv, D), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.zeros((B, Lk, Hkv, D), dtype=torch.float32, device=q.device)
    for name, t, shp in (("dq", dq, (B, Lq, Hq, D)), ("dk", dk, (B, Lk, Hkv, D)), ("dv", dv, (B, Lk, Hkv, D))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {list(shp)}")
    s = _resolve(stream)
    cu_dev, cu_host, nseq = _cu(cu_seqlens, q.device, s)
    qm = ctypes.byref(qmap) if qmap else None
    km = ctypes.byref(kmap) if kmap else None
    nbytes = lib().usp_block_attn_bwd_workspace_size(Lq, Lk, MASK[mask], qm, km, int(causal), int(window),
                                                     int(n_sink), _ptr(cu_host), nseq)
    ws = _workspace(nbytes, q.device, s)
    _check(lib().usp_block_attn_bwd(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(dout, torch.bfloat16, "dout"), _dev(lse, torch.float32, "lse"), _dev(delta, torch.float32, "delta"),
        _dev(dq, torch.float32, "dq"), _dev(dk, torch.float32, "dk"), _dev(dv, torch.float32, "dv"),
        B, Lq, Lk, Hq, Hkv, D, float(softmax_scale), MASK[mask], qm, km, int(causal), int(window), int(n_sink),
        _ptr(cu_dev), _ptr(cu_host), nseq, float(softcap),
        _slopes(alibi_slopes, Hq), _ptr(ws), nbytes, ctypes.c_void_p(s.cuda_stream)))
    return dq, dk, dv


def default_split_keys(B: int, S: int, Hkv: int) -> int:
    """Keys per cache piece: up to 1024 (longer streams per wave, fewer partials), but small enough that
    the split kernel runs at least ~2048 waves (8 per CU of the 256, two per SIMD), since one wave handles
    one (piece, batch row, KV head) and the kernel's rate follows the waves per CU."""
    return max(32, min(1024, (S * B * Hkv // 2048) // 32 * 32))


def decode_split_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, kv_lens=None, split_keys: Optional[int] = None,
                     window: int = 0, n_sink: int = 0, softmax_scale: float = 0.0, softcap: float = 0.0,
                     alibi_slopes: Optional[torch.Tensor] = None, out_part=None, lse_part=None,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Partials of the cache pieces (usp_decode_split_fwd): q [B,Lq,Hq,D], cache k / v [B,S,Hkv,D] bf16;
    alibi_slopes [Hq] f32 on the device.  Returns (out_part [n,B,Lq,Hq,D], lse_part [n,B,Hq,Lq]) f32."""
    B, Lq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    if split_keys is None:
        split_keys = default_split_keys(B, S, Hkv)
    n = (S + split_keys - 1) // split_keys
    if out_part is None:
        out_part = torch.empty((n, B, Lq, Hq, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n, B, Hq, Lq), dtype=torch.float32, device=q.device)
    s = _resolve(stream)
    lens_host = lens_dev = None
    if kv_lens is not None:
        vals = [int(x) for x in kv_lens]
        lens_host = torch.tensor(vals, dtype=torch.int32)
        lens_dev = _host_to_device_on(vals, torch.int32, q.device, s)
    _check(lib().usp_decode_split_fwd(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        ctypes.c_void_p(lens_dev.data_ptr()) if lens_dev is not None else None,
        ctypes.c_void_p(lens_host.data_ptr()) if lens_host is not None else None,
        _dev(out_part, torch.float32, "out_part"), _dev(lse_part, torch.float32, "lse_part"),
        B, Lq, S, Hq, Hkv, D, split_keys, float(softmax_scale), int(window), int(n_sink), float(softcap),
        _slopes(alibi_slopes, Hq), ctypes.c_void_p(s.cuda_stream)))
    return out_part, lse_part


def decode_merge(out_part: torch.Tensor, lse_part: torch.Tensor, *, out_dtype=torch.float32, out=None, lse=None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Combines the piece partials (usp_decode_merge): out [B,Lq,Hq,D], lse [B,Hq,Lq].  out_part and
    lse_part are scratch (overwritten when there are more than 64 pieces)."""
    n, B, Lq, Hq, D = out_part.shape
    if out is None:
        out = torch.empty((B, Lq, Hq, D), dtype=out_dtype, device=out_part.device)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=out_part.device)
    _check(lib().usp_decode_merge(_dev(out_part, torch.float32, "out_part"), _dev(lse_part, torch.float32, "lse_part"),
                                  n, B, Lq, Hq, D, _dev(out, None, "out"), DT[out.dtype], _dev(lse, torch.float32, "lse"),
                                  _stream(stream)))
    return out, lse


def decode_fwd(q, k, v, **kw) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode then the merge; keyword arguments of decode_split_fwd plus out_dtype."""
    out_dtype = kw.pop("out_dtype", torch.float32)
    parts = decode_split_fwd(q, k, v, **kw)
    return decode_merge(*parts, out_dtype=out_dtype)


def lse_merge(out_acc: torch.Tensor, lse_acc: torch.Tensor, out_part: torch.Tensor, lse_part: torch.Tensor,
              row_begin: int = 0, row_end: Optional[int] = None, stream=None) -> None:
    """In-place merge of (out_part, lse_part) into (out_acc, lse_acc)."""
    B, L, H, D = out_acc.shape
    row_end = L if row_end is None else row_end
    _check(lib().usp_lse_merge(_dev(out_acc, torch.float32, "out_acc"), _dev(lse_acc, torch.float32, "lse_acc"),
                               _dev(out_part, torch.float32, "out_part"), _dev(lse_part, torch.float32, "lse_part"),
                               B, L, H, D, row_begin, row_end, _stream(stream)))


class RingCall:
    """A prepared usp_ring_fwd call: arguments, outputs and workspace are
    allocated once; ``run()`` only enqueues the kernels."""

    def __init__(self, q: torch.Tensor, k: Optional[torch.Tensor], v: Optional[torch.Tensor], *, impl: str,
                 ring_degree: int, ulysses_degree: int = 1, stripe_block: int = 1, causal: bool = False,
                 window: int = 0, n_sink: int = 0, cu_seqlens=None, softmax_scale: float = 0.0, rank: int = -1,
                 ulysses_rank: int = 0, input_order: str = "natural", out_dtype=torch.float32,
                 merge_mode: int = 0, qkv_packed: bool = False, softcap: float = 0.0,
                 alibi_slopes: Optional[torch.Tensor] = None, out_layout: str = "heads",
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
        """q, k, v as [B,S,H,D] (varlen [T,H,D]); with qkv_packed, q is the packed [B,S,3,H,D] (varlen
        [T,3,H,D]) tensor and k, v are None.  alibi_slopes: [Hq] f32 on the device, over all heads.
        out_layout (one rank's share): "heads" -> out [B,L,Hq/ud,D], lse [B,Hq/ud,L] (head group u);
        "seq" -> out [B,L,Hq,D], lse [B,Hq,L] after the Ulysses head -> seq relayout, of which this
        call writes head group u (``out`` / ``lse`` may be given to let the ud calls share them)."""
        varlen = cu_seqlens is not None
        if qkv_packed:
            if varlen:
                S, _, Hq, D = q.shape
                B = 1
            else:
                B, S, _, Hq, D = q.shape
            Hkv = Hq
        elif varlen:
            S, Hq, D = q.shape
            B = 1
            Hkv = k.shape[1]
        else:
            B, S, Hq, D = q.shape
            Hkv = k.shape[2]
        N, ud = ring_degree, ulysses_degree
        L = S // N
        Hl = Hq // ud
        layout = {"heads": 0, "seq": 1}[out_layout]
        if rank < 0:
            out_shape = (S, Hq, D) if varlen else (B, S, Hq, D)
            lse_shape = (Hq, S) if varlen else (B, Hq, S)
        else:
            Ho = Hq if layout == 1 else Hl
            out_shape = (L, Ho, D) if varlen else (B, L, Ho, D)
            lse_shape = (Ho, L) if varlen else (B, Ho, L)
        self.q, self.k, self.v = q, k, v
        self.out = out if out is not None else torch.empty(out_shape, dtype=out_dtype, device=q.device)
        self.lse = lse if lse is not None else torch.empty(lse_shape, dtype=torch.float32, device=q.device)
        if tuple(self.out.shape) != out_shape or self.out.dtype != out_dtype:
            raise ValueError(f"out must be {list(out_shape)} {out_dtype}")
        if tuple(self.lse.shape) != lse_shape:
            raise ValueError(f"lse must be {list(lse_shape)}")
        cu_dev, cu_host, nseq = _cu(cu_seqlens, q.device)
        if cu_dev is not None:
            # construction only: the device copy is complete before any stream a run() uses
            torch.cuda.current_stream().synchronize()
        self._cu = (cu_dev, cu_host)
        a = RingArgs()
        a.q = _dev(q, torch.bfloat16, "q").value
        a.k = None if qkv_packed else _dev(k, torch.bfloat16, "k").value
        a.v = None if qkv_packed else _dev(v, torch.bfloat16, "v").value
        a.qkv_packed = int(bool(qkv_packed))
        a.out, a.lse = self.out.data_ptr(), self.lse.data_ptr()
        a.B, a.S, a.Hq, a.Hkv, a.D = B, S, Hq, Hkv, D
        a.softmax_scale = float(softmax_scale)
        a.causal, a.window, a.n_sink = int(causal), int(window), int(n_sink)
        a.cu_seqlens_dev = cu_dev.data_ptr() if cu_dev is not None else None
        a.cu_seqlens_host = cu_host.data_ptr() if cu_host is not None else None
        a.nseq = nseq
        a.impl, a.ring_degree, a.ulysses_degree, a.stripe_block = IMPL[impl], N, ud, stripe_block
        a.rank, a.ulysses_rank = rank, ulysses_rank
        a.input_order = {"natural": 0, "permuted": 1}[input_order]
        a.out_dtype = DT[out_dtype]
        a.merge_mode = merge_mode
        a.softcap = float(softcap)
        sp = _slopes(alibi_slopes, Hq)
        a.alibi_slopes = sp.value if sp is not None else None
        a.out_layout = layout
        self.alibi_slopes = alibi_slopes
        self.args = a
        self.q_rows = L if rank >= 0 else S
        self.Hl, self.Hkl = Hl, Hkv // ud
        self.B_, self.S_, self.D_ = B, S, D
        nbytes = lib().usp_ring_fwd_workspace_size(ctypes.byref(a))
        if nbytes == 0:
            # either nothing is needed or the arguments are invalid: let the call report which
            self.workspace = None
        else:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        self.ws_bytes = nbytes

    def run(self, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        ws = ctypes.c_void_p(self.workspace.data_ptr()) if self.workspace is not None else None
        _check(lib().usp_ring_fwd(ctypes.byref(self.args), ws, self.ws_bytes, _stream(stream)))
        return self.out, self.lse

    def stage(self, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """The q, k, v rows exactly as this call's attention kernels read them (usp_ring_stage):
        q [B, rows, Hq/ud, D] (rows = L for one rank, S for all), k / v [B, S, Hkv/ud, D] rank-major;
        varlen drops B."""
        dev = self.q.device
        qs = torch.empty((self.B_, self.q_rows, self.Hl, self.D_), dtype=torch.bfloat16, device=dev)
        ks = torch.empty((self.B_, self.S_, self.Hkl, self.D_), dtype=torch.bfloat16, device=dev)
        vs = torch.empty_like(ks)
        _check(lib().usp_ring_stage(ctypes.byref(self.args), _ptr(qs), _ptr(ks), _ptr(vs), _stream(stream)))
        if self._cu[0] is not None:
            qs, ks, vs = qs[0], ks[0], vs[0]
        return qs, ks, vs

    def capture(self) -> "torch.cuda.CUDAGraph":
        """Records one usp_ring_fwd call into a HIP graph (torch.cuda.CUDAGraph) over this call's
        buffers.  The call only enqueues kernels (its tile plans are built on the device), so it is
        recorded as it stands; ``graph.replay()`` reruns it on the same inputs / outputs."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(stream=torch.cuda.current_stream())
        return graph


class RingBwdCall:
    """A prepared usp_ring_bwd call for the forward described by ``fwd`` (a
    RingCall that has run): dout has the shape of fwd.out; gradients are
    allocated once; ``run()`` only enqueues the kernels."""

    def __init__(self, fwd: RingCall, dout: torch.Tensor):
        if tuple(dout.shape) != tuple(fwd.out.shape):
            raise ValueError("dout must have the shape of the forward output")
        a = fwd.args
        self.fwd, self.dout = fwd, dout
        dev = fwd.q.device
        varlen = fwd._cu[0] is not None
        N, ud = a.ring_degree, a.ulysses_degree
        L = a.S // N
        if a.rank < 0:
            dq_shape, kv_rows = (a.B, a.S, a.Hq, a.D), a.S
        else:
            dq_shape, kv_rows = (a.B, L, a.Hq // ud, a.D), a.S
        kv_shape = (a.B, kv_rows, a.Hkv // ud, a.D)
        if varlen:
            dq_shape, kv_shape = dq_shape[1:], kv_shape[1:]
        self.dq = torch.empty(dq_shape, dtype=torch.float32, device=dev)
        self.dk = torch.empty(kv_shape, dtype=torch.float32, device=dev)
        self.dv = torch.empty(kv_shape, dtype=torch.float32, device=dev)
        b = RingBwdArgs()
        b.fwd = a
        b.dout = _dev(dout, torch.bfloat16, "dout").value
        b.dq, b.dk, b.dv = self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr()
        self.args = b
        nbytes = lib().usp_ring_bwd_workspace_size(ctypes.byref(b))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.ws_bytes = nbytes

    def run(self, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        _check(lib().usp_ring_bwd(ctypes.byref(self.args), ctypes.c_void_p(self.workspace.data_ptr()),
                                  self.ws_bytes, _stream(stream)))
        return self.dq, self.dk, self.dv

    def capture(self) -> "torch.cuda.CUDAGraph":
        """Records one usp_ring_bwd call into a HIP graph (see RingCall.capture); the gradients are
        zeroed by a kernel inside the call, so replays recompute them."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(stream=torch.cuda.current_stream())
        return graph


def ring_fwd(q, k, v, **kw) -> Tuple[torch.Tensor, torch.Tensor]:
    """All ring steps on one device (usp_ring_fwd); see RingCall for arguments."""
    call = RingCall(q, k, v, **kw)
    out = call.run()
    # the workspace goes back to torch's stream-ordered cache, so later work on this stream is
    # ordered after the call; other streams may not reuse it before the call has run
    _on_stream(call.workspace, torch.cuda.current_stream())
    return out


# ---------------------------------------------------------------- timing
KERNEL_CLASSES = {"attn": 0, "permute": 1, "relayout": 2, "merge": 3, "bwd_dq": 4, "bwd_dkdv": 5,
                  "bwd_delta": 6, "decode": 7, "decode_merge": 8, "plan": 9}


def timing_enable(on: bool = True) -> None:
    _check(lib().usp_timing_enable(int(on)))


def timing_reset() -> None:
    _check(lib().usp_timing_reset())


def timing_read(kernel_class: str) -> Tuple[float, int]:
    """(total milliseconds, launches) recorded for one kernel class."""
    ms = ctypes.c_double(0.0)
    n = _I64(0)
    _check(lib().usp_timing_read(KERNEL_CLASSES[kernel_class], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------- planner
def plan_block(Lq: int, Lk: int, D: int = 128, *, mask: str = "positional", qmap: Optional[PosMap] = None,
               kmap: Optional[PosMap] = None, causal: bool = False, window: int = 0, n_sink: int = 0,
               cu_seqlens=None, accumulate: bool = False):
    """Host-only tile plan (usp_plan_block): (items [n,8] int32, runs [m,4] int32, tile_m, tile_n)."""
    L = lib()
    cu_host = None if cu_seqlens is None else torch.tensor(list(cu_seqlens), dtype=torch.int32)
    nseq = 0 if cu_host is None else cu_host.numel() - 1
    cu_p = ctypes.c_void_p(cu_host.data_ptr()) if cu_host is not None else None
    ni, nr = _I64(0), _I64(0)
    tm, tn = ctypes.c_int32(0), ctypes.c_int32(0)
    qm = ctypes.byref(qmap) if qmap else None
    km = ctypes.byref(kmap) if kmap else None
    _check(L.usp_plan_block(Lq, Lk, D, MASK[mask], qm, km, int(causal), int(window), int(n_sink), cu_p, nseq,
                            int(accumulate), None, 0, None, 0, ctypes.byref(ni), ctypes.byref(nr),
                            ctypes.byref(tm), ctypes.byref(tn)))
    items = torch.zeros((max(1, ni.value), 8), dtype=torch.int32)
    runs = torch.zeros((max(1, nr.value), 4), dtype=torch.int32)
    _check(L.usp_plan_block(Lq, Lk, D, MASK[mask], qm, km, int(causal), int(window), int(n_sink), cu_p, nseq,
                            int(accumulate), ctypes.c_void_p(items.data_ptr()), ni.value,
                            ctypes.c_void_p(runs.data_ptr()), nr.value, ctypes.byref(ni), ctypes.byref(nr),
                            ctypes.byref(tm), ctypes.byref(tn)))
    return items[:ni.value], runs[:nr.value], tm.value, tn.value


def plan_block_kv(Lq: int, Lk: int, D: int = 128, *, mask: str = "positional", qmap: Optional[PosMap] = None,
                  kmap: Optional[PosMap] = None, causal: bool = False, window: int = 0, n_sink: int = 0,
                  cu_seqlens=None):
    """Host-only transposed plan of the dK / dV kernel (usp_plan_block_kv):
    (items [n,8] int32, runs [m,4] int32, tile_k, tile_q)."""
    L = lib()
    cu_host = None if cu_seqlens is None else torch.tensor(list(cu_seqlens), dtype=torch.int32)
    nseq = 0 if cu_host is None else cu_host.numel() - 1
    cu_p = ctypes.c_void_p(cu_host.data_ptr()) if cu_host is not None else None
    ni, nr = _I64(0), _I64(0)
    tk, tq = ctypes.c_int32(0), ctypes.c_int32(0)
    qm = ctypes.byref(qmap) if qmap else None
    km = ctypes.byref(kmap) if kmap else None
    _check(L.usp_plan_block_kv(Lq, Lk, D, MASK[mask], qm, km, int(causal), int(window), int(n_sink), cu_p, nseq,
                               None, 0, None, 0, ctypes.byref(ni), ctypes.byref(nr), ctypes.byref(tk),
                               ctypes.byref(tq)))
    items = torch.zeros((max(1, ni.value), 8), dtype=torch.int32)
    runs = torch.zeros((max(1, nr.value), 4), dtype=torch.int32)
    _check(L.usp_plan_block_kv(Lq, Lk, D, MASK[mask], qm, km, int(causal), int(window), int(n_sink), cu_p, nseq,
                               ctypes.c_void_p(items.data_ptr()), ni.value, ctypes.c_void_p(runs.data_ptr()),
                               nr.value, ctypes.byref(ni), ctypes.byref(nr), ctypes.byref(tk), ctypes.byref(tq)))
    return items[:ni.value], runs[:nr.value], tk.value, tq.value


def plan_block_device(Lq: int, Lk: int, *, mask: str = "positional", qmap: Optional[PosMap] = None,
                      kmap: Optional[PosMap] = None, causal: bool = False, window: int = 0, n_sink: int = 0,
                      cu_seqlens=None, accumulate: bool = False, kv_tiles: bool = False, device="cuda"):
    """The device planner's plan of one block (usp_plan_block_device), read back:
    (items [n,8] int32 in the kernels' order, runs [n*slots,4] int32, run_slots)."""
    L = lib()
    s = torch.cuda.current_stream()
    cu_dev, cu_host, nseq = _cu(cu_seqlens, device, s)
    qm = ctypes.byref(qmap) if qmap else None
    km = ctypes.byref(kmap) if kmap else None
    n, slots, need = _I64(0), ctypes.c_int32(0), _SZ(0)
    args = (Lq, Lk, MASK[mask], qm, km, int(causal), int(window), int(n_sink), _ptr(cu_dev), _ptr(cu_host), nseq,
            int(accumulate), int(kv_tiles))
    _check(L.usp_plan_block_device(*args, None, 0, ctypes.byref(n), ctypes.byref(slots), ctypes.byref(need),
                                   ctypes.c_void_p(s.cuda_stream)))
    ws = torch.zeros(max(1, need.value), dtype=torch.uint8, device=device)
    _check(L.usp_plan_block_device(*args, _ptr(ws), need.value, ctypes.byref(n), ctypes.byref(slots),
                                   ctypes.byref(need), ctypes.c_void_p(s.cuda_stream)))
    torch.cuda.synchronize()
    nc = n.value
    roff = (nc * 32 + 255) // 256 * 256
    items = ws[:nc * 32].view(torch.int32).view(nc, 8).cpu()
    runs = ws[roff:roff + nc * slots.value * 16].view(torch.int32).view(-1, 4).cpu()
    return items, runs, slots.value
