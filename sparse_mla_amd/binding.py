"""ctypes binding of libmla_decode (include/mla_decode.h), one function per
C entry point with the same name.  Argument marshalling only: every step of
the decode runs in the library's HIP kernels; torch provides device memory
and the current stream.  Importing this module loads the library and raises
if it has not been built (``python -m sparse_mla_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_DECODE_LIB selects another build of the same library (e.g. a debug build).
LIB_PATH = os.environ.get("MLA_DECODE_LIB", os.path.join(_HERE, "libmla_decode.so"))

MLA_FLAG_VALIDATE = 1
MLA_FLAG_WRITE_SCORES = 2
MLA_DEV_INDEX_OUT_OF_RANGE = 1
MLA_DEV_DUPLICATE_INDEX = 2
MLA_DEV_EMPTY_SELECTION = 4
HEADS, NOPE, ROPE, LATENT, VALUE = 128, 128, 64, 512, 128
MAX_SLOTS_PER_SPLIT = 1024

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_mla_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _i64, _u32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)


def _sig(name, res, args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = args
    return fn


_abi_version = _sig("mla_abi_version", ctypes.c_int, [])
_status_string = _sig("mla_status_string", ctypes.c_char_p, [ctypes.c_int])
_last_hip_error = _sig("mla_last_hip_error", ctypes.c_int, [])
_plan = _sig("mla_plan", ctypes.c_int, [_i32, _i32, _i32, _i32, ctypes.POINTER(_i32)])
_workspace_bytes = _sig("mla_workspace_bytes", _sz, [_i32, _i32])
_absorb = _sig("mla_absorb_q", ctypes.c_int, [_p, _i64, _i64, _p, _p, _i32, _p])
_decode = _sig("mla_sparse_decode", ctypes.c_int, [
    _p, _p, _i64, _i64,            # q_abs q_pe q_pe_sb q_pe_sh
    _p, _i64, _i64,                # kv kv_sb kv_st
    _p, _i64, _i64,                # pe pe_sb pe_st
    _p, _i32,                      # seq_lens max_len
    _p, _i32, _f32, _i32,          # indices k_max scale B
    _i32, _p, _sz,                 # num_splits workspace ws_bytes
    _p, _p,                        # o_latent lse
    _u32, _p, _i64,                # flags bitmap bitmap_words
    _p, _p, _p,                    # scores status stream
])
_combine = _sig("mla_combine", ctypes.c_int, [_p, _sz, _i32, _i32, _p, _p, _p, _p])
_value_up = _sig("mla_value_up", ctypes.c_int, [_p, _p, _p, _i64, _i64, _i32, _p])
_combine_value_up = _sig("mla_combine_value_up", ctypes.c_int,
                         [_p, _sz, _i32, _i32, _p, _p, _i64, _i64, _p, _p, _p])
_dequant = _sig("mla_dequant_wkv_b_fp8", ctypes.c_int, [_p, _p, _p, _p])
_output_proj = _sig("mla_output_proj", ctypes.c_int, [_p, _i64, _p, _p, _i64, _i32, _p])
MODEL_DIM = 7168


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _status_string(status).decode()
        if status == 6:
            msg += f" (hipError {_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        raise MLAError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (ROCm) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dim")


def _bsh(t: torch.Tensor):
    """(B, H, D) view strides of a [B, H, D] or [B, 1, H, D] tensor."""
    if t.dim() == 4:
        if t.shape[1] != 1:
            raise ValueError("only one query position per sequence (decode)")
        return t.shape[0], t.shape[2], t.stride(0), t.stride(2)
    return t.shape[0], t.shape[1], t.stride(0), t.stride(1)


def mla_abi_version() -> int:
    return _abi_version()


def mla_plan(B: int, k_max: int, dense: bool, num_cus: Optional[int] = None):
    """Key splits per sequence for a launch."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count \
            if torch.cuda.is_available() else 256
    s = _i32()
    _check("mla_plan", _plan(B, k_max, int(bool(dense)), num_cus, ctypes.byref(s)))
    return s.value


def mla_workspace_bytes(B: int, num_splits: int) -> int:
    return int(_workspace_bytes(B, num_splits))


def mla_absorb_q(q_nope: torch.Tensor, wkv_b: torch.Tensor, q_abs: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    _need(q_nope, "q_nope", torch.bfloat16)
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    B, H, sb, sh = _bsh(q_nope)
    if H != HEADS or q_nope.shape[-1] != NOPE or tuple(wkv_b.shape) != (HEADS * (NOPE + VALUE), LATENT):
        raise ValueError("shape mismatch with the fixed model dimensions")
    if not wkv_b.is_contiguous():
        raise ValueError("wkv_b must be contiguous")
    if q_abs is None:
        q_abs = torch.empty((B, HEADS, LATENT), dtype=torch.bfloat16, device=q_nope.device)
    _need(q_abs, "q_abs", torch.bfloat16, 3)
    if tuple(q_abs.shape) != (B, HEADS, LATENT) or not q_abs.is_contiguous():
        raise ValueError("q_abs must be a contiguous [B,128,512] tensor")
    _check("mla_absorb_q", _absorb(_ptr(q_nope), sb, sh, _ptr(wkv_b), _ptr(q_abs), B, _stream(stream)))
    return q_abs


def mla_sparse_decode(q_abs, q_pe, kv, pe, seq_lens, max_len: int, indices, scale: float,
                      num_splits: int, workspace, o_latent, lse=None,
                      flags: int = 0, bitmap=None, scores=None, status=None, k_max=None, stream=None):
    """kv [B, L, >=512 cols used as 512] and pe [B, L, 64] views (any strides with
    a unit last stride); indices int32 [B, k] or None (dense, k_max = max_len)."""
    _need(q_abs, "q_abs", torch.bfloat16, 3)
    _need(q_pe, "q_pe", torch.bfloat16)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(pe, "pe", torch.bfloat16, 3)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B = q_abs.shape[0]
    Bq, Hq, qsb, qsh = _bsh(q_pe)
    if Bq != B or Hq != HEADS or q_pe.shape[-1] != ROPE or kv.shape[-1] != LATENT or pe.shape[-1] != ROPE:
        raise ValueError("shape mismatch with the fixed model dimensions")
    if kv.shape[0] < B or pe.shape[0] < B or seq_lens.shape[0] != B or kv.shape[1] < max_len or pe.shape[1] < max_len:
        raise ValueError("cache or seq_lens too small")
    if indices is not None:
        _need(indices, "indices", torch.int32, 2)
        if not indices.is_contiguous() or indices.shape[0] != B:
            raise ValueError("indices must be a contiguous int32 [B, k] tensor")
        k_max = indices.shape[1]
    elif k_max is None:
        k_max = max_len
    words = 0
    if bitmap is not None:
        _need(bitmap, "bitmap", torch.int32, 2)
        words = bitmap.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_sparse_decode", _decode(
        _ptr(q_abs), _ptr(q_pe), qsb, qsh,
        _ptr(kv), kv.stride(0), kv.stride(1),
        _ptr(pe), pe.stride(0), pe.stride(1),
        _ptr(seq_lens), int(max_len),
        _ptr(indices), int(k_max), float(scale), B,
        int(num_splits), _ptr(workspace), ws_bytes,
        _ptr(o_latent), _ptr(lse),
        int(flags), _ptr(bitmap), words,
        _ptr(scores), _ptr(status), _stream(stream)))


def mla_combine(workspace, B: int, num_splits: int, o_latent, lse=None, status=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_combine", _combine(_ptr(workspace), ws_bytes, B, num_splits, _ptr(o_latent), _ptr(lse),
                                   _ptr(status), _stream(stream)))


def mla_value_up(o_latent: torch.Tensor, wkv_b: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    _need(o_latent, "o_latent", torch.bfloat16, 3)
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    B = o_latent.shape[0]
    if not o_latent.is_contiguous() or tuple(o_latent.shape) != (B, HEADS, LATENT):
        raise ValueError("o_latent must be a contiguous [B,128,512] tensor")
    if out is None:
        out = torch.empty((B, 1, HEADS, VALUE), dtype=torch.bfloat16, device=o_latent.device)
    _need(out, "out", torch.bfloat16)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != HEADS or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,128,128] or [B,128,128]")
    _check("mla_value_up", _value_up(_ptr(o_latent), _ptr(wkv_b), _ptr(out), sb, sh, B, _stream(stream)))
    return out


def mla_combine_value_up(workspace, B: int, num_splits: int, wkv_b: torch.Tensor,
                         out: Optional[torch.Tensor] = None, lse=None, status=None, stream=None) -> torch.Tensor:
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    if out is None:
        out = torch.empty((B, 1, HEADS, VALUE), dtype=torch.bfloat16, device=wkv_b.device)
    _need(out, "out", torch.bfloat16)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != HEADS or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,128,128] or [B,128,128]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_combine_value_up", _combine_value_up(_ptr(workspace), ws_bytes, B, num_splits, _ptr(wkv_b),
                                                     _ptr(out), sb, sh, _ptr(lse), _ptr(status), _stream(stream)))
    return out


def mla_output_proj(x: torch.Tensor, wo: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """x: the value-up output, bf16 [B, 1, 128, 128] or [B, 16384] (each row's
    16384 values contiguous); wo: bf16 [7168, 16384], contiguous.  Returns
    out bf16 [B, 1, 7168] (or writes `out`, [B, 1, 7168] or [B, 7168])."""
    _need(x, "x", torch.bfloat16)
    _need(wo, "wo", torch.bfloat16, 2)
    B = x.shape[0]
    xf = x.reshape(B, -1)
    if xf.shape[1] != HEADS * VALUE or xf.stride(1) != 1 or xf.data_ptr() != x.data_ptr():
        raise ValueError("x must hold 16384 contiguous values per sequence")
    if tuple(wo.shape) != (MODEL_DIM, HEADS * VALUE) or not wo.is_contiguous():
        raise ValueError("wo must be a contiguous [7168, 16384] tensor")
    if out is None:
        out = torch.empty((B, 1, MODEL_DIM), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16)
    of = out.reshape(B, -1)
    if of.shape[1] != MODEL_DIM or of.stride(1) != 1 or of.data_ptr() != out.data_ptr():
        raise ValueError("out must be [B, 1, 7168] or [B, 7168] with contiguous rows")
    _check("mla_output_proj", _output_proj(_ptr(x), xf.stride(0), _ptr(wo), _ptr(out), of.stride(0), B,
                                           _stream(stream)))
    return out


def mla_dequant_wkv_b_fp8(w_fp8: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    _need(w_fp8, "w_fp8", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 2)
    if tuple(w_fp8.shape) != (HEADS * (NOPE + VALUE), LATENT) or tuple(scales.shape) != (256, 4):
        raise ValueError("w_fp8 must be [32768,512] and scales [256,4]")
    if not (w_fp8.is_contiguous() and scales.is_contiguous()):
        raise ValueError("w_fp8 and scales must be contiguous")
    if out is None:
        out = torch.empty(w_fp8.shape, dtype=torch.bfloat16, device=w_fp8.device)
    _check("mla_dequant_wkv_b_fp8", _dequant(_ptr(w_fp8), _ptr(scales), _ptr(out), _stream(stream)))
    return out


@dataclass
class DecodeBuffers:
    """Device buffers of one decode step for a fixed (B, k_max, plan)."""
    B: int
    k_max: int
    num_splits: int
    q_abs: torch.Tensor
    o_latent: torch.Tensor
    lse: torch.Tensor
    out: torch.Tensor
    workspace: Optional[torch.Tensor]

    @staticmethod
    def allocate(B: int, k_max: int, dense: bool, device="cuda", num_splits=None):
        if num_splits is None:
            num_splits = mla_plan(B, k_max, dense)
        ws = mla_workspace_bytes(B, num_splits)
        return DecodeBuffers(
            B=B, k_max=k_max, num_splits=num_splits,
            q_abs=torch.empty((B, HEADS, LATENT), dtype=torch.bfloat16, device=device),
            o_latent=torch.empty((B, HEADS, LATENT), dtype=torch.bfloat16, device=device),
            lse=torch.empty((B, HEADS), dtype=torch.float32, device=device),
            out=torch.empty((B, 1, HEADS, VALUE), dtype=torch.bfloat16, device=device),
            workspace=torch.empty(ws, dtype=torch.uint8, device=device) if ws else None,
        )


def decode_step(bufs: DecodeBuffers, q_nope, q_pe, kv, pe, wkv_b, seq_lens, max_len, indices, scale,
                flags=0, bitmap=None, scores=None, status=None, stream=None, fused=True) -> torch.Tensor:
    """One decode step enqueued on one stream: absorb, sparse decode, then
    combine + value-up (one fused launch when there are splits and ``fused``;
    with fused, bufs.o_latent is not written when num_splits > 1)."""
    mla_absorb_q(q_nope, wkv_b, bufs.q_abs, stream=stream)
    mla_sparse_decode(bufs.q_abs, q_pe, kv, pe, seq_lens, max_len, indices, scale,
                      bufs.num_splits, bufs.workspace, bufs.o_latent, bufs.lse,
                      flags=flags, bitmap=bitmap, scores=scores, status=status,
                      k_max=bufs.k_max, stream=stream)
    if bufs.num_splits > 1 and fused:
        mla_combine_value_up(bufs.workspace, bufs.B, bufs.num_splits, wkv_b, bufs.out, lse=bufs.lse,
                             status=status, stream=stream)
    else:
        mla_combine(bufs.workspace, bufs.B, bufs.num_splits, bufs.o_latent, bufs.lse, status=status,
                    stream=stream)
        mla_value_up(bufs.o_latent, wkv_b, bufs.out, stream=stream)
    return bufs.out
