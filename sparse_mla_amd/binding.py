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
MAX_SLOTS_PER_SPLIT = 2048

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
_workspace_bytes_h = _sig("mla_workspace_bytes_heads", _sz, [_i32, _i32, _i32])
_absorb_h = _sig("mla_absorb_q_heads", ctypes.c_int, [_i32, _p, _i64, _i64, _p, _p, _i32, _p])
_decode_h = _sig("mla_sparse_decode_heads", ctypes.c_int, [_i32] + [
    _p, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _i32, _f32, _i32,
    _i32, _p, _sz, _p, _p, _u32, _p, _i64, _p, _p, _p])
_combine_h = _sig("mla_combine_heads", ctypes.c_int, [_i32, _p, _sz, _i32, _i32, _p, _p, _p, _p])
_value_up_h = _sig("mla_value_up_heads", ctypes.c_int, [_i32, _p, _p, _p, _i64, _i64, _i32, _p])
_combine_value_up_h = _sig("mla_combine_value_up_heads", ctypes.c_int,
                           [_i32, _p, _sz, _i32, _i32, _p, _p, _i64, _i64, _p, _p, _p])
HEAD_COUNTS = (16, 32, 64, 128)
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
_decode_noalloc = _sig("mla_sparse_decode_noalloc", ctypes.c_int, [
    _p, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _i32, _f32, _i32,
    _i32, _p, _p, _u32, _p, _i64, _p, _p, _p,
])
_noalloc_scratch_bytes = _sig("mla_noalloc_scratch_bytes", _sz, [])
_prefill_ws = _sig("mla_prefill_workspace_bytes", _sz, [_i32, _i32, _i32])
_prefill = _sig("mla_sparse_prefill", ctypes.c_int, [
    _p, _i64, _i64, _p, _i64, _i64,  # q_nope st sh, q_pe st sh
    _p, _i64, _i64, _p, _i64, _i64,  # kv sb st, pe sb st
    _p, _p, _i32, _f32,              # wkv_b indices k_max scale
    _i32, _i32, _i32, _p, _sz,       # B T num_splits workspace ws_bytes
    _p, _i64, _i64, _p,              # out st sh lse
    _u32, _p, _i64, _p, _p,          # flags bitmap words status stream
])
_combine = _sig("mla_combine", ctypes.c_int, [_p, _sz, _i32, _i32, _p, _p, _p, _p])
_value_up = _sig("mla_value_up", ctypes.c_int, [_p, _p, _p, _i64, _i64, _i32, _p])
_combine_value_up = _sig("mla_combine_value_up", ctypes.c_int,
                         [_p, _sz, _i32, _i32, _p, _p, _i64, _i64, _p, _p, _p])
_dequant = _sig("mla_dequant_wkv_b_fp8", ctypes.c_int, [_p, _p, _p, _p])
_absorb_fp8 = _sig("mla_absorb_q_fp8", ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _i32, _p, _p])
_value_up_fp8 = _sig("mla_value_up_fp8", ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i32, _p, _p])
_combine_value_up_fp8 = _sig("mla_combine_value_up_fp8", ctypes.c_int,
                             [_p, _sz, _i32, _i32, _p, _p, _p, _i64, _i64, _p, _p, _p])
_output_proj = _sig("mla_output_proj", ctypes.c_int, [_p, _i64, _p, _p, _i64, _i32, _p])
_output_proj_pack = _sig("mla_output_proj_pack", ctypes.c_int, [_p, _p, _p])
_output_proj_packed = _sig("mla_output_proj_packed", ctypes.c_int, [_p, _i64, _p, _p, _i64, _i32, _p])
_output_proj_split_ws = _sig("mla_output_proj_split_workspace_bytes", _sz, [_i32])
_output_proj_split = _sig("mla_output_proj_split", ctypes.c_int, [_p, _i64, _p, _p, _i64, _i32, _p, _sz, _p])
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


def mla_workspace_bytes(B: int, num_splits: int, heads: int = HEADS) -> int:
    return int(_workspace_bytes_h(heads, B, num_splits))


def _heads(H: int) -> int:
    if H not in HEAD_COUNTS:
        raise ValueError(f"head count {H} not one of {HEAD_COUNTS}")
    return H


def mla_absorb_q(q_nope: torch.Tensor, wkv_b: torch.Tensor, q_abs: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """q_nope [B, 1, H, 128] or [B, H, 128] with H = 128 or a head-sharded
    share (16, 32, 64; wkv_b then holds those heads' H * 256 rows)."""
    _need(q_nope, "q_nope", torch.bfloat16)
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    B, H, sb, sh = _bsh(q_nope)
    _heads(H)
    if q_nope.shape[-1] != NOPE or tuple(wkv_b.shape) != (H * (NOPE + VALUE), LATENT):
        raise ValueError("shape mismatch with the fixed model dimensions")
    if not wkv_b.is_contiguous():
        raise ValueError("wkv_b must be contiguous")
    if q_abs is None:
        q_abs = torch.empty((B, H, LATENT), dtype=torch.bfloat16, device=q_nope.device)
    _need(q_abs, "q_abs", torch.bfloat16, 3)
    if tuple(q_abs.shape) != (B, H, LATENT) or not q_abs.is_contiguous():
        raise ValueError("q_abs must be a contiguous [B,H,512] tensor")
    _check("mla_absorb_q", _absorb_h(H, _ptr(q_nope), sb, sh, _ptr(wkv_b), _ptr(q_abs), B, _stream(stream)))
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
    B, H = q_abs.shape[0], _heads(q_abs.shape[1])
    Bq, Hq, qsb, qsh = _bsh(q_pe)
    if Bq != B or Hq != H or q_pe.shape[-1] != ROPE or kv.shape[-1] != LATENT or pe.shape[-1] != ROPE:
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
    _check("mla_sparse_decode", _decode_h(
        H, _ptr(q_abs), _ptr(q_pe), qsb, qsh,
        _ptr(kv), kv.stride(0), kv.stride(1),
        _ptr(pe), pe.stride(0), pe.stride(1),
        _ptr(seq_lens), int(max_len),
        _ptr(indices), int(k_max), float(scale), B,
        int(num_splits), _ptr(workspace), ws_bytes,
        _ptr(o_latent), _ptr(lse),
        int(flags), _ptr(bitmap), words,
        _ptr(scores), _ptr(status), _stream(stream)))


def mla_noalloc_scratch_bytes() -> int:
    return int(_noalloc_scratch_bytes())


def mla_sparse_decode_noalloc(q_abs, q_pe, kv, pe, seq_lens, max_len: int, indices, scale: float,
                              num_splits: int, o_latent, lse=None, flags: int = 0, bitmap=None, scores=None,
                              status=None, k_max=None, stream=None):
    """mla_sparse_decode with the split partials in the library's static
    scratch and the merge into o_latent / lse done by the same call (no
    workspace argument, no allocation)."""
    _need(q_abs, "q_abs", torch.bfloat16, 3)
    _need(q_pe, "q_pe", torch.bfloat16)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(pe, "pe", torch.bfloat16, 3)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(o_latent, "o_latent", torch.bfloat16, 3)
    B = q_abs.shape[0]
    Bq, Hq, qsb, qsh = _bsh(q_pe)
    if Bq != B or Hq != HEADS or q_pe.shape[-1] != ROPE or kv.shape[-1] != LATENT or pe.shape[-1] != ROPE:
        raise ValueError("shape mismatch with the fixed model dimensions")
    if kv.shape[0] < B or pe.shape[0] < B or seq_lens.shape[0] != B or kv.shape[1] < max_len or pe.shape[1] < max_len:
        raise ValueError("cache or seq_lens too small")
    if tuple(o_latent.shape) != (B, HEADS, LATENT) or not o_latent.is_contiguous():
        raise ValueError("o_latent must be a contiguous [B,128,512] tensor")
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
    _check("mla_sparse_decode_noalloc", _decode_noalloc(
        _ptr(q_abs), _ptr(q_pe), qsb, qsh,
        _ptr(kv), kv.stride(0), kv.stride(1),
        _ptr(pe), pe.stride(0), pe.stride(1),
        _ptr(seq_lens), int(max_len),
        _ptr(indices), int(k_max), float(scale), B,
        int(num_splits), _ptr(o_latent), _ptr(lse),
        int(flags), _ptr(bitmap), words,
        _ptr(scores), _ptr(status), _stream(stream)))


def mla_prefill_workspace_bytes(B: int, T: int, num_splits: int) -> int:
    return int(_prefill_ws(B, T, num_splits))


def _rows_of(t: torch.Tensor, name: str, B: int, T: int, D: int):
    """(row stride, head stride) of a [B, T, 128, D] tensor whose B*T query
    rows are evenly spaced (row r = b*T + s at r * row stride)."""
    if t.dim() != 4 or tuple(t.shape) != (B, T, HEADS, D) or t.stride(-1) != 1:
        raise ValueError(f"{name} must be [B, T, 128, {D}] with unit inner stride")
    if B > 1 and t.stride(0) != T * t.stride(1):
        raise ValueError(f"{name}: the B*T query rows must be evenly spaced")
    return t.stride(1), t.stride(2)


def mla_sparse_prefill(q_nope, q_pe, kv, pe, wkv_b, indices, scale: float, num_splits=None, workspace=None,
                       out=None, lse=None, flags: int = 0, bitmap=None, status=None, stream=None):
    """Sparse prefill of B prompts of T tokens: q_nope [B,T,128,128], q_pe
    [B,T,128,64], kv [B,>=T,512] and pe [B,>=T,64] views of the prompts'
    latent and rotary keys, indices int32 [B,T,k] (or None: every causal
    key).  Returns out bf16 [B,T,128,128]."""
    _need(q_nope, "q_nope", torch.bfloat16)
    _need(q_pe, "q_pe", torch.bfloat16)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(pe, "pe", torch.bfloat16, 3)
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    B, T = q_nope.shape[0], q_nope.shape[1]
    qn_st, qn_sh = _rows_of(q_nope, "q_nope", B, T, NOPE)
    qp_st, qp_sh = _rows_of(q_pe, "q_pe", B, T, ROPE)
    if kv.shape[0] < B or pe.shape[0] < B or kv.shape[1] < T or pe.shape[1] < T or kv.shape[2] != LATENT \
            or pe.shape[2] != ROPE:
        raise ValueError("kv / pe must cover the B prompts' T positions")
    if tuple(wkv_b.shape) != (HEADS * (NOPE + VALUE), LATENT) or not wkv_b.is_contiguous():
        raise ValueError("wkv_b must be a contiguous [32768, 512] tensor")
    if indices is not None:
        _need(indices, "indices", torch.int32, 3)
        if not indices.is_contiguous() or tuple(indices.shape[:2]) != (B, T):
            raise ValueError("indices must be a contiguous int32 [B, T, k] tensor")
        k_max = indices.shape[2]
    else:
        k_max = T
    if num_splits is None:
        num_splits = mla_plan(B * T, k_max, indices is None)
    ws_need = mla_prefill_workspace_bytes(B, T, num_splits)
    if workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q_nope.device)
    if out is None:
        out = torch.empty((B, T, HEADS, VALUE), dtype=torch.bfloat16, device=q_nope.device)
    o_st, o_sh = _rows_of(out, "out", B, T, VALUE)
    words = 0
    if bitmap is not None:
        _need(bitmap, "bitmap", torch.int32, 2)
        words = bitmap.shape[1]
    _check("mla_sparse_prefill", _prefill(
        _ptr(q_nope), qn_st, qn_sh, _ptr(q_pe), qp_st, qp_sh,
        _ptr(kv), kv.stride(0), kv.stride(1), _ptr(pe), pe.stride(0), pe.stride(1),
        _ptr(wkv_b), _ptr(indices), int(k_max), float(scale),
        B, T, int(num_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), o_st, o_sh, _ptr(lse), int(flags), _ptr(bitmap), words, _ptr(status), _stream(stream)))
    return out


def mla_combine(workspace, B: int, num_splits: int, o_latent, lse=None, status=None, stream=None):
    """The heads come from o_latent [B, H, 512]."""
    H = _heads(o_latent.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_combine", _combine_h(H, _ptr(workspace), ws_bytes, B, num_splits, _ptr(o_latent), _ptr(lse),
                                     _ptr(status), _stream(stream)))


def mla_value_up(o_latent: torch.Tensor, wkv_b: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    _need(o_latent, "o_latent", torch.bfloat16, 3)
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    B, H = o_latent.shape[0], _heads(o_latent.shape[1])
    if not o_latent.is_contiguous() or tuple(o_latent.shape) != (B, H, LATENT):
        raise ValueError("o_latent must be a contiguous [B,H,512] tensor")
    if tuple(wkv_b.shape) != (H * (NOPE + VALUE), LATENT):
        raise ValueError("wkv_b must hold the H heads' rows")
    if out is None:
        out = torch.empty((B, 1, H, VALUE), dtype=torch.bfloat16, device=o_latent.device)
    _need(out, "out", torch.bfloat16)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != H or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,H,128] or [B,H,128]")
    _check("mla_value_up", _value_up_h(H, _ptr(o_latent), _ptr(wkv_b), _ptr(out), sb, sh, B, _stream(stream)))
    return out


def mla_combine_value_up(workspace, B: int, num_splits: int, wkv_b: torch.Tensor,
                         out: Optional[torch.Tensor] = None, lse=None, status=None, stream=None) -> torch.Tensor:
    """The heads come from wkv_b's rows (H * 256)."""
    _need(wkv_b, "wkv_b", torch.bfloat16, 2)
    H = _heads(wkv_b.shape[0] // (NOPE + VALUE))
    if out is None:
        out = torch.empty((B, 1, H, VALUE), dtype=torch.bfloat16, device=wkv_b.device)
    _need(out, "out", torch.bfloat16)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != H or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,H,128] or [B,H,128]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_combine_value_up", _combine_value_up_h(H, _ptr(workspace), ws_bytes, B, num_splits, _ptr(wkv_b),
                                                       _ptr(out), sb, sh, _ptr(lse), _ptr(status), _stream(stream)))
    return out


def _output_proj_args(x, wo, out):
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
    return B, xf.stride(0), out, of.stride(0)


def mla_output_proj(x: torch.Tensor, wo: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """x: the value-up output, bf16 [B, 1, 128, 128] or [B, 16384] (each row's
    16384 values contiguous); wo: bf16 [7168, 16384], contiguous.  Returns
    out bf16 [B, 1, 7168] (or writes `out`, [B, 1, 7168] or [B, 7168])."""
    B, x_sb, out, out_sb = _output_proj_args(x, wo, out)
    _check("mla_output_proj", _output_proj(_ptr(x), x_sb, _ptr(wo), _ptr(out), out_sb, B, _stream(stream)))
    return out


def mla_output_proj_pack(wo: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The output-projection weight repacked for mla_output_proj_packed (one-time
    set-up): a bf16 tensor of wo's shape holding the same values in groups of
    28 rows stored chunk by chunk."""
    _need(wo, "wo", torch.bfloat16, 2)
    if tuple(wo.shape) != (MODEL_DIM, HEADS * VALUE) or not wo.is_contiguous():
        raise ValueError("wo must be a contiguous [7168, 16384] tensor")
    if out is None:
        out = torch.empty_like(wo)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != tuple(wo.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [7168, 16384] tensor")
    _check("mla_output_proj_pack", _output_proj_pack(_ptr(wo), _ptr(out), _stream(stream)))
    return out


def mla_output_proj_packed(x: torch.Tensor, wo_packed: torch.Tensor, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """mla_output_proj with the weight from mla_output_proj_pack (bit-identical
    result)."""
    B, x_sb, out, out_sb = _output_proj_args(x, wo_packed, out)
    _check("mla_output_proj_packed", _output_proj_packed(_ptr(x), x_sb, _ptr(wo_packed), _ptr(out), out_sb, B,
                                                         _stream(stream)))
    return out


def mla_output_proj_split_workspace_bytes(B: int) -> int:
    return int(_output_proj_split_ws(B))


def mla_output_proj_split(x: torch.Tensor, wo: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mla_output_proj with the inputs split in four (fp32 partial sums in
    `workspace`, a uint8 tensor of at least mla_output_proj_split_workspace_bytes(B)
    bytes, allocated here when not given); same arguments and result up to
    the rounding order of the fp32 sums."""
    B, x_sb, out, out_sb = _output_proj_args(x, wo, out)
    if workspace is None:
        workspace = torch.empty(mla_output_proj_split_workspace_bytes(B), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check("mla_output_proj_split", _output_proj_split(_ptr(x), x_sb, _ptr(wo), _ptr(out), out_sb, B,
                                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def _need_fp8_weight(w_fp8, w_scale):
    _need(w_fp8, "w_fp8", torch.uint8, 2)
    _need(w_scale, "w_scale", torch.float32, 2)
    if tuple(w_fp8.shape) != (HEADS * (NOPE + VALUE), LATENT) or tuple(w_scale.shape) != (256, 4):
        raise ValueError("w_fp8 must be [32768,512] and w_scale [256,4]")
    if not (w_fp8.is_contiguous() and w_scale.is_contiguous()):
        raise ValueError("w_fp8 and w_scale must be contiguous")


def mla_absorb_q_fp8(q_nope, w_fp8, w_scale, q_abs=None, w_formed=None, stream=None):
    """mla_absorb_q with the block-scaled fp8 weight read directly."""
    _need(q_nope, "q_nope", torch.bfloat16)
    _need_fp8_weight(w_fp8, w_scale)
    B, H, sb, sh = _bsh(q_nope)
    if H != HEADS or q_nope.shape[-1] != NOPE:
        raise ValueError("shape mismatch with the fixed model dimensions")
    if q_abs is None:
        q_abs = torch.empty((B, HEADS, LATENT), dtype=torch.bfloat16, device=q_nope.device)
    if tuple(q_abs.shape) != (B, HEADS, LATENT) or not q_abs.is_contiguous():
        raise ValueError("q_abs must be a contiguous [B,128,512] tensor")
    _check("mla_absorb_q_fp8", _absorb_fp8(_ptr(q_nope), sb, sh, _ptr(w_fp8), _ptr(w_scale), _ptr(q_abs), B,
                                           _ptr(w_formed), _stream(stream)))
    return q_abs


def mla_value_up_fp8(o_latent, w_fp8, w_scale, out=None, w_formed=None, stream=None):
    """mla_value_up with the block-scaled fp8 weight read directly."""
    _need(o_latent, "o_latent", torch.bfloat16, 3)
    _need_fp8_weight(w_fp8, w_scale)
    B = o_latent.shape[0]
    if not o_latent.is_contiguous() or tuple(o_latent.shape) != (B, HEADS, LATENT):
        raise ValueError("o_latent must be a contiguous [B,128,512] tensor")
    if out is None:
        out = torch.empty((B, 1, HEADS, VALUE), dtype=torch.bfloat16, device=o_latent.device)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != HEADS or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,128,128] or [B,128,128]")
    _check("mla_value_up_fp8", _value_up_fp8(_ptr(o_latent), _ptr(w_fp8), _ptr(w_scale), _ptr(out), sb, sh, B,
                                             _ptr(w_formed), _stream(stream)))
    return out


def mla_combine_value_up_fp8(workspace, B: int, num_splits: int, w_fp8, w_scale, out=None, lse=None, status=None,
                             stream=None):
    """mla_combine_value_up with the block-scaled fp8 weight read directly."""
    _need_fp8_weight(w_fp8, w_scale)
    if out is None:
        out = torch.empty((B, 1, HEADS, VALUE), dtype=torch.bfloat16, device=w_fp8.device)
    Bo, Ho, sb, sh = _bsh(out)
    if Bo != B or Ho != HEADS or out.shape[-1] != VALUE:
        raise ValueError("out must be [B,1,128,128] or [B,128,128]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_combine_value_up_fp8", _combine_value_up_fp8(
        _ptr(workspace), ws_bytes, B, num_splits, _ptr(w_fp8), _ptr(w_scale), _ptr(out), sb, sh, _ptr(lse),
        _ptr(status), _stream(stream)))
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
    def allocate(B: int, k_max: int, dense: bool, device="cuda", num_splits=None, heads: int = HEADS):
        """Buffers for B sequences of `heads` heads (128, or a head-sharded
        share: 16, 32, 64)."""
        if num_splits is None:
            num_splits = mla_plan(B, k_max, dense)
        ws = mla_workspace_bytes(B, num_splits, _heads(heads))
        return DecodeBuffers(
            B=B, k_max=k_max, num_splits=num_splits,
            q_abs=torch.empty((B, heads, LATENT), dtype=torch.bfloat16, device=device),
            o_latent=torch.empty((B, heads, LATENT), dtype=torch.bfloat16, device=device),
            lse=torch.empty((B, heads), dtype=torch.float32, device=device),
            out=torch.empty((B, 1, heads, VALUE), dtype=torch.bfloat16, device=device),
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


class StepLauncher:
    """One decode step's C calls with their arguments marshalled once.

    Built from the same tensors as ``decode_step`` (their dtypes and shapes
    checked here, nothing enqueued), it keeps the raw ctypes argument tuples
    of mla_absorb_q, mla_sparse_decode and mla_combine_value_up (or
    mla_value_up when the plan has one split), so that each step costs three
    foreign calls and no Python-side work; the library still checks every
    argument on each call.  The tensors must stay alive and unchanged while
    the launcher is used.  Calling it enqueues one step on ``stream`` and
    raises on a non-zero status."""

    def __init__(self, bufs: DecodeBuffers, q_nope, q_pe, kv, pe, wkv_b, seq_lens, max_len, indices, scale,
                 stream=None, w_fp8=None, w_scale=None):
        """With w_fp8 and w_scale (and wkv_b None) the step reads the
        block-scaled fp8 weight directly (mla_absorb_q_fp8,
        mla_combine_value_up_fp8 / mla_value_up_fp8)."""
        fp8 = w_fp8 is not None
        if fp8:
            _need_fp8_weight(w_fp8, w_scale)
            wkv_b = w_fp8
        for t, name, dt in ((q_nope, "q_nope", torch.bfloat16), (q_pe, "q_pe", torch.bfloat16),
                            (kv, "kv", torch.bfloat16), (pe, "pe", torch.bfloat16),
                            (wkv_b, "wkv_b", torch.uint8 if fp8 else torch.bfloat16),
                            (seq_lens, "seq_lens", torch.int32)):
            _need(t, name, dt)
        B = bufs.B
        Hq = _bsh(q_nope)[1]
        if (_bsh(q_nope)[:2] != (B, Hq) or _bsh(q_pe)[:2] != (B, Hq) or q_nope.shape[-1] != NOPE
                or q_pe.shape[-1] != ROPE or kv.dim() != 3 or pe.dim() != 3 or kv.shape[-1] != LATENT
                or pe.shape[-1] != ROPE or kv.shape[0] < B or pe.shape[0] < B or seq_lens.shape != (B,)
                or kv.shape[1] < max_len or pe.shape[1] < max_len
                or (not fp8 and tuple(wkv_b.shape) != (Hq * (NOPE + VALUE), LATENT)) or not wkv_b.is_contiguous()):
            raise ValueError("shape mismatch with the fixed model dimensions or the buffers")
        if indices is not None:
            _need(indices, "indices", torch.int32, 2)
            if not indices.is_contiguous() or indices.shape[0] != B:
                raise ValueError("indices must be a contiguous int32 [B, k] tensor")
        st = _stream(stream)
        B = bufs.B
        H = _heads(_bsh(q_nope)[1])
        if fp8 and H != HEADS:
            raise ValueError("the fp8 weight path takes all 128 heads")
        _, _, qn_sb, qn_sh = _bsh(q_nope)
        _, _, qp_sb, qp_sh = _bsh(q_pe)
        _, _, o_sb, o_sh = _bsh(bufs.out)
        ws_bytes = 0 if bufs.workspace is None else bufs.workspace.numel()
        k_max = bufs.k_max if indices is None else indices.shape[1]
        absorb = ((_absorb_fp8, "mla_absorb_q_fp8", (_ptr(q_nope), qn_sb, qn_sh, _ptr(w_fp8), _ptr(w_scale),
                                                     _ptr(bufs.q_abs), B, None, st)) if fp8 else
                  (_absorb_h, "mla_absorb_q", (H, _ptr(q_nope), qn_sb, qn_sh, _ptr(wkv_b), _ptr(bufs.q_abs), B, st)))
        self._calls = [
            absorb,
            (_decode_h, "mla_sparse_decode", (
                H, _ptr(bufs.q_abs), _ptr(q_pe), qp_sb, qp_sh,
                _ptr(kv), kv.stride(0), kv.stride(1), _ptr(pe), pe.stride(0), pe.stride(1),
                _ptr(seq_lens), int(max_len), _ptr(indices), int(k_max), float(scale), B,
                bufs.num_splits, _ptr(bufs.workspace), ws_bytes, _ptr(bufs.o_latent), _ptr(bufs.lse),
                0, None, 0, None, None, st)),
        ]
        if bufs.num_splits > 1 and fp8:
            self._calls.append((_combine_value_up_fp8, "mla_combine_value_up_fp8", (
                _ptr(bufs.workspace), ws_bytes, B, bufs.num_splits, _ptr(w_fp8), _ptr(w_scale), _ptr(bufs.out), o_sb,
                o_sh, _ptr(bufs.lse), None, st)))
        elif bufs.num_splits > 1:
            self._calls.append((_combine_value_up_h, "mla_combine_value_up", (
                H, _ptr(bufs.workspace), ws_bytes, B, bufs.num_splits, _ptr(wkv_b), _ptr(bufs.out), o_sb, o_sh,
                _ptr(bufs.lse), None, st)))
        elif fp8:
            self._calls.append((_value_up_fp8, "mla_value_up_fp8", (
                _ptr(bufs.o_latent), _ptr(w_fp8), _ptr(w_scale), _ptr(bufs.out), o_sb, o_sh, B, None, st)))
        else:
            self._calls.append((_value_up_h, "mla_value_up", (
                H, _ptr(bufs.o_latent), _ptr(wkv_b), _ptr(bufs.out), o_sb, o_sh, B, st)))
        # The separate merge of the split partials (for timing the attention
        # part alone): mla_combine into bufs.o_latent and bufs.lse.
        self._combine = (_combine_h, "mla_combine", (H, _ptr(bufs.workspace), ws_bytes, B, bufs.num_splits,
                                                     _ptr(bufs.o_latent), _ptr(bufs.lse), None, st))

    @staticmethod
    def _run(call):
        fn, name, args = call
        r = fn(*args)
        if r:
            _check(name, r)

    def __call__(self):
        for call in self._calls:
            self._run(call)

    def decode(self):
        """Only the mla_sparse_decode call of the step (reads bufs.q_abs as
        the last absorb left it)."""
        self._run(self._calls[1])

    def combine(self):
        """mla_combine of the split partials (a no-op with one split)."""
        self._run(self._combine)
