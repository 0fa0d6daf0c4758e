"""ctypes loader and argument marshalling for the C oracle (``mla_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Arrays are converted to
float64 here; bf16 and fp8 inputs are decoded by exact type conversion, never
by any arithmetic of the method.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

ORACLE_ERR_INDEX_RANGE = 1
ORACLE_ERR_EMPTY = 4
ORACLE_ERR_ARG = 8

_lib = None


def build(force: bool = True) -> str:
    """Compile ``mla_oracle.c`` with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def load(path: str | None = None):
    """Load the built oracle library, building it first if it is absent.

    ``path`` loads another build of the same source (the tests use this to
    check that deliberately broken copies of the oracle fail the pins)."""
    global _lib
    if path is not None or _lib is None:
        if path is None and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path or _LIB)
        d, i64, p = ctypes.c_double, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            i64, i64, i64, i64, i64, i64,   # B H Dn Dc Dr Dv
            p, p,                           # q_nope q_pe
            p, i64, i64,                    # kv kv_sb kv_st
            p, i64, i64,                    # pe pe_sb pe_st
            p, p, p, i64, d,                # wkv_b seq_lens indices k_max scale
            p, p, p, p,                     # q_abs o_lat out lse
            p, i64,                         # attended att_stride
            p, p,                           # weights scores
        ]
        lib.oracle_dequant_fp8.restype = ctypes.c_int
        lib.oracle_dequant_fp8.argtypes = [p, p, i64, i64, i64, p, p]
        lib.oracle_e4m3_to_double.restype = d
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [d]
        lib.oracle_absorb.restype = ctypes.c_int
        lib.oracle_absorb.argtypes = [i64, i64, i64, i64, i64, p, p, p]
        lib.oracle_value_up.restype = ctypes.c_int
        lib.oracle_value_up.argtypes = [i64, i64, i64, i64, i64, p, p, p]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [
            i64, i64, i64, i64, i64, i64, i64,   # B T H Dn Dc Dr Dv
            p, p,                                # q_nope q_pe
            p, i64, i64,                         # kv kv_sb kv_st
            p, i64, i64,                         # pe pe_sb pe_st
            p, p, i64, d,                        # wkv_b indices k_max scale
            p, p, p,                             # out lse attended
        ]
        lib.oracle_output_proj.restype = ctypes.c_int
        lib.oracle_output_proj.argtypes = [i64, i64, i64, p, p, p]
        if path is not None:
            return lib
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor or array (bf16, fp32, ...) to float64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _np(x, dtype) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(q_nope, q_pe, kv, pe, wkv_b, seq_lens, indices, scale,
           want_weights=False, want_attended=False, att_len=None, lib=None):
    """Run the C oracle.

    Shapes (any float dtype; converted exactly to float64):
      q_nope [B, H, Dn] (a [B, 1, H, Dn] tensor is accepted), q_pe [B, H, Dr],
      kv [B, L, Dc], pe [B, L, Dr], wkv_b [H*(Dn+Dv), Dc],
      seq_lens [B] int, indices [B, k] int or None (dense over t < L_b).

    Returns a dict with q_abs, o_lat, out [B, H, Dv], lse [B, H], status and,
    on request, weights/scores [B, H, k] and attended [B, att_len] (uint8).
    ``lib`` selects another loaded build (default: the built oracle).
    """
    lib = lib or load()
    qn = _f64(q_nope)
    qr = _f64(q_pe)
    if qn.ndim == 4:
        qn = qn.reshape(qn.shape[0], qn.shape[2], qn.shape[3])
        qr = qr.reshape(qr.shape[0], qr.shape[2], qr.shape[3])
    B, H, Dn = qn.shape
    Dr = qr.shape[2]
    kvd = _f64(kv)
    ped = _f64(pe)
    Dc = kvd.shape[2]
    w = _f64(wkv_b)
    Dv = w.shape[0] // H - Dn
    assert w.shape == (H * (Dn + Dv), Dc)
    lens = _np(seq_lens, np.int32)
    assert lens.shape == (B,)
    assert int(lens.max(initial=0)) <= kvd.shape[1], "cache shorter than a sequence length"
    idx = None if indices is None else _np(indices, np.int64)
    k_max = 0 if idx is None else idx.shape[1]
    q_abs = np.empty((B, H, Dc))
    o_lat = np.empty((B, H, Dc))
    out = np.empty((B, H, Dv))
    lse = np.empty((B, H))
    weights = np.empty((B, H, k_max)) if (want_weights and idx is not None) else None
    scores = np.empty((B, H, k_max)) if (want_weights and idx is not None) else None
    att = None
    if want_attended:
        n = int(att_len if att_len is not None else kvd.shape[1])
        assert n >= int(lens.max(initial=0))
        att = np.zeros((B, n), dtype=np.uint8)
    st = lib.oracle_decode(
        B, H, Dn, Dc, Dr, Dv,
        _ptr(qn), _ptr(qr),
        _ptr(kvd), kvd.shape[1] * Dc, Dc,
        _ptr(ped), ped.shape[1] * Dr, Dr,
        _ptr(w), _ptr(lens), _ptr(idx), k_max, float(scale),
        _ptr(q_abs), _ptr(o_lat), _ptr(out), _ptr(lse),
        _ptr(att), 0 if att is None else att.shape[1],
        _ptr(weights), _ptr(scores),
    )
    if st & ORACLE_ERR_ARG:
        raise ValueError("oracle_decode: bad arguments")
    if st & ORACLE_ERR_INDEX_RANGE:
        raise IndexError("oracle_decode: an index is out of range for its sequence")
    res = dict(q_abs=q_abs, o_lat=o_lat, out=out, lse=lse, status=st)
    if weights is not None:
        res["weights"] = weights
        res["scores"] = scores
    if att is not None:
        res["attended"] = att
    return res


def prefill(q_nope, q_pe, kv, pe, wkv_b, indices, scale, want_attended=False, lib=None):
    """Sparse prefill in the full-sequence (MHA) form, fp64.

    q_nope [B, T, H, Dn], q_pe [B, T, H, Dr] (queries of the prompt's T
    positions), kv [B, >=T, Dc], pe [B, >=T, Dr] (latent and rotary key of
    each prompt position; only the first T are keys), wkv_b [H*(Dn+Dv), Dc],
    indices [B, T, k] int (the indexer's selection of each query; -1 is
    padding) or None (every causal key).  Returns a dict with out
    [B, T, H, Dv], lse [B, T, H], status and, on request, attended
    [B, T, T] (uint8)."""
    lib = lib or load()
    qn = _f64(q_nope)
    qr = _f64(q_pe)
    B, T, H, Dn = qn.shape
    Dr = qr.shape[3]
    kvd = _f64(kv)
    ped = _f64(pe)
    Dc = kvd.shape[2]
    assert kvd.shape[1] >= T and ped.shape[1] >= T
    w = _f64(wkv_b)
    Dv = w.shape[0] // H - Dn
    assert w.shape == (H * (Dn + Dv), Dc)
    idx = None if indices is None else _np(indices, np.int64)
    k_max = 0 if idx is None else idx.shape[2]
    if idx is not None:
        assert idx.shape[:2] == (B, T)
    out = np.empty((B, T, H, Dv))
    lse = np.empty((B, T, H))
    att = np.zeros((B, T, T), dtype=np.uint8) if want_attended else None
    st = lib.oracle_prefill(B, T, H, Dn, Dc, Dr, Dv, _ptr(qn), _ptr(qr),
                            _ptr(kvd), kvd.shape[1] * Dc, Dc, _ptr(ped), ped.shape[1] * Dr, Dr,
                            _ptr(w), _ptr(idx), k_max, float(scale), _ptr(out), _ptr(lse), _ptr(att))
    if st & ORACLE_ERR_ARG:
        raise ValueError("oracle_prefill: bad arguments")
    if st & ORACLE_ERR_INDEX_RANGE:
        raise IndexError("oracle_prefill: an index is outside the prompt")
    res = dict(out=out, lse=lse, status=st)
    if att is not None:
        res["attended"] = att
    return res


def _bhd(x):
    a = _f64(x)
    if a.ndim == 4:
        a = a.reshape(a.shape[0], a.shape[2], a.shape[3])
    return np.ascontiguousarray(a)


def absorb(q_nope, wkv_b, lib=None):
    """Step 2 alone: q_abs [B,H,Dc] from q_nope [B,H,Dn] (or [B,1,H,Dn])."""
    lib = lib or load()
    q = _bhd(q_nope)
    w = _f64(wkv_b)
    B, H, Dn = q.shape
    Dc = w.shape[1]
    Dv = w.shape[0] // H - Dn
    out = np.empty((B, H, Dc))
    if lib.oracle_absorb(B, H, Dn, Dc, Dv, _ptr(q), _ptr(w), _ptr(out)):
        raise ValueError("oracle_absorb: bad arguments")
    return out


def value_up(o_lat, wkv_b, Dn=128, lib=None):
    """Step 7 alone: out [B,H,Dv] from o_lat [B,H,Dc]."""
    lib = lib or load()
    o = _bhd(o_lat)
    w = _f64(wkv_b)
    B, H, Dc = o.shape
    Dv = w.shape[0] // H - Dn
    out = np.empty((B, H, Dv))
    if lib.oracle_value_up(B, H, Dn, Dc, Dv, _ptr(o), _ptr(w), _ptr(out)):
        raise ValueError("oracle_value_up: bad arguments")
    return out


def output_proj(x, wo, lib=None):
    """Output projection alone: out [B, Dout] from the head outputs x
    ([B, Din], or [B, 1, H, Dv] flattened per sequence) and wo [Dout, Din]."""
    lib = lib or load()
    a = _f64(x)
    a = np.ascontiguousarray(a.reshape(a.shape[0], -1))
    w = np.ascontiguousarray(_f64(wo))
    B, Din = a.shape
    Dout = w.shape[0]
    if w.shape[1] != Din:
        raise ValueError("wo must be [Dout, Din] with Din = the flattened head outputs")
    out = np.empty((B, Dout))
    if lib.oracle_output_proj(B, Din, Dout, _ptr(a), _ptr(w), _ptr(out)):
        raise ValueError("oracle_output_proj: bad arguments")
    return out


def dequant_fp8(w_fp8, scales, block=128):
    """Oracle dequantisation of block-scaled E4M3FN weights.

    ``w_fp8`` holds raw codes (uint8 [rows, cols]); ``scales`` fp32
    [ceil(rows/block), ceil(cols/block)].  Returns (bf16 bit patterns as
    uint16, exact products as float64).
    """
    lib = load()
    w = _np(w_fp8, np.uint8)
    s = _np(scales, np.float32)
    rows, cols = w.shape
    out16 = np.empty((rows, cols), dtype=np.uint16)
    exact = np.empty((rows, cols))
    st = lib.oracle_dequant_fp8(_ptr(w), _ptr(s), rows, cols, block, _ptr(out16), _ptr(exact))
    if st:
        raise ValueError("oracle_dequant_fp8: bad arguments")
    return out16, exact


def e4m3_to_double(code: int) -> float:
    return load().oracle_e4m3_to_double(int(code))


def double_to_bf16_bits(x: float) -> int:
    return int(load().oracle_double_to_bf16(float(x)))


def bf16_bits_to_double(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (type conversion: bits << 16 as fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
