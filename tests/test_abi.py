"""CPU tests of the C-ABI library: it loads, exports every symbol that
include/mla_decode.h declares, and rejects bad arguments on the host with the
documented status codes before anything is enqueued (no GPU is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")
LIB = os.path.join(ROOT, "sparse_mla_amd", "libmla_decode.so")

OK, NULLP, BADDIM, ALIGN, WS, UNSUP, HIP, RANGE, SCRATCH = range(9)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from sparse_mla_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    p, i32, i64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                 ctypes.c_float, ctypes.c_size_t)
    L.mla_sparse_decode.argtypes = [p, p, i64, i64, p, i64, i64, p, i64, i64, p, i32, p, i32, f32, i32,
                                    i32, p, sz, p, p, u32, p, i64, p, p, p]
    L.mla_sparse_decode_noalloc.argtypes = [p, p, i64, i64, p, i64, i64, p, i64, i64, p, i32, p, i32, f32, i32,
                                            i32, p, p, u32, p, i64, p, p, p]
    L.mla_noalloc_scratch_bytes.restype = sz
    L.mla_absorb_q.argtypes = [p, i64, i64, p, p, i32, p]
    L.mla_value_up.argtypes = [p, p, p, i64, i64, i32, p]
    L.mla_combine.argtypes = [p, sz, i32, i32, p, p, p, p]
    L.mla_combine_value_up.argtypes = [p, sz, i32, i32, p, p, i64, i64, p, p, p]
    L.mla_dequant_wkv_b_fp8.argtypes = [p, p, p, p]
    L.mla_output_proj.argtypes = [p, i64, p, p, i64, i32, p]
    L.mla_output_proj_packed.argtypes = [p, i64, p, p, i64, i32, p]
    L.mla_output_proj_pack.argtypes = [p, p, p]
    L.mla_workspace_bytes.restype = sz
    L.mla_workspace_bytes.argtypes = [i32, i32]
    L.mla_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32)]
    L.mla_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "mla_sparse_decode" in names and len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/mla_decode.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 2
    for code in range(9):
        assert lib.mla_status_string(code) != b"unknown status"
    assert lib.mla_last_hip_error() == 0


def test_workspace_bytes(lib):
    assert lib.mla_workspace_bytes(64, 1) == 0
    assert lib.mla_workspace_bytes(64, 2) == 2 * 64 * 128 * (512 * 2 + 2 * 4)
    assert lib.mla_workspace_bytes(0, 2) == 0 and lib.mla_workspace_bytes(4, 65) == 0


def test_plan(lib):
    s = ctypes.c_int32()
    for B, k, dense in [(1, 1001, 1), (32, 2048, 0), (64, 2048, 0), (128, 2048, 0), (64, 8192, 1), (7, 5000, 0)]:
        assert lib.mla_plan(B, k, dense, 256, ctypes.byref(s)) == OK
        assert 1 <= s.value <= 64
        chunk = -(-(-(-k // s.value)) // 32) * 32
        assert (s.value - 1) * chunk < k  # no empty split
        if not dense:
            assert chunk <= 2048
    # The shapes the benchmark runs: one workgroup per CU where the keys allow.
    for B, k, dense, want in [(64, 2048, 0, 4), (32, 2048, 0, 8), (1, 1001, 1, 32)]:
        assert lib.mla_plan(B, k, dense, 256, ctypes.byref(s)) == OK and s.value == want
    assert lib.mla_plan(0, 10, 0, 256, ctypes.byref(s)) == BADDIM


FAKE = 1 << 20  # a 16-byte aligned non-null address: never dereferenced (errors come first)


def _decode(lib, **kw):
    a = dict(q_abs=FAKE, q_pe=FAKE, q_pe_sb=128 * 64, q_pe_sh=64, kv=FAKE, kv_sb=576 * 100, kv_st=576,
             pe=FAKE + 1024, pe_sb=576 * 100, pe_st=576, seq_lens=FAKE, max_len=100, indices=FAKE, k_max=64,
             scale=0.07, B=2, S=1, ws=None, ws_bytes=0, o_lat=FAKE, lse=None, flags=0, bitmap=None,
             words=0, scores=None, status=None, stream=None)
    a.update(kw)
    return lib.mla_sparse_decode(a["q_abs"], a["q_pe"], a["q_pe_sb"], a["q_pe_sh"], a["kv"], a["kv_sb"],
                                 a["kv_st"], a["pe"], a["pe_sb"], a["pe_st"], a["seq_lens"], a["max_len"],
                                 a["indices"], a["k_max"], a["scale"], a["B"], a["S"], a["ws"],
                                 a["ws_bytes"], a["o_lat"], a["lse"], a["flags"], a["bitmap"], a["words"],
                                 a["scores"], a["status"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q_abs=None), NULLP),
    (dict(seq_lens=None), NULLP),
    (dict(B=0), BADDIM),
    (dict(k_max=0), BADDIM),
    (dict(max_len=0), BADDIM),
    (dict(S=0), BADDIM),
    (dict(S=65), BADDIM),
    (dict(indices=None, k_max=50), BADDIM),          # dense needs k_max >= max_len
    (dict(k_max=4097, S=2), BADDIM),                         # > 2048 slots in one split
    (dict(kv=FAKE + 8), ALIGN),
    (dict(kv_st=580), ALIGN),
    (dict(q_pe_sh=60), ALIGN),
    (dict(kv_st=504, pe_st=504), UNSUP),
    (dict(pe_st=56), UNSUP),
    (dict(max_len=2000000, kv_sb=576 * 2000000, pe_sb=576 * 2000000), RANGE),
    (dict(q_pe_sh=8 * 1100000), RANGE),               # q_pe span of one sequence > 2 GiB
    (dict(o_lat=None), NULLP),
    (dict(S=2, ws=None), NULLP),
    (dict(S=2, ws=FAKE, ws_bytes=100), WS),
    (dict(flags=1), NULLP),                           # VALIDATE without bitmap/status
    (dict(flags=1, bitmap=FAKE, status=FAKE, words=3), BADDIM),
    (dict(flags=2), NULLP),                           # WRITE_SCORES without scores
])
def test_decode_rejects_bad_arguments(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_other_entry_points_reject_bad_arguments(lib):
    assert lib.mla_absorb_q(None, 0, 0, FAKE, FAKE, 1, None) == NULLP
    assert lib.mla_absorb_q(FAKE, 16384, 128, FAKE, FAKE, 0, None) == BADDIM
    assert lib.mla_absorb_q(FAKE + 4, 16384, 128, FAKE, FAKE, 1, None) == ALIGN
    assert lib.mla_absorb_q(FAKE, 16384, 127, FAKE, FAKE, 1, None) == ALIGN
    assert lib.mla_absorb_q(FAKE, 1 << 28, 128, FAKE, FAKE, 9, None) == RANGE   # 32-bit row offsets
    assert lib.mla_value_up(FAKE, None, FAKE, 16384, 128, 1, None) == NULLP
    assert lib.mla_value_up(FAKE, FAKE, FAKE, 16384, 128, 70000, None) == BADDIM
    assert lib.mla_combine(None, 0, 4, 1, FAKE, None, None, None) == OK   # one split: no-op
    assert lib.mla_combine(None, 0, 4, 2, FAKE, None, None, None) == NULLP
    assert lib.mla_combine(FAKE, 10, 4, 2, FAKE, None, None, None) == WS
    assert lib.mla_combine_value_up(FAKE, 1 << 30, 4, 1, FAKE, FAKE, 16384, 128, None, None, None) == BADDIM
    assert lib.mla_combine_value_up(FAKE, 10, 4, 2, FAKE, FAKE, 16384, 128, None, None, None) == WS
    assert lib.mla_dequant_wkv_b_fp8(None, FAKE, FAKE, None) == NULLP
    assert lib.mla_dequant_wkv_b_fp8(FAKE + 2, FAKE, FAKE, None) == ALIGN


PEAKS_HEADER = os.path.join(ROOT, "include", "mla_peaks.h")
PEAKS_LIB = os.path.join(ROOT, "sparse_mla_amd", "libmla_peaks.so")


@pytest.fixture(scope="module")
def peaks():
    if not os.path.exists(PEAKS_LIB):
        from sparse_mla_amd import build
        build.build()
    L = ctypes.CDLL(PEAKS_LIB)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.mlap_stream_read.argtypes = [p, sz, i32, p, p]
    L.mlap_row_gather.argtypes = [p, sz, p, i32, i32, p, p]
    L.mlap_mfma_bf16.argtypes = [i32, i32, p, p]
    return L


def test_peaks_exports_every_declared_symbol(peaks):
    text = re.sub(r"/\*.*?\*/", "", open(PEAKS_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mlap_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mlap_mfma_bf16", "mlap_row_gather", "mlap_stream_read"]
    for n in names:
        assert hasattr(peaks, n), f"{n} declared in include/mla_peaks.h but not exported"


def test_peaks_reject_bad_arguments(peaks):
    # Return 1 (argument rejected) before any launch: fake, aligned addresses
    # are never dereferenced on these paths.
    a = 1 << 20
    assert peaks.mlap_stream_read(None, 1024, 4, a, None) == 1
    assert peaks.mlap_stream_read(a, 0, 4, a, None) == 1
    assert peaks.mlap_stream_read(a, 1000, 4, a, None) == 1      # not a multiple of 16
    assert peaks.mlap_stream_read(a + 8, 1024, 4, a, None) == 1  # misaligned
    assert peaks.mlap_stream_read(a, 1024, 0, a, None) == 1
    assert peaks.mlap_row_gather(a, 1 << 20, a, 4, 48, a, None) == 1      # not a multiple of 32
    assert peaks.mlap_row_gather(a, 1 << 20, a, 4, 2048, a, None) == 1    # above 1024
    assert peaks.mlap_row_gather(a, 1 << 33, a, 4, 512, a, None) == 1     # beyond 32-bit offsets
    assert peaks.mlap_row_gather(a, 1 << 20, None, 4, 512, a, None) == 1
    assert peaks.mlap_row_gather(a, 1 << 20, a, 0, 512, a, None) == 1
    assert peaks.mlap_mfma_bf16(0, 10, a, None) == 1
    assert peaks.mlap_mfma_bf16(4, 0, a, None) == 1
    assert peaks.mlap_mfma_bf16(4, 10, None, None) == 1


def test_output_proj_host_checks(lib):
    a = 1 << 20  # fake aligned addresses: never dereferenced on these paths
    assert lib.mla_output_proj(None, 16384, a, a, 7168, 4, None) == NULLP
    assert lib.mla_output_proj(a, 16384, None, a, 7168, 4, None) == NULLP
    assert lib.mla_output_proj(a, 16384, a, a, 7168, 0, None) == BADDIM
    assert lib.mla_output_proj(a, 16384, a, a, 7168, 65537, None) == BADDIM
    assert lib.mla_output_proj(a, 16376, a, a, 7168, 4, None) == BADDIM    # rows would overlap
    assert lib.mla_output_proj(a, 16384, a, a, 7000, 4, None) == BADDIM
    assert lib.mla_output_proj(a + 8, 16384, a, a, 7168, 4, None) == ALIGN
    assert lib.mla_output_proj(a, 16388, a, a, 7168, 4, None) == ALIGN     # stride not a multiple of 8
    assert lib.mla_output_proj(a, 16384, a + 8, a, 7168, 4, None) == ALIGN
    assert lib.mla_output_proj(a, 16384, a, a + 1, 7168, 4, None) == ALIGN


def test_output_proj_packed_host_checks(lib):
    a = 1 << 20
    assert lib.mla_output_proj_pack(None, a, None) == NULLP
    assert lib.mla_output_proj_pack(a, None, None) == NULLP
    assert lib.mla_output_proj_pack(a + 8, a, None) == ALIGN
    assert lib.mla_output_proj_pack(a, a + 2, None) == ALIGN
    f = lib.mla_output_proj_packed
    assert f(None, 16384, a, a, 7168, 4, None) == NULLP
    assert f(a, 16384, a, a, 7168, 0, None) == BADDIM
    assert f(a, 16384, a + 8, a, 7168, 4, None) == ALIGN
    assert f(a, 1 << 26, a, a, 7168, 4, None) == RANGE


def test_noalloc_host_checks(lib):
    """mla_sparse_decode_noalloc rejects plans whose partials exceed its
    static scratch, and bad arguments, on the host before it looks up the
    scratch or enqueues anything."""
    a = FAKE
    assert lib.mla_noalloc_scratch_bytes() == 40 << 20
    args = [a, a, 128 * 64, 64, a, 576 * 2048, 576, a + 1024, 576 * 2048, 576, a, 2048, a, 2048, 0.07, 128,
            64, a, None, 0, None, 0, None, None, None]
    assert lib.mla_workspace_bytes(128, 64) > lib.mla_noalloc_scratch_bytes()
    assert lib.mla_sparse_decode_noalloc(*args) == SCRATCH
    args[15], args[16] = 2, 2          # B = 2, two splits: fits the scratch
    args[0] = None
    assert lib.mla_sparse_decode_noalloc(*args) == NULLP
    args[0] = a
    args[17] = None                    # o_latent
    assert lib.mla_sparse_decode_noalloc(*args) == NULLP
    args[17] = a + 8
    assert lib.mla_sparse_decode_noalloc(*args) == ALIGN


def test_heads_host_checks(lib):
    """The head-sharded calls take 16, 32, 64 or 128 heads and reject others
    on the host (MLA_ERR_UNSUPPORTED); workspace sizes scale with the heads."""
    a = FAKE
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mla_workspace_bytes_heads.restype = sz
    lib.mla_workspace_bytes_heads.argtypes = [i32, i32, i32]
    lib.mla_absorb_q_heads.argtypes = [i32, p, i64, i64, p, p, i32, p]
    lib.mla_value_up_heads.argtypes = [i32, p, p, p, i64, i64, i32, p]
    lib.mla_combine_heads.argtypes = [i32, p, sz, i32, i32, p, p, p, p]
    for H in (16, 32, 64, 128):
        assert lib.mla_workspace_bytes_heads(H, 64, 4) == 4 * 64 * H * (512 * 2 + 2 * 4)
    assert lib.mla_workspace_bytes_heads(128, 64, 4) == lib.mla_workspace_bytes(64, 4)
    assert lib.mla_workspace_bytes_heads(48, 64, 4) == 0
    for H in (0, 8, 48, 96, 256):
        assert lib.mla_absorb_q_heads(H, a, 8192, 128, a, a, 4, None) == UNSUP
        assert lib.mla_value_up_heads(H, a, a, a, 8192, 128, 4, None) == UNSUP
        assert lib.mla_combine_heads(H, a, 1 << 30, 4, 2, a, None, None, None) == UNSUP
    assert lib.mla_absorb_q_heads(64, None, 8192, 128, a, a, 4, None) == NULLP
