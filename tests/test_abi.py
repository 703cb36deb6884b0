"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-side validation rejects bad arguments with the
documented status codes before anything is launched.

Validation makes no HIP call, so these run on a machine without a GPU; no call
here reaches a kernel launch (every argument block is invalid in some way).
"""

import ctypes
import os
import re
import subprocess

import pytest

from io_aware_tiled_10_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fb._LIB_PATH), reason="libfa.so not built")

OK, NULL, SHAPE, DTYPE, STRIDE, UNSUP, WS, DEV, LAUNCH, ARG = range(10)
FAKE = 0x7F0000000000  # a 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_calls():
    assert declared_functions() == sorted(fb.EXPORTED)


def test_library_exports_every_declared_symbol():
    h = fb.lib()
    for name in declared_functions():
        assert hasattr(h, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fb._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(fa_\w+)", out))
    assert set(declared_functions()) <= exported


def test_ceiling_library_exports_its_header_and_rejects_bad_arguments():
    header = os.path.join(ROOT, "include", "fa_ceiling.h")
    path = os.path.join(ROOT, "io_aware_tiled_10_amd", "libfa_ceiling.so")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    declared = set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text))
    assert declared == {"fa_ceiling_mfma", "fa_ceiling_mfma_flops", "fa_ceiling_stream"}
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert declared <= set(re.findall(r"\sT\s(fa_\w+)", out))
    h = ctypes.CDLL(path)
    h.fa_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    h.fa_ceiling_mfma_flops.restype = ctypes.c_double
    h.fa_ceiling_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    # invalid arguments return 1 before any launch
    assert h.fa_ceiling_mfma(None, 1, 1, 0, None) == 1
    assert h.fa_ceiling_mfma(FAKE, 0, 1, 0, None) == 1
    assert h.fa_ceiling_mfma(FAKE, 1, 0, 0, None) == 1
    assert h.fa_ceiling_mfma(FAKE, 1, 1, 2, None) == 1
    # 8 waves x 16 products of 32 x 32 x 16 per trip
    assert h.fa_ceiling_mfma_flops(3, 5) == 3 * 8 * 5 * 16 * 2 * 32 * 32 * 16
    h.fa_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    ok_bytes = 32768 * 4
    assert h.fa_ceiling_stream(None, ok_bytes, FAKE, 4, None) == 1
    assert h.fa_ceiling_stream(FAKE, ok_bytes, None, 4, None) == 1
    assert h.fa_ceiling_stream(FAKE, ok_bytes, FAKE, 0, None) == 1
    assert h.fa_ceiling_stream(FAKE, 0, FAKE, 4, None) == 1
    assert h.fa_ceiling_stream(FAKE, ok_bytes + 16, FAKE, 4, None) == 1  # not whole trips
    assert h.fa_ceiling_stream(FAKE, ok_bytes, FAKE, 3, None) == 1      # slices of unequal trips
    assert h.fa_ceiling_stream(FAKE + 8, ok_bytes, FAKE, 4, None) == 1  # misaligned


def test_status_strings_and_version():
    h = fb.lib()
    for s in range(10):
        assert h.fa_status_str(s).decode().startswith("FA_")
    assert h.fa_status_str(1234).decode() == "FA_ERR_UNKNOWN"
    assert h.fa_version() >> 16 == 1


def good_fwd(**kw):
    a = fb.FwdArgs(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, kv_lens=None,
                   q_stride=fb.c_i64x3(2 * 8 * 128, 8 * 128, 128), k_stride=fb.c_i64x3(2 * 8 * 128, 8 * 128, 128),
                   v_stride=fb.c_i64x3(2 * 8 * 128, 8 * 128, 128), o_stride=fb.c_i64x3(2 * 8 * 128, 8 * 128, 128),
                   B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=128, in_dtype=fb.FA_BF16, out_dtype=fb.FA_BF16,
                   scale=0.088, causal=0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


FWD_BAD = [
    ({"B": 0}, SHAPE), ({"Hq": 3, "Hkv": 2}, SHAPE), ({"Hkv": 4}, SHAPE), ({"Nq": -1}, SHAPE),
    ({"Nk": -2}, SHAPE), ({"D": 96}, UNSUP), ({"D": 256}, UNSUP),
    ({"in_dtype": 7}, DTYPE), ({"out_dtype": 9}, DTYPE),
    ({"in_dtype": fb.FA_F32, "out_dtype": fb.FA_BF16}, DTYPE),
    ({"in_dtype": fb.FA_F32, "out_dtype": fb.FA_F32, "D": 128}, UNSUP),
    ({"scale": 0.0}, ARG), ({"scale": -1.0}, ARG), ({"scale": float("inf")}, ARG),
    ({"scale": float("nan")}, ARG), ({"causal": 2}, ARG),
    ({"q": None}, NULL), ({"k": None}, NULL), ({"v": None}, NULL), ({"o": None}, NULL),
    ({"q": FAKE + 2}, STRIDE), ({"o": FAKE + 8}, STRIDE),
    ({"q_stride": fb.c_i64x3(2 * 8 * 128, 8 * 128, 100)}, STRIDE),
    ({"k_stride": fb.c_i64x3(-1, 8 * 128, 128)}, STRIDE),
    ({"lse": FAKE + 2}, STRIDE),
]


@pytest.mark.parametrize("change,status", FWD_BAD)
def test_fwd_rejects_bad_arguments(change, status):
    a = good_fwd(**change)
    assert fb.lib().fa_fwd(ctypes.byref(a), None) == status


def test_fwd_null_args_and_empty_query():
    assert fb.lib().fa_fwd(None, None) == NULL
    # Nq == 0 is a valid request that launches nothing
    assert fb.lib().fa_fwd(ctypes.byref(good_fwd(Nq=0)), None) == OK


def good_bwd(**kw):
    st = fb.c_i64x3(2 * 8 * 128, 8 * 128, 128)
    a = fb.BwdArgs(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                   kv_lens=None, q_stride=st, k_stride=st, v_stride=st, o_stride=st, do_stride=st,
                   dq_stride=st, dk_stride=st, dv_stride=st, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, D=128,
                   dtype=fb.FA_BF16, scale=0.088, causal=1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BWD_BAD = [
    ({"dtype": fb.FA_F32}, DTYPE), ({"D": 32}, UNSUP), ({"Hq": 3}, SHAPE),
    ({"lse": None}, NULL), ({"dq": None}, NULL), ({"dk": None}, NULL), ({"dout": None}, NULL),
    ({"dv": FAKE + 4}, STRIDE), ({"do_stride": fb.c_i64x3(0, 0, 3)}, STRIDE),
    ({"scale": 0.0}, ARG), ({"causal": -1}, ARG),
]


@pytest.mark.parametrize("change,status", BWD_BAD)
def test_bwd_rejects_bad_arguments(change, status):
    a = good_bwd(**change)
    assert fb.lib().fa_bwd(ctypes.byref(a), FAKE, 1 << 30, None) == status
    assert fb.lib().fa_bwd_workspace_bytes(ctypes.byref(a)) == 0


def test_bwd_workspace_query_and_too_small_workspace():
    a = good_bwd(B=2, Hq=16, Hkv=16, Nq=4096, Nk=4096)
    need = fb.lib().fa_bwd_workspace_bytes(ctypes.byref(a))
    rows = 2 * 16 * 4096
    assert need == rows * 8  # LSE log2 e and -D_i per query row, two fp32 planes
    assert fb.lib().fa_bwd(ctypes.byref(a), FAKE, need - 1, None) == WS
    assert fb.lib().fa_bwd(ctypes.byref(a), None, need, None) == WS
    assert fb.lib().fa_bwd(ctypes.byref(a), FAKE + 4, need, None) == WS


def good_dec(**kw):
    a = fb.DecodeArgs(q=FAKE, k_cache=FAKE, v_cache=FAKE, seq_lens=FAKE, o=FAKE, lse=FAKE,
                      q_stride=fb.c_i64x2(32 * 128, 128), k_stride=fb.c_i64x3(8 * 4096 * 128, 4096 * 128, 128),
                      v_stride=fb.c_i64x3(8 * 4096 * 128, 4096 * 128, 128), o_stride=fb.c_i64x2(32 * 128, 128),
                      Bs=4, Hq=32, Hkv=8, D=128, cache_len=4096, max_len=4096, split_len=2048,
                      in_dtype=fb.FA_BF16, out_dtype=fb.FA_BF16, scale=0.088)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


DEC_BAD = [
    ({"max_len": 5000}, SHAPE), ({"split_len": 100}, SHAPE), ({"split_len": 0}, SHAPE),
    ({"Hq": 30}, SHAPE), ({"Bs": -1}, SHAPE), ({"Bs": 70000}, SHAPE), ({"D": 80}, UNSUP),
    ({"in_dtype": fb.FA_F32}, DTYPE), ({"out_dtype": 5}, DTYPE), ({"seq_lens": None}, NULL),
    ({"k_cache": None}, NULL), ({"q": FAKE + 2}, STRIDE), ({"scale": -0.5}, ARG),
]


@pytest.mark.parametrize("change,status", DEC_BAD)
def test_decode_rejects_bad_arguments(change, status):
    a = good_dec(**change)
    assert fb.lib().fa_decode(ctypes.byref(a), FAKE, 1 << 30, None) == status


def test_decode_workspace_query():
    a = good_dec(Bs=64, max_len=4096, cache_len=32768)
    need = fb.lib().fa_decode_workspace_bytes(ctypes.byref(a))
    rows = 64 * 32 * 2
    assert need == rows * 128 * 4 + rows * 4
    assert fb.lib().fa_decode(ctypes.byref(a), FAKE, need - 1, None) == WS
    assert fb.lib().fa_decode(ctypes.byref(good_dec(Bs=0)), None, 0, None) == OK


@pytest.mark.parametrize("change,status", DEC_BAD)
def test_decode_noalloc_rejects_bad_arguments(change, status):
    # the same validation as fa_decode, before the static array is looked up
    assert fb.lib().fa_decode_noalloc(ctypes.byref(good_dec(**change)), None) == status


def test_decode_noalloc_rejects_work_beyond_its_static_array():
    # 64 sequences x 32 heads x 16 chunks of partials fit the 32 MiB array; 33 chunks
    # (a longer cache) need more and are refused before anything is looked up or launched
    fits = good_dec(Bs=64, max_len=32768, cache_len=32768, split_len=2048)
    assert fb.lib().fa_decode_workspace_bytes(ctypes.byref(fits)) <= fb.DECODE_NOALLOC_MAX_WORKSPACE_BYTES
    big = good_dec(Bs=64, max_len=33 * 2048, cache_len=33 * 2048, split_len=2048)
    assert fb.lib().fa_decode_workspace_bytes(ctypes.byref(big)) > fb.DECODE_NOALLOC_MAX_WORKSPACE_BYTES
    assert fb.lib().fa_decode_noalloc(ctypes.byref(big), None) == WS
    assert fb.lib().fa_decode_noalloc(ctypes.byref(good_dec(Bs=0)), None) == OK


def good_varlen(**kw):
    a = fb.FwdVarlenArgs(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE,
                         q_stride=fb.c_i64x2(4 * 128, 128), k_stride=fb.c_i64x2(2 * 128, 128),
                         v_stride=fb.c_i64x2(2 * 128, 128), o_stride=fb.c_i64x2(4 * 128, 128),
                         B=3, Hq=4, Hkv=2, D=128, total_q=100, total_k=120, max_seqlen_q=60,
                         in_dtype=fb.FA_BF16, out_dtype=fb.FA_BF16, scale=0.088, causal=1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


VARLEN_BAD = [
    ({"B": 0}, SHAPE), ({"Hq": 3}, SHAPE), ({"total_q": -1}, SHAPE), ({"max_seqlen_q": 101}, SHAPE),
    ({"total_k": -5}, SHAPE), ({"D": 96}, UNSUP), ({"in_dtype": fb.FA_F32, "out_dtype": fb.FA_F32}, DTYPE),
    ({"out_dtype": 4}, DTYPE), ({"scale": 0.0}, ARG), ({"causal": 3}, ARG),
    ({"cu_seqlens_q": None}, NULL), ({"cu_seqlens_k": None}, NULL), ({"k": None}, NULL),
    ({"q": FAKE + 8}, STRIDE), ({"cu_seqlens_k": FAKE + 2}, STRIDE),
    ({"k_stride": fb.c_i64x2(2 * 128, 3)}, STRIDE), ({"lse": FAKE + 1}, STRIDE),
]


@pytest.mark.parametrize("change,status", VARLEN_BAD)
def test_fwd_varlen_rejects_bad_arguments(change, status):
    assert fb.lib().fa_fwd_varlen(ctypes.byref(good_varlen(**change)), None) == status


def test_fwd_varlen_empty_batches_launch_nothing():
    assert fb.lib().fa_fwd_varlen(None, None) == NULL
    assert fb.lib().fa_fwd_varlen(ctypes.byref(good_varlen(total_q=0, max_seqlen_q=0)), None) == OK
    assert fb.lib().fa_fwd_varlen(ctypes.byref(good_varlen(max_seqlen_q=0)), None) == OK


def good_paged(**kw):
    a = fb.DecodePagedArgs(q=FAKE, k_pages=FAKE, v_pages=FAKE, block_table=FAKE, seq_lens=FAKE,
                           o=FAKE, lse=FAKE, q_stride=fb.c_i64x2(32 * 128, 128),
                           k_stride=fb.c_i64x3(8 * 16 * 128, 16 * 128, 128),
                           v_stride=fb.c_i64x3(8 * 16 * 128, 16 * 128, 128),
                           o_stride=fb.c_i64x2(32 * 128, 128), table_stride=256,
                           Bs=4, Hq=32, Hkv=8, D=128, num_pages=1024, page_size=16,
                           max_pages_per_seq=256, max_len=4096, split_len=2048,
                           in_dtype=fb.FA_BF16, out_dtype=fb.FA_BF16, scale=0.088)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


PAGED_BAD = [
    ({"page_size": 8}, SHAPE), ({"page_size": 48}, SHAPE), ({"page_size": 0}, SHAPE),
    ({"max_len": 4097}, SHAPE), ({"table_stride": 255}, SHAPE), ({"num_pages": -1}, SHAPE),
    ({"split_len": 1000}, SHAPE), ({"split_len": 8192}, SHAPE), ({"Hq": 30}, SHAPE), ({"D": 80}, UNSUP),
    ({"in_dtype": fb.FA_F32}, DTYPE), ({"scale": float("nan")}, ARG),
    ({"block_table": None}, NULL), ({"seq_lens": None}, NULL), ({"v_pages": None}, NULL),
    ({"block_table": FAKE + 2}, STRIDE), ({"k_pages": FAKE + 4}, STRIDE),
    ({"page_size": 1 << 20, "max_pages_per_seq": 1, "table_stride": 1,
      "k_stride": fb.c_i64x3(1 << 30, 1 << 7, 8 * 128)}, SHAPE),
]


@pytest.mark.parametrize("change,status", PAGED_BAD)
def test_decode_paged_rejects_bad_arguments(change, status):
    a = good_paged(**change)
    assert fb.lib().fa_decode_paged(ctypes.byref(a), FAKE, 1 << 30, None) == status
    assert fb.lib().fa_decode_paged_workspace_bytes(ctypes.byref(a)) == 0


def test_decode_paged_workspace_query():
    a = good_paged(Bs=64)
    need = fb.lib().fa_decode_paged_workspace_bytes(ctypes.byref(a))
    rows = 64 * 32 * 2
    assert need == rows * 128 * 4 + rows * 4
    assert fb.lib().fa_decode_paged(ctypes.byref(a), FAKE, need - 1, None) == WS
    assert fb.lib().fa_decode_paged(ctypes.byref(good_paged(Bs=0)), None, 0, None) == OK


def good_quant(**kw):
    a = fb.QuantizeArgs(x=FAKE, codes=FAKE, scales=FAKE, x_stride=fb.c_i64x3(4 * 100 * 128, 100 * 128, 128),
                        codes_stride=fb.c_i64x3(4 * 100 * 128, 100 * 128, 128), B=1, H=4, N=100, D=128, block=64)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


QUANT_BAD = [({"B": 0}, SHAPE), ({"N": -1}, SHAPE), ({"block": 32}, UNSUP), ({"D": 64}, UNSUP),
             ({"x": None}, NULL), ({"scales": None}, NULL), ({"codes": FAKE + 8}, STRIDE),
             ({"codes_stride": fb.c_i64x3(0, 0, 120)}, STRIDE), ({"scales": FAKE + 2}, STRIDE)]


@pytest.mark.parametrize("change,status", QUANT_BAD)
def test_quantize_fp8_rejects_bad_arguments(change, status):
    assert fb.lib().fa_quantize_fp8(ctypes.byref(good_quant(**change)), None) == status


def good_fp8(**kw):
    st8 = fb.c_i64x3(2 * 8 * 128, 8 * 128, 128)
    st = fb.c_i64x3(2 * 8 * 128, 8 * 128, 128)
    a = fb.FwdFp8Args(q=FAKE, k=FAKE, v=FAKE, q_scales=FAKE, k_scales=FAKE, o=FAKE, lse=FAKE, kv_lens=None,
                      q_stride=st8, k_stride=st8, v_stride=st, o_stride=st, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=128,
                      block=64, out_dtype=fb.FA_BF16, scale=0.088, causal=0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


FP8_BAD = [({"D": 64}, UNSUP), ({"block": 128}, UNSUP), ({"Hq": 3, "Hkv": 2}, SHAPE), ({"out_dtype": 6}, DTYPE),
           ({"scale": 0.0}, ARG), ({"causal": 5}, ARG), ({"q_scales": None}, NULL), ({"k_scales": None}, NULL),
           ({"v": None}, NULL), ({"q": FAKE + 4}, STRIDE), ({"q_stride": fb.c_i64x3(0, 0, 100)}, STRIDE),
           ({"k_scales": FAKE + 1}, STRIDE)]


@pytest.mark.parametrize("change,status", FP8_BAD)
def test_fwd_fp8_rejects_bad_arguments(change, status):
    assert fb.lib().fa_fwd_fp8(ctypes.byref(good_fp8(**change)), None) == status
    assert fb.lib().fa_fwd_fp8(ctypes.byref(good_fp8(Nq=0)), None) == OK


@pytest.mark.parametrize("p", [-0.1, 1.0, 1.5, float("nan")])
def test_dropout_rejects_bad_probability(p):
    assert fb.lib().fa_fwd_dropout(ctypes.byref(good_fwd()), p, 1, None) == ARG
    assert fb.lib().fa_bwd_dropout(ctypes.byref(good_bwd()), p, 1, FAKE, 1 << 30, None) == ARG


def test_dropout_rejects_fp32_and_bad_args_first():
    a = good_fwd(in_dtype=fb.FA_F32, out_dtype=fb.FA_F32, D=64)
    assert fb.lib().fa_fwd_dropout(ctypes.byref(a), 0.1, 1, None) == UNSUP
    assert fb.lib().fa_fwd_dropout(ctypes.byref(good_fwd(D=96)), 0.1, 1, None) == UNSUP
    assert fb.lib().fa_bwd_dropout(ctypes.byref(good_bwd(dtype=fb.FA_F32)), 0.1, 1, FAKE, 1 << 30, None) == DTYPE
    assert fb.lib().fa_fwd_dropout(None, 0.1, 1, None) == NULL
    assert fb.lib().fa_bwd_dropout(None, 0.1, 1, None, 0, None) == NULL


def test_row_pitches_beyond_8_mib_are_rejected():
    big = (1 << 22) + 8  # elements: bf16 rows of just over 8 MiB
    assert fb.lib().fa_fwd(ctypes.byref(good_fwd(k_stride=fb.c_i64x3(0, 0, big))), None) == SHAPE
    st = fb.c_i64x3(0, 0, big)
    assert fb.lib().fa_bwd(ctypes.byref(good_bwd(dq_stride=st)), FAKE, 1 << 30, None) == SHAPE
    assert fb.lib().fa_decode(ctypes.byref(good_dec(v_stride=fb.c_i64x3(0, 0, big))), FAKE, 1 << 30, None) == SHAPE
    assert fb.lib().fa_fwd_varlen(ctypes.byref(good_varlen(q_stride=fb.c_i64x2(big, 128))), None) == SHAPE
    assert fb.lib().fa_quantize_fp8(ctypes.byref(good_quant(x_stride=fb.c_i64x3(0, 0, big))), None) == SHAPE


def test_noalloc_limit_matches_the_header():
    m = re.search(r"#define FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fb.DECODE_NOALLOC_MAX_WORKSPACE_BYTES
