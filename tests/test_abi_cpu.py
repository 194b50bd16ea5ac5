"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/mla_decode.h declares, and validates arguments before any HIP call.
No compute call is made here."""

import ctypes
import os
import re

import pytest

import mla_latent_cache_decode_amd as mla
from mla_latent_cache_decode_amd._lib import make_params, MlaDecodeParams

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla_decode.h")


def _lib():
    return mla.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(mla.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_params_struct_layout_matches_header():
    # 11 int32 + 1 float, no padding
    assert ctypes.sizeof(MlaDecodeParams) == 48


def test_row_sizes():
    assert mla.kv_row_bytes("bf16") == 1152
    assert mla.kv_row_stride("bf16") == 1152
    assert mla.kv_row_bytes("fp8") == 594
    assert mla.kv_row_stride("fp8") == 608
    # the 512-dimension FP8 row of the DeepSeek-R1 record, constraint (2)
    assert mla.kv_row_bytes("fp8", 448, 64) == 528
    assert mla.kv_row_stride("fp8", 448, 64) == 528
    # its fp4 variant: 288 bytes at 512 dimensions; 324 (stride 336) at 576
    assert mla.kv_row_bytes("fp4", 448, 64) == 288
    assert mla.kv_row_bytes("fp4") == 324
    assert mla.kv_row_stride("fp4") == 336
    lib = _lib()
    assert lib.mla_kv_row_bytes(7, 512, 64) == 0
    assert lib.mla_kv_row_bytes(1, 500, 64) == 0        # not a multiple of 32
    assert lib.mla_kv_row_bytes(0, 0, 64) == 0


def test_status_strings():
    lib = _lib()
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_ARGUMENT"), (2, "MLA_ERR_UNSUPPORTED"),
                       (3, "MLA_ERR_WORKSPACE_TOO_SMALL"), (4, "MLA_ERR_HIP"), (5, "MLA_ERR_OUT_OF_MEMORY")]:
        assert lib.mla_status_string(code).decode() == name
    assert lib.mla_status_string(99).decode() == "MLA_ERR_UNKNOWN"
    assert lib.mla_decode_abi_version() == 1


def _init(**over):
    kw = dict(max_batch=4, max_blocks_per_seq=16, softmax_scale=0.072)
    kw.update(over)
    p = make_params(**kw)
    for k in ("struct_size",):
        if k in over:
            setattr(p, k, over[k])
    h = ctypes.c_void_p(1234)
    st = _lib().mla_decode_init(ctypes.byref(p), ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("over,expected", [
    (dict(max_batch=0), 1),
    (dict(s_q=0), 1),
    (dict(s_q=9), 1),
    (dict(n_h=100), 1),
    (dict(n_h=0), 1),
    (dict(d_c=0), 1),
    (dict(block_size=0), 1),
    (dict(max_blocks_per_seq=0), 1),
    (dict(kv_dtype=5), 1),
    (dict(kv_dtype=3), 1),
    (dict(softmax_scale=0.0), 1),
    (dict(softmax_scale=float("nan")), 1),
    (dict(softmax_scale=-1.0), 1),
    (dict(num_workers=-1), 1),
    (dict(flags=4), 1),
    (dict(flags=2), 1),          # only MLA_FLAG_KV_WITHIN_4GIB is defined
    (dict(flags=-1), 1),
    (dict(d_c=448), 2),          # valid request, instantiated for the fp8 cache only
    (dict(d_c=448, kv_dtype="fp4"), 2),
    (dict(d_c=384, kv_dtype="fp8"), 2),
    (dict(d_c=448, d_r=0, kv_dtype="fp8"), 2),
    (dict(block_size=48), 2),    # page blocks: powers of two from 16 to 256
    (dict(block_size=8), 2),
    (dict(block_size=512), 2),
])
def test_init_rejects_before_any_hip_call(over, expected):
    st, h = _init(**over)
    assert st == expected
    assert h is None


def test_init_rejects_wrong_struct_size():
    p = make_params(max_batch=4, max_blocks_per_seq=16, softmax_scale=0.07)
    p.struct_size = 40
    h = ctypes.c_void_p()
    assert _lib().mla_decode_init(ctypes.byref(p), ctypes.byref(h)) == 1


def test_init_null_arguments():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.mla_decode_init(None, ctypes.byref(h)) == 1
    p = make_params(max_batch=4, max_blocks_per_seq=16, softmax_scale=0.07)
    assert lib.mla_decode_init(ctypes.byref(p), None) == 1


@pytest.mark.parametrize("block_size", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("flags", [0, 1], ids=["no_flags", "kv_within_4gib"])
def test_valid_params_without_a_gpu_report_hip_error(block_size, flags):
    import torch
    if torch.cuda.is_available():
        pytest.skip("this host has a GPU")
    st, h = _init(block_size=block_size, flags=flags)
    assert st == 4 and h is None


def test_fp8_narrow_row_passes_host_validation():
    # d_c = 448, d_r = 64: the record's 528-byte fp8 row
    import torch
    if torch.cuda.is_available():
        pytest.skip("this host has a GPU")
    st, h = _init(d_c=448, kv_dtype="fp8")
    assert st == 4 and h is None


def test_null_handle_paths():
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_decode_workspace_size(None, 1, ctypes.byref(n)) == 1
    assert lib.mla_decode_run(None, None, None, None, None, 1, None, None, None, 0, None) == 1
    assert lib.mla_decode_sparse_workspace_size(None, 1, 2048, ctypes.byref(n)) == 1
    assert lib.mla_decode_sparse_run(None, None, None, None, None, None, 2048, 1, None, None, None, 0, None) == 1
    assert lib.mla_decode_free(None) == 0
    assert lib.mla_decode_set_profile_events(None, None, None) == 1
    assert lib.mla_decode_get_info(None, None, None, None) == 1
