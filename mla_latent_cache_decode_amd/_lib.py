"""ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the HIP library.
PyTorch tensors are accepted for device memory and the current stream; the
binding checks their dtype, device, shape and contiguity on the host and
passes raw pointers.  There is no fallback: if the library is missing the
import fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_DECODE_LIB_PATH may name another build of the same sources (the host
# AddressSanitizer build that the ABI test makes); by default the in-tree one
LIB_PATH = os.environ.get("MLA_DECODE_LIB_PATH") or os.path.join(_PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_ERR_OUT_OF_MEMORY = 5

# the caller guarantees the whole cache lies within 0xFFFFF000 bytes of its
# base (include/mla_decode.h): the sparse gathers then use 32-bit offsets
MLA_FLAG_KV_WITHIN_4GIB = 1
KV_WINDOW_BYTES = 0xFFFFF000
# the per-GPU scratch of mla_decode_run_noalloc (include/mla_decode.h)
NOALLOC_SCRATCH_BYTES = 128 << 20

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3_E8M0 = 1
MLA_KV_FP4_E2M1_E8M0 = 2
KV_DTYPES = {"bf16": MLA_KV_BF16, "fp8": MLA_KV_FP8_E4M3_E8M0, "fp4": MLA_KV_FP4_E2M1_E8M0}

# every symbol include/mla_decode.h declares
EXPORTED_SYMBOLS = (
    "mla_decode_init",
    "mla_decode_workspace_size",
    "mla_decode_run",
    "mla_decode_run_noalloc",
    "mla_decode_sparse_workspace_size",
    "mla_decode_sparse_run",
    "mla_decode_set_profile_events",
    "mla_decode_get_info",
    "mla_decode_free",
    "mla_kv_row_bytes",
    "mla_kv_row_stride",
    "mla_status_string",
    "mla_decode_abi_version",
)


class MlaDecodeParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("n_h", ctypes.c_int32),
        ("d_c", ctypes.c_int32),
        ("d_r", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("num_workers", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and type the shared library.  Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # Load torch first: its bundled HIP runtime (same SONAME) then satisfies
    # this library's dependency, so the process has exactly one HIP runtime
    # and torch's streams, events and allocations are valid here.
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m mla_latent_cache_decode_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mla_decode_init.argtypes = [ctypes.POINTER(MlaDecodeParams), ctypes.POINTER(vp)]
    lib.mla_decode_init.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [vp, i32, ctypes.POINTER(sz)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    lib.mla_decode_run.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.mla_decode_run.restype = ctypes.c_int
    lib.mla_decode_run_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.mla_decode_run_noalloc.restype = ctypes.c_int
    lib.mla_decode_sparse_workspace_size.argtypes = [vp, i32, i32, ctypes.POINTER(sz)]
    lib.mla_decode_sparse_workspace_size.restype = ctypes.c_int
    lib.mla_decode_sparse_run.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.mla_decode_sparse_run.restype = ctypes.c_int
    lib.mla_decode_set_profile_events.argtypes = [vp, vp, vp]
    lib.mla_decode_set_profile_events.restype = ctypes.c_int
    lib.mla_decode_get_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.mla_decode_get_info.restype = ctypes.c_int
    lib.mla_decode_free.argtypes = [vp]
    lib.mla_decode_free.restype = ctypes.c_int
    lib.mla_kv_row_bytes.argtypes = [i32, i32, i32]
    lib.mla_kv_row_bytes.restype = sz
    lib.mla_kv_row_stride.argtypes = [i32, i32, i32]
    lib.mla_kv_row_stride.restype = sz
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_decode_abi_version.argtypes = []
    lib.mla_decode_abi_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().mla_status_string(int(status)).decode()
    except ImportError:
        return f"status {status}"


def kv_row_bytes(kv_dtype: str, d_c: int = 512, d_r: int = 64) -> int:
    return int(load_library().mla_kv_row_bytes(KV_DTYPES[kv_dtype], d_c, d_r))


def kv_row_stride(kv_dtype: str, d_c: int = 512, d_r: int = 64) -> int:
    return int(load_library().mla_kv_row_stride(KV_DTYPES[kv_dtype], d_c, d_r))


def make_params(*, max_batch: int, s_q: int = 1, n_h: int = 128, d_c: int = 512, d_r: int = 64,
                block_size: int = 64, max_blocks_per_seq: int, kv_dtype: str = "bf16",
                softmax_scale: float, num_workers: int = 0, flags: int = 0) -> MlaDecodeParams:
    return MlaDecodeParams(ctypes.sizeof(MlaDecodeParams), max_batch, s_q, n_h, d_c, d_r, block_size,
                           max_blocks_per_seq, KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype,
                           softmax_scale, num_workers, flags)


class MlaDecode:
    """One configured decode (a host handle).  ``run`` enqueues on the current stream."""

    def __init__(self, **kw):
        self._lib = load_library()
        self.params = make_params(**kw)
        h = ctypes.c_void_p()
        st = self._lib.mla_decode_init(ctypes.byref(self.params), ctypes.byref(h))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_init")
        self._h = h
        self._ws = None

    # -- info -------------------------------------------------------------
    def info(self) -> dict:
        w, r, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = self._lib.mla_decode_get_info(self._h, ctypes.byref(w), ctypes.byref(r), ctypes.byref(c))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_get_info")
        return {"num_workers": w.value, "row_groups": r.value, "compute_units": c.value}

    def workspace_size(self, batch: int) -> int:
        n = ctypes.c_size_t()
        st = self._lib.mla_decode_workspace_size(self._h, int(batch), ctypes.byref(n))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_workspace_size")
        return n.value

    def alloc_workspace(self, batch: int, device="cuda"):
        import torch
        n = self.workspace_size(batch)
        # torch's caching allocator returns >= 512-byte aligned blocks
        return torch.empty(max(n, 1), dtype=torch.uint8, device=device)

    def set_profile_events(self, ev_start: Optional[int], ev_stop: Optional[int]) -> None:
        st = self._lib.mla_decode_set_profile_events(self._h, ev_start, ev_stop)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_set_profile_events")

    # -- the decode ---------------------------------------------------------
    def run(self, q, kv, block_table, seq_lens, out, lse=None, workspace=None, stream=None) -> None:
        import torch
        p = self.params
        batch = int(seq_lens.shape[0])
        d = p.d_c + p.d_r
        _check(q, (batch, p.s_q, p.n_h, d), torch.bfloat16, "q")
        _check(out, (batch, p.s_q, p.n_h, p.d_c), torch.float32, "out")
        if lse is not None:
            _check(lse, (batch, p.s_q, p.n_h), torch.float32, "lse")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch \
                or block_table.shape[1] != p.max_blocks_per_seq or not block_table.is_contiguous():
            raise ValueError("block_table must be contiguous int32 [batch, max_blocks_per_seq]")
        if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be contiguous int32 [batch]")
        if not kv.is_contiguous() or not kv.is_cuda:
            raise ValueError("kv pages must be a contiguous device tensor")
        for t in (q, out, block_table, seq_lens) + ((lse,) if lse is not None else ()):
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
        if workspace is None:
            if self._ws is None or self._ws.numel() < self.workspace_size(batch):
                self._ws = self.alloc_workspace(batch, device=q.device)
            workspace = self._ws
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        st = self._lib.mla_decode_run(
            self._h, q.data_ptr(), kv.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), batch,
            out.data_ptr(), lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), stream)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_run")

    def run_noalloc(self, q, kv, block_table, seq_lens, out, lse=None, stream=None) -> None:
        """``run`` through mla_decode_run_noalloc: no workspace, the library's
        per-GPU scratch instead (calls that overlap on one GPU race)."""
        import torch
        p = self.params
        batch = int(seq_lens.shape[0])
        _check(q, (batch, p.s_q, p.n_h, p.d_c + p.d_r), torch.bfloat16, "q")
        _check(out, (batch, p.s_q, p.n_h, p.d_c), torch.float32, "out")
        if lse is not None:
            _check(lse, (batch, p.s_q, p.n_h), torch.float32, "lse")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch \
                or block_table.shape[1] != p.max_blocks_per_seq or not block_table.is_contiguous():
            raise ValueError("block_table must be contiguous int32 [batch, max_blocks_per_seq]")
        if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be contiguous int32 [batch]")
        if not kv.is_contiguous() or not kv.is_cuda:
            raise ValueError("kv pages must be a contiguous device tensor")
        for t in (q, out, block_table, seq_lens) + ((lse,) if lse is not None else ()):
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        st = self._lib.mla_decode_run_noalloc(
            self._h, q.data_ptr(), kv.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), batch,
            out.data_ptr(), lse.data_ptr() if lse is not None else None, stream)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_run_noalloc")

    # -- the sparse (top-k) decode -------------------------------------------
    def sparse_workspace_size(self, batch: int, topk: int) -> int:
        n = ctypes.c_size_t()
        st = self._lib.mla_decode_sparse_workspace_size(self._h, int(batch), int(topk), ctypes.byref(n))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_sparse_workspace_size")
        return n.value

    def alloc_sparse_workspace(self, batch: int, topk: int, device="cuda"):
        import torch
        return torch.empty(max(self.sparse_workspace_size(batch, topk), 1), dtype=torch.uint8, device=device)

    def run_sparse(self, q, kv, block_table, seq_lens, indices, out, lse=None, workspace=None,
                   stream=None) -> None:
        """Each query attends to the tokens its row of ``indices`` (int32
        [batch, s_q, topk], -1 = padding) lists; see mla_decode_sparse_run."""
        import torch
        p = self.params
        batch = int(seq_lens.shape[0])
        _check(q, (batch, p.s_q, p.n_h, p.d_c + p.d_r), torch.bfloat16, "q")
        _check(out, (batch, p.s_q, p.n_h, p.d_c), torch.float32, "out")
        if lse is not None:
            _check(lse, (batch, p.s_q, p.n_h), torch.float32, "lse")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch \
                or block_table.shape[1] != p.max_blocks_per_seq or not block_table.is_contiguous():
            raise ValueError("block_table must be contiguous int32 [batch, max_blocks_per_seq]")
        if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be contiguous int32 [batch]")
        if indices.dtype != torch.int32 or indices.dim() != 3 or tuple(indices.shape[:2]) != (batch, p.s_q) \
                or not indices.is_contiguous():
            raise ValueError("indices must be contiguous int32 [batch, s_q, topk]")
        if not kv.is_contiguous() or not kv.is_cuda:
            raise ValueError("kv pages must be a contiguous device tensor")
        for t in (q, out, block_table, seq_lens, indices) + ((lse,) if lse is not None else ()):
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
        topk = int(indices.shape[2])
        if workspace is None:
            workspace = self.alloc_sparse_workspace(batch, topk, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        st = self._lib.mla_decode_sparse_run(
            self._h, q.data_ptr(), kv.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), indices.data_ptr(),
            topk, batch, out.data_ptr(), lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), stream)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_sparse_run")

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.mla_decode_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
