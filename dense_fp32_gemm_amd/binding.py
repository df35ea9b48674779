"""ctypes binding of libgemm_f32.so (include/gemm_f32.h), same names.

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  ``matmul`` is a convenience over ``gemm_f32`` that takes torch
tensors for device memory and the current torch stream; it validates layout
and raises on any non-zero status.  There is no fallback: if the library is
missing and cannot be built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgemm_f32.so")

GEMM_F32_OK = 0
GEMM_F32_ERR_DIM = 1
GEMM_F32_ERR_LD = 2
GEMM_F32_ERR_NULL = 3
GEMM_F32_ERR_LAUNCH = 4
GEMM_F32_ERR_CONFIG = 5
GEMM_F32_ERR_ALIGN = 6
GEMM_F32_ERR_SCRATCH = 7
GEMM_F32_SCRATCH_BYTES = 4 << 20

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str = "gemm_f32"):
        self.status = status
        super().__init__(f"{what}: status {status} ({gemm_f32_status_string(status)})")


def load() -> ctypes.CDLL:
    """The HIP library (built in-tree first if it is not there yet)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            from . import build
            build.build()
        lib = ctypes.CDLL(LIBRARY)
        i, p = ctypes.c_int, ctypes.c_void_p
        gemm_args = [i, i, i, p, i, p, i, p, i, p]
        lib.gemm_f32.argtypes = gemm_args
        lib.gemm_f32.restype = i
        lib.gemm_f32_with_config.argtypes = [i] + gemm_args
        lib.gemm_f32_with_config.restype = i
        lib.gemm_f32_num_configs.argtypes = []
        lib.gemm_f32_num_configs.restype = i
        lib.gemm_f32_config_name.argtypes = [i]
        lib.gemm_f32_config_name.restype = ctypes.c_char_p
        ip = ctypes.POINTER(ctypes.c_int)
        lib.gemm_f32_config_info.argtypes = [i, ip, ip, ip, ip, ip]
        lib.gemm_f32_config_info.restype = i
        lib.gemm_f32_describe.argtypes = [i, i, i, i, p, i, p, i, p, i, ctypes.c_char_p, i]
        lib.gemm_f32_describe.restype = i
        lib.gemm_f32_ws_size.argtypes = [i, i, i]
        lib.gemm_f32_ws_size.restype = ctypes.c_size_t
        lib.gemm_f32_ws.argtypes = [i, i, i, p, i, p, i, p, i, p, ctypes.c_size_t, p]
        lib.gemm_f32_ws.restype = i
        lib.gemm_f32_ws_noalloc.argtypes = gemm_args
        lib.gemm_f32_ws_noalloc.restype = i
        lib.gemm_f32_device_peak.argtypes = [i, ip, ip, ctypes.POINTER(ctypes.c_double)]
        lib.gemm_f32_device_peak.restype = i
        lib.gemm_f32_status_string.argtypes = [i]
        lib.gemm_f32_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


INT32_MIN, INT32_MAX = -(1 << 31), (1 << 31) - 1


def _ints(**vals):
    """Refuses values a C int cannot hold: ctypes would wrap them silently
    (2^32 + 1000 becomes 1000), turning an oversized size or leading
    dimension into a different, valid-looking one."""
    for name, v in vals.items():
        if not INT32_MIN <= int(v) <= INT32_MAX:
            raise ValueError(f"{name} = {v} does not fit the C ABI's 32-bit int")


# --- the C ABI, one function per exported symbol ---------------------------
def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """C := A . B on `stream`; A, B, C are device addresses (ints)."""
    _ints(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return load().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_with_config(config, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    _ints(config=config, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return load().gemm_f32_with_config(config, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_num_configs() -> int:
    return load().gemm_f32_num_configs()


def gemm_f32_config_name(config: int) -> str:
    return load().gemm_f32_config_name(config).decode()


def gemm_f32_config_info(config: int, occupancy: bool = False) -> dict:
    """{'bm', 'bn', 'bk', 'threads'} (+ 'blocks_per_cu' if occupancy, needs a GPU)."""
    vals = [ctypes.c_int(0) for _ in range(5)]
    ptrs = [ctypes.byref(v) for v in vals]
    if not occupancy:
        ptrs[4] = None
    rc = load().gemm_f32_config_info(config, *ptrs)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_config_info")
    out = dict(bm=vals[0].value, bn=vals[1].value, bk=vals[2].value, threads=vals[3].value)
    if occupancy:
        out["blocks_per_cu"] = vals[4].value
    return out


def gemm_f32_ws_size(M, N, K) -> int:
    """Workspace bytes the split-K plan for this shape needs (0: not split)."""
    _ints(M=M, N=N, K=K)
    return load().gemm_f32_ws_size(M, N, K)


def gemm_f32_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=0) -> int:
    """C := A . B, split over K through `workspace` when the shape calls for it."""
    _ints(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return load().gemm_f32_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream)


def gemm_f32_ws_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """C := A . B like gemm_f32_ws, split over K through the library's own
    static scratch (allocates nothing; overlapping calls on one GPU race)."""
    _ints(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return load().gemm_f32_ws_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_device_peak(device: int = 0) -> dict:
    """{'compute_units', 'clock_khz', 'tflops'}: the FP32 matrix-core peak derived
    from the device's properties (needs a GPU)."""
    cu, khz, tf = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_double(0.0)
    rc = load().gemm_f32_device_peak(device, ctypes.byref(cu), ctypes.byref(khz), ctypes.byref(tf))
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_device_peak")
    return dict(compute_units=cu.value, clock_khz=khz.value, tflops=tf.value)


def gemm_f32_describe(config, M, N, K, A, lda, B, ldb, C, ldc) -> tuple[int, str]:
    """(status, description) of what gemm_f32_with_config would enqueue."""
    _ints(config=config, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    buf = ctypes.create_string_buffer(256)
    rc = load().gemm_f32_describe(config, M, N, K, A, lda, B, ldb, C, ldc, buf, len(buf))
    return rc, buf.value.decode()


def gemm_f32_status_string(status: int) -> str:
    return load().gemm_f32_status_string(status).decode()


def config_names() -> list[str]:
    return [gemm_f32_config_name(c) for c in range(gemm_f32_num_configs())]


# --- torch convenience -------------------------------------------------------
def _row_major(t, rows: int, cols: int, name: str) -> int:
    """Leading dimension of a 2-D float32 CUDA tensor with unit column stride."""
    import torch
    if t.dtype != torch.float32 or t.dim() != 2 or not t.is_cuda:
        raise TypeError(f"{name} must be a 2-D float32 tensor on a GPU")
    if tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(rows, cols)}")
    s0, s1 = t.stride()
    if rows > 0 and cols > 1 and s1 != 1:
        raise ValueError(f"{name} must have unit column stride")
    if rows > 1 and s0 < cols:
        raise ValueError(f"{name} rows overlap")
    return max(s0 if rows > 1 else cols, cols, 1)


def matmul(A, B, out=None, config: int = -1, stream=None):
    """out = A @ B via gemm_f32 on the current (or given) torch stream."""
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda = _row_major(A, M, K, "A")
    ldb = _row_major(B, K, N, "B")
    _ints(M=M, N=N, K=K, lda=lda, ldb=ldb)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    ldc = _row_major(out, M, N, "out")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    rc = gemm_f32_with_config(config, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                              out.data_ptr(), ldc, stream.cuda_stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc)
    return out
