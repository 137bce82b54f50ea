"""Python binding of libdtm_gemm.so, the MI355X (gfx950) blocked GEMM C = A·B
and the row softmax.

The C ABI is declared in ``include/dtm_gemm.h`` and ``include/dtm_softmax.h``;
the functions here have the same names and only marshal arguments (sizes, device pointers, element
strides, dtype codes and the current HIP stream) into it.  Every step of the
computation runs in the library's HIP kernels.  PyTorch provides device memory
and streams.

There is no fallback: if the shared library is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdtm_gemm.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libdtm_gemm_debug.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADER = os.path.join(INCLUDE, "dtm_gemm.h")
HEADERS = [HEADER, os.path.join(INCLUDE, "dtm_softmax.h")]

# dtm_dtype
DTM_F32, DTM_F16, DTM_BF16 = 0, 1, 2
# dtm_status
STATUS = {
    0: "DTM_OK", 1: "DTM_ERR_INVALID_DIM", 2: "DTM_ERR_NULL_POINTER", 3: "DTM_ERR_DTYPE",
    4: "DTM_ERR_STRIDE", 5: "DTM_ERR_ALIAS", 6: "DTM_ERR_CONFIG", 7: "DTM_ERR_WORKSPACE",
    8: "DTM_ERR_DEVICE", 9: "DTM_ERR_LAUNCH", 10: "DTM_ERR_POINTER", 11: "DTM_ERR_SCRATCH",
}
globals().update({v: k for k, v in STATUS.items()})
# dtm_kernel
KERNELS = {0: "none", 1: "zero_fill", 2: "generic", 3: "mfma_f16", 4: "mfma_f32",
           5: "generic_fp16acc", 6: "mfma_f16_wavek"}
DTM_KERNEL_NONE, DTM_KERNEL_ZERO_FILL, DTM_KERNEL_GENERIC = 0, 1, 2
DTM_KERNEL_MFMA_F16, DTM_KERNEL_MFMA_F32 = 3, 4
DTM_KERNEL_GENERIC_FP16ACC = 5  # negative control: fp16 accumulator, forced only
DTM_KERNEL_MFMA_F16_WAVEK = 6   # 128 x 128 tiles, K loop split across the 4 waves
DTM_LAYOUT_A_M_CONTIG, DTM_LAYOUT_B_K_CONTIG = 1, 2


class TileConfig(ctypes.Structure):
    """dtm_tile_config: zero fields mean "the selector chooses"."""

    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("dp_rows", ctypes.c_int32), ("workspace_limit", ctypes.c_uint64)]


class Plan(ctypes.Structure):
    """dtm_plan."""

    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("grid_m", ctypes.c_int64), ("grid_n", ctypes.c_int64),
                ("k_iters", ctypes.c_int64), ("split_k", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("fast_path", ctypes.c_int32),
                ("ragged", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("dp_rows", ctypes.c_int64)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel_name"] = KERNELS.get(self.kernel, "unknown")
        return d


# dtm_softmax_form
SOFTMAX_FORMS = {0: "none", 1: "wave", 2: "block", 3: "online", 4: "split"}


class SoftmaxPlan(ctypes.Structure):
    """dtm_softmax_plan."""

    _fields_ = [("form", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("chunks", ctypes.c_int32),
                ("chunk_elems", ctypes.c_int32), ("vectorized", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("passes", ctypes.c_int32),
                ("parts", ctypes.c_int32)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["form_name"] = SOFTMAX_FORMS.get(self.form, "unknown")
        return d


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str = "gemm"):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {gemm_status_string(status)}")


_lib = None


def _load(path):
    """Load a build of the library at `path` and declare its C signatures."""
    L = ctypes.CDLL(path)
    i64, vp, i32, u64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    ops = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i32, i32]
    L.gemm.argtypes = ops + [vp]
    L.gemm.restype = i32
    L.gemm_plan.argtypes = ops + [ctypes.POINTER(TileConfig), ctypes.POINTER(Plan)]
    L.gemm_plan.restype = i32
    L.gemm_ex.argtypes = ops + [ctypes.POINTER(TileConfig), vp, u64, vp]
    L.gemm_ex.restype = i32
    L.gemm_status_string.argtypes = [i32]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_kernel_name.argtypes = [i32]
    L.gemm_kernel_name.restype = ctypes.c_char_p
    L.gemm_set_pointer_checks.argtypes = [i32]
    L.gemm_set_pointer_checks.restype = i32
    L.gemm_ex_noalloc.argtypes = ops + [ctypes.POINTER(TileConfig), vp]
    L.gemm_ex_noalloc.restype = i32
    L.gemm_noalloc_scratch_bytes.argtypes = []
    L.gemm_noalloc_scratch_bytes.restype = u64
    L.gemm_mfma_probe.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    L.gemm_mfma_probe.restype = i32
    L.gemm_workspace_reserve.argtypes = [u64, vp]
    L.gemm_workspace_reserve.restype = i32
    L.gemm_workspace_release.argtypes = [vp]
    L.gemm_workspace_release.restype = i32
    L.gemm_workspace_reserved.argtypes = [vp]
    L.gemm_workspace_reserved.restype = u64
    sops = [i64, i64, vp, i64, i64, vp, i64, i64, i32, i32]
    L.row_softmax.argtypes = sops + [vp]
    L.row_softmax.restype = i32
    L.row_softmax_plan.argtypes = sops + [ctypes.POINTER(SoftmaxPlan)]
    L.row_softmax_plan.restype = i32
    return L


def lib():
    """The loaded libdtm_gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = _load(LIB_PATH)
    return _lib


_debug_lib = None


def debug_lib():
    """The extra-barrier debug build, libdtm_gemm_debug.so (same C ABI; every
    K iteration of the LDS-staged kernels waits for all memory operations and
    the whole workgroup).  Raises if it has not been built
    (`python -m dense_tiled_matrix_amd.build --debug-barriers`)."""
    global _debug_lib
    if _debug_lib is None:
        if not os.path.exists(DEBUG_LIB_PATH):
            raise RuntimeError(f"{DEBUG_LIB_PATH} is missing: build it with "
                               "`python -m dense_tiled_matrix_amd.build --debug-barriers`")
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def header_functions():
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def set_pointer_checks(on: bool) -> bool:
    """Turn the library's debug pointer checks on or off (gemm_set_pointer_checks);
    returns the previous setting."""
    return bool(lib().gemm_set_pointer_checks(1 if on else 0))


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(int(status)).decode()


def gemm_kernel_name(kernel: int) -> str:
    return lib().gemm_kernel_name(int(kernel)).decode()


# ---------------------------------------------------------------- workspace

# The selector's split plans keep slices x rows x N x 4 bytes of fp32 partials:
# 16 MiB for 512 x 512 in 16 slices, up to ~128 MiB for the last tile-rows of a
# C near 8192 wide in 16 slices.  A smaller reservation only splits less.
DEFAULT_WORKSPACE_BYTES = 256 << 20


def _current_cuda(device):
    import torch

    return torch.device(device) if device is not None else \
        torch.device("cuda", torch.cuda.current_device())


def reserve_workspace(nbytes: int = DEFAULT_WORKSPACE_BYTES, stream=None, device=None) -> None:
    """Reserve (at least) ``nbytes`` of library workspace for ``stream``
    (default: torch's current stream) through ``gemm_workspace_reserve``.

    ``gemm``/``row_softmax`` never allocate: a plan that splits K keeps its
    fp32 partials in this workspace and splits only as far as they fit, so
    without a reservation such shapes run unsplit.  This call may allocate
    and wait for the stream; make it before timing or graph capture."""
    import torch

    dev = _current_cuda(device)
    with torch.cuda.device(dev):
        st = lib().gemm_workspace_reserve(int(nbytes), _stream(dev, stream))
    if st != DTM_OK:
        raise GemmError(st, "gemm_workspace_reserve")


def release_workspace(stream=None, device=None) -> None:
    """Free the workspace reserved for ``stream`` (``gemm_workspace_release``)."""
    import torch

    dev = _current_cuda(device)
    with torch.cuda.device(dev):
        st = lib().gemm_workspace_release(_stream(dev, stream))
    if st != DTM_OK:
        raise GemmError(st, "gemm_workspace_release")


def workspace_reserved(stream=None, device=None) -> int:
    """Bytes reserved for ``stream`` (``gemm_workspace_reserved``)."""
    import torch

    dev = _current_cuda(device)
    with torch.cuda.device(dev):
        return int(lib().gemm_workspace_reserved(_stream(dev, stream)))


def gemm_mfma_probe_raw(in_dtype, layout, paired, A, B, C, stream=None):
    """``gemm_mfma_probe`` on raw device pointers; returns the status."""
    s = ctypes.c_void_p(0 if stream is None else int(stream))
    return lib().gemm_mfma_probe(in_dtype, layout, paired, A, B, C, s)


# ---------------------------------------------------------------- tensors


def _dtype_code(dt) -> int:
    import torch

    codes = {torch.float32: DTM_F32, torch.float16: DTM_F16, torch.bfloat16: DTM_BF16}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}; expected float32, float16 or bfloat16")
    return codes[dt]


def _torch_dtype(code_or_dtype):
    import torch

    if code_or_dtype is None or isinstance(code_or_dtype, torch.dtype):
        return code_or_dtype
    return {DTM_F32: torch.float32, DTM_F16: torch.float16, DTM_BF16: torch.bfloat16}[code_or_dtype]


def _operands(a, b, out, out_dtype):
    import torch

    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    if a.dtype != b.dtype:
        raise TypeError(f"a and b must share a dtype ({a.dtype} vs {b.dtype})")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: a is {tuple(a.shape)}, b is {tuple(b.shape)}")
    if out is None:
        odt = _torch_dtype(out_dtype) or torch.float32
        out = torch.empty((M, N), dtype=odt, device=a.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    return M, N, K, out


def _device_of(*tensors):
    """The one CUDA device all ``tensors`` live on; ValueError otherwise (a
    host pointer handed to a kernel would fault the GPU, not fail)."""
    devs = {t.device for t in tensors}
    if len(devs) != 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"every tensor must be on a CUDA device, got {dev}")
    return dev


def _on_device(device, call):
    """Run ``call()`` with ``device`` as the current HIP device."""
    import torch

    if device.index is None or device.index == torch.cuda.current_device():
        return call()
    with torch.cuda.device(device):
        return call()


def _args(a, b, out, M, N, K):
    return (M, N, K, a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
            b.stride(1), out.data_ptr(), out.stride(0), out.stride(1), _dtype_code(a.dtype),
            _dtype_code(out.dtype))


def _stream(device, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _config(config):
    if config is None:
        return None
    if isinstance(config, TileConfig):
        return ctypes.byref(config)
    c = TileConfig(**config)
    return ctypes.byref(c)


def gemm(a, b, out=None, out_dtype=None, stream=None):
    """C = a @ b on the GPU through the C ``gemm``; returns ``out``.

    ``a`` (M x K) and ``b`` (K x N) are device tensors of one dtype (float32,
    float16 or bfloat16) with any strides; ``out`` (M x N) may be given, else
    it is allocated with ``out_dtype`` (default float32).  All must live on
    one CUDA device (ValueError otherwise).  The call is asynchronous on
    ``stream`` (default: torch's current stream); split-K plans use the
    workspace reserved for that stream (``reserve_workspace``).
    """
    M, N, K, out = _operands(a, b, out, out_dtype)
    dev = _device_of(a, b, out)
    st = _on_device(dev, lambda: lib().gemm(*_args(a, b, out, M, N, K), _stream(dev, stream)))
    if st != DTM_OK:
        raise GemmError(st, "gemm")
    return out


def gemm_ex(a, b, out=None, out_dtype=None, config=None, workspace=None, stream=None,
            library=None):
    """``gemm`` with a forced tile configuration (a dict of dtm_tile_config
    fields or a TileConfig) and an optional workspace tensor.  ``library``:
    another build of the library to call (e.g. ``debug_lib()``)."""
    M, N, K, out = _operands(a, b, out, out_dtype)
    dev = _device_of(a, b, out, *([workspace] if workspace is not None else []))
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    L = library if library is not None else lib()
    st = _on_device(dev, lambda: L.gemm_ex(*_args(a, b, out, M, N, K), _config(config),
                                           ws_ptr, ws_bytes, _stream(dev, stream)))
    if st != DTM_OK:
        raise GemmError(st, "gemm_ex")
    return out


def gemm_plan(a, b, out=None, out_dtype=None, config=None) -> dict:
    """The plan ``gemm``/``gemm_ex`` would launch (host only, no GPU needed).

    Tensors may live on any device: only shapes, strides, dtypes and pointer
    values are read.
    """
    M, N, K, out = _operands(a, b, out, out_dtype)
    p = Plan()
    st = lib().gemm_plan(*_args(a, b, out, M, N, K), _config(config), ctypes.byref(p))
    if st != DTM_OK:
        raise GemmError(st, "gemm_plan")
    return p.as_dict()


def gemm_plan_raw(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                  stride_cn, in_dtype, out_dtype, config=None):
    """``gemm_plan`` on raw integers; returns ``(status, plan_dict)``."""
    p = Plan()
    st = lib().gemm_plan(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                         stride_cn, in_dtype, out_dtype, _config(config), ctypes.byref(p))
    return st, p.as_dict()


def gemm_raw(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm, stride_cn,
             in_dtype, out_dtype, stream=None):
    """``gemm`` on raw integers (device pointers); returns the status."""
    s = ctypes.c_void_p(0 if stream is None else int(stream))
    return lib().gemm(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                      stride_cn, in_dtype, out_dtype, s)


def gemm_ex_raw(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                stride_cn, in_dtype, out_dtype, config=None, workspace=0, workspace_bytes=0,
                stream=None):
    """``gemm_ex`` on raw integers (device pointers); returns the status."""
    s = ctypes.c_void_p(0 if stream is None else int(stream))
    return lib().gemm_ex(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                         stride_cn, in_dtype, out_dtype, _config(config), workspace or None,
                         workspace_bytes, s)


def gemm_ex_noalloc(a, b, out=None, out_dtype=None, config=None, stream=None):
    """``gemm_ex`` without any workspace argument or reservation, through the
    C ``gemm_ex_noalloc``: split-K partials go to the library's fixed device
    array (``gemm_noalloc_scratch_bytes()`` bytes).  Calls that overlap on one
    GPU race on that array."""
    M, N, K, out = _operands(a, b, out, out_dtype)
    dev = _device_of(a, b, out)
    st = _on_device(dev, lambda: lib().gemm_ex_noalloc(*_args(a, b, out, M, N, K),
                                                       _config(config), _stream(dev, stream)))
    if st != DTM_OK:
        raise GemmError(st, "gemm_ex_noalloc")
    return out


def gemm_ex_noalloc_raw(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                        stride_cn, in_dtype, out_dtype, config=None, stream=None):
    """``gemm_ex_noalloc`` on raw integers (device pointers); returns the status."""
    s = ctypes.c_void_p(0 if stream is None else int(stream))
    return lib().gemm_ex_noalloc(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                 stride_cm, stride_cn, in_dtype, out_dtype, _config(config), s)


def gemm_noalloc_scratch_bytes() -> int:
    return int(lib().gemm_noalloc_scratch_bytes())


# ---------------------------------------------------------------- row softmax


def _softmax_operands(x, out, out_dtype):
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x columns)")
    if out is None:
        import torch

        odt = _torch_dtype(out_dtype) or x.dtype
        out = torch.empty(x.shape, dtype=odt, device=x.device)
    elif tuple(out.shape) != tuple(x.shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(x.shape)}")
    return out


def _softmax_args(x, out):
    M, N = x.shape
    return (M, N, x.data_ptr(), x.stride(0), x.stride(1), out.data_ptr(), out.stride(0),
            out.stride(1), _dtype_code(x.dtype), _dtype_code(out.dtype))


def row_softmax(x, out=None, out_dtype=None, stream=None):
    """Softmax over the columns of each row of the 2-D device tensor ``x``
    through the C ``row_softmax``; returns ``out`` (allocated with
    ``out_dtype``, default x's dtype, when not given; it may be ``x`` itself
    for an in-place call)."""
    out = _softmax_operands(x, out, out_dtype)
    dev = _device_of(x, out)
    st = _on_device(dev, lambda: lib().row_softmax(*_softmax_args(x, out), _stream(dev, stream)))
    if st != DTM_OK:
        raise GemmError(st, "row_softmax")
    return out


def row_softmax_plan(x, out=None, out_dtype=None) -> dict:
    """The plan ``row_softmax`` would launch (host only)."""
    out = _softmax_operands(x, out, out_dtype)
    p = SoftmaxPlan()
    st = lib().row_softmax_plan(*_softmax_args(x, out), ctypes.byref(p))
    if st != DTM_OK:
        raise GemmError(st, "row_softmax_plan")
    return p.as_dict()


def row_softmax_raw(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn, in_dtype,
                    out_dtype, stream=None):
    """``row_softmax`` on raw integers (device pointers); returns the status."""
    s = ctypes.c_void_p(0 if stream is None else int(stream))
    return lib().row_softmax(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn, in_dtype,
                             out_dtype, s)


def row_softmax_plan_raw(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn, in_dtype,
                         out_dtype):
    """``row_softmax_plan`` on raw integers; returns ``(status, plan_dict)``."""
    p = SoftmaxPlan()
    st = lib().row_softmax_plan(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn,
                                in_dtype, out_dtype, ctypes.byref(p))
    return st, p.as_dict()
