"""ctypes binding of libgemm_mkl.so: argument marshalling only.

Every step of the GEMM runs in the HIP library.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libgemm_mkl.so")

F32, F16, BF16 = 0, 1, 2
EPI_IDENTITY, EPI_RELU, EPI_SILU = 0, 1, 2
STATUS = {
    0: "OK",
    -1: "INVALID_VALUE",
    -2: "UNSUPPORTED_DTYPE",
    -3: "UNSUPPORTED_EPILOGUE",
    -4: "WORKSPACE",
    -5: "HIP_ERROR",
    -6: "NOT_AVAILABLE",
}
OPT_FORCE_GENERAL = 1
OPT_STREAMK = 2
OPT_NO_STREAMK = 4
OPT_PERSISTENT = 8
OPT_NO_PERSISTENT = 16
OPT_FIXUP = 32
OPT_NO_FIXUP = 64
OPT_FIXUP_RECOMPUTE = 128
NOALLOC_SCRATCH_BYTES = 32 << 20   # GEMM_MKL_NOALLOC_SCRATCH_BYTES

DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}
EPILOGUE_CODES = {"identity": EPI_IDENTITY, "relu": EPI_RELU, "silu": EPI_SILU}


class GemmMklError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"gemm_mkl status {status} ({STATUS.get(status, '?')}): {message}")
        self.status = status


class Opts(ctypes.Structure):
    _fields_ = [
        ("prefetch_stages", ctypes.c_int32),
        ("split_k", ctypes.c_int32),
        ("config_id", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("config_id", ctypes.c_int32),
        ("prefetch_stages", ctypes.c_int32),
        ("split_k", ctypes.c_int32),
        ("general", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("streamk", ctypes.c_int32),
        ("counter_bytes", ctypes.c_int32),
        ("persistent", ctypes.c_int32),
        ("packed", ctypes.c_int32),
        ("fixup", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


EXPORTS = (
    "gemm_mkl",
    "gemm_mkl_ex",
    "gemm_mkl_noalloc",
    "gemm_mkl_grouped",
    "gemm_mkl_grouped_config",
    "gemm_mkl_opts_init",
    "gemm_mkl_get_plan",
    "gemm_mkl_tile_order",
    "gemm_mkl_workspace_size",
    "gemm_mkl_release_workspace",
    "gemm_mkl_status_string",
    "gemm_mkl_num_configs",
    "gemm_mkl_config_name",
    "gemm_mkl_version",
    "gemm_mkl_rms_norm",
    "gemm_mkl_rms_norm_ex",
    "gemm_mkl_rms_norm_variant",
    "gemm_mkl_rms_norm_num_variants",
    "gemm_mkl_rms_norm_variant_name",
)

_lib = None


def load(path: str = LIB_PATH):
    """Load and type the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m tiled_dense_gemm_mkl_amd.build); there is no fallback path")
    # torch's wheel carries its own HIP runtime.  Loaded first, it is the copy
    # this library binds to (same soname); loaded after this library, it
    # comes in beside the system runtime that this library would then have
    # bound, and two runtimes in one process share no devices, streams or
    # memory (calls then fail with "no ROCm-capable device").
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gemm_mkl.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.gemm_mkl.restype = i32
    lib.gemm_mkl_ex.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, vp, ctypes.POINTER(Opts)]
    lib.gemm_mkl_ex.restype = i32
    lib.gemm_mkl_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, vp, ctypes.POINTER(Opts)]
    lib.gemm_mkl_noalloc.restype = i32
    lib.gemm_mkl_grouped.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp, ctypes.POINTER(Opts)]
    lib.gemm_mkl_grouped.restype = i32
    lib.gemm_mkl_grouped_config.argtypes = [i64, i64, i64, i64, i32, i32, ctypes.POINTER(Opts)]
    lib.gemm_mkl_grouped_config.restype = i32
    lib.gemm_mkl_opts_init.argtypes = [ctypes.POINTER(Opts)]
    lib.gemm_mkl_opts_init.restype = None
    lib.gemm_mkl_get_plan.argtypes = [i64, i64, i64, i64, i32, i32, ctypes.POINTER(Opts), ctypes.POINTER(Plan)]
    lib.gemm_mkl_get_plan.restype = i32
    lib.gemm_mkl_tile_order.argtypes = [i64, i64, i64, i64, i32, i32, ctypes.POINTER(Opts), ctypes.c_void_p, i64]
    lib.gemm_mkl_tile_order.restype = i32
    lib.gemm_mkl_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.gemm_mkl_workspace_size.restype = ctypes.c_size_t
    lib.gemm_mkl_release_workspace.argtypes = []
    lib.gemm_mkl_release_workspace.restype = i32
    lib.gemm_mkl_status_string.argtypes = [i32]
    lib.gemm_mkl_status_string.restype = ctypes.c_char_p
    lib.gemm_mkl_num_configs.argtypes = []
    lib.gemm_mkl_num_configs.restype = i32
    lib.gemm_mkl_config_name.argtypes = [i32]
    lib.gemm_mkl_config_name.restype = ctypes.c_char_p
    lib.gemm_mkl_version.argtypes = []
    lib.gemm_mkl_version.restype = i32
    lib.gemm_mkl_rms_norm.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, i32, vp]
    lib.gemm_mkl_rms_norm.restype = i32
    lib.gemm_mkl_rms_norm_ex.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, i32, vp, i32]
    lib.gemm_mkl_rms_norm_ex.restype = i32
    lib.gemm_mkl_rms_norm_variant.argtypes = [i64, i64, i32, i32]
    lib.gemm_mkl_rms_norm_variant.restype = i32
    lib.gemm_mkl_rms_norm_num_variants.argtypes = []
    lib.gemm_mkl_rms_norm_num_variants.restype = i32
    lib.gemm_mkl_rms_norm_variant_name.argtypes = [i32]
    lib.gemm_mkl_rms_norm_variant_name.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gemm_mkl_status_string(int(status)).decode()


def make_opts(prefetch_stages=None, split_k=None, config_id=None, force_general=False,
              workspace_ptr=None, workspace_bytes=0, streamk=None, persistent=None, fixup=None,
              fixup_recompute=False) -> Opts:
    o = Opts()
    load().gemm_mkl_opts_init(ctypes.byref(o))
    if prefetch_stages is not None:
        o.prefetch_stages = int(prefetch_stages)
    if split_k is not None:
        o.split_k = int(split_k)
    if config_id is not None:
        o.config_id = int(config_id)
    if force_general:
        o.flags |= OPT_FORCE_GENERAL
    if streamk is True:
        o.flags |= OPT_STREAMK
    elif streamk is False:
        o.flags |= OPT_NO_STREAMK
    if persistent is True:
        o.flags |= OPT_PERSISTENT
    elif persistent is False:
        o.flags |= OPT_NO_PERSISTENT
    if fixup is True:
        o.flags |= OPT_FIXUP
    elif fixup is False:
        o.flags |= OPT_NO_FIXUP
    if fixup_recompute:
        o.flags |= OPT_FIXUP_RECOMPUTE
    if workspace_ptr is not None:
        o.workspace = int(workspace_ptr)
        o.workspace_bytes = int(workspace_bytes)
    return o


# ------------------------------------------------------------------ raw C-ABI calls

def gemm_mkl(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream=None) -> int:
    """The C entry point, unchanged: device pointers as ints, returns the status."""
    return load().gemm_mkl(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream)


def gemm_mkl_ex(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream=None, opts: Opts | None = None) -> int:
    return load().gemm_mkl_ex(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream,
                              ctypes.byref(opts) if opts is not None else None)


def gemm_mkl_noalloc(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream=None,
                     opts: Opts | None = None) -> int:
    """The allocation-free entry point (its workspace is the library's fixed
    device scratch of NOALLOC_SCRATCH_BYTES); returns the status."""
    return load().gemm_mkl_noalloc(A_ptr, B_ptr, C_ptr, M, N, K, L, dtype, epilogue, stream,
                                   ctypes.byref(opts) if opts is not None else None)


def gemm_mkl_grouped(A_ptr, B_ptr, C_ptr, offs_ptr, G, total_m, N, K, dtype, epilogue, stream=None,
                     opts: Opts | None = None) -> int:
    return load().gemm_mkl_grouped(A_ptr, B_ptr, C_ptr, offs_ptr, G, total_m, N, K, dtype, epilogue, stream,
                                   ctypes.byref(opts) if opts is not None else None)


def grouped_config(G, total_m, N, K, dtype, epilogue, opts: Opts | None = None) -> int:
    """Configuration id gemm_mkl_grouped would use (raises on a negative status)."""
    st = load().gemm_mkl_grouped_config(G, total_m, N, K, dtype, epilogue,
                                        ctypes.byref(opts) if opts is not None else None)
    if st < 0:
        raise GemmMklError(st, status_string(st))
    return st


def gemm_mkl_rms_norm(x_ptr, w_ptr, y_ptr, rows, hidden, eps, dtype, stream=None, variant=-1) -> int:
    """The RMSNorm entry point (gemm_mkl_rms_norm_ex): device pointers as ints
    (w_ptr None for no weight), returns the status."""
    return load().gemm_mkl_rms_norm_ex(x_ptr, w_ptr, y_ptr, rows, hidden, eps, dtype, stream, variant)


def rms_norm_variant(rows, hidden, dtype, aligned=True) -> int:
    """Variant gemm_mkl_rms_norm picks for these sizes (raises on a negative status)."""
    st = load().gemm_mkl_rms_norm_variant(rows, hidden, dtype, 1 if aligned else 0)
    if st < 0:
        raise GemmMklError(st, status_string(st))
    return st


def rms_norm_variant_names() -> list[str]:
    lib = load()
    return [lib.gemm_mkl_rms_norm_variant_name(i).decode() for i in range(lib.gemm_mkl_rms_norm_num_variants())]


def get_plan(M, N, K, L, dtype, epilogue, opts: Opts | None = None) -> dict:
    p = Plan()
    st = load().gemm_mkl_get_plan(M, N, K, L, dtype, epilogue,
                                  ctypes.byref(opts) if opts is not None else None, ctypes.byref(p))
    if st != 0:
        raise GemmMklError(st, status_string(st))
    return p.as_dict()


def tile_order(M, N, K, L, dtype, epilogue, opts: Opts | None = None):
    """int32 array [grid, 4]: (batch, K split, tile row, tile column) of each
    workgroup of the plan's data-parallel grid, in workgroup order."""
    import numpy as np

    grid = get_plan(M, N, K, L, dtype, epilogue, opts)["grid"]
    out = np.zeros((max(grid, 0), 4), dtype=np.int32)
    st = load().gemm_mkl_tile_order(M, N, K, L, dtype, epilogue,
                                    ctypes.byref(opts) if opts is not None else None,
                                    out.ctypes.data, out.size)
    if st != 0:
        raise GemmMklError(st, status_string(st))
    return out


def workspace_size(M, N, K, L, dtype, split_k=0) -> int:
    return int(load().gemm_mkl_workspace_size(M, N, K, L, dtype, split_k))


def release_workspace() -> None:
    st = load().gemm_mkl_release_workspace()
    if st != 0:
        raise GemmMklError(st, status_string(st))


def config_names() -> list[str]:
    lib = load()
    return [lib.gemm_mkl_config_name(i).decode() for i in range(lib.gemm_mkl_num_configs())]


# ------------------------------------------------------------------ torch front end

def _torch_dtype_code(t) -> int:
    import torch

    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}: expected float32, float16 or bfloat16")
    return codes[t.dtype]


def _workspace_args(workspace, device):
    """(pointer, bytes) of a caller workspace tensor, or (None, 0) for none.

    The kernels write the workspace at its raw address, so a tensor in host
    memory or on another GPU would be an invalid device access: it is
    rejected here, as is one whose bytes are not contiguous.
    """
    import torch

    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}, got one on {workspace.device}")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def gemm(a, b, epilogue: str = "identity", out=None, *, prefetch_stages=None, split_k=None,
         config_id=None, force_general=False, workspace=None, stream=None, streamk=None, persistent=None,
         fixup=None, fixup_recompute=False):
    """C = epilogue(a @ b^T) per batch, on the GPU through libgemm_mkl.

    a: [L, M, K] or [M, K]; b: [L, N, K] or [N, K] (same dtype, on one GPU,
    contiguous).  Returns [L, M, N] (or [M, N]) in the operand dtype.
    """
    import torch

    if epilogue not in EPILOGUE_CODES:
        raise ValueError(f"unknown epilogue {epilogue!r}: expected one of {sorted(EPILOGUE_CODES)}")
    if not (isinstance(a, torch.Tensor) and isinstance(b, torch.Tensor)):
        raise TypeError("a and b must be torch tensors")
    if a.device.type != "cuda" or b.device != a.device:
        raise ValueError("a and b must be on the same GPU")
    if a.dtype != b.dtype:
        raise TypeError(f"dtype mismatch: a is {a.dtype}, b is {b.dtype}")
    squeeze = a.dim() == 2
    if squeeze:
        if b.dim() != 2:
            raise ValueError("a and b must both be 2-D or both 3-D")
        a3, b3 = a.unsqueeze(0), b.unsqueeze(0)
    else:
        if a.dim() != 3 or b.dim() != 3:
            raise ValueError("a must be [L, M, K] and b [L, N, K]")
        a3, b3 = a, b
    L, M, K = a3.shape
    Lb, N, Kb = b3.shape
    if Lb != L or Kb != K:
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}")
    if not (a3.is_contiguous() and b3.is_contiguous()):
        raise ValueError("a and b must be contiguous (K innermost)")
    if out is None:
        out3 = torch.empty((L, M, N), dtype=a.dtype, device=a.device)
    else:
        out3 = out.unsqueeze(0) if squeeze else out
        if tuple(out3.shape) != (L, M, N) or out3.dtype != a.dtype or not out3.is_contiguous() \
                or out3.device != a.device:
            raise ValueError("out must be a contiguous [L, M, N] tensor of the operand dtype on the same GPU")
    ws_ptr, ws_bytes = _workspace_args(workspace, a.device)
    opts = make_opts(prefetch_stages, split_k, config_id, force_general, ws_ptr, ws_bytes or 0, streamk, persistent,
                     fixup, fixup_recompute)
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        st = gemm_mkl_ex(a3.data_ptr(), b3.data_ptr(), out3.data_ptr(), M, N, K, L,
                         _torch_dtype_code(a), EPILOGUE_CODES[epilogue], s.cuda_stream, opts)
    if st != 0:
        raise GemmMklError(st, status_string(st))
    return out3[0] if squeeze else out3


def gemm_grouped(a, b, offs, epilogue: str = "identity", out=None, *, prefetch_stages=None, config_id=None,
                 stream=None):
    """Grouped GEMM on the GPU through libgemm_mkl.

    a: [total_m, K]; b: [G, N, K]; offs: int32 [G] cumulative row ends of the
    groups (on the same GPU).  Returns c [total_m, N] with the rows of group g
    equal to epilogue(a[rows of g] @ b[g]^T); rows outside every group are left
    as they are in `out` (uninitialised when out is None).
    """
    import torch

    if epilogue not in EPILOGUE_CODES:
        raise ValueError(f"unknown epilogue {epilogue!r}: expected one of {sorted(EPILOGUE_CODES)}")
    if not all(isinstance(x, torch.Tensor) for x in (a, b, offs)):
        raise TypeError("a, b and offs must be torch tensors")
    if a.device.type != "cuda" or b.device != a.device or offs.device != a.device:
        raise ValueError("a, b and offs must be on the same GPU")
    if a.dtype != b.dtype:
        raise TypeError(f"dtype mismatch: a is {a.dtype}, b is {b.dtype}")
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous():
        raise TypeError("offs must be a contiguous 1-D int32 tensor")
    if a.dim() != 2 or b.dim() != 3:
        raise ValueError("a must be [total_m, K] and b [G, N, K]")
    total_m, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or offs.shape[0] != G:
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, offs {tuple(offs.shape)}")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (K innermost)")
    if out is None:
        out = torch.empty((total_m, N), dtype=a.dtype, device=a.device)
    elif tuple(out.shape) != (total_m, N) or out.dtype != a.dtype or not out.is_contiguous() \
            or out.device != a.device:
        raise ValueError("out must be a contiguous [total_m, N] tensor of the operand dtype on the same GPU")
    opts = make_opts(prefetch_stages, None, config_id)
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        st = gemm_mkl_grouped(a.data_ptr(), b.data_ptr(), out.data_ptr(), offs.data_ptr(), G, total_m, N, K,
                              _torch_dtype_code(a), EPILOGUE_CODES[epilogue], s.cuda_stream, opts)
    if st != 0:
        raise GemmMklError(st, status_string(st))
    return out


def rms_norm(x, weight=None, eps: float = 1e-6, out=None, *, variant: int = -1, stream=None):
    """RMSNorm over the last axis on the GPU through libgemm_mkl:
    y = x * rsqrt(mean(x^2) + eps) * weight, computed in fp32, rounded once to
    x's dtype.

    x: [..., hidden] contiguous; weight: [hidden] of x's dtype or None (no
    weight); out: like x, may be x itself (in place).
    """
    import torch

    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a torch tensor on a GPU")
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous tensor with at least one dimension")
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if weight is not None:
        if not isinstance(weight, torch.Tensor) or weight.device != x.device or weight.dtype != x.dtype \
                or tuple(weight.shape) != (hidden,) or not weight.is_contiguous():
            raise ValueError("weight must be a contiguous [hidden] tensor of x's dtype on x's GPU")
    if out is None:
        out = torch.empty_like(x)
    elif tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous tensor shaped and typed like x on x's GPU")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        st = gemm_mkl_rms_norm(x.data_ptr(), weight.data_ptr() if weight is not None else None, out.data_ptr(),
                               rows, hidden, float(eps), _torch_dtype_code(x), s.cuda_stream, variant)
    if st != 0:
        raise GemmMklError(st, status_string(st))
    return out
