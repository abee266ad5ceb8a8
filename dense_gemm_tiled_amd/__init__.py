"""dense_gemm_tiled_amd -- MI355X (gfx950) dense GEMM, Python binding.

A thin ctypes layer over libtcgemm.so (C ABI in include/tcgemm.h).  PyTorch is
used only for device memory and streams: every GEMM runs in the library's HIP
kernels, enqueued on torch's current stream.  There is no fallback path: if
the library is not built, every call raises.

    import dense_gemm_tiled_amd as tg
    tg.gemm(a, b, c, alpha=1.0, beta=0.0, transpose_a=False, transpose_b=False)

computes c = alpha * op(a) @ op(b) + beta * c in place (tensorcore "GEMM",
section "Surface"), where a is stored [M,K] or, transposed, [K,M]; b is
stored [K,N] or, transposed, [N,K]; c is [M,N].  3-D tensors make a batched
call (one launch for all problems).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

__all__ = [
    "gemm", "plan", "TcGemmError", "last_kernel", "dispatch_count", "time_next_gemm", "library_path",
    "load_library", "F32", "F16", "BF16", "I8", "I32", "status_name", "DescT",
    "BatchedDescT", "PlanInfoT",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtcgemm.so")

# tc_dtype_t
F32, F16, BF16, I8, I32 = 0, 1, 2, 3, 4
_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", I8: "i8", I32: "i32"}

# tc_status_t
_STATUS = {0: "TC_OK", 1: "TC_ERR_INVALID_ARGUMENT", 2: "TC_ERR_UNSUPPORTED",
           3: "TC_ERR_OVERFLOW", 4: "TC_ERR_ALIASING", 5: "TC_ERR_OUT_OF_MEMORY",
           6: "TC_ERR_DEVICE"}


def status_name(code: int) -> str:
    return _STATUS.get(int(code), "TC_ERR_UNKNOWN(%d)" % code)


class TcGemmError(RuntimeError):
    """A libtcgemm call returned an error status."""

    def __init__(self, status: int, message: str):
        self.status = int(status)
        self.message = message
        super().__init__("%s: %s" % (status_name(status), message))


class DescT(ctypes.Structure):
    """tc_gemm_desc"""
    _fields_ = [("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("a_dtype", ctypes.c_int), ("b_dtype", ctypes.c_int),
                ("c_dtype", ctypes.c_int), ("accum_dtype", ctypes.c_int),
                ("transpose_a", ctypes.c_bool), ("transpose_b", ctypes.c_bool),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("lda", ctypes.c_int32), ("ldb", ctypes.c_int32), ("ldc", ctypes.c_int32)]


class BatchedDescT(ctypes.Structure):
    """tc_gemm_batched_desc"""
    _fields_ = [("base", DescT), ("batch", ctypes.c_int32),
                ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_c", ctypes.c_int64)]


class EpilogueT(ctypes.Structure):
    """tc_epilogue"""
    _fields_ = [("bias", ctypes.c_void_p), ("bias_stride", ctypes.c_int64),
                ("activation", ctypes.c_int), ("col_scale", ctypes.c_void_p),
                ("scale_stride", ctypes.c_int64)]


# tc_activation_t
ACTIVATIONS = {"none": 0, "relu": 1, "gelu_tanh": 2}


class PlanInfoT(ctypes.Structure):
    """tc_plan_info"""
    _fields_ = [("kernel", ctypes.c_char * 128),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("k_per_split", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("launches", ctypes.c_int32), ("band", ctypes.c_int32)]


# Every symbol include/tcgemm.h declares, with its ctypes signature.
_VP = ctypes.c_void_p
_SIGNATURES = {
    "tc_context_create": (ctypes.c_int, [ctypes.POINTER(_VP)]),
    "tc_context_destroy": (None, [_VP]),
    "tc_stream_create": (ctypes.c_int, [_VP, ctypes.POINTER(_VP)]),
    "tc_stream_wrap": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(_VP)]),
    "tc_stream_sync": (ctypes.c_int, [_VP]),
    "tc_stream_destroy": (None, [_VP]),
    "tc_gemm": (ctypes.c_int, [_VP, ctypes.POINTER(DescT), _VP, _VP, _VP]),
    "tc_gemm_async": (ctypes.c_int, [_VP, ctypes.POINTER(DescT), _VP, _VP, _VP, _VP]),
    "tc_gemm_batched": (ctypes.c_int, [_VP, ctypes.POINTER(BatchedDescT), _VP, _VP, _VP]),
    "tc_gemm_batched_async": (ctypes.c_int,
                              [_VP, ctypes.POINTER(BatchedDescT), _VP, _VP, _VP, _VP]),
    "tc_gemm_batched_async_noalloc": (ctypes.c_int,
                                      [_VP, ctypes.POINTER(BatchedDescT), _VP, _VP, _VP, _VP]),
    "tc_gemm_epilogue": (ctypes.c_int, [_VP, ctypes.POINTER(BatchedDescT),
                                        ctypes.POINTER(EpilogueT), _VP, _VP, _VP]),
    "tc_gemm_epilogue_async": (ctypes.c_int, [_VP, ctypes.POINTER(BatchedDescT),
                                              ctypes.POINTER(EpilogueT), _VP, _VP, _VP, _VP]),
    "tc_gemm_plan": (ctypes.c_int, [_VP, ctypes.POINTER(BatchedDescT),
                                    ctypes.POINTER(PlanInfoT)]),
    "tc_set_autotune": (ctypes.c_int, [_VP, ctypes.c_int]),
    "tc_autotune_entries": (ctypes.c_int64, [_VP]),
    "tc_last_kernel": (ctypes.c_char_p, [_VP]),
    "tc_dispatch_count": (ctypes.c_uint64, [_VP]),
    "tc_time_next_gemm": (ctypes.c_int, [_VP, _VP, _VP]),
    "tc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tc_last_error": (ctypes.c_char_p, [_VP]),
    "tc_tile_of_workgroup": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32)]),
    "tc_version": (ctypes.c_char_p, []),
}

_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtcgemm.so (built in-tree by dense_gemm_tiled_amd.build).

    Raises RuntimeError if it is missing: there is no other implementation.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            "libtcgemm.so is not built (%s); run `python -m dense_gemm_tiled_amd.build` "
            "or __graft_entry__.build()" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------------ context / streams
_ctx: Dict[int, int] = {}                       # device -> tc_context*
_streams: Dict[Tuple[int, int], int] = {}      # (device, hipStream_t) -> tc_stream*


def _check(status: int, ctx: Optional[int]) -> None:
    if status != 0:
        msg = load_library().tc_last_error(ctx)
        raise TcGemmError(status, (msg or b"").decode())


def _context(device: int) -> int:
    h = _ctx.get(device)
    if h is None:
        out = _VP()
        _check(load_library().tc_context_create(ctypes.byref(out)), None)
        h = out.value
        _ctx[device] = h
    return h


def _current_raw_stream(device: int) -> int:
    """torch's current stream on `device` as a hipStream_t (an int)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(device))
    return int(torch.cuda.current_stream(device).cuda_stream)


def _torch_stream(device: int, stream=None) -> Tuple[int, int]:
    handle = _current_raw_stream(device) if stream is None else int(stream.cuda_stream)
    key = (device, handle)
    s = _streams.get(key)
    ctx = _context(device)
    if s is None:
        import torch
        out = _VP()
        with torch.cuda.device(device):
            _check(load_library().tc_stream_wrap(ctx, _VP(handle), ctypes.byref(out)), ctx)
        s = out.value
        _streams[key] = s
    return ctx, s


def last_kernel(device: int = 0) -> str:
    return (load_library().tc_last_kernel(_context(device)) or b"").decode()


def dispatch_count(device: int = 0) -> int:
    return int(load_library().tc_dispatch_count(_context(device)))


def time_next_gemm(start, end, device: int = 0) -> None:
    """Have the next GEMM call record torch.cuda.Event `start` and `end` on
    its stream right around its main GEMM kernel (see tc_time_next_gemm).
    The events must already exist on the device (recorded once)."""
    ctx = _context(device)
    _check(load_library().tc_time_next_gemm(ctx, _VP(start.cuda_event), _VP(end.cuda_event)), ctx)


# ------------------------------------------------------------------ descriptors
def _dtype_code(t) -> int:
    import torch
    table = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
             torch.int8: I8, torch.int32: I32}
    if t.dtype not in table:
        raise TcGemmError(2, "unsupported tensor dtype %s" % t.dtype)
    return table[t.dtype]


def _ld(t) -> int:
    """Leading dimension (elements) of the last two dims of a row-major view."""
    if t.stride(-1) != 1 and t.size(-1) > 1:
        raise TcGemmError(1, "the last dimension must be contiguous (stride 1)")
    if t.size(-2) <= 1:
        return int(t.size(-1))
    return int(t.stride(-2))


def make_desc(a, b, c, alpha: float = 1.0, beta: float = 0.0,
              transpose_a: bool = False, transpose_b: bool = False) -> BatchedDescT:
    """Build the batched descriptor for tensors a, b, c (2-D or 3-D)."""
    if a.dim() not in (2, 3) or b.dim() not in (2, 3) or c.dim() not in (2, 3):
        raise TcGemmError(1, "operands must be 2-D or 3-D tensors")
    M, N = int(c.size(-2)), int(c.size(-1))
    K = int(a.size(-2) if transpose_a else a.size(-1))
    a_m = int(a.size(-1) if transpose_a else a.size(-2))
    b_k, b_n = (int(b.size(-1)), int(b.size(-2))) if transpose_b else (int(b.size(-2)), int(b.size(-1)))
    if a_m != M or b_n != N or b_k != K:
        raise TcGemmError(1, "shape mismatch: op(a) %dx%d, op(b) %dx%d, c %dx%d"
                          % (a_m, K, b_k, b_n, M, N))
    batch = int(c.size(0)) if c.dim() == 3 else 1
    for t in (a, b):
        if t.dim() == 3 and int(t.size(0)) != batch:
            raise TcGemmError(1, "batch sizes differ")
    ad, bd, cd = _dtype_code(a), _dtype_code(b), _dtype_code(c)
    accum = I32 if ad == I8 else F32
    desc = BatchedDescT()
    base = desc.base
    base.M, base.N, base.K = M, N, K
    base.a_dtype, base.b_dtype, base.c_dtype, base.accum_dtype = ad, bd, cd, accum
    base.transpose_a, base.transpose_b = bool(transpose_a), bool(transpose_b)
    base.alpha, base.beta = float(alpha), float(beta)
    base.lda, base.ldb, base.ldc = _ld(a), _ld(b), _ld(c)
    desc.batch = batch
    desc.stride_a = int(a.stride(0)) if a.dim() == 3 else 0
    desc.stride_b = int(b.stride(0)) if b.dim() == 3 else 0
    desc.stride_c = int(c.stride(0)) if c.dim() == 3 else 0
    return desc


# ------------------------------------------------------------------ API
def _column_vector(c, t, name: str, dtype) -> Tuple[int, int]:
    """(pointer, per-problem stride) of a [N] or [batch, N] GPU tensor."""
    N = int(c.size(-1))
    if not t.is_cuda or t.dtype != dtype:
        raise TcGemmError(1, "%s must be a GPU tensor of dtype %s" % (name, dtype))
    if int(t.size(-1)) != N or (t.size(-1) > 1 and t.stride(-1) != 1):
        raise TcGemmError(1, "%s must hold N contiguous values per problem" % name)
    stride = 0
    if t.dim() == 2:
        batch = int(c.size(0)) if c.dim() == 3 else 1
        if int(t.size(0)) != batch:
            raise TcGemmError(1, "%s has %d rows for %d problems" % (name, t.size(0), batch))
        stride = int(t.stride(0))
    elif t.dim() != 1:
        raise TcGemmError(1, "%s must be 1-D or 2-D" % name)
    return t.data_ptr(), stride


def make_epilogue(c, bias=None, activation: Optional[str] = None, col_scale=None) -> EpilogueT:
    """tc_epilogue for output c: bias is a GPU tensor of c's dtype and
    col_scale a float32 GPU tensor, each holding N values per problem ([N],
    shared by a batch, or [batch, N] with contiguous rows); activation is
    None, "none", "relu" or "gelu_tanh"."""
    import torch
    ep = EpilogueT()
    act = "none" if activation is None else activation
    if act not in ACTIVATIONS:
        raise TcGemmError(1, "unknown activation %r" % (activation,))
    ep.activation = ACTIVATIONS[act]
    ep.bias, ep.bias_stride, ep.col_scale, ep.scale_stride = None, 0, None, 0
    if bias is not None:
        ep.bias, ep.bias_stride = _column_vector(c, bias, "bias", c.dtype)
    if col_scale is not None:
        ep.col_scale, ep.scale_stride = _column_vector(c, col_scale, "col_scale", torch.float32)
    return ep


# Descriptors of the shapes seen so far (a call rebuilds none: its fields
# depend only on the key), bounded.
_desc_cache: Dict[tuple, BatchedDescT] = {}


def _desc_of(a, b, c, alpha, beta, transpose_a, transpose_b):
    """The descriptor of a call and a ctypes reference to it, cached per
    (types, shapes, strides, scalars, transposes)."""
    key = (a.dtype, b.dtype, c.dtype, a.shape, b.shape, c.shape, a.stride(), b.stride(),
           c.stride(), alpha, beta, transpose_a, transpose_b)
    d = _desc_cache.get(key)
    if d is None:
        desc = make_desc(a, b, c, alpha, beta, transpose_a, transpose_b)
        d = (desc, ctypes.byref(desc))
        if len(_desc_cache) < 4096:
            _desc_cache[key] = d
    return d


def gemm(a, b, c, *, alpha: float = 1.0, beta: float = 0.0, transpose_a: bool = False,
         transpose_b: bool = False, stream=None, bias=None, activation: Optional[str] = None,
         col_scale=None):
    """c = activation(alpha * (op(a) @ op(b)) * col_scale + beta * c + bias) on
    c's device, enqueued on torch's current stream (or `stream`).  Without
    bias, activation and col_scale this is the plain product
    (tc_gemm_batched_async), with any of them the fused epilogue
    (tc_gemm_epilogue_async); int8 a and b with a float c need col_scale
    (per-column dequantization).  Returns c."""
    if not (a.is_cuda and b.is_cuda and c.is_cuda):
        raise TcGemmError(1, "a, b and c must be GPU tensors")
    device = c.get_device()
    desc, dref = _desc_of(a, b, c, alpha, beta, transpose_a, transpose_b)
    lib = _lib if _lib is not None else load_library()
    ctx, s = _torch_stream(device, stream)
    if bias is None and activation is None and col_scale is None:
        st = lib.tc_gemm_batched_async(ctx, dref, a.data_ptr(), b.data_ptr(), c.data_ptr(), s)
    else:
        ep = make_epilogue(c, bias, activation, col_scale)
        st = lib.tc_gemm_epilogue_async(ctx, dref, ctypes.byref(ep), a.data_ptr(), b.data_ptr(),
                                        c.data_ptr(), s)
    if st != 0:
        _check(st, ctx)
    return c


def gemm_sync(a, b, c, *, alpha: float = 1.0, beta: float = 0.0, transpose_a: bool = False,
              transpose_b: bool = False):
    """Synchronous form: runs on the library context's own stream after
    synchronizing the device, and returns when c holds the result."""
    import torch
    device = c.device.index if c.device.index is not None else 0
    desc = make_desc(a, b, c, alpha, beta, transpose_a, transpose_b)
    torch.cuda.synchronize(device)
    lib = load_library()
    ctx = _context(device)
    with torch.cuda.device(device):
        st = lib.tc_gemm_batched(ctx, ctypes.byref(desc), _VP(a.data_ptr()), _VP(b.data_ptr()),
                                 _VP(c.data_ptr()))
    _check(st, ctx)
    return c


def set_autotune(enable: bool, device: int = 0) -> None:
    """Turn first-call autotuning on or off for the device's context (see
    tc_set_autotune)."""
    ctx = _context(device)
    _check(load_library().tc_set_autotune(ctx, int(bool(enable))), ctx)


def autotune_entries(device: int = 0) -> int:
    return int(load_library().tc_autotune_entries(_context(device)))


def plan(desc: BatchedDescT) -> dict:
    """Validate and plan a descriptor on the host (no GPU needed)."""
    lib = load_library()
    info = PlanInfoT()
    st = lib.tc_gemm_plan(None, ctypes.byref(desc), ctypes.byref(info))
    _check(st, None)
    out = {name: getattr(info, name) for name, _ in PlanInfoT._fields_}
    out["kernel"] = info.kernel.decode()
    return out
