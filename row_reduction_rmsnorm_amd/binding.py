"""ctypes binding of librowreduce.so (the C ABI declared in include/rowreduce.h).

Argument marshalling only: every operation runs in the library's HIP kernels.
PyTorch supplies device memory (tensors' data pointers) and the stream
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is missing or cannot be loaded, importing it raises.

The diagnostics build librowreduce_diag.so (include/rowreduce_diag.h: the
same kernel object plus a forced variant, the all-reduce self-test and the
streaming copy) is loaded only by ``diag_lib()``, ``forced_variant()``,
``rr_selftest_wave_allreduce`` and ``rr_stream_copy``, for tests and
measurement.
"""
import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree builds; ROWREDUCE_LIB may name another build of the library.
LIB_PATH = os.environ.get("ROWREDUCE_LIB") or os.path.join(HERE, "librowreduce.so")
DIAG_LIB_PATH = os.path.join(HERE, "librowreduce_diag.so")

RR_F32 = 0
RR_BF16 = 1
F32 = RR_F32
BF16 = RR_BF16

RR_OK = 0
RR_ERR_INVALID_ARG = 1
RR_ERR_UNSUPPORTED = 2
RR_ERR_WORKSPACE = 3
RR_ERR_HIP = 4

RR_OP_RMSNORM = 0
RR_OP_FUSED_ADD_RMSNORM = 1
RR_OP_SOFTMAX = 2
RR_OP_LAYERNORM = 3
RR_OP_SOFTMAX_CAUSAL = 4

RR_VARIANT_AUTO = 0
RR_VARIANT_WAVE = 1
RR_VARIANT_BLOCK = 2
RR_VARIANT_SPLIT = 3
RR_VARIANT_LOOP = 4
RR_VARIANT_SPLIT_ONE_KERNEL = 5
RR_VARIANT_SUBWAVE = 6
RR_VARIANT_SPLIT_TWO_KERNELS = 7
VARIANT_NAMES = {0: "auto", 1: "wave", 2: "block", 3: "split", 4: "loop", 5: "split1", 6: "subwave", 7: "split2"}

# Every function include/rowreduce.h declares.
EXPORTS = (
    "rr_rmsnorm", "rr_fused_add_rmsnorm", "rr_layernorm", "rr_softmax_rows_workspace_bytes",
    "rr_softmax_rows", "rr_softmax_rows_ex_workspace_bytes", "rr_softmax_rows_ex",
    "rr_rmsnorm_strided", "rr_fused_add_rmsnorm_strided", "rr_layernorm_strided",
    "rr_softmax_rows_strided", "rr_softmax_rows_strided_noalloc",
    "rr_status_string", "rr_last_error_message", "rr_query_plan",
)
# The one-kernel split's default wait (rowreduce_diag.h), 100 MHz ticks.
SPLIT_WAIT_TICKS_DEFAULT = 4000
# What include/rowreduce_diag.h adds in the diagnostics build.
DIAG_EXPORTS = ("rr_set_variant_override", "rr_selftest_wave_allreduce", "rr_stream_copy",
                "rr_set_split_wait_ticks", "rr_split_fallbacks")


class RowReduceError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class rr_softmax_opts(ctypes.Structure):
    _fields_ = [
        ("log_output", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("causal_period", ctypes.c_int64),
        ("causal_offset", ctypes.c_int64),
    ]


def make_softmax_opts(log_output=False, causal_period=None, causal_offset=0):
    """Options struct; causal_period None means no causal rule."""
    o = rr_softmax_opts()
    o.log_output = int(log_output)
    if causal_period is not None:
        o.causal = 1
        o.causal_period = int(causal_period)
        o.causal_offset = int(causal_offset)
    return o


class rr_plan(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("waves_per_row", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("vecs_per_lane", ctypes.c_int32),
        ("vec_elems", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("chunks_per_row", ctypes.c_int64),
        ("work_items", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("row_shift", ctypes.c_int32),
    ]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["variant_name"] = VARIANT_NAMES.get(self.variant, "?")
        return d


_LIB = None
_DIAG = None
_ROUTED = None     # the diagnostics build while forced_variant() is active


def lib():
    """The loaded library (built in-tree on first use if it is not there);
    inside forced_variant(), the diagnostics build."""
    global _LIB
    if _ROUTED is not None:
        return _ROUTED
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        if os.environ.get("ROWREDUCE_LIB"):
            raise ImportError(f"ROWREDUCE_LIB={LIB_PATH} does not exist")
        from . import build as _build
        _build.build()
    _LIB = load_library(LIB_PATH)
    return _LIB


def diag_lib():
    """The diagnostics build (built in-tree on first use if it is not there)."""
    global _DIAG
    if _DIAG is not None:
        return _DIAG
    if not os.path.exists(DIAG_LIB_PATH):
        from . import build as _build
        _build.build()
    _DIAG = load_library(DIAG_LIB_PATH)
    return _DIAG


@contextlib.contextmanager
def forced_variant(variant: int):
    """Run every call of this module inside the block through the
    diagnostics build with `variant` (an rr_variant code) forced, then
    restore automatic choice and the product library.  For tests and
    measurement; not thread-safe."""
    global _ROUTED
    D = diag_lib()
    st = D.rr_set_variant_override(int(variant))
    if st != RR_OK:
        raise RowReduceError(st, f"rr_set_variant_override({variant}): {D.rr_status_string(st).decode()}: "
                                 f"{D.rr_last_error_message().decode()}")
    prev = _ROUTED
    _ROUTED = D
    try:
        yield D
    finally:
        D.rr_set_variant_override(RR_VARIANT_AUTO)
        _ROUTED = prev


def load_library(path):
    """A ctypes handle on a build of the library at `path` with every
    declared function's argument and result types set (lib() uses it for
    the library itself; the race-stress tests use it for the stress build)."""
    try:
        L = ctypes.CDLL(path)
    except OSError as e:
        raise ImportError(f"cannot load {path}: {e}") from e
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    L.rr_rmsnorm.argtypes = [vp, vp, vp, i64, i64, f32, i32, vp]
    L.rr_fused_add_rmsnorm.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.rr_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.rr_softmax_rows_workspace_bytes.argtypes = [i64, i64, i32, i32]
    L.rr_softmax_rows_workspace_bytes.restype = ctypes.c_size_t
    L.rr_softmax_rows.argtypes = [vp, vp, i64, i64, i32, i32, vp, ctypes.c_size_t, vp]
    po = ctypes.POINTER(rr_softmax_opts)
    L.rr_softmax_rows_ex_workspace_bytes.argtypes = [i64, i64, i32, i32, po]
    L.rr_softmax_rows_ex_workspace_bytes.restype = ctypes.c_size_t
    L.rr_softmax_rows_ex.argtypes = [vp, vp, i64, i64, i32, i32, po, vp, ctypes.c_size_t, vp]
    L.rr_rmsnorm_strided.argtypes = [vp, i64, vp, i64, vp, i64, i64, f32, i32, vp]
    L.rr_fused_add_rmsnorm_strided.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, f32, i32, vp]
    L.rr_layernorm_strided.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, f32, i32, vp]
    L.rr_softmax_rows_strided.argtypes = [vp, i64, vp, i64, i64, i64, i32, i32, po, vp,
                                          ctypes.c_size_t, vp]
    L.rr_softmax_rows_strided_noalloc.argtypes = [vp, i64, vp, i64, i64, i64, i32, i32, po, vp]
    L.rr_status_string.argtypes = [i32]
    L.rr_status_string.restype = ctypes.c_char_p
    L.rr_last_error_message.argtypes = []
    L.rr_last_error_message.restype = ctypes.c_char_p
    L.rr_query_plan.argtypes = [i32, i64, i64, i32, i32, i32, ctypes.POINTER(rr_plan)]
    for f in ("rr_rmsnorm", "rr_fused_add_rmsnorm", "rr_layernorm", "rr_softmax_rows",
              "rr_softmax_rows_ex", "rr_query_plan", "rr_rmsnorm_strided",
              "rr_fused_add_rmsnorm_strided", "rr_layernorm_strided", "rr_softmax_rows_strided",
              "rr_softmax_rows_strided_noalloc"):
        getattr(L, f).restype = i32
    # the diagnostics build's additions (absent from the product library)
    if hasattr(L, "rr_set_variant_override"):
        L.rr_set_variant_override.argtypes = [i32]
        L.rr_selftest_wave_allreduce.argtypes = [vp, vp, i64, i32, vp]
        L.rr_stream_copy.argtypes = [vp, vp, i64, vp]
        L.rr_set_split_wait_ticks.argtypes = [ctypes.c_uint64]
        L.rr_split_fallbacks.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
        for f in DIAG_EXPORTS:
            getattr(L, f).restype = i32
    return L


def status_string(status: int) -> str:
    return lib().rr_status_string(int(status)).decode()


def last_error_message() -> str:
    return lib().rr_last_error_message().decode()


def check(status: int, what: str = "") -> None:
    if status != RR_OK:
        raise RowReduceError(status, f"{what}: {status_string(status)}: {last_error_message()}")


# ----------------------------------------------------------------------------
# raw C-ABI calls (integers for pointers and streams)
# ----------------------------------------------------------------------------

def raw_rmsnorm(y, x, gamma, M, H, eps, dtype, stream):
    return lib().rr_rmsnorm(y, x, gamma, M, H, eps, dtype, stream)


def raw_fused_add_rmsnorm(y, residual, x, gamma, M, H, eps, dtype, stream):
    return lib().rr_fused_add_rmsnorm(y, residual, x, gamma, M, H, eps, dtype, stream)


def raw_layernorm(y, x, gamma, beta, M, H, eps, dtype, stream):
    return lib().rr_layernorm(y, x, gamma, beta, M, H, eps, dtype, stream)


def raw_softmax_rows(y, x, M, N, in_dtype, out_dtype, workspace, workspace_bytes, stream):
    return lib().rr_softmax_rows(y, x, M, N, in_dtype, out_dtype, workspace, workspace_bytes,
                                 stream)


def rr_softmax_rows_workspace_bytes(M: int, N: int, in_dtype: int, out_dtype: int) -> int:
    return int(lib().rr_softmax_rows_workspace_bytes(M, N, in_dtype, out_dtype))


def _opts_ref(opts):
    return ctypes.byref(opts) if opts is not None else None


def raw_softmax_rows_ex(y, x, M, N, in_dtype, out_dtype, opts, workspace, workspace_bytes, stream):
    """opts: an rr_softmax_opts or None."""
    return lib().rr_softmax_rows_ex(y, x, M, N, in_dtype, out_dtype, _opts_ref(opts), workspace,
                                    workspace_bytes, stream)


def raw_rmsnorm_strided(y, ldy, x, ldx, gamma, M, H, eps, dtype, stream):
    return lib().rr_rmsnorm_strided(y, ldy, x, ldx, gamma, M, H, eps, dtype, stream)


def raw_fused_add_rmsnorm_strided(y, ldy, residual, ldr, x, ldx, gamma, M, H, eps, dtype, stream):
    return lib().rr_fused_add_rmsnorm_strided(y, ldy, residual, ldr, x, ldx, gamma, M, H, eps, dtype,
                                              stream)


def raw_layernorm_strided(y, ldy, x, ldx, gamma, beta, M, H, eps, dtype, stream):
    return lib().rr_layernorm_strided(y, ldy, x, ldx, gamma, beta, M, H, eps, dtype, stream)


def raw_softmax_rows_strided(y, ldy, x, ldx, M, N, in_dtype, out_dtype, opts, workspace,
                             workspace_bytes, stream):
    return lib().rr_softmax_rows_strided(y, ldy, x, ldx, M, N, in_dtype, out_dtype, _opts_ref(opts),
                                         workspace, workspace_bytes, stream)


def raw_softmax_rows_strided_noalloc(y, ldy, x, ldx, M, N, in_dtype, out_dtype, opts, stream):
    return lib().rr_softmax_rows_strided_noalloc(y, ldy, x, ldx, M, N, in_dtype, out_dtype, _opts_ref(opts),
                                                 stream)


def rr_softmax_rows_ex_workspace_bytes(M: int, N: int, in_dtype: int, out_dtype: int, opts=None) -> int:
    return int(lib().rr_softmax_rows_ex_workspace_bytes(M, N, in_dtype, out_dtype, _opts_ref(opts)))


def rr_query_plan(op: int, M: int, N: int, in_dtype: int, out_dtype: int, aligned16=True):
    """aligned16: True/1 vector-aligned rows; False/0 element access; 2 rows
    at a common offset within a vector (see include/rowreduce.h)."""
    p = rr_plan()
    mode = 2 if aligned16 == 2 else (1 if aligned16 else 0)
    check(lib().rr_query_plan(op, M, N, in_dtype, out_dtype, mode, ctypes.byref(p)), "rr_query_plan")
    return p.as_dict()


# ----------------------------------------------------------------------------
# tensor-level calls (marshalling only)
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RR_F32
    if t.dtype == torch.bfloat16:
        return RR_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream_of(t, stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _rows(t):
    if t.dim() == 0:
        raise ValueError("need at least one dimension")
    n = t.shape[-1]
    m = t.numel() // n if n else 0
    return m, n


def _rows_ld(t):
    """(M, N, row stride) of a tensor whose rows are contiguous and evenly
    spaced: unit stride in the last dimension, and leading dimensions that
    flatten to one (each stride the next one times its size)."""
    if t.dim() == 0:
        raise ValueError("need at least one dimension")
    if not t.is_cuda:
        raise ValueError("tensors must live on a GPU device")
    n = t.shape[-1]
    m = t.numel() // n if n else 0
    if n > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must have unit stride")
    if t.dim() == 1:
        return m, n, n
    for i in range(t.dim() - 2):
        if t.shape[i] > 1 and t.stride(i) != t.stride(i + 1) * t.shape[i + 1]:
            raise ValueError("leading dimensions must flatten to one row dimension")
    ld = t.stride(-2) if t.shape[-2] > 1 else n
    return m, n, max(ld, n) if m <= 1 else ld


def rr_rmsnorm_strided(y, x, gamma, eps: float, stream=None) -> None:
    """rr_rmsnorm on views whose rows are evenly spaced (a column slice)."""
    _need_cuda(gamma)
    M, H, ldx = _rows_ld(x)
    My, Hy, ldy = _rows_ld(y)
    if (My, Hy) != (M, H) or gamma.shape != (H,):
        raise ValueError("y must match x and gamma must be [H]")
    dt = dtype_code(x)
    if dtype_code(y) != dt or dtype_code(gamma) != dt:
        raise TypeError("x, y and gamma must share one dtype")
    check(raw_rmsnorm_strided(y.data_ptr(), ldy, x.data_ptr(), ldx, gamma.data_ptr(), M, H,
                              float(eps), dt, _stream_of(x, stream)), "rr_rmsnorm_strided")


def rr_fused_add_rmsnorm_strided(y, residual, x, gamma, eps: float, stream=None) -> None:
    _need_cuda(gamma)
    M, H, ldx = _rows_ld(x)
    My, Hy, ldy = _rows_ld(y)
    Mr, Hr, ldr = _rows_ld(residual)
    if (My, Hy) != (M, H) or (Mr, Hr) != (M, H) or gamma.shape != (H,):
        raise ValueError("y and residual must match x and gamma must be [H]")
    dt = dtype_code(x)
    if any(dtype_code(t) != dt for t in (y, residual, gamma)):
        raise TypeError("all tensors must share one dtype")
    check(raw_fused_add_rmsnorm_strided(y.data_ptr(), ldy, residual.data_ptr(), ldr, x.data_ptr(),
                                        ldx, gamma.data_ptr(), M, H, float(eps), dt,
                                        _stream_of(x, stream)), "rr_fused_add_rmsnorm_strided")


def rr_layernorm_strided(y, x, gamma, beta, eps: float, stream=None) -> None:
    _need_cuda(gamma)
    M, H, ldx = _rows_ld(x)
    My, Hy, ldy = _rows_ld(y)
    if (My, Hy) != (M, H) or gamma.shape != (H,) or (beta is not None and beta.shape != (H,)):
        raise ValueError("y must match x and gamma, beta must be [H]")
    dt = dtype_code(x)
    if dtype_code(y) != dt or dtype_code(gamma) != dt or (beta is not None and dtype_code(beta) != dt):
        raise TypeError("all tensors must share one dtype")
    bp = None
    if beta is not None:
        _need_cuda(beta)
        bp = beta.data_ptr()
    check(raw_layernorm_strided(y.data_ptr(), ldy, x.data_ptr(), ldx, gamma.data_ptr(), bp, M, H,
                                float(eps), dt, _stream_of(x, stream)), "rr_layernorm_strided")


def rr_softmax_rows_strided(y, x, opts=None, workspace=None, stream=None) -> None:
    M, N, ldx = _rows_ld(x)
    My, Ny, ldy = _rows_ld(y)
    if (My, Ny) != (M, N):
        raise ValueError("y must match x")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need_cuda(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(raw_softmax_rows_strided(y.data_ptr(), ldy, x.data_ptr(), ldx, M, N, dtype_code(x),
                                   dtype_code(y), opts, ws_ptr, ws_bytes, _stream_of(x, stream)),
          "rr_softmax_rows_strided")


def rr_softmax_rows_strided_noalloc(y, x, opts=None, stream=None) -> None:
    """rr_softmax_rows_strided with the split row's slots in the library's
    static scratch array (no workspace, nothing allocated)."""
    M, N, ldx = _rows_ld(x)
    My, Ny, ldy = _rows_ld(y)
    if (My, Ny) != (M, N):
        raise ValueError("y must match x")
    check(raw_softmax_rows_strided_noalloc(y.data_ptr(), ldy, x.data_ptr(), ldx, M, N, dtype_code(x),
                                           dtype_code(y), opts, _stream_of(x, stream)),
          "rr_softmax_rows_strided_noalloc")


def rr_rmsnorm(y, x, gamma, eps: float, stream=None) -> None:
    """y = x * rsqrt(mean(x^2) + eps) * gamma over the last dimension."""
    _need_cuda(y, x, gamma)
    M, H = _rows(x)
    if y.shape != x.shape or gamma.shape != (H,):
        raise ValueError("y must match x and gamma must be [H]")
    dt = dtype_code(x)
    if dtype_code(y) != dt or dtype_code(gamma) != dt:
        raise TypeError("x, y and gamma must share one dtype")
    check(raw_rmsnorm(y.data_ptr(), x.data_ptr(), gamma.data_ptr(), M, H, float(eps), dt,
                      _stream_of(x, stream)), "rr_rmsnorm")


def rr_fused_add_rmsnorm(y, residual, x, gamma, eps: float, stream=None) -> None:
    """residual <- residual + x (rounded to the dtype); y = rmsnorm(residual) * gamma."""
    _need_cuda(y, residual, x, gamma)
    M, H = _rows(x)
    if y.shape != x.shape or residual.shape != x.shape or gamma.shape != (H,):
        raise ValueError("y and residual must match x and gamma must be [H]")
    dt = dtype_code(x)
    if any(dtype_code(t) != dt for t in (y, residual, gamma)):
        raise TypeError("all tensors must share one dtype")
    check(raw_fused_add_rmsnorm(y.data_ptr(), residual.data_ptr(), x.data_ptr(),
                                gamma.data_ptr(), M, H, float(eps), dt,
                                _stream_of(x, stream)), "rr_fused_add_rmsnorm")


def rr_layernorm(y, x, gamma, beta, eps: float, stream=None) -> None:
    """y = (x - mean) * rsqrt(var + eps) * gamma + beta over the last dimension
    (beta may be None)."""
    _need_cuda(y, x, gamma)
    M, H = _rows(x)
    if y.shape != x.shape or gamma.shape != (H,) or (beta is not None and beta.shape != (H,)):
        raise ValueError("y must match x; gamma and beta must be [H]")
    dt = dtype_code(x)
    if dtype_code(y) != dt or dtype_code(gamma) != dt:
        raise TypeError("x, y, gamma and beta must share one dtype")
    bp = None
    if beta is not None:
        _need_cuda(beta)
        if dtype_code(beta) != dt:
            raise TypeError("x, y, gamma and beta must share one dtype")
        bp = beta.data_ptr()
    check(raw_layernorm(y.data_ptr(), x.data_ptr(), gamma.data_ptr(), bp, M, H, float(eps), dt,
                        _stream_of(x, stream)), "rr_layernorm")


def rr_softmax_rows(y, x, workspace=None, stream=None) -> None:
    """Row softmax of x into y over the last dimension (y may be x when dtypes match).

    workspace: a uint8 device tensor of at least rr_softmax_rows_workspace_bytes
    bytes when that is non-zero."""
    _need_cuda(y, x)
    M, N = _rows(x)
    if y.shape != x.shape:
        raise ValueError("y must match x")
    din, dout = dtype_code(x), dtype_code(y)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need_cuda(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(raw_softmax_rows(y.data_ptr(), x.data_ptr(), M, N, din, dout, ws_ptr, ws_bytes,
                           _stream_of(x, stream)), "rr_softmax_rows")


def rr_softmax_rows_ex(y, x, opts=None, workspace=None, stream=None) -> None:
    """rr_softmax_rows with an rr_softmax_opts (log output, causal rule)."""
    _need_cuda(y, x)
    M, N = _rows(x)
    if y.shape != x.shape:
        raise ValueError("y must match x")
    din, dout = dtype_code(x), dtype_code(y)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need_cuda(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(raw_softmax_rows_ex(y.data_ptr(), x.data_ptr(), M, N, din, dout, opts, ws_ptr, ws_bytes,
                              _stream_of(x, stream)), "rr_softmax_rows_ex")


def rr_selftest_wave_allreduce(out, inp, kind: int, stream=None) -> None:
    _need_cuda(out, inp)
    per = 128 if kind == 2 else 64
    if inp.numel() % per or out.numel() != inp.numel():
        raise ValueError("bad self-test sizes")
    D = diag_lib()
    st = D.rr_selftest_wave_allreduce(inp.data_ptr(), out.data_ptr(), inp.numel() // per, int(kind),
                                      _stream_of(inp, stream))
    if st != RR_OK:
        raise RowReduceError(st, f"rr_selftest_wave_allreduce: {D.rr_last_error_message().decode()}")


def rr_stream_copy(dst, src, stream=None) -> None:
    """dst <- src, every byte, by the diagnostics build's streaming copy (a
    measurement reference: the practical bar for an operation moving the same
    bytes)."""
    _need_cuda(dst, src)
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("rr_stream_copy: contiguous tensors of equal byte size required")
    D = diag_lib()
    st = D.rr_stream_copy(dst.data_ptr(), src.data_ptr(), nb, _stream_of(src, stream))
    if st != RR_OK:
        raise RowReduceError(st, f"rr_stream_copy: {D.rr_last_error_message().decode()}")


def split_fallbacks(reset: bool = False) -> int:
    """The current device's count, in the diagnostics build, of one-kernel
    split chunks summarised again because their wait expired (reset clears
    it afterwards).  Only calls made through the diagnostics build count
    there (forced_variant(), split_wait() or diag_lib() directly)."""
    D = diag_lib()
    n = ctypes.c_uint32(0)
    st = D.rr_split_fallbacks(ctypes.byref(n), 1 if reset else 0)
    if st != RR_OK:
        raise RowReduceError(st, f"rr_split_fallbacks: {D.rr_last_error_message().decode()}")
    return int(n.value)


@contextlib.contextmanager
def split_wait(ticks: int):
    """Run every call of this module inside the block through the
    diagnostics build with the one-kernel split's wait set to `ticks` of the
    100 MHz clock (0: give up at once), then restore the default wait and
    the product library.  For tests; not thread-safe."""
    global _ROUTED
    D = diag_lib()
    st = D.rr_set_split_wait_ticks(int(ticks))
    if st != RR_OK:
        raise RowReduceError(st, f"rr_set_split_wait_ticks: {D.rr_last_error_message().decode()}")
    prev = _ROUTED
    _ROUTED = D
    try:
        yield D
    finally:
        D.rr_set_split_wait_ticks(SPLIT_WAIT_TICKS_DEFAULT)
        _ROUTED = prev


# ----------------------------------------------------------------------------
# allocating conveniences (outputs and workspace come from torch)
# ----------------------------------------------------------------------------

def rmsnorm(x, gamma, eps: float, out=None):
    y = _torch().empty_like(x) if out is None else out
    rr_rmsnorm(y, x, gamma, eps)
    return y


def layernorm(x, gamma, beta, eps: float, out=None):
    y = _torch().empty_like(x) if out is None else out
    rr_layernorm(y, x, gamma, beta, eps)
    return y


def fused_add_rmsnorm(x, residual, gamma, eps: float, out=None):
    """Updates residual in place and returns y."""
    y = _torch().empty_like(x) if out is None else out
    rr_fused_add_rmsnorm(y, residual, x, gamma, eps)
    return y


def softmax_workspace(x, out_dtype):
    torch = _torch()
    M, N = _rows(x)
    n = rr_softmax_rows_workspace_bytes(M, N, dtype_code(x),
                                        RR_F32 if out_dtype == torch.float32 else RR_BF16)
    return torch.empty(n, dtype=torch.uint8, device=x.device) if n else None


def softmax_rows_ex(x, out_dtype=None, out=None, log_output=False, causal_period=None,
                    causal_offset=0, workspace=None):
    """Softmax or log-softmax of each row; with causal_period, row i keeps
    the keys j <= (i mod causal_period) + causal_offset (the rest is never
    read and comes out as 0, or -inf for log output)."""
    torch = _torch()
    opts = make_softmax_opts(log_output, causal_period, causal_offset)
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if workspace is None:
        M, N = _rows(x)
        n = rr_softmax_rows_ex_workspace_bytes(M, N, dtype_code(x), dtype_code(out), opts)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    rr_softmax_rows_ex(out, x, opts, workspace)
    return out


def softmax_rows(x, out_dtype=None, out=None, workspace=None):
    torch = _torch()
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if workspace is None:
        workspace = softmax_workspace(x, out.dtype)
    rr_softmax_rows(out, x, workspace)
    return out
