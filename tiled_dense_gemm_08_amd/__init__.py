"""Python binding of libtg.so, the gfx950 tiled fp16 GEMM (+ fused bias + ReLU).

The functions named tg_* mirror the C ABI in include/tg.h one to one: they
take raw device pointers (ints) and sizes and return the tg_status code.
`gemm` and `gemm_bias_relu` marshal torch tensors (device memory and the
current stream only) into those calls; every step of the computation runs in
the library's HIP kernels.  The library must be built (see build.py); there
is no fallback: importing this package fails if libtg.so is missing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtg.so")
# the LDS-poison debug build of the same sources (build.py), for tests
POISON_LIB_PATH = os.path.join(HERE, "libtg_poison.so")

TG_DTYPE_F16 = 1
TG_DTYPE_F32 = 2
TG_DTYPE_I32 = 3   # int8 operands, int32 C
TG_CEILING_OPERAND_BYTES = 131072   # operand buffer of tg_mfma_ceiling

TG_SUCCESS = 0
TG_ERROR_INVALID_VALUE = 1
TG_ERROR_NOT_DEVICE_MEMORY = 2
TG_ERROR_UNSUPPORTED = 3
TG_ERROR_LAUNCH = 4
TG_ERROR_FILE = 5
TG_ERROR_WORKSPACE = 6

TG_OP_N = 0
TG_OP_T = 1

# every function declared in include/tg.h and include/tg_diag.h
EXPORTED = ("tg_gemm", "tg_gemm_bias_relu", "tg_gemm_ex", "tg_status_string", "tg_num_configs",
            "tg_config_info", "tg_config_supports", "tg_select_config",
            "tg_gemm_with_config", "tg_tuning_load", "tg_tuning_clear", "tg_tuning_count",
            "tg_splitk_workspace_bytes", "tg_gemm_ws", "tg_gemm_ws_static", "tg_select_plan",
            "tg_attention_fwd", "tg_mfma_ceiling", "tg_version")


class TgError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, tg_status_string(status)))


class ConfigDesc(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("block_k", ctypes.c_int), ("stages", ctypes.c_int), ("waves_m", ctypes.c_int),
                ("waves_n", ctypes.c_int), ("mfma", ctypes.c_int), ("direct_lds", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("ops", ctypes.c_int), ("elem_bytes", ctypes.c_int),
                ("whole_k", ctypes.c_int), ("name", ctypes.c_char_p)]


def load_library(path=LIB_PATH):
    """A build of the library at `path` with every C ABI function declared."""
    # The library must run on the same HIP runtime as the framework that owns
    # the device memory.  PyTorch ships its own libamdhip64; importing it
    # first makes libtg.so bind to that copy instead of loading a second
    # runtime that would not know torch's allocations.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError("%s is not built; run `python tiled_dense_gemm_08_amd/build.py`"
                          % path)
    L = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    gemm_args = [I64, I64, I64, I64, I64, I64, I, P]
    L.tg_gemm.argtypes = [P, P, P] + gemm_args
    L.tg_gemm.restype = I
    L.tg_gemm_bias_relu.argtypes = [P, P, P, P] + gemm_args
    L.tg_gemm_bias_relu.restype = I
    L.tg_gemm_ex.argtypes = [I, I, P, P, P, P] + gemm_args
    L.tg_gemm_ex.restype = I
    L.tg_gemm_with_config.argtypes = [I, I, I, P, P, P, P] + gemm_args
    L.tg_gemm_with_config.restype = I
    L.tg_status_string.argtypes = [I]
    L.tg_status_string.restype = ctypes.c_char_p
    L.tg_num_configs.argtypes = []
    L.tg_num_configs.restype = I
    L.tg_config_info.argtypes = [I, ctypes.POINTER(ConfigDesc)]
    L.tg_config_info.restype = I
    shape_args = [P, P, P, P, I64, I64, I64, I64, I64, I64, I]
    L.tg_config_supports.argtypes = [I, I, I] + shape_args
    L.tg_config_supports.restype = I
    L.tg_select_config.argtypes = [I, I] + shape_args
    L.tg_select_config.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    SZ = ctypes.c_size_t
    L.tg_splitk_workspace_bytes.argtypes = [I64, I64, I]
    L.tg_splitk_workspace_bytes.restype = SZ
    L.tg_gemm_ws.argtypes = [I, I, I, I, P, P, P, P, I64, I64, I64, I64, I64, I64, I, P, SZ, P]
    L.tg_gemm_ws.restype = I
    L.tg_gemm_ws_static.argtypes = [I, I, I, I, P, P, P, P, I64, I64, I64, I64, I64, I64, I, P]
    L.tg_gemm_ws_static.restype = I
    L.tg_select_plan.argtypes = [I, I] + shape_args + [SZ, IP, IP, IP, ctypes.POINTER(SZ)]
    L.tg_select_plan.restype = I
    L.tg_attention_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P,
                                   ctypes.c_float, I, P]
    L.tg_attention_fwd.restype = I
    L.tg_tuning_load.argtypes = [ctypes.c_char_p, IP, IP, IP]
    L.tg_tuning_load.restype = I
    L.tg_tuning_clear.argtypes = []
    L.tg_tuning_clear.restype = I
    L.tg_tuning_count.argtypes = []
    L.tg_tuning_count.restype = I
    L.tg_mfma_ceiling.argtypes = [I, P, P, I64, I64, P]
    L.tg_mfma_ceiling.restype = I
    L.tg_version.argtypes = []
    L.tg_version.restype = ctypes.c_char_p
    return L


lib = load_library()


# ------------------------------------------------------------ raw C ABI --
def tg_gemm(A, B, C, M, N, K, lda, ldb, ldc, c_dtype, stream=0):
    return lib.tg_gemm(A, B, C, M, N, K, lda, ldb, ldc, c_dtype, stream or None)


def tg_gemm_bias_relu(A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, stream=0):
    return lib.tg_gemm_bias_relu(A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, stream or None)


def tg_gemm_ex(op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, stream=0):
    return lib.tg_gemm_ex(op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype,
                          stream or None)


def tg_gemm_with_config(config_id, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, stream=0,
                        op_a=TG_OP_N, op_b=TG_OP_N):
    return lib.tg_gemm_with_config(config_id, op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc,
                                   c_dtype, stream or None)


def tg_status_string(status):
    return lib.tg_status_string(status).decode()


def tg_num_configs():
    return lib.tg_num_configs()


def tg_config_info(config_id):
    d = ConfigDesc()
    st = lib.tg_config_info(config_id, ctypes.byref(d))
    if st != TG_SUCCESS:
        raise TgError(st, "tg_config_info(%d)" % config_id)
    return {f: (getattr(d, f).decode() if f == "name" else getattr(d, f)) for f, _ in d._fields_}


def tg_config_supports(config_id, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype,
                       op_a=TG_OP_N, op_b=TG_OP_N):
    return lib.tg_config_supports(config_id, op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc,
                                  c_dtype)


def tg_select_config(A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, op_a=TG_OP_N,
                     op_b=TG_OP_N):
    return lib.tg_select_config(op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype)


def tg_splitk_workspace_bytes(M, N, splits):
    return lib.tg_splitk_workspace_bytes(M, N, splits)


def tg_gemm_ws(config_id, splits, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, workspace,
               workspace_bytes, stream=0, op_a=TG_OP_N, op_b=TG_OP_N):
    return lib.tg_gemm_ws(config_id, splits, op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc,
                          c_dtype, workspace, workspace_bytes, stream or None)


def tg_gemm_ws_static(config_id, splits, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype,
                      stream=0, op_a=TG_OP_N, op_b=TG_OP_N):
    return lib.tg_gemm_ws_static(config_id, splits, op_a, op_b, A, B, bias, C, M, N, K, lda, ldb,
                                 ldc, c_dtype, stream or None)


TG_STATIC_SCRATCH_BYTES = 64 << 20   # the library's workspace of tg_gemm_ws_static

SIZE_MAX = ctypes.c_size_t(-1).value


def tg_select_plan(A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, workspace_bytes=SIZE_MAX,
                   op_a=TG_OP_N, op_b=TG_OP_N):
    """What tg_gemm_ws(-1, 0, ...) runs with that much workspace:
    (status, config id, slices, packed-operand mask (1: A, 2: B), workspace bytes used)."""
    cid, sp, packed, used = ctypes.c_int(-2), ctypes.c_int(-2), ctypes.c_int(-1), ctypes.c_size_t(0)
    st = lib.tg_select_plan(op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype,
                            workspace_bytes, ctypes.byref(cid), ctypes.byref(sp),
                            ctypes.byref(packed), ctypes.byref(used))
    return st, cid.value, sp.value, packed.value, used.value


def _strides3(st):
    a = (ctypes.c_int64 * 3)(*[int(x) for x in st])
    return a


def tg_attention_fwd(Q, K, V, O, lse, B, H, Hkv, Lq, Lk, d, q_strides, k_strides, v_strides,
                     o_strides, scale, causal, stream=0):
    return lib.tg_attention_fwd(Q, K, V, O, lse, B, H, Hkv, Lq, Lk, d, _strides3(q_strides),
                                _strides3(k_strides), _strides3(v_strides),
                                _strides3(o_strides), scale, int(causal), stream or None)


def tg_tuning_load(path):
    """Returns (status, loaded, skipped, error_line)."""
    loaded, skipped, line = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_int(-1)
    st = lib.tg_tuning_load(None if path is None else os.fsencode(path), ctypes.byref(loaded),
                            ctypes.byref(skipped), ctypes.byref(line))
    return st, loaded.value, skipped.value, line.value


def tg_tuning_clear():
    return lib.tg_tuning_clear()


def tg_tuning_count():
    return lib.tg_tuning_count()


def tg_mfma_ceiling(mfma, operands, sink, iters, workgroups, stream=0):
    return lib.tg_mfma_ceiling(mfma, operands, sink, iters, workgroups, stream or None)


def tg_version():
    return lib.tg_version().decode()


def load_tuning(path):
    """Load a tuning cache file (written by `sweep --tune`); raises TgError
    naming the offending line.  Returns (loaded, skipped)."""
    st, loaded, skipped, line = tg_tuning_load(path)
    if st != TG_SUCCESS:
        raise TgError(st, "tg_tuning_load(%s) line %d" % (path, line))
    return loaded, skipped


def configs():
    return [tg_config_info(i) for i in range(tg_num_configs())]


# --------------------------------------------------- torch marshalling --
def _dtype_code(t):
    import torch
    if t == torch.float16:
        return TG_DTYPE_F16
    if t == torch.float32:
        return TG_DTYPE_F32
    raise TypeError("output dtype must be float16 or float32, got %s" % t)


def _matrix(t, name):
    """Pointer and leading dimension of a row-major 2-D tensor."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.size(0) > 1 and t.stride(1) != 1 or t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major (unit column stride)" % name)
    ld = t.stride(0) if t.size(0) > 1 else t.size(1)
    return t.data_ptr(), max(ld, t.size(1))


def _operand(t, name):
    """Pointer, leading dimension and orientation of an operand tensor: a
    row-major tensor is used as stored (TG_OP_N); a tensor with unit row
    stride (a transposed view of a row-major array) is passed as the stored
    array with TG_OP_T."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.stride(1) == 1 or t.size(1) == 1:
        p, ld = _matrix(t, name)
        return p, ld, TG_OP_N
    if t.stride(0) == 1 or t.size(0) == 1:
        p, ld = _matrix(t.t(), name)
        return p, ld, TG_OP_T
    raise ValueError("%s must be row-major or a transposed row-major view" % name)


def gemm(a, b, out=None, out_dtype=None, bias=None, config=None, stream=None, workspace=None,
         splits=0):
    """C = A.B (or max(A.B + bias, 0) when bias is given) with libtg.

    a: (M, K) float16, b: (K, N) float16 on the current device, each row-major
    or a transposed view of a row-major array (passed with TG_OP_T, no copy);
    out: optional preallocated (M, N) float16/float32 row-major tensor.
    config: None (dispatcher's choice) or a configuration id.
    workspace: optional device tensor (any dtype, contiguous) passed to
    tg_gemm_ws, which may then slice K or pack operands into it; splits: 0
    lets the dispatcher choose, n >= 1 forces n slices (needs a workspace when
    n > 1).  workspace_bytes(...) gives the size the fastest plan uses.
    """
    import torch
    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("A and B must be float16")
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (M, N)))
    pa, lda, op_a = _operand(a, "A")
    pb, ldb, op_b = _operand(b, "B")
    pc, ldc = _matrix(out, "C")
    code = _dtype_code(out.dtype)
    pbias = 0
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() != 1 or bias.numel() < N or bias.stride(0) != 1:
            raise ValueError("bias must be a contiguous float32 vector of length N")
        pbias = bias.data_ptr()
    s = (stream if stream is not None else torch.cuda.current_stream(a.device)).cuda_stream
    if workspace is not None or splits:
        pw, nw = 0, 0
        if workspace is not None:
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
            pw, nw = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = tg_gemm_ws(-1 if config is None else config, splits, pa, pb, pbias or None, pc,
                        M, N, K, lda, ldb, ldc, code, pw or None, nw, s, op_a=op_a, op_b=op_b)
    elif config is not None:
        st = tg_gemm_with_config(config, pa, pb, pbias or None, pc, M, N, K, lda, ldb, ldc,
                                 code, s, op_a=op_a, op_b=op_b)
    elif op_a or op_b:
        st = tg_gemm_ex(op_a, op_b, pa, pb, pbias or None, pc, M, N, K, lda, ldb, ldc, code, s)
    elif bias is not None:
        st = tg_gemm_bias_relu(pa, pb, pbias, pc, M, N, K, lda, ldb, ldc, code, s)
    else:
        st = tg_gemm(pa, pb, pc, M, N, K, lda, ldb, ldc, code, s)
    if st != TG_SUCCESS:
        raise TgError(st, "tg_gemm")
    return out


def workspace_bytes(a, b, out_dtype=None, bias=None):
    """Workspace bytes tg_gemm_ws's fastest plan uses for these operands (0:
    none).  Touches no device state."""
    import torch
    M, K = a.shape
    N = b.shape[1]
    pa, lda, op_a = _operand(a, "A")
    pb, ldb, op_b = _operand(b, "B")
    code = _dtype_code(out_dtype or torch.float16)
    # the stand-in C address only has to be aligned: the plan does not read it
    st, _, _, _, used = tg_select_plan(pa, pb, bias.data_ptr() if bias is not None else None,
                                       256, M, N, K, lda, ldb, N, code, op_a=op_a, op_b=op_b)
    if st != TG_SUCCESS:
        raise TgError(st, "tg_select_plan")
    return used


def gemm_bias_relu(a, b, bias, out=None, out_dtype=None, config=None, stream=None,
                   workspace=None, splits=0):
    return gemm(a, b, out=out, out_dtype=out_dtype, bias=bias, config=config, stream=stream,
                workspace=workspace, splits=splits)


def attention(q, k, v, causal=False, scale=None, out=None, return_lse=False, stream=None):
    """Fused attention forward with libtg: q (B, H, Lq, d), k and v (B, Hkv, Lk, d)
    float16 views on the current device whose last dimension is contiguous
    (any strides otherwise, e.g. a (B, L, H, d) tensor permuted to (B, H, L, d));
    returns out (B, H, Lq, d) float16 and, with return_lse, lse (B, H, Lq)
    float32.  scale defaults to 1/sqrt(d)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.float16 or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("%s must be a 4-D float16 tensor with a contiguous last dim" % n)
    B, H, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if tuple(v.shape) != (Bk, Hkv, Lk, dk) or Bk != B or dk != d:
        raise ValueError("shapes do not match: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                                  tuple(v.shape)))
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=torch.float16, device=q.device)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device) if return_lse else None
    scale = (1.0 / d ** 0.5) if scale is None else scale
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    st = tg_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None, B, H, Hkv, Lq, Lk, d,
                          q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3],
                          scale, causal, s)
    if st != TG_SUCCESS:
        raise TgError(st, "tg_attention_fwd")
    return (out, lse) if return_lse else out
