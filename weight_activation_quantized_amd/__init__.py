"""Quantized linear layers for AMD Instinct MI355X (gfx950): W4A16 and W8A8_INT8.

A thin binding over the C ABI of ``libmq.so`` (declared in ``include/mq.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, allocates outputs with ``torch.empty`` and passes
device pointers and the current HIP stream. There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.

Entry points (same names as the C ABI, without the ``mq_`` prefix):

    quant_per_token_int8(x)                          -> (xq, s_tok); x fp16 or bf16
    w8a8_scaled_mm(xq, s_tok, wq, s_ch)              -> y  (fp16, or bf16 with out_dtype)
    w8a8_mm_i32(xq, wq)                              -> acc (int32)
    w4a16_gemm(x, qweight, scales, qzeros, group)    -> y  (x's dtype: fp16 or bf16); K split on small grids
    w4a16_gemm_workspace_bytes(M, N, K, group)       -> int
    w4a16_gemv(x, qweight, scales, qzeros, group)    -> y  (x's dtype), M <= 64
    w4a16_gemv_workspace_bytes(M, N, K, group)       -> int
    w4a16_block_weights(qweight)                     -> qweight_blocked (decode layout, once per matrix)
    w4a16_gemv_blocked(x, qweight_blocked, scales, qzeros, group) -> y (x's dtype), M <= 64
    w4a16_gemv_blocked_workspace_bytes(M, N, K, group) -> int

    (W4A16 group: 32, 64 or 128 rows per scale / zero point, or -1 for one
    per output column over all of K: scales [1, N], qzeros [1, N/8].)

    kv_quant(x, bits)                                -> (codes, params) per (token, head) row

    int4_reorder(words, order)                       -> words in the library's field order
    int4_transpose(words, order)                     -> [B, A/8] from a 4-bit [A, B] packed along B
    u16_transpose(scales)                            -> [B, A] (fp16 scales [N, K/G] -> [K/G, N])

and two compositions used by a model's linear layer:

    w4a16_linear(x, qweight, scales, qzeros, group)  GEMV for M <= 64 (decode layout if qweight_blocked
                                                     is given), else GEMM
    w8a8_linear(x, wq, s_ch)                         quantize x (fp16 or bf16) per token, then scaled GEMM
                                                     (one fused kernel for 1-4 tokens, see mq.h; a workspace otherwise)
    w8a8_linear_noalloc(x, wq, s_ch)                 the same (fp16) with the library's own scratch: no allocation
"""

import ctypes
import os

__all__ = [
    "MqError", "library", "LIB_PATH",
    "quant_per_token_int8", "w8a8_scaled_mm", "w8a8_mm_i32",
    "w4a16_gemm", "w4a16_gemv", "w4a16_gemv_workspace_bytes",
    "w4a16_linear", "w8a8_linear", "GEMV_MAX_M",
    "w4a16_block_weights", "w4a16_gemv_blocked", "w4a16_gemv_blocked_workspace_bytes",
    "w8a8_linear_workspace_bytes", "w4a16_gemm_workspace_bytes", "kv_quant",
    "AWQ_FIELD_ORDER", "int4_reorder", "int4_transpose", "u16_transpose",
    "w8a8_linear_noalloc", "NOALLOC_SCRATCH_BYTES",
]

# The in-tree build; MQ_LIBRARY names another build of the same library (for
# example the host-sanitized one that the CPU tests load).
LIB_PATH = os.environ.get("MQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmq.so")
GEMV_MAX_M = 64

STATUS_NAMES = {
    0: "MQ_OK", 1: "MQ_ERR_NULL", 2: "MQ_ERR_SHAPE", 3: "MQ_ERR_ALIGN", 4: "MQ_ERR_UNSUPPORTED",
    5: "MQ_ERR_WORKSPACE", 6: "MQ_ERR_ALIAS", 7: "MQ_ERR_HIP",
}


class MqError(RuntimeError):
    """A libmq call returned a non-OK status."""

    def __init__(self, status, detail):
        self.status = int(status)
        self.status_name = STATUS_NAMES.get(self.status, f"status {status}")
        self.detail = detail
        super().__init__(f"{self.status_name}: {detail}")


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_PROTOTYPES = {
    "mq_abi_version": (ctypes.c_int, []),
    "mq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mq_last_error": (ctypes.c_char_p, []),
    "mq_quant_per_token_int8": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "mq_w8a8_scaled_mm": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "mq_w8a8_mm_i32": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "mq_w4a16_gemm_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "mq_w4a16_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_w4a16_gemv_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "mq_w4a16_gemv": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_w4a16_block_weights": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "mq_w8a8_linear_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "mq_kv_quant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_int32, _P]),
    "mq_kv_quant_bf16": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_int32, _P]),
    "mq_w8a8_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_quant_per_token_int8_bf16": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "mq_w8a8_scaled_mm_bf16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "mq_w8a8_linear_bf16": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_w8a8_linear_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "mq_int4_reorder": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "mq_int4_transpose": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "mq_u16_transpose": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "mq_w4a16_gemv_blocked_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "mq_w4a16_gemv_blocked": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t,
                                             _P]),
    "mq_w4a16_gemm_bf16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_w4a16_gemv_bf16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "mq_w4a16_gemv_blocked_bf16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P,
                                                  ctypes.c_size_t, _P]),
}


def library():
    """The loaded ``libmq.so`` (ctypes) with prototypes set. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m weight_activation_quantized_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        detail = library().mq_last_error()
        raise MqError(status, detail.decode() if detail else "")


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_tensor(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_of(t, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _out(out, shape, dtype, like, name):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _dev_tensor(out, name, dtype, len(shape))
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(out.shape)})")
    return out


def _half_dtype(t, name):
    """fp16 or bf16: the activation dtypes the entry points take."""
    torch = _torch()
    if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16:
        return torch.bfloat16
    if isinstance(t, torch.Tensor) and t.dtype == torch.float16:
        return torch.float16
    raise TypeError(f"{name} must be a float16 or bfloat16 tensor")


def quant_per_token_int8(x, out=None, s_out=None, stream=None):
    """Per-token int8 quantization of fp16 or bf16 x[M, K] -> (xq int8 [M, K], s_tok fp32 [M])."""
    torch = _torch()
    dt = _half_dtype(x, "x")
    _dev_tensor(x, "x", dt, 2)
    M, K = x.shape
    xq = _out(out, (M, K), torch.int8, x, "out")
    s = _out(s_out, (M,), torch.float32, x, "s_out")
    fn = library().mq_quant_per_token_int8_bf16 if dt == torch.bfloat16 else library().mq_quant_per_token_int8
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), xq.data_ptr(), s.data_ptr(), M, K, _stream_of(x, stream)))
    return xq, s


def w8a8_scaled_mm(xq, s_tok, wq, s_ch, out=None, stream=None, out_dtype=None):
    """y[M, N] = (xq[M, K] . wq[N, K]^T) * s_tok[:, None] * s_ch[None, :] in
    fp16 (default) or bf16 (``out_dtype=torch.bfloat16``, or a bf16 ``out``)."""
    torch = _torch()
    _dev_tensor(xq, "xq", torch.int8, 2)
    _dev_tensor(wq, "wq", torch.int8, 2)
    _dev_tensor(s_tok, "s_tok", torch.float32, 1)
    _dev_tensor(s_ch, "s_ch", torch.float32, 1)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or s_tok.shape[0] != M or s_ch.shape[0] != N:
        raise ValueError("shape mismatch between xq, s_tok, wq and s_ch")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float16
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("out_dtype must be float16 or bfloat16")
    y = _out(out, (M, N), out_dtype, xq, "out")
    fn = library().mq_w8a8_scaled_mm_bf16 if out_dtype == torch.bfloat16 else library().mq_w8a8_scaled_mm
    with torch.cuda.device(xq.device):
        _check(fn(xq.data_ptr(), s_tok.data_ptr(), wq.data_ptr(), s_ch.data_ptr(), y.data_ptr(), M, N, K,
                  _stream_of(xq, stream)))
    return y


def w8a8_mm_i32(xq, wq, out=None, stream=None):
    """Debug: raw int32 accumulator acc[M, N] = xq[M, K] . wq[N, K]^T."""
    torch = _torch()
    _dev_tensor(xq, "xq", torch.int8, 2)
    _dev_tensor(wq, "wq", torch.int8, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq must share K")
    acc = _out(out, (M, N), torch.int32, xq, "out")
    with torch.cuda.device(xq.device):
        _check(library().mq_w8a8_mm_i32(xq.data_ptr(), wq.data_ptr(), acc.data_ptr(), M, N, K,
                                        _stream_of(xq, stream)))
    return acc


def _w4a16_shapes(x, qweight, scales, qzeros, group):
    torch = _torch()
    _dev_tensor(x, "x", _half_dtype(x, "x"), 2)
    _dev_tensor(qweight, "qweight", torch.int32, 2)
    _dev_tensor(scales, "scales", torch.float16, 2)
    _dev_tensor(qzeros, "qzeros", torch.int32, 2)
    M, K = x.shape
    N = qweight.shape[1] * 8
    if qweight.shape[0] != K:
        raise ValueError("qweight must be [K, N/8]")
    G = K if group == -1 else group
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of the group size")
    if tuple(scales.shape) != (K // G, N) or tuple(qzeros.shape) != (K // G, N // 8):
        raise ValueError("scales must be [K/G, N] and qzeros [K/G, N/8]")
    return M, N, K


def w4a16_gemm_workspace_bytes(M, N, K, group=128):
    """Workspace bytes that let ``w4a16_gemm`` split K on small tile grids (0: never splits)."""
    return int(library().mq_w4a16_gemm_workspace_bytes(M, N, K, group))


def w4a16_gemm(x, qweight, scales, qzeros, group=128, out=None, workspace=None, stream=None):
    """W4A16 GEMM: y[M, N] = x[M, K] . dequant(qweight, scales, qzeros), x and y
    fp16 or bf16 (the weight rounded once to x's dtype).

    ``workspace``: a uint8 GPU tensor of at least ``w4a16_gemm_workspace_bytes``
    bytes (allocated if None and the shape splits K); ``False`` never splits.
    """
    torch = _torch()
    M, N, K = _w4a16_shapes(x, qweight, scales, qzeros, group)
    y = _out(out, (M, N), x.dtype, x, "out")
    if workspace is False:
        workspace = None
    elif workspace is None:
        need = w4a16_gemm_workspace_bytes(M, N, K, group) if M else 0
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = library().mq_w4a16_gemm_bf16 if x.dtype == torch.bfloat16 else library().mq_w4a16_gemm
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(),
                  y.data_ptr(), M, N, K, group, ws_ptr, ws_bytes, _stream_of(x, stream)))
    return y


def w4a16_gemv_workspace_bytes(M, N, K, group=128):
    """Workspace bytes ``w4a16_gemv`` needs (0 if none)."""
    return int(library().mq_w4a16_gemv_workspace_bytes(M, N, K, group))


def w4a16_gemv(x, qweight, scales, qzeros, group=128, out=None, workspace=None, stream=None):
    """W4A16 GEMV for decode (M <= 64); x and y fp16 or bf16.

    ``workspace``: a uint8 GPU tensor of at least ``w4a16_gemv_workspace_bytes``
    bytes (allocated if None); its contents do not matter. Calls sharing a
    workspace must be ordered on the GPU (for example, the same stream).
    """
    torch = _torch()
    M, N, K = _w4a16_shapes(x, qweight, scales, qzeros, group)
    y = _out(out, (M, N), x.dtype, x, "out")
    need = w4a16_gemv_workspace_bytes(M, N, K, group)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = library().mq_w4a16_gemv_bf16 if x.dtype == torch.bfloat16 else library().mq_w4a16_gemv
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(),
                  y.data_ptr(), M, N, K, group, ws_ptr, ws_bytes, _stream_of(x, stream)))
    return y


def w4a16_block_weights(qweight, out=None, stream=None):
    """Reorder qweight [K, N/8] into the column-blocked decode layout (N % 32 == 0).

    Returns an int32 tensor of shape [K/64, 8*N]: row P holds the bytes of
    rows 64P .. 64P+63 of every 32-output strip in the order the blocked GEMV
    streams them (see ``mq.h``). Run once per weight matrix.
    """
    torch = _torch()
    _dev_tensor(qweight, "qweight", torch.int32, 2)
    K, NP = qweight.shape
    N = NP * 8
    if N % 32:
        raise ValueError("the blocked layout needs N % 32 == 0")
    if K % 64:
        raise ValueError("the blocked layout needs K % 128 == 0")
    qb = _out(out, (K // 64, 8 * N), torch.int32, qweight, "out")
    with torch.cuda.device(qweight.device):
        _check(library().mq_w4a16_block_weights(qweight.data_ptr(), qb.data_ptr(), N, K,
                                                _stream_of(qweight, stream)))
    return qb


def w4a16_gemv_blocked_workspace_bytes(M, N, K, group=128):
    """Workspace bytes ``w4a16_gemv_blocked`` needs (0 if none)."""
    return int(library().mq_w4a16_gemv_blocked_workspace_bytes(M, N, K, group))


def w4a16_gemv_blocked(x, qweight_blocked, scales, qzeros, group=128, out=None, workspace=None, stream=None):
    """W4A16 GEMV for decode (M <= 64) on weights from ``w4a16_block_weights``; x and y fp16 or bf16."""
    torch = _torch()
    _dev_tensor(x, "x", _half_dtype(x, "x"), 2)
    _dev_tensor(qweight_blocked, "qweight_blocked", torch.int32, 2)
    _dev_tensor(scales, "scales", torch.float16, 2)
    _dev_tensor(qzeros, "qzeros", torch.int32, 2)
    M, K = x.shape
    N = scales.shape[1]
    G = K if group == -1 else group
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of the group size")
    if tuple(qweight_blocked.shape) != (K // 64, 8 * N) or N % 32:
        raise ValueError("qweight_blocked must be [K/64, 8*N] (from w4a16_block_weights)")
    if tuple(scales.shape) != (K // G, N) or tuple(qzeros.shape) != (K // G, N // 8):
        raise ValueError("scales must be [K/G, N] and qzeros [K/G, N/8]")
    y = _out(out, (M, N), x.dtype, x, "out")
    need = w4a16_gemv_blocked_workspace_bytes(M, N, K, group)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = library().mq_w4a16_gemv_blocked_bf16 if x.dtype == torch.bfloat16 else library().mq_w4a16_gemv_blocked
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), qweight_blocked.data_ptr(), scales.data_ptr(), qzeros.data_ptr(), y.data_ptr(), M, N,
                  K, group, ws_ptr, ws_bytes, _stream_of(x, stream)))
    return y


def w4a16_linear(x, qweight, scales, qzeros, group=128, out=None, stream=None, qweight_blocked=None):
    """W4A16 linear layer: a GEMV for M <= 64 (decode), the GEMM otherwise
    (prefill). With ``qweight_blocked`` (``w4a16_block_weights(qweight)``,
    converted once when the layer is loaded) decode runs the GEMV on the
    decode layout, the faster one; without it, the GEMV on [K, N/8]."""
    if x.shape[0] <= GEMV_MAX_M:
        if qweight_blocked is not None:
            return w4a16_gemv_blocked(x, qweight_blocked, scales, qzeros, group, out=out, stream=stream)
        return w4a16_gemv(x, qweight, scales, qzeros, group, out=out, stream=stream)
    return w4a16_gemm(x, qweight, scales, qzeros, group, out=out, stream=stream)


def w8a8_linear_workspace_bytes(M, K):
    """Workspace bytes ``w8a8_linear`` needs for the two-kernel path (the one-token fused path
    leaves it unused)."""
    return int(library().mq_w8a8_linear_workspace_bytes(M, K))


def w8a8_linear(x, wq, s_ch, out=None, workspace=None, stream=None):
    """W8A8_INT8 linear layer from fp16 or bf16 x (y in x's dtype): per-token
    int8 quantization, then the scaled int8 GEMM (one fused kernel for one
    to four tokens, see mq.h). Bit-identical to ``w8a8_scaled_mm(*quant_per_token_int8(x), wq,
    s_ch, out_dtype=x.dtype)``."""
    torch = _torch()
    dt = _half_dtype(x, "x")
    _dev_tensor(x, "x", dt, 2)
    _dev_tensor(wq, "wq", torch.int8, 2)
    _dev_tensor(s_ch, "s_ch", torch.float32, 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or s_ch.shape[0] != N:
        raise ValueError("wq must be [N, K] and s_ch [N]")
    y = _out(out, (M, N), dt, x, "out")
    need = w8a8_linear_workspace_bytes(M, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(x.device):
        fn = library().mq_w8a8_linear_bf16 if dt == torch.bfloat16 else library().mq_w8a8_linear
        _check(fn(x.data_ptr(), wq.data_ptr(), s_ch.data_ptr(), y.data_ptr(), M, N, K, ws_ptr, ws_bytes,
                  _stream_of(x, stream)))
    return y


# Bytes of the library-owned scratch behind ``w8a8_linear_noalloc`` (per GPU).
NOALLOC_SCRATCH_BYTES = 33816576


def w8a8_linear_noalloc(x, wq, s_ch, out=None, stream=None):
    """``w8a8_linear`` for fp16 x without a workspace: the library keeps the
    codes and per-token scales in its own scratch array on each GPU (for
    callers that cannot allocate, e.g. under graph capture). Needs
    ``w8a8_linear_workspace_bytes(M, K) <= NOALLOC_SCRATCH_BYTES``. Calls that
    may overlap in time on one GPU share that scratch and must be serialized
    by the caller (one stream suffices). With ``out`` given, allocates nothing."""
    torch = _torch()
    _dev_tensor(x, "x", torch.float16, 2)
    _dev_tensor(wq, "wq", torch.int8, 2)
    _dev_tensor(s_ch, "s_ch", torch.float32, 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or s_ch.shape[0] != N:
        raise ValueError("wq must be [N, K] and s_ch [N]")
    y = _out(out, (M, N), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        _check(library().mq_w8a8_linear_noalloc(x.data_ptr(), wq.data_ptr(), s_ch.data_ptr(), y.data_ptr(), M, N, K,
                                                _stream_of(x, stream)))
    return y


def kv_quant(x, bits=8, codes=None, params=None, stream=None):
    """Online KV-cache quantization per (token, head) row: x [..., head_dim] fp16
    or bf16 -> (codes uint8 [..., head_dim] (8 bits) or [..., head_dim/2] (4
    bits, two per byte, element 2i low), params fp32 [..., 2] = (scale, min))."""
    torch = _torch()
    if (not isinstance(x, torch.Tensor) or x.dtype not in (torch.float16, torch.bfloat16)
            or x.device.type != "cuda"):
        raise TypeError("x must be a float16 or bfloat16 GPU tensor")
    if not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be contiguous with at least one dimension")
    D = x.shape[-1]
    lead = tuple(x.shape[:-1])
    rows = x.numel() // D if D else 0
    cshape = lead + ((D,) if bits == 8 else (D // 2,))
    codes = _out(codes, cshape, torch.uint8, x, "codes")
    params = _out(params, lead + (2,), torch.float32, x, "params")
    with torch.cuda.device(x.device):
        fn = library().mq_kv_quant_bf16 if x.dtype == torch.bfloat16 else library().mq_kv_quant
        _check(fn(x.data_ptr(), codes.data_ptr(), params.data_ptr(), rows, D, bits, _stream_of(x, stream)))
    return codes, params


# Field order of AWQ-style checkpoint words: field j holds element
# 8c + AWQ_FIELD_ORDER[j] of the row's span (a reading; the pages name the
# format but not its bits).
AWQ_FIELD_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def _order_arg(order):
    if order is None:
        return None
    vals = [int(v) for v in order]
    if len(vals) != 8:
        raise ValueError("order must have 8 entries")
    return (ctypes.c_uint8 * 8)(*[v & 0xFF for v in vals])


def int4_reorder(src, order, out=None, stream=None):
    """int32 words of 4-bit values in another field order (field j holding
    element 8c + order[j]) -> the library's order, same shape (e.g. an
    AWQ-style qweight [K, N/8] or qzeros [K/G, N/8])."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or src.dtype != torch.int32 or src.device.type != "cuda":
        raise TypeError("src must be an int32 GPU tensor")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    out = _out(out, tuple(src.shape), torch.int32, src, "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    with torch.cuda.device(src.device):
        _check(library().mq_int4_reorder(src.data_ptr(), out.data_ptr(), src.numel(), _order_arg(order),
                                         _stream_of(src, stream)))
    return out


def int4_transpose(src, order=None, out=None, stream=None):
    """int32 [A, B/8] (a 4-bit [A, B] matrix packed along B in `order`) ->
    int32 [B, A/8], its transpose packed along A in the library's order
    (e.g. weights stored [N, K/8] -> qweight [K, N/8])."""
    torch = _torch()
    _dev_tensor(src, "src", torch.int32, 2)
    A, B = src.shape[0], src.shape[1] * 8
    if A % 8:
        raise ValueError("the row count of src must be a multiple of 8")
    out = _out(out, (B, A // 8), torch.int32, src, "out")
    with torch.cuda.device(src.device):
        _check(library().mq_int4_transpose(src.data_ptr(), out.data_ptr(), A, B, _order_arg(order),
                                           _stream_of(src, stream)))
    return out


def u16_transpose(src, out=None, stream=None):
    """[A, B] 16-bit tensor (fp16 scales) -> [B, A] (e.g. scales stored
    [N, K/G] -> [K/G, N])."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or src.dtype not in (torch.float16, torch.int16, torch.bfloat16):
        raise TypeError("src must be a 16-bit GPU tensor")
    _dev_tensor(src, "src", src.dtype, 2)
    A, B = src.shape
    out = _out(out, (B, A), src.dtype, src, "out")
    with torch.cuda.device(src.device):
        _check(library().mq_u16_transpose(src.data_ptr(), out.data_ptr(), A, B, _stream_of(src, stream)))
    return out
