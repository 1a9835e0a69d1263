"""Thin ctypes binding of the C ABI in ``include/migemm.h``.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmigemm.so``.  If the library is not built, every call raises
instead of falling back to anything else.

Tensor-level functions take torch CUDA tensors (torch is used for device
memory and streams only) and check what the C ABI cannot see: dtype, device,
and the layout the C contract fixes (column-major GEMM operands given as
strides (1, rows); contiguous row-major GEMV operands).
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmigemm.so")

ERRORS = {0: "ok", -1: "negative dimension", -2: "null pointer with a non-zero extent",
          -3: "output overlaps an input", -4: "pointer or size not aligned as the entry point requires",
          -5: "configuration not offered", -6: "dimension beyond the supported range"}

F16, BF16 = 0, 1
F8E4M3, F8E5M2, I8 = 2, 3, 4          # 8-bit inputs of gemm_tn_q_ex


class MigemmError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        msg = ERRORS.get(code, "HIP error %d" % code if code > 0 else "error %d" % code)
        super().__init__("%s: %s (code %d)" % (where, msg, code))


class Plan(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("waves", ctypes.c_int), ("group_m", ctypes.c_int), ("xcd_remap", ctypes.c_int),
                ("vec_a", ctypes.c_int), ("vec_b", ctypes.c_int), ("grid", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int), ("tile", ctypes.c_int), ("a_kmajor", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None

# exported symbol -> (restype, argtypes); also the list the export test checks
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
SIGNATURES = {
    "gemm_f16": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "gemm_bf16": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "gemv_bf16": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "gemm_ex": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gemm_tn_f16": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "gemm_tn_bf16": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "gemm_tn_ex": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gemv_bf16_ex": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "gemm_tn_fp8_e4m3": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P]),
    "gemm_tn_fp8_e5m2": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P]),
    "gemm_tn_i8": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P]),
    "gemm_tn_q_ex": (_I, [_I, _P, _P, _P, _I, _I, _I, ctypes.c_float, _I, _I, _I, _P]),
    "gemm_splitk_ex": (_I, [_I, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P]),
    "migemm_splitk_splits": (_I, [_I, _I, _I, _I, _I]),
    "migemm_splitk_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "migemm_tile_coord": (_I, [_I64, _I64, _I64, _I64, _I64,
                               ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "migemm_gemm_plan_for": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(Plan)]),
    "migemm_gemm_tn_plan_for": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(Plan)]),
    "migemm_gemv_plan_for": (_I, [_P, _P, _P, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "migemm_strerror": (ctypes.c_char_p, [_I]),
    "migemm_abi_version": (_I, []),
    "migemm_hbm_read": (_I, [_P, ctypes.c_size_t, _P, _P]),
    "attention_decode_bf16": (_I, [_P, _P, _P, _P, _P, _P] + [_I] * 7 +
                              [ctypes.c_float, _I, _I, _P, ctypes.c_size_t, _P]),
    "attention_decode_bf16_noalloc": (_I, [_P, _P, _P, _P, _P, _P] + [_I] * 7 +
                                      [ctypes.c_float, _I, _I, _P]),
    "migemm_attention_segments": (_I, [_I, _I, _I, _I]),
    "migemm_attention_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "migemm_hbm_read_sink_words": (_I, []),
    "migemm_clock_probe": (_I, [_P, _I, _I, _P]),
    "migemm_gemm_clocked": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
}


def lib():
    """Load libmigemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmigemm.so is not built (run __graft_entry__.build() or "
                               "python bf16_gemm_decode_amd/build.py); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(code, where):
    if code != 0:
        raise MigemmError(code, where)


# ---- raw pointer level (device addresses as ints) ----------------------------

def gemm_f16_ptr(A, B, C, M, N, K, stream=0):
    return lib().gemm_f16(A, B, C, M, N, K, stream or None)


def gemm_bf16_ptr(A, B, C, M, N, K, stream=0):
    return lib().gemm_bf16(A, B, C, M, N, K, stream or None)


def gemm_ex_ptr(dtype, A, B, C, M, N, K, tile=0, group_m=0, xcd_remap=1, stream=0):
    return lib().gemm_ex(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, stream or None)


def gemm_tn_ex_ptr(dtype, At, B, C, M, N, K, tile=0, group_m=0, xcd_remap=1, stream=0):
    return lib().gemm_tn_ex(dtype, At, B, C, M, N, K, tile, group_m, xcd_remap, stream or None)


def gemv_bf16_ptr(W, X, Y, M, K, n, stream=0):
    return lib().gemv_bf16(W, X, Y, M, K, n, stream or None)


def gemv_bf16_ex_ptr(W, X, Y, M, K, n, rows_per_block=0, stream=0):
    return lib().gemv_bf16_ex(W, X, Y, M, K, n, rows_per_block, stream or None)


def tile_coord(wg, num_pid_m, num_pid_n, group_m, num_xcd):
    pm, pn = _I64(), _I64()
    _check(lib().migemm_tile_coord(wg, num_pid_m, num_pid_n, group_m, num_xcd,
                                   ctypes.byref(pm), ctypes.byref(pn)), "migemm_tile_coord")
    return pm.value, pn.value


def gemm_plan(dtype, A, B, C, M, N, K, tile=0, group_m=0, xcd_remap=1, a_kmajor=False):
    p = Plan()
    fn = lib().migemm_gemm_tn_plan_for if a_kmajor else lib().migemm_gemm_plan_for
    code = fn(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, ctypes.byref(p))
    return code, p.as_dict()


def gemv_route(W, X, Y, M, K, n, rows_per_block=0):
    """(code, route) of gemv_bf16_ex's checks and kernel choice: route 0 no
    launch, 1 vector kernel, 14 4x4x4 MFMA kernel, 15 batch kernel, 18
    row-balanced batch kernel, 19 wide row-balanced kernel, 9 gemm_tn."""
    r = _I()
    code = lib().migemm_gemv_plan_for(W, X, Y, M, K, n, rows_per_block, ctypes.byref(r))
    return code, r.value


# ---- torch tensor level --------------------------------------------------------

def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _colmajor_ok(t, rows, cols):
    """Element (i, j) at offset i + j*rows (strides of size-1 dims ignored)."""
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        return False
    if t.numel() == 0:
        return True
    s0, s1 = t.stride()
    return (s0 == 1 or rows == 1) and (s1 == rows or cols == 1)


def _require(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def gemm(A, B, C=None, stream=None, tile=0, group_m=0, xcd_remap=1):
    """C = A @ B for column-major 2-D tensors (strides (1, rows)).  Dtype
    float16 -> gemm_f16, bfloat16 -> gemm_bf16.  C is allocated column-major
    when not given.  Launches on `stream` (default: torch's current stream)."""
    import torch
    dt = A.dtype
    if dt not in (torch.float16, torch.bfloat16):
        raise TypeError("A must be float16 or bfloat16")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    _require(A, dt, "A")
    _require(B, dt, "B")
    if C is None:
        C = torch.empty((N, M), dtype=dt, device=A.device).t()
    _require(C, dt, "C")
    for t, r, c, nm in ((A, M, K, "A"), (B, K, N, "B"), (C, M, N, "C")):
        if not _colmajor_ok(t, r, c):
            raise ValueError("%s must be column-major %dx%d (strides (1, %d))" % (nm, r, c, r))
    code = lib().gemm_ex(F16 if dt == torch.float16 else BF16, A.data_ptr(), B.data_ptr(),
                         C.data_ptr(), M, N, K, tile, group_m, xcd_remap, _stream_handle(stream))
    _check(code, "gemm")
    return C


def gemv(W, X, Y=None, stream=None, rows_per_block=0):
    """Y = X @ W^T, bfloat16, row-major contiguous W [M,K], X [n,K], Y [n,M]."""
    import torch
    _require(W, torch.bfloat16, "W")
    _require(X, torch.bfloat16, "X")
    M, K = W.shape
    n, K2 = X.shape
    if K2 != K:
        raise ValueError("K differs: %d vs %d" % (K, K2))
    if not (W.is_contiguous() and X.is_contiguous()):
        raise ValueError("W and X must be contiguous row-major")
    if Y is None:
        Y = torch.empty((n, M), dtype=torch.bfloat16, device=W.device)
    _require(Y, torch.bfloat16, "Y")
    if tuple(Y.shape) != (n, M) or not Y.is_contiguous():
        raise ValueError("Y must be contiguous row-major %dx%d" % (n, M))
    code = lib().gemv_bf16_ex(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, K, n,
                              rows_per_block, _stream_handle(stream))
    _check(code, "gemv")
    return Y


def hbm_read(buf, sink, stream=None):
    """Streaming-read probe over a CUDA tensor `buf` (bytes = buf's size)."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().migemm_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(),
                                 _stream_handle(stream)), "hbm_read")


def hbm_read_sink_words():
    return lib().migemm_hbm_read_sink_words()


def attention_decode(Q, Kc, Vc, block_table, seq_lens, Out, Hkv, block_size, scale,
                     max_seq_len, num_segments=0, workspace=None, stream=None):
    """Tensor wrapper of attention_decode_bf16.  Q, Out: [B, Hq, D] bfloat16
    CUDA tensors; Kc, Vc: [num_blocks, block_size, Hkv, D] bfloat16;
    block_table: [B, max_blocks] int32; seq_lens: [B] int32.  Allocates the
    workspace when none is given (a uint8 CUDA tensor of the needed size)."""
    import torch
    B, Hq, D = Q.shape
    num_blocks = Kc.shape[0]
    max_blocks = block_table.shape[1]
    for t in (Q, Kc, Vc, Out):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("Q, Kc, Vc, Out must be contiguous bfloat16 CUDA tensors")
    for t in (block_table, seq_lens):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("block_table and seq_lens must be contiguous int32 CUDA tensors")
    S = num_segments or lib().migemm_attention_segments(B, Hq, Hkv, max_seq_len)
    need = lib().migemm_attention_workspace_bytes(B, Hq, D, S)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
    _check(lib().attention_decode_bf16(Q.data_ptr(), Kc.data_ptr(), Vc.data_ptr(),
                                       block_table.data_ptr(), seq_lens.data_ptr(), Out.data_ptr(),
                                       B, Hq, Hkv, D, block_size, max_blocks, num_blocks, scale,
                                       max_seq_len, S, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream)), "attention_decode_bf16")
    return Out
