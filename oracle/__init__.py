"""CPU oracle for the column-major GEMM, the decode GEMV and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never imports, links or calls it, and it shares no code with the
HIP path.  The arithmetic lives in ``oracle.c`` (FP64 triple loop, exact
16-bit decode, single RNE rounding); this module only marshals numpy arrays
and implements the acceptance rule.

Decode attention (DCU decode page, sections 6.1 and 6.3) uses the same
rule with S_abs = sum_l p_l |v_ld| and a relative factor derived per output
from L, D and the scores' magnitude (``attention_rel``).

Acceptance rule (per checked element, C_ref the oracle's rounded result):
    |C_gpu - C_ref| <= 2e-3 * S_abs + ulp_out(C_ref)
with S_abs = sum_k |a_mk| |b_kn| and ulp_out the spacing of the output format
at |C_ref|; non-finite values must agree in class (NaN, or Inf of one sign).
The 2e-3 factor is at least twice Higham's gamma_K = K u / (1 - K u),
u = 2^-24, for every K used here (gamma_16384 = 9.77e-4), so any FP32
summation order passes; the one ulp absorbs the GPU's second rounding.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FP16 = 0
BF16 = 1
_FMT = {"f16": FP16, "fp16": FP16, "float16": FP16,
        "bf16": BF16, "bfloat16": BF16}

_lib = None


def fmt_id(fmt) -> int:
    return fmt if isinstance(fmt, int) else _FMT[fmt]


def lib():
    """Load liboracle.so, building it with gcc only when none is built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.oracle_decode.restype = ctypes.c_double
        L.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint16]
        L.oracle_encode.restype = ctypes.c_uint16
        L.oracle_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        L.oracle_decode_array.argtypes = [ctypes.c_int, u16p, f64p, ctypes.c_int64]
        L.oracle_encode_array.argtypes = [ctypes.c_int, f64p, u16p, ctypes.c_int64]
        L.oracle_gemm.restype = ctypes.c_int64
        L.oracle_gemm.argtypes = [ctypes.c_int, u16p, u16p, u16p, f64p, f64p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_gemm_sampled.restype = ctypes.c_int64
        L.oracle_gemm_sampled.argtypes = [ctypes.c_int, u16p, u16p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, i64p,
                                          ctypes.c_int64, u16p, f64p, f64p]
        L.oracle_gemv.restype = ctypes.c_int64
        L.oracle_gemv.argtypes = [ctypes.c_int, u16p, u16p, u16p, f64p, f64p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_grouped_tile.restype = None
        L.oracle_grouped_tile.argtypes = [ctypes.c_int64] * 4 + [i64p, i64p]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_grouped_order.restype = None
        L.oracle_grouped_order.argtypes = [ctypes.c_int64] * 3 + [i64p, i64p]
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.oracle_attention.restype = ctypes.c_int64
        L.oracle_attention.argtypes = [ctypes.c_int, u16p, u16p, u16p, i32p, i32p] + \
            [ctypes.c_int] * 6 + [ctypes.c_double, u16p, f64p, f64p, f64p]
        L.oracle_attention_segmented.restype = None
        L.oracle_attention_segmented.argtypes = [ctypes.c_int, u16p, u16p, u16p, i32p, i32p] + \
            [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int, u16p, f64p]
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.oracle_decode8.restype = ctypes.c_double
        L.oracle_decode8.argtypes = [ctypes.c_int, ctypes.c_uint8]
        L.oracle_decode8_array.argtypes = [ctypes.c_int, u8p, f64p, ctypes.c_int64]
        L.oracle_gemm_tn_q.restype = ctypes.c_int64
        L.oracle_gemm_tn_q.argtypes = [ctypes.c_int, u8p, u8p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_float, i64p, ctypes.c_int64,
                                       u16p, f64p, f64p]
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected raw 16-bit patterns as uint16, got %s" % a.dtype)
    return a


def decode(bits, fmt) -> np.ndarray:
    """Exact float64 values of an array of 16-bit patterns."""
    b = _u16(bits)
    out = np.empty(b.shape, np.float64)
    lib().oracle_decode_array(fmt_id(fmt), _p(b, ctypes.c_uint16),
                              _p(out, ctypes.c_double), b.size)
    return out


def encode(values, fmt) -> np.ndarray:
    """Round float64 values to 16-bit patterns (nearest-even, one step)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_encode_array(fmt_id(fmt), _p(v, ctypes.c_double),
                              _p(out, ctypes.c_uint16), v.size)
    return out


class GemmResult:
    """Oracle output: ``bits`` (rounded), ``exact`` (float64 sum), ``sabs``
    (sum of |a||b|), ``macs`` (multiply-adds performed)."""

    def __init__(self, bits, exact, sabs, macs):
        self.bits, self.exact, self.sabs, self.macs = bits, exact, sabs, macs


def gemm(A, B, M, N, K, fmt) -> GemmResult:
    """C = A x B, column-major, every entry.  A, B: flat uint16 patterns,
    A(m,k) = A[m + k*M], B(k,n) = B[k + n*K].  Results are flat, length M*N,
    C(m,n) at index m + n*M."""
    A, B = _u16(A).ravel(), _u16(B).ravel()
    assert A.size == M * K and B.size == K * N
    C = np.empty(M * N, np.uint16)
    Cx = np.empty(M * N, np.float64)
    S = np.empty(M * N, np.float64)
    macs = lib().oracle_gemm(fmt_id(fmt), _p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                             _p(C, ctypes.c_uint16), _p(Cx, ctypes.c_double),
                             _p(S, ctypes.c_double), M, N, K)
    return GemmResult(C, Cx, S, macs)


def gemm_sampled(A, B, M, N, K, idx, fmt) -> GemmResult:
    """The same quantities at flat output indices idx (m + n*M)."""
    A, B = _u16(A).ravel(), _u16(B).ravel()
    assert A.size == M * K and B.size == K * N
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < M * N)
    C = np.empty(idx.size, np.uint16)
    Cx = np.empty(idx.size, np.float64)
    S = np.empty(idx.size, np.float64)
    macs = lib().oracle_gemm_sampled(fmt_id(fmt), _p(A, ctypes.c_uint16),
                                     _p(B, ctypes.c_uint16), M, N, K,
                                     _p(idx, ctypes.c_int64), idx.size,
                                     _p(C, ctypes.c_uint16), _p(Cx, ctypes.c_double),
                                     _p(S, ctypes.c_double))
    return GemmResult(C, Cx, S, macs)


def gemv(W, X, M, K, n, fmt="bf16") -> GemmResult:
    """Y = X W^T: W row-major [M,K], X row-major [n,K]; Y row-major [n,M]."""
    W, X = _u16(W).ravel(), _u16(X).ravel()
    assert W.size == M * K and X.size == n * K
    Y = np.empty(n * M, np.uint16)
    Yx = np.empty(n * M, np.float64)
    S = np.empty(n * M, np.float64)
    macs = lib().oracle_gemv(fmt_id(fmt), _p(W, ctypes.c_uint16), _p(X, ctypes.c_uint16),
                             _p(Y, ctypes.c_uint16), _p(Yx, ctypes.c_double),
                             _p(S, ctypes.c_double), M, K, n)
    return GemmResult(Y, Yx, S, macs)


class AttentionResult(GemmResult):
    """Oracle attention output: ``bits``, ``exact`` (double), ``sabs``
    (sum_l p_l |v_ld|), ``macs``, and ``qk_abs`` per (b, h): the largest
    |scale| * sum_d |q_d k_ld| over the cached tokens."""

    def __init__(self, bits, exact, sabs, macs, qk_abs):
        super().__init__(bits, exact, sabs, macs)
        self.qk_abs = qk_abs


def _att_args(Q, Kc, Vc, block_table, seq_lens):
    Q, Kc, Vc = _u16(Q).ravel(), _u16(Kc).ravel(), _u16(Vc).ravel()
    bt = np.ascontiguousarray(block_table, np.int32).ravel()
    sl = np.ascontiguousarray(seq_lens, np.int32).ravel()
    return Q, Kc, Vc, bt, sl


def attention(Q, Kc, Vc, block_table, seq_lens, B, Hq, Hkv, D, block_size, max_blocks,
              scale, fmt="bf16") -> AttentionResult:
    """Decode attention, the plain definition (DCU decode page, section 6.1):
    out[b,h,:] = softmax(scale * q K^T) V over the seq_lens[b] cached tokens
    of kv head h // (Hq // Hkv).  Q, out: [B, Hq, D]; Kc, Vc: paged
    [block, token_in_block, Hkv, D]; block_table: [B, max_blocks] page ids."""
    Q, Kc, Vc, bt, sl = _att_args(Q, Kc, Vc, block_table, seq_lens)
    n = B * Hq * D
    out = np.empty(n, np.uint16)
    ox = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    qka = np.empty(B * Hq, np.float64)
    macs = lib().oracle_attention(fmt_id(fmt), _p(Q, ctypes.c_uint16), _p(Kc, ctypes.c_uint16),
                                  _p(Vc, ctypes.c_uint16), _p(bt, ctypes.c_int32),
                                  _p(sl, ctypes.c_int32), B, Hq, Hkv, D, block_size, max_blocks,
                                  scale, _p(out, ctypes.c_uint16), _p(ox, ctypes.c_double),
                                  _p(S, ctypes.c_double), _p(qka, ctypes.c_double))
    return AttentionResult(out, ox, S, macs, qka)


def attention_segmented(Q, Kc, Vc, block_table, seq_lens, B, Hq, Hkv, D, block_size,
                        max_blocks, scale, nseg, fmt="bf16"):
    """The page's segmented algorithm (section 6.3) in double: returns
    (rounded bits, double values)."""
    Q, Kc, Vc, bt, sl = _att_args(Q, Kc, Vc, block_table, seq_lens)
    n = B * Hq * D
    out = np.empty(n, np.uint16)
    ox = np.empty(n, np.float64)
    lib().oracle_attention_segmented(fmt_id(fmt), _p(Q, ctypes.c_uint16), _p(Kc, ctypes.c_uint16),
                                     _p(Vc, ctypes.c_uint16), _p(bt, ctypes.c_int32),
                                     _p(sl, ctypes.c_int32), B, Hq, Hkv, D, block_size,
                                     max_blocks, scale, nseg, _p(out, ctypes.c_uint16),
                                     _p(ox, ctypes.c_double))
    return out, ox


Q_FMT = {"f8e4m3": 2, "f8e5m2": 3, "i8": 4}


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        a = a.view(np.uint8) if a.dtype == np.int8 else a.astype(np.uint8)
    return a.ravel()


def decode8(bits, fmt) -> np.ndarray:
    """Exact values of 8-bit codes: OCP FP8 E4M3 / E5M2 or INT8."""
    b = _u8(bits)
    out = np.empty(b.size, np.float64)
    lib().oracle_decode8_array(Q_FMT[fmt], _p(b, ctypes.c_uint8), _p(out, ctypes.c_double), b.size)
    return out


def gemm_tn_q(At, B, M, N, K, fmt, scale, idx=None) -> GemmResult:
    """8-bit GEMM, A k-major: C(m,n) = BF16(scale * sum_k At[k+m*K] B[k+n*K])
    (INT8: through FP32 as the output is defined; see oracle.c), column-major
    M x N, or the entries at flat indices idx.  sabs = |scale| sum |a||b|."""
    At, B = _u8(At), _u8(B)
    count = M * N if idx is None else len(idx)
    ix = None if idx is None else np.ascontiguousarray(idx, np.int64)
    bits = np.empty(count, np.uint16)
    ex = np.empty(count, np.float64)
    S = np.empty(count, np.float64)
    macs = lib().oracle_gemm_tn_q(Q_FMT[fmt], _p(At, ctypes.c_uint8), _p(B, ctypes.c_uint8),
                                  M, N, K, scale,
                                  None if ix is None else _p(ix, ctypes.c_int64), count,
                                  _p(bits, ctypes.c_uint16), _p(ex, ctypes.c_double),
                                  _p(S, ctypes.c_double))
    return GemmResult(bits, ex, S, macs)


def gamma(n, u=2.0 ** -24):
    """Higham's gamma_n = n u / (1 - n u)."""
    return n * u / (1.0 - n * u)


def attention_rel(ref: AttentionResult, seq_lens, Hq, D):
    """Relative bound, per output element, for an FP32 evaluation of decode
    attention in any order (scores summed over D, exponentials, sums over L,
    one merge): 2 * |scale| * gamma_D * sum_d |q k| (a score error scales
    both numerator and denominator terms by up to e^eps) + 2 * gamma_L (the
    sums of numerator and denominator) + 16 u (exp, division, merge)."""
    sl = np.asarray(seq_lens, np.int64)
    B = sl.size
    L = np.repeat(sl, Hq)                                   # per (b, h)
    rel = 2 * ref.qk_abs * gamma(D) + 2 * np.array([gamma(max(int(x), 1)) for x in L]) + 16 * 2.0 ** -24
    return np.repeat(rel, D).reshape(B * Hq * D)


def grouped_tile(pid, num_pid_m, num_pid_n, group_m):
    """Grouped tile ordering of the FlagGems Hygon page: pid -> (pid_m, pid_n)."""
    pm, pn = ctypes.c_int64(), ctypes.c_int64()
    lib().oracle_grouped_tile(pid, num_pid_m, num_pid_n, group_m,
                              ctypes.byref(pm), ctypes.byref(pn))
    return pm.value, pn.value


def set_threads(n):
    """OpenMP threads for the oracle's loops from now on (results do not
    depend on it); returns the previous count."""
    return lib().oracle_set_threads(int(n))


def grouped_order(num_pid_m, num_pid_n, group_m):
    """The whole grouped ordering as a table: entry p is program p's tile
    (pid_m, pid_n), built by walking the tiles group by group."""
    n = num_pid_m * num_pid_n
    pm = np.zeros(n, np.int64)
    pn = np.zeros(n, np.int64)
    lib().oracle_grouped_order(num_pid_m, num_pid_n, group_m, _p(pm, ctypes.c_int64),
                               _p(pn, ctypes.c_int64))
    return list(zip(pm.tolist(), pn.tolist()))


# ---- acceptance rule -------------------------------------------------------

_PARAMS = {FP16: (10, -14), BF16: (7, -126)}   # stored mantissa bits, emin


def ulp_out(ref_values, fmt) -> np.ndarray:
    """Spacing of the output format at |v|: 2^(max(e, emin) - mbits) with
    e = floor(log2|v|); at v = 0 the smallest subnormal spacing."""
    mbits, emin = _PARAMS[fmt_id(fmt)]
    v = np.abs(np.asarray(ref_values, np.float64))
    v = np.where(np.isfinite(v), v, 0.0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.where(v > 0, np.maximum(e, emin), emin)
    return np.ldexp(1.0, (e - mbits).astype(np.int64))


def check(got_bits, ref: GemmResult, fmt, rel=2e-3):
    """Apply the acceptance rule.  Returns (ok, report dict)."""
    f = fmt_id(fmt)
    got = decode(np.asarray(got_bits, np.uint16), f)
    want = decode(ref.bits, f)
    fin_w, fin_g = np.isfinite(want), np.isfinite(got)
    bad_class = (fin_w != fin_g)
    nf = ~fin_w & ~fin_g
    bad_class |= nf & (np.isnan(want) != np.isnan(got))
    bad_class |= nf & ~np.isnan(want) & (np.sign(want) != np.sign(got))
    both = fin_w & fin_g
    err = np.zeros(got.shape)
    err[both] = np.abs(got[both] - want[both])
    bound = rel * ref.sabs + ulp_out(want, f)
    bad_val = both & (err > bound)
    bad = bad_class | bad_val
    ratio = np.where(both, err / bound, 0.0)
    rep = {"checked": int(got.size), "bad": int(bad.sum()),
           "max_err": float(err.max()) if err.size else 0.0,
           "max_ratio": float(ratio.max()) if ratio.size else 0.0,
           "first_bad": np.nonzero(bad)[0][:8].tolist()}
    return (rep["bad"] == 0), rep
