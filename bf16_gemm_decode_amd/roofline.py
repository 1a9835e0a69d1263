"""Work, traffic and roofline arithmetic for the GEMM and the decode GEMV.

The roofline is the simplified form of the DCU decode page (forum.sourcefind.cn
db785961), section 3: attainable = min(compute peak, bandwidth x intensity),
intensity = FLOP per byte moved.  GEMM work is 2*M*N*K (MTT S4000 GEMM
write-up, section 2).  Bytes are algorithmic: every operand read once and the
output written once.  Units: GB = 1e9 B, TFLOP = 1e12 FLOP.
"""

# MI355X published peaks (dense, no sparsity).
MI355X = {
    "cus": 256,
    "xcds": 8,
    "clock_ghz": 2.4,
    "hbm_GBps": 8000.0,
    "mfma_f16_tflops": 2500.0,
    "mfma_bf16_tflops": 2500.0,
    "mfma_fp8_tflops": 5000.0,
    "mfma_int8_tops": 5000.0,
    "valu_fp32_tflops": 157.3,
    "valu_fp64_tflops": 78.6,
}


def gemm_flop(M, N, K):
    return 2.0 * M * N * K


def gemm_bytes(M, N, K, elt=2):
    return float(elt) * (M * K + K * N + M * N)


def gemv_flop(M, K, n):
    return 2.0 * n * M * K


def gemv_bytes(M, K, n, elt=2):
    """W [M,K] read once, X [n,K] read once, Y [n,M] written once."""
    return float(elt) * (M * K + n * K + n * M)


def intensity(flop, nbytes):
    return flop / nbytes


def bandwidth_roof_tflops(bw_GBps, flop_per_byte):
    return bw_GBps * flop_per_byte / 1000.0


def attainable_tflops(peak_tflops, bw_GBps, flop_per_byte):
    return min(peak_tflops, bandwidth_roof_tflops(bw_GBps, flop_per_byte))


def bound(peak_tflops, bw_GBps, flop_per_byte):
    """'hbm' below the ridge point, 'compute' at or above it."""
    return "hbm" if bandwidth_roof_tflops(bw_GBps, flop_per_byte) < peak_tflops else "compute"


def ridge(peak_tflops, bw_GBps):
    """Intensity (FLOP/byte) where the two roofs meet."""
    return peak_tflops * 1000.0 / bw_GBps


def seconds_at(amount, rate):
    return amount / rate


def attention_bytes(seq_lens, Hq, Hkv, D, block_size, elt=2):
    """Decode attention (one query token per sequence): every cached K and V
    row of the kv heads read once, Q read once, the output written once, and
    the block-table entries of the used pages read once."""
    kv = sum(2.0 * elt * int(L) * Hkv * D for L in seq_lens)
    pages = sum(4.0 * (-(-int(L) // block_size)) for L in seq_lens)
    return kv + pages + 2.0 * elt * len(seq_lens) * Hq * D


def attention_flop(seq_lens, Hq, D):
    """q.k and prob*v: 4 * L * Hq * D per sequence (softmax not counted)."""
    return sum(4.0 * int(L) * Hq * D for L in seq_lens)
