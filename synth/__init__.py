"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.

This module holds none of the method's arithmetic: it only draws random
numbers and stores them as 16-bit patterns, using numpy's float64->float16
conversion and torch's float32->bfloat16 conversion (both round to nearest
even).  Both the HIP path and the CPU oracle receive what it returns.

Input recipe (the pages fix shapes and distributions, not the generator):
  * one ``numpy.random.default_rng(seed)`` (PCG64) per workload;
  * operands are drawn in argument order -- A then B for the GEMM, W then X
    for the GEMV -- each filled in its own flat storage order (column-major
    index for GEMM operands, row-major for GEMV operands);
  * FP16: float64 draw -> nearest-even binary16.  BF16: float64 draw ->
    nearest-even float32 -> nearest-even bfloat16;
  * "N(0, s)" means standard deviation s.
"""
import numpy as np

F16 = "f16"
BF16 = "bf16"

# The five workloads of the pages (shapes from the S4000 GEMM write-up's
# contest size and the DCU decode page's gate/up projection).
WORKLOADS = {
    "gemm_512_f16": dict(kind="gemm", M=512, N=512, K=512, fmt=F16,
                         dist=("uniform", 1.0, 1.0), seed=0),
    "gemm_8192x8192x16384_f16": dict(kind="gemm", M=8192, N=8192, K=16384, fmt=F16,
                                     dist=("uniform", 1.0, 1.0), seed=1),
    "gemm_5000x3000x4100_bf16": dict(kind="gemm", M=5000, N=3000, K=4100, fmt=BF16,
                                     dist=("normal", 1.0, 1.0), seed=2),
    "gemv_34816x5120_bf16": dict(kind="gemv", M=34816, K=5120, fmt=BF16,
                                 n_values=(1, 4, 16), seed=3),
    "prefill_4096x34816x5120_bf16": dict(kind="gemm", M=4096, N=34816, K=5120, fmt=BF16,
                                         dist=("normal", 1.0, 0.02), seed=4),
    # decode attention of the DCU page's head shape (16 query heads, 4 KV
    # heads, head dim 256, BF16, pages of 784 tokens), one query token,
    # Q, K, V ~ N(0, 1), scale 1/sqrt(D)
    "attention_decode_16q4kv_d256_bf16": dict(kind="attention", Hq=16, Hkv=4, D=256,
                                              block_size=784, lengths=(8192, 16384, 32768),
                                              B=1, fmt=BF16, seed=5),
}


def to_bits(values, fmt) -> np.ndarray:
    """Store float64 values as 16-bit patterns (uint16), nearest-even."""
    v = np.asarray(values, dtype=np.float64)
    if fmt == F16:
        return v.astype(np.float16).view(np.uint16)
    if fmt == BF16:
        import torch
        t = torch.from_numpy(np.ascontiguousarray(v.astype(np.float32)))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(fmt)


def from_bits(bits, fmt) -> np.ndarray:
    """float32 view of 16-bit patterns (for quick looks; exact for both)."""
    b = np.asarray(bits, np.uint16)
    if fmt == F16:
        return b.view(np.float16).astype(np.float32)
    if fmt == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(fmt)


def _draw(rng, size, kind, scale):
    if kind == "uniform":
        return rng.uniform(-scale, scale, size)
    if kind == "normal":
        return rng.normal(0.0, scale, size)
    raise ValueError(kind)


def gemm_operands(M, N, K, fmt, dist=("uniform", 1.0, 1.0), seed=0):
    """A (M x K) and B (K x N), column-major, as flat uint16 arrays.
    dist = (kind, scale_A, scale_B): uniform[-s, s] or normal(0, s)."""
    kind, sa, sb = dist
    rng = np.random.default_rng(seed)
    A = to_bits(_draw(rng, M * K, kind, sa), fmt)
    B = to_bits(_draw(rng, K * N, kind, sb), fmt)
    return A, B


def gemv_operands(M, K, n, seed=3, sigma_w=0.02, sigma_x=1.0, fmt=BF16):
    """W row-major [M, K] ~ N(0, sigma_w), X row-major [n, K] ~ N(0, sigma_x)."""
    rng = np.random.default_rng(seed)
    W = to_bits(rng.normal(0.0, sigma_w, M * K), fmt)
    X = to_bits(rng.normal(0.0, sigma_x, n * K), fmt)
    return W, X


def workload_operands(name, n=None):
    w = WORKLOADS[name]
    if w["kind"] == "gemm":
        return gemm_operands(w["M"], w["N"], w["K"], w["fmt"], w["dist"], w["seed"])
    return gemv_operands(w["M"], w["K"], n, seed=w["seed"], fmt=w["fmt"])


def attention_operands(B, Hq, Hkv, D, seq_lens, block_size, seed, sigma=1.0, spare_blocks=3,
                       fmt=BF16):
    """Decode-attention inputs.  Q [B, Hq, D] and the paged caches K, V
    [num_blocks, block_size, Hkv, D] ~ N(0, sigma) (drawn in that order, flat
    storage order); block_table [B, max_blocks] int32: each sequence takes
    ceil(L / block_size) pages from a seeded permutation of all pages (so
    pages are scattered), unused entries -1."""
    rng = np.random.default_rng(seed)
    seq_lens = [int(x) for x in seq_lens]
    need = [-(-L // block_size) for L in seq_lens]
    max_blocks = max(1, max(need) if need else 1)
    nblocks = sum(need) + spare_blocks
    Q = to_bits(rng.normal(0.0, sigma, B * Hq * D), fmt)
    K = to_bits(rng.normal(0.0, sigma, nblocks * block_size * Hkv * D), fmt)
    V = to_bits(rng.normal(0.0, sigma, nblocks * block_size * Hkv * D), fmt)
    perm = rng.permutation(nblocks)
    bt = np.full((B, max_blocks), -1, np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return dict(Q=Q, K=K, V=V, block_table=bt, seq_lens=np.array(seq_lens, np.int32),
                max_blocks=max_blocks, num_blocks=nblocks, B=B, Hq=Hq, Hkv=Hkv, D=D,
                block_size=block_size)


def q8_operands(M, N, K, fmt, seed, sigma=1.0):
    """8-bit operands of the k-major GEMM: At row-major [M, K] then B as N
    columns of K, flat uint8 codes.  FP8 (fmt 'f8e4m3' / 'f8e5m2'): N(0,
    sigma) drawn in float32 and converted to torch's OCP float8 types
    (nearest even); INT8 ('i8'): integers uniform in [-128, 127]."""
    rng = np.random.default_rng(seed)
    if fmt == "i8":
        At = rng.integers(-128, 128, M * K).astype(np.int8).view(np.uint8)
        B = rng.integers(-128, 128, N * K).astype(np.int8).view(np.uint8)
        return At, B
    import torch
    dt = {"f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}[fmt]

    def enc(n):
        x = torch.from_numpy(rng.normal(0.0, sigma, n).astype(np.float32))
        return x.to(dt).view(torch.uint8).numpy().copy()
    At = enc(M * K)
    B = enc(N * K)
    return At, B


def to_q8(values, fmt) -> np.ndarray:
    """Codes of the 8-bit formats for values they hold exactly (small
    integers): INT8 two's complement ('i8'), or torch's OCP float8 types
    ('f8e4m3', 'f8e5m2'); flat uint8."""
    v = np.asarray(values, dtype=np.float64).ravel()
    if fmt == "i8":
        return v.astype(np.int8).view(np.uint8)
    import torch
    dt = {"f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}[fmt]
    return torch.from_numpy(v.astype(np.float32)).to(dt).view(torch.uint8).numpy().copy()


def sample_indices(M, N, seed, count=4096):
    """``count`` distinct flat output indices (m + n*M) drawn with
    default_rng(1000 + seed), plus the four corners, sorted."""
    total = M * N
    rng = np.random.default_rng(1000 + seed)
    idx = rng.choice(total, size=min(count, total), replace=False)
    corners = np.array([0, M - 1, (N - 1) * M, total - 1], np.int64)
    return np.unique(np.concatenate([idx.astype(np.int64), corners]))


def small_ints(rng, size, lo, hi):
    """Integers in [lo, hi] as float64 (exact in every 16-bit format here)."""
    return rng.integers(lo, hi + 1, size).astype(np.float64)


def identity_colmajor(n):
    """n x n identity, column-major flat float64."""
    return np.eye(n, dtype=np.float64).ravel(order="F")


def cyclic_shift_colmajor(n, s=1):
    """Permutation matrix P (n x n) with P(i, (i + s) mod n) = 1, column-major
    flat float64 -- not symmetric for n > 2 and s != 0, n/2."""
    P = np.zeros((n, n))
    P[np.arange(n), (np.arange(n) + s) % n] = 1.0
    return P.ravel(order="F")


def mod5_pattern(i, j, a, b):
    """Small-integer operand pattern ((a*i + b*j) mod 5) - 2, values in
    [-2, 2], as float64 (exact in every 16-bit format here), broadcast over
    index arrays i and j.  For a fixed j it takes only five distinct rows
    over i (the row for j depends on b*j mod 5 alone), so an operand of
    billions of elements can be assembled on the device from five short rows,
    while any of its rows or columns can be rebuilt on the host from the same
    formula."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    return (((a * i + b * j) % 5) - 2).astype(np.float64)


def _exact_dim(h, t, L, D):
    """Head-dim slot of logical token t in kv head h for the exact-class V:
    h = 0: t mod D; h = 1: the run of L/D consecutive tokens t lies in
    (together these two identify every token of a sequence of L <= D*D);
    h = 2, 3: mixed.  Consecutive tokens never share a slot in kv head 0."""
    t = np.asarray(t, dtype=np.int64)
    if h % 4 == 0:
        return t % D
    if h % 4 == 1:
        return (t // max(1, L // D)) % D
    if h % 4 == 2:
        return (t + t // 16) % D
    return (5 * t + t // 64) % D


def attention_exact_operands(seq_len, kind, Hq=16, Hkv=4, D=256, block_size=784, seed=7,
                             spare_blocks=3, fmt=BF16):
    """Decode-attention inputs whose output every correct implementation
    with FP32 sums returns bit for bit (one sequence, power-of-two seq_len).

    The page layout and the block table are those of attention_operands
    (scattered pages); unused pages keep N(0, 1) values.  For every logical
    token t of kv head h, V holds 1 in head-dim slot _exact_dim(h, t) and 0
    elsewhere, so each output is (number of counted tokens mapped to its
    slot) / (number of counted tokens): small integers over a power of two.
      * kind "uniform": Q = 0, every score is 0, every token is counted;
      * kind "mask": query head h holds 1024 in head-dim h mod D, zeros
        elsewhere; in the kv head's dims of its query heads K holds 0 for
        an exactly half of the tokens (a seeded choice per kv head) and
        -1024 for the rest, so the scores are 0 or -2^20 * scale: weights
        exactly 1 or (after the exponential underflows) exactly 0.
    Returns the attention_operands dict plus 'counted' [Hkv, L] (bool)."""
    if seq_len <= 0 or seq_len & (seq_len - 1):
        raise ValueError("seq_len must be a power of two")
    op = attention_operands(1, Hq, Hkv, D, [seq_len], block_size, seed, spare_blocks=spare_blocks,
                            fmt=fmt)
    rng = np.random.default_rng(seed + 1)
    L, G = seq_len, Hq // Hkv
    t = np.arange(L)
    page = op["block_table"][0][t // block_size].astype(np.int64)
    row = (page * block_size + t % block_size)          # cache row of logical token t
    V = op["V"].reshape(-1, Hkv, D).copy()
    K = op["K"].reshape(-1, Hkv, D).copy()
    one, zero, neg = to_bits([1.0, 0.0, -1024.0], fmt)
    counted = np.ones((Hkv, L), bool)
    for h in range(Hkv):
        V[row, h, :] = zero
        V[row, h, _exact_dim(h, t, L, D)] = one
        if kind == "mask":
            keep = np.zeros(L, bool)
            keep[rng.permutation(L)[:L // 2]] = True
            counted[h] = keep
            dims = [(h * G + j) % D for j in range(G)]
            for d in dims:
                K[row, h, d] = np.where(keep, zero, neg)
    if kind == "uniform":
        Q = np.full(Hq * D, zero, np.uint16)
    elif kind == "mask":
        Q = np.full((Hq, D), zero, np.uint16)
        Q[np.arange(Hq), np.arange(Hq) % D] = to_bits([1024.0], fmt)[0]
        Q = Q.reshape(-1)
    else:
        raise ValueError(kind)
    op.update(Q=Q, K=K.reshape(-1), V=V.reshape(-1), counted=counted)
    return op
