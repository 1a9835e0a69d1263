"""Shared helpers for the GPU parity tests: device buffers with guard bands,
calls through the C ABI, and checks against the oracle."""
import numpy as np

import oracle
import synth

SENTINEL = 0xFFFF
GUARD = 4096


def dev(bits):
    """uint16 numpy array -> int16 CUDA tensor holding the same bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy().view(np.uint16)


class Guarded:
    """An output buffer of `count` uint16 with GUARD sentinel words on both
    sides; `ptr` is the address of the first output element."""

    def __init__(self, count, guard=GUARD):
        import torch
        self.count, self.guard = count, guard
        self.buf = torch.full((count + 2 * guard,), -1, dtype=torch.int16, device="cuda")
        self.ptr = self.buf.data_ptr() + 2 * guard

    def out(self):
        return host(self.buf[self.guard:self.guard + self.count])

    def guards_intact(self):
        h = host(self.buf)
        return bool(np.all(h[:self.guard] == SENTINEL) and np.all(h[self.guard + self.count:] == SENTINEL))


def gemm_gpu(A_bits, B_bits, M, N, K, fmt, tile=0, group_m=0, xcd_remap=1, stream=0, c_shift=0):
    """Run the library GEMM through the C ABI; returns (C bits, guards ok,
    inputs unchanged).  c_shift moves C by that many elements (4: C on an
    8-byte but not a 16-byte boundary)."""
    import torch
    from bf16_gemm_decode_amd import binding
    dA, dB = dev(A_bits), dev(B_bits)
    cA, cB = dA.clone(), dB.clone()
    C = Guarded(M * N, GUARD + c_shift)
    code = binding.gemm_ex_ptr(binding.F16 if fmt == "f16" else binding.BF16,
                               dA.data_ptr(), dB.data_ptr(), C.ptr, M, N, K,
                               tile, group_m, xcd_remap, stream)
    assert code == 0, "gemm_ex returned %d" % code
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(dA, cA) and torch.equal(dB, cB))
    return C.out(), C.guards_intact(), unchanged


def gemm_tn_gpu(At_bits, B_bits, M, N, K, fmt, tile=0, group_m=0, xcd_remap=1, stream=0, c_shift=0):
    """gemm_tn_ex through the C ABI (A given k-major: A(m,k) = At[k + m*K]);
    returns (C bits, guards ok, inputs unchanged)."""
    import torch
    from bf16_gemm_decode_amd import binding
    dA, dB = dev(At_bits), dev(B_bits)
    cA, cB = dA.clone(), dB.clone()
    C = Guarded(M * N, GUARD + c_shift)
    code = binding.gemm_tn_ex_ptr(binding.F16 if fmt == "f16" else binding.BF16,
                                  dA.data_ptr(), dB.data_ptr(), C.ptr, M, N, K,
                                  tile, group_m, xcd_remap, stream)
    assert code == 0, "gemm_tn_ex returned %d" % code
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(dA, cA) and torch.equal(dB, cB))
    return C.out(), C.guards_intact(), unchanged


def gemm_tn_q_gpu(At, B, M, N, K, fmt, scale, tile=0, stream=0, c_shift=0):
    """gemm_tn_q_ex (8-bit At, B; BF16 C) through the C ABI; returns (C bits,
    guards ok, inputs unchanged)."""
    import torch
    from bf16_gemm_decode_amd import binding
    q = {"f8e4m3": binding.F8E4M3, "f8e5m2": binding.F8E5M2, "i8": binding.I8}[fmt]
    dA = torch.from_numpy(np.ascontiguousarray(At).view(np.uint8)).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B).view(np.uint8)).cuda()
    cA, cB = dA.clone(), dB.clone()
    C = Guarded(M * N, GUARD + c_shift)
    code = binding.lib().gemm_tn_q_ex(q, dA.data_ptr(), dB.data_ptr(), C.ptr, M, N, K, scale,
                                      tile, 0, 1, stream)
    assert code == 0, "gemm_tn_q_ex returned %d" % code
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(dA, cA) and torch.equal(dB, cB))
    return C.out(), C.guards_intact(), unchanged


def kmajor_to_colmajor(At_bits, M, K):
    """A(m,k) = At[k + m*K]  ->  column-major A[m + k*M] (a pure relayout)."""
    return np.ascontiguousarray(np.asarray(At_bits).reshape(M, K).T).reshape(-1)


def gemv_gpu(W_bits, X_bits, M, K, n, rows_per_block=0, stream=0):
    import torch
    from bf16_gemm_decode_amd import binding
    dW, dX = dev(W_bits), dev(X_bits)
    cW, cX = dW.clone(), dX.clone()
    Y = Guarded(n * M)
    code = binding.gemv_bf16_ex_ptr(dW.data_ptr(), dX.data_ptr(), Y.ptr, M, K, n,
                                    rows_per_block, stream)
    assert code == 0, "gemv_bf16_ex returned %d" % code
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(dW, cW) and torch.equal(dX, cX))
    return Y.out(), Y.guards_intact(), unchanged


def assert_parity(got, ref, fmt, what):
    ok, rep = oracle.check(got, ref, fmt)
    assert ok, "%s: %s" % (what, rep)
    return rep


def attention_exact_expected(op, Hq, D):
    """Closed form of an exact-class attention input (synth.attention_exact_operands):
    output (h, d) = (counted tokens of kv head h's group mapped to slot d) /
    (counted tokens), as BF16 bits.  Both counts are integers and the
    denominator a power of two, so the value is exact before one rounding."""
    Hkv = op["Hkv"]
    L = int(op["seq_lens"][0])
    t = np.arange(L)
    exp = np.zeros((Hq, D))
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        cnt = op["counted"][kvh]
        c = np.bincount(synth._exact_dim(kvh, t[cnt], L, D), minlength=D)
        exp[h] = c / cnt.sum()
    return synth.to_bits(exp.ravel(), "bf16")


def exact_mismatches(got_bits, ref_bits):
    """Number of outputs whose bits differ (exact-class comparison)."""
    return int(np.count_nonzero(np.asarray(got_bits, np.uint16) != np.asarray(ref_bits, np.uint16)))
