"""GPU parity for operands of more than 2^31 elements (about 8.6 GB each), for
k-major A operands (8- and 16-bit) of more than 2^32 bytes, and for a paged KV
cache past 2^31 bytes: byte offsets past 32 bits, the per-step
rebasing of the buffer descriptors and the 64-bit row and page offsets of the
decode kernels.

The GEMM and GEMV operands follow synth.mod5_pattern, entries in [-2, 2]:
every partial sum is an integer below 2^24, so FP32 accumulation is exact in
any order and the one rounding to 16 bits is deterministic -- results are
compared bit for bit.  The pattern has five distinct rows, so the large
operand is assembled on the device by repeating them (torch indexing:
plumbing, no arithmetic of the method); the oracle computes the product
restricted to the sampled rows and columns, built on the host from the same
formula.  The attention case places seeded pages near the end of a large,
otherwise zero cache and checks against the oracle on the same pages
compacted."""
import numpy as np
import pytest

import oracle
import synth
from helpers import dev

pytestmark = pytest.mark.gpu


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _edge_indices(n, extra):
    """first, last and a few interior indices of 0..n-1, sorted, unique"""
    return np.unique(np.array([0, 1, n // 3, n // 2, n - 2, n - 1] + extra, dtype=np.int64) % n)


@pytest.mark.parametrize("fmt,big", [("f16", "A"), ("bf16", "B")])
def test_gemm_operand_past_2g_elements(fmt, big):
    import torch
    from bf16_gemm_decode_amd import binding
    K = 4100                                   # 4-byte rows: the k loop stops at 4096, then the tail
    M, N = ((1 << 20) + 8, 264) if big == "A" else (264, (1 << 20) + 8)
    assert (M if big == "A" else N) * K > 2 ** 31
    print("case large", big, fmt, (M, N, K), flush=True)
    # A(m, k) = ((m + 3k) mod 5) - 2: k-row k of the column-major A is row
    # class 3k mod 5; B(k, n) = ((k + 2n) mod 5) - 2: column n is class 2n mod 5
    arows = torch.stack([dev(synth.to_bits(synth.mod5_pattern(np.arange(M), c, 1, 1), fmt)) for c in range(5)])
    bcols = torch.stack([dev(synth.to_bits(synth.mod5_pattern(np.arange(K), c, 1, 1), fmt)) for c in range(5)])
    kidx = torch.arange(K, device="cuda") * 3 % 5
    nidx = torch.arange(N, device="cuda") * 2 % 5
    dA = arows[kidx].reshape(-1)               # [K][M]: A[m + k*M]
    dB = bcols[nidx].reshape(-1)               # [N][K]: B[k + n*K]
    del arows, bcols
    dC = torch.full((M * N,), 0x7C01, dtype=torch.int16, device="cuda")   # NaN marker
    code, plan = binding.gemm_plan(binding.F16 if fmt == "f16" else binding.BF16,
                                   dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K)
    assert code == 0 and plan["tile"] == 16          # the ping-pong tile, 4-byte B rows
    print("plan tile", plan["tile"], "grid", plan["grid"], flush=True)
    code = binding.gemm_ex_ptr(binding.F16 if fmt == "f16" else binding.BF16,
                               dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K)
    assert code == 0
    torch.cuda.synchronize()
    ms = _edge_indices(M, [(1 << 31) // K, (1 << 31) // K + 1, 257, 4095])
    ns = _edge_indices(N, [(1 << 31) // K, 255, 256, 4097])
    got = dC.view(M * N)[torch.from_numpy(ms[:, None] + ns[None, :] * M).cuda().reshape(-1)]
    got = got.cpu().numpy().view(np.uint16).reshape(len(ms), len(ns))
    # the product restricted to those rows and columns
    kk = np.arange(K)
    Asub = synth.to_bits(synth.mod5_pattern(ms[:, None], kk[None, :], 1, 3).ravel(order="F"), fmt)
    Bsub = synth.to_bits(synth.mod5_pattern(kk[:, None], ns[None, :], 1, 2).ravel(order="F"), fmt)
    ref = oracle.gemm(Asub, Bsub, len(ms), len(ns), K, fmt)
    want = ref.bits.reshape(len(ns), len(ms)).T          # column-major [ms x ns]
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
    del dA, dB, dC
    _free()


@pytest.mark.parametrize("fmt,big,tile", [("f8e4m3", "A", 17), ("f8e5m2", "B", 17), ("i8", "A", 10),
                                          ("i8", "B", 10), ("bf16", "A", 10), ("f16", "B", 10)])
def test_gemm_kmajor_operand_past_4g_bytes(fmt, big, tile):
    # A k-major (At[k + m*K]), 8- or 16-bit, one operand of more than 2^32
    # bytes, on the automatic tile (asserted).  K = 4112 units: whole 64-unit
    # stages, then a 16-unit tail.
    import torch
    from bf16_gemm_decode_amd import binding
    q8 = fmt in ("f8e4m3", "f8e5m2", "i8")
    esize = 1 if q8 else 2
    K = 4112
    M, N = ((1 << 20) + 8, 264) if big == "A" else (264, (1 << 20) + 8)
    assert (M if big == "A" else N) * K * esize > 2 ** 32
    print("case large k-major", big, fmt, (M, N, K), flush=True)

    def enc(v):
        return synth.to_q8(v, fmt) if q8 else synth.to_bits(v, fmt)

    def todev(codes):
        return torch.from_numpy(codes if q8 else codes.view(np.int16)).cuda()

    # A(m, k) = ((m + 3k) mod 5) - 2: row m of At is class m mod 5;
    # B(k, n) = ((k + 2n) mod 5) - 2: column n is class 2n mod 5
    kk = np.arange(K)
    arows = torch.stack([todev(enc(synth.mod5_pattern(c, kk, 1, 3))) for c in range(5)])
    bcols = torch.stack([todev(enc(synth.mod5_pattern(kk, c, 1, 1))) for c in range(5)])
    dA = arows[torch.arange(M, device="cuda") % 5].reshape(-1)         # [M][K]
    dB = bcols[torch.arange(N, device="cuda") * 2 % 5].reshape(-1)     # [N][K]
    del arows, bcols
    dC = torch.full((M * N,), 0x7FC1, dtype=torch.int16, device="cuda")   # NaN marker
    dtype = {"f8e4m3": binding.F8E4M3, "f8e5m2": binding.F8E5M2, "i8": binding.I8,
             "bf16": binding.BF16, "f16": binding.F16}[fmt]
    code, plan = binding.gemm_plan(dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K,
                                   a_kmajor=True)
    assert code == 0 and plan["tile"] == tile, plan
    print("plan tile", plan["tile"], "grid", plan["grid"], flush=True)
    if q8:
        code = binding.lib().gemm_tn_q_ex(dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K,
                                          1.0, 0, 0, 1, None)
    else:
        code = binding.gemm_tn_ex_ptr(dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K)
    assert code == 0
    torch.cuda.synchronize()
    big_dim = M if big == "A" else N
    cross = (1 << 32) // (K * esize)           # first row / column past 2^32 bytes
    ms = _edge_indices(M, [cross, cross + 1, 257, 4095] if big == "A" else [127, 128, 255])
    ns = _edge_indices(N, [cross, cross + 1, 255, 4097] if big == "B" else [127, 128, 255])
    assert big_dim - 1 > cross
    got = dC.view(M * N)[torch.from_numpy(ms[:, None] + ns[None, :] * M).cuda().reshape(-1)]
    got = got.cpu().numpy().view(np.uint16).reshape(len(ms), len(ns))
    # the product restricted to those rows and columns; every partial sum is
    # an integer below 2^24, so the results are exact and compared bit for bit
    Asub = enc(synth.mod5_pattern(ms[:, None], kk[None, :], 1, 3).ravel())     # [ms][K]
    Bsub = enc(synth.mod5_pattern(kk[None, :], ns[:, None], 1, 2).ravel())     # [ns][K]
    if q8:
        ref = oracle.gemm_tn_q(Asub, Bsub, len(ms), len(ns), K, fmt, 1.0)
    else:
        ref = oracle.gemm(np.ascontiguousarray(Asub.reshape(len(ms), K).T).reshape(-1), Bsub,
                          len(ms), len(ns), K, fmt)
    want = ref.bits.reshape(len(ns), len(ms)).T          # column-major [ms x ns]
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
    del dA, dB, dC
    _free()


@pytest.mark.parametrize("n", [1, 4, 16])
def test_gemv_weight_past_2g_elements(n):
    import torch
    from bf16_gemm_decode_amd import binding
    M, K = (1 << 19) + 3, 4104
    assert M * K > 2 ** 31
    print("case large gemv", (M, K, n), flush=True)
    # W[j][k] = ((3k + j) mod 5) - 2: row j is class j mod 5;
    # X[i][k] = ((k + 2i) mod 5) - 2
    wrows = torch.stack([dev(synth.to_bits(synth.mod5_pattern(np.arange(K), c, 3, 1), "bf16")) for c in range(5)])
    dW = wrows[torch.arange(M, device="cuda") % 5].reshape(-1)
    del wrows
    kk = np.arange(K)
    X = synth.to_bits(synth.mod5_pattern(kk[None, :], np.arange(n)[:, None], 1, 2).ravel(), "bf16")
    dX = dev(X)
    dY = torch.full((n * M,), 0x7FC1, dtype=torch.int16, device="cuda")
    code = binding.gemv_bf16_ptr(dW.data_ptr(), dX.data_ptr(), dY.data_ptr(), M, K, n)
    assert code == 0
    torch.cuda.synchronize()
    js = _edge_indices(M, [(1 << 31) // K, (1 << 31) // K + 1, 4099])
    got = dY.view(n, M)[:, torch.from_numpy(js).cuda()].cpu().numpy().view(np.uint16)
    Wsub = synth.to_bits(synth.mod5_pattern(kk[None, :], js[:, None], 3, 1).ravel(), "bf16")
    ref = oracle.gemv(Wsub, X, len(js), K, n)
    assert np.array_equal(got, ref.bits.reshape(n, len(js)))
    del dW, dX, dY
    _free()


def test_attention_cache_past_2g_bytes():
    # Paged caches of 2000 pages of 784 tokens (3.3 GB each at 4 KV heads,
    # head dim 256): the sequences' pages sit near the end, past 2^31 bytes
    # from the cache base.  Only those pages hold data; the oracle takes the
    # same pages compacted, with the block table renumbered.
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    Hq, Hkv, D, bs, NB = 16, 4, 256, 784, 2000
    op = synth.attention_operands(2, Hq, Hkv, D, [3000, 1500], bs, seed=77)
    page = bs * Hkv * D
    big = np.array([NB - 1 - 7 * p for p in range(op["num_blocks"])], np.int64)   # compact page -> big page
    assert int(big.min()) * page * 2 > 2 ** 31
    print("case large attention cache", NB, "pages, live pages", big.tolist(), flush=True)
    dK = torch.zeros(NB * page, dtype=torch.int16, device="cuda")
    dV = torch.zeros(NB * page, dtype=torch.int16, device="cuda")
    idx = torch.from_numpy(big).cuda()
    dK.view(NB, page)[idx] = dev(op["K"]).view(-1, page)
    dV.view(NB, page)[idx] = dev(op["V"]).view(-1, page)
    bt = op["block_table"].astype(np.int64)
    bt_big = np.where(bt >= 0, big[np.maximum(bt, 0)], -1).astype(np.int32)
    dbt = torch.from_numpy(np.ascontiguousarray(bt_big)).cuda()
    dsl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
    dQ = dev(op["Q"])
    out = torch.full((2 * Hq * D,), -1, dtype=torch.int16, device="cuda")
    scale = 1.0 / 16
    for S in (0, 16):
        segs = S or L.migemm_attention_segments(2, Hq, Hkv, 3000)
        wsb = L.migemm_attention_workspace_bytes(2, Hq, D, segs)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        code = L.attention_decode_bf16(dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), dbt.data_ptr(),
                                       dsl.data_ptr(), out.data_ptr(), 2, Hq, Hkv, D, bs, op["max_blocks"],
                                       NB, scale, 3000, S, ws.data_ptr(), wsb, None)
        assert code == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        ref = oracle.attention(op["Q"], op["K"], op["V"], op["block_table"], op["seq_lens"], 2, Hq, Hkv,
                               D, bs, op["max_blocks"], scale)
        ok, rep = oracle.check(got, ref, "bf16", rel=oracle.attention_rel(ref, op["seq_lens"], Hq, D))
        assert ok, ("large cache", S, rep)
    del dK, dV
    _free()
