"""GPU parity of the split-K GEMM (gemm_splitk_ex) through the C ABI against
the CPU oracle: both layouts of A, both 16-bit types, the three tiles that
take slices, slice counts that divide K and ones that leave a short last
slice (or fewer slices than asked), launches whose loads all lie in range
and ragged ones, every output at small sizes and sampled
outputs of a long-K product with the automatic slice count."""
import numpy as np
import pytest

import oracle
import synth
from helpers import Guarded, assert_parity, dev, kmajor_to_colmajor

pytestmark = pytest.mark.gpu


def _splitk(A, B, M, N, K, fmt, a_kmajor, splits, tile=0):
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    dA, dB = dev(A), dev(B)
    cA, cB = dA.clone(), dB.clone()
    C = Guarded(M * N)
    ws_bytes = max(16, L.migemm_splitk_workspace_bytes(M, N, max(splits, 32)))
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
    code = L.gemm_splitk_ex(0 if fmt == "f16" else 1, a_kmajor, dA.data_ptr(), dB.data_ptr(), C.ptr,
                            M, N, K, splits, tile, 0, 1, ws.data_ptr(), ws_bytes, None)
    assert code == 0, code
    torch.cuda.synchronize()
    assert torch.equal(dA, cA) and torch.equal(dB, cB), "inputs modified"
    assert C.guards_intact(), "write outside C"
    return C.out()


CASES = [
    # M, N, K, a_kmajor, splits, tile
    # (a column-major A needs M a multiple of 8 for the 16-byte loads)
    (304, 200, 4136, 0, 2, 9), (300, 200, 4136, 1, 3, 9), (520, 264, 2048, 0, 4, 10),
    (520, 264, 2048, 1, 4, 10), (136, 70, 8200, 0, 8, 13), (130, 70, 8200, 1, 5, 13),
    (256, 128, 192, 0, 3, 9), (64, 64, 4096, 1, 0, 0), (1000, 40, 3000, 0, 6, 0),
    # every load in range (M, N multiples of 256, K of 64): tile 10's slices
    # load through global addresses
    (512, 256, 4096, 0, 4, 10), (512, 256, 4096, 1, 4, 10),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_splitk_parity(case, fmt):
    M, N, K, ak, S, tile = CASES[case]
    print("case splitk", CASES[case], fmt, flush=True)
    A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 700 + case)
    got = _splitk(A, B, M, N, K, fmt, ak, S, tile)
    Acm = kmajor_to_colmajor(A, M, K) if ak else A
    assert_parity(got, oracle.gemm(Acm, B, M, N, K, fmt), fmt, "splitk %s %s" % (CASES[case], fmt))


def test_splitk_long_k_sampled():
    M, N, K = 1024, 1024, 65536
    print("case splitk long K", flush=True)
    A, B = synth.gemm_operands(M, N, K, "bf16", ("normal", 1.0, 1.0), 777)
    got = _splitk(A, B, M, N, K, "bf16", 0, 0)
    idx = synth.sample_indices(M, N, 777, 2048)
    assert_parity(got[idx], oracle.gemm_sampled(A, B, M, N, K, idx, "bf16"), "bf16", "splitk long K")
