"""attention_decode_bf16_noalloc (partials in the library's per-GPU device
array, no allocation) against attention_decode_bf16 with a caller
workspace: bit-identical outputs on two calls in a row, the second smaller,
through the C ABI."""
import numpy as np
import pytest

import synth
from helpers import dev, host

pytestmark = pytest.mark.gpu


def _both(op, scale, S):
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    B, Hq, Hkv, D = op["B"], op["Hq"], op["Hkv"], op["D"]
    dQ, dK, dV = dev(op["Q"]), dev(op["K"]), dev(op["V"])
    bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
    mlen = int(max(op["seq_lens"]))
    segs = S or L.migemm_attention_segments(B, Hq, Hkv, mlen)
    need = L.migemm_attention_workspace_bytes(B, Hq, D, segs)
    assert need <= (8 << 20)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    out_ws = torch.full((B * Hq * D,), -1, dtype=torch.int16, device="cuda")
    out_na = torch.full((B * Hq * D,), -1, dtype=torch.int16, device="cuda")
    args = (dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), bt.data_ptr(), sl.data_ptr())
    shape = (B, Hq, Hkv, D, op["block_size"], op["max_blocks"], op["num_blocks"], scale, mlen, S)
    code = L.attention_decode_bf16(*args, out_ws.data_ptr(), *shape, ws.data_ptr(), ws.numel(), None)
    assert code == 0, code
    code = L.attention_decode_bf16_noalloc(*args, out_na.data_ptr(), *shape, None)
    assert code == 0, code
    torch.cuda.synchronize()
    return host(out_ws), host(out_na)


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    w = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    # first: the page's head shape, 2 sequences of 8192 and 5000 tokens, automatic segments
    op = synth.attention_operands(2, w["Hq"], w["Hkv"], w["D"], [8192, 5000], w["block_size"], seed=71)
    print("case noalloc 1: B 2, 16q/4kv, d256, L 8192/5000, S auto", flush=True)
    a, b = _both(op, 1.0 / 16, 0)
    assert np.array_equal(a, b)
    assert np.all(a != 0xFFFF)
    # second, smaller: fewer heads, smaller head dim and segments, fewer tokens
    op2 = synth.attention_operands(1, 8, 2, 128, [300], 16, seed=72)
    print("case noalloc 2: B 1, 8q/2kv, d128, L 300, S 4", flush=True)
    a2, b2 = _both(op2, 0.125, 4)
    assert np.array_equal(a2, b2)
    assert np.all(a2 != 0xFFFF)
