"""GPU parity of attention_decode_bf16 (through the C ABI) against the CPU
oracle: every output at small and page-shaped sizes, scattered pages, group
sizes 1-8, head dims 64-256, empty and single-token sequences, segment counts
from 1 to more segments than tokens, and the DCU page's 32-vs-16 segment
agreement at its head shape (16 query heads, 4 KV heads, head dim 256, pages
of 784 tokens) for 8K, 16K and 32K cached tokens."""
import numpy as np
import pytest

import oracle
import synth
from helpers import dev, host

pytestmark = pytest.mark.gpu


def _gpu(op, scale, S, max_seq_len=None):
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    B, Hq, Hkv, D = op["B"], op["Hq"], op["Hkv"], op["D"]
    dQ, dK, dV = dev(op["Q"]), dev(op["K"]), dev(op["V"])
    cK, cV = dK.clone(), dV.clone()
    bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
    guard = 256
    out = torch.full((B * Hq * D + 2 * guard,), -1, dtype=torch.int16, device="cuda")
    mlen = int(max(op["seq_lens"])) if max_seq_len is None else max_seq_len
    segs = S or L.migemm_attention_segments(B, Hq, Hkv, mlen)
    need = L.migemm_attention_workspace_bytes(B, Hq, D, segs)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")   # counters start at zero
    code = L.attention_decode_bf16(dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), bt.data_ptr(),
                                   sl.data_ptr(), out.data_ptr() + 2 * guard, B, Hq, Hkv, D,
                                   op["block_size"], op["max_blocks"], op["num_blocks"], scale,
                                   mlen, S, ws.data_ptr(), ws.numel(), None)
    assert code == 0, code
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[:guard] == 0xFFFF) and np.all(o[-guard:] == 0xFFFF), "write outside Out"
    assert torch.equal(dK, cK) and torch.equal(dV, cV), "cache modified"
    return o[guard:-guard]


def _ref(op, scale):
    return oracle.attention(op["Q"], op["K"], op["V"], op["block_table"], op["seq_lens"], op["B"],
                            op["Hq"], op["Hkv"], op["D"], op["block_size"], op["max_blocks"], scale)


def _parity(op, scale, S, what):
    got = _gpu(op, scale, S)
    ref = _ref(op, scale)
    rel = oracle.attention_rel(ref, op["seq_lens"], op["Hq"], op["D"])
    ok, rep = oracle.check(got, ref, "bf16", rel=rel)
    assert ok, "%s: %s" % (what, rep)
    return got, ref


CASES = [
    # B, Hq, Hkv, D, seq_lens, block_size
    (1, 1, 1, 64, [1], 1),
    (2, 4, 2, 64, [100, 37], 16),
    (3, 8, 2, 128, [0, 500, 1], 32),
    (1, 16, 4, 256, [1000], 784),
    (2, 8, 1, 256, [3000, 2999], 64),
    (2, 2, 2, 128, [129, 7], 5),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("S", [0, 1, 3, 16, 32])
def test_parity_shapes_and_segments(case, S):
    B, Hq, Hkv, D, lens, bs = CASES[case]
    print("case", CASES[case], "S", S, flush=True)
    op = synth.attention_operands(B, Hq, Hkv, D, lens, bs, seed=50 + case)
    _parity(op, 1.0 / np.sqrt(D), S, "case %d S %d" % (case, S))


def test_more_segments_than_tokens_and_other_scales():
    op = synth.attention_operands(2, 4, 1, 64, [5, 40], 3, seed=60)
    for S, scale in ((64, 0.125), (1024, 1.0), (7, -0.5)):
        print("case S", S, "scale", scale, flush=True)
        _parity(op, scale, S, "S %d scale %g" % (S, scale))


def test_empty_sequences_give_zeros():
    op = synth.attention_operands(3, 4, 2, 128, [0, 10, 0], 8, seed=61)
    got = _gpu(op, 0.1, 4)
    D, Hq = 128, 4
    assert np.all(got[:Hq * D] == 0) and np.all(got[2 * Hq * D:] == 0)
    assert np.any(got[Hq * D:2 * Hq * D] != 0)


def test_lengths_past_the_block_table_are_clamped():
    op = synth.attention_operands(1, 2, 1, 64, [48], 16, seed=62)    # 3 pages
    op2 = dict(op)
    op2["seq_lens"] = np.array([10 ** 6], np.int32)                  # beyond 3 * 16
    got = _gpu(op2, 0.2, 8, max_seq_len=48)
    ref = _ref(op, 0.2)
    ok, rep = oracle.check(got, ref, "bf16", rel=oracle.attention_rel(ref, [48], 2, 64))
    assert ok, rep


@pytest.mark.parametrize("L", [8192, 16384, 32768])
def test_page_head_shape_32_vs_16_segments(L):
    # DCU page section 7: at 16 Q / 4 KV heads, head dim 256, pages of 784,
    # the 32-segment output differs from the 16-segment one by at most
    # 2.44e-4 (max abs) and 1.58e-5 (mean abs); both meet the oracle's bound
    w = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    op = synth.attention_operands(1, w["Hq"], w["Hkv"], w["D"], [L], w["block_size"], seed=w["seed"])
    scale = 1.0 / np.sqrt(w["D"])
    print("case page shape L", L, flush=True)
    g16, ref = _parity(op, scale, 16, "S 16 L %d" % L)
    g32, _ = _parity(op, scale, 32, "S 32 L %d" % L)
    a16 = oracle.decode(g16, "bf16")
    a32 = oracle.decode(g32, "bf16")
    d = np.abs(a32 - a16)
    assert np.all(np.isfinite(a16)) and np.all(np.isfinite(a32))
    assert d.max() <= 2.44e-4 and d.mean() <= 1.58e-5, (d.max(), d.mean())
    # and the automatic choice for this chip
    _parity(op, scale, 0, "automatic L %d" % L)


@pytest.mark.parametrize("kind", ["uniform", "mask"])
@pytest.mark.parametrize("L", [8192, 16384, 32768])
def test_page_head_shape_exact_class(kind, L):
    # DCU page sections 6.3 and 7 (16 Q / 4 KV heads, head dim 256, pages of
    # 784): inputs whose output every correct FP32 implementation returns
    # bit for bit (synth.attention_exact_operands), with the automatic, 16
    # and 32 segments.  One missing, extra or misread token anywhere (a
    # segment or page tail) changes the bits: see the oracle controls.
    from helpers import attention_exact_expected, exact_mismatches
    w = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    op = synth.attention_exact_operands(L, kind)
    scale = 1.0 / np.sqrt(w["D"])
    ref = _ref(op, scale)
    assert np.array_equal(ref.bits, attention_exact_expected(op, w["Hq"], w["D"]))
    for S in (0, 16, 32):
        print("case exact", kind, "L", L, "S", S, flush=True)
        got = _gpu(op, scale, S)
        assert exact_mismatches(got, ref.bits) == 0, (kind, L, S, exact_mismatches(got, ref.bits))


@pytest.mark.parametrize("L", [8192, 16384, 32768])
def test_page_head_shape_automatic_vs_16_and_32_segments(L):
    # the automatic segment count against the page's 16 and 32 with the
    # page's section 7 bound (max abs <= 2.44e-4, mean abs <= 1.58e-5)
    w = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    op = synth.attention_operands(1, w["Hq"], w["Hkv"], w["D"], [L], w["block_size"], seed=w["seed"])
    scale = 1.0 / np.sqrt(w["D"])
    print("case auto vs 16/32 L", L, flush=True)
    auto = oracle.decode(_gpu(op, scale, 0), "bf16")
    for S in (16, 32):
        other = oracle.decode(_gpu(op, scale, S), "bf16")
        d = np.abs(auto - other)
        assert d.max() <= 2.44e-4 and d.mean() <= 1.58e-5, (S, d.max(), d.mean())



def test_one_workspace_many_shapes():
    # one workspace serves calls of different shapes and segment counts in
    # a row; every result meets the oracle's bound
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    cases = [(2, 8, 2, 128, [300, 77], 16, 1), (1, 16, 4, 256, [2000], 784, 16),
             (3, 4, 4, 64, [50, 0, 129], 8, 17), (1, 16, 4, 256, [4000], 784, 128),
             (2, 8, 1, 128, [999, 1], 32, 1024), (1, 2, 2, 64, [5], 4, 40)]
    for i, (B, Hq, Hkv, D, lens, bs, S) in enumerate(cases):
        print("case shared workspace", i, B, Hq, Hkv, D, lens, bs, S, flush=True)
        op = synth.attention_operands(B, Hq, Hkv, D, lens, bs, seed=80 + i)
        scale = 1.0 / np.sqrt(D)
        dQ, dK, dV = dev(op["Q"]), dev(op["K"]), dev(op["V"])
        bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
        out = torch.empty(B * Hq * D, dtype=torch.int16, device="cuda")
        assert L.migemm_attention_workspace_bytes(B, Hq, D, S) <= ws.numel()
        code = L.attention_decode_bf16(dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), bt.data_ptr(),
                                       sl.data_ptr(), out.data_ptr(), B, Hq, Hkv, D, op["block_size"],
                                       op["max_blocks"], op["num_blocks"], scale, max(lens), S,
                                       ws.data_ptr(), ws.numel(), None)
        assert code == 0, code
        torch.cuda.synchronize()
        ref = _ref(op, scale)
        ok, rep = oracle.check(host(out), ref, "bf16", rel=oracle.attention_rel(ref, op["seq_lens"], Hq, D))
        assert ok, (i, rep)


def test_graph_replays_match_eager():
    # the call (segment and merge kernels) captured in a HIP graph and
    # replayed several times, with eager work in between: every replay
    # equals the eager result bit for bit
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    w = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    op = synth.attention_operands(1, w["Hq"], w["Hkv"], w["D"], [8192], w["block_size"], seed=w["seed"])
    scale = 1.0 / np.sqrt(w["D"])
    dQ, dK, dV = dev(op["Q"]), dev(op["K"]), dev(op["V"])
    bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
    S = L.migemm_attention_segments(1, w["Hq"], w["Hkv"], 8192)
    ws = torch.empty(L.migemm_attention_workspace_bytes(1, w["Hq"], w["D"], S), dtype=torch.uint8, device="cuda")
    out = torch.empty(w["Hq"] * w["D"], dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()

    def call():
        return L.attention_decode_bf16(dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), bt.data_ptr(),
                                       sl.data_ptr(), out.data_ptr(), 1, w["Hq"], w["Hkv"], w["D"],
                                       op["block_size"], op["max_blocks"], op["num_blocks"], scale, 8192, S,
                                       ws.data_ptr(), ws.numel(), s.cuda_stream)
    with torch.cuda.stream(s):
        assert call() == 0
    s.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        assert call() == 0
    for r in range(4):
        print("case graph replay", r, flush=True)
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        _ = (dQ.float() * 2).sum().item()                # eager work between replays
