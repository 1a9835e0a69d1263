"""GPU tests of the boundary's stream contract: calls on a non-null stream are
stream-ordered, the library keeps no state between calls, and a call on a
non-null stream makes no allocation and no synchronization, so it can be
captured into a graph.

Every entry point (GEMM on tiles 16 and auto, the k-major GEMM, the GEMV at
one and sixteen tokens, the FP8 GEMM on tile 17, split-K with its reduce, and
split-KV decode attention with its merge) first runs alone on the null stream
(synchronous); those results are checked against the oracle where cheap and
serve as the reference. Then all of them run overlapped on three streams, and
as one captured graph replayed three times with eager fills and
synchronizations between the replays. Every result must equal the reference
bit for bit: each kernel's arithmetic order is fixed by its launch, so any
difference would be shared state or a broken ordering."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, dev, host

pytestmark = pytest.mark.gpu


def _jobs():
    """(name, output tensor size, run(stream_handle, out_ptr) -> code, oracle check or None)"""
    import torch
    from bf16_gemm_decode_amd import binding
    L = binding.lib()
    keep = []                                   # device inputs and workspaces, alive with the jobs
    jobs = []

    def put(bits):
        t = dev(bits)
        keep.append(t)
        return t.data_ptr()

    # GEMM, FP16, ping-pong tile; BF16 on the automatic tile
    M, N, K = 520, 600, 332
    A, B = synth.gemm_operands(M, N, K, "f16", ("uniform", 1.0, 1.0), seed=71)
    pa, pb = put(A), put(B)
    jobs.append(("gemm f16 tile 16", M * N,
                 lambda s, c, pa=pa, pb=pb: binding.gemm_ex_ptr(binding.F16, pa, pb, c, 520, 600, 332, 16, 0, 1, s),
                 lambda got, A=A, B=B: assert_parity(got, oracle.gemm(A, B, 520, 600, 332, "f16"), "f16", "gemm")))
    A2, B2 = synth.gemm_operands(1000, 700, 1100, "bf16", ("normal", 1.0, 1.0), seed=72)
    pa2, pb2 = put(A2), put(B2)
    jobs.append(("gemm bf16 auto", 1000 * 700,
                 lambda s, c: binding.gemm_ex_ptr(binding.BF16, pa2, pb2, c, 1000, 700, 1100, 0, 0, 1, s), None))
    # k-major GEMM
    At, Bt = synth.gemm_operands(300, 200, 272, "bf16", ("normal", 1.0, 1.0), seed=73)
    pat, pbt = put(At), put(Bt)
    jobs.append(("gemm_tn bf16", 300 * 200,
                 lambda s, c: binding.gemm_tn_ex_ptr(binding.BF16, pat, pbt, c, 300, 200, 272, 0, 0, 1, s), None))
    # GEMV, one and sixteen tokens
    for n in (1, 16):
        W, X = synth.gemv_operands(4099, 1032, n, seed=74 + n)
        pw, px = put(W), put(X)
        chk = (lambda got, W=W, X=X: assert_parity(got, oracle.gemv(W, X, 4099, 1032, 1), "bf16", "gemv")) \
            if n == 1 else None
        jobs.append(("gemv n=%d" % n, n * 4099,
                     lambda s, c, pw=pw, px=px, n=n: binding.gemv_bf16_ex_ptr(pw, px, c, 4099, 1032, n, 0, s), chk))
    # FP8 GEMM on the double-rate tile
    Aq, Bq = synth.q8_operands(520, 264, 1024, "f8e4m3", seed=76)
    tq = [torch.from_numpy(Aq).cuda(), torch.from_numpy(Bq).cuda()]
    keep.extend(tq)
    jobs.append(("fp8 tile 17", 520 * 264,
                 lambda s, c: L.gemm_tn_q_ex(binding.F8E4M3, tq[0].data_ptr(), tq[1].data_ptr(), c, 520, 264, 1024,
                                             0.75, 17, 0, 1, s), None))
    # split-K: each call its own workspace
    As, Bs = synth.gemm_operands(520, 264, 2048, "f16", ("uniform", 1.0, 1.0), seed=77)
    pas, pbs = put(As), put(Bs)
    wsb = L.migemm_splitk_workspace_bytes(520, 264, 4)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    keep.append(ws)
    jobs.append(("split-K", 520 * 264,
                 lambda s, c: L.gemm_splitk_ex(0, 0, pas, pbs, c, 520, 264, 2048, 4, 10, 0, 1, ws.data_ptr(), wsb,
                                               s), None))
    # decode attention, 16 segments
    op = synth.attention_operands(2, 8, 1, 256, [3000, 2999], 64, seed=78)
    dQ, dK, dV = dev(op["Q"]), dev(op["K"]), dev(op["V"])
    bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
    need = L.migemm_attention_workspace_bytes(2, 8, 256, 16)
    wsa = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    keep.extend([dQ, dK, dV, bt, sl, wsa])
    jobs.append(("attention", 2 * 8 * 256,
                 lambda s, c: L.attention_decode_bf16(dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), bt.data_ptr(),
                                                      sl.data_ptr(), c, 2, 8, 1, 256, op["block_size"],
                                                      op["max_blocks"], op["num_blocks"], 0.0625, 3000, 16,
                                                      wsa.data_ptr(), wsa.numel(), s), None))
    return jobs, keep


def _outputs(jobs):
    import torch
    return [torch.full((size,), -1, dtype=torch.int16, device="cuda") for _, size, _, _ in jobs]


def test_overlapped_streams_and_graph_replays():
    import torch
    jobs, keep = _jobs()
    torch.cuda.synchronize()
    # alone, synchronous (null stream)
    ref = _outputs(jobs)
    torch.cuda.synchronize()
    for (name, _, run, chk), out in zip(jobs, ref):
        print("case serial", name, flush=True)
        assert run(None, out.data_ptr()) == 0, name
        if chk is not None:
            chk(host(out))
    torch.cuda.synchronize()

    # overlapped on three streams, twice, no synchronization in between
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = [_outputs(jobs) for _ in range(2)]
    torch.cuda.synchronize()
    print("case overlapped streams", flush=True)
    for rep in range(2):
        for i, (name, _, run, _) in enumerate(jobs):
            assert run(streams[(i + rep) % 3].cuda_stream, outs[rep][i].data_ptr()) == 0, name
    torch.cuda.synchronize()
    for rep in range(2):
        for (name, _, _, _), got, want in zip(jobs, outs[rep], ref):
            assert torch.equal(got, want), "overlapped %s (pass %d) differs" % (name, rep)

    # captured once, replayed three times
    static = _outputs(jobs)
    torch.cuda.synchronize()
    print("case graph capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        for (name, _, run, _), out in zip(jobs, static):
            assert run(s, out.data_ptr()) == 0, name
    torch.cuda.synchronize()
    for rep in range(3):
        print("case graph replay", rep, flush=True)
        for t in static:
            t.fill_(-1)                                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, _, _, _), got, want in zip(jobs, static, ref):
            assert torch.equal(got, want), "graph replay %d: %s differs" % (rep, name)
    del g, keep
    torch.cuda.synchronize()
