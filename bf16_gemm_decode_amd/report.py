"""Per-workload timing report of the hot path on one GPU.

Measures every workload of the method's test matrix with the seeded synthetic
inputs of `synth` (the same recipes the parity tests use):

  * 512^3 FP16 GEMM (launch-latency bound), the 8192 x 8192 x 16384 FP16 GEMM,
    the ragged 5000 x 3000 x 4100 BF16 GEMM;
  * the decode GEMV Y = X W^T (W 34816 x 5120 BF16) at n = 1, 4, 16 tokens,
    and the same product at n = 16 .. 256 through gemm_tn_bf16 (MFMA);
  * the prefill GEMM 4096 x 34816 x 5120 BF16 over the grouped-ordering width
    GROUP_M in {1, 4, 8, 16} x the tiles that fit it, in both of its layouts
    (column-major X through gemm_ex, row-major X and W through gemm_tn_ex);
  * the streaming-read probe;
  * split-KV decode attention at 16 query / 4 KV heads, head dim 256, pages
    of 784 tokens, for 1 sequence of 8K, 16K, 32K tokens and batches of 8 x 8K
    and 32 x 4K, at 16, 32 and the automatic number of segments (the caches
    rotate over disjoint page sets of > 600 MB so they do not stay in the
    MALL).

Times are kernel durations from HIP events around back-to-back launches on
one stream (median and minimum of `--rounds` rounds).  TFLOP/s use the
algorithmic 2*M*N*K, GB/s the algorithmic bytes; "util" is the fraction of
the 2.5 PFLOP/s dense FP16/BF16 MFMA peak (of 8 TB/s for the GEMV).  Outputs
are not checked here: the test suite does that.

Usage (GPU):  python -m bf16_gemm_decode_amd.report [--out report.md] [--rounds 5]
"""
import argparse
import json
import os
import subprocess
import sys

from . import binding, roofline as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _timer(torch, stream, fn, launches, rounds):
    for _ in range(2):
        fn(0)
    stream.synchronize()
    ts = []
    for r in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            code = fn(i)
            assert code == 0, code
        e1.record(stream)
        stream.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3 / launches)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def _dev(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _smi():
    """Clock / power / temperature as printed by amd-smi, if it runs here."""
    for cmd in (["amd-smi", "metric", "-g", "0", "--clock", "--power", "--temperature"],
                ["rocm-smi", "--showclocks", "--showpower", "--showtemp"]):
        try:
            out = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if out.returncode == 0 and out.stdout.strip():
            return "$ " + " ".join(cmd) + "\n" + out.stdout.strip()
    return "(no amd-smi / rocm-smi output available)"


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--out", default=None, help="write a markdown summary here")
    p.add_argument("--rounds", type=int, default=5)
    p.add_argument("--skip-prefill-grid", action="store_true")
    p.add_argument("--sections", default="gemm,decode,prefill,attention,q8,splitk",
                   help="comma list of gemm, decode, prefill, attention, q8, splitk")
    p.add_argument("--decode-tiles", default="0",
                   help="gemm_tn tiles to time for the decode batches (0 = automatic)")
    p.add_argument("--attn-segments", default="16,32,0",
                   help="segment counts to time for the attention (0 = automatic)")
    a = p.parse_args(argv)

    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import synth

    torch.cuda.set_device(0)
    s = torch.cuda.Stream()
    h = s.cuda_stream
    L = binding.lib()
    rows = []
    peak = rf.MI355X["mfma_f16_tflops"]
    hbm = rf.MI355X["hbm_GBps"]
    smi_before = _smi()

    def gemm_row(name, code_dt, dA, dB, dC, M, N, K, tile=0, gm=0, tn=False, launches=None):
        fn_c = L.gemm_tn_ex if tn else L.gemm_ex
        launches = launches or max(3, min(200, int(2e-3 / max(rf.gemm_flop(M, N, K) / 1.0e15, 1e-6))))
        med, mn = _timer(torch, s, lambda i: fn_c(code_dt, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(),
                                                  M, N, K, tile, gm, 1, h), launches, a.rounds)
        _, plan = binding.gemm_plan(code_dt, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K,
                                    tile, gm, 1, a_kmajor=tn)
        tf = rf.gemm_flop(M, N, K) / med / 1e12
        r = {"workload": name, "M": M, "N": N, "K": K, "layout": "A k-major" if tn else "column-major",
             "tile": plan["tile"], "tile_mnk": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
             "group_m": plan["group_m"], "grid": plan["grid"], "launches": launches,
             "median_us": round(med * 1e6, 2), "min_us": round(mn * 1e6, 2),
             "tflops": round(tf, 1), "util": round(tf / peak, 4)}
        rows.append(r)
        print(json.dumps(r), flush=True)
        return r

    def operands(name):
        w = synth.WORKLOADS[name]
        A, B = synth.workload_operands(name)
        code_dt = binding.F16 if w["fmt"] == "f16" else binding.BF16
        return w, code_dt, _dev(torch, A), _dev(torch, B)

    sections = a.sections.split(",")
    # --- GEMMs ------------------------------------------------------------
    for name in (("gemm_512_f16", "gemm_8192x8192x16384_f16", "gemm_5000x3000x4100_bf16")
                 if "gemm" in sections else ()):
        w, code_dt, dA, dB = operands(name)
        dC = torch.empty(w["M"] * w["N"], dtype=torch.int16, device="cuda")
        gemm_row(name, code_dt, dA, dB, dC, w["M"], w["N"], w["K"])
        del dA, dB, dC

    # --- decode GEMV and its batched MFMA form ------------------------------
    wv = synth.WORKLOADS["gemv_34816x5120_bf16"]
    if "decode" not in sections:
        wv = None
    M, K = (wv["M"], wv["K"]) if wv else (0, 0)
    W, _ = synth.gemv_operands(M, K, 1, seed=wv["seed"]) if wv else (None, None)
    copies = [_dev(torch, W)] if wv else []
    for _ in range(3 if wv else 0):
        copies.append(copies[0].clone())        # 4 x 356.5 MB: W cannot stay in the MALL
    probe_buf = torch.empty((4 << 30) // 4, dtype=torch.int32, device="cuda")
    probe_buf.fill_(7)
    sink = torch.zeros(binding.hbm_read_sink_words(), dtype=torch.int32, device="cuda")
    pmed, pmin = _timer(torch, s, lambda i: L.migemm_hbm_read(probe_buf.data_ptr(), 4 << 30,
                                                               sink.data_ptr(), h), 5, a.rounds)
    probe = (4 << 30) / pmed / 1e9
    rows.append({"workload": "hbm_read probe (4 GiB)", "median_us": round(pmed * 1e6, 1),
                 "GBps": round(probe, 1), "util": round(probe / hbm, 4)})
    print(json.dumps(rows[-1]), flush=True)
    if wv:
        wb = M * K * 2          # one copy of W; launches rotate over 4 disjoint regions like the GEMV
        wmed, wmin = _timer(torch, s, lambda i: L.migemm_hbm_read(probe_buf.data_ptr() + (i % 4) * wb, wb,
                                                                   sink.data_ptr(), h), 5, a.rounds)
        rows.append({"workload": "hbm_read probe (W's %.1f MB)" % (wb / 1e6), "median_us": round(wmed * 1e6, 1),
                     "min_us": round(wmin * 1e6, 1), "GBps": round(wb / wmed / 1e9, 1),
                     "util": round(wb / wmed / 1e9 / hbm, 4)})
        print(json.dumps(rows[-1]), flush=True)
    del probe_buf
    for n in ((1, 2, 3, 4, 8, 16) if wv else ()):
        _, X = synth.gemv_operands(M, K, n, seed=wv["seed"])
        dX = _dev(torch, X)
        dY = torch.empty(n * M, dtype=torch.int16, device="cuda")
        # rows_per_block 0: the automatic path; 2: the row-blocked vector kernel
        for rpb, path in ((0, "gemv_bf16 (automatic)"), (2, "gemv_bf16_ex vector kernel, rows_per_block 2")):
            med, mn = _timer(torch, s, lambda i: L.gemv_bf16_ex(copies[i % 4].data_ptr(), dX.data_ptr(),
                                                                 dY.data_ptr(), M, K, n, rpb, h),
                             40, a.rounds)
            gb = rf.gemv_bytes(M, K, n) / med / 1e9
            r = {"workload": "gemv_34816x5120_bf16: " + path, "n": n, "median_us": round(med * 1e6, 2),
                 "min_us": round(mn * 1e6, 2), "GBps": round(gb, 1), "util": round(gb / hbm, 4),
                 "frac_of_probe": round(gb / probe, 4)}
            rows.append(r)
            print(json.dumps(r), flush=True)
    # the DCU page's section 6.2 knob: output rows of W per workgroup of the
    # vector kernel, one token
    _, X1 = synth.gemv_operands(M, K, 1, seed=wv["seed"]) if wv else (None, None)
    dX1 = _dev(torch, X1) if wv else None
    dY1 = torch.empty(M, dtype=torch.int16, device="cuda") if wv else None
    for rpb in ((2, 4, 8, 16, 32) if wv else ()):
        med, mn = _timer(torch, s, lambda i: L.gemv_bf16_ex(copies[i % 4].data_ptr(), dX1.data_ptr(),
                                                             dY1.data_ptr(), M, K, 1, rpb, h), 40, a.rounds)
        gb = rf.gemv_bytes(M, K, 1) / med / 1e9
        r = {"workload": "gemv_34816x5120_bf16: rows_per_block sweep (vector kernel)", "n": 1,
             "rows_per_block": rpb, "median_us": round(med * 1e6, 2), "min_us": round(mn * 1e6, 2),
             "GBps": round(gb, 1), "util": round(gb / hbm, 4), "frac_of_probe": round(gb / probe, 4)}
        rows.append(r)
        print(json.dumps(r), flush=True)
    for n in ((4, 8, 16, 32, 64, 128, 256) if wv else ()):
        _, X = synth.gemv_operands(M, K, n, seed=wv["seed"])
        dX = _dev(torch, X)
        dY = torch.empty(n * M, dtype=torch.int16, device="cuda")
        for tile in (int(t) for t in a.decode_tiles.split(",")):
            if binding.gemm_plan(binding.BF16, copies[0].data_ptr(), dX.data_ptr(), dY.data_ptr(),
                                 M, n, K, tile, 0, 1, a_kmajor=True)[0] != 0:
                continue
            med, mn = _timer(torch, s, lambda i: L.gemm_tn_ex(binding.BF16, copies[i % 4].data_ptr(),
                                                               dX.data_ptr(), dY.data_ptr(), M, n, K,
                                                               tile, 0, 1, h), 20, a.rounds)
            gb = rf.gemv_bytes(M, K, n) / med / 1e9
            tf = rf.gemm_flop(M, n, K) / med / 1e12
            _, plan = binding.gemm_plan(binding.BF16, copies[0].data_ptr(), dX.data_ptr(),
                                        dY.data_ptr(), M, n, K, tile, 0, 1, a_kmajor=True)
            r = {"workload": "decode batch Y = X W^T via gemm_tn_bf16", "n": n, "tile": plan["tile"],
                 "tile_mnk": [plan["tile_m"], plan["tile_n"], plan["tile_k"]], "grid": plan["grid"],
                 "median_us": round(med * 1e6, 2), "min_us": round(mn * 1e6, 2), "GBps": round(gb, 1),
                 "util": round(gb / hbm, 4), "frac_of_probe": round(gb / probe, 4), "tflops": round(tf, 1)}
            rows.append(r)
            print(json.dumps(r), flush=True)
    del copies

    # --- prefill: GROUP_M x tile ------------------------------------------
    if not a.skip_prefill_grid and "prefill" in sections:
        w, code_dt, dA, dB = operands("prefill_4096x34816x5120_bf16")
        Mp, Np, Kp = w["M"], w["N"], w["K"]
        dC = torch.empty(Mp * Np, dtype=torch.int16, device="cuda")
        for tile in (16, 10, 9, 2, 3):
            for gm in (1, 4, 8, 16):
                gemm_row("prefill_4096x34816x5120_bf16", code_dt, dA, dB, dC, Mp, Np, Kp, tile, gm,
                         launches=10)
        # row-major X [4096, 5120] and W [34816, 5120] as gemm_tn(At = W, B = X): Y row-major
        At = dB                                           # W row-major: B(k,n) = W[n][k]
        Xr = dA.view(Kp, Mp).t().contiguous().view(-1)   # X row-major [4096, 5120]
        Y = torch.empty(Mp * Np, dtype=torch.int16, device="cuda")
        for tile in (10, 7, 9):
            for gm in (1, 4, 8, 16):
                gemm_row("prefill_4096x34816x5120_bf16 (Y = X W^T, row-major)", code_dt, At, Xr, Y,
                         Np, Mp, Kp, tile, gm, tn=True, launches=10)

    # --- decode attention over the paged cache ------------------------------
    wa = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]
    for B, Lq in (((1, 8192), (1, 16384), (1, 32768), (8, 8192), (32, 4096))
                  if "attention" in sections else ()):
        Hq, Hkv, D, bs = wa["Hq"], wa["Hkv"], wa["D"], wa["block_size"]
        per = 2 * 2 * Lq * Hkv * D                      # KV bytes of one sequence
        copies = max(1, -(-(600 << 20) // (per * B)))    # > 2x the MALL across rotations
        op = synth.attention_operands(B * copies, Hq, Hkv, D, [Lq] * (B * copies), bs,
                                      seed=wa["seed"])
        dQ, dK, dV = _dev(torch, op["Q"]), _dev(torch, op["K"]), _dev(torch, op["V"])
        bt = torch.from_numpy(np.ascontiguousarray(op["block_table"], np.int32)).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(op["seq_lens"], np.int32)).cuda()
        out = torch.empty(B * copies * Hq * D, dtype=torch.int16, device="cuda")
        mb = op["max_blocks"]
        nbytes = rf.attention_bytes([Lq] * B, Hq, Hkv, D, bs)
        for S in (int(x) for x in a.attn_segments.split(",")):
            segs = S or L.migemm_attention_segments(B, Hq, Hkv, Lq)
            wsb = L.migemm_attention_workspace_bytes(B, Hq, D, segs)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

            def call(i, S=S, ws=ws, wsb=wsb):
                c = i % copies                           # sequences c*B .. c*B+B-1
                return L.attention_decode_bf16(
                    dQ.data_ptr() + c * B * Hq * D * 2, dK.data_ptr(), dV.data_ptr(),
                    bt.data_ptr() + c * B * mb * 4, sl.data_ptr() + c * B * 4,
                    out.data_ptr() + c * B * Hq * D * 2, B, Hq, Hkv, D, bs, mb, op["num_blocks"],
                    1.0 / np.sqrt(D), Lq, S, ws.data_ptr(), wsb, h)
            med, mn = _timer(torch, s, call, 40, a.rounds)
            gb = nbytes / med / 1e9
            r = {"workload": "attention_decode_16q4kv_d256_bf16 (page 784)", "B": B, "L": Lq,
                 "segments": segs, "requested": S, "median_us": round(med * 1e6, 2),
                 "min_us": round(mn * 1e6, 2), "GBps": round(gb, 1), "util": round(gb / hbm, 4),
                 "frac_of_probe": round(gb / probe, 4),
                 "workspace_bytes": wsb}
            rows.append(r)
            print(json.dumps(r), flush=True)
        del dQ, dK, dV, op

    # --- 8-bit GEMMs (k-major A) at the headline size ---------------------
    if "q8" in sections:
        Mq, Nq, Kq = 8192, 8192, 16384
        g = torch.Generator(device="cuda")
        g.manual_seed(11)

        def codes(n, fmt):
            c = torch.randint(0, 256, (n,), dtype=torch.int32, device="cuda", generator=g)
            if fmt == binding.F8E4M3:
                c = torch.where((c & 0x7F) == 0x7F, c ^ 1, c)      # no NaN codes
            elif fmt == binding.F8E5M2:
                c = torch.where((c & 0x7C) == 0x7C, c & ~0x40, c)  # no inf / NaN codes
            return c.to(torch.uint8)
        dC = torch.empty(Mq * Nq, dtype=torch.int16, device="cuda")
        for q, qname, pk in ((binding.F8E4M3, "fp8 e4m3", rf.MI355X["mfma_fp8_tflops"]),
                             (binding.F8E5M2, "fp8 e5m2", rf.MI355X["mfma_fp8_tflops"]),
                             (binding.I8, "int8", rf.MI355X["mfma_int8_tops"])):
            dA, dB = codes(Mq * Kq, q), codes(Nq * Kq, q)
            # the automatic tile; for FP8 also tile 10 (the half-rate MFMA) beside it
            for qtile in ((0, 10) if q != binding.I8 else (0,)):
                med, mn = _timer(torch, s, lambda i: L.gemm_tn_q_ex(q, dA.data_ptr(), dB.data_ptr(),
                                                                     dC.data_ptr(), Mq, Nq, Kq, 1.0, qtile,
                                                                     0, 1, h), 10, a.rounds)
                _, plan = binding.gemm_plan(q, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), Mq, Nq, Kq,
                                            qtile, a_kmajor=True)
                tf = rf.gemm_flop(Mq, Nq, Kq) / med / 1e12
                r = {"workload": "gemm_tn %s 8192x8192x16384 (BF16 out)" % qname, "M": Mq, "N": Nq,
                     "K": Kq, "layout": "A k-major", "tile": plan["tile"],
                     "tile_mnk": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
                     "group_m": plan["group_m"], "median_us": round(med * 1e6, 2),
                     "min_us": round(mn * 1e6, 2), "tflops": round(tf, 1), "util": round(tf / pk, 4)}
                rows.append(r)
                print(json.dumps(r), flush=True)
            del dA, dB
        # the BF16 kernel on the same layout, for comparison
        dA = torch.randn(Mq * Kq, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
        dB = torch.randn(Nq * Kq, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
        gemm_row("gemm_tn bf16 8192x8192x16384 (comparison)", binding.BF16, dA, dB, dC, Mq, Nq,
                 Kq, tn=True, launches=10)
        del dA, dB, dC

    # --- split-K on shapes whose tiles do not fill the chip -----------------
    if "splitk" in sections:
        gk = torch.Generator(device="cuda")
        gk.manual_seed(13)
        ws = torch.empty(1 << 28, dtype=torch.float32, device="cuda")          # 1 GiB
        for (Ms, Ns, Ks) in ((1024, 1024, 65536), (2048, 2048, 65536), (2048, 2048, 16384),
                             (4096, 1024, 32768), (8192, 1024, 16384), (512, 512, 131072)):
            dA = torch.randn(Ms * Ks, device="cuda", generator=gk).to(torch.bfloat16).view(torch.int16)
            dB = torch.randn(Ks * Ns, device="cuda", generator=gk).to(torch.bfloat16).view(torch.int16)
            dC = torch.empty(Ms * Ns, dtype=torch.int16, device="cuda")
            gemm_row("gemm_ex (no split)", binding.BF16, dA, dB, dC, Ms, Ns, Ks, launches=10)
            med, mn = _timer(torch, s, lambda i: L.gemm_splitk_ex(binding.BF16, 0, dA.data_ptr(), dB.data_ptr(),
                                                                   dC.data_ptr(), Ms, Ns, Ks, 0, 0, 0, 1,
                                                                   ws.data_ptr(), ws.numel() * 4, h),
                             10, a.rounds)
            tf = rf.gemm_flop(Ms, Ns, Ks) / med / 1e12
            r = {"workload": "gemm_splitk_ex (automatic: %d slices)" % L.migemm_splitk_splits(binding.BF16, 0, Ms, Ns, Ks),
                 "M": Ms, "N": Ns, "K": Ks, "layout": "column-major", "median_us": round(med * 1e6, 2),
                 "min_us": round(mn * 1e6, 2), "tflops": round(tf, 1), "util": round(tf / peak, 4)}
            rows.append(r)
            print(json.dumps(r), flush=True)
            del dA, dB, dC
        del ws

    smi_after = _smi()
    if a.out:
        with open(a.out, "w") as f:
            f.write("# Per-workload report\n\n")
            f.write("command: `python -m bf16_gemm_decode_amd.report %s`\n\n"
                    % " ".join(sys.argv[1:] if argv is None else argv))
            f.write("Kernel durations from HIP events around back-to-back launches (median / min of "
                    "%d rounds); util = fraction of the dense peak of the row's type (2.5 PFLOP/s "
                    "FP16/BF16, 5.0 PFLOP/s FP8, 5.0 POP/s INT8) or of 8 TB/s (GEMV, attention, "
                    "probe); for the attention GB/s counts the algorithmic bytes (K and V read once, "
                    "Q, block table, output), the workspace partials not included.\n\n"
                    % a.rounds)
            f.write("| workload | shape / n | layout | tile | GROUP_M | median us | min us | TFLOP/s | GB/s | util | of probe |\n")
            f.write("|---|---|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                shape = ("%dx%dx%d" % (r["M"], r["N"], r["K"]) if "M" in r else
                         "n=%d rows_per_block=%d" % (r["n"], r["rows_per_block"]) if "rows_per_block" in r else
                         "n=%d" % r["n"] if "n" in r else
                         "B=%d L=%d S=%d" % (r["B"], r["L"], r["segments"]) if "L" in r else "")
                tile = ("%d (%s)" % (r["tile"], "x".join(str(v) for v in r["tile_mnk"]))
                        if "tile_mnk" in r else str(r.get("tile", "")))
                f.write("| %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |\n" % (
                    r["workload"], shape, r.get("layout", ""), tile, r.get("group_m", ""),
                    r.get("median_us", ""), r.get("min_us", ""), r.get("tflops", ""),
                    r.get("GBps", ""), r.get("util", ""), r.get("frac_of_probe", "")))
            f.write("\n## GPU state\n\nbefore:\n```\n%s\n```\nafter:\n```\n%s\n```\n" % (smi_before, smi_after))
        print("wrote", a.out)


if __name__ == "__main__":
    main()
