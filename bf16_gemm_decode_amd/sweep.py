"""Time GEMM tile configurations and grouped-ordering widths on one shape.

Usage (on a GPU machine):
  python -m bf16_gemm_decode_amd.sweep --shape 4096,34816,5120 --dtype bf16 \
      --tiles 1,2,3 --group-m 1,4,8,16 --xcd 1 [--tn]

Prints one JSON line per configuration: average kernel time over --reps
launches (HIP events on the launch stream) and TFLOP/s = 2*M*N*K / time,
with the fraction of the 2.5 PFLOP/s dense FP16/BF16 MFMA peak.  Inputs are
seeded random data (normal(0,1) for A, normal(0,0.02) for B); outputs are not
checked here -- the test suite does that.
"""
import argparse
import json

from . import binding, roofline


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--shape", default="8192,8192,16384")
    p.add_argument("--dtype", default="f16", choices=["f16", "bf16"])
    p.add_argument("--tiles", default="1")
    p.add_argument("--group-m", default="8")
    p.add_argument("--xcd", default="1")
    p.add_argument("--reps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--tn", action="store_true",
                   help="time gemm_tn_ex (A supplied k-major) instead of gemm_ex")
    a = p.parse_args(argv)

    import torch
    M, N, K = (int(v) for v in a.shape.split(","))
    dt = torch.float16 if a.dtype == "f16" else torch.bfloat16
    code_dt = binding.F16 if a.dtype == "f16" else binding.BF16
    g = torch.Generator(device="cuda").manual_seed(0)
    A = torch.randn(M * K, generator=g, device="cuda").to(dt)
    B = (torch.randn(K * N, generator=g, device="cuda") * 0.02).to(dt)
    C = torch.empty(M * N, dtype=dt, device="cuda")
    torch.cuda.synchronize()   # inputs are drawn on the default stream; the launches go to s
    s = torch.cuda.Stream()
    L = binding.lib()
    flop = roofline.gemm_flop(M, N, K)
    peak = roofline.MI355X["mfma_f16_tflops"]
    for tile in (int(t) for t in a.tiles.split(",")):
        for gm in (int(v) for v in a.group_m.split(",")):
            for xcd in (int(v) for v in a.xcd.split(",")):
                fn = L.gemm_tn_ex if a.tn else L.gemm_ex

                def run():
                    return fn(code_dt, A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                              tile, gm, xcd, s.cuda_stream)
                rc = run()
                if rc != 0:
                    print(json.dumps({"tile": tile, "group_m": gm, "xcd_remap": xcd, "error": rc}))
                    continue
                for _ in range(a.warmup):
                    run()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(s)
                for _ in range(a.reps):
                    run()
                e1.record(s)
                s.synchronize()
                t = e0.elapsed_time(e1) / 1e3 / a.reps
                _, plan = binding.gemm_plan(code_dt, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                                            M, N, K, tile, gm, xcd, a_kmajor=a.tn)
                tf = flop / t / 1e12
                print(json.dumps({"shape": [M, N, K], "dtype": a.dtype, "a_layout": "k-major" if a.tn else "m-major",
                                  "tile": tile,
                                  "tile_mnk": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
                                  "group_m": plan["group_m"], "xcd_remap": xcd,
                                  "grid": plan["grid"], "ms": round(t * 1e3, 4),
                                  "tflops": round(tf, 1), "frac_peak": round(tf / peak, 4)}),
                      flush=True)


if __name__ == "__main__":
    main()
