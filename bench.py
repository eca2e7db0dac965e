"""Benchmark of the DiT flash self-attention forward on one MI355X.

Default: the BF16 path at the FLUX-1024^2 shape (B=1, H=24, S=4608, D=128),
attention TFLOPS = 4 * B * H * S^2 * D / time, inputs resident in HBM.
A step is one attn_fwd_bf16 call; K steps are timed with HIP events recorded
on the stream the kernel is launched on (defaults: 200 warmup steps, then 1000
timed ones, about a quarter second: long enough for steady clocks).  The same line also reports the Sage
mode at that shape ("sage" = prepare + attention, "sage_core" = attention on
prepared tensors), the roofline of the dominant kernel and the CPU oracle's
throughput on a bounded row sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --copy-calibration     # plain copy for PMC byte scaling
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "int8": 5033.2}  # 256 CU x 2.4 GHz x 4096 / 8192 per clk
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {"attn_fwd_bf16": ["image_dit_amd/csrc/attn_bf16.hip", "image_dit_amd/csrc/common.hpp"]}


def kernel_sha(name):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, workload):
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.md" % (name, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_sha(name):
        return None
    return float(m_b.group(1))


def time_launches(fn, stream, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def cpu_baseline(w, q, k, v, target_s=20.0):
    """The oracle's exact fp64 attention on a bounded sample of query rows."""
    import oracle
    from image_dit_amd import synth
    rows = synth.sample_rows(w.B, w.S, w.H, n=256, seed=w.seed + 2)
    t0 = time.perf_counter()
    oracle.attn_rows(q, k, v, w.scale, rows=rows)
    t_small = time.perf_counter() - t0
    n = int(min(w.B * w.H * w.S, max(256, 256 * target_s / max(t_small, 1e-3))))
    rows = synth.sample_rows(w.B, w.S, w.H, n=n, seed=w.seed + 2)
    t0 = time.perf_counter()
    oracle.attn_rows(q, k, v, w.scale, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.S * w.D * len(rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d query rows of %s (exact fp64 attention over all %d keys), %.1f s; "
                      "value = 4*S*D*rows / time" % (len(rows), w.name, w.S, dt)}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="flux1024")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sage", action="store_true", help="time the BF16 path only")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the attention of one GPU's heads is the "
              "measured unit (heads shard across GPUs with no exchange); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import image_dit_amd as ia
    from image_dit_amd import cost, synth

    if args.copy_calibration:
        copy_calibration()
        return

    w = synth.WORKLOADS[args.workload]
    q, k, v = synth.workload_qkv(w)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    stream = torch.cuda.Stream()
    flops = cost.attn_flops(w.B, w.H, w.S, w.D)

    def bf16_step():
        ia.attn_fwd_bf16(qd, kd, vd, w.scale, out=out, stream=stream)

    ms = time_launches(bf16_step, stream, args.steps, args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12

    modes = {}
    if not args.no_sage:
        prepared = ia.sage_prepare(qd, kd, vd, w.scale, stream=stream)
        sout = torch.empty_like(qd)

        def prep_step():
            ia.sage_prepare(qd, kd, vd, w.scale, out=prepared, stream=stream)

        def core_step():
            ia.sage_attn_fwd(prepared, w.S, w.H, w.scale, out=sout, stream=stream)

        def sage_step():
            prep_step()
            core_step()

        ms_prep = time_launches(prep_step, stream, args.steps, args.warmup)
        ms_core = time_launches(core_step, stream, args.steps, args.warmup)
        ms_sage = time_launches(sage_step, stream, args.steps, args.warmup)
        peak8 = PEAK_TFLOPS["int8"]
        modes = {
            "sage": {"ms": ms_sage, "tflops": flops / (ms_sage * 1e-3) / 1e12},
            "sage_core": {"ms": ms_core, "tflops": flops / (ms_core * 1e-3) / 1e12,
                          "frac_of_8bit_peak": flops / (ms_core * 1e-3) / 1e12 / peak8},
            "sage_prepare": {"ms": ms_prep,
                             "gbs": cost.sage_prepare_bytes(w.B, w.H, w.S, w.D) / (ms_prep * 1e-3) / 1e9,
                             "frac_of_hbm_peak": cost.sage_prepare_bytes(w.B, w.H, w.S, w.D) / (ms_prep * 1e-3) / 1e9 / PEAK_HBM_GBS},
        }

    traffic = measured_traffic("attn_fwd_bf16", w.name)
    line = {
        "metric": "attention TFLOPS (4*B*H*S^2*D/s) at FLUX/Wan DiT shapes; % of MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn BF16 Q/K/V)",
        "config": {"workload": "%s self-attention, BF16 path" % w.name, "B": w.B, "H": w.H, "S": w.S,
                   "D": w.D, "causal": False},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": tflops / PEAK_TFLOPS["bf16"],
                     "traffic": traffic,
                     "kernel": "attn_fwd_bf16_kernel", "algorithmic_flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": cost.attn_bytes_bf16(w.B, w.H, w.S, w.D)},
        "modes": modes,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
