"""Benchmark of the DiT flash self-attention forward on one MI355X.

Headline: the BF16 path at the FLUX-1024^2 shape (B=1, H=24, S=4608, D=128),
attention TFLOPS = 4 * B * H * S^2 * D / time, inputs resident in HBM.  A step
is one BF16 attention call (attn_fwd_bf16_ws, which at this shape runs the plain
attn_fwd_bf16 kernel).  W warm-up steps, then exactly K timed steps, timed
with HIP events recorded on the stream the kernel is launched on; events at the
quarter marks give the first- and last-quarter ms per step (the clock regime).

The same JSON line carries one row per (workload, mode) for the DiT shapes:
  bf16       attn_fwd_bf16_ws (the plain attn_fwd_bf16 kernel unless the last round of
             query tiles is split)                vs the BF16 MFMA peak
  sage       sage_prepare + sage_attn_fwd_ws    vs the 8-bit MFMA peak
  sage_core  sage_attn_fwd_ws on prepared tensors (the plain sage_attn_fwd kernel
             unless the last round of query tiles is split)   vs the 8-bit MFMA peak
  prepare    sage_prepare                       vs the HBM peak (algorithmic bytes)
and rows of the path's variants, on a base workload's tensors (the _ws entry points):
  bf16_X, sage_core_X   X = causal (key window (-1, 0)), gqa4 (H_kv = H / 4), text512
                        (cross-attention to 512 tokens); TFLOPS count the visible pairs only
  prepare_xform         sage_prepare_ex with RMSNorm + RoPE (rope_dim 128) fused
  prepare_smoothk       sage_prepare_ex with K smoothing (one more read of K)
Rows are timed first, each for at least --row-ms milliseconds, and the headline
follows the last one with no idle gap (its inputs are made beforehand): the
shader clock drops within a fraction of a second of idling and takes longer
than a short timed loop to recover, so a headline timed after an idle gap
measures the clock ramp, not the kernel.  The FLUX-1024
Sage rows use the K-bias workload of that shape.  Row inputs other than the
headline's are drawn on the GPU from a seeded generator (same distribution).

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--rows all|none|W:M,...]
    python bench.py --only wan720p:bf16,wan720p:sage_core --reps 3   # profiling runs
    python bench.py --copy-calibration     # plain copy for PMC byte scaling
    python bench.py --ceilings             # library GEMM and copy rates (practical ceilings)
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# 256 CU x 2.4 GHz x (4096 BF16 | 8192 FP8/INT8) per CU per clock
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "int8": 5033.2}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "attn_fwd_bf16": ["image_dit_amd/csrc/attn_bf16.hip", "image_dit_amd/csrc/common.hpp"],
    "sage_attn_fwd": ["image_dit_amd/csrc/attn_sage.hip", "image_dit_amd/csrc/common.hpp"],
    "sage_prepare": ["image_dit_amd/csrc/prepare.hip", "image_dit_amd/csrc/common.hpp"],
}
# Variants of the path (cross-attention to text tokens, grouped heads, a causal key window,
# the fused Q/K transform and K smoothing in prepare), each on a base workload's tensors:
# attention variants count only the visible (query, key) pairs, prepare variants their own bytes.
VARIANTS = {
    "causal": dict(window=(-1, 0)),   # bottom-right aligned: query i sees keys 0..i
    "gqa4": dict(hkv_div=4),          # H_kv = H / 4 (the first H / 4 heads of K and V)
    "text512": dict(s_kv=512),        # cross-attention to 512 tokens (the first 512 of K and V)
}
PREP_VARIANTS = {
    "xform": dict(rope_dim=128),      # RMSNorm (seeded weights) + rotate-half RoPE on all 128 channels
    "smoothk": dict(smooth_k=True),   # K's channel mean subtracted before INT8
}
MODES = (("bf16", "sage", "sage_core", "prepare")
         + tuple("%s_%s" % (m, v) for v in VARIANTS for m in ("bf16", "sage_core"))
         + tuple("prepare_%s" % v for v in PREP_VARIANTS))
# largest first; the FLUX-1024 rows last, right before the headline at that shape
DEFAULT_ROWS = ["wan720p:bf16", "wan720p:sage", "wan720p:sage_core", "wan720p:prepare",
                "flux2048:bf16", "flux2048:sage", "flux2048:sage_core", "flux2048:prepare",
                "hunyuan720p:bf16", "hunyuan720p:sage", "hunyuan720p:sage_core", "hunyuan720p:prepare",
                "wan720p:bf16_text512", "wan720p:sage_core_text512", "wan720p:prepare_xform",
                "wan720p:prepare_smoothk",
                "flux2048:bf16_causal", "flux2048:sage_core_causal", "flux2048:bf16_gqa4",
                "flux2048:sage_core_gqa4",
                "flux1024:prepare_xform", "flux1024:prepare_smoothk",
                "flux1024:prepare", "flux1024:sage_core", "flux1024:sage"]


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


def timed(fn, stream, steps, warmup, marks=(0.25, 0.75)):
    """ms per call over `steps` calls after `warmup` untimed ones, plus the ms
    per call of the first and last quarter of the timed calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    cut = sorted({0, steps} | {int(round(steps * m)) for m in marks})
    ev = {i: torch.cuda.Event(enable_timing=True) for i in cut}
    ev[0].record(stream)
    for i in range(steps):
        fn()
        if i + 1 in ev:
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[steps]) / steps
    q1, q3 = cut[1], cut[-2]
    first = ev[0].elapsed_time(ev[q1]) / max(q1, 1)
    last = ev[q3].elapsed_time(ev[steps]) / max(steps - q3, 1)
    return total, first, last


def timed_for(fn, stream, min_ms, min_reps=3):
    """Time `fn` for at least min_ms milliseconds (after two warm-up calls)."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1), 1e-3)
    reps = max(min_reps, int(math.ceil(min_ms / est)))
    ms, _, _ = timed(fn, stream, reps, 0)
    return ms, reps


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


def ceilings(seconds=2.0, n=8192):
    """Sustained throughput of plain library work on this board: hipBLASLt GEMMs through
    torch (BF16 matmul, FP8 e4m3 _scaled_mm, INT8 _int_mm, n x n x n) and a 1 GiB device
    copy, each run back to back for `seconds`.  These are the practical MFMA and HBM
    ceilings under the board's power limit, next to which the kernels' fractions of the
    published peaks are read."""
    import torch
    dev = torch.device("cuda")

    def sustain(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps, t0 = 0, time.perf_counter()
        e0.record()
        while True:
            for _ in range(10):
                fn()
            reps += 10
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > seconds:
                break
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"seconds_each": seconds, "gemm_n": n}
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    ms = sustain(lambda: a @ b)
    out["bf16_gemm_tflops"] = 2.0 * n ** 3 / ms / 1e9
    del a, b
    a8 = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn)
    b8 = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn).t()
    one = torch.ones((), device=dev)
    ms = sustain(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
    out["fp8_gemm_tflops"] = 2.0 * n ** 3 / ms / 1e9
    del a8, b8
    ai = torch.randint(-127, 128, (n, n), device=dev, dtype=torch.int8)
    bi = torch.randint(-127, 128, (n, n), device=dev, dtype=torch.int8)
    ms = sustain(lambda: torch._int_mm(ai, bi))
    out["int8_gemm_tops"] = 2.0 * n ** 3 / ms / 1e9
    del ai, bi
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = sustain(lambda: dst.copy_(src))
    out["copy_gbs"] = 2.0 * (1 << 30) / ms / 1e6  # bytes read + written
    out["peaks"] = {"bf16_tflops": PEAK_TFLOPS["bf16"], "fp8_int8_tflops": PEAK_TFLOPS["fp8"],
                    "hbm_gbs": PEAK_HBM_GBS}
    print(json.dumps(out), flush=True)


class Inputs:
    """Device inputs and output buffers of one workload, made once."""

    def __init__(self, w, dev, qkv=None):
        import torch
        from image_dit_amd import synth
        self.w = w
        if qkv is None:
            qkv = synth.make_qkv_device(w.B, w.S, w.H, dev, w.D, seed=w.seed, k_bias_std=w.k_bias_std)
        self.q, self.k, self.v = (t.to(dev) for t in qkv)
        self.out = torch.empty_like(self.q)
        self._prep = None
        self._var, self._pvar = {}, {}
        import image_dit_amd as ia
        # the BF16 and Sage rows run the _ws entry points: the last, partial round of query tiles
        # is split over every CU where that pays (workspace size > 0), else they are the plain
        # kernels; one workspace serves both (one call at a time)
        self.ws_bytes = max(ia.bf16_workspace_size(w.B, w.S, w.S, w.H, w.H),
                            ia.sage_attn_workspace_size(w.B, w.S, w.S, w.H, w.H))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev) if self.ws_bytes else None

    def prepared(self, stream):
        import image_dit_amd as ia
        if self._prep is None:
            self._prep = ia.sage_prepare(self.q, self.k, self.v, self.w.scale, stream=stream)
        return self._prep

    def variant(self, name, stream):
        """Tensors of an attention variant: (k, v, prepared, window, H_kv, S_kv, workspace)."""
        import torch
        import image_dit_amd as ia
        if name not in self._var:
            spec, w = VARIANTS[name], self.w
            window = spec.get("window", (-1, -1))
            H_kv = w.H // spec.get("hkv_div", 1)
            S_kv = spec.get("s_kv", w.S)
            if H_kv == w.H and S_kv == w.S:
                k, v, prep = self.k, self.v, self.prepared(stream)
            else:
                k = self.k[:, :S_kv, :H_kv].contiguous()
                v = self.v[:, :S_kv, :H_kv].contiguous()
                prep = ia.sage_prepare_ex(self.q, k, v, w.scale, stream=stream)
            nb = max(ia.bf16_workspace_size(w.B, w.S, S_kv, w.H, H_kv, window),
                     ia.sage_attn_workspace_size(w.B, w.S, S_kv, w.H, H_kv, window))
            ws = torch.zeros(nb, dtype=torch.uint8, device=self.q.device) if nb else None
            self._var[name] = (k, v, prep, window, H_kv, S_kv, ws)
        return self._var[name]

    def prep_variant(self, name):
        """Arguments of a prepare variant (and its own outputs, so the base prepared tensors
        stay as they are)."""
        import torch
        import image_dit_amd as ia
        from image_dit_amd import synth
        if name not in self._pvar:
            spec, w, dev = PREP_VARIANTS[name], self.w, self.q.device
            kw = {}
            if spec.get("rope_dim"):
                cos, sin = synth.make_rope_tables(w.S, spec["rope_dim"])
                kw.update(q_norm_w=synth.make_norm_weight(seed=1).to(dev),
                          k_norm_w=synth.make_norm_weight(seed=2).to(dev),
                          rope_cos=cos.to(dev), rope_sin=sin.to(dev), rope_dim=spec["rope_dim"])
            if spec.get("smooth_k"):
                nb = ia.sage_workspace_size(w.B, w.S, w.H)
                kw.update(smooth_k=True, k_mean=torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev),
                          workspace=torch.empty(max(nb, 16), dtype=torch.uint8, device=dev))
            specs = ia._prepared_specs(w.B, w.S, w.H, w.D, w.S, w.H)
            kw["out"] = tuple(torch.empty(shape, dtype=dt, device=dev) for _, shape, dt in specs)
            self._pvar[name] = kw
        return self._pvar[name]


def mode_fn(inp, mode, stream):
    import image_dit_amd as ia
    w = inp.w
    if mode == "bf16":
        return lambda: ia.attn_fwd_bf16_ws(inp.q, inp.k, inp.v, w.scale, out=inp.out, workspace=inp.ws,
                                           stream=stream)
    prep = inp.prepared(stream)
    if mode == "prepare":
        return lambda: ia.sage_prepare(inp.q, inp.k, inp.v, w.scale, out=prep, stream=stream)
    if mode == "sage_core":
        return lambda: ia.sage_attn_fwd_ws(prep, w.S, w.S, w.H, w.H, w.scale, out=inp.out, workspace=inp.ws,
                                           stream=stream)
    if mode == "sage":
        def f():
            ia.sage_prepare(inp.q, inp.k, inp.v, w.scale, out=prep, stream=stream)
            ia.sage_attn_fwd_ws(prep, w.S, w.S, w.H, w.H, w.scale, out=inp.out, workspace=inp.ws,
                                stream=stream)
        return f
    base, _, var = mode.partition("_")
    if mode.startswith("sage_core_"):
        base, var = "sage_core", mode[len("sage_core_"):]
    if base == "prepare" and var in PREP_VARIANTS:
        kw = inp.prep_variant(var)
        return lambda: ia.sage_prepare_ex(inp.q, inp.k, inp.v, w.scale, stream=stream, **kw)
    if var in VARIANTS:
        k, v, vprep, window, H_kv, S_kv, ws = inp.variant(var, stream)
        if base == "bf16":
            return lambda: ia.attn_fwd_bf16_ws(inp.q, k, v, w.scale, window=window, out=inp.out, workspace=ws,
                                               stream=stream)
        if base == "sage_core":
            return lambda: ia.sage_attn_fwd_ws(vprep, w.S, S_kv, w.H, H_kv, w.scale, window=window, out=inp.out,
                                               workspace=ws, stream=stream)
    raise ValueError(mode)


def row_record(w, mode, ms, reps):
    from image_dit_amd import cost
    flops = cost.attn_flops(w.B, w.H, w.S, w.D)
    rec = {"workload": w.name, "mode": mode, "B": w.B, "H": w.H, "S": w.S, "ms": ms, "reps": reps}
    var = mode.rsplit("_", 1)[-1] if "_" in mode and mode != "sage_core" else ""
    if var in VARIANTS:
        spec = VARIANTS[var]
        window = spec.get("window", (-1, -1))
        H_kv, S_kv = w.H // spec.get("hkv_div", 1), spec.get("s_kv", w.S)
        flops = cost.attn_flops_ex(w.B, w.H, w.S, S_kv, w.D, window)
        rec.update(S_kv=S_kv, H_kv=H_kv, window=list(window), flop=flops)
    if mode.startswith("prepare_"):
        spec = PREP_VARIANTS[var]
        nbytes = cost.sage_prepare_bytes_ex(w.B, w.H, w.S, w.S, w.H, w.D, rope_dim=spec.get("rope_dim", 0),
                                            smooth_k=spec.get("smooth_k", False))
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec.update(bound="hbm", gbs=gbs, algorithmic_bytes=nbytes, peak=PEAK_HBM_GBS,
                   frac=gbs / PEAK_HBM_GBS)
        return rec
    if mode == "prepare":
        nbytes = cost.sage_prepare_bytes(w.B, w.H, w.S, w.D)
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec.update(bound="hbm", gbs=gbs, algorithmic_bytes=nbytes, peak=PEAK_HBM_GBS,
                   frac=gbs / PEAK_HBM_GBS)
    else:
        tf = flops / (ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS["bf16" if mode.startswith("bf16") else "int8"]
        rec.update(bound="mfma", tflops=tf, peak=peak, frac=tf / peak)
    return rec


def parse_rows(spec):
    from image_dit_amd import synth
    if spec in ("", "none"):
        return []
    items = DEFAULT_ROWS if spec == "all" else [x for x in spec.split(",") if x]
    out = []
    for it in items:
        wname, mode = it.split(":")
        if mode not in MODES:
            raise SystemExit("unknown mode %r (one of %s)" % (mode, ", ".join(MODES)))
        if wname == "flux1024" and mode != "bf16":
            wname = "flux1024_kbias"  # the Sage configuration of this shape carries the K bias
        if wname not in synth.WORKLOADS:
            raise SystemExit("unknown workload %r" % wname)
        out.append((wname, mode))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rows", default="all", help="per-config rows: all, none or workload:mode,...")
    ap.add_argument("--row-ms", type=float, default=200.0, help="minimum timed ms per row")
    ap.add_argument("--only", default="", help="run only these rows, --reps calls each (profiling)")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceilings", action="store_true",
                    help="sustained library GEMM and copy rates (the practical ceilings)")
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
    if args.ceilings:
        ceilings()
        return

    ia.load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream()
    inputs = {}

    def get_inputs(name, qkv=None):
        if name not in inputs:
            inputs[name] = Inputs(synth.WORKLOADS[name], dev, qkv)
        return inputs[name]

    if args.only:
        for wname, mode in parse_rows(args.only):
            inp = get_inputs(wname)
            fn = mode_fn(inp, mode, stream)
            ms, _, _ = timed(fn, stream, args.reps, 1)
            print(json.dumps(row_record(inp.w, mode, ms, args.reps)), flush=True)
            inputs.clear()
            torch.cuda.empty_cache()
        return

    # headline inputs first (host-generated: the CPU baseline uses the same tensors)
    w = synth.WORKLOADS["flux1024"]
    q, k, v = synth.workload_qkv(w)
    head = Inputs(w, dev, (q, k, v))
    head_fn = mode_fn(head, "bf16", stream)

    # ---- per-config rows (time-sized); one workload's buffers at a time
    rows = []
    t_rows = time.perf_counter()
    for wname, mode in parse_rows(args.rows):
        if wname not in inputs:
            inputs.clear()
            torch.cuda.empty_cache()
        inp = get_inputs(wname)
        ms, reps = timed_for(mode_fn(inp, mode, stream), stream, args.row_ms)
        rows.append(row_record(inp.w, mode, ms, reps))
    t_rows = time.perf_counter() - t_rows

    # ---- headline: FLUX-1024 BF16, exactly W warm-up + K timed steps
    ms, first, last = timed(head_fn, stream, args.steps, args.warmup)
    inputs.clear()
    flops = cost.attn_flops(w.B, w.H, w.S, w.D)
    tflops = flops / (ms * 1e-3) / 1e12
    rows.insert(0, dict(row_record(w, "bf16", ms, args.steps), headline=True))

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
        "config": {"workload": "flux1024 self-attention, BF16 path", "B": w.B, "H": w.H, "S": w.S,
                   "D": w.D, "causal": False},
        "clock_regime": {"first_quarter_ms_per_step": first, "last_quarter_ms_per_step": last,
                         "timed_after": "%d per-config rows (%.1f s), no idle gap" % (len(rows) - 1, t_rows)},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": tflops / PEAK_TFLOPS["bf16"],
                     "traffic": measured_traffic("attn_fwd_bf16", w.name),
                     "kernel": "attn_fwd_bf16_kernel", "algorithmic_flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": cost.attn_bytes_bf16(w.B, w.H, w.S, w.D)},
        "rows": rows,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
