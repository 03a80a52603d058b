"""Benchmark of one latent MoE layer forward on one MI355X.

A step is one pass of the whole layer (input norm when configured, router,
top-k, permutation, down-projection, grouped GEMM1 + SwiGLU, grouped GEMM2 +
per-expert norm, combine, up-projection + residual gate) over one batch of
seeded synthetic input of the 816B-A42B layer shape (d=8192, latent 4096,
256 SwiGLU experts 4096->4096->4096, top-8 softmax gating, bf16 weights),
with every input already resident in HBM.

Default workload: decode, T=64 tokens (also timed with the Infinity Cache
flushed between calls).  Further line items time the prefill regime
(T=8192), skewed routing (T=16384), MXFP4 weights (4 chunks of 8192) and
the Muse sublayer around the same layer (sigmoid router with a correction
bias, latent pre-norm, input-scaled output norm, alpha/beta residual gate)
at T=64 and T=8192.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA (fp8 x fp4 runs at the fp8 rate)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(p, counts) -> dict:
    """Algorithmic HBM bytes of one forward (one chunk): every weight byte of
    the touched experts, the router and both projections read once, x read,
    out written.  Weights take 2 bytes (bf16, fp16) or 4.25 bits (MXFP4)."""
    touched = int((counts > 0).sum())
    wb = 0.53125 if p.weights == "mxfp4" else 2
    per_expert_w1 = 2 * p.F * p.L * wb
    per_expert_w2 = p.L * p.F * wb
    dense = p.n * p.d * 2 + (p.L * p.d + p.d * p.L) * wb
    TK = p.chunk_T * p.k
    act = p.chunk_T * p.d * 2 + p.chunk_T * p.d * 4
    gemm1 = touched * per_expert_w1 + TK * p.L * 2 + TK * p.F * 2   # W1 + gathered z rows + act rows
    return {"touched": touched, "total": touched * (per_expert_w1 + per_expert_w2) + dense + act, "gemm1": gemm1}


def layer_flops(p) -> dict:
    """FLOPs of one pass over all chunks of preset p."""
    T = p.chunk_T * p.chunks
    per_tok = 2 * p.d * p.n + 2 * p.d * p.L + p.k * (2 * p.L * 2 * p.F + 2 * p.F * p.L) + 2 * p.L * p.d
    return {"total": T * per_tok, "gemm1": T * p.k * 2 * p.L * 2 * p.F,
            "experts": T * p.k * (2 * p.L * 2 * p.F + 2 * p.F * p.L)}


def recorded_traffic(name: str):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    record under profiles/, or None when the kernel sources changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if csrc_hash() != rec.get("source_sha256_16"):
        return None
    return rec["traffic_bytes"]


def recorded_mfma_counters(workload: str):
    """Per-kernel MFMA-busy share, clock and TFLOP/s of the prefill GEMMs from
    the committed rocprofv3 counter record, or None when the kernel sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "prefill_T8192_mfma_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if csrc_hash() != rec.get("source_sha256_16"):
        return None
    return {r["role"]: {"mfma_busy": r["mfma_busy"], "clock_GHz": r["clock_GHz"], "TFLOPs": r["TFLOPs"]}
            for r in rec[workload]}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def csrc_hash() -> str:
    """Digest of the kernel sources (all of csrc/, in name order)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sparse_mixture_experts_router_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h")):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def vendor_gemm_reference(torch) -> None:
    """Times the vendor GEMM library (torch.bmm / torch.mm) on the layer's GEMM shapes with N(0,1) operands (and
    one with zeros), fp16 and bf16: the rate a library GEMM reaches on this chip and data, printed as one JSON line."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = []

    def timed(fn, flop, label, dt):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        n = 10
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        res.append({"shape": label, "dtype": dt, "ms": round(ms, 3), "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1)})
        log(res[-1])

    for dt in (torch.float16, torch.bfloat16):
        name = "fp16" if dt == torch.float16 else "bf16"
        a = torch.randn(256, 256, 4096, device=dev, dtype=dt, generator=g)
        b = torch.randn(256, 4096, 8192, device=dev, dtype=dt, generator=g)
        timed(lambda: torch.bmm(a, b), 2.0 * 256 * 256 * 4096 * 8192,
              "256 experts x [256 x 4096] @ [4096 x 8192] (GEMM1's shape, every expert at 256 rows)", name)
        del a, b
        a = torch.randn(8192, 8192, device=dev, dtype=dt, generator=g)
        b = torch.randn(8192, 4096, device=dev, dtype=dt, generator=g)
        timed(lambda: torch.mm(a, b), 2.0 * 8192 * 8192 * 4096, "[8192 x 8192] @ [8192 x 4096] (down-projection)", name)
        b = torch.randn(8192, 8192, device=dev, dtype=dt, generator=g)
        timed(lambda: torch.mm(a, b), 2.0 * 8192 ** 3, "[8192 x 8192] @ [8192 x 8192], N(0,1) operands", name)
        a.zero_()
        b.zero_()
        timed(lambda: torch.mm(a, b), 2.0 * 8192 ** 3, "[8192 x 8192] @ [8192 x 8192], zero operands", name)
        del a, b
        torch.cuda.empty_cache()
    print(json.dumps({"vendor_gemm": res}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--only-prefill", action="store_true", help="only the prefill workload (profiling runs)")
    ap.add_argument("--only", default=None, metavar="PRESET",
                    help="only the named workload preset (c1m, c2, c3, c4c, c4i, c4q, m1, m2), for profiling runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the cache-flushed decode timing and the skewed (T=16384) and MXFP4 (4 x 8192) workloads")
    ap.add_argument("--weight-format", choices=["bf16", "f16"], default="f16",
                    help="storage of expert_w1, expert_w2, up_w: the bf16 checkpoint as is, or converted once "
                         "(before timing, value-exact) to fp16 so the fp16 GEMMs read it without converting")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run the library's plain 16-byte copy of MIB MiB (5 times), to calibrate HBM counters")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor GEMM library (torch) on the layer's GEMM shapes, as a reference rate")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_mixture_experts_router_amd as moe
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.rand(n // 4, dtype=torch.float32, device="cuda")  # random bits: constant data reads as far fewer bytes
        b = torch.empty_like(a)
        moe.moe_hbm_copy(b, a, n)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            moe.moe_hbm_copy(b, a, n)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        print(json.dumps({"copy_bytes": n, "copy_GBps": round(2 * n / dt / 1e9, 1)}))
        return
    if args.vendor_gemm:
        vendor_gemm_reference(torch)
        return
    moe.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    p = synthetic.PRESETS["c1"]
    t0 = time.time()
    host = synthetic.layer_params(p)
    log("layer generated in %.1f s" % (time.time() - t0))
    W = {k: to_dev(v) for k, v in host.items()}
    wfmt = args.weight_format
    gains = {"router_bias": None, "gamma_in": None, "gamma_expert": W["gamma_ex"], "res_gate": W["gate"]}

    def make_desc(T, pr, wf):
        return moe.make_desc(T, pr.d, pr.L, pr.n, pr.k, pr.F, expert_kind=pr.kind, act=pr.act, router=pr.router_w,
                             weights=wf, in_norm=pr.in_norm, expert_norm=pr.expert_norm, res_gate=pr.res_gate,
                             eps_in=pr.eps_in, eps_expert=pr.eps_expert, interm=pr.interm, router_fn=pr.router_fn,
                             out_mult=pr.out_mult, routed_scale=pr.routed_scale, latent_norm=pr.latent_norm,
                             eps_latent=pr.eps_latent, out_norm=pr.out_norm, eps_out=pr.eps_out, res_tau=pr.res_tau,
                             res_floor=pr.res_floor, act_quant=pr.act_quant)

    stream = torch.cuda.current_stream()

    def run_workload(pr, steps, warmup, Wd=None, gd=None, wf=None):
        """steps timed passes of preset pr (all of its chunks per pass, chunk_T tokens each)."""
        Wd, gd, wf = Wd or W, gd or gains, wf or wfmt
        T = pr.chunk_T
        desc = make_desc(T, pr, wf)
        x_host = synthetic.inputs(pr, chunk=0) if pr.chunks > 1 else synthetic.inputs(pr)
        xs = [to_dev(x_host)] + [to_dev(synthetic.inputs(pr, chunk=c)) for c in range(1, pr.chunks)]
        out = torch.empty((T, pr.d), dtype=torch.float32, device=dev)
        ws = torch.empty(moe.moe_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        counts = torch.empty(pr.n, dtype=torch.int32, device=dev)

        def fwd(c, dbg=None, s=None):
            moe.moe_layer_forward(desc, xs[c], Wd["router_w"], Wd["down_w"], Wd["w1"], Wd["w2"], Wd["up_w"], gd,
                                  out, workspace=ws, dbg=dbg, stream=s or stream)

        def timed(step):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / steps

        def eager_step():
            for c in range(pr.chunks):
                fwd(c)

        fwd(0, {"expert_counts": counts})
        torch.cuda.synchronize()
        for _ in range(warmup):
            eager_step()
        eager_ms = timed(eager_step)
        # the same step as one HIP graph (the forward launches kernels only: no
        # allocation, no memset), reported beside the plain calls
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in range(pr.chunks):
                fwd(c, s=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for c in range(pr.chunks):
                fwd(c, s=cap)
        for _ in range(warmup):
            graph.replay()
        graph_ms = timed(graph.replay)
        # per-stage times in a separate eager pass (the stage events add gaps of their own)
        evs = [[moe.StageEvents() for _ in range(pr.chunks)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            for c in range(pr.chunks):
                fwd(c, {"stage_events": evs[i][c].address})
        torch.cuda.synchronize()
        stages = {}
        skip = set()
        if pr.in_norm == "none":
            skip.add("in_norm")
        if pr.out_norm == "none" and pr.res_gate != "muse":
            skip.add("resgate")  # the linear gate runs in the up-projection's epilogue
        ran = [s for s in moe.STAGES if s not in skip]
        for s in ran:
            v = [sum(e.elapsed_ms(s) or 0.0 for e in row) for row in evs]
            if any(v):
                stages[s] = sum(v) / len(v)
        for row in evs:
            for e in row:
                e.close()
        del graph
        return {"T": T * pr.chunks, "ms": eager_ms, "graph_ms": graph_ms, "stages": stages,
                "counts": counts.cpu().numpy(), "x": x_host, "fwd": fwd}

    def flushed_ms(r, steps):
        """Median event-timed ms of one call after writing 1 GiB of scratch, so no weight, router or
        projection byte is left in the 256 MB Infinity Cache from the previous call."""
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ms = []
        for i in range(steps):
            scratch.fill_(i & 255)
            e0.record(stream)
            r["fwd"](0)
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        del scratch
        return float(np.median(ms))

    def to_f16_format():
        # expert_w1, expert_w2 and up_w converted in place, once, outside every timed region
        for key in ("w1", "w2", "up_w"):
            moe.moe_convert_bf16_to_f16(W[key], W[key], W[key].numel())
        torch.cuda.synchronize()

    # The bf16 checkpoint as given (no conversion), decode and prefill, before the fp16 format is made
    bf16_ckpt = None
    if args.only_prefill:
        args.only = "c2"
    if wfmt == "f16" and not args.no_extra and not args.only:
        rb = run_workload(p, args.steps, args.warmup, wf="bf16")
        bf16_ckpt = {"decode_T64": {"ms_per_step": round(rb["ms"], 4),
                                    "tokens_per_s": round(p.chunk_T / (rb["ms"] * 1e-3), 1),
                                    "stage_ms": {k: round(v, 4) for k, v in rb["stages"].items()}}}
        log("bf16 checkpoint, decode T=%d: %.3f ms/step" % (p.chunk_T, rb["ms"]))
        if not args.no_prefill:
            pc = synthetic.PRESETS["c2"]
            rb2 = run_workload(pc, 3, 1, wf="bf16")
            bf16_ckpt["prefill_T8192"] = {
                "ms_per_step": round(rb2["ms"], 4), "tokens_per_s": round(pc.chunk_T / (rb2["ms"] * 1e-3), 1),
                "TFLOPs": round(layer_flops(pc)["total"] / (rb2["ms"] * 1e-3) / 1e12, 1),
                "stage_ms": {k: round(v, 4) for k, v in rb2["stages"].items()}}
            log("bf16 checkpoint, prefill T=%d: %.3f ms/step" % (pc.chunk_T, rb2["ms"]))
        bf16_ckpt["note"] = ("expert_w1, expert_w2 and up_w read as bf16 and converted to fp16 per fragment "
                             "inside the GEMMs; same results bit for bit as the fp16 weight format")
    if wfmt == "f16":
        to_f16_format()

    def preset_gains(pr, dev_w):
        gv = {k: to_dev(v) for k, v in synthetic.gains(pr).items()}
        return {"router_bias": gv.get("bias"), "gamma_in": gv.get("gamma_in"), "gamma_expert": gv.get("gamma_ex"),
                "res_gate": gv.get("gate"), "gamma_latent": gv.get("gamma_lat"), "gamma_out": gv.get("gamma_out")}

    if args.only:
        # one workload alone (profiling runs): the preset's weight format and parameter vectors
        po = synthetic.PRESETS[args.only]
        Wo, wfo = W, wfmt
        if po.weights == "mxfp4":
            W.clear()  # the bf16 layer is not needed: free its 24 GB first
            torch.cuda.empty_cache()
            Wo = {k: to_dev(v) for k, v in synthetic.layer_params(po).items()}
            wfo = "mxfp4"
        ro = run_workload(po, args.prefill_steps, 2, Wd=Wo, gd=preset_gains(po, Wo), wf=wfo)
        tf = layer_flops(po)["total"] / (ro["ms"] * 1e-3) / 1e12
        log("%s (T=%d x %d): %.3f ms/step, %.1f TFLOP/s; stages %s" % (
            args.only, po.chunk_T, po.chunks, ro["ms"], tf, {k: round(v, 4) for k, v in ro["stages"].items()}))
        return

    # ---- decode (headline) ----
    r = run_workload(p, args.steps, args.warmup)
    by = layer_bytes(p, r["counts"])
    fl = layer_flops(p)
    tok_s = p.chunk_T / (r["ms"] * 1e-3)
    g1_ms = r["stages"]["gemm1"]
    g1_gbs = by["gemm1"] / (g1_ms * 1e-3) / 1e9
    log("decode T=%d: %.3f ms/step (as a HIP graph %.3f), %.0f tok/s, layer %.0f GB/s; stages %s" % (
        p.chunk_T, r["ms"], r["graph_ms"], tok_s, by["total"] / (r["ms"] * 1e-3) / 1e9,
        {k: round(v, 4) for k, v in r["stages"].items()}))

    result = {
        "metric": "MoE-layer tokens/s at T=64 (decode; T=8192 prefill under secondary)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp16 MFMA operands (bf16 checkpoint weights stored as fp16: exact for magnitudes in "
                  "[2^-17, 65504], smaller ones round to fp16 subnormals), fp32 accumulate"
                  if wfmt == "f16" else "bf16 weights, fp16 activations, fp32 accumulate"),
        "data": "synthetic (seeded Philox normals, random-init weights of the 816B-A42B layer shape)",
        "config": {"workload": "latent MoE layer, decode T=64", "T": p.chunk_T, "d_model": p.d, "d_latent": p.L,
                   "d_ff": p.F, "n_experts": p.n, "top_k": p.k, "weights": p.weights, "weight_storage": wfmt,
                   "touched_experts": by["touched"], "layer_bytes": by["total"],
                   "layer_GBps": round(by["total"] / (r["ms"] * 1e-3) / 1e9, 1),
                   "layer_frac_hbm": round(by["total"] / (r["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "graph_ms_per_step": round(r["graph_ms"], 4),
                   "stage_ms": {k: round(v, 4) for k, v in r["stages"].items()}},
        "roofline": {"kernel": "gemm_stream_kernel (grouped GEMM1 + SwiGLU)", "bound": "hbm",
                     "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(g1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("decode_T64_gemm1_traffic.json"),
                     "bytes_per_launch": by["gemm1"], "avg_launch_ms": round(g1_ms, 4)},
    }

    if bf16_ckpt:
        result["bf16_checkpoint"] = bf16_ckpt
    if not args.no_extra:
        fm = flushed_ms(r, args.steps)
        result["decode_cache_flushed"] = {
            "ms_median": round(fm, 4), "tokens_per_s": round(p.chunk_T / (fm * 1e-3), 1),
            "layer_GBps": round(by["total"] / (fm * 1e-3) / 1e9, 1),
            "note": "1 GiB written before each call: nothing of the previous call is left in the 256 MB "
                    "Infinity Cache (the headline steps run back to back)"}
        log("decode T=%d, cache flushed between calls: %.3f ms" % (p.chunk_T, fm))

    # ---- prefill (secondary) ----
    if not args.no_prefill:
        p2 = synthetic.PRESETS["c2"]
        r2 = run_workload(p2, args.prefill_steps, 2)
        fl2 = layer_flops(p2)
        tf = fl2["total"] / (r2["ms"] * 1e-3) / 1e12
        g1 = r2["stages"]["gemm1"]
        g1_tf = fl2["gemm1"] / (g1 * 1e-3) / 1e12
        by2 = layer_bytes(p2, r2["counts"])
        log("prefill T=%d: %.3f ms/step, %.0f tok/s, %.1f TFLOP/s; stages %s" % (
            p2.chunk_T, r2["ms"], p2.chunk_T / (r2["ms"] * 1e-3), tf, {k: round(v, 4) for k, v in r2["stages"].items()}))
        result["secondary"] = {
            "workload": "latent MoE layer, prefill T=8192", "value": round(p2.chunk_T / (r2["ms"] * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(r2["ms"], 4), "graph_ms_per_step": round(r2["graph_ms"], 4),
            "steps": args.prefill_steps,
            "layer_TFLOPs": round(tf, 1), "layer_frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
            "stage_ms": {k: round(v, 4) for k, v in r2["stages"].items()},
            # at ~256 rows per expert GEMM1 does ~240 FLOP per byte it must move, below the chip's
            # 2.5 PFLOP/s / 8 TB/s = 312 FLOP/B balance: HBM bounds it (2.3 ms vs 1.8 ms of MFMA)
            "roofline": {"kernel": "gemm_big_kernel + gemm_wide_kernel, grouped GEMM1 + SwiGLU (full-tile and "
                                   "wide-tile launches, timed together by the stage's HIP events)",
                         "bound": "hbm", "achieved": round(by2["gemm1"] / (g1 * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(by2["gemm1"] / (g1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": by2["gemm1"], "avg_launch_ms": round(g1, 4),
                         "traffic": recorded_traffic("prefill_T8192_gemm1_traffic.json"),
                         "mfma_view": {"flops": fl2["gemm1"], "achieved_TFLOPs": round(g1_tf, 1),
                                       "peak_TFLOPs": BF16_PEAK_TFLOPS,
                                       "frac": round(g1_tf / BF16_PEAK_TFLOPS, 4),
                                       "counters": recorded_mfma_counters("c2")}}}

    # ---- the skewed and MXFP4 workloads ----
    def report(pr, rr, label):
        flx, byx = layer_flops(pr), layer_bytes(pr, rr["counts"])
        toks = pr.chunk_T * pr.chunks
        d = {"workload": label, "tokens_per_s": round(toks / (rr["ms"] * 1e-3), 1), "ms_per_step": round(rr["ms"], 4),
             "graph_ms_per_step": round(rr["graph_ms"], 4),
             "TFLOPs": round(flx["total"] / (rr["ms"] * 1e-3) / 1e12, 1),
             "frac_mfma": round(flx["total"] / (rr["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
             "weight_and_io_GBps": round(byx["total"] * pr.chunks / (rr["ms"] * 1e-3) / 1e9, 1),
             "touched_experts_chunk0": byx["touched"], "stage_ms": {k: round(v, 4) for k, v in rr["stages"].items()}}
        log("%s: %.3f ms/step, %.0f tok/s, %.1f TFLOP/s" % (label, rr["ms"], d["tokens_per_s"], d["TFLOPs"]))
        return d

    if not args.no_extra:
        p3 = synthetic.PRESETS["c3"]
        g3 = dict(gains)
        g3["router_bias"] = to_dev(synthetic.zipf_bias(p3.n))
        result["skewed"] = report(p3, run_workload(p3, 5, 1, gd=g3),
                                  "T=16384, Zipf(1.2) selection bias (hottest expert most of the tokens)")
        t0 = time.time()
        host4 = synthetic.layer_params(synthetic.PRESETS["c4i"])  # MXFP4 forms of the same draws
        W4 = {k: to_dev(v) for k, v in host4.items()}
        del host4
        log("MXFP4 layer generated in %.1f s" % (time.time() - t0))
        result["mxfp4"] = {}
        for name in ("c4c", "c4i"):
            p4 = synthetic.PRESETS[name]
            g4 = {"router_bias": None, "gamma_in": W4["gamma_in"], "gamma_expert": W4["gamma_ex"], "res_gate": W4["gate"]}
            result["mxfp4"][p4.in_norm] = report(p4, run_workload(p4, 3, 1, Wd=W4, gd=g4, wf="mxfp4"),
                                                 "MXFP4 weights, 4 chunks of T=8192, input norm %s" % p4.in_norm)
        # the same workload with MXFP8 activations at the expert GEMMs (the scaled fp8 x fp4 MFMA)
        p4 = synthetic.PRESETS["c4q"]
        g4 = {"router_bias": None, "gamma_in": W4["gamma_in"], "gamma_expert": W4["gamma_ex"], "res_gate": W4["gate"]}
        rq = report(p4, run_workload(p4, 3, 1, Wd=W4, gd=g4, wf="mxfp4"),
                    "MXFP4 weights and MXFP8 expert-GEMM activations, 4 chunks of T=8192, input norm centered")
        flq = layer_flops(p4)
        rq["frac_fp8_mfma"] = round(rq["TFLOPs"] / FP8_PEAK_TFLOPS, 4)
        rq["note"] = ("TFLOPs and frac_mfma count every FLOP of the layer against the bf16 peak; the expert GEMMs "
                      "(%.0f%% of the FLOPs) run on the fp8 x fp4 MFMA, whose dense peak is %.0f TFLOP/s" % (
                          100.0 * flq["experts"] / flq["total"], FP8_PEAK_TFLOPS))
        result["mxfp4"]["mxfp8_activations"] = rq
        # the decode batch on the same MXFP4 weights
        p1m = synthetic.PRESETS["c1m"]
        g1m = {"router_bias": None, "gamma_in": None, "gamma_expert": W4["gamma_ex"], "res_gate": W4["gate"]}
        r1m = run_workload(p1m, args.steps, args.warmup, Wd=W4, gd=g1m, wf="mxfp4")
        by1m = layer_bytes(p1m, r1m["counts"])
        result["mxfp4"]["decode_T64"] = {
            "workload": "MXFP4 weights, decode T=64", "ms_per_step": round(r1m["ms"], 4),
            "graph_ms_per_step": round(r1m["graph_ms"], 4),
            "tokens_per_s": round(p1m.chunk_T / (r1m["ms"] * 1e-3), 1),
            "layer_bytes": by1m["total"], "layer_GBps": round(by1m["total"] / (r1m["ms"] * 1e-3) / 1e9, 1),
            "layer_frac_hbm": round(by1m["total"] / (r1m["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "touched_experts": by1m["touched"],
            # the grouped GEMM1 on MXFP4 codes (4.25 bits a weight) and its scale words: algorithmic bytes over
            # its event-timed stage
            "gemm1_GBps": round(by1m["gemm1"] / (r1m["stages"]["gemm1"] * 1e-3) / 1e9, 1),
            "gemm1_frac_hbm": round(by1m["gemm1"] / (r1m["stages"]["gemm1"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stage_ms": {k: round(v, 4) for k, v in r1m["stages"].items()}}
        log("MXFP4 weights, decode T=64: %.3f ms/step, %.0f tok/s, layer %.0f GB/s" % (
            r1m["ms"], p1m.chunk_T / (r1m["ms"] * 1e-3), by1m["total"] / (r1m["ms"] * 1e-3) / 1e9))
        del W4
        torch.cuda.empty_cache()

    # ---- the Muse sublayer around the same layer ----
    if not args.no_extra:
        result["muse"] = {}
        for name, steps, label in (("m1", args.steps, "decode T=64"), ("m2", 5, "prefill T=8192")):
            pm = synthetic.PRESETS[name]
            gv = {k: to_dev(v) for k, v in synthetic.gains(pm).items()}
            gm = {"router_bias": gv.get("bias"), "gamma_in": gv.get("gamma_in"), "gamma_expert": gv.get("gamma_ex"),
                  "res_gate": gv.get("gate"), "gamma_latent": gv.get("gamma_lat"), "gamma_out": gv.get("gamma_out")}
            result["muse"][name] = report(pm, run_workload(pm, steps, 2, gd=gm),
                                          "Muse sublayer (sigmoid router + bias, C_pre, output norm, alpha/beta "
                                          "gate), " + label)

    # ---- CPU oracle baseline on a bounded sample of the decode workload ----
    if not args.no_cpu_baseline:
        import oracle
        cfg = p.cfg()
        t = dict(host)
        t["x"] = r["x"]
        # passes over the whole decode batch until about cpu_seconds of work (rows are independent)
        toks = np.arange(p.chunk_T)
        passes, m, el = 0, 0, 0.0
        while el < args.cpu_seconds and passes < 1000:
            t1 = time.perf_counter()
            oracle.forward(cfg, t, tokens=toks)
            el += time.perf_counter() - t1
            passes += 1
            m += len(toks)
        cores = oracle.threads()
        result["cpu_baseline"] = {"value": round(m / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                                  "cpu_model": cpu_model(),
                                  "sample": "%d passes over the T=%d decode batch (%d token rows), fp64 oracle, "
                                            "%.1f s" % (passes, p.chunk_T, m, el)}
        log("cpu oracle: %d token rows in %.1f s on %d threads" % (m, el, cores))
        if not args.no_prefill:
            # the prefill batch: routing (router, top-k, weights) of all its tokens, and the whole layer on a
            # seeded sample of them (exact per token: rows are independent)
            p2 = synthetic.PRESETS["c2"]
            x2 = synthetic.inputs(p2)
            t2 = dict(host, x=x2)
            t1 = time.perf_counter()
            oracle.forward(p2.cfg(), t2, want_outputs=False)
            el_r = time.perf_counter() - t1
            sub = synthetic.sample_tokens(p2.T, 256, seed=77)
            t1 = time.perf_counter()
            oracle.forward(p2.cfg(), t2, tokens=sub)
            el_f = time.perf_counter() - t1
            result["cpu_baseline"]["prefill_T8192"] = {
                "routing_tokens_per_s": round(p2.T / el_r, 1), "layer_tokens_per_s": round(len(sub) / el_f, 3),
                "sample": "routing of all %d tokens (%.1f s); the whole layer on %d seeded tokens (%.1f s)" % (
                    p2.T, el_r, len(sub), el_f)}
            log("cpu oracle, prefill batch: routing %d tokens in %.1f s, layer on %d tokens in %.1f s" % (
                p2.T, el_r, len(sub), el_f))

    print(json.dumps(result))


if __name__ == "__main__":
    main()
