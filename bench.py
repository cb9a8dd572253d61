#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE forward on one MI355X.

One step = one pass of the whole hot path on one batch of synthetic input:
  moe_dispatch -> moe_expert_gate_up (SiLU*up fused) -> moe_expert_down
  -> moe_reduce_fused,
exactly the kernels moe_routed_forward launches after the dispatch, called
stage by stage so that HIP events (recorded on the stream the kernels run
on) time every kernel inside the timed region.

Workload of the headline value (the metric's T = 512 case): the
DeepSeek-shaped decode layer, T=512, d_hidden=7168, d_expert=2048, E=256
routed experts, top-8, bf16, seeded synthetic x / weights / router (no
dataset, random-init weights). The same JSON line carries, at its end, the
metric's T = 4096 case (the prefill layer of the same shapes, "t4096"), the
Zipf-skewed T = 4096 routed forward ("skewed"), its standalone reduce
("reduce_skewed"), the two small workloads and the quantised / weighted
variants in compact form; the full per-kernel detail goes to stderr.

Timing protocol (after the reduce PR's measurement section): warm-up steps,
then the K timed steps split into 3 trials; before every step a 512 MB
device buffer is read (summed), which evicts the 4 MB L2s and the 256 MB
last-level cache, so no step reads its inputs from a cache the previous
step filled, and leaves no dirty lines for the step's own reads to write
back (--flush-mode write fills the buffer instead); each step is bracketed by HIP events; the value is the median
of the 3 trial means of the event span (flush excluded). The CPU oracle is
timed on bounded samples of the workloads under "cpu_baseline".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pmc_grouped_gemm_gate_up_deepseek_decode.md")
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_routed_moe_amd", "csrc", f)
                for f in ("grouped_gemm.hpp", "grouped_gemm.hip", "common.hpp")]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2,
                    help="index into synthetic.CONFIGS for the main line (default 2: decode T=512); "
                         "with --dump-routing, -1 is the MFMA probe's routing")
    ap.add_argument("--block-m", type=int, default=None,
                    help="row block size of every timed workload (default: chosen per workload)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MB of device memory passed over before every timed step (0 = no flush)")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read",
                    help="read (sum) or write (fill) the flush buffer")
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--no-t4096", action="store_true",
                    help="skip the T=4096 prefill, skewed and small workloads")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the standalone reduce, the MFMA probe, the gate and the variants")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="tokens of the decode workload the oracle runs for the CPU baseline")
    ap.add_argument("--only", default=None,
                    help="comma-separated subset of the extra legs to run (t4096, skewed, small, "
                         "reduce, probe, gate, fp8, w8a8, w4a8, mx, weighted, fused, w4a8_gemm)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--dump-routing", default=None, metavar="FILE",
                    help="only write the workload's routing (ids, weights) for moe_bench_driver")
    ap.add_argument("--dump-reduce", default=None, metavar="FILE",
                    help="only write the skewed workload's standalone-reduce positions and "
                         "weights for moe_bench_driver")
    return ap.parse_args()


def gemm_source_sha():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, or None if it is missing or was taken on other kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != gemm_source_sha():
        return None
    return float(val.group(1))


def workload_numbers(d, tables_sizes, weights="16bit", weighted_down=False):
    """Algorithmic FLOPs and bytes of one step, per kernel (units in the
    design notes): weights of the experts that receive rows once (FP8: 1
    byte each, W4A8: half a byte, plus a 4-byte scale per row), x read once,
    h / expert_out written and read once, y written once; W4A8 / MX / W8A8
    add the quantised copies of x and h (and their scales), written once and
    read once."""
    T, H, D, E, K = d["T"], d["H"], d["D"], d["E"], d["K"]
    b = d["x"].element_size()
    wb = {"16bit": b, "fp8": 1, "w8a8": 1, "w4a8": 0.5, "mx": 0.5 + 1 / 32}[weights]
    sc = 4 if weights in ("fp8", "w4a8", "w8a8") else 0   # scale bytes per weight row
    n_valid = int(tables_sizes.sum())
    e_active = int((tables_sizes > 0).sum())
    P = T * K
    w_gate_up = int(e_active * 2 * D * (H * wb + sc))
    w_down = int(e_active * H * (D * wb + sc))
    out = dict(n_valid=n_valid, e_active=e_active)
    if weights in ("w4a8", "mx", "w8a8"):
        # int8 / E4M3 + a 4-byte scale per row, or E4M3 + an E8M0 byte per 32 values
        ab = 1 + 1 / 32 if weights == "mx" else 1
        rs = 0 if weights == "mx" else 4
        out["quant_x_bytes"] = int(T * H * b + T * H * ab + T * rs)
        out["gate_up_bytes"] = int(w_gate_up + T * H * ab + T * rs + n_valid * D * b)
        out["quant_h_bytes"] = int(P * D * b + P * D * ab + P * rs)
        out["down_bytes"] = int(w_down + n_valid * D * ab + n_valid * rs + n_valid * H * b)
    else:
        out["gate_up_bytes"] = w_gate_up + T * H * b + n_valid * D * b
        out["down_bytes"] = w_down + n_valid * D * b + n_valid * H * b
    out["reduce_bytes"] = n_valid * H * b + T * H * b + P * 8
    if weighted_down:   # the down GEMM reads a weight per row; the reduce reads none
        out["down_bytes"] += n_valid * 4
        out["reduce_bytes"] -= P * 4
    out["dispatch_bytes"] = P * 8 + n_valid * 12 + P * 8 + 12 * E
    out["flops_gate_up"] = 4 * n_valid * H * D
    out["flops_down"] = 2 * n_valid * H * D
    out["flops"] = out["flops_gate_up"] + out["flops_down"]
    out["b_min"] = w_gate_up + w_down + 2 * T * H * b + P * 8
    return out


class Flusher:
    """Passes over a `mb`-MB device buffer on the current stream, more than
    the 256 MB last-level cache and the L2s together, so that what a timed
    call reads next comes from HBM. mode "read" sums the buffer (the caches
    are left holding clean lines of it); mode "write" fills it, which leaves
    up to the L2s' size of dirty lines that the timed call's own reads then
    write back to HBM."""

    def __init__(self, dev, mb, mode="read"):
        import torch
        self.buf = torch.ones(max(mb, 0) << 20, dtype=torch.uint8, device=dev) if mb > 0 else None
        self.mode = mode
        self.sum_dtype = torch.int32
        self.v = 0
        self.sink = None

    def __call__(self):
        if self.buf is None:
            return
        if self.mode == "read":
            self.sink = self.buf.sum(dtype=self.sum_dtype)
        else:
            self.v ^= 1
            self.buf.fill_(self.v)


def trial_slices(steps, trials):
    """Splits `steps` timed steps into `trials` consecutive trials (sizes differ by <= 1)."""
    trials = max(1, min(trials, steps))
    sizes = [steps // trials + (1 if i < steps % trials else 0) for i in range(trials)]
    out, i = [], 0
    for n in sizes:
        out.append(slice(i, i + n))
        i += n
    return out


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def timed_calls(fn, n_marks, steps, warmup, flush, trials):
    """Runs fn(events) `warmup` times untimed, then `steps` times, each after
    flush(); fn records n_marks + 1 events. Returns the median over the
    trials of the trial means of the span (first to last event) and of each
    interval between consecutive events, in ms."""
    import torch
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_marks + 1)]
    for _ in range(warmup):
        flush()
        fn(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        fn(events[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    spans = [ev[0].elapsed_time(ev[n_marks]) for ev in events]
    parts = [[ev[j].elapsed_time(ev[j + 1]) for ev in events] for j in range(n_marks)]
    sl = trial_slices(steps, trials)
    tmean = lambda v: [sum(v[s]) / (s.stop - s.start) for s in sl]
    return dict(span=median(tmean(spans)), parts=[median(tmean(p)) for p in parts],
                trial_spans=[round(x, 4) for x in tmean(spans)], wall_incl_flush=wall)


def time_workload(cfg, steps, warmup, block_m, dev, flush, trials, weights="16bit",
                  weighted_down=False, fused=False):
    """One workload's step timed kernel by kernel. weights "fp8" / "w4a8" /
    "mx" / "w8a8": the expert weights are quantized once (timed on its own,
    not part of the step) and the step runs that path's GEMMs (W4A8 / MX /
    W8A8 quantise x and h inside the step, each a timed kernel of its own).
    weighted_down (16-bit weights): the routing weight applied in the down
    GEMM's epilogue, then an unweighted reduce. fused (16-bit weights,
    block_m <= 32): gate/up and down in the fused expert kernel, h kept on
    chip."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S

    t_gen = time.time()
    d = S.make_moe_inputs(cfg, device=dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    quant_ms = None
    if weights != "16bit":
        qfn = {"fp8": mr.quantize_fp8_rows, "w8a8": mr.quantize_fp8_rows,
               "w4a8": mr.quantize_int4_rows, "mx": mr.quantize_mx_weights}[weights]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        q = [qfn(d[n]) for n in ("w_gate", "w_up", "w_down")]
        ev[1].record()
        torch.cuda.synchronize()
        quant_ms = ev[0].elapsed_time(ev[1])
        d["w_gate"], d["w_up"], d["w_down"] = q
    T, H, D, E, K = d["T"], d["H"], d["D"], d["E"], d["K"]
    block_m = block_m or mr.default_block_m(T, K, E, weights)
    ids, w = d["topk_ids"], d["topk_weights"]
    x, wg, wu, wd = d["x"], d["w_gate"], d["w_up"], d["w_down"]
    tables = mr.MoeTables(T, K, E, block_m, dev)
    if weights == "w4a8":
        ws, h, eo, xq, sx, hq, sh = mr.forward_w4a8_workspace(tables, H, D, x.dtype)
    elif weights == "mx":
        ws, h, eo, xq, sx, hq, sh = mr.forward_mx_workspace(tables, H, D, x.dtype)
    elif weights == "w8a8":
        ws, h, eo, xq, sx, hq, sh = mr.forward_w8a8_workspace(tables, H, D, x.dtype)
    elif fused:
        ws, eo = mr.fused_workspace(tables, H, x.dtype)
    else:
        ws, h, eo = mr.forward_workspace(tables, H, D, x.dtype)
    if weights in ("w4a8", "mx", "w8a8"):
        names = ["dispatch", "quant_x", "gate_up", "quant_h", "down", "reduce"]
    elif fused:
        names = ["dispatch", "experts", "reduce"]
    else:
        names = ["dispatch", "gate_up", "down", "reduce"]
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    pos = tables.token_topk_to_pos.view(T, K)
    wt = tables.topk_weights.view(T, K)

    def step(ev):
        ev[0].record()
        mr.moe_dispatch(ids, w, E, block_m=block_m, tables=tables)
        ev[1].record()
        if weights == "w4a8":
            mr.quantize_int8_rows(x, q=xq, scales=sx)
            ev[2].record()
            mr.moe_expert_gate_up_w4a8(xq, sx, wg, wu, tables, x.dtype, h=h)
            ev[3].record()
            mr.quantize_int8_rows(h, q=hq, scales=sh)
            ev[4].record()
            mr.moe_expert_down_w4a8(hq, sh, wd, tables, x.dtype, expert_out=eo)
            ev[5].record()
        elif weights == "mx":
            mr.quantize_mx_rows(x, mr.MX_FP8, codes=xq, scales=sx)
            ev[2].record()
            mr.moe_expert_gate_up_mx(xq, sx, wg, wu, tables, x.dtype, h=h)
            ev[3].record()
            mr.quantize_mx_rows(h, mr.MX_FP8, codes=hq, scales=sh)
            ev[4].record()
            mr.moe_expert_down_mx(hq, sh, wd, tables, x.dtype, expert_out=eo)
            ev[5].record()
        elif weights == "w8a8":
            mr.quantize_fp8_act_rows(x, q=xq, scales=sx)
            ev[2].record()
            mr.moe_expert_gate_up_w8a8(xq, sx, wg, wu, tables, x.dtype, h=h)
            ev[3].record()
            mr.quantize_fp8_act_rows(h, q=hq, scales=sh)
            ev[4].record()
            mr.moe_expert_down_w8a8(hq, sh, wd, tables, x.dtype, expert_out=eo)
            ev[5].record()
        elif fused:
            mr.moe_expert_fused(x, wg, wu, wd, tables, expert_out=eo)
            ev[2].record()
        else:
            if weights == "fp8":
                mr.moe_expert_gate_up_w8(x, wg, wu, tables, h=h)
                ev[2].record()
                mr.moe_expert_down_w8(h, wd, tables, expert_out=eo)
            else:
                mr.moe_expert_gate_up(x, wg, wu, tables, h=h)
                ev[2].record()
                if weighted_down:
                    mr.moe_expert_down_weighted(h, wd, tables, expert_out=eo)
                else:
                    mr.moe_expert_down(h, wd, tables, expert_out=eo)
            ev[3].record()
        mr.moe_reduce_fused(eo, pos, None if weighted_down else wt, y=y)
        ev[len(names)].record()

    t = timed_calls(step, len(names), steps, warmup, flush, trials)
    per = dict(zip(names, t["parts"]))
    sizes = tables.group_sizes.cpu()
    nums = workload_numbers(d, sizes, weights, weighted_down)
    if fused:   # h is neither written nor read
        nums["experts_bytes"] = nums["gate_up_bytes"] + nums["down_bytes"] - 2 * nums["n_valid"] * D * x.element_size()
        nums["flops_experts"] = nums["flops"]
    return dict(d=d, tables=tables, block_m=block_m, ms=t["span"], trial_ms=t["trial_spans"],
                wall_incl_flush_ms=t["wall_incl_flush"], kernel_ms=per, nums=nums, gen_s=t_gen,
                quant_ms=quant_ms, weights=weights, name=cfg["name"], dtype=cfg["dtype"])


def mfma_peak(weights, dtype="bf16"):
    # W4A8 runs int8 MFMA (5.0 POP/s dense), MX the FP8 x FP4 scaled MFMA and
    # W8A8 the FP8 MFMA (5.0 PFLOP/s); the others bf16 / fp16 MFMA.
    if dtype == "f32":
        return 157.3
    return {"w4a8": MFMA_INT8_PEAK_TOPS, "mx": MFMA_FP8_PEAK_TFLOPS,
            "w8a8": MFMA_FP8_PEAK_TFLOPS}.get(weights, MFMA_BF16_PEAK_TFLOPS)


def summarize(r):
    nums, per = r["nums"], r["kernel_ms"]
    ms = r["ms"]
    peak = mfma_peak(r.get("weights"), r.get("dtype", "bf16"))
    gbs = lambda nbytes, t_ms: nbytes / (t_ms * 1e-3) / 1e9
    kernels = {}
    for n in per:
        key = n + "_bytes"
        kernels[n] = {"ms": round(per[n], 4), "algo_bytes": nums[key],
                      "GB_s": round(gbs(nums[key], per[n]), 1),
                      "hbm_frac": round(gbs(nums[key], per[n]) / HBM_PEAK_GBS, 4)}
    for n, key in (("gate_up", "flops_gate_up"), ("down", "flops_down"),
                   ("experts", "flops_experts")):
        if n not in per:
            continue
        kernels[n]["TFLOP_s" if r.get("weights") != "w4a8" else "TOP_s"] = \
            round(nums[key] / (per[n] * 1e-3) / 1e12, 2)
        t_roof = max(nums[n + "_bytes"] / (HBM_PEAK_GBS * 1e9), nums[key] / (peak * 1e12)) * 1e3
        kernels[n]["roofline_frac"] = round(t_roof / per[n], 4)
    tflops = nums["flops"] / (ms * 1e-3) / 1e12
    hbm = gbs(nums["b_min"], ms)
    t_roof_ms = max(nums["b_min"] / (HBM_PEAK_GBS * 1e9), nums["flops"] / (peak * 1e12)) * 1e3
    return dict(workload=r["name"], ms_per_layer=round(ms, 4), trial_ms=r["trial_ms"],
                TFLOP_s=round(tflops, 2), HBM_GB_s=round(hbm, 1),
                hbm_frac=round(hbm / HBM_PEAK_GBS, 4),
                mfma_frac=round(tflops / peak, 4),
                roofline_frac=round(t_roof_ms / ms, 4), roofline_ms=round(t_roof_ms, 4),
                flops=nums["flops"], b_min_bytes=nums["b_min"], n_valid=nums["n_valid"],
                active_experts=nums["e_active"], block_m=r["block_m"], kernels=kernels,
                quantize_ms=None if r.get("quant_ms") is None else round(r["quant_ms"], 3))


def compact(s):
    """The JSON line's short form of a workload summary: ms/layer, fractions
    of the roofline / HBM / MFMA peaks, and ms and roofline fraction per
    kernel."""
    k = s["kernels"]
    return {"ms": s["ms_per_layer"], "roof": s["roofline_frac"], "hbm": s["hbm_frac"],
            "mfma": s["mfma_frac"], "TF": s["TFLOP_s"],
            "k_ms": {n: k[n]["ms"] for n in k},
            "k_roof": {n: k[n]["roofline_frac"] for n in ("gate_up", "down", "experts") if n in k}}


def run_workload(cfg, args, dev, flush, **kw):
    import torch
    r = time_workload(cfg, args.steps, args.warmup, args.block_m, dev, flush, args.trials, **kw)
    r.pop("d")
    r.pop("tables")
    torch.cuda.empty_cache()
    s = summarize(r)
    print("# %s %s: %.4f ms/layer (trials %s), %.2f TFLOP/s, %.1f GB/s, roofline %.3f"
          % (cfg["name"], kw, s["ms_per_layer"], s["trial_ms"], s["TFLOP_s"], s["HBM_GB_s"],
             s["roofline_frac"]), file=sys.stderr, flush=True)
    return s


def time_w4a8_gemm(args, dev, flush):
    """The plain W4A8 GEMM (moe_w4a8_gemm) at the tutorial's two serving
    shapes, N = 3584, K = 18944: M = 1 (a GEMV-like decode step) and M = 32
    (a small batch). Seeded int8 A and random packed int4 B (34 MB, flushed
    from the caches before every call)."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    out = []
    N, K = 3584, 18944
    g = torch.Generator(device=dev).manual_seed(11)
    B = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.int16).to(torch.uint8)
    for name, M in (("gemv_like", 1), ("small_batch", 32)):
        A = torch.randint(-127, 128, (M, K), generator=g, device=dev, dtype=torch.int16).to(torch.int8)
        Ct = torch.empty((N, M), dtype=torch.int32, device=dev)

        def call(ev):
            ev[0].record()
            mr.w4a8_gemm(A, B, Ct=Ct)
            ev[1].record()
        ms = timed_calls(call, 1, args.steps, args.warmup, flush, args.trials)["span"]
        nbytes = N * K // 2 + M * K + N * M * 4
        out.append({"workload": "W4A8 GEMM %s M=%d N=%d K=%d" % (name, M, N, K),
                    "us": round(ms * 1e3, 2), "algo_bytes": nbytes,
                    "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    return out


def time_reduce(args, dev, flush):
    """The skewed workload's standalone moe_reduce_fused: expert_out [32768,
    7168], 10 % of the slots masked, in bf16 and in the quantized form (FP8
    E4M3 rows with a scale per row in, FP8 out with a scale per token), and
    the decode-shaped reduce (512 x 8 x 7168 bf16, every slot valid: the
    reduce PR's headline case). Bytes: the valid rows read once, y written
    once, positions and weights (and the scales) read once."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    cfg = S.CONFIGS[4]
    T, K, H = cfg["T"], cfg["K"], cfg["H"]
    d = S.make_reduce_inputs(T, K, H, dtype="bf16", seed=cfg["seed"], device=dev)
    x, pos, w = d["expert_out"], d["token_topk_to_pos"], d["topk_weights"]
    n_valid = int((pos >= 0).sum())
    out = []

    def timed(fn):
        def call(ev):
            ev[0].record()
            fn()
            ev[1].record()
        return timed_calls(call, 1, args.steps, args.warmup, flush, args.trials)["span"]

    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: mr.moe_reduce_fused(x, pos, w, y=y))
    out.append(("bf16", "skewed standalone reduce 4096x8x7168 bf16, 10% slots masked", ms,
                n_valid * H * 2 + T * H * 2 + T * K * 8))
    del y

    x8 = x.to(torch.float8_e4m3fn)
    del x, d
    g = torch.Generator().manual_seed(cfg["seed"] + 1)
    x_sf = (torch.rand(T * K, generator=g) * 0.05 + 0.01).to(dev)
    sf = (torch.rand(T, generator=g) * 4 + 1).to(dev)
    y8 = torch.empty(T, H, dtype=torch.float8_e4m3fn, device=dev)
    ms = timed(lambda: mr.moe_reduce_fused(x8, pos, w, y=y8, x_sf=x_sf, sf=sf))
    out.append(("fp8", "skewed standalone reduce 4096x8x7168 fp8 e4m3 + x_sf in, fp8 + sf out",
                ms, n_valid * H + T * H + T * K * 8 + n_valid * 4 + T * 4))
    del x8, y8

    Td = 512
    dd = S.make_reduce_inputs(Td, K, H, dtype="bf16", seed=2, mask_frac=0.0, device=dev)
    yd = torch.empty(Td, H, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: mr.moe_reduce_fused(dd["expert_out"], dd["token_topk_to_pos"],
                                           dd["topk_weights"], y=yd))
    out.append(("decode", "decode-shaped standalone reduce 512x8x7168 bf16", ms,
                Td * K * H * 2 + Td * H * 2 + Td * K * 8))
    res = {}
    for key, name, ms, nbytes in out:
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[key] = {"workload": name, "us": round(ms * 1e3, 2), "algo_bytes": nbytes,
                    "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return res


PROBE_CFG = dict(name="mfma-probe", dtype="bf16", T=4096, H=7168, D=2048, E=1, K=1,
                 renorm=False, zipf=False, seed=7)


def mfma_probe(args, dev, flush):
    """Labelled MFMA probe (not a workload of the metric): the gate/up and
    down kernels on one expert receiving 4096 rows (T=4096, top-1, E=1,
    d_hidden=7168, d_expert=2048): 16 row blocks of 256 share one expert's
    weights, so the kernels run compute-bound at the prefill tile shapes."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    cfg = PROBE_CFG
    d = S.make_moe_inputs(cfg, device=dev)
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 1, block_m=256)
    ws, h, eo = mr.forward_workspace(tables, cfg["H"], cfg["D"], torch.bfloat16)
    res = {}
    for name, fn, flops in (
            ("gate_up", lambda: mr.moe_expert_gate_up(d["x"], d["w_gate"], d["w_up"], tables, h=h),
             4 * 4096 * 7168 * 2048),
            ("down", lambda: mr.moe_expert_down(h, d["w_down"], tables, expert_out=eo),
             2 * 4096 * 7168 * 2048)):
        def call(ev, fn=fn):
            ev[0].record()
            fn()
            ev[1].record()
        ms = timed_calls(call, 1, args.steps, args.warmup, flush, args.trials)["span"]
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "TFLOP_s": round(tf, 1),
                     "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    res["workload"] = "MFMA probe: one expert, 4096 rows, 7168x2048 bf16, block_m 256"
    return res


def time_gate(args, dev, flush):
    """The router gate (moe_gate) at the decode and prefill shapes: logits
    [T, 256] from x [T, 7168] and an fp32 router [256, 7168], top-8, softmax,
    renormalised. An fp32 vector-ALU kernel (one fma chain per logit): FLOPs
    2*T*E*H against the fp32 vector peak; bytes x + router + logits + ids +
    weights."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    res = []
    for ci in (2, 3):
        cfg = S.CONFIGS[ci]
        d = S.make_moe_inputs(cfg, device=dev, weights=False)
        T, H, E, K = cfg["T"], cfg["H"], cfg["E"], cfg["K"]
        out = (torch.empty(T, K, dtype=torch.int32, device=dev),
               torch.empty(T, K, dtype=torch.float32, device=dev),
               torch.empty(T, E, dtype=torch.float32, device=dev))

        def call(ev):
            ev[0].record()
            mr.moe_gate(d["x"], d["router"], K, renorm=cfg["renorm"], out=out)
            ev[1].record()
        ms = timed_calls(call, 1, args.steps, args.warmup, flush, args.trials)["span"]
        flops = 2.0 * T * E * H
        nbytes = T * H * 2 + E * H * 4 + T * E * 4 + T * K * 8
        tf = flops / (ms * 1e-3) / 1e12
        res.append({"workload": "router gate, %s (T=%d, E=%d, H=%d, top-%d)"
                                % (cfg["name"], T, E, H, K),
                    "us": round(ms * 1e3, 2), "TFLOP_s": round(tf, 2),
                    "fp32_vector_frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                    "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del d
    return res


def host_info():
    """nproc (usable and online), the CPU model and the socket count of this host."""
    model, sockets = None, set()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name") and model is None:
                model = line.split(":", 1)[1].strip()
            elif line.startswith("physical id"):
                sockets.add(line.split(":", 1)[1].strip())
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "cpus_online": os.cpu_count(),
            "cpu_model": model, "sockets": len(sockets) or None}


def oracle_forward_seconds(cfg, n_tokens, dev, threads=None):
    """Seconds the oracle takes for the dispatch of the whole batch plus the
    forward of its first n_tokens tokens, and the token count used. The
    seeded inputs are generated on the device (the same values as on the
    host) and the experts those tokens use are copied to the host first;
    neither is timed."""
    import numpy as np
    import torch

    import oracle
    import synthetic as S
    d = S.make_moe_inputs(cfg, device=dev)
    T, K, E = cfg["T"], cfg["K"], cfg["E"]
    n = min(n_tokens, T)
    ids = d["topk_ids"].cpu().numpy()
    w = d["topk_weights"].cpu().numpy()
    sub = ids[:n]
    used = np.unique(sub[sub >= 0])
    remap = np.full(E, -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sub_ids = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
    sel = torch.from_numpy(used).long().to(dev)
    if cfg["dtype"] == "f32":
        st, dt = (lambda t: t.contiguous().cpu().numpy()), oracle.F32
    else:
        st = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        dt = oracle.BF16 if cfg["dtype"] == "bf16" else oracle.F16
    args = (st(d["x"][:n]), st(d["w_gate"][sel]), st(d["w_up"][sel]), st(d["w_down"][sel]))
    del d
    torch.cuda.empty_cache()
    prev = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        t0 = time.perf_counter()
        oracle.dispatch(ids, w, E, 32)
        oracle.moe_forward(dt, *args, sub_ids, w[:n], tokens=np.arange(n, dtype=np.int32))
        sec = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(prev)
    return sec, n


def cpu_baseline(args, dev):
    """The oracle (as it stands) on bounded samples: the decode workload's
    first --cpu-tokens tokens (the reported value, scaled to the layer), the
    tiny workload whole and the mid-size one on 64 tokens at all threads and
    at 1 thread, and the two T = 4096 workloads on 24 tokens."""
    import oracle
    import synthetic as S
    threads = oracle.num_threads()
    per = {}
    main = None
    for ci, n_tok, one in ((2, args.cpu_tokens, False), (0, 64, True), (1, 64, True),
                           (3, 24, False), (4, 24, False)):
        cfg = S.CONFIGS[ci]
        sec, n = oracle_forward_seconds(cfg, n_tok, dev)
        ms = sec * 1e3 * cfg["T"] / n
        e = {"ms_layer": round(ms, 1), "tokens": n}
        if one:
            sec1, _ = oracle_forward_seconds(cfg, n_tok, dev, threads=1)
            e["ms_layer_1thread"] = round(sec1 * 1e3 * cfg["T"] / n, 1)
        per[cfg["name"]] = e
        if ci == 2:
            main = (ms, n, sec)
        print("# cpu oracle %s: %s" % (cfg["name"], e), file=sys.stderr, flush=True)
    ms, n, sec = main
    return {"value": round(ms, 1), "unit": "ms/layer", "cores": threads, "kind": "oracle",
            "sample": "oracle dispatch of all 4096 pairs + forward of %d of 512 tokens of the "
                      "seeded decode workload (%.1f s), scaled by 512/%d; per_config: the other "
                      "workloads on the token counts given, also scaled to a layer" % (n, sec, n),
            "host": host_info(), "per_config": per}


def dump_routing(cfg, block_m, path):
    """Write {magic, T, K, E, H, D, dtype, block_m} + ids + weights for the C++
    driver (mixture_experts_routed_moe_amd/moe_bench_driver routing FILE)."""
    import numpy as np

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    d = S.make_moe_inputs(cfg, device="cpu", weights=False)
    T, H, D, E, K = d["T"], d["H"], d["D"], d["E"], d["K"]
    block_m = block_m or mr.default_block_m(T, K, E)
    code = {"f16": 0, "bf16": 1, "f32": 2}[cfg["dtype"]]
    hdr = np.array([0x4d6f4531, T, K, E, H, D, code, block_m], np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(d["topk_ids"].numpy().astype(np.int32).tobytes())
        f.write(d["topk_weights"].numpy().astype(np.float32).tobytes())
    print(json.dumps({"routing_dump": path, "workload": cfg["name"], "block_m": int(block_m)}))


def dump_reduce(path):
    """Write {magic, T, K, H} + positions + weights of the skewed workload's
    standalone reduce for the C++ driver (moe_bench_driver reduce FILE)."""
    import numpy as np

    import synthetic as S
    cfg = S.CONFIGS[4]
    T, K, H = cfg["T"], cfg["K"], cfg["H"]
    d = S.make_reduce_inputs(T, K, H, dtype="bf16", seed=cfg["seed"], device="cpu", rows=False)
    hdr = np.array([0x4d6f4532, T, K, H], np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(d["token_topk_to_pos"].numpy().astype(np.int32).tobytes())
        f.write(d["topk_weights"].numpy().astype(np.float32).tobytes())
    print(json.dumps({"reduce_dump": path, "T": T, "K": K, "H": H}))


def copy_calibration(dev):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 3}))


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE=%d)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import synthetic as S
    if args.dump_routing:
        cfg = PROBE_CFG if args.workload == -1 else S.CONFIGS[args.workload]
        dump_routing(cfg, args.block_m or (256 if args.workload == -1 else None),
                     args.dump_routing)
        return
    if args.dump_reduce:
        dump_reduce(args.dump_reduce)
        return
    import torch
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    legs = set(args.only.split(",")) if args.only else None
    want = lambda leg: legs is None or leg in legs
    flush = Flusher(dev, args.flush_mb, args.flush_mode)

    cfg = S.CONFIGS[args.workload]
    main_r = time_workload(cfg, args.steps, args.warmup, args.block_m, dev, flush, args.trials)
    main_s = summarize(main_r)
    print("# %s: %.4f ms/layer (trials %s), %.1f GB/s (%.1f%% of HBM peak), gen %.1fs"
          % (cfg["name"], main_s["ms_per_layer"], main_s["trial_ms"], main_s["HBM_GB_s"],
             100 * main_s["hbm_frac"], main_r["gen_s"]), file=sys.stderr, flush=True)
    print("# main detail: %s" % json.dumps(main_s), file=sys.stderr, flush=True)
    del main_r["d"], main_r["tables"]
    torch.cuda.empty_cache()

    tail = {}          # compact entries, printed last in the JSON line
    detail = {}
    if not args.no_t4096 and args.workload == 2:
        for key, ci in (("tiny", 0), ("mid", 1), ("t4096", 3), ("skewed", 4)):
            if key in ("tiny", "mid") and not want("small"):
                continue
            if key in ("t4096", "skewed") and not want(key):
                continue
            s = run_workload(S.CONFIGS[ci], args, dev, flush)
            detail[key] = s
            tail[key] = dict(compact(s), n_act=s["active_experts"])
    extras = {}
    variants = {}
    if not args.no_extras:
        if want("reduce"):
            extras["reduce_skewed"] = time_reduce(args, dev, flush)
            torch.cuda.empty_cache()
            tail["reduce_skewed"] = {k: {"us": v["us"], "hbm": v["hbm_frac"]}
                                     for k, v in extras["reduce_skewed"].items()}
        if want("probe"):
            extras["mfma_probe"] = mfma_probe(args, dev, flush)
            torch.cuda.empty_cache()
            tail["mfma_probe"] = {k: extras["mfma_probe"][k]["mfma_frac"] for k in ("gate_up", "down")}
        if want("gate"):
            extras["gate"] = time_gate(args, dev, flush)
            torch.cuda.empty_cache()
        for leg, kw in (("fp8", dict(weights="fp8")), ("w8a8", dict(weights="w8a8")),
                        ("w4a8", dict(weights="w4a8")), ("mx", dict(weights="mx")),
                        ("weighted", dict(weighted_down=True)), ("fused", dict(fused=True))):
            if not want(leg):
                continue
            if leg == "w8a8" and not hasattr(__import__("mixture_experts_routed_moe_amd"),
                                             "moe_expert_gate_up_w8a8"):
                continue
            for ci in ((2,) if leg == "fused" else (2, 3)):
                s = run_workload(S.CONFIGS[ci], args, dev, flush, **kw)
                extras.setdefault(leg, {})["T%d" % S.CONFIGS[ci]["T"]] = s
                variants["%s_T%d" % (leg, S.CONFIGS[ci]["T"])] = [s["ms_per_layer"],
                                                                  s["roofline_frac"]]
        if want("w4a8_gemm"):
            extras["w4a8_gemm"] = time_w4a8_gemm(args, dev, flush)
            torch.cuda.empty_cache()
        print("# extras: %s" % json.dumps(extras), file=sys.stderr, flush=True)
    if detail:
        print("# workloads: %s" % json.dumps(detail), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, dev)
        print("# cpu baseline: %s" % json.dumps(cpu), file=sys.stderr, flush=True)

    gu = main_s["kernels"]["gate_up"]
    achieved = gu["GB_s"]
    traffic = counter_traffic()
    line = {
        "metric": "routed-MoE fwd ms/layer + TFLOP/s & HBM GB/s vs peak at T=512, T=4096",
        "value": main_s["ms_per_layer"],
        "unit": "ms/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_s["ms_per_layer"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else cfg["dtype"],
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init expert weights, "
                "N(0,0.02) router, softmax top-k)",
        "config": {"workload": cfg["name"], "T": cfg["T"], "d_hidden": cfg["H"],
                   "d_expert": cfg["D"], "n_routed_experts": cfg["E"], "top_k": cfg["K"],
                   "block_m": main_s["block_m"]},
        "roofline": {"bound": "hbm", "kernel": "grouped_gemm gate/up (SiLU*up fused)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algo_bytes_per_launch": gu["algo_bytes"],
                     "avg_launch_ms": gu["ms"]},
        "cpu_baseline": cpu,
        "protocol": "%d trials x ~%d steps, median of trial means; %d MB %s flush before each "
                    "step" % (args.trials, max(1, args.steps // max(1, args.trials)),
                              args.flush_mb, args.flush_mode),
        "TFLOP_s": main_s["TFLOP_s"], "HBM_GB_s": main_s["HBM_GB_s"],
        "hbm_frac": main_s["hbm_frac"], "mfma_frac": main_s["mfma_frac"],
        "roofline_frac": main_s["roofline_frac"],
        "kernels": {n: [k["ms"], k["hbm_frac"]] for n, k in main_s["kernels"].items()},
        "variants": variants or None,
    }
    for key in ("tiny", "mid", "mfma_probe", "reduce_skewed", "skewed", "t4096"):
        if key in tail:
            line[key] = tail[key]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
