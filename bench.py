#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE forward on one MI355X.

One step = one pass of the whole hot path on one batch of synthetic input:
  moe_dispatch -> moe_expert_gate_up (SiLU*up fused) -> moe_expert_down
  -> moe_reduce_fused,
exactly the kernels moe_routed_forward launches after the dispatch, called
stage by stage so that HIP events (recorded on the stream the kernels run
on) time every kernel inside the timed region.

Workload (the metric's T = 512 case): the DeepSeek-shaped decode layer,
T=512, d_hidden=7168, d_expert=2048, E=256 routed experts, top-8, bf16,
seeded synthetic x / weights / router (no dataset, random-init weights).
The same line also carries the metric's T = 4096 case (the prefill layer
of the same shapes) under "t4096", and the CPU oracle timed on a bounded
sample of the decode workload under "cpu_baseline".

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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2,
                    help="index into synthetic.CONFIGS for the main line (default 2: decode T=512)")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--no-t4096", action="store_true", help="skip the T=4096 prefill case")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the standalone reduce and the MFMA probe")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=512,
                    help="tokens of the decode workload the oracle runs for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--dump-routing", default=None, metavar="FILE",
                    help="only write the workload's routing (ids, weights) for moe_bench_driver")
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
    h / expert_out written and read once, y written once; W4A8 adds the int8
    copies of x and h (and their scales), written once and read once."""
    T, H, D, E, K = d["T"], d["H"], d["D"], d["E"], d["K"]
    b = d["x"].element_size()
    wb = {"16bit": b, "fp8": 1, "w4a8": 0.5, "mx": 0.5 + 1 / 32}[weights]
    sc = 4 if weights in ("fp8", "w4a8") else 0   # scale bytes per weight row
    n_valid = int(tables_sizes.sum())
    e_active = int((tables_sizes > 0).sum())
    P = T * K
    w_gate_up = int(e_active * 2 * D * (H * wb + sc))
    w_down = int(e_active * H * (D * wb + sc))
    out = dict(n_valid=n_valid, e_active=e_active)
    if weights in ("w4a8", "mx"):
        # int8 + a 4-byte scale per row, or E4M3 + an E8M0 byte per 32 values
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


def time_workload(cfg, steps, warmup, block_m, dev, weights="16bit", weighted_down=False):
    """One workload's step timed kernel by kernel. weights "fp8" / "w4a8":
    the expert weights are quantized once (moe_quantize_fp8_rows /
    moe_quantize_int4_rows, timed on its own, not part of the step) and the
    step runs the FP8-weight GEMMs, or the W4A8 path (x and h quantised to
    int8 inside the step, each a timed kernel of its own). weighted_down
    (16-bit weights): the routing weight applied in the down GEMM's
    epilogue, then an unweighted reduce."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S

    t_gen = time.time()
    d = S.make_moe_inputs(cfg, device=dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    quant_ms = None
    if weights != "16bit":
        qfn = {"fp8": mr.quantize_fp8_rows, "w4a8": mr.quantize_int4_rows,
               "mx": mr.quantize_mx_weights}[weights]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        q = [qfn(d[n]) for n in ("w_gate", "w_up", "w_down")]
        ev[1].record()
        torch.cuda.synchronize()
        quant_ms = ev[0].elapsed_time(ev[1])
        d["w_gate"], d["w_up"], d["w_down"] = q
    T, H, D, E, K = d["T"], d["H"], d["D"], d["E"], d["K"]
    block_m = block_m or mr.default_block_m(T, K, E)
    ids, w = d["topk_ids"], d["topk_weights"]
    x, wg, wu, wd = d["x"], d["w_gate"], d["w_up"], d["w_down"]
    tables = mr.MoeTables(T, K, E, block_m, dev)
    if weights == "w4a8":
        ws, h, eo, xq, sx, hq, sh = mr.forward_w4a8_workspace(tables, H, D, x.dtype)
        names = ["dispatch", "quant_x", "gate_up", "quant_h", "down", "reduce"]
    elif weights == "mx":
        ws, h, eo, xq, sx, hq, sh = mr.forward_mx_workspace(tables, H, D, x.dtype)
        names = ["dispatch", "quant_x", "gate_up", "quant_h", "down", "reduce"]
    else:
        ws, h, eo = mr.forward_workspace(tables, H, D, x.dtype)
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

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    for _ in range(warmup):
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = {n: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps
           for j, n in enumerate(names)}
    span = sum(ev[0].elapsed_time(ev[len(names)]) for ev in events) / steps
    sizes = tables.group_sizes.cpu()
    nums = workload_numbers(d, sizes, weights, weighted_down)
    return dict(d=d, tables=tables, block_m=block_m, wall_ms=wall_ms, event_ms=span,
                kernel_ms=per, nums=nums, gen_s=t_gen, quant_ms=quant_ms, weights=weights)


def summarize(r):
    nums, per = r["nums"], r["kernel_ms"]
    ms = r["wall_ms"]
    gbs = lambda nbytes, t_ms: nbytes / (t_ms * 1e-3) / 1e9
    kernels = {}
    for n in per:
        key = n + "_bytes"
        kernels[n] = {"ms": round(per[n], 4), "algo_bytes": nums[key],
                      "GB_s": round(gbs(nums[key], per[n]), 1),
                      "hbm_frac": round(gbs(nums[key], per[n]) / HBM_PEAK_GBS, 4)}
    for n, key in (("gate_up", "flops_gate_up"), ("down", "flops_down")):
        kernels[n]["TFLOP_s" if r.get("weights") != "w4a8" else "TOP_s"] = \
            round(nums[key] / (per[n] * 1e-3) / 1e12, 2)
    # W4A8 runs int8 MFMA (5.0 POP/s dense), MX the FP8 x FP4 scaled MFMA
    # (5.0 PFLOP/s at the FP8 rate); the others bf16 / fp16 MFMA
    peak = {"w4a8": MFMA_INT8_PEAK_TOPS, "mx": MFMA_FP8_PEAK_TFLOPS}.get(r.get("weights"),
                                                                      MFMA_BF16_PEAK_TFLOPS)
    tflops = nums["flops"] / (ms * 1e-3) / 1e12
    hbm = gbs(nums["b_min"], ms)
    t_roof_ms = max(nums["b_min"] / (HBM_PEAK_GBS * 1e9), nums["flops"] / (peak * 1e12)) * 1e3
    return dict(ms_per_layer=round(ms, 4), event_ms_per_layer=round(r["event_ms"], 4),
                TFLOP_s=round(tflops, 2), HBM_GB_s=round(hbm, 1),
                hbm_frac=round(hbm / HBM_PEAK_GBS, 4),
                mfma_frac=round(tflops / peak, 4),
                roofline_frac=round(t_roof_ms / ms, 4), roofline_ms=round(t_roof_ms, 4),
                flops=nums["flops"], b_min_bytes=nums["b_min"], n_valid=nums["n_valid"],
                active_experts=nums["e_active"], block_m=r["block_m"], kernels=kernels)


def _time_rotating(fn, inputs, steps, warmup):
    """Average ms of fn(inp) over `steps` calls cycling through `inputs`
    (copies whose total exceeds the 256 MB last-level cache, so every call
    reads its rows from HBM)."""
    import torch
    for i in range(warmup):
        fn(inputs[i % len(inputs)])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn(inputs[i % len(inputs)])
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def time_w4a8_gemm(steps, warmup, dev):
    """The plain W4A8 GEMM (moe_w4a8_gemm) at the tutorial's two serving
    shapes, N = 3584, K = 18944: M = 1 (a GEMV-like decode step) and M = 32
    (a small batch). Seeded int8 A and random packed int4 B; 10 copies of B
    rotate so each call reads its weights from HBM."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    out = []
    N, K = 3584, 18944
    g = torch.Generator(device=dev).manual_seed(11)
    Bs = [torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.int16)
          .to(torch.uint8) for _ in range(10)]
    for name, M in (("gemv_like", 1), ("small_batch", 32)):
        A = torch.randint(-127, 128, (M, K), generator=g, device=dev, dtype=torch.int16).to(torch.int8)
        Ct = torch.empty((N, M), dtype=torch.int32, device=dev)
        ms = _time_rotating(lambda B: mr.w4a8_gemm(A, B, Ct=Ct), Bs, steps, warmup)
        nbytes = N * K // 2 + M * K + N * M * 4
        out.append({"workload": "W4A8 GEMM %s M=%d N=%d K=%d" % (name, M, N, K),
                    "us": round(ms * 1e3, 2), "algo_bytes": nbytes,
                    "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    return out


def time_reduce(steps, warmup, dev):
    """The skewed workload's standalone moe_reduce_fused: expert_out [32768,
    7168], 10 % of the slots masked, in bf16 and in the quantized form (FP8
    E4M3 rows with a scale per row in, FP8 out with a scale per token). Bytes:
    the valid rows read once, y written once, positions and weights (and the
    scales) read once."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    cfg = S.CONFIGS[4]
    T, K, H = cfg["T"], cfg["K"], cfg["H"]
    d = S.make_reduce_inputs(T, K, H, dtype="bf16", seed=cfg["seed"], device=dev)
    x, pos, w = d["expert_out"], d["token_topk_to_pos"], d["topk_weights"]
    n_valid = int((pos >= 0).sum())
    out = []

    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    xs = [x, x.clone()]
    ms = _time_rotating(lambda xi: mr.moe_reduce_fused(xi, pos, w, y=y), xs, steps, warmup)
    nbytes = n_valid * H * 2 + T * H * 2 + T * K * 8
    out.append(("skewed standalone reduce 4096x8x7168 bf16, 10% slots masked", ms, nbytes))
    del xs, y

    x8 = [x.to(torch.float8_e4m3fn) for _ in range(3)]
    del x, d
    g = torch.Generator().manual_seed(cfg["seed"] + 1)
    x_sf = (torch.rand(T * K, generator=g) * 0.05 + 0.01).to(dev)
    sf = (torch.rand(T, generator=g) * 4 + 1).to(dev)
    y8 = torch.empty(T, H, dtype=torch.float8_e4m3fn, device=dev)
    ms = _time_rotating(lambda xi: mr.moe_reduce_fused(xi, pos, w, y=y8, x_sf=x_sf, sf=sf), x8,
                        steps, warmup)
    nbytes = n_valid * H + T * H + T * K * 8 + n_valid * 4 + T * 4
    out.append(("skewed standalone reduce 4096x8x7168 fp8 e4m3 + x_sf in, fp8 + sf out", ms,
                nbytes))
    res = []
    for name, ms, nbytes in out:
        gbs = nbytes / (ms * 1e-3) / 1e9
        res.append({"workload": name, "ms": round(ms, 4), "algo_bytes": nbytes,
                    "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    return res


def mfma_probe(steps, warmup, dev):
    """Labelled MFMA probe (not a workload of the metric): the gate/up and
    down kernels on one expert receiving 4096 rows (T=4096, top-1, E=1,
    d_hidden=7168, d_expert=2048): 16 row blocks of 256 share one expert's
    weights, so the kernels run compute-bound at the prefill tile shapes."""
    import torch

    import mixture_experts_routed_moe_amd as mr
    import synthetic as S
    cfg = dict(name="mfma-probe", dtype="bf16", T=4096, H=7168, D=2048, E=1, K=1,
               renorm=False, zipf=False, seed=7)
    d = S.make_moe_inputs(cfg, device=dev)
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 1, block_m=256)
    ws, h, eo = mr.forward_workspace(tables, cfg["H"], cfg["D"], torch.bfloat16)
    res = {}
    for name, fn, flops in (
            ("gate_up", lambda: mr.moe_expert_gate_up(d["x"], d["w_gate"], d["w_up"], tables, h=h),
             4 * 4096 * 7168 * 2048),
            ("down", lambda: mr.moe_expert_down(h, d["w_down"], tables, expert_out=eo),
             2 * 4096 * 7168 * 2048)):
        for _ in range(warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "TFLOP_s": round(tf, 1),
                     "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    res["workload"] = "MFMA probe: one expert, 4096 rows, 7168x2048 bf16, block_m 256"
    return res


def time_gate(steps, warmup, dev):
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
        fn = lambda: mr.moe_gate(d["x"], d["router"], K, renorm=cfg["renorm"], out=out)
        for _ in range(warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        flops = 2.0 * T * E * H
        nbytes = T * H * 2 + E * H * 4 + T * E * 4 + T * K * 8
        tf = flops / (ms * 1e-3) / 1e12
        res.append({"workload": "router gate, %s (T=%d, E=%d, H=%d, top-%d)" % (cfg["name"], T, E,
                                                                               H, K),
                    "us": round(ms * 1e3, 2), "TFLOP_s": round(tf, 2),
                    "fp32_vector_frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                    "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del d
    return res


def cpu_baseline(r, n_tokens):
    """The oracle (as it stands) on the first n_tokens tokens of the workload,
    plus its dispatch of the whole batch; time scaled to the whole layer."""
    import numpy as np
    import torch

    import oracle

    d = r["d"]
    T, K, E = d["T"], d["K"], d["E"]
    n_tokens = min(n_tokens, T)
    tokens = np.arange(n_tokens, dtype=np.int32)
    ids = d["topk_ids"].cpu().numpy()
    w = d["topk_weights"].cpu().numpy()
    sub = ids[:n_tokens]
    used = np.unique(sub[sub >= 0])
    remap = np.full(E, -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sub_ids = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
    sel = torch.from_numpy(used).long().to(d["x"].device)
    bits = lambda t: t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    xs, gs, us, ds = (bits(d["x"][:n_tokens]), bits(d["w_gate"][sel]), bits(d["w_up"][sel]),
                      bits(d["w_down"][sel]))
    t0 = time.perf_counter()
    oracle.dispatch(ids, w, E, r["block_m"])
    t_disp = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.moe_forward(oracle.BF16, xs, gs, us, ds, sub_ids, w[:n_tokens], tokens=tokens)
    t_fwd = time.perf_counter() - t0
    ms = (t_disp + t_fwd * T / n_tokens) * 1e3
    return {"value": round(ms, 1), "unit": "ms/layer", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "oracle forward on %d of %d tokens (%d routed pairs, %.1f s) scaled by "
                      "T/%d, plus its dispatch of all %d pairs (%.3f s); same seeded "
                      "decode workload" % (n_tokens, T, n_tokens * K, t_fwd, n_tokens, T * K,
                                           t_disp)}


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
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE=%d)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import synthetic as S
    if args.dump_routing:
        dump_routing(S.CONFIGS[args.workload], args.block_m, args.dump_routing)
        return
    import torch
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return

    cfg = S.CONFIGS[args.workload]
    main_r = time_workload(cfg, args.steps, args.warmup, args.block_m, dev)
    main_s = summarize(main_r)
    print("# %s: %.4f ms/layer, %.1f GB/s (%.1f%% of HBM peak), gen %.1fs"
          % (cfg["name"], main_s["ms_per_layer"], main_s["HBM_GB_s"], 100 * main_s["hbm_frac"],
             main_r["gen_s"]), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(main_r, args.cpu_tokens)
        print("# cpu baseline: %s" % json.dumps(cpu), file=sys.stderr, flush=True)
    main_d = main_r.pop("d")
    del main_d, main_r["tables"]
    torch.cuda.empty_cache()

    t4096 = None
    if not args.no_t4096 and args.workload == 2:
        r3 = time_workload(S.CONFIGS[3], args.steps, args.warmup, None, dev)
        r3.pop("d")
        r3.pop("tables")
        torch.cuda.empty_cache()
        t4096 = summarize(r3)
        t4096["workload"] = S.CONFIGS[3]["name"]
        print("# %s: %.4f ms/layer, %.2f TFLOP/s, %.1f GB/s"
              % (S.CONFIGS[3]["name"], t4096["ms_per_layer"], t4096["TFLOP_s"],
                 t4096["HBM_GB_s"]), file=sys.stderr, flush=True)

    extras = {}
    if not args.no_extras:
        extras["reduce_skewed"] = time_reduce(args.steps, args.warmup, dev)
        torch.cuda.empty_cache()
        extras["mfma_probe"] = mfma_probe(args.steps, args.warmup, dev)
        torch.cuda.empty_cache()
        extras["gate"] = time_gate(args.steps, args.warmup, dev)
        torch.cuda.empty_cache()
        fp8 = {}
        for ci in (2, 3):
            r8 = time_workload(S.CONFIGS[ci], args.steps, args.warmup, None, dev, weights="fp8")
            r8.pop("d")
            r8.pop("tables")
            torch.cuda.empty_cache()
            s8 = summarize(r8)
            s8["quantize_ms"] = round(r8["quant_ms"], 3)
            s8["workload"] = S.CONFIGS[ci]["name"] + " with FP8 E4M3 expert weights (per-row scales)"
            fp8["T%d" % S.CONFIGS[ci]["T"]] = s8
        extras["fp8_weights"] = fp8
        w4 = {}
        for ci in (2, 3):
            r4 = time_workload(S.CONFIGS[ci], args.steps, args.warmup, None, dev, weights="w4a8")
            r4.pop("d")
            r4.pop("tables")
            torch.cuda.empty_cache()
            s4 = summarize(r4)
            s4["quantize_ms"] = round(r4["quant_ms"], 3)
            s4["workload"] = (S.CONFIGS[ci]["name"] + " with W4A8 experts (int4 weights, per-row "
                              "scales; int8 activations, per-row scales)")
            w4["T%d" % S.CONFIGS[ci]["T"]] = s4
        extras["w4a8"] = w4
        mx = {}
        for ci in (2, 3):
            rm = time_workload(S.CONFIGS[ci], args.steps, args.warmup, None, dev, weights="mx")
            rm.pop("d")
            rm.pop("tables")
            torch.cuda.empty_cache()
            sm = summarize(rm)
            sm["quantize_ms"] = round(rm["quant_ms"], 3)
            sm["workload"] = (S.CONFIGS[ci]["name"] + " with MX experts (MXFP4 weights, MXFP8 "
                              "activations, E8M0 scales per 32 values)")
            mx["T%d" % S.CONFIGS[ci]["T"]] = sm
        extras["mx"] = mx
        wdn = {}
        for ci in (2, 3):
            rw = time_workload(S.CONFIGS[ci], args.steps, args.warmup, None, dev,
                               weighted_down=True)
            rw.pop("d")
            rw.pop("tables")
            torch.cuda.empty_cache()
            sw = summarize(rw)
            sw["workload"] = (S.CONFIGS[ci]["name"] + " with the routing weight in the down "
                              "epilogue and an unweighted reduce")
            wdn["T%d" % S.CONFIGS[ci]["T"]] = sw
        extras["weighted_down"] = wdn
        extras["w4a8_gemm"] = time_w4a8_gemm(args.steps, args.warmup, dev)
        torch.cuda.empty_cache()
        print("# %s" % json.dumps(extras), file=sys.stderr, flush=True)

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
        "TFLOP_s": main_s["TFLOP_s"], "HBM_GB_s": main_s["HBM_GB_s"],
        "hbm_frac": main_s["hbm_frac"], "mfma_frac": main_s["mfma_frac"],
        "roofline_frac": main_s["roofline_frac"],
        "roofline": {"bound": "hbm", "kernel": "grouped_gemm gate/up (SiLU*up fused)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algo_bytes_per_launch": gu["algo_bytes"],
                     "avg_launch_ms": gu["ms"]},
        "kernels": main_s["kernels"],
        "t4096": t4096,
        "reduce_skewed": extras.get("reduce_skewed"),
        "mfma_probe": extras.get("mfma_probe"),
        "gate": extras.get("gate"),
        "fp8_weights": extras.get("fp8_weights"),
        "w4a8": extras.get("w4a8"),
        "w4a8_gemm": extras.get("w4a8_gemm"),
        "weighted_down": extras.get("weighted_down"),
        "mx": extras.get("mx"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
