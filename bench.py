"""Benchmark: W4A8 GEMM TOPS and weight-stream GB/s on the Llama-2-70B linear
shapes (N=28672,K=8192 and N=8192,K=28672; group 128) for M in
{1, 16, 128, 1024, 4096}, on one MI355X.

One step = the ten W4A8 GEMMs of that sweep (fp16 output, fused epilogue),
inputs resident in HBM.  Each GEMM slot owns a distinct copy of its packed
weights (10 x 121 MB), so a slot's weights are evicted from the 256 MB
Infinity Cache by the others before they are read again.

Prints one JSON line.  `value` = whole-step TOPS (sum of 2*M*N*K over the
step / step time).  Per-slot kernel times come from HIP events recorded on
the stream the kernels run on.  `cpu_baseline` times the CPU oracle (decode
+ int32 GEMM + epilogue) on a bounded sample of the same sweep.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402  (seeded inputs and shapes only)

METRIC = ("W4A8 GEMM TOPS + weight-stream GB/s at Llama-7B/70B linear shapes, "
          "M=1..4096")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
CFG = wl.LLAMA70B_SWEEP
DOMINANT_SLOT = "upgate:M4096"  # 4096 x 28672 x 8192: the largest share of a step
MS = (1, 16, 128, 1024, 4096)


def weight_bytes(N, K, g):
    return N * K // 2 + 2 * N * (K // g)


def algo_bytes(M, N, K, g):
    """Weights + scales + X + sx + Y (fp16): what the method must move."""
    return weight_bytes(N, K, g) + 4 * N + M * K + 4 * M + 2 * M * N


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", default="", help="run one slot, e.g. upgate:M4096")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp8", action="store_true")
    p.add_argument("--no-ablation", action="store_true")
    p.add_argument("--no-moe", action="store_true")
    p.add_argument("--cpu-sample-cols", type=int, default=256)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain 256 MiB device-to-device copies (the known-size "
                        "kernel that scales the HBM byte counters)")
    return p.parse_args()


def _code_only(text):
    """C/C++ source without comments and blank space: the part of a kernel
    source that the compiler sees (string and character literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest():
    """sha256 of the kernel sources without their comments: counter readings
    taken from other code no longer describe the kernels that run."""
    import hashlib
    d = os.path.join(ROOT, "w4a8_quantized_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def profiled_traffic(slot_name):
    """HBM bytes per launch of `slot_name`'s kernel from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by
    what the same counter reads for a copy of known size), or None when no
    summary exists or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{slot_name.replace(':', '_')}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != source_digest():
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None
    return round((fetch + write) * 1024.0)


def calibrate_copy():
    """Plain device-to-device copies of 256 MiB (read 256 MiB, write
    256 MiB per dispatch) for scaling FETCH_SIZE / WRITE_SIZE readings."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 4}), flush=True)


def cpu_baseline(slots_desc, ncols):
    """Oracle (test infrastructure) timed on the host cores: identity decode,
    int32 GEMM and fp16 epilogue for every slot of the sweep, restricted to
    `ncols` output channels per slot; scaled to the full step."""
    import numpy as np
    import oracle
    import workloads as wl
    total_ops_full = 0.0
    t_scaled = 0.0
    per_pair = {}
    for (tag, M, N, K, g, pair) in slots_desc:
        if pair not in per_pair:
            # numpy draws row-major: a smaller draw with the same seed is
            # exactly the leading rows of the full matrices the GPU uses
            W = wl.gen_weights(ncols, K, wl.seed_w(CFG, pair))
            X = wl.gen_activations(max(MS), K, wl.seed_x(CFG, max(MS)),
                                   wl.seed_outliers(CFG))
            X8_all, sx_all = oracle.quant_sym_rows(X, 127)
            per_pair[pair] = (oracle.w4a8_pack(W, g), X8_all, sx_all)
        pk, X8_all, sx_all = per_pair[pair]
        X8, sx = X8_all[:M], sx_all[:M]
        t0 = time.perf_counter()
        oracle.w4a8_gemm(X8, sx, pk, g)
        dt = time.perf_counter() - t0
        t_scaled += dt * (N / ncols)
        total_ops_full += 2.0 * M * N * K
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": total_ops_full / t_scaled / 1e12, "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"each of the 10 GEMMs of the sweep on {ncols} of its N output "
                      f"channels (decode + int32 GEMM + fp16 epilogue), time scaled by "
                      f"N/{ncols}; {t_scaled:.1f} s projected for one full step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import numpy as np
    import torch
    import w4a8_quantized_gemm_amd as w4
    import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    pairs = wl.nk_pairs(CFG)           # [(28672, 8192), (8192, 28672)]
    tags = {pairs[0]: "upgate", pairs[1]: "down"}
    g = 128

    # ---- inputs: packed weights (one copy per slot), activations per shape
    slots = []
    for pi, (N, K) in enumerate(pairs):
        Wf = torch.from_numpy(wl.gen_weights(N, K, wl.seed_w(CFG, pi))).to(dev)
        pk = w4.pack(Wf, group=g)
        del Wf
        Xf = torch.from_numpy(wl.gen_activations(max(MS), K, wl.seed_x(CFG, max(MS)),
                                                 wl.seed_outliers(CFG))).to(dev)
        Xq, sx = w4.quant_act(Xf)
        del Xf
        for M in MS:
            name = f"{tags[(N, K)]}:M{M}"
            if args.only and args.only != name:
                continue
            copy = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in pk.items()}
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            slots.append({"name": name, "M": M, "N": N, "K": K, "pair": pi, "pk": copy,
                          "X": Xq[:M], "sx": sx[:M], "Y": Y})
        del pk
    torch.cuda.synchronize()
    if not slots:
        print(f"unknown slot {args.only}", file=sys.stderr)
        sys.exit(2)

    # HIP events inside the timed region bracket only the dominant slot (the
    # largest share of the step), whose kernel the roofline reports: each
    # further event pair cost about 6 us of step time (measured: events on
    # the four M >= 1024 slots, 2.065 ms per step; on this slot alone, 2.047,
    # equal to none).
    evslots = ([i for i, s in enumerate(slots) if s["name"] == DOMINANT_SLOT]
               or list(range(len(slots))))
    evpos = {i: j for j, i in enumerate(evslots)}

    def step(evs=None):
        for i, s in enumerate(slots):
            ev = evs is not None and i in evpos
            if ev:
                evs[evpos[i]][0].record(stream)
            w4.gemm(s["X"], s["sx"], s["pk"], out=s["Y"])
            if ev:
                evs[evpos[i]][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in evslots] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ev_us = {}
    for i in evslots:
        times = np.array([evs[k][evpos[i]][0].elapsed_time(evs[k][evpos[i]][1])
                          for k in range(args.steps)]) * 1e3
        ev_us[i] = times

    # Per-slot figures of the other slots, outside the timed region: bursts
    # of back-to-back launches rotating through the weight copies of all
    # slots of the same shape (5 x 121 MB, more than the 256 MB Infinity
    # Cache), so a launch never finds its weights cached; events bracket the
    # burst only, so a launch's figure includes the gap to the next dispatch.
    burst_us = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i, s in enumerate(slots):
        if i in ev_us:
            continue
        copies = [t["pk"] for t in slots if t["pair"] == s["pair"]]
        reps = 20
        for r in range(2):
            w4.gemm(s["X"], s["sx"], copies[r % len(copies)], out=s["Y"])
        e0.record(stream)
        for r in range(reps):
            w4.gemm(s["X"], s["sx"], copies[r % len(copies)], out=s["Y"])
        e1.record(stream)
        torch.cuda.synchronize()
        burst_us[i] = e0.elapsed_time(e1) * 1e3 / reps

    sweep = []
    total_ops = 0.0
    kern_ms_sum = 0.0
    for i, s in enumerate(slots):
        M, N, K = s["M"], s["N"], s["K"]
        us = float(np.mean(ev_us[i])) if i in ev_us else burst_us[i]
        ops = 2.0 * M * N * K
        total_ops += ops
        kern_ms_sum += us / 1e3
        wgbs = weight_bytes(N, K, g) / (us * 1e-6) / 1e9
        row = {"slot": s["name"], "M": M, "N": N, "K": K, "group": g,
               "us_mean": round(us, 2),
               "timing": "events in timed region" if i in ev_us else "back-to-back burst",
               "tops": round(ops / (us * 1e-6) / 1e12, 2),
               "weight_stream_gbs": round(wgbs, 1),
               "hbm_frac_algo": round(algo_bytes(M, N, K, g) / (us * 1e-6) / 1e9
                                      / HBM_PEAK_GBS, 4),
               "mfma_frac": round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
        if i in ev_us:
            row["us_min"] = round(float(ev_us[i].min()), 2)
        else:
            row["launches_per_burst"] = 20
        sweep.append(row)

    value = total_ops / (ms_per_step * 1e-3) / 1e12

    def roof(slot_name, bound):
        e = next((x for x in sweep if x["slot"] == slot_name), None)
        if e is None:
            return None
        if bound == "mfma":
            a = 2.0 * e["M"] * e["N"] * e["K"] / (e["us_mean"] * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": INT8_PEAK_TOPS,
                    "unit": "TFLOP/s", "frac": round(a / INT8_PEAK_TOPS, 4),
                    "traffic": profiled_traffic(slot_name), "kernel_slot": slot_name,
                    "us_per_launch": e["us_mean"], "timing": e["timing"]}
        a = algo_bytes(e["M"], e["N"], e["K"], g) / (e["us_mean"] * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(slot_name),
                "kernel_slot": slot_name,
                "us_per_launch": e["us_mean"], "timing": e["timing"]}

    # dominant kernel: the slot with the largest share of the step (among
    # those timed with events inside the timed region)
    dom = max((sweep[i] for i in evslots), key=lambda e: e["us_mean"])
    dom_bound = "mfma" if dom["M"] >= 1024 else "hbm"
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "llama2-70b linear sweep (W4A8, group 128)",
                   "shapes_NK": [list(p) for p in pairs], "M": list(MS),
                   "slots": [s["name"] for s in slots], "out": "fp16",
                   "weights_per_slot_MB": round(weight_bytes(*pairs[0], g) / 1e6, 1),
                   "parallelism": "single GPU"},
        "roofline": roof(dom["slot"], dom_bound),
        "roofline_decode": roof("upgate:M16", "hbm") or roof("down:M16", "hbm"),
        "kernel_ms_per_step": round(kern_ms_sum, 4),
        "sweep": sweep,
    }

    # ---- decode ablation on the matrix-core slots (outside the timed step):
    # the production LiquidQuant decode interleaved with the matrix cores, the
    # conventional signed affine decode, and the LiquidQuant decode done per
    # K-step in one block, all three on the 32 x 32 x 32 tile kernel.  Same
    # codes, same results bit for bit.
    if not args.no_ablation:
        abl = []
        names = {w4.ABL_LQQ: "lqq", w4.ABL_AFFINE16: "affine16", w4.ABL_LQQ_COARSE: "lqq_coarse"}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for sl in slots:
            if sl["M"] < 1024:
                continue
            row = {"slot": sl["name"]}
            # the weight copies of every slot of this shape in turn, as in the
            # sweep's bursts, so that no launch finds its weights in the cache
            copies = [t["pk"] for t in slots if t["pair"] == sl["pair"]]
            for v, nm in names.items():
                w4.gemm_ablation(v, sl["X"], sl["sx"], copies[-1], out=sl["Y"])
                reps = 2 * len(copies)
                e0.record(stream)
                for r in range(reps):
                    w4.gemm_ablation(v, sl["X"], sl["sx"], copies[r % len(copies)], out=sl["Y"])
                e1.record(stream)
                torch.cuda.synchronize()
                row[nm + "_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
            # the production kernel choice for the same slot (from the sweep)
            row["w4a8_gemm_us"] = next(r["us_mean"] for r in sweep if r["slot"] == sl["name"])
            row["affine16_vs_lqq"] = round(row["affine16_us"] / row["lqq_us"], 3)
            row["coarse_vs_lqq"] = round(row["lqq_coarse_us"] / row["lqq_us"], 3)
            abl.append(row)
        out["ablation"] = abl

    # ---- W4A8 against W8A8 on the same skeletons (the first quantisation
    # level alone, 1 byte per weight, no decode), per slot of the sweep: the
    # memory-bound slots should favour W4A8's halved weight stream, the
    # compute-bound ones show what the decode costs against none
    if not args.no_ablation and not args.only:
        cmp_rows = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for pi, (N, K) in enumerate(pairs):
            Wf = torch.from_numpy(wl.gen_weights(N, K, wl.seed_w(CFG, pi))).to(dev)
            pk8 = w4.pack_w8(Wf)
            # two copies used alternately: each is evicted from the 256 MB
            # Infinity Cache by the other between its uses
            pk8b = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in pk8.items()}
            del Wf
            for sl in slots:
                if sl["pair"] != pi:
                    continue
                for _ in range(3):
                    w4.gemm_w8a8(sl["X"], sl["sx"], pk8, out=sl["Y"])
                reps = 10 if sl["M"] >= 1024 else 20
                e0.record(stream)
                for r in range(reps):
                    w4.gemm_w8a8(sl["X"], sl["sx"], pk8 if r % 2 == 0 else pk8b, out=sl["Y"])
                e1.record(stream)
                torch.cuda.synchronize()
                us8 = e0.elapsed_time(e1) * 1e3 / reps
                w4us = next(x["us_mean"] for x in sweep if x["slot"] == sl["name"])
                cmp_rows.append({"slot": sl["name"], "w8a8_us": round(us8, 2), "w4a8_us": w4us,
                                 "w8a8_vs_w4a8": round(us8 / w4us, 3)})
            del pk8, pk8b
        out["w8a8_compare"] = {"note": "W8A8 timed back-to-back alternating two weight "
                                       "copies (events over 10-20 launches); W4A8 from the "
                                       "sweep (rotating weight copies)",
                               "results": cmp_rows}

    # ---- grouped (mixture-of-experts) GEMM: Mixtral-8x7B expert layers, 8
    # experts with top-2 routing drawn from a seeded generator (each token to
    # two distinct experts), synthetic weights and activations of those shapes
    if not args.no_moe and not args.only:
        rng = np.random.default_rng(8)
        E, g_moe = 8, 128
        moe = []
        for (Nm, Km, tag) in ((14336, 4096, "up"), (4096, 14336, "down")):
            Ws = torch.from_numpy(np.stack([wl.gen_weights(Nm, Km, 800 + e) for e in range(E)]))
            pkm = w4.pack_experts(Ws.to(dev), group=g_moe)
            del Ws
            # two copies of the expert weights used in turn (2 x 240 MB)
            pkms = [pkm, {k: (v.clone() if torch.is_tensor(v) else v) for k, v in pkm.items()}]
            for T in (16, 2048):
                picks = np.stack([rng.choice(E, 2, replace=False) for _ in range(T)])
                counts = np.bincount(picks.ravel(), minlength=E)
                offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
                Mm = int(counts.sum())
                Xm = torch.from_numpy(wl.gen_activations(Mm, Km, 900 + T, 901)).to(dev)
                Xq_m, sx_m = w4.quant_act(Xm)
                Ym = torch.empty((Mm, Nm), dtype=torch.float16, device=dev)
                mr = int(counts.max())
                for r in range(3):
                    w4.gemm_grouped(Xq_m, sx_m, offs, pkms[r % 2], mr, out=Ym)
                reps = 10
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for r in range(reps):
                    w4.gemm_grouped(Xq_m, sx_m, offs, pkms[r % 2], mr, out=Ym)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                active = int((counts > 0).sum())
                wbytes = active * weight_bytes(Nm, Km, g_moe)
                moe.append({"layer": tag, "N": Nm, "K": Km, "tokens": T, "rows": Mm,
                            "max_rows_per_expert": mr, "active_experts": active,
                            "us": round(us, 2),
                            "tops": round(2.0 * Mm * Nm * Km / (us * 1e-6) / 1e12, 2),
                            "weight_stream_gbs": round(wbytes / (us * 1e-6) / 1e9, 1)})
            del pkm, pkms
        out["variant_moe"] = {"workload": "Mixtral-8x7B expert layers, 8 experts top-2, "
                                          "W4A8 group 128, fp16 out; events over 10 back-to-back "
                                          "launches alternating two copies of the expert weights",
                              "results": moe}

    # ---- FP8 variants (INT4 weights x e4m3 activations), reported alongside:
    # per-channel scales, and per-group scales folded into the FP8 weights
    # with a per-tensor rescale; prefill shape and a 16-token decode shape
    if not args.no_fp8 and not args.only:
        sh = wl.CONFIGS[wl.FP8_VARIANT].shapes[0]
        Wf = torch.from_numpy(wl.gen_weights(sh.N, sh.K, wl.seed_w(wl.FP8_VARIANT))).to(dev)
        pk8 = w4.pack(Wf, mode=w4.PACK_INT4_SYM)
        pk8g = w4.pack_fp8g(Wf, group=128)
        del Wf
        # weight copies used in turn, more bytes than the 256 MB Infinity
        # Cache, so no launch finds its weights cached from the previous use
        ncp = int(300e6 // (sh.N * sh.K // 2)) + 1
        cps8 = [pk8] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in pk8.items()}
                        for _ in range(ncp - 1)]
        cps8g = [pk8g] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in pk8g.items()}
                          for _ in range(ncp - 1)]
        Xf = torch.from_numpy(wl.gen_activations(sh.M, sh.K, wl.seed_x(wl.FP8_VARIANT),
                                                 wl.seed_outliers(wl.FP8_VARIANT))).to(dev)
        X8, sx8 = w4.quant_act_fp8(Xf)
        del Xf

        def timed(fn, reps):
            for r in range(3):
                fn(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for r in range(reps):
                fn(r)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        res = {}
        for M in (sh.M, 16):
            Yb = torch.empty((M, sh.N), dtype=torch.bfloat16, device=dev)
            Xm, sxm = X8[:M], sx8[:M]
            for tag, fn in (("per_channel",
                             lambda r: w4.gemm_fp8(Xm, sxm, cps8[r % ncp], out=Yb)),
                            ("group128_folded",
                             lambda r: w4.gemm_fp8g(Xm, sxm, cps8g[r % ncp], out=Yb))):
                us = timed(fn, 20)
                tf = 2.0 * M * sh.N * sh.K / (us * 1e-6) / 1e12
                wb = sh.N * sh.K / 2 + (sh.N * 4 if tag == "per_channel"
                                        else sh.N * sh.K // 128 * 4 + 4)
                ab = wb + M * sh.K + M * 4 + M * sh.N * 2
                res[f"{tag}_M{M}"] = {"us": round(us, 2), "tflops": round(tf, 2),
                                      "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4),
                                      "hbm_frac_algo": round(ab / (us * 1e-6) / 1e9
                                                             / HBM_PEAK_GBS, 4)}
        out["variant_fp8"] = {"workload": f"int4-fp8 N={sh.N} K={sh.K}, M={sh.M} and 16, "
                                          "bf16 out; events over 20 back-to-back launches "
                                          f"rotating {ncp} weight copies",
                              "results": res}
        del pk8, pk8g, cps8, cps8g, X8

    # ---- per-token activation quantisation, the step before every GEMM:
    # fp16 X -> INT8 codes (W4A8) or e4m3 codes (W4FP8) plus float32 row
    # scales, at the sweep's activation shapes.  HBM bound: 2 bytes read and
    # 1 written per value; copies of X used in turn past 512 MB in total
    # where that fits, so the large shapes stream from HBM (the 16-row ones
    # are a few hundred KB and launch bound whatever the copies).
    if not args.no_ablation and not args.only:
        qres = []
        for (M, K) in ((16, 8192), (16, 28672), (4096, 8192), (4096, 28672)):
            ncp = max(2, min(8, int(512e6 // (M * K * 2)) + 1))
            Xs = [torch.randn((M, K), device=dev).to(torch.float16) for _ in range(ncp)]
            Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
            Xe = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sq = torch.empty(M, dtype=torch.float32, device=dev)
            row = {"M": M, "K": K, "x_copies": ncp}
            for tag, fn, Yq in (("int8", lambda r: w4.quant_act(Xs[r % ncp], out=(Xq, sq)), Xq),
                                ("e4m3", lambda r: w4.quant_act_fp8(Xs[r % ncp], out=(Xe, sq)),
                                 Xe)):
                # the launches are captured in a HIP graph and replayed: the
                # 16-row kernels take less time than a launch from Python
                reps = 20
                fn(reps - 1)
                torch.cuda.synchronize()
                want = Yq.clone()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    for r in range(3):
                        fn(r)
                torch.cuda.current_stream().wait_stream(side)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for r in range(reps):
                        fn(r)
                graph.replay()
                torch.cuda.synchronize()
                if not torch.equal(Yq, want):
                    raise RuntimeError(f"quant_act {tag} {M}x{K}: graph replay differs")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                del graph
                ab = 3 * M * K + 4 * M
                row[tag + "_us"] = round(us, 2)
                row[tag + "_gbs"] = round(ab / (us * 1e-6) / 1e9, 1)
                row[tag + "_hbm_frac"] = round(ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            qres.append(row)
            del Xs, Xq, Xe, sq
        out["variant_quant_act"] = {"workload": "fp16 activations -> per-token INT8 / e4m3 + "
                                                "float32 scales; events around one replay of a "
                                                "HIP graph of 20 launches rotating x_copies "
                                                "copies of X",
                                    "results": qres}

    if not args.no_cpu_baseline and not args.only:
        desc = [(s["name"], s["M"], s["N"], s["K"], g, s["pair"]) for s in slots]
        out["cpu_baseline"] = cpu_baseline(desc, args.cpu_sample_cols)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
