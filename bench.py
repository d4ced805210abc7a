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
    p.add_argument("--only", default="",
                   help="run one slot, e.g. upgate:M4096, or fp8 / moe / quant for that "
                        "variant alone")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp8", action="store_true")
    p.add_argument("--no-ablation", action="store_true")
    p.add_argument("--no-moe", action="store_true")
    p.add_argument("--no-7b", action="store_true")
    p.add_argument("--cpu-sample-cols", type=int, default=4096,
                   help="output channels per slot in the all-core oracle sample")
    p.add_argument("--cpu-sample-cols-1core", type=int, default=256,
                   help="output channels per slot in the one-core oracle sample")
    p.add_argument("--cpu-baseline-only", action="store_true",
                   help="only time the oracle sample (no GPU) and print its JSON")
    p.add_argument("--sustain-ms", type=float, default=100.0,
                   help="untimed whole steps run for about this long before the warm-up "
                        "steps, so the timed steps see the sustained clock (0: none)")
    p.add_argument("--bursts", type=int, default=5,
                   help="bursts of 20 back-to-back launches per slot outside the timed step")
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
    kv = _profile_kv(f"traffic_{slot_name.replace(':', '_')}.txt")
    if kv is None:
        return None
    try:
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None
    return round((fetch + write) * 1024.0)


def _profile_kv(name):
    """key: value lines of profiles/<name>.txt, or None when the file is
    missing or its counters were taken from other kernel code."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    return kv


def profiled_mfma(slot_name, M, N, K, us_per_launch):
    """Matrix-core counters per launch of `slot_name`'s kernel from the
    committed summary: INT8 matrix-core operations counted (MOPS x 512)
    against the algorithmic 2*M*N*K, the fraction of SIMD cycles the matrix
    core was busy, and the shader clock the busy cycles imply."""
    kv = _profile_kv(f"mfma_{slot_name.replace(':', '_')}.txt")
    if kv is None:
        return None
    try:
        mops = float(kv["mfma_mops_i8_per_dispatch"])
        busy = float(kv["mfma_busy_cycles_per_dispatch"])
        gui = float(kv["grbm_gui_active_per_dispatch"])
        simds = float(kv["simds"])
    except (KeyError, ValueError):
        return None
    return {"int8_ops_counted": mops * 512.0, "int8_ops_algorithmic": 2.0 * M * N * K,
            "busy_frac": round(busy / (gui * simds), 4),
            "gui_active_cycles": gui,
            "clock_ghz_implied": round(gui / (us_per_launch * 1e3), 3)}


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


def sweep_desc():
    """(name, M, N, K, group, pair) of every slot of the sweep (no GPU)."""
    pairs = wl.nk_pairs(CFG)
    tags = {pairs[0]: "upgate", pairs[1]: "down"}
    return [(f"{tags[(N, K)]}:M{M}", M, N, K, 128, pi)
            for pi, (N, K) in enumerate(pairs) for M in MS]


def cpu_baseline(slots_desc, ncols):
    """Oracle (test infrastructure) timed on the host cores: identity decode,
    int32 GEMM and fp16 epilogue for every slot of the sweep, restricted to
    `ncols` output channels per slot; scaled to the full step."""
    import oracle
    total_ops_full = 0.0
    t_scaled = 0.0
    t_real = 0.0
    per_pair = {}
    for (tag, M, N, K, g, pair) in slots_desc:
        if pair not in per_pair:
            # numpy draws row-major: a smaller draw with the same seed is
            # exactly the leading rows of the full matrices the GPU uses
            W = wl.gen_weights(min(ncols, N), K, wl.seed_w(CFG, pair))
            X = wl.gen_activations(max(MS), K, wl.seed_x(CFG, max(MS)),
                                   wl.seed_outliers(CFG))
            X8_all, sx_all = oracle.quant_sym_rows(X, 127)
            per_pair[pair] = (oracle.w4a8_pack(W, g), X8_all, sx_all)
        pk, X8_all, sx_all = per_pair[pair]
        X8, sx = X8_all[:M], sx_all[:M]
        t0 = time.perf_counter()
        oracle.w4a8_gemm(X8, sx, pk, g)
        dt = time.perf_counter() - t0
        t_real += dt
        t_scaled += dt * (N / min(ncols, N))
        total_ops_full += 2.0 * M * N * K
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": round(total_ops_full / t_scaled / 1e12, 5), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"each of the 10 GEMMs of the sweep on {ncols} of its N output "
                      f"channels (decode + int32 GEMM + fp16 epilogue): {t_real:.1f} s of "
                      f"oracle time, scaled by N/{ncols} to {t_scaled:.1f} s for one full step"}


def cpu_baseline_one_core(ncols):
    """The same oracle sample in a child process limited to one thread."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                          "--cpu-sample-cols", str(ncols)], env=env, capture_output=True,
                         text=True, timeout=600)
    if res.returncode != 0:
        return {"error": res.stderr[-300:]}
    return json.loads(res.stdout.strip().splitlines()[-1])


def _smi_sample():
    """One `amd-smi metric --clock --power --json` reading: mean shader clock
    over the XCDs, memory clock (MHz) and socket power (W)."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    res = subprocess.run([exe, "metric", "--clock", "--power", "--json"], capture_output=True,
                         text=True, timeout=30)
    d = json.loads(res.stdout)
    g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
    gfx = [v["clk"]["value"] for k, v in g["clock"].items()
           if k.startswith("gfx") and isinstance(v.get("clk"), dict)]
    mem = g["clock"]["mem_0"]["clk"]["value"]
    power = g["power"]["socket_power"]["value"]
    return {"gfx_mhz": sum(gfx) / len(gfx), "mem_mhz": mem, "socket_power_w": power}


def clocks_under_load(launch, n_samples=4, limit_s=20.0):
    """Clocks and power read by amd-smi while `launch` (one GEMM) runs back
    to back: a sampler thread takes readings after a settling pause while
    this thread keeps the GPU queue full."""
    import threading
    import torch
    samples, errors = [], []

    def sampler():
        time.sleep(0.5)
        while len(samples) < n_samples and len(errors) < 2:
            try:
                samples.append(_smi_sample())
            except Exception as e:  # the tool is optional on a host
                errors.append(repr(e)[:200])

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.time()
    th.start()
    launches = 0
    while th.is_alive() and time.time() - t0 < limit_s:
        for _ in range(20):
            launch()
        launches += 20
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    if not samples:
        return {"error": errors[0] if errors else "no reading"}
    mean = lambda k: round(sum(x[k] for x in samples) / len(samples), 1)
    return {"gfx_mhz_mean": mean("gfx_mhz"),
            "gfx_mhz_min": round(min(x["gfx_mhz"] for x in samples), 1),
            "mem_mhz": mean("mem_mhz"), "socket_power_w_mean": mean("socket_power_w"),
            "socket_power_w_max": max(x["socket_power_w"] for x in samples),
            "samples": len(samples), "launches": launches}


def decode_target(sweep, target=0.70):
    """Fraction of the 8 TB/s HBM peak (algorithmic bytes) that each slot
    with M <= 16 reaches back to back, against the 70 % target."""
    fr = {e["slot"]: e["hbm_frac_algo"] for e in sweep
          if int(e["slot"].split(":M")[1]) <= 16 and e.get("hbm_frac_algo") is not None}
    return {"target_hbm_frac": target, "slots": fr,
            "met": bool(fr) and all(v >= target for v in fr.values())}


def sustain(torch, stream, launch, pool, ms=100.0):
    """About `ms` milliseconds (wall clock) of untimed back-to-back launches
    (launch(pool[r % len(pool)]), eight between synchronisations), so that
    what is timed next runs at the clock the chip holds under sustained
    load.  Measured on one box: after 50 ms idle, 20 back-to-back launches of
    4096 x 28672 x 8192 took 823 us each, 714 us after 100 ms of load; at
    16 x 8192 x 28672, 27.0 against 24.1 us.  `stream` is where the launches
    go (torch's current stream)."""
    t_start = time.perf_counter()
    r = 0
    while r < 20000 and (time.perf_counter() - t_start) * 1e3 < ms:
        for _ in range(8):
            launch(pool[r % len(pool)])
            r += 1
        torch.cuda.synchronize()


def graph_bursts(torch, stream, launch, pool, Yout, n, reps=20):
    """Per-launch microseconds of `reps` launches (launch(pool[r % len(pool)]))
    captured once in a HIP graph, so a launch's figure is the GPU's (kernel
    plus dispatch gap) even where a Python launch takes longer than the
    kernel.  Two replays, each followed by a synchronisation, are first
    checked against the eager result; then, after about 100 ms of untimed
    replays, n replays run back to back on `stream` (the GPU kept busy, as in
    the sweep: this part is power-bound, and idle gaps would raise its
    clock), each bracketed by events, and the output of the last is checked
    again."""
    import numpy as np
    launch(pool[(reps - 1) % len(pool)])
    torch.cuda.synchronize()
    want = Yout.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in range(3):
            launch(pool[r % len(pool)])
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(reps):
            launch(pool[r % len(pool)])
    for _ in range(2):
        Yout.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(Yout, want):
            raise RuntimeError("graph replay differs from the eager result")
    sustain(torch, stream, lambda _: graph.replay(), [None])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        graph.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    if not torch.equal(Yout, want):
        raise RuntimeError("graph replay differs from the eager result")
    out_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 / reps for i in range(n)]
    del graph
    return np.array(out_us)


def moe_variant(w4, wl, torch, dev, stream, n=5):
    """Grouped (mixture-of-experts) GEMM: Mixtral-8x7B expert layers, 8
    experts with top-2 routing drawn from a seeded generator (each token to
    two distinct experts), synthetic weights and activations of those
    shapes, at 16 and 2048 tokens."""
    import numpy as np
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
            offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
                                    ).to(dev)
            Mm = int(counts.sum())
            Xm = torch.from_numpy(wl.gen_activations(Mm, Km, 900 + T, 901)).to(dev)
            Xq_m, sx_m = w4.quant_act(Xm)
            Ym = torch.empty((Mm, Nm), dtype=torch.float16, device=dev)
            mr = int(counts.max())
            launch = (lambda pk, Xq_m=Xq_m, sx_m=sx_m, offs=offs, mr=mr, Ym=Ym:
                      w4.gemm_grouped(Xq_m, sx_m, offs, pk, mr, out=Ym))
            sustain(torch, stream, launch, pkms)
            reps = 10
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            ts = []
            for _ in range(n):
                e0.record(stream)
                for r in range(reps):
                    launch(pkms[r % 2])
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / reps)
            us = float(np.median(ts))
            active = int((counts > 0).sum())
            wbytes = active * weight_bytes(Nm, Km, g_moe)
            moe.append({"layer": tag, "N": Nm, "K": Km, "tokens": T, "rows": Mm,
                        "max_rows_per_expert": mr, "active_experts": active,
                        "us": round(us, 2), "us_min": round(min(ts), 2),
                        "us_max": round(max(ts), 2),
                        "tops": round(2.0 * Mm * Nm * Km / (us * 1e-6) / 1e12, 2),
                        "weight_stream_gbs": round(wbytes / (us * 1e-6) / 1e9, 1)})
        del pkm, pkms
    return {"workload": "Mixtral-8x7B expert layers, 8 experts top-2, W4A8 group 128, fp16 "
                        f"out; median over {n} bursts of 10 back-to-back launches alternating "
                        "two copies of the expert weights",
            "results": moe}


def quant_variant(w4, torch, dev, stream, n=5):
    """Per-token activation quantisation, the step before every GEMM: fp16 X
    -> INT8 codes (W4A8) or e4m3 codes (W4FP8) plus float32 row scales, at
    the sweep's activation shapes.  HBM bound: 2 bytes read and 1 written
    per value; copies of X used in turn past 512 MB in total where that
    fits, so the large shapes stream from HBM (the 16-row ones are a few
    hundred KB and launch bound whatever the copies)."""
    import numpy as np
    qres = []
    for (M, K) in ((16, 8192), (16, 28672), (4096, 8192), (4096, 28672)):
        ncp = max(2, min(8, int(512e6 // (M * K * 2)) + 1))
        Xs = [torch.randn((M, K), device=dev).to(torch.float16) for _ in range(ncp)]
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        Xe = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sq = torch.empty(M, dtype=torch.float32, device=dev)
        row = {"M": M, "K": K, "x_copies": ncp}
        for tag, fn, Yq in (("int8", lambda i: w4.quant_act(Xs[i], out=(Xq, sq)), Xq),
                            ("e4m3", lambda i: w4.quant_act_fp8(Xs[i], out=(Xe, sq)), Xe)):
            # the launches are captured in a HIP graph and replayed: the
            # 16-row kernels take less time than a launch from Python
            ts = graph_bursts(torch, stream, fn, list(range(ncp)), Yq, n)
            us = float(np.median(ts))
            ab = 3 * M * K + 4 * M
            row[tag + "_us"] = round(us, 2)
            row[tag + "_gbs"] = round(ab / (us * 1e-6) / 1e9, 1)
            row[tag + "_hbm_frac"] = round(ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        qres.append(row)
        del Xs, Xq, Xe, sq
    return {"workload": "fp16 activations -> per-token INT8 / e4m3 + float32 scales; median "
                        "over back-to-back replays of a HIP graph of 20 launches rotating "
                        "x_copies copies of X",
            "results": qres}


def fp8_variant(w4, wl, torch, dev, stream, n=5):
    """FP8 variants (INT4 weights x e4m3 activations), reported alongside the
    W4A8 sweep: per-channel scales, and per-group scales folded into the FP8
    weights with a per-tensor rescale; the prefill shape and a 16-token
    decode shape."""
    import numpy as np
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

    res = {}
    for M in (sh.M, 16):
        Yb = torch.empty((M, sh.N), dtype=torch.bfloat16, device=dev)
        Xm, sxm = X8[:M], sx8[:M]
        for tag, fn, pool in (("per_channel",
                               lambda pk: w4.gemm_fp8(Xm, sxm, pk, out=Yb), cps8),
                              ("group128_folded",
                               lambda pk: w4.gemm_fp8g(Xm, sxm, pk, out=Yb), cps8g)):
            ts = graph_bursts(torch, stream, fn, pool, Yb, n)
            us = float(np.median(ts))
            tf = 2.0 * M * sh.N * sh.K / (us * 1e-6) / 1e12
            wb = sh.N * sh.K / 2 + (sh.N * 4 if tag == "per_channel"
                                    else sh.N * sh.K // 128 * 4 + 4)
            ab = wb + M * sh.K + M * 4 + M * sh.N * 2
            res[f"{tag}_M{M}"] = {"us": round(us, 2), "us_min": round(float(ts.min()), 2),
                                  "us_max": round(float(ts.max()), 2), "tflops": round(tf, 2),
                                  "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4),
                                  "hbm_frac_algo": round(ab / (us * 1e-6) / 1e9
                                                         / HBM_PEAK_GBS, 4)}
    return {"workload": f"int4-fp8 N={sh.N} K={sh.K}, M={sh.M} and 16, bf16 out; median over "
                        f"{n} back-to-back replays of a HIP graph of 20 launches rotating {ncp} "
                        "weight copies (a Python launch takes longer than the 16-row kernels), "
                        "the output checked against the eager result",
            "results": res}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(sweep_desc(), args.cpu_sample_cols)), flush=True)
        return

    import numpy as np
    import torch
    import w4a8_quantized_gemm_amd as w4
    import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.only == "fp8":
        # the FP8 variant alone, for the profiler
        print(json.dumps({"variant_fp8": fp8_variant(w4, wl, torch, dev, stream, args.bursts)}),
              flush=True)
        return
    if args.only == "quant":
        # the activation quantisation alone, for the profiler
        print(json.dumps({"variant_quant_act": quant_variant(w4, torch, dev, stream,
                                                             args.bursts)}), flush=True)
        return
    if args.only == "moe":
        # the grouped GEMM alone, for the profiler
        print(json.dumps({"variant_moe": moe_variant(w4, wl, torch, dev, stream, args.bursts)}),
              flush=True)
        return
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
            # one weight copy per slot; a slot run alone (--only) rotates
            # through copies past 512 MB so that, as in the full step, no
            # launch finds its weights in the 256 MB Infinity Cache
            ncp = 1 if not args.only else -(-600_000_000 // weight_bytes(N, K, g))
            copies = [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in pk.items()}
                      for _ in range(ncp)]
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            slots.append({"name": name, "M": M, "N": N, "K": K, "pair": pi, "pks": copies,
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

    def step(k, evs=None):
        for i, s in enumerate(slots):
            ev = evs is not None and i in evpos
            if ev:
                evs[evpos[i]][0].record(stream)
            w4.gemm(s["X"], s["sx"], s["pks"][k % len(s["pks"])], out=s["Y"])
            if ev:
                evs[evpos[i]][1].record(stream)

    # Before the W warm-up steps, whole steps run untimed for about
    # --sustain-ms milliseconds: the chip's clock ramps up under load over
    # tens of milliseconds, so without this the first timed steps run below
    # the clock the chip holds in sustained use (see sustain()).
    sustain_steps = 0
    if args.sustain_ms > 0:
        step(0)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        while sustain_steps < 1000 and (time.perf_counter() - t_start) * 1e3 < args.sustain_ms:
            for _ in range(4):
                step(sustain_steps)
                sustain_steps += 1
            torch.cuda.synchronize()
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in evslots] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k])
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
    # Several bursts per slot give the median and the spread.
    reps = 20

    def bursts(launch, pool, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sustain(torch, stream, launch, pool)
        out_us = []
        for _ in range(n):
            e0.record(stream)
            for r in range(reps):
                launch(pool[r % len(pool)])
            e1.record(stream)
            torch.cuda.synchronize()
            out_us.append(e0.elapsed_time(e1) * 1e3 / reps)
        return np.array(out_us)

    burst_us = {}
    for i, s in enumerate(slots):
        if i in ev_us:
            continue
        pool = [pk for t in slots if t["pair"] == s["pair"] for pk in t["pks"]]
        burst_us[i] = bursts(lambda pk, s=s: w4.gemm(s["X"], s["sx"], pk, out=s["Y"]), pool,
                             args.bursts)

    sweep = []
    total_ops = 0.0
    kern_ms_sum = 0.0
    for i, s in enumerate(slots):
        M, N, K = s["M"], s["N"], s["K"]
        ts = ev_us[i] if i in ev_us else burst_us[i]
        # events in the timed region: the mean launch time; bursts: the median burst
        us = float(np.mean(ts)) if i in ev_us else float(np.median(ts))
        ops = 2.0 * M * N * K
        total_ops += ops
        kern_ms_sum += us / 1e3
        wgbs = weight_bytes(N, K, g) / (us * 1e-6) / 1e9
        row = {"slot": s["name"], "M": M, "N": N, "K": K, "group": g,
               "us": round(us, 2),
               "timing": "events in timed region" if i in ev_us else "back-to-back bursts",
               "us_median": round(float(np.median(ts)), 2),
               "us_min": round(float(ts.min()), 2), "us_max": round(float(ts.max()), 2),
               "tops": round(ops / (us * 1e-6) / 1e12, 2),
               "weight_stream_gbs": round(wgbs, 1),
               "hbm_frac_algo": round(algo_bytes(M, N, K, g) / (us * 1e-6) / 1e9
                                      / HBM_PEAK_GBS, 4),
               "mfma_frac": round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
        if i in ev_us:
            row["launches"] = len(ts)
        else:
            row["bursts"] = len(ts)
            row["launches_per_burst"] = reps
        sweep.append(row)

    value = total_ops / (ms_per_step * 1e-3) / 1e12

    def roof(slot_name, bound):
        e = next((x for x in sweep if x["slot"] == slot_name), None)
        if e is None:
            return None
        if bound == "mfma":
            a = 2.0 * e["M"] * e["N"] * e["K"] / (e["us"] * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": INT8_PEAK_TOPS,
                    "unit": "TFLOP/s", "frac": round(a / INT8_PEAK_TOPS, 4),
                    "traffic": profiled_traffic(slot_name),
                    "mfma_counters": profiled_mfma(slot_name, e["M"], e["N"], e["K"], e["us"]),
                    "kernel_slot": slot_name,
                    "us_per_launch": e["us"], "timing": e["timing"]}
        a = algo_bytes(e["M"], e["N"], e["K"], g) / (e["us"] * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(slot_name),
                "kernel_slot": slot_name,
                "us_per_launch": e["us"], "timing": e["timing"]}

    # dominant kernel: the slot with the largest share of the step (among
    # those timed with events inside the timed region)
    dom = max((sweep[i] for i in evslots), key=lambda e: e["us"])
    dom_bound = "mfma" if dom["M"] >= 1024 else "hbm"
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "sustain_steps": sustain_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "llama2-70b linear sweep (W4A8, group 128)",
                   "shapes_NK": [list(p) for p in pairs], "M": list(MS),
                   "slots": [s["name"] for s in slots], "out": "fp16",
                   "weights_per_slot_MB": round(weight_bytes(*pairs[0], g) / 1e6, 1),
                   "parallelism": "single GPU"},
        "roofline": roof(dom["slot"], dom_bound),
        "roofline_decode": roof("upgate:M16", "hbm") or roof("down:M16", "hbm"),
        # the decode target (70 % of HBM bandwidth at M <= 16), assessed on
        # the back-to-back figures, launch gaps included
        "decode_target": decode_target(sweep),
        "kernel_ms_per_step": round(kern_ms_sum, 4),
        "sweep": sweep,
    }

    # ---- shader / memory clock and socket power while the dominant slot's
    # GEMM runs back to back (amd-smi readings; the clock the chip holds
    # under this load is what bounds the matrix-core kernels)
    if not args.only:
        ds = next(s for s in slots if s["name"] == DOMINANT_SLOT)
        out["clocks_under_load"] = dict(
            clocks_under_load(lambda: w4.gemm(ds["X"], ds["sx"], ds["pks"][0], out=ds["Y"])),
            slot=DOMINANT_SLOT)

    # ---- Llama-2-7B shapes, reported beside the 70B sweep (not part of the
    # timed step): attention-projection decode (M = 1, 4, 16 on 4096 x 4096)
    # and MLP prefill (2048 tokens on 11008 x 4096 and 4096 x 11008), group
    # 64.  Each shape rotates through weight copies past 600 MB (68 copies of
    # the 8.9 MB decode weights), so no launch finds its weights in the
    # 256 MB Infinity Cache; several bursts of back-to-back launches each.
    if not args.no_7b and not args.only:
        rows7 = []
        for cfg in (wl.LLAMA7B_DECODE, wl.LLAMA7B_PREFILL):
            for pi, (N, K) in enumerate(wl.nk_pairs(cfg)):
                g7 = 64
                Wf = torch.from_numpy(wl.gen_weights(N, K, wl.seed_w(cfg, pi))).to(dev)
                pk7 = w4.pack(Wf, group=g7)
                del Wf
                ncp = -(-600_000_000 // weight_bytes(N, K, g7))
                pool = [pk7] + [{k: (v.clone() if torch.is_tensor(v) else v)
                                 for k, v in pk7.items()} for _ in range(ncp - 1)]
                for sh in wl.CONFIGS[cfg].shapes:
                    if (sh.N, sh.K) != (N, K):
                        continue
                    M = sh.M
                    Xf = torch.from_numpy(wl.gen_activations(M, K, wl.seed_x(cfg, M),
                                                             wl.seed_outliers(cfg))).to(dev)
                    X7, sx7 = w4.quant_act(Xf)
                    del Xf
                    Y7 = torch.empty((M, N), dtype=torch.float16, device=dev)
                    ts = graph_bursts(torch, stream, lambda pk, X7=X7, sx7=sx7, Y7=Y7:
                                      w4.gemm(X7, sx7, pk, out=Y7), pool, Y7, args.bursts)
                    us = float(np.median(ts))
                    ops = 2.0 * M * N * K
                    ab = algo_bytes(M, N, K, g7)
                    bound = "hbm" if M <= 16 else "mfma"
                    frac = (ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS if bound == "hbm"
                            else ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS)
                    rows7.append({"shape": sh.name, "M": M, "N": N, "K": K, "group": g7,
                                  "us_median": round(us, 2), "us_min": round(float(ts.min()), 2),
                                  "us_max": round(float(ts.max()), 2),
                                  "tops": round(ops / (us * 1e-6) / 1e12, 2),
                                  "weight_stream_gbs": round(weight_bytes(N, K, g7)
                                                             / (us * 1e-6) / 1e9, 1),
                                  "bound": bound, "frac_of_peak": round(frac, 4),
                                  "weight_copies": ncp})
                del pool, pk7
        out["llama7b"] = {"workload": "llama2-7b linear shapes (W4A8, group 64), fp16 out; "
                                      "median over back-to-back replays of a HIP graph of 20 "
                                      "launches rotating weight copies past 600 MB (a Python "
                                      "launch takes longer than the decode kernels); decode rows "
                                      "against 8 TB/s (algorithmic bytes), prefill rows "
                                      "against 5 POP/s",
                          "results": rows7}

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
            # the weight copies of every slot of this shape in turn, as in the
            # sweep's bursts, so that no launch finds its weights in the cache
            copies = [pk for t in slots if t["pair"] == sl["pair"] for pk in t["pks"]]
            fns = {nm: (lambda pk, v=v, sl=sl: w4.gemm_ablation(v, sl["X"], sl["sx"], pk,
                                                                 out=sl["Y"]))
                   for v, nm in names.items()}
            # the production kernel choice for the same slot, in the same loop
            fns["w4a8_gemm"] = lambda pk, sl=sl: w4.gemm(sl["X"], sl["sx"], pk, out=sl["Y"])
            reps = 2 * len(copies)
            sustain(torch, stream, fns["lqq"], copies)
            times = {nm: [] for nm in fns}
            # the variants interleaved, one burst each per round, medians over
            # the rounds, so that drift of the clock affects them alike
            for _ in range(args.bursts):
                for nm, fn in fns.items():
                    e0.record(stream)
                    for r in range(reps):
                        fn(copies[r % len(copies)])
                    e1.record(stream)
                    torch.cuda.synchronize()
                    times[nm].append(e0.elapsed_time(e1) * 1e3 / reps)
            row = {"slot": sl["name"]}
            for nm, v in times.items():
                row[nm + "_us"] = round(float(np.median(v)), 2)
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
                pool4 = [pk for t in slots if t["pair"] == pi for pk in t["pks"]]
                f8 = lambda r, sl=sl: w4.gemm_w8a8(sl["X"], sl["sx"], pk8 if r % 2 == 0 else pk8b,
                                                   out=sl["Y"])
                f4 = lambda r, sl=sl, pool4=pool4: w4.gemm(sl["X"], sl["sx"],
                                                          pool4[r % len(pool4)], out=sl["Y"])
                sustain(torch, stream, f8, [0, 1])
                reps = 10 if sl["M"] >= 1024 else 20
                t8, t4 = [], []
                # W8A8 and W4A8 bursts interleaved, medians over the rounds
                for _ in range(args.bursts):
                    for fn, acc in ((f8, t8), (f4, t4)):
                        e0.record(stream)
                        for r in range(reps):
                            fn(r)
                        e1.record(stream)
                        torch.cuda.synchronize()
                        acc.append(e0.elapsed_time(e1) * 1e3 / reps)
                us8, us4 = float(np.median(t8)), float(np.median(t4))
                cmp_rows.append({"slot": sl["name"], "w8a8_us": round(us8, 2),
                                 "w4a8_us": round(us4, 2), "w8a8_vs_w4a8": round(us8 / us4, 3)})
            del pk8, pk8b
        out["w8a8_compare"] = {"note": "medians over rounds of interleaved bursts of 10-20 "
                                       "back-to-back launches: W8A8 alternating two weight "
                                       "copies, W4A8 rotating the sweep's weight copies of the "
                                       "same shape",
                               "results": cmp_rows}

    # ---- grouped (mixture-of-experts) GEMM, Mixtral-8x7B expert layers
    if not args.no_moe and not args.only:
        out["variant_moe"] = moe_variant(w4, wl, torch, dev, stream, args.bursts)

    if not args.no_fp8 and not args.only:
        out["variant_fp8"] = fp8_variant(w4, wl, torch, dev, stream, args.bursts)

    # ---- per-token activation quantisation, the step before every GEMM
    if not args.no_ablation and not args.only:
        out["variant_quant_act"] = quant_variant(w4, torch, dev, stream, args.bursts)

    if not args.no_cpu_baseline and not args.only:
        out["cpu_baseline"] = cpu_baseline(sweep_desc(), args.cpu_sample_cols)
        out["cpu_baseline"]["one_core"] = cpu_baseline_one_core(args.cpu_sample_cols_1core)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
