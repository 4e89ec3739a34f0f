"""Benchmark of the NVFP4 weight-only projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode pass of the 27B-style dense MLP at M = 1: the gate/up
GEMV (K=5120 -> N=17408) followed by the down GEMV (K=17408 -> N=5120), each
through the C ABI on packed weights already resident in HBM.  `value` is the
algorithmic bytes of the step (packed codes + e4m3 scales + x + y + g) per
second.  Each step uses a different copy of the packed weights, cycling
through >= 512 MB of copies, so the 256 MB Infinity Cache cannot serve them.

Also measured and reported in the same JSON line:
  roofline      the GEMV kernel: bytes per launch / mean launch duration (HIP
                events on the launch stream around the timed region, whose
                launches are all this kernel) vs 8 TB/s;
                `traffic` from the rocprofv3 FETCH_SIZE/WRITE_SIZE summary in
                profiles/ when it was taken on the current kernel source.
  prefill_gemm  the M = 512 prefill chunk (qkv 5120->14336, gate/up
                5120->17408) as the binding calls it (fp16 staging kernel +
                GEMM on fp16 operands): TFLOP/s vs 2.517 PFLOP/s dense
                bf16/fp16, with the time of the bf16-operand path (no
                workspace) beside it; `traffic` (HBM bytes per GEMM launch,
                mean of the two) from the rocprofv3 counter summary in
                profiles/ when current.
  shapes        the other workloads' GEMVs (M = 7 verify, lm-head, 4B shapes).
  verify_sweep  the speculative-verify GEMV over M = 1..16 rows for both MLP
                matrices (gate/up 5120->17408, down 17408->5120): GB/s and the
                fraction of 8 TB/s per M.
  fused_gate_up the MLP's gate and up weights as one fused 2F x K NVFP4
                projection with the silu(gate)*up epilogue (bf16 out), F = 17408,
                K = 5120: the GEMV at M = 1 and M = 7 and the GEMM at M = 512,
                each beside the plain projection over the same packed weight
                (fp32 out, no epilogue).
  pack          the one-time weight swizzle (read + write bytes / s).
  lm_head_argmax  the lm-head GEMV (M = 1 decode, M = 7 verify) with the fused
                greedy argmax and no logits written, beside the plain GEMV
                writing the logits followed by torch.argmax.
  quantize      the load-time NVFP4 conversion of bf16 weights (fused gate/up
                34816 x 5120 and lm-head 248320 x 5120): algorithmic bytes
                (bf16 in, codes + scales out) / s; two launches, the first
                reads w for its max, the second reads it again to quantize.
  graph_replay  the decode step captured as a HIP graph and replayed (the
                launch path a serving loop would use).
  prepared_calls  the decode step through prepared launchers (host time per
                launch without the binding's per-call checks).
  cpu_baseline  the CPU oracle on the decode step, on the host cores, and on
                one thread for the tiny case, the decode step and the 4B pair.
  device_state_before_timing  clock levels (sysfs) and the processes holding
                a GPU (amdsmi, in this process; idle check).
  host          os.cpu_count(), the CPUs this process may run on, OMP_NUM_THREADS.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2517.0          # 256 CU x 4096 flop/clk x 2.4 GHz, dense
MALL_DEFEAT_BYTES = 512 << 20
METRIC = "NVFP4 projection GB/s & % HBM peak (M=1); TFLOP/s & % MFMA peak (M=512)"


def algo_bytes(M, N, K):
    """Packed codes + e4m3 scales + bf16 x + fp32 y + the fp32 global scale."""
    return N * K // 2 + N * K // 16 + 2 * M * K + 4 * M * N + 4


def src_digest(name):
    path = os.path.join(ROOT, "nvfp4_weight_only_q4proj_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(profile, digest, launch_bytes):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when absent or taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def head_start(torch, ms):
    """Queue a spin kernel so the host can enqueue the timed launches while
    the GPU is busy: the timed region then measures back-to-back kernels,
    not the host's launch rate."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def timed_region(torch, launches, steps):
    """HIP events on the launch stream (the current stream, which the binding
    launches on) around `launches` run back to back behind a head start.
    Returns (ms per step, host seconds spent enqueueing)."""
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    head_start(torch, 0.05 * len(launches) + 5)
    h0 = time.perf_counter()
    t0.record(stream)
    for fn in launches:
        fn()
    t1.record(stream)
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, host_s


def single_thread_oracle(oracle, synth, dec):
    """The oracle on one host thread: the 512 x 256 tiny case (median of 3
    runs), one decode step (gate/up + down, one run) and the 4B-style
    up/down pair (one run each); seconds and algorithmic GB/s."""
    res = {}

    def run(cases, reps):
        times = []
        for _ in range(reps):
            t = time.perf_counter()
            for c in cases:
                oracle.proj(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, nthreads=1)
            times.append(time.perf_counter() - t)
        el = sorted(times)[len(times) // 2]
        b = sum(algo_bytes(c.M, c.N, c.K) for c in cases)
        return {"s": round(el, 4), "gbs": round(b / el / 1e9, 4)}

    res["tiny_512x256_M1"] = run(synth.workload_cases("tiny"), 3)
    res["decode_step_M1"] = run(dec, 1)
    for c in synth.workload_cases("lmh", only=["up_4b", "down_4b"]):
        res[f"{c.name}_{c.N}x{c.K}_M1"] = run([c], 1)
    return res


def device_state():
    """Shader and memory clock levels and the processes holding a GPU, read
    from sysfs just before timing (an idle check: no other process should
    hold the GPU).  No child process is started: under a profiler every
    process inherits its preloaded library, which initialises the GPU."""
    import glob
    state = {"clocks": {}, "gpu_pids": None}
    for card in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        try:
            if open(os.path.join(card, "vendor")).read().strip() != "0x1002":
                continue
            levels = {}
            for clk in ("sclk", "mclk"):
                lines = open(os.path.join(card, f"pp_dpm_{clk}")).read().split("\n")
                cur = [ln for ln in lines if ln.strip().endswith("*")]
                levels[clk] = {"current": cur[0].split(":", 1)[1].strip(" *") if cur else None,
                               "levels": [ln.split(":", 1)[1].strip(" *") for ln in lines
                                          if ":" in ln]}
            state["clocks"][os.path.basename(os.path.dirname(card))] = levels
        except (OSError, IndexError):
            continue
    state["gpu_pids"], state["gpu_processes_source"] = gpu_processes()
    return state


def gpu_processes():
    """(pids of the other processes that hold a GPU, where the list came
    from): amdsmi's per-GPU process list, read in this process before it
    touches the GPU; the kfd sysfs directory when amdsmi is unusable."""
    me = os.getpid()
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            pids = set()
            for h in amdsmi.amdsmi_get_processor_handles():
                for proc in amdsmi.amdsmi_get_gpu_process_list(h):
                    pid = proc.get("pid") if isinstance(proc, dict) else None
                    if isinstance(pid, int) and pid != me:
                        pids.add(pid)
            return sorted(pids), "amdsmi"
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # noqa: BLE001 - any amdsmi failure falls back
        err = f"amdsmi: {type(e).__name__}: {e}"[:200]
    try:
        return sorted(int(p) for p in os.listdir("/sys/class/kfd/kfd/proc")
                      if p.isdigit() and int(p) != me), "kfd sysfs"
    except OSError:
        return None, err + "; no kfd sysfs process list"


def graph_replay(torch, launches, steps_per_pass, passes):
    """`launches` (steps_per_pass steps) captured once as a HIP graph and
    replayed `passes` times back to back behind a head start.  Returns (ms
    per step, host microseconds per replay call)."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in launches:
            fn()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    head_start(torch, 0.05 * len(launches) * passes + 5)
    h0 = time.perf_counter()
    t0.record(stream)
    for _ in range(passes):
        graph.replay()
    t1.record(stream)
    host_us = (time.perf_counter() - h0) / passes * 1e6
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (passes * steps_per_pass), host_us


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall-time bound of the cpu_baseline sample")
    ap.add_argument("--only", choices=["dec", "pre", "shapes", "verify", "mlp", "argmax", "quant",
                                       "all"],
                    default="all",
                    help="restrict the run (for profiling one kernel)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the projection would shard across GPUs by "
              "output columns or by k, and no multi-GPU path is implemented.",
              file=sys.stderr)
        sys.exit(2)

    smi = device_state()

    import numpy as np
    import torch

    import nvfp4_weight_only_q4proj_amd as q4
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    def upload(case, copies):
        mat = case.matrix
        codes = torch.from_numpy(mat.codes.reshape(-1)).to(dev)
        scales = torch.from_numpy(mat.scales.reshape(-1)).to(dev)
        pc, ps = q4.pack_weight(codes, scales, mat.N, mat.K)
        reps = [(pc, ps)] + [(pc.clone(), ps.clone()) for _ in range(copies - 1)]
        x = torch.from_numpy(case.x.view(np.int16)).to(dev)
        y = torch.empty((case.M, mat.N), dtype=torch.float32, device=dev)
        del codes, scales
        return {"case": case, "w": reps, "x": x, "y": y, "g": mat.g}

    def copies_for(step_bytes):
        return max(2, -(-MALL_DEFEAT_BYTES // step_bytes))

    def launcher(kind, u, i):
        # "gemm": the binding's default (fp16 operands staged in its GEMM
        # scratch where gemm_staging_pays, else bf16); "gemm_bf16": no
        # workspace, bf16 operands (one kernel); "gemm_fp16": always staged
        c = u["case"]
        pc, ps = u["w"][i % len(u["w"])]
        if kind == "gemv":
            return lambda: q4.q4proj_gemv(pc, ps, u["g"], u["x"], u["y"], c.M, c.N, c.K)
        ws = {"gemm": None, "gemm_bf16": False,
              "gemm_fp16": q4.gemm_scratch(dev, q4.q4proj_gemm_workspace_bytes(c.M, c.N, c.K))}[kind]
        return lambda: q4.q4proj_gemm(pc, ps, u["g"], u["x"], u["y"], c.M, c.N, c.K, workspace=ws)

    out = {"metric": METRIC, "device_state_before_timing": smi,
           "host": {"cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
                    "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}}

    # ---- decode step: gate/up + down GEMV at M = 1 -------------------------
    dec = synth.workload_cases("dec")
    step_bytes = sum(algo_bytes(c.M, c.N, c.K) for c in dec)
    ncopy = copies_for(step_bytes)
    dec_u = [upload(c, ncopy) for c in dec]
    torch.cuda.synchronize()

    if args.only in ("dec", "all"):
        for i in range(args.warmup):
            for u in dec_u:
                launcher("gemv", u, i)()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        step_ms, host_s = timed_region(
            torch, [launcher("gemv", u, args.warmup + i) for i in range(args.steps) for u in dec_u],
            args.steps)
        wall = time.perf_counter() - wall0
        # every launch in the timed region is the decode GEMV kernel, so its
        # mean duration per launch is the region's time over the launch count
        # (launch gaps included, which only lowers the figure)
        gemv_ms = step_ms / len(dec_u)
        launch_bytes = step_bytes / len(dec_u)
        achieved = launch_bytes / (gemv_ms * 1e-3) / 1e9
        digest = src_digest("q4p_gemv.hip")
        traffic = read_traffic("gemv_dec_traffic.txt", digest, launch_bytes)
        value = step_bytes / (step_ms * 1e-3) / 1e9
        out.update({
            "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,0.02) bf16 weights, two-level NVFP4; x ~ N(0,1) bf16)",
            "config": {"workload": "decode M=1, 27B-style MLP: gate/up 5120->17408 + down "
                                   "17408->5120 NVFP4 GEMV",
                       "M": 1, "shapes": [[c.N, c.K] for c in dec],
                       "bytes_per_step": step_bytes, "weight_copies": ncopy,
                       "rotation_bytes": ncopy * sum(
                           u["w"][0][0].numel() + u["w"][0][1].numel() for u in dec_u)},
            "tokens_per_s": round(1.0 / (step_ms * 1e-3), 1),
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "gemv_sk_kernel<1, 4, false, 0>",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic, "mean_launch_us": round(gemv_ms * 1e3, 3),
                         "bytes_per_launch": launch_bytes,
                         "kernel_source_sha256_16": digest},
            "device": {"name": props.name, "cus": props.multi_processor_count,
                       "arch": getattr(props, "gcnArchName", "")},
            "wall_s_timed": round(wall, 4),
            "host_enqueue_us_per_launch": round(host_s / (args.steps * len(dec_u)) * 1e6, 2),
        })
        # the same step as a captured graph: one pass over every weight copy
        # (ncopy steps) per graph, replayed back to back
        passes = max(1, args.steps // ncopy)
        g_ms, g_host = graph_replay(
            torch, [launcher("gemv", u, i) for i in range(ncopy) for u in dec_u], ncopy, passes)
        out["graph_replay"] = {
            "ms_per_step": round(g_ms, 5), "steps": passes * ncopy,
            "gbs": round(step_bytes / (g_ms * 1e-3) / 1e9, 1),
            "launches_per_graph": ncopy * len(dec_u),
            "host_us_per_replay": round(g_host, 2),
            "note": "the decode step captured as a HIP graph (torch.cuda.CUDAGraph over the "
                    "C-ABI calls, caller-owned buffers, no allocation per call)"}
        # the same launches through prepared calls: the binding's checks run
        # once per (weight copy, matrix), each step only calls the C entry
        prep = [[q4.prepare_gemv(pc, ps, u["g"], u["x"], u["y"], u["case"].M, u["case"].N,
                                 u["case"].K) for (pc, ps) in u["w"]] for u in dec_u]
        p_ms, p_host = timed_region(
            torch, [prep[j][(args.warmup + i) % ncopy] for i in range(args.steps)
                    for j in range(len(dec_u))], args.steps)
        out["prepared_calls"] = {
            "ms_per_step": round(p_ms, 5), "gbs": round(step_bytes / (p_ms * 1e-3) / 1e9, 1),
            "host_enqueue_us_per_launch": round(p_host / (args.steps * len(dec_u)) * 1e6, 2),
            "note": "the decode step through prepare_gemv launchers (arguments checked and "
                    "converted once; the C ABI still validates every call)"}

    # ---- prefill chunk: M = 512 GEMM --------------------------------------
    if args.only in ("pre", "all"):
        pre = synth.workload_cases("pre")
        pre_bytes = sum(algo_bytes(c.M, c.N, c.K) for c in pre)
        pre_u = [upload(c, copies_for(pre_bytes)) for c in pre]
        torch.cuda.synchronize()
        for i in range(max(3, args.warmup // 4)):
            for u in pre_u:
                launcher("gemm", u, i)()
                launcher("gemm_bf16", u, i)()
                launcher("gemm_fp16", u, i)()
        torch.cuda.synchronize()
        gsteps = max(10, args.steps // 4)
        per = {}
        tot_flop = tot_ms = 0.0
        for u in pre_u:
            c = u["case"]
            # the projection as called by default, and each operand path forced;
            # five alternating rounds, medians (the engine clock under this load
            # drifts by a few per cent between timed regions)
            runs = {"gemm": [], "gemm_bf16": [], "gemm_fp16": []}
            for rnd in range(5):
                for kind in runs:
                    t_ms, _ = timed_region(torch, [launcher(kind, u, i) for i in range(gsteps)],
                                           gsteps)
                    runs[kind].append(t_ms)
            ms, ms_b, ms_h = (sorted(runs[k])[2] for k in ("gemm", "gemm_bf16", "gemm_fp16"))
            flop = 2.0 * c.M * c.N * c.K
            tot_flop += flop
            tot_ms += ms
            per[c.name] = {"M": c.M, "N": c.N, "K": c.K, "us": round(ms * 1e3, 2),
                           "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                           "mfma_frac": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           "staged": bool(q4.gemm_staging_pays(c.M, c.N, c.K)),
                           "bf16_operands_us": round(ms_b * 1e3, 2),
                           "fp16_operands_us": round(ms_h * 1e3, 2)}
        tflops = tot_flop / (tot_ms * 1e-3) / 1e12
        out["prefill_gemm"] = {
            "workload": "prefill chunk M=512: qkv 5120->14336 + gate/up 5120->17408",
            "tflops": round(tflops, 1), "unit": "TFLOP/s",
            "note": "medians of five alternating rounds. us: the projection as the binding "
                    "calls it by default (staged: "
                    "gemm_xprep_kernel stages the activations as fp16, then gemm_kernel runs on "
                    "fp16 operands, both inside the timed region; not staged: gemm_kernel on "
                    "bf16 operands); bf16_operands_us / fp16_operands_us: each path forced. "
                    "All three give the same results bit for bit",
            "roofline": {"bound": "mfma", "kernel": "gemm_kernel (+ gemm_xprep_kernel where staged)",
                         "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": read_traffic("gemm_pre_counters.txt", src_digest("q4p_gemm.hip"),
                                                 None),
                         "kernel_source_sha256_16": src_digest("q4p_gemm.hip")},
            "tokens_per_s": round(512 / (tot_ms * 1e-3), 1),
            "per_matrix": per, "steps": gsteps}
        del pre_u

    # ---- the other decode-type shapes, the pack step ------------------------
    if args.only in ("shapes", "all"):
        shapes = {}
        for wl in ("mtp", "lmh"):
            for c in synth.workload_cases(wl):
                b = algo_bytes(c.M, c.N, c.K)
                u = upload(c, copies_for(b))
                n = max(10, args.steps // 4)
                for i in range(3):
                    launcher("gemv", u, i)()
                ms, _ = timed_region(torch, [launcher("gemv", u, i) for i in range(n)], n)
                shapes[f"{wl}/{c.name}"] = {"M": c.M, "N": c.N, "K": c.K,
                                            "us": round(ms * 1e3, 2),
                                            "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                                            "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                del u
        out["shapes"] = shapes
        # pack: read canonical + write packed bytes of the lm-head weight
        lm = synth.workload_cases("lmh", only=["lm_head"])[0].matrix
        codes = torch.from_numpy(lm.codes.reshape(-1)).to(dev)
        scales = torch.from_numpy(lm.scales.reshape(-1)).to(dev)
        pc = torch.empty(q4.q4proj_packed_codes_bytes(lm.N, lm.K), dtype=torch.uint8, device=dev)
        ps = torch.empty(q4.q4proj_packed_scales_bytes(lm.N, lm.K), dtype=torch.uint8, device=dev)
        for i in range(2):
            q4.q4proj_pack(codes, scales, lm.N, lm.K, pc, ps)
        ms, _ = timed_region(
            torch, [lambda: q4.q4proj_pack(codes, scales, lm.N, lm.K, pc, ps)] * 5, 5)
        moved = codes.numel() + scales.numel() + pc.numel() + ps.numel()
        out["pack"] = {"N": lm.N, "K": lm.K, "us": round(ms * 1e3, 1),
                       "gbs": round(moved / (ms * 1e-3) / 1e9, 1)}
        del codes, scales, pc, ps

    # ---- speculative verify: M = 1..16 rows at once ------------------------
    if args.only in ("verify", "all"):
        sweep = {}
        for c in synth.workload_cases("mtp"):
            N, K = c.N, c.K
            u = upload(c, copies_for(algo_bytes(16, N, K)))
            ys = {}
            per_m = {}
            n = max(10, args.steps // 8)
            for M in range(1, 17):
                xm = torch.from_numpy(synth.x_bf16(7, 40 + M, M, K).view(np.int16)).to(dev)
                ym = torch.empty((M, N), dtype=torch.float32, device=dev)
                ys[M] = (xm, ym)

                def vlaunch(i, M=M, xm=xm, ym=ym):
                    pc, ps = u["w"][i % len(u["w"])]
                    return lambda: q4.q4proj_gemv(pc, ps, u["g"], xm, ym, M, N, K)

                for i in range(3):
                    vlaunch(i)()
                ms, _ = timed_region(torch, [vlaunch(i) for i in range(n)], n)
                b = algo_bytes(M, N, K)
                per_m[M] = {"us": round(ms * 1e3, 2), "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            sweep[f"{c.name} {K}->{N}"] = per_m
            del u, ys
        out["verify_sweep"] = {
            "workload": "speculative verify: M = 1..16 activation rows through the NVFP4 GEMV "
                        "(MLP gate/up 5120->17408 and down 17408->5120)",
            "kernel": "gemv_sk_kernel<ceil(M/4), 4, KR, 0> (KR: joined k-ranges)",
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
            "per_matrix": sweep, "launches_per_M": max(10, args.steps // 8),
            "kernel_source_sha256_16": src_digest("q4p_gemv.hip")}

    # ---- fused gate/up + silu(gate)*up ------------------------------------
    if args.only in ("mlp", "all"):
        (c,) = synth.workload_cases("mlp")
        F, K = c.N // 2, c.K
        fused = {}
        for M in (1, 7):
            cm = synth.Case("mlp", c.name, M, c.matrix,
                            c.x if M == 1 else synth.x_bf16(5, 10 + M, M, K))
            b_plain = algo_bytes(M, 2 * F, K)
            u = upload(cm, copies_for(b_plain))
            h = torch.empty((M, F), dtype=torch.int16, device=dev)
            ws = torch.zeros(q4.q4proj_silu_mul_workspace_bytes(M, F, K), dtype=torch.uint8,
                             device=dev)

            def fused_launch(i, u=u, h=h, ws=ws, M=M):
                pc, ps = u["w"][i % len(u["w"])]
                return lambda: q4.q4proj_gemv_silu_mul(pc, ps, u["g"], u["x"], h, M, F, K,
                                                       workspace=ws)

            n = max(10, args.steps // 4)
            for i in range(3):
                fused_launch(i)()
                launcher("gemv", u, i)()
            ms_f, _ = timed_region(torch, [fused_launch(i) for i in range(n)], n)
            ms_p, _ = timed_region(torch, [launcher("gemv", u, i) for i in range(n)], n)
            b_fused = 2 * F * K // 2 + 2 * F * K // 16 + 2 * M * K + 2 * M * F + 4
            fused[f"M={M}"] = {
                "M": M, "F": F, "K": K, "us": round(ms_f * 1e3, 2),
                "gbs": round(b_fused / (ms_f * 1e-3) / 1e9, 1),
                "hbm_frac": round(b_fused / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "plain_gemv_2F_us": round(ms_p * 1e3, 2)}
            del u, h, ws
        # the M = 512 prefill chunk through the matrix-core path
        (cp,) = synth.workload_cases("pre", only=["gate_up"])
        M = cp.M
        cm = synth.Case("mlp", c.name, M, c.matrix, cp.x)
        u = upload(cm, copies_for(algo_bytes(M, 2 * F, K)))
        h = torch.empty((M, F), dtype=torch.int16, device=dev)

        def fused_gemm(i, u=u, h=h, ws=None):
            pc, ps = u["w"][i % len(u["w"])]
            return lambda: q4.q4proj_gemm_silu_mul(pc, ps, u["g"], u["x"], h, M, F, K, workspace=ws)

        n = max(10, args.steps // 8)
        for i in range(3):
            fused_gemm(i)()
            fused_gemm(i, ws=False)()
            launcher("gemm", u, i)()
        ms_f, _ = timed_region(torch, [fused_gemm(i) for i in range(n)], n)
        ms_fb, _ = timed_region(torch, [fused_gemm(i, ws=False) for i in range(n)], n)
        ms_p, _ = timed_region(torch, [launcher("gemm", u, i) for i in range(n)], n)
        flop = 2.0 * M * 2 * F * K
        fused[f"M={M}"] = {
            "M": M, "F": F, "K": K, "us": round(ms_f * 1e3, 2),
            "tflops": round(flop / (ms_f * 1e-3) / 1e12, 1),
            "mfma_frac": round(flop / (ms_f * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "bf16_operands_us": round(ms_fb * 1e3, 2),
            "plain_gemm_2F_us": round(ms_p * 1e3, 2)}
        del u, h
        out["fused_gate_up"] = {
            "workload": "fused gate/up 5120 -> 2x17408 NVFP4 projection + silu(gate)*up -> bf16",
            "kernels": ["gemv_sk_kernel<ROWS, 4, false, true> (M <= 16)",
                        "gemm_xprep_kernel + gemm_kernel<4, 1, true> (M = 512)"],
            "per_M": fused,
            "kernel_source_sha256_16": {"gemv": src_digest("q4p_gemv.hip"),
                                        "gemm": src_digest("q4p_gemm.hip")}}

    # ---- lm-head with the fused greedy argmax ------------------------------
    if args.only in ("argmax", "all"):
        (c,) = synth.workload_cases("lmh", only=["lm_head"])
        N, K = c.N, c.K
        lm = {}
        for M in (1, 7):
            cm = synth.Case("lmh", c.name, M, c.matrix,
                            c.x if M == 1 else synth.x_bf16(4, 20 + M, M, K))
            u = upload(cm, copies_for(algo_bytes(M, N, K)))
            val = torch.empty(M, dtype=torch.float32, device=dev)
            idx = torch.empty(M, dtype=torch.int64, device=dev)
            ws = torch.zeros(q4.q4proj_argmax_workspace_bytes(M, N, K), dtype=torch.uint8,
                             device=dev)

            def fused(i, u=u, val=val, idx=idx, ws=ws, M=M):
                pc, ps = u["w"][i % len(u["w"])]
                return lambda: q4.q4proj_gemv_argmax(pc, ps, u["g"], u["x"], None, val, idx,
                                                     M, N, K, workspace=ws)

            def unfused(i, u=u):
                f = launcher("gemv", u, i)
                return lambda: (f(), torch.argmax(u["y"], dim=1))

            n = max(10, args.steps // 8)
            for i in range(3):
                fused(i)()
                unfused(i)()
            ms_f, _ = timed_region(torch, [fused(i) for i in range(n)], n)
            ms_u, _ = timed_region(torch, [unfused(i) for i in range(n)], n)
            b = N * K // 2 + N * K // 16 + 2 * M * K + 12 * M + 4
            lm[f"M={M}"] = {"M": M, "N": N, "K": K, "us": round(ms_f * 1e3, 2),
                            "gbs": round(b / (ms_f * 1e-3) / 1e9, 1),
                            "hbm_frac": round(b / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "gemv_plus_torch_argmax_us": round(ms_u * 1e3, 2)}
            del u, val, idx, ws
        out["lm_head_argmax"] = {
            "workload": "lm-head 5120 -> 248320 NVFP4 GEMV + greedy argmax, no logits written",
            "kernel": "gemv_sk_kernel<ROWS, 4, false, 2>", "per_M": lm,
            "kernel_source_sha256_16": src_digest("q4p_gemv.hip")}

    # ---- NVFP4 quantizer --------------------------------------------------
    if args.only in ("quant", "all"):
        quant = {}
        gen = torch.Generator(device=dev)
        for name, N, K in (("gate_up_fused", 34816, 5120), ("lm_head", 248320, 5120)):
            gen.manual_seed(6)
            w = (torch.randn(N * K, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            codes = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
            scales = torch.empty(N * K // 16, dtype=torch.uint8, device=dev)
            gq = torch.empty(1, dtype=torch.float32, device=dev)
            ws = torch.empty(q4.q4proj_quantize_workspace_bytes(N, K), dtype=torch.uint8,
                             device=dev)
            run = lambda: q4.q4proj_quantize(w, N, K, codes, scales, gq, workspace=ws)
            for _ in range(2):
                run()
            n = 5
            ms, _ = timed_region(torch, [run] * n, n)
            b = 2 * N * K + N * K // 2 + N * K // 16 + 4
            quant[name] = {"N": N, "K": K, "us": round(ms * 1e3, 1),
                           "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                           "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "read_bytes_per_weight": 4, "algorithmic_bytes": b}
            del w, codes, scales, gq, ws
        out["quantize"] = {"workload": "bf16 -> NVFP4 (codes, e4m3 scales, g), synthetic "
                                       "N(0, 0.02) weights", "per_matrix": quant,
                           "kernels": ["quant_amax_kernel", "quant_kernel"],
                           "kernel_source_sha256_16": src_digest("q4p_quant.hip")}

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # ---- CPU baseline: the oracle on the decode step ----------------------
    if not args.skip_cpu and args.only in ("dec", "all"):
        import oracle
        nthreads = oracle.default_threads()
        reps = 0
        t = time.perf_counter()
        while True:
            for c in dec:
                oracle.proj(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t
            if el >= args.cpu_seconds or reps >= 50:
                break
        out["cpu_baseline"] = {"value": round(step_bytes * reps / el / 1e9, 3), "unit": "GB/s",
                               "cores": nthreads, "kind": "oracle",
                               "host_cpu_count": os.cpu_count(),
                               "threads_rule": "one oracle thread per CPU this process may run "
                                               "on (its affinity mask), not os.cpu_count()",
                               "sample": f"{reps} full decode steps (gate/up + down, M=1, "
                                         f"all rows) in {el:.2f} s, fp64",
                               "tokens_per_s": round(reps / el, 2),
                               "single_thread": single_thread_oracle(oracle, synth, dec)}

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
