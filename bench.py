"""Benchmark of the fused 8-bit AdamW step with a stochastically rounded bf16 write.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gptneo-6.7b]
                    [--algo adamw|lion|momentum]

One step = one opt8_adamw_step call over the whole parameter list (every
tensor: dequantise, AdamW in fp32, stochastic bf16 param write, block absmax,
requantise); --algo lion / momentum time the one-state rules on the same list.
Inputs are synthetic and already resident in HBM when the timed region starts;
a small pool of gradient sets gives each step fresh gradients without
generating them inside the timed region.  Without --steps/--warmup, both loops
run at least 20 / 10 steps and at least a quarter of a second each (a list of
many small tensors steps in about 0.26 ms; the GPU clock needs tens of
milliseconds to settle).  Prints ONE JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
# The GPU's clock takes tens of milliseconds to settle after the first launches: a
# short step (a list of many small tensors takes about 0.26 ms) warms up and is timed
# over at least this long, so the rate is the one a training loop sees.
MIN_WARM_S = 0.25
MIN_TIMED_S = 0.25
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
METRIC = "Gparams/s per optimizer step and % of HBM peak BW, 1 MI355X"
BLOCK = 2048
STATE_BYTES = {0: 1, 1: 2, 2: 4}


def algorithmic_bytes(mode: int, n: int, one_state: bool = False) -> int:
    """Bytes each element's step must move once: read grad, param, state; write param, state."""
    if one_state:   # m only: g 2 + p 2+2 + m r/w (8-bit 1+1 and 8 B absmax per block, bf16 2+2, fp32 4+4)
        if mode == 0:
            return 8 * n + 8 * ((n + BLOCK - 1) // BLOCK)
        return 10 * n if mode == 1 else 14 * n
    if mode == 0:   # 8-bit: 2+2+1+1 in, 2+1+1 out, plus absmax r/w (2 x 4 B in, 2 x 4 B out) per block
        return 10 * n + 16 * ((n + BLOCK - 1) // BLOCK)
    if mode == 1:   # bf16 state: g 2 + p 2+2 + m, v 2+2 in / 2+2 out
        return 14 * n
    return 22 * n   # fp32 state: g 2 + p 2+2 + m, v 4+4 in / 4+4 out


def profiled_traffic(kernel: str, workload: str, key: str = "traffic_bytes"):
    """A figure (default: HBM bytes per launch) from a committed rocprofv3 summary of this
    exact kernel build and workload, or None."""
    import glob
    from precision_optimizer_step_amd.build import kernel_fingerprint
    fp = kernel_fingerprint()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        text = open(path).read()
        if "bench-traffic" not in text:
            continue
        block = text.split("bench-traffic", 1)[1].split("```", 1)[0]
        kv = dict(ln.split(": ", 1) for ln in block.strip().splitlines() if ": " in ln)
        if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("fingerprint") == fp:
            return float(kv[key]) if key in kv else None
    return None


def probe_bandwidth(dev, words=1 << 27, reps=5):
    """Best GB/s of the streaming probe over grid sizes from the resident count to 32 times it
    (a grid larger than what fits lets finished workgroups be replaced, which the step kernels
    need too): 1 read + 1 write stream, and 3 read + 2 write streams (the 8-bit step's 6 B
    read : 4 B written per element); and of the probe with the 8-bit step's own access pattern
    (four read and three write streams in 2048-element blocks, no arithmetic), the best of one
    and two adjacent blocks per wave over grids from 2 to 256 workgroups per CU."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "precision_optimizer_step_amd", "libopt8_probe.so")
    if not os.path.exists(path):
        return {}
    lib = ctypes.CDLL(path)
    lib.opt8_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    inp = torch.empty(3 * words * 16, dtype=torch.uint8, device=dev).random_(0, 255)
    out = torch.empty(2 * words * 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {}
    for name, nin, nout in (("copy", 1, 1), ("mix", 3, 2)):
        best = 0.0
        for grid in (cus * 8, cus * 16, cus * 32, cus * 64, cus * 128, cus * 256):
            def run():
                assert lib.opt8_probe_stream(inp.data_ptr(), out.data_ptr(), words, nin, nout, grid,
                                             stream) == 0
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = max(best, (nin + nout) * words * 16 * reps / (e0.elapsed_time(e1) / 1000.0) / 1e9)
        res[name] = round(best, 1)
    del inp, out
    # the 8-bit step's own access pattern (10 B per element, no arithmetic)
    lib.opt8_probe_pattern.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                 ctypes.c_void_p]
    nblocks = 1 << 18
    n = nblocks * BLOCK
    g = torch.empty(n, dtype=torch.int16, device=dev).random_(-32768, 32767)
    p = torch.empty(n, dtype=torch.int16, device=dev).random_(-32768, 32767)
    m = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
    v = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
    for per_wave in (1, 2):
        best = 0.0
        for grid in (cus * 2, cus * 4, cus * 8, cus * 16, cus * 32, cus * 64, cus * 128, cus * 256):
            def run():
                assert lib.opt8_probe_pattern(g.data_ptr(), p.data_ptr(), m.data_ptr(), v.data_ptr(), nblocks,
                                              grid, per_wave, stream) == 0
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = max(best, 10 * n * reps / (e0.elapsed_time(e1) / 1000.0) / 1e9)
        res[f"pattern_8bit_{per_wave}"] = round(best, 1)
    res["pattern_8bit"] = max(res["pattern_8bit_1"], res["pattern_8bit_2"])
    del g, p, m, v
    torch.cuda.empty_cache()
    return res


class ClockSampler:
    """GFX (per XCD) and memory clocks of the GPU torch uses, read from the driver's metrics
    table (amdsmi) by a host thread; empty if amdsmi is unavailable.  The table refreshes
    only every few hundred milliseconds, so the clocks are sampled while the step runs back
    to back for a few seconds, and samples from the first second are dropped.  Also read: the
    socket power, and the share of the sampled time the firmware spent holding the package
    power limit (the PPT residency counter against the metrics' millisecond accumulation
    counter)."""

    def __init__(self, pci_bus=None, period_s=0.05, settle_s=1.0):
        import threading
        self.period, self.settle = period_s, settle_s
        self.gfx, self.xcd, self.mem, self.power = [], [], [], []
        self.acc = []   # (accumulation_counter, ppt_residency_acc) per sample
        self.cap_w = None
        self.err = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            # the handle of the GPU torch uses: the same PCI bus number
            match = [h for h in handles
                     if pci_bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == pci_bus]
            if len(match) != 1 and len(handles) != 1:
                raise RuntimeError(f"cannot tell which of {len(handles)} GPUs is in use")
            self.handle = match[0] if len(match) == 1 else handles[0]
            self.smi.amdsmi_get_gpu_metrics_info(self.handle)
            try:   # microwatts
                self.cap_w = amdsmi.amdsmi_get_power_cap_info(self.handle)["power_cap"] / 1e6
            except Exception:
                self.cap_w = None
        except Exception as e:   # no amdsmi or no permission: the clock is reported as unknown
            self.smi = None
            self.err = f"{type(e).__name__}: {e}"

    def _loop(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
                if time.perf_counter() - t0 >= self.settle:
                    self.gfx.append(float(m["current_gfxclk"]))
                    self.mem.append(float(m["current_uclk"]))
                    xs = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float))]
                    if xs:
                        self.xcd.append(xs)
                    if isinstance(m.get("current_socket_power"), (int, float)):
                        self.power.append(float(m["current_socket_power"]))
                    a, r = m.get("accumulation_counter"), m.get("ppt_residency_acc")
                    if isinstance(a, (int, float)) and isinstance(r, (int, float)):
                        self.acc.append((a, r))
            except Exception as e:
                self.err = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.smi is not None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self, note):
        if not self.gfx:
            return {"gfx_mhz": None, "mem_mhz": None, "samples": 0, "source": "amdsmi gpu metrics",
                    "note": self.err or "no samples"}
        g, m = sorted(self.gfx), sorted(self.mem)
        out = {"gfx_mhz": {"median": g[len(g) // 2], "min": g[0], "max": g[-1]},
               "mem_mhz": {"median": m[len(m) // 2], "min": m[0], "max": m[-1]},
               "samples": len(g), "source": "amdsmi gpu metrics (current_gfxclk, current_uclk)", "note": note}
        if self.xcd:
            per = list(zip(*self.xcd))
            out["gfx_mhz_per_xcd_median"] = [sorted(x)[len(x) // 2] for x in per]
        if self.power:
            pw = sorted(self.power)
            out["socket_power_w"] = {"median": pw[len(pw) // 2], "max": pw[-1], "cap": self.cap_w}
        if len(self.acc) >= 2 and self.acc[-1][0] > self.acc[0][0]:
            out["power_limited_frac"] = round((self.acc[-1][1] - self.acc[0][1]) / (self.acc[-1][0] - self.acc[0][0]), 3)
        return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 20, and enough for about %.2f s)" % MIN_TIMED_S)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 10, and enough for about %.2f s)" % MIN_WARM_S)
    ap.add_argument("--workload", default="gptneo-6.7b")
    ap.add_argument("--grad-pool", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--round", choices=("stochastic", "nearest"), default="stochastic",
                    help="parameter rounding (nearest: the deterministic baseline, for the SR overhead)")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="untimed phase after the timed steps in which the GPU clock is sampled (0: skip)")
    ap.add_argument("--cpu-cap-elems", type=int, default=1 << 24,
                    help="oracle leg: elements taken from the start of each tensor of the fixed subset")
    ap.add_argument("--algo", choices=("adamw", "lion", "momentum"), default="adamw",
                    help="update rule (lion / momentum: one 8-bit state, the same machinery)")
    ap.add_argument("--state-round", choices=("nearest", "stochastic"), default="nearest",
                    help="8-bit state rounding: nearest codebook entry, or stochastic between neighbours")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from precision_optimizer_step_amd import opt8
    from workloads import gen, shapes

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    opt8.opt8_init_codebooks()
    try:
        w = shapes.get(args.workload)
    except ValueError as e:
        print(json.dumps({"error": str(e)}))
        sys.exit(2)
    one_state = args.algo != "adamw"
    algo_id = {"adamw": 0, "lion": 1, "momentum": 2}[args.algo]
    step_fn = {"adamw": opt8.opt8_adamw_step, "lion": opt8.opt8_lion_step,
               "momentum": opt8.opt8_momentum_step}[args.algo]
    # hyperparameters: the workload's for AdamW; Lion at a tenth of its lr with beta2 0.99
    # (the usual Lion setting), momentum 0.9 at the workload's lr
    lr = w.lr / 10 if args.algo == "lion" else w.lr
    beta2 = 0.99 if args.algo == "lion" else w.beta2

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- inputs in HBM
    t0 = time.time()
    if args.steps is None or args.warmup is None:
        pool = max(1, args.grad_pool)
    else:
        pool = max(1, min(args.grad_pool, args.steps + args.warmup))
    tensors = []
    modes = {0: 0, 1: 0, 2: 0}
    alg = {0: 0, 1: 0, 2: 0}
    for tid, spec in enumerate(w.tensors):
        n = spec.numel
        mode = 1 if w.state_mode == "bf16" else opt8.opt8_default_mode(n)
        P = torch.empty(n, dtype=torch.bfloat16, device=dev)
        gen.param_init_device(spec, w, tid, P)
        grads = []
        for k in range(pool):
            G = torch.empty(n, dtype=torch.bfloat16, device=dev)
            gen.grad_init_device(spec, w, k + 1, tid, G)
            grads.append(G)
        AM = AV = None
        if mode == 0:
            M = torch.full((n,), 127, dtype=torch.uint8, device=dev)
            V = torch.zeros(n, dtype=torch.uint8, device=dev)
            nb = (n + BLOCK - 1) // BLOCK
            AM = torch.zeros(nb, dtype=torch.float32, device=dev)
            AV = torch.zeros(nb, dtype=torch.float32, device=dev)
        elif mode == 1:
            M = torch.zeros(n, dtype=torch.bfloat16, device=dev)
            V = torch.zeros(n, dtype=torch.bfloat16, device=dev)
        else:
            M = torch.zeros(n, dtype=torch.float32, device=dev)
            V = torch.zeros(n, dtype=torch.float32, device=dev)
        if one_state:
            V = AV = None
        tensors.append(dict(tid=tid, mode=mode, n=n, P=P, grads=grads, M=M, V=V, AM=AM, AV=AV))
        modes[mode] += n
        alg[mode] += algorithmic_bytes(mode, n, one_state)
    torch.cuda.synchronize()
    total = sum(t["n"] for t in tensors)
    log(f"workload {w.name}: {len(tensors)} tensors, {total} params, inputs built in {time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    lists = [opt8.tensor_array(opt8.make_tensor(t["P"], t["grads"][k], t["M"], t["V"], t["AM"], t["AV"],
                                                tensor_id=t["tid"], mode=t["mode"]) for t in tensors)
             for k in range(pool)]

    rnd = opt8.OPT8_ROUND_NEAREST if args.round == "nearest" else opt8.OPT8_ROUND_STOCHASTIC
    srnd = opt8.OPT8_STATE_ROUND_STOCHASTIC if args.state_round == "stochastic" else opt8.OPT8_STATE_ROUND_NEAREST

    def step(t):
        hp = opt8.make_hparams(lr, w.beta1, beta2, w.eps, w.weight_decay, step=t, seed=w.seed,
                               param_round=rnd, state_round=srnd)
        step_fn(lists[(t - 1) % pool], hp)

    # ---------------------------------------------------------------- timing
    # step 1 (zero state) is timed on its own inside the warmup: its blocks start from absmax 0
    t_step = 1
    step1_ms = None
    warmup = 0
    est_s = None
    if args.warmup is None or args.warmup > 0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(t_step)
        e1.record()
        torch.cuda.synchronize()
        step1_ms = e0.elapsed_time(e1)
        t_step += 1
        warmup = 1
        if args.warmup is None:
            # chunks of steps until a quarter second has passed; the last chunk's
            # rate sizes the default timed loop
            c0 = time.perf_counter()
            chunk = 9
            while True:
                c1 = time.perf_counter()
                for _ in range(chunk):
                    step(t_step)
                    t_step += 1
                torch.cuda.synchronize()
                warmup += chunk
                est_s = (time.perf_counter() - c1) / chunk
                if warmup >= 10 and time.perf_counter() - c0 >= MIN_WARM_S:
                    break
                chunk = max(8, min(4 * chunk, int(0.05 / est_s)))
        else:
            c1 = time.perf_counter()
            for _ in range(args.warmup - 1):
                step(t_step)
                t_step += 1
            torch.cuda.synchronize()
            warmup = args.warmup
            if args.warmup > 1:
                est_s = (time.perf_counter() - c1) / (args.warmup - 1)
    steps = args.steps
    if steps is None:
        steps = max(20, math.ceil(MIN_TIMED_S / est_s)) if est_s else 20
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(steps):
        starts[k].record()
        step(t_step)
        ends[k].record()
        t_step += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # the GPU clock under this step: the step again back to back for about clock_s seconds
    # (untimed), the driver's clocks sampled meanwhile
    clock_s = args.clock_seconds
    clocks = ClockSampler(getattr(torch.cuda.get_device_properties(dev), "pci_bus_id", None))
    n_clock = 0
    if clock_s > 0 and clocks.smi is not None:
        est_ms = max(wall * 1000.0 / steps, 0.05)
        with clocks:
            c0 = time.perf_counter()
            while time.perf_counter() - c0 < clock_s:
                for _ in range(max(1, int(200.0 / est_ms))):
                    step(t_step)
                    t_step += 1
                    n_clock += 1
                torch.cuda.synchronize()
    clock_note = (f"sampled every 50 ms while {n_clock} more steps ran back to back after the timed ones "
                  f"(about {clock_s:.0f} s, untimed), the first second dropped")
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1000.0 / steps
    ev_avg = sum(ev_ms) / len(ev_ms)
    value = total / (ms_per_step / 1000.0) / 1e9
    log(f"wall {ms_per_step:.3f} ms/step; events per step: avg {ev_avg:.3f} min {min(ev_ms):.3f} "
        f"max {max(ev_ms):.3f} ms")

    # dominant kernel: the largest share of algorithmic bytes
    dom = max(alg, key=lambda k: alg[k])
    only_dom = all(v == 0 for k, v in modes.items() if k != dom)
    kernel_ms = ev_avg if only_dom else None
    roof = None
    if kernel_ms:
        achieved = alg[dom] / (kernel_ms / 1000.0) / 1e9
        kname = {0: "step_kernel<8bit>", 1: "step_kernel<bf16>", 2: "step_kernel<fp32>"}[dom]
        if one_state:
            kname = kname[:-1] + f",{args.algo}>"
        if srnd and dom == 0:
            kname = kname[:-1] + ",sr-state>"
        traffic = profiled_traffic(kname, w.name)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": int(traffic) if traffic else None,
                "valu_issue_frac": profiled_traffic(kname, w.name, "valu_issue_frac"),
                # rocprofv3's VALU-busy figure (SQ_ACTIVE_INST_VALU x 4 / SIMDs / cycles), from the profile of the same kernel fingerprint
                "valu_busy": profiled_traffic(kname, w.name, "valu_busy"),
                "frac_of_attainable": None,
                "kernel": kname,
                "algorithmic_bytes_per_launch": alg[dom], "avg_launch_ms": round(kernel_ms, 4)}
        ragged = sum(1 for t in tensors if t["mode"] == 0 and t["n"] % BLOCK)
        if dom == 0 and ragged:
            # the library launches the last partial blocks of 8-bit tensors separately: the
            # HIP events bracket both launches, and the bytes are those of both
            roof["kernel"] = kname + " + its last-partial-block launch"
            roof["note"] = (f"one step is two launches (full blocks; the last partial block of each of "
                            f"{ragged} tensors), timed and counted together")

    # attainable streaming bandwidth on this machine: the probe kernels (libopt8_probe.so) with a
    # plain 1:1 copy and with the step's own 3:2 read:write mix, 16-byte accesses
    attain = probe_bandwidth(dev)
    if roof and attain.get("mix"):
        roof["frac_of_attainable"] = round(roof["achieved"] / attain["mix"], 4)
    if roof and dom == 0 and not one_state and attain.get("pattern_8bit"):
        roof["frac_of_step_pattern"] = round(roof["achieved"] / attain["pattern_8bit"], 4)

    # ---------------------------------------------------------------- CPU baseline (oracle) + parity
    # The oracle, single-threaded, on a bounded fixed subset of the list: the embeddings, every
    # tensor of the first and the last layer and the final LayerNorm, each tensor cut to its
    # first --cpu-cap-elems elements (whole blocks, so the cut changes no result).  Its inputs
    # are the state left by the timed steps and the next gradient set; the GPU then runs one
    # more step (untimed) over the whole list, and its outputs for the subset are compared
    # with the oracle's element by element.  The oracle's rate, times the list's element
    # count, gives an extrapolated single-core time for a whole step.
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        subset = [tid for tid in shapes.subset_for_sampling(w) if tid < len(tensors)]
        if len(subset) < 2:
            # lists without the model layout (many small tensors, one tensor): their first
            # tensors, up to one cap's worth of elements
            subset, acc = [], 0
            for t in tensors:
                if acc >= args.cpu_cap_elems:
                    break
                subset.append(t["tid"])
                acc += min(t["n"], args.cpu_cap_elems)
        sd = {0: np.uint8, 1: np.uint16, 2: np.float32}

        def host(t, lo, hi, dtype):
            if t is None:
                return None
            h = t[lo:hi].detach().cpu()
            if h.dtype == torch.bfloat16:
                h = h.view(torch.int16)
            return h.numpy().view(dtype).copy()
        gi = (t_step - 1) % pool
        inputs = []
        for tid in subset:
            t = tensors[tid]
            n = min(t["n"], args.cpu_cap_elems)
            nb = (n + BLOCK - 1) // BLOCK
            inputs.append(dict(t=t, n=n, p=host(t["P"], 0, n, np.uint16), g=host(t["grads"][gi], 0, n, np.uint16),
                               m=host(t["M"], 0, n, sd[t["mode"]]), v=host(t["V"], 0, n, sd[t["mode"]]),
                               am=host(t["AM"], 0, nb, np.float32), av=host(t["AV"], 0, nb, np.float32)))
        step(t_step)                   # one more GPU step, outside the timed region
        torch.cuda.synchronize()
        hp = oracle.Hparams(lr=lr, beta1=w.beta1, beta2=beta2, eps=w.eps, weight_decay=w.weight_decay,
                            step=t_step, seed=w.seed, param_round=rnd, state_round=srnd)
        n_el = sum(x["n"] for x in inputs)
        mism = {"param": 0, "state": 0, "absmax": 0}
        max_step = 0
        cpu_s = 0.0
        for x in inputs:
            t, n = x["t"], x["n"]
            nb = (n + BLOCK - 1) // BLOCK
            c0t = time.perf_counter()
            if one_state:
                pw, mw, amw = oracle.step_tensor_1state(algo_id, t["mode"], x["p"], x["g"], x["m"], x["am"], hp,
                                                        t["tid"])
                want = [pw, mw, None, amw, None]
            else:
                want = list(oracle.step_tensor(t["mode"], x["p"], x["g"], x["m"], x["v"], x["am"], x["av"], hp,
                                               t["tid"]))
            cpu_s += time.perf_counter() - c0t
            got = [host(t["P"], 0, n, np.uint16), host(t["M"], 0, n, sd[t["mode"]]),
                   host(t["V"], 0, n, sd[t["mode"]]), host(t["AM"], 0, nb, np.float32),
                   host(t["AV"], 0, nb, np.float32)]
            mism["param"] += int(np.count_nonzero(got[0] != want[0]))
            for k in (1, 2):
                if want[k] is not None:
                    a_, b_ = got[k].view(np.uint8 if want[k].dtype == np.uint8 else
                                         np.uint16 if want[k].dtype == np.uint16 else np.uint32), \
                        want[k].view(np.uint8 if want[k].dtype == np.uint8 else
                                     np.uint16 if want[k].dtype == np.uint16 else np.uint32)
                    mism["state"] += int(np.count_nonzero(a_ != b_))
                    if want[k].dtype == np.uint8:
                        max_step = max(max_step, int(np.abs(a_.astype(np.int64) - b_.astype(np.int64)).max(initial=0)))
            for k in (3, 4):
                if want[k] is not None:
                    gk, wk = got[k].astype(np.float64), want[k].astype(np.float64)
                    mism["absmax"] += int(np.count_nonzero(
                        (np.isnan(gk) != np.isnan(wk)) | (np.abs(gk - wk) > 1e-6 * np.abs(wk))))
        rate = n_el / cpu_s
        names = [w.tensors[tid].name for tid in subset]
        layers = sorted({n.split(".")[0] for n in names if "." in n and not n.startswith("ln_f")},
                        key=lambda x: (len(x), x))
        which = ", ".join([n for n in names if "." not in n] + [f"layer {x}" for x in layers]
                          + [n for n in names if n.startswith("ln_f")]) if len(names) > 3 else ", ".join(names)
        if len(which) > 160:
            which = f"{names[0]} ... {names[-1]}"
        cpu = {"value": round(rate / 1e9, 6), "unit": "Gparams/s", "cores": 1, "kind": "oracle",
               "sample": f"one step of {n_el} elements: the first min(numel, {args.cpu_cap_elems}) elements of "
                         f"each of {len(subset)} tensors ({which}); {cpu_s:.1f} s, numpy, "
                         f"single thread, of {os.cpu_count()} host cores",
               "extrapolated_full_step_s": round(total / rate, 1),
               "extrapolated": "full-list single-core time = the subset's elements/s x the list's elements"}
        parity = {"elements": n_el, "tensors": len(subset), "step": t_step,
                  "mismatch_param": mism["param"], "mismatch_state": mism["state"],
                  "mismatch_absmax": mism["absmax"], "max_code_distance": max_step,
                  "allowed_per_kind": int(1e-5 * n_el),
                  "ok": mism["absmax"] == 0 and max_step <= 1 and
                  max(mism["param"], mism["state"]) <= int(1e-5 * n_el)}
        log(f"oracle: {n_el} elements in {cpu_s:.2f}s; parity of the extra step: {parity}")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tensors": len(tensors), "params": total,
                   "state": "bf16-sr" if w.state_mode == "bf16" else "8bit+fp32<4096",
                   "param_round": args.round, "algo": args.algo, "state_round": args.state_round,
                   "grad_pool": pool, "hbm_pct_of_peak": round(100 * sum(alg.values()) / (ms_per_step / 1000.0)
                                                              / 1e9 / HBM_PEAK_GBPS, 2),
                   "attainable_copy_GBps": attain.get("copy"),
                   "attainable_3r2w_GBps": attain.get("mix"),
                   "attainable_8bit_step_pattern_GBps": attain.get("pattern_8bit"),
                   "attainable_8bit_step_pattern_one_block_per_wave_GBps": attain.get("pattern_8bit_1")},
        "roofline": roof,
        "timing": {"median_ms": round(sorted(ev_ms)[len(ev_ms) // 2], 4), "min_ms": round(min(ev_ms), 4),
                   "max_ms": round(max(ev_ms), 4),
                   "step1_ms": round(step1_ms, 4) if step1_ms is not None else None},
        "cpu_baseline": cpu,
        "parity": parity,
        "gpu_clock": clocks.summary(clock_note),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
