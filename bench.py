"""Benchmark of the fused 8-bit AdamW step with a stochastically rounded bf16 write.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gptneo-6.7b]
                    [--algo adamw|lion|momentum]

One step = one opt8_adamw_step call over the whole parameter list (every
tensor: dequantise, AdamW in fp32, stochastic bf16 param write, block absmax,
requantise); --algo lion / momentum time the one-state rules on the same list.
Inputs are synthetic and already resident in HBM when the timed region starts;
a small pool of gradient sets gives each step fresh gradients without
generating them inside the timed region.  Prints ONE JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
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
    """Best GB/s of the streaming probe over three grid sizes: 1 read + 1 write stream, and
    3 read + 2 write streams (the 8-bit step's 6 B read : 4 B written per element); and of the
    probe with the 8-bit step's own access pattern (four read and three write streams in
    2048-element blocks, no arithmetic), the best of one and two adjacent blocks per wave."""
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
        for grid in (cus * 8, cus * 16, cus * 32):
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
        for grid in (cus * 2, cus * 3, cus * 4, cus * 8):
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gptneo-6.7b")
    ap.add_argument("--grad-pool", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--round", choices=("stochastic", "nearest"), default="stochastic",
                    help="parameter rounding (nearest: the deterministic baseline, for the SR overhead)")
    ap.add_argument("--cpu-sample-elems", type=int, default=128 * 1024 * 1024)
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
    w = shapes.get(args.workload)
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
    for w_i in range(args.warmup):
        if w_i == 0:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(t_step)
            e1.record()
            torch.cuda.synchronize()
            step1_ms = e0.elapsed_time(e1)
        else:
            step(t_step)
        t_step += 1
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record()
        step(t_step)
        ends[k].record()
        t_step += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1000.0 / args.steps
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

    # attainable streaming bandwidth on this machine: the probe kernels (libopt8_probe.so) with a
    # plain 1:1 copy and with the step's own 3:2 read:write mix, 16-byte accesses
    attain = probe_bandwidth(dev)
    if roof and attain.get("mix"):
        roof["frac_of_attainable"] = round(roof["achieved"] / attain["mix"], 4)
    if roof and dom == 0 and not one_state and attain.get("pattern_8bit"):
        roof["frac_of_step_pattern"] = round(roof["achieved"] / attain["pattern_8bit"], 4)

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        big = max(tensors, key=lambda t: t["n"] if t["mode"] == dom else -1)
        n = min(big["n"], args.cpu_sample_elems)
        sd = {0: np.uint8, 1: np.uint16, 2: np.float32}[big["mode"]]

        def host(t, dtype):
            h = t[:n].detach().cpu()
            if h.dtype == torch.bfloat16:
                h = h.view(torch.int16)
            return h.numpy().view(dtype).copy()
        p, g = host(big["P"], np.uint16), host(big["grads"][0], np.uint16)
        m = host(big["M"], sd)
        v = host(big["V"], sd) if big["V"] is not None else None
        am = big["AM"][: (n + BLOCK - 1) // BLOCK].cpu().numpy() if big["AM"] is not None else None
        av = big["AV"][: (n + BLOCK - 1) // BLOCK].cpu().numpy() if big["AV"] is not None else None
        hp = oracle.Hparams(lr=lr, beta1=w.beta1, beta2=beta2, eps=w.eps,
                            weight_decay=w.weight_decay, step=t_step, seed=w.seed, state_round=srnd)
        c0t = time.perf_counter()
        if one_state:
            oracle.step_tensor_1state(algo_id, big["mode"], p, g, m, am, hp, big["tid"])
        else:
            oracle.step_tensor(big["mode"], p, g, m, v, am, av, hp, big["tid"])
        cpu_s = time.perf_counter() - c0t
        cpu = {"value": round(n / cpu_s / 1e9, 6), "unit": "Gparams/s", "cores": 1, "kind": "oracle",
               "sample": f"one step of the first {n} elements of tensor {w.tensors[big['tid']].name} "
                         f"({cpu_s:.1f} s, numpy single thread, of {os.cpu_count()} host cores)"}
        log(f"oracle: {n} elements in {cpu_s:.2f}s")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
