"""Benchmark of the fused 8-bit block-wise optimizer step on one MI355X.

Default workload: 8-bit AdamW (wd 0.01), one 4096x4096 fp32 parameter tensor,
block 256, synthetic seeded inputs already resident in HBM.  One "step" is one
fused kernel launch over the whole tensor (decode, update, absmax, re-encode,
parameter write).  To keep the 256 MB Infinity Cache from serving the ~270 MB
working set, consecutive steps rotate over R independent replicas (parameters,
gradients, codes, absmax), so every step streams its bytes from HBM.

Output: one JSON line (rank 0) with the throughput, the kernel's roofline
position (algorithmic bytes / average launch time from HIP events on the launch
stream) and the CPU oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np
import torch

from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W

METRIC = "8-bit Adam step: Gelem/s and achieved HBM GB/s (% of peak) at 4096×4096 fp32"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public spec
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def workload_by_name(name):
    table = {
        "adamw_fp32_b256": lambda: W.c2_adamw_4096("f32", 256),
        "adamw_fp32_b2048": lambda: W.c2_adamw_4096("f32", 2048),
        "adamw_fp16_b256": lambda: W.c2_adamw_4096("f16", 256),
        "adamw_fp16_b2048": lambda: W.c2_adamw_4096("f16", 2048),
        "ademamix_bf16_b256": W.c3_ademamix_4096,
        "momentum_fp16_skip0": lambda: W.c4_embedding("momentum", False),
        "momentum_fp16_skip1": lambda: W.c4_embedding("momentum", True),
        "lion_fp16_skip0": lambda: W.c4_embedding("lion", False),
        "lion_fp16_skip1": lambda: W.c4_embedding("lion", True),
        "adam_fp32_256x256": W.c1_adam_256,
    }
    return table[name]()


class Replica:
    """Device buffers of one independent copy of the workload's single tensor."""

    def __init__(self, wl, r, dev):
        t = wl.tensors[0]
        self.n = n = t.numel
        hp = wl.hp
        B = hp["blocksize"]
        nb = (n + B - 1) // B
        dt = TORCH_DT[t.dtype]
        k1 = 2 if hp["optimizer"] == "ademamix" else 1
        self.two = hp["optimizer"] in ("adam", "adamw", "ademamix")
        p = W.normal_f32([wl.seed, 1, 0, r], n, wl.p_scale)
        g = W.normal_f32([wl.seed, 2, 0, r], n, wl.g_scale)
        if wl.zero_row_frac:
            rows = t.shape[0]
            mask = W.zero_row_mask([wl.seed, 3, 0, r], rows, wl.zero_row_frac)
            g.reshape(rows, -1)[mask] = 0.0
        self.p = torch.from_numpy(p).to(dev).to(dt)
        self.g = torch.from_numpy(g).to(dev).to(dt)
        self.s1 = torch.zeros(k1 * n, dtype=torch.uint8, device=dev)
        self.a1 = torch.zeros(k1 * nb, dtype=torch.float32, device=dev)
        self.s2 = torch.zeros(n, dtype=torch.uint8, device=dev) if self.two else None
        self.a2 = torch.zeros(nb, dtype=torch.float32, device=dev) if self.two else None

    def step(self, hp, t, q1, q2):
        if self.two:
            bitopt.step_8bit_blockwise_2state(hp, t, self.p, self.g, self.s1, self.s2, self.a1, self.a2, q1, q2)
        else:
            bitopt.step_8bit_blockwise_1state(hp, t, self.p, self.g, self.s1, self.a1, q1)


def cpu_baseline(wl, target_s=15.0):
    """The oracle, as it stands, on a bounded sample of the same workload's blocks."""
    import oracle
    t = wl.tensors[0]
    hp = wl.hp
    B = hp["blocksize"]
    n_all = t.numel
    threads = oracle.get_threads()

    def run(nblocks):
        n = min(n_all, nblocks * B)
        p = W.to_dtype(W.normal_f32([wl.seed, 1, 0, 0], n_all, wl.p_scale, 0, n), t.dtype)
        g = W.to_dtype(W.normal_f32([wl.seed, 2, 0, 0], n_all, wl.g_scale, 0, n), t.dtype)
        nb = (n + B - 1) // B
        k1 = 2 if hp["optimizer"] == "ademamix" else 1
        two = hp["optimizer"] in ("adam", "adamw", "ademamix")
        s1, a1 = np.zeros(k1 * n, np.uint8), np.zeros(k1 * nb, np.float32)
        s2 = np.zeros(n, np.uint8) if two else None
        a2 = np.zeros(nb, np.float32) if two else None
        q1, q2 = oracle.dynamic_map(True), oracle.dynamic_map(False)
        t0 = time.perf_counter()
        oracle.step_8bit(hp, 1, p, g, t.dtype, s1, a1, q1, s2, a2, q2 if two else None)
        return n, time.perf_counter() - t0

    n, dt = run(max(1, 65536 // B))                     # calibration: 64K elements
    want = int(n * target_s / max(dt, 1e-6))
    n, dt = run(max(1, min(n_all, want) // B))
    return {"value": n / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} elements ({(n + B - 1) // B} blocks of {B}) of the same workload, "
                      f"1 step, {dt:.1f} s on {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="adamw_fp32_b256")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the optimizer step is per-rank local (blocks are independent), "
              "and this build has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    wl = workload_by_name(args.workload)
    t = wl.tensors[0]
    hp = dict(wl.hp)
    n = t.numel
    B = hp["blocksize"]
    ns = {"adam": 2, "adamw": 2, "ademamix": 3, "momentum": 1, "lion": 1}[hp["optimizer"]]
    bpe = W.bytes_per_element(t.dtype, ns, B)
    q1 = bitopt.create_dynamic_map(True).to(dev)
    q2 = bitopt.create_dynamic_map(False).to(dev)
    reps = [Replica(wl, r, dev) for r in range(args.replicas)]
    torch.cuda.synchronize()

    step_no = 0
    for i in range(args.warmup):
        step_no += 1
        reps[i % len(reps)].step(hp, step_no, q1, q2)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(args.steps):
        step_no += 1
        reps[k % len(reps)].step(hp, step_no, q1, q2)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)])   # ms
    total_ms = ev[0].elapsed_time(ev[-1])
    avg_ms = total_ms / args.steps
    value = n * args.steps / (total_ms / 1e3) / 1e9
    achieved = bpe * n / (avg_ms / 1e3) / 1e9

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gelem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(avg_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "optimizer": hp["optimizer"], "shape": list(t.shape),
                   "param_dtype": t.dtype, "blocksize": B, "weight_decay": hp.get("weight_decay", 0.0),
                   "skip_zeros": bool(hp.get("skip_zeros", False)), "replicas": len(reps)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_elem": bpe, "kernel_ms_median": round(float(np.median(per)), 5),
                     "kernel_ms_p10": round(float(np.percentile(per, 10)), 5),
                     "kernel_ms_p90": round(float(np.percentile(per, 90)), 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
