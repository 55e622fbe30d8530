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
import csv
import glob
import hashlib
import json
import os
import subprocess
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
        "rmsprop_fp32_b256": lambda: W.f2_one_state_4096("rmsprop", "f32"),
        "rmsprop_bf16_b256": lambda: W.f2_one_state_4096("rmsprop", "bf16"),
        "adagrad_fp32_b256": lambda: W.f2_one_state_4096("adagrad", "f32"),
        "adagrad_bf16_b256": lambda: W.f2_one_state_4096("adagrad", "bf16"),
        "adamw_fp32_tensorwise": lambda: W.f3_tensorwise_4096("f32"),
        "adamw_bf16_tensorwise": lambda: W.f3_tensorwise_4096("bf16"),
        "adamw_fp32_b256_paged": lambda: W.f4_paged_4096("f32"),
        "adamw_fp32_b256_staged": lambda: W.f4_staged_4096("f32"),
        "adamw_fp32_b256_pooled": lambda: W.f4_pooled_4096("f32", 1 << 24, 2),
        "adamw_fp32_b256_pooled_thrash": lambda: W.f4_pooled_4096("f32", 1 << 22, 3),
        "adam_fp32_256x256": W.c1_adam_256,
        "adam_fp32_1024x9": W.adam_small_1024x9,
        "adamw32_fp32_4096": lambda: W.adamw_32bit_4096("f32"),
        "adamw32_bf16_4096": lambda: W.adamw_32bit_4096("bf16"),
        "gpt_1p3b": W.c5_gpt_1p3b,
        "quantize_fp32_b256": lambda: W.codec_4096("quantize", "f32"),
        "dequantize_fp32_b256": lambda: W.codec_4096("dequantize", "f32"),
        "quantize_bf16_b256": lambda: W.codec_4096("quantize", "bf16"),
    }
    return table[name]()


NUM_STATES = {"adam": 2, "adamw": 2, "ademamix": 3, "momentum": 1, "lion": 1, "rmsprop": 1, "adagrad": 1}


def tensorwise_bytes_per_element(dtype: str, optimizer: str, max_unorm: float = 0.0) -> float:
    """The two-pass tensor-wide step: pass 1 reads g, the codes and (when the state
    update uses it, or with max_unorm) p; pass 2 reads and writes like the block-wise
    step."""
    ps = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    ns = NUM_STATES[optimizer]
    needs_p = optimizer in ("momentum", "rmsprop", "adagrad") or max_unorm > 0.0
    return (3 * ps + 2 * ns) + (ps + ns + (ps if needs_p else 0))


def workload_bytes(wl) -> float:
    """Algorithmic HBM bytes of one step over every tensor of the workload (the codec
    workloads: values read or written once, codes written or read once, one absmax per
    block)."""
    if wl.extra.get("codec"):
        t = wl.tensors[0]
        ps = {"f32": 4, "f16": 2, "bf16": 2}[t.dtype]
        return (ps + 1 + 4.0 / wl.hp["blocksize"]) * t.numel
    ns = NUM_STATES[wl.hp["optimizer"]]
    total = 0.0
    for t in wl.tensors:
        if t.eightbit and wl.hp["blocksize"] == 0:
            total += tensorwise_bytes_per_element(t.dtype, wl.hp["optimizer"], wl.hp.get("max_unorm", 0.0)) * t.numel
        elif t.eightbit:
            total += W.bytes_per_element(t.dtype, ns, wl.hp["blocksize"]) * t.numel
        else:   # 32-bit states: read+write p, read g, read+write each fp32 state
            ps = {"f32": 4, "f16": 2, "bf16": 2}[t.dtype]
            total += (3 * ps + ns * 8) * t.numel
    return total


def replica_grad(wl, r):
    """The fp32 gradient of replica r of a single-tensor workload (rows zeroed for the
    skip_zeros workloads)."""
    t = wl.tensors[0]
    g = W.normal_f32([wl.seed, 2, 0, r], t.numel, wl.g_scale)
    if wl.zero_row_frac:
        rows = t.shape[0]
        mask = W.zero_row_mask([wl.seed, 3, 0, r], rows, wl.zero_row_frac)
        g.reshape(rows, -1)[mask] = 0.0
    return g


def skip_aware_bytes(wl, g_dev, full_bytes):
    """With skip_zeros, a block whose gradients are all zero needs only its gradient
    read: the algorithmic bytes of a step over gradient g."""
    t = wl.tensors[0]
    n, B = t.numel, wl.hp["blocksize"]
    nbk = (n + B - 1) // B
    pad = torch.zeros(nbk * B, device=g_dev.device)
    pad[:n] = g_dev.float().abs()
    live = int((pad.view(nbk, B).amax(1) > 0).sum().item())
    gsz = {"f32": 4, "f16": 2, "bf16": 2}[t.dtype]
    return full_bytes * live / nbk + gsz * B * (nbk - live)


class Model:
    """Device buffers of every tensor of a multi-tensor workload: one plan built up
    front, each step one bitopt_step_multi_planned call (one launch per tensor kind)."""

    def __init__(self, wl, dev):
        import ctypes
        hp = wl.hp
        B = hp["blocksize"]
        two = hp["optimizer"] in ("adam", "adamw", "ademamix")
        k1 = 2 if hp["optimizer"] == "ademamix" else 1
        self.bufs = []
        arr = (bitopt.Tensor * len(wl.tensors))()
        for i, t in enumerate(wl.tensors):
            n = t.numel
            nb = (n + B - 1) // B
            dt = TORCH_DT[t.dtype]
            p = torch.from_numpy(W.normal_f32([wl.seed, 1, i], n, wl.p_scale)).to(dev).to(dt)
            g = torch.from_numpy(W.normal_f32([wl.seed, 2, i, 1], n, wl.g_scale)).to(dev).to(dt)
            sd = torch.uint8 if t.eightbit else torch.float32
            s1 = torch.zeros(k1 * n, dtype=sd, device=dev)
            s2 = torch.zeros(n, dtype=sd, device=dev) if two else None
            a1 = torch.zeros(k1 * nb, device=dev) if t.eightbit else None
            a2 = torch.zeros(nb, device=dev) if (t.eightbit and two) else None
            self.bufs.append((p, g, s1, s2, a1, a2))
            ptr = lambda x: None if x is None else x.data_ptr()
            arr[i] = bitopt.Tensor(p.data_ptr(), g.data_ptr(), s1.data_ptr(), ptr(s2), ptr(a1), ptr(a2), n,
                                   bitopt.DTYPES[dt], 1 if t.eightbit else 0)
        self.arr = arr
        self.count = len(wl.tensors)
        self.ws = torch.empty(bitopt.multi_workspace_bytes(self.count), dtype=torch.uint8, device=dev)
        self.n = sum(t.numel for t in wl.tensors)
        # the descriptor table is written once (bitopt_multi_plan_build); each step is
        # then kernel launches only (bitopt_step_multi_planned)
        self.plan = bitopt.MultiPlanC()
        h = bitopt.make_hparams(hp)
        rc = bitopt.lib().bitopt_multi_plan_build(ctypes.byref(h), arr, self.count, ctypes.c_void_p(self.ws.data_ptr()),
                                                  self.ws.numel(), ctypes.byref(self.plan),
                                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise bitopt.BitoptError(rc, bitopt.last_error())
        self.launches_per_step = self.plan.nlaunch

    def launcher(self, hp, q1, q2):
        import ctypes
        L = bitopt.lib()
        h = bitopt.make_hparams(hp)
        self._keep = h
        f = L.bitopt_step_multi_planned
        plan = ctypes.byref(self.plan)
        args = (ctypes.c_void_p(q1.data_ptr()), ctypes.c_void_p(q2.data_ptr()),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

        def launch(t):
            rc = f(plan, ctypes.byref(h), t, *args)
            if rc != 0:
                raise bitopt.BitoptError(rc, bitopt.last_error())
        return launch


class CodecReplica:
    """Device buffers of one copy of a codec workload: values, codes, absmax."""

    def __init__(self, wl, r, dev):
        t = wl.tensors[0]
        self.kind = wl.extra["codec"]
        self.n = n = t.numel
        self.B = B = wl.hp["blocksize"]
        dt = TORCH_DT[t.dtype]
        self.x = torch.from_numpy(W.normal_f32([wl.seed, 1, 0, r], n, wl.g_scale)).to(dev).to(dt)
        self.q = bitopt.create_dynamic_map(True).to(dev)
        self.codes, self.absmax = bitopt.quantize_blockwise(self.x, self.q, B)
        self.out = torch.empty_like(self.x)
        self.p = self.x
        self.eightbit = True

    def step(self, hp, t, q1, q2):
        if self.kind == "quantize":
            bitopt.quantize_blockwise(self.x, self.q, self.B, codes=self.codes, absmax=self.absmax)
        else:
            bitopt.dequantize_blockwise(self.codes, self.absmax, self.q, self.B, out=self.out)

    def raw_launcher(self, hp, q1, q2):
        import ctypes
        L = bitopt.lib()
        ptr = lambda x: ctypes.c_void_p(x.data_ptr())
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        dt = bitopt.DTYPES[self.x.dtype]
        if self.kind == "quantize":
            f, args = L.bitopt_quantize_blockwise, (ptr(self.x), dt, self.n, ptr(self.q), self.B, ptr(self.codes),
                                                    ptr(self.absmax), stream)
        else:
            f, args = L.bitopt_dequantize_blockwise, (ptr(self.codes), ptr(self.absmax), ptr(self.q), self.n, self.B,
                                                      ptr(self.out), dt, stream)

        def launch(t):
            rc = f(*args)
            if rc != 0:
                raise bitopt.BitoptError(rc, bitopt.last_error())
        return launch


class Replica:
    """Device buffers of one independent copy of the workload's single tensor (8-bit
    states with their absmax, or fp32 states for the 32-bit step)."""

    def __init__(self, wl, r, dev):
        t = wl.tensors[0]
        self.eightbit = t.eightbit
        self.n = n = t.numel
        hp = wl.hp
        B = hp["blocksize"]
        self.tensorwise = B == 0
        nb = 1 if self.tensorwise else (n + B - 1) // B
        dt = TORCH_DT[t.dtype]
        k1 = 2 if hp["optimizer"] == "ademamix" else 1
        self.two = hp["optimizer"] in ("adam", "adamw", "ademamix")
        self.ws = torch.empty(bitopt.tensorwise_workspace_bytes(), dtype=torch.uint8, device=dev)
        p = W.normal_f32([wl.seed, 1, 0, r], n, wl.p_scale)
        g = replica_grad(wl, r)
        self.p = torch.from_numpy(p).to(dev).to(dt)
        self.g = torch.from_numpy(g).to(dev).to(dt)
        self.staged = wl.extra.get("paged") == "staged"
        if self.staged:
            # state paged through device staging buffers around each step
            self.staging = torch.empty(bitopt.paged_staging_bytes(hp, wl.extra["chunk"]), dtype=torch.uint8,
                                       device=dev)
            self.copy_streams = (torch.cuda.Stream(), torch.cuda.Stream())
        self.pool = None
        if wl.extra.get("paged") == "pooled":
            # host-resident state behind an HBM page pool
            self.pool = bitopt.PagePool(hp, wl.extra["page"], nframes=wl.extra["frames"], device=dev)
        if wl.extra.get("paged"):
            # optimizer state in pinned host memory mapped into the GPU address space
            def z(numel, dt):
                t_ = bitopt.host_state(numel, dt)
                t_.zero_()
                return t_
        else:
            def z(numel, dt):
                return torch.zeros(numel, dtype=dt, device=dev)
        sd = torch.uint8 if self.eightbit else torch.float32
        self.s1 = z(k1 * n, sd)
        self.s2 = z(n, sd) if self.two else None
        self.a1 = z(k1 * nb, torch.float32) if self.eightbit else None
        self.a2 = z(nb, torch.float32) if (self.two and self.eightbit) else None

    def step(self, hp, t, q1, q2):
        if self.pool is not None:
            self.pool.step(hp, t, self.p, self.g, self.s1, self.a1, q1, self.s2, self.a2, q2 if self.two else None)
            return
        if self.staged:
            bitopt.step_8bit_paged(hp, t, self.p, self.g, self.s1, self.a1, q1, self.s2, self.a2,
                                   q2 if self.two else None, staging=self.staging, h2d_stream=self.copy_streams[0],
                                   d2h_stream=self.copy_streams[1])
            return
        if not self.eightbit:
            if self.two:
                bitopt.step_32bit_2state(hp, t, self.p, self.g, self.s1, self.s2)
            else:
                bitopt.step_32bit_1state(hp, t, self.p, self.g, self.s1)
        elif self.tensorwise:
            bitopt.step_8bit_tensorwise(hp, t, self.p, self.g, self.s1, self.a1, q1, self.s2, self.a2,
                                        q2 if self.two else None, workspace=self.ws)
        elif self.two:
            bitopt.step_8bit_blockwise_2state(hp, t, self.p, self.g, self.s1, self.s2, self.a1, self.a2, q1, q2)
        else:
            bitopt.step_8bit_blockwise_1state(hp, t, self.p, self.g, self.s1, self.a1, q1)

    def raw_launcher(self, hp, q1, q2):
        """The same call with its ctypes arguments built once (the timed loop's host
        cost then stays far below a kernel's duration)."""
        import ctypes
        L = bitopt.lib()
        h = bitopt.make_hparams(hp)
        ptr = lambda x: ctypes.c_void_p(x.data_ptr())
        dt = bitopt.DTYPES[self.p.dtype]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        opt = lambda x: None if x is None else ptr(x)
        head = (ctypes.byref(h), )
        if self.pool is not None:
            f = L.bitopt_step_8bit_pooled
            head = (self.pool.handle, ctypes.byref(h))
            tail = (ptr(self.s1), opt(self.s2), ptr(self.a1), opt(self.a2), ptr(q1), ptr(q2) if self.two else None,
                    stream)
        elif self.staged:
            f = L.bitopt_step_8bit_paged
            tail = (ptr(self.s1), opt(self.s2), ptr(self.a1), opt(self.a2), ptr(q1), ptr(q2) if self.two else None,
                    ptr(self.staging), self.staging.numel(), ctypes.c_void_p(self.copy_streams[0].cuda_stream),
                    ctypes.c_void_p(self.copy_streams[1].cuda_stream), stream)
        elif not self.eightbit:
            f = L.bitopt_step_32bit_2state if self.two else L.bitopt_step_32bit_1state
            tail = (ptr(self.s1), ptr(self.s2), stream) if self.two else (ptr(self.s1), stream)
        elif self.tensorwise:
            f = L.bitopt_step_8bit_tensorwise
            tail = (ptr(self.s1), opt(self.s2), ptr(self.a1), opt(self.a2), ptr(q1),
                    ptr(q2) if self.two else None, ptr(self.ws), stream)
        elif self.two:
            f = L.bitopt_step_8bit_blockwise_2state
            tail = (ptr(self.s1), ptr(self.s2), ptr(self.a1), ptr(self.a2), ptr(q1), ptr(q2), stream)
        else:
            f = L.bitopt_step_8bit_blockwise_1state
            tail = (ptr(self.s1), ptr(self.a1), ptr(q1), stream)
        mid = (ptr(self.p), ptr(self.g), dt, self.n)
        self._keep = h

        def launch(t):
            rc = f(*head, t, *mid, *tail)
            if rc != 0:
                raise bitopt.BitoptError(rc, bitopt.last_error())
        return launch


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, target_s=15.0):
    """The oracle, as it stands, on a bounded sample of the same workload.  A single
    tensor: a prefix of it (whole blocks) when one pass over all of it would exceed
    the target time, else repeated full steps until about target_s seconds.  A
    multi-tensor workload: every small (32-bit) tensor in full plus a prefix of each
    8-bit tensor, in the workload's proportions of 8-bit and 32-bit elements."""
    import oracle
    if len(wl.tensors) > 1:
        return cpu_baseline_multi(wl, target_s)
    t = wl.tensors[0]
    hp = wl.hp
    B = hp["blocksize"]
    n_all = t.numel
    threads = oracle.get_threads()
    k1 = 2 if hp["optimizer"] == "ademamix" else 1
    two = hp["optimizer"] in ("adam", "adamw", "ademamix")
    q1, q2 = oracle.dynamic_map(True), oracle.dynamic_map(False)

    def run(n, steps):
        p = W.to_dtype(W.normal_f32([wl.seed, 1, 0, 0], n_all, wl.p_scale, 0, n), t.dtype)
        g = W.to_dtype(W.normal_f32([wl.seed, 2, 0, 0], n_all, wl.g_scale, 0, n), t.dtype)
        nb = 1 if B == 0 else (n + B - 1) // B
        if not t.eightbit:                             # the 32-bit step: fp32 states, no codec
            m1 = np.zeros(k1 * n, np.float32)
            m2 = np.zeros(n, np.float32) if two else None
            t0 = time.perf_counter()
            for step in range(1, steps + 1):
                oracle.step_32bit(hp, step, p, g, t.dtype, m1, m2)
            return time.perf_counter() - t0
        s1, a1 = np.zeros(k1 * n, np.uint8), np.zeros(k1 * nb, np.float32)
        s2 = np.zeros(n, np.uint8) if two else None
        a2 = np.zeros(nb, np.float32) if two else None
        t0 = time.perf_counter()
        for step in range(1, steps + 1):
            oracle.step_8bit(hp, step, p, g, t.dtype, s1, a1, q1, s2, a2, q2 if two else None)
        return time.perf_counter() - t0

    if B == 0:                                         # tensor-wide: one block, the whole tensor
        n, steps = n_all, 1
    else:
        n0 = min(n_all, 256 * B)
        dt0 = run(n0, 1)                               # calibration
        per_elem = dt0 / n0
        if per_elem * n_all <= target_s:
            n, steps = n_all, max(1, int(target_s / (per_elem * n_all)))
        else:
            n, steps = max(B, int(target_s / per_elem) // B * B), 1
    dt = run(n, steps)
    what = "the whole tensor" if n == n_all else f"the first {n} elements ({n // B} blocks of {B})"
    return {"value": n * steps / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{what} of the same workload, {steps} step(s), {dt:.1f} s on {threads} threads"}


def cpu_baseline_codec(wl, target_s=15.0):
    """The oracle's codec on the same values: repeated whole-tensor passes for about
    target_s seconds."""
    import oracle
    t = wl.tensors[0]
    B = wl.hp["blocksize"]
    x = W.to_dtype(W.normal_f32([wl.seed, 1, 0, 0], t.numel, wl.g_scale), t.dtype)
    q = oracle.dynamic_map(True)
    codes, absmax = oracle.quantize_blockwise(x, t.dtype, q, B)
    run = (lambda: oracle.quantize_blockwise(x, t.dtype, q, B)) if wl.extra["codec"] == "quantize" else \
        (lambda: oracle.dequantize_blockwise(codes, absmax, q, B, t.dtype))
    t0 = time.perf_counter()
    run()
    one = time.perf_counter() - t0
    reps = max(1, int(target_s / max(one, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    dt = time.perf_counter() - t0
    threads = oracle.get_threads()
    return {"value": t.numel * reps / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the whole tensor, {reps} pass(es), {dt:.1f} s on {threads} threads "
                      f"({'OpenMP over blocks' if wl.extra['codec'] == 'quantize' else 'one thread: a plain loop'})"}


def cpu_baseline_multi(wl, target_s=15.0):
    import oracle
    hp = wl.hp
    B = hp["blocksize"]
    threads = oracle.get_threads()
    two = hp["optimizer"] in ("adam", "adamw", "ademamix")
    k1 = 2 if hp["optimizer"] == "ademamix" else 1
    q1, q2 = oracle.dynamic_map(True), oracle.dynamic_map(False)
    big = [(i, t) for i, t in enumerate(wl.tensors) if t.eightbit]
    small = [(i, t) for i, t in enumerate(wl.tensors) if not t.eightbit]

    def run(per_tensor_blocks):
        total, secs = 0, 0.0
        for i, t in big:
            n = min(t.numel, per_tensor_blocks * B)
            p = W.to_dtype(W.normal_f32([wl.seed, 1, i], t.numel, wl.p_scale, 0, n), t.dtype)
            g = W.to_dtype(W.normal_f32([wl.seed, 2, i, 1], t.numel, wl.g_scale, 0, n), t.dtype)
            nb = (n + B - 1) // B
            s1, a1 = np.zeros(k1 * n, np.uint8), np.zeros(k1 * nb, np.float32)
            s2 = np.zeros(n, np.uint8) if two else None
            a2 = np.zeros(nb, np.float32) if two else None
            t0 = time.perf_counter()
            oracle.step_8bit(hp, 1, p, g, t.dtype, s1, a1, q1, s2, a2, q2 if two else None)
            secs += time.perf_counter() - t0
            total += n
        for i, t in small:
            n = t.numel
            p = W.to_dtype(W.normal_f32([wl.seed, 1, i], n, wl.p_scale), t.dtype)
            g = W.to_dtype(W.normal_f32([wl.seed, 2, i, 1], n, wl.g_scale), t.dtype)
            m1 = np.zeros(k1 * n, np.float32)
            m2 = np.zeros(n, np.float32) if two else None
            t0 = time.perf_counter()
            oracle.step_32bit(hp, 1, p, g, t.dtype, m1, m2)
            secs += time.perf_counter() - t0
            total += n
        return total, secs

    n0, dt0 = run(16)                                  # calibration
    blocks = max(16, int(16 * target_s / max(dt0, 1e-6)))
    n, dt = run(blocks)
    return {"value": n / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"one step over {len(big)} 8-bit tensors (the first {blocks} blocks of {B} of each) and the "
                      f"{len(small)} 32-bit tensors in full ({n} elements), {dt:.1f} s on {threads} threads"}


def source_hash() -> str:
    """Hash of the HIP library's sources: HBM traffic counted by the profiler is
    reported only while the kernels are unchanged since the counters were taken."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_optimizers_block_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the step kernel from the committed counter summary,
    or None if there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


COPY_ELEMS = 64 << 20          # calibration copy: 64 Mi fp32 = 256 MiB read + 256 MiB written


def copy_calibration(dev):
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def _rocprof(args, outdir, extra, env=None, result=None):
    """Run the benchmark under rocprofv3; its JSON line goes to result["bench"] when
    a dict is given."""
    cmd = ["rocprofv3", *extra, "--output-format", "csv", "-d", outdir, "-o", "run", "--",
           sys.executable, os.path.abspath(__file__), *args]
    print("+ " + " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=env, timeout=300, stdout=subprocess.PIPE, text=True)
    sys.stdout.write(r.stdout)
    sys.stdout.flush()
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 failed ({r.returncode}): {' '.join(cmd)}")
    if result is not None:
        for line in reversed(r.stdout.strip().splitlines()):
            if line.startswith("{"):
                result["bench"] = json.loads(line)
                break
    # as recorded: the repository root as <repo>, the interpreter as python
    shown = ["python" if c == sys.executable else c.replace(ROOT, "<repo>") for c in cmd]
    return " ".join(shown)


def _csv_rows(outdir, suffix):
    rows = []
    for f in glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def kernel_is_8bit(kname: str) -> bool:
    """Whether a step kernel's name (k_step<dtype, optimizer, blocksize, 8-bit, ...>)
    is the 8-bit instantiation."""
    args = kname[kname.index("<") + 1:kname.index(">")].split(",")
    return args[3].strip() == "true"


def profile(workload: str, outdir: str, steps: int, counter_groups=(), counter_warmup: int = 3):
    """Kernel trace plus FETCH_SIZE and WRITE_SIZE passes (each its own run) of the
    benchmark, and one more run per group of extra counters (e.g. SQ_INSTS_VALU);
    writes <workload>.md and .json into outdir (the summaries kept under profiles/
    are these files)."""
    env = dict(os.environ, TMPDIR="/tmp")
    outdir = os.path.abspath(outdir)
    # The trace pass is the benchmark's own command (its default warm-up and timed
    # launches), so the trace's average duration is taken over the same launches the
    # benchmark times; the counter passes count bytes, which do not depend on clocks,
    # over `steps` launches.
    cmds = {}
    traced = {}
    cmds["trace"] = _rocprof(["--workload", workload, "--no-cpu-baseline"], os.path.join(outdir, "trace"),
                             ["--kernel-trace", "--stats"], env, traced)
    tb = traced.get("bench") or {}
    base = ["--workload", workload, "--steps", str(steps), "--warmup", "3", "--no-cpu-baseline", "--copy-calibration"]
    cmds["fetch"] = _rocprof(base, os.path.join(outdir, "fetch"), ["--pmc", "FETCH_SIZE"], env)
    cmds["write"] = _rocprof(base, os.path.join(outdir, "write"), ["--pmc", "WRITE_SIZE"], env)
    # extra counter passes warm up like the timed run when asked to (instruction counts
    # depend on the step: early steps take the exact 16-bit parameter path more often)
    base_nc = ["--workload", workload, "--steps", str(steps), "--warmup", str(counter_warmup), "--no-cpu-baseline"]
    for gi, group in enumerate(counter_groups):
        cmds[f"counters{gi}"] = _rocprof(base_nc, os.path.join(outdir, f"counters{gi}"), ["--pmc", *group], env)
    run = {"workload": workload, "source_hash": source_hash(), "commands": cmds, "traced_bench": tb,
           "steps": steps, "counter_groups": [list(g) for g in counter_groups], "counter_warmup": counter_warmup}
    with open(os.path.join(outdir, "run.json"), "w") as f:
        json.dump(run, f, indent=1)
    summarize_profile(workload, outdir)


# FETCH_SIZE and WRITE_SIZE per KiB copied, as the 256 MiB calibration copy reads them
# in the profiled runs (FETCH_SIZE counts half of the bytes read on this part).
NOMINAL_SCALE = (2.0, 1.0)


def summarize_profile(workload: str, outdir: str):
    """The <workload>.md / .json summaries from the raw output of profile() in outdir
    (its run.json records the commands, the traced run's benchmark line and the
    library source hash at the time of the run)."""
    outdir = os.path.abspath(outdir)
    with open(os.path.join(outdir, "run.json")) as f:
        run = json.load(f)
    cmds, tb, steps = run["commands"], run["traced_bench"] or {}, run["steps"]
    counter_groups, counter_warmup = run["counter_groups"], run["counter_warmup"]
    stats = [r for r in _csv_rows(os.path.join(outdir, "trace"), "kernel_stats.csv")]
    # the dominant library kernel (a multi-tensor step launches one kernel per tensor kind)
    step_stats = sorted((r for r in stats if "bitopt::" in r["Name"]), key=lambda r: -float(r["TotalDurationNs"]))
    kname = step_stats[0]["Name"]
    avg_ns = float(step_stats[0]["AverageNs"])
    calls = int(step_stats[0]["Calls"])
    # the same kernel over the traced run's timed launches only (its last ones), the
    # figure comparable with that run's time per step
    trace = [r for r in _csv_rows(os.path.join(outdir, "trace"), "kernel_trace.csv") if r["Kernel_Name"] == kname]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace]
    t_steps, t_warm = int(tb.get("steps") or 0), int(tb.get("warmup") or 0)
    per_step = max(1, round(len(dur) / (t_steps + t_warm))) if t_steps + t_warm else 1
    timed = dur[-per_step * t_steps:] if t_steps and dur else dur
    timed_ns = sum(timed) / len(timed) if timed else avg_ns

    def counter(name, sub):
        rows = [r for r in _csv_rows(os.path.join(outdir, sub), "counter_collection.csv") if r["Counter_Name"] == name]
        step = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == kname]
        if not step:      # names spelled differently in the two outputs: any library kernel
            step = [float(r["Counter_Value"]) for r in rows if "bitopt::" in r["Kernel_Name"]]
        # the calibration copy is the runtime's device-to-device blit kernel, by far the
        # largest blit of the run (paged workloads' host copies may use blit kernels too)
        blits = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        vmax = max(blits)
        copy = [v for v in blits if v >= 0.5 * vmax]
        return step, copy

    fs, fc = counter("FETCH_SIZE", "fetch")
    ws, wc = counter("WRITE_SIZE", "write")
    # the timed launches are the last `steps` step-kernel dispatches of each run
    fs, ws = fs[-steps:], ws[-steps:]
    copy_kib = COPY_ELEMS * 4 / 1024.0
    f_scale = copy_kib / (sum(fc) / len(fc))
    w_scale = copy_kib / (sum(wc) / len(wc))
    fetch_b = sum(fs) / len(fs) * f_scale * 1024.0
    write_b = sum(ws) / len(ws) * w_scale * 1024.0
    wl = workload_by_name(workload)
    if len(wl.tensors) > 1 and "k_step" in kname:
        # only the tensors of the dominant kernel's kind (8-bit or 32-bit states)
        quant = kernel_is_8bit(kname)
        wl = W.Workload(**{**wl.__dict__, "tensors": [t for t in wl.tensors if t.eightbit == quant]})
    alg = workload_bytes(wl)
    if wl.hp.get("skip_zeros"):
        # block liveness: the zeroed rows (no N(0, 1e-2) sample rounds to zero in 16 bits)
        alg = skip_aware_bytes(wl, torch.from_numpy(replica_grad(wl, 0)), alg)
    kelems = sum(t.numel for t in wl.tensors)
    unit = wl.extra.get("chunk") or wl.extra.get("page")
    if unit and unit < kelems:
        # staged or pooled state: one launch per chunk or page (4096x4096 splits evenly)
        alg = alg * unit / kelems
        kelems = unit
    extra = {}
    for gi, group in enumerate(counter_groups):
        rows = _csv_rows(os.path.join(outdir, f"counters{gi}"), "counter_collection.csv")
        for name in group:
            per = {}
            for r in rows:
                if r["Counter_Name"] != name or "bitopt::" not in r["Kernel_Name"]:
                    continue
                if r["Kernel_Name"] != kname and any(x["Kernel_Name"] == kname for x in rows):
                    continue
                key = r.get("Dispatch_Id", str(len(per)))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            vals = [per[k] for k in sorted(per, key=lambda k: int(k) if k.isdigit() else 0)][-steps:]
            if vals:
                extra[name] = sum(vals) / len(vals)
    d = {"workload": workload, "kernel": kname, "source_hash": run["source_hash"],
         "kernel_trace_calls": calls, "kernel_trace_avg_us": avg_ns / 1e3,
         "kernel_timed_launches": len(timed), "kernel_timed_avg_us": timed_ns / 1e3,
         "kernel_launches_per_step": per_step,
         "fetch_kib_per_launch": sum(fs) / len(fs), "write_kib_per_launch": sum(ws) / len(ws),
         "copy_calibration": {"bytes_each_way": COPY_ELEMS * 4, "fetch_kib": sum(fc) / len(fc),
                              "write_kib": sum(wc) / len(wc), "fetch_scale": f_scale, "write_scale": w_scale},
         "traffic_bytes_per_launch": fetch_b + write_b, "algorithmic_bytes_per_launch": alg,
         "kernel_elements": kelems, "counters_per_launch": extra,
         "traced_run": {"ms_per_step": tb.get("ms_per_step"), "value": tb.get("value"), "unit": tb.get("unit"),
                        "frac": (tb.get("roofline") or {}).get("frac"), "steps": tb.get("steps")},
         "commands": cmds}
    with open(os.path.join(outdir, f"{workload}.json"), "w") as f:
        json.dump(d, f, indent=1)
    with open(os.path.join(outdir, f"{workload}.md"), "w") as f:
        f.write(f"# {workload}: rocprofv3 summary\n\n")
        f.write(f"Kernel: `{kname}`\n\n")
        f.write("| figure | value |\n|---|---|\n")
        f.write(f"| kernel-trace calls | {calls} |\n")
        f.write(f"| kernel-trace average duration, all calls (warm-up included) | {avg_ns / 1e3:.2f} us |\n")
        f.write(f"| kernel-trace average duration, the traced run's {len(timed)} timed launches "
                f"({per_step} per step) | {timed_ns / 1e3:.2f} us |\n")
        if tb:
            f.write(f"| the traced run's own benchmark line: time per step (launch to launch) | "
                    f"{tb['ms_per_step'] * 1e3:.2f} us ({tb['value']} {tb['unit']}, {tb['roofline']['frac']} of peak) |\n")
        f.write(f"| algorithmic bytes per launch | {alg / 1e6:.1f} MB |\n")
        f.write(f"| algorithmic GB/s at the timed-launch average | {alg / timed_ns:.0f} "
                f"({alg / timed_ns / HBM_PEAK_GBS:.4f} of the 8000 GB/s peak) |\n")
        f.write(f"| FETCH_SIZE per launch (raw) | {sum(fs) / len(fs):.0f} KiB |\n")
        f.write(f"| WRITE_SIZE per launch (raw) | {sum(ws) / len(ws):.0f} KiB |\n")
        f.write(f"| copy calibration (256 MiB each way): FETCH_SIZE / WRITE_SIZE | "
                f"{sum(fc) / len(fc):.0f} / {sum(wc) / len(wc):.0f} KiB -> scale {f_scale:.4f} / {w_scale:.4f} |\n")
        f.write(f"| HBM traffic per launch (scaled) | {(fetch_b + write_b) / 1e6:.1f} MB "
                f"({(fetch_b + write_b) / alg:.3f} x algorithmic) |\n")
        if abs(f_scale / NOMINAL_SCALE[0] - 1.0) > 0.02 or abs(w_scale / NOMINAL_SCALE[1] - 1.0) > 0.02:
            nb_ = (sum(fs) / len(fs) * NOMINAL_SCALE[0] + sum(ws) / len(ws) * NOMINAL_SCALE[1]) * 1024.0
            f.write(f"| the same at the copy factors {NOMINAL_SCALE[0]:.1f} / {NOMINAL_SCALE[1]:.1f} that the "
                    f"other runs measure (this run's copy counts read low) | {nb_ / 1e6:.1f} MB "
                    f"({nb_ / alg:.3f} x algorithmic) |\n")
        f.write(f"| library source hash | {run['source_hash']} |\n\n")
        if extra:
            f.write("| counter | per launch | per element (x64 for per-wave counts) |\n|---|---|---|\n")
            for name, v in extra.items():
                wave = name.startswith("SQ_INSTS") or name in ("SQ_LDS_BANK_CONFLICT", "SQ_WAVES")
                per_el = v * 64 / kelems if wave else v / kelems
                f.write(f"| {name} | {v:.6g} | {per_el:.4g} |\n")
            f.write(f"\nElements updated by the kernel per launch: {kelems}.\n\n")
        pc = (f" --profile-counters '{';'.join(','.join(g) for g in counter_groups)}' --profile-warmup {counter_warmup}"
              if counter_groups else "")
        f.write(f"Made by `python bench.py --profile <outdir> --workload {workload} --profile-steps {steps}{pc}` "
                "(from the repository root), which runs the profiler passes below from /tmp with "
                "TMPDIR=/tmp; raw output stays in the -d directories.  The trace pass is the benchmark's "
                "default command (1000 warm-up and 1000 timed steps); the timed-launch average covers the "
                "kernel's launches in its timed steps, the figure comparable with that run's time per step.  "
                "Counter passes run `--profile-steps` steps after their own warm-up; per-launch counter "
                "figures are averages over those steps.\n\n")
        for k, c in cmds.items():
            f.write(f"- {k}: `{c}`\n")
    print(json.dumps(d))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the GPU reaches its sustained clocks only after tens of ms of back-to-back
    # launches: with 10 warm-up steps the 4096x4096 steps measure 4-7% slower
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="adamw_fp32_b256")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 256 MiB with torch (profiler scale factor)")
    ap.add_argument("--profile", metavar="OUTDIR",
                    help="run the benchmark under rocprofv3 (kernel trace, FETCH_SIZE, WRITE_SIZE); "
                         "raw output and the <workload>.md/.json summaries go to OUTDIR")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--profile-counters", default="",
                    help="extra counter passes for --profile: groups separated by ';', counters by ','")
    ap.add_argument("--profile-warmup", type=int, default=3, help="warm-up launches of the extra counter passes")
    ap.add_argument("--profile-summarize", metavar="OUTDIR",
                    help="only rewrite the summaries from the raw output an earlier --profile left in OUTDIR")
    args = ap.parse_args()
    if args.profile_summarize:
        summarize_profile(args.workload, args.profile_summarize)
        return
    if args.profile:
        groups = [[c for c in g.split(",") if c] for g in args.profile_counters.split(";") if g.strip()]
        profile(args.workload, args.profile, args.profile_steps, groups, args.profile_warmup)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the optimizer step is per-rank local (blocks are independent), "
              "and this library has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    wl = workload_by_name(args.workload)
    hp = dict(wl.hp)
    B = hp["blocksize"]
    multi = len(wl.tensors) > 1
    q1 = bitopt.create_dynamic_map(True).to(dev)
    q2 = bitopt.create_dynamic_map(False).to(dev)
    if multi:
        model = Model(wl, dev)
        n = model.n
        step_bytes = workload_bytes(wl)
        launchers = [model.launcher(hp, q1, q2)]
    else:
        t = wl.tensors[0]
        n = t.numel
        step_bytes = workload_bytes(wl)
        reps = [(CodecReplica if wl.extra.get("codec") else Replica)(wl, r, dev) for r in range(args.replicas)]
        launchers = None
        if hp.get("skip_zeros"):
            step_bytes = skip_aware_bytes(wl, reps[0].g, step_bytes)
    torch.cuda.synchronize()

    step_no = 0
    if multi:
        for i in range(args.warmup):
            step_no += 1
            launchers[0](step_no)
    else:
        for i in range(args.warmup):
            step_no += 1
            reps[i % len(reps)].step(hp, step_no, q1, q2)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    launch = launchers if multi else [r.raw_launcher(hp, q1, q2) for r in reps]
    # timed region: K back-to-back launches between two events on the launch stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    for k in range(args.steps):
        step_no += 1
        launch[k % len(launch)](step_no)
    host_us = (time.perf_counter() - h0) * 1e6 / args.steps
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # distribution of single launches (separate pass, an event pair around each)
    nd = min(args.steps, 50)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nd)]
    for k in range(nd):
        step_no += 1
        ev[2 * k].record(stream)
        launch[k % len(launch)](step_no)
        ev[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(dev)
    per = np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(nd)])   # ms
    avg_ms = total_ms / args.steps
    value = n * args.steps / (total_ms / 1e3) / 1e9
    achieved = step_bytes / (avg_ms / 1e3) / 1e9

    # the parameter dtype of the workload (element arithmetic is fp32, states are u8 codes)
    dtype = "+".join(sorted({t.dtype for t in wl.tensors}, key=lambda d: -sum(
        x.numel for x in wl.tensors if x.dtype == d)))
    if multi:
        cfg = {"workload": wl.name, "optimizer": hp["optimizer"], "tensors": len(wl.tensors),
               "params": n, "eightbit_params": sum(t.numel for t in wl.tensors if t.eightbit),
               "param_dtype": "bf16 (8-bit states), f32 (32-bit states)", "blocksize": B,
               "launches_per_step": model.launches_per_step, "arithmetic": "f32", "state_dtype": "u8"}
    else:
        cfg = {"workload": wl.name, "optimizer": hp["optimizer"], "shape": list(t.shape),
               "param_dtype": t.dtype, "blocksize": B, "weight_decay": hp.get("weight_decay", 0.0),
               "skip_zeros": bool(hp.get("skip_zeros", False)), "replicas": len(reps),
               "arithmetic": "f32", "state_dtype": "u8" if t.eightbit else "f32"}
        if wl.extra.get("paged") == "pooled":
            cfg["state_memory"] = (f"pinned host, cached in an HBM page pool of {wl.extra['frames']} frames of "
                                   f"{wl.extra['page']} elements")
        elif wl.extra.get("paged") == "staged":
            cfg["state_memory"] = f"pinned host, paged through HBM staging in chunks of {wl.extra['chunk']} elements"
        elif wl.extra.get("paged"):
            cfg["state_memory"] = "pinned host, read and written in place over the host link"
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gelem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(avg_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(args.workload),
                     "algorithmic_bytes_per_step": step_bytes,
                     "kernel_ms_median": round(float(np.median(per)), 5),
                     "kernel_ms_p10": round(float(np.percentile(per, 10)), 5),
                     "kernel_ms_p90": round(float(np.percentile(per, 90)), 5),
                     "host_us_per_launch": round(host_us, 2)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_codec if wl.extra.get("codec") else cpu_baseline)(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
