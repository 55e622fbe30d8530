"""GPU: the multi-tensor step (one launch per tensor kind) is bit-identical to the
per-tensor entry points, for every optimizer, over mixed 8-bit / 32-bit tensors of
all dtypes, ragged and unaligned sizes, and empty tensors; and it matches the
oracle on small tensors."""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, as_f32, param_rtol, to_dev, to_host

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
OPTS = {
    "adam": dict(optimizer="adam", lr=1e-3, weight_decay=0.01),
    "ademamix": dict(optimizer="ademamix", lr=1e-3, beta3=0.9999, alpha=5.0, t_alpha=3, t_beta3=3),
    "momentum": dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01),
    "lion": dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01),
    "rmsprop": dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8, weight_decay=0.01),
    "adagrad": dict(optimizer="adagrad", lr=0.01, eps=1e-10, weight_decay=0.01),
}
# (n, dtype, is_8bit)
SPECS = [(5000, "f32", True), (4096, "bf16", True), (70000, "f16", True), (2048, "f32", False),
         (1000, "bf16", False), (0, "f32", True), (3, "f32", True), (8192 + 16, "bf16", True),
         (4095, "f32", False), (40000, "f32", True), (3000, "f16", False), (77, "f16", False)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _make(name, bs, seed):
    hp = OPTS[name]
    two = name in ("adam", "ademamix")
    k = 2 if name == "ademamix" else 1
    ts = []
    for i, (n, dt, eight) in enumerate(SPECS):
        nb = (n + bs - 1) // bs
        p = W.to_dtype(W.normal_f32([seed, 1, i], n, 0.02), dt)
        sd = torch.uint8 if eight else torch.float32
        t = dict(p=to_dev(p, dt) if n else torch.zeros(0, dtype=TDT[dt], device="cuda"),
                 state1=torch.zeros(k * n, dtype=sd, device="cuda"),
                 state2=torch.zeros(n, dtype=sd, device="cuda") if two else None,
                 absmax1=torch.zeros(k * nb, device="cuda") if eight else None,
                 absmax2=torch.zeros(nb, device="cuda") if (eight and two) else None,
                 is_8bit=eight, dt=dt, n=n, p0=p)
        ts.append(t)
    return ts


def _per_tensor(hp, step, t, q1, q2):
    if t["n"] == 0:
        return
    two = hp["optimizer"] in ("adam", "ademamix")
    if t["is_8bit"]:
        if two:
            bitopt.step_8bit_blockwise_2state(hp, step, t["p"], t["g"], t["state1"], t["state2"], t["absmax1"],
                                              t["absmax2"], q1, q2)
        else:
            bitopt.step_8bit_blockwise_1state(hp, step, t["p"], t["g"], t["state1"], t["absmax1"], q1)
    else:
        if two:
            bitopt.step_32bit_2state(hp, step, t["p"], t["g"], t["state1"], t["state2"])
        else:
            bitopt.step_32bit_1state(hp, step, t["p"], t["g"], t["state1"])


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("name", list(OPTS))
def test_multi_equals_per_tensor(name, bs):
    hp = dict(OPTS[name], blocksize=bs)
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    A, Bt = _make(name, bs, 10), _make(name, bs, 10)
    ws = None
    for step in (1, 2, 3):
        for i, (ta, tb) in enumerate(zip(A, Bt)):
            g = W.to_dtype(W.normal_f32([11, 2, i, step], ta["n"], 0.01), ta["dt"])
            gd = to_dev(g, ta["dt"]) if ta["n"] else torch.zeros(0, dtype=TDT[ta["dt"]], device="cuda")
            ta["g"] = gd
            tb["g"] = gd
        ws = bitopt.step_multi(hp, step, A, q1, q2, workspace=ws)
        for tb in Bt:
            _per_tensor(hp, step, tb, q1, q2)
        torch.cuda.synchronize()
        for ta, tb in zip(A, Bt):
            for key in ("p", "state1", "state2", "absmax1", "absmax2"):
                if ta[key] is None:
                    continue
                np.testing.assert_array_equal(to_host(ta[key]), to_host(tb[key]), err_msg=f"{key} n={ta['n']}")


def test_multi_matches_oracle():
    """Small tensors of every kind, adam, 3 steps: multi launch vs the oracle."""
    hp = dict(OPTS["adam"], blocksize=256)
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    T = _make("adam", 256, 20)
    qs, qu = oracle.dynamic_map(True), oracle.dynamic_map(False)
    ref = []
    for t in T:
        n = t["n"]
        nb = (n + 255) // 256
        if t["is_8bit"]:
            ref.append(dict(p=t["p0"].copy(), s1=np.zeros(n, np.uint8), s2=np.zeros(n, np.uint8),
                            a1=np.zeros(nb, np.float32), a2=np.zeros(nb, np.float32)))
        else:
            ref.append(dict(p=t["p0"].copy(), s1=np.zeros(n, np.float32), s2=np.zeros(n, np.float32)))
    cmp = Compare()
    for step in (1, 2, 3):
        gs = []
        for i, t in enumerate(T):
            g = W.to_dtype(W.normal_f32([21, 2, i, step], t["n"], 0.01), t["dt"])
            gs.append(g)
            t["g"] = to_dev(g, t["dt"]) if t["n"] else torch.zeros(0, dtype=TDT[t["dt"]], device="cuda")
        bitopt.step_multi(hp, step, T, q1, q2)
        for t, r, g in zip(T, ref, gs):
            if t["n"] == 0:
                continue
            if t["is_8bit"]:
                oracle.step_8bit(hp, step, r["p"], g, t["dt"], r["s1"], r["a1"], qs, r["s2"], r["a2"], qu)
            else:
                oracle.step_32bit(hp, step, r["p"], g, t["dt"], r["s1"], r["s2"])
        torch.cuda.synchronize()
        for t, r in zip(T, ref):
            if t["n"] == 0:
                continue
            cmp.values(as_f32(to_host(t["p"], t["dt"]), t["dt"]), as_f32(r["p"], t["dt"]), param_rtol(t["dt"]), "p")
            if t["is_8bit"]:
                cmp.codes(to_host(t["state1"]), r["s1"], "s1")
                cmp.codes(to_host(t["state2"]), r["s2"], "s2")
                cmp.values(to_host(t["absmax1"]), r["a1"], param_rtol(t["dt"]), "a1", kind="a")
                cmp.values(to_host(t["absmax2"]), r["a2"], param_rtol(t["dt"]), "a2", kind="a")
            else:
                cmp.values(to_host(t["state1"]), r["s1"], 1e-6, "m", kind="a")
                cmp.values(to_host(t["state2"]), r["s2"], 1e-6, "v", kind="a")
    print("\n[multi vs oracle] " + cmp.summary())


@pytest.mark.parametrize("name", ["adam", "ademamix", "lion"])
def test_multi_plan_steps_equal_per_tensor(name):
    """A plan built once and stepped three times (bitopt_step_multi_planned) gives the
    per-tensor calls' results bit for bit; the plan survives changing gradients (same
    buffers, new contents)."""
    bs = 256
    hp = dict(OPTS[name], blocksize=bs)
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    A, Bt = _make(name, bs, 30), _make(name, bs, 30)
    for ta, tb in zip(A, Bt):
        ta["g"] = torch.zeros(ta["n"], dtype=TDT[ta["dt"]], device="cuda")
        tb["g"] = ta["g"]
    plan = bitopt.MultiPlan(hp, A)
    assert plan.c.count == sum(1 for t in A if t["n"] > 0)
    for step in (1, 2, 3):
        for i, ta in enumerate(A):
            if ta["n"]:
                ta["g"].copy_(to_dev(W.to_dtype(W.normal_f32([31, 2, i, step], ta["n"], 0.01), ta["dt"]), ta["dt"]))
        plan.step(hp, step, q1, q2)
        for tb in Bt:
            _per_tensor(hp, step, tb, q1, q2)
        torch.cuda.synchronize()
        for ta, tb in zip(A, Bt):
            for key in ("p", "state1", "state2", "absmax1", "absmax2"):
                if ta[key] is not None:
                    np.testing.assert_array_equal(to_host(ta[key]), to_host(tb[key]), err_msg=f"{key} n={ta['n']}")
