"""GPU: the per-tensor and tensor-wide steps captured into a HIP graph (through
torch.cuda.graph) and replayed several times -- with eager work and synchronisation
between the replays -- give, replay after replay, exactly the result of the same
calls made eagerly.  The steps enqueue kernels only (no memset or copy nodes)."""
import numpy as np
import pytest
import torch

from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _state(n, nb, two, k=1):
    return dict(s1=torch.zeros(k * n, dtype=torch.uint8, device="cuda"), a1=torch.zeros(k * nb, device="cuda"),
                s2=torch.zeros(n, dtype=torch.uint8, device="cuda") if two else None,
                a2=torch.zeros(nb, device="cuda") if two else None)


def _compare(a, b, what):
    for key in a:
        if a[key] is not None:
            np.testing.assert_array_equal(to_host(a[key]), to_host(b[key]), err_msg=f"{what} {key}")


@pytest.mark.parametrize("mode", ["blockwise", "tensorwise"])
def test_captured_step_replays_like_eager(mode):
    n = 3 * 4096 + 77
    bs = 0 if mode == "tensorwise" else 256
    hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=bs)
    nb = 1 if bs == 0 else (n + bs - 1) // bs
    p0 = W.normal_f32([1800, 1], n, 0.02)
    g = to_dev(W.normal_f32([1800, 2], n, 0.01), "f32")
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    A = dict(p=to_dev(p0, "f32"), **_state(n, nb, True))        # stepped by the graph
    B = dict(p=to_dev(p0, "f32"), **_state(n, nb, True))        # stepped eagerly
    ws = {"A": torch.empty(bitopt.tensorwise_workspace_bytes(), dtype=torch.uint8, device="cuda"),
          "B": torch.empty(bitopt.tensorwise_workspace_bytes(), dtype=torch.uint8, device="cuda")}

    def step(S, key):
        if mode == "tensorwise":
            bitopt.step_8bit_tensorwise(hp, 1, S["p"], g, S["s1"], S["a1"], q1, S["s2"], S["a2"], q2,
                                        workspace=ws[key])
        else:
            bitopt.step_8bit_blockwise_2state(hp, 1, S["p"], g, S["s1"], S["s2"], S["a1"], S["a2"], q1, q2)

    # warm the step up on a side stream (as torch.cuda.graph expects), then capture it
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        C = dict(p=to_dev(p0, "f32"), **_state(n, nb, True))
        step(C, "A")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(A, "A")
    torch.cuda.synchronize()
    for r in range(4):
        graph.replay()
        step(B, "B")
        scratch = torch.randn(1 << 20, device="cuda").sum()      # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        _compare(A, B, f"replay {r}")


def test_captured_multi_plan_step_replays_like_eager():
    """The planned multi-tensor step enqueues kernels only, so it can be captured: one
    graph per step number (the per-step scalars are captured with the launch), replayed
    in order t = 1, 2, 3 and again, each replay equal to the eager planned step at the
    same t on a twin set of tensors."""
    hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=256)
    specs = [(5000, "f32", True), (4096, "bf16", True), (3000, "f16", True), (2048, "f32", False), (77, "bf16", False)]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()

    def make():
        ts = []
        for i, (n, dt, eight) in enumerate(specs):
            nb = (n + 255) // 256
            sd = torch.uint8 if eight else torch.float32
            ts.append(dict(p=to_dev(W.to_dtype(W.normal_f32([1900, 1, i], n, 0.02), dt), dt),
                           g=to_dev(W.to_dtype(W.normal_f32([1900, 2, i], n, 0.01), dt), dt),
                           state1=torch.zeros(n, dtype=sd, device="cuda"), state2=torch.zeros(n, dtype=sd, device="cuda"),
                           absmax1=torch.zeros(nb, device="cuda") if eight else None,
                           absmax2=torch.zeros(nb, device="cuda") if eight else None, is_8bit=eight))
        return ts

    A, B = make(), make()
    pa, pb = bitopt.MultiPlan(hp, A), bitopt.MultiPlan(hp, B)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on a scratch copy, as torch.cuda.graph expects
        C = make()
        bitopt.MultiPlan(hp, C).step(hp, 1, q1, q2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for t in (1, 2, 3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pa.step(hp, t, q1, q2)
        graphs[t] = g
    torch.cuda.synchronize()
    for rnd in range(2):
        for t in (1, 2, 3):
            graphs[t].replay()
            pb.step(hp, t, q1, q2)
            scratch = torch.randn(1 << 18, device="cuda").sum()
            torch.cuda.synchronize()
            assert torch.isfinite(scratch)
            for ta, tb in zip(A, B):
                for key in ("p", "state1", "state2", "absmax1", "absmax2"):
                    if ta[key] is not None:
                        np.testing.assert_array_equal(to_host(ta[key]), to_host(tb[key]), err_msg=f"round {rnd} t {t} {key}")


@pytest.mark.parametrize("opt", ["adam", "ademamix"])
def test_captured_device_scalar_step_follows_the_step_number(opt):
    """bitopt_step_multi_planned_dscalars reads the per-step scalars from device memory:
    ONE captured graph, its scalar buffer rewritten before each replay with step t's
    values (bias corrections; AdEMAMix's alpha and beta3 schedules), steps t = 1..5
    exactly as the eager planned step at t = 1..5 on a twin set of tensors."""
    if opt == "adam":
        hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=256)
    else:
        hp = dict(optimizer="ademamix", lr=1e-3, beta3=0.9999, alpha=5.0, t_alpha=4, t_beta3=4, blocksize=256)
    k = 2 if opt == "ademamix" else 1
    specs = [(5000, "f32", True), (4096, "bf16", True), (3008, "f16", True), (2048, "f32", False)]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    print(f"\n[case] device-scalar graph replay {opt}", flush=True)

    def make():
        ts = []
        for i, (n, dt, eight) in enumerate(specs):
            nb = (n + 255) // 256
            sd = torch.uint8 if eight else torch.float32
            ts.append(dict(p=to_dev(W.to_dtype(W.normal_f32([1910, 1, i], n, 0.02), dt), dt),
                           g=to_dev(W.to_dtype(W.normal_f32([1910, 2, i], n, 0.01), dt), dt),
                           state1=torch.zeros(k * n, dtype=sd, device="cuda"),
                           state2=torch.zeros(n, dtype=sd, device="cuda"),
                           absmax1=torch.zeros(k * nb, device="cuda") if eight else None,
                           absmax2=torch.zeros(nb, device="cuda") if eight else None, is_8bit=eight))
        return ts

    A, B = make(), make()
    pa, pb = bitopt.MultiPlan(hp, A), bitopt.MultiPlan(hp, B)
    scal = torch.zeros(bitopt.device_scalars_bytes(), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on a scratch copy, as torch.cuda.graph expects
        C = make()
        scal.copy_(bitopt.device_scalars(hp, 1))
        bitopt.MultiPlan(hp, C).step_dscalars(hp, scal, q1, q2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.step_dscalars(hp, scal, q1, q2)
    torch.cuda.synchronize()
    for t in range(1, 6):
        scal.copy_(bitopt.device_scalars(hp, t))
        g.replay()
        pb.step(hp, t, q1, q2)
        scratch = torch.randn(1 << 18, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for ta, tb in zip(A, B):
            for key in ("p", "state1", "state2", "absmax1", "absmax2"):
                if ta[key] is not None:
                    np.testing.assert_array_equal(to_host(ta[key]), to_host(tb[key]), err_msg=f"t {t} {key}")
