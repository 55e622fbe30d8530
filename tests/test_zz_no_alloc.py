"""GPU: the allocation-free tensor-wide step (bitopt_step_8bit_tensorwise_noalloc)
gives exactly the results of bitopt_step_8bit_tensorwise with a caller workspace, on
two calls in a row -- the second with a smaller tensor, so the shared scratch array
still holds the first call's partial results -- for a 2-state and a 1-state
optimizer, with and without max_unorm, and over several steps."""
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


def _state(n, two, k=1):
    return dict(s1=torch.zeros(k * n, dtype=torch.uint8, device="cuda"), a1=torch.zeros(k, device="cuda"),
                s2=torch.zeros(n, dtype=torch.uint8, device="cuda") if two else None,
                a2=torch.zeros(1, device="cuda") if two else None)


CASES = [
    ("adam", "f32", dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=0)),
    ("ademamix", "bf16", dict(optimizer="ademamix", lr=1e-3, beta3=0.9999, alpha=5.0, t_alpha=3, t_beta3=3,
                              blocksize=0, max_unorm=0.01)),
    ("momentum", "f16", dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01, blocksize=0,
                             skip_zeros=True)),
]


@pytest.mark.parametrize("name,dtype,hp", CASES, ids=[c[0] for c in CASES])
def test_noalloc_tensorwise_equals_workspace_call(name, dtype, hp):
    assert bitopt.lib().bitopt_tensorwise_scratch_bytes() >= bitopt.tensorwise_workspace_bytes()
    two = name in ("adam", "ademamix")
    k = 2 if name == "ademamix" else 1
    q1, q2 = bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda()
    ws = torch.empty(bitopt.tensorwise_workspace_bytes(), dtype=torch.uint8, device="cuda")
    for call, n in enumerate((1536 * 1024 + 333, 70 * 1024 + 16)):     # second call: smaller
        print(f"\n[case] noalloc {name} {dtype} call {call} n={n}", flush=True)
        p0 = W.to_dtype(W.normal_f32([2000 + call, 1], n, 0.02), dtype)
        A = dict(p=to_dev(p0, dtype), **_state(n, two, k))     # the allocation-free call
        B = dict(p=to_dev(p0, dtype), **_state(n, two, k))     # the call with a workspace
        for t in (1, 2, 3):
            g = W.normal_f32([2000 + call, 2, t], n, 0.01)
            if hp.get("skip_zeros"):
                g[: n // 3] = 0.0
            gd = to_dev(W.to_dtype(g, dtype), dtype)
            bitopt.step_8bit_tensorwise_noalloc(hp, t, A["p"], gd, A["s1"], A["a1"], q1, A["s2"], A["a2"],
                                                q2 if two else None)
            bitopt.step_8bit_tensorwise(hp, t, B["p"], gd, B["s1"], B["a1"], q1, B["s2"], B["a2"],
                                        q2 if two else None, workspace=ws)
            torch.cuda.synchronize()
            for key in A:
                if A[key] is not None:
                    np.testing.assert_array_equal(to_host(A[key]), to_host(B[key]), err_msg=f"call {call} t {t} {key}")
