"""Checkpoint round trip: the whole optimizer state of the 8-bit step is the buffers
the caller owns (codes, absmax, parameters; the step counter is the caller's).
Saving them to bytes and loading them into fresh device buffers gives a next step
bit-identical to the one taken from the original buffers, and both equal the
oracle's step."""
import io

import numpy as np
import pytest
import torch

from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, Quant8, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = [
    (dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, blocksize=256), "bf16"),
    (dict(optimizer="ademamix", lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, t_alpha=10,
          t_beta3=10, eps=1e-8, weight_decay=0.01, blocksize=2048), "f16"),
    (dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01, blocksize=256), "f32"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _grad(seed, t, n, dtype):
    return W.to_dtype(W.normal_f32([seed, 2, t], n, 0.01), dtype)


@pytest.mark.parametrize("hp,dtype", CASES, ids=[c[0]["optimizer"] for c in CASES])
def test_checkpoint_round_trip(hp, dtype):
    n, seed = 3 * 2048 + 77, 2100
    print(f"\n[checkpoint] {hp['optimizer']} {dtype} B={hp['blocksize']} n={n}", flush=True)
    q = Quant8(hp, W.to_dtype(W.normal_f32([seed, 1], n, 0.02), dtype), dtype)
    cmp = Compare()
    for t in (1, 2, 3):
        g = _grad(seed, t, n, dtype)
        q.step_gpu(t, to_dev(g, dtype))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")

    # save every caller-owned buffer, load it into fresh device memory
    torch.cuda.synchronize()
    buf = io.BytesIO()
    torch.save({k: v.cpu() for k, v in q.d.items() if v is not None}, buf)
    buf.seek(0)
    loaded = torch.load(buf, weights_only=True)
    r = Quant8(hp, np.zeros(n, q.o["p"].dtype), dtype)
    r.d = {k: loaded[k].cuda() for k in loaded}
    for k in r.d:
        assert r.d[k].data_ptr() != q.d[k].data_ptr()

    g = _grad(seed, 4, n, dtype)
    q.step_gpu(4, to_dev(g, dtype))
    r.step_gpu(4, to_dev(g, dtype))
    q.step_oracle(4, g)
    torch.cuda.synchronize()
    for k in q.d:
        if q.d[k] is not None:
            np.testing.assert_array_equal(to_host(r.d[k]).view(np.uint8), to_host(q.d[k]).view(np.uint8),
                                          err_msg=f"{k} after the restored step")
    q.compare(cmp, "step 4")
    print("  " + cmp.summary(), flush=True)
