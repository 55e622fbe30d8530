"""A tensor of more than 2^31 elements: 64-bit element, block and tile indexing.

The inputs are drawn on the device by torch's seeded generator (not by the library
under test); the oracle follows sampled blocks -- the first ones, those around
element 2^31, random ones and the ragged last block -- each as a one-block tensor
started from the device's pre-step state of that block (blocks are independent).
About 22 GB of device memory."""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from parity import Compare, as_f32, param_rtol, to_host

pytestmark = pytest.mark.gpu

N = 2 ** 31 + 3 * 256 + 77
B = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 32 * 2 ** 30:
        pytest.skip("needs 32 GiB of free device memory")
    bitopt.lib()


def _blocks(nb):
    mid = 2 ** 31 // B
    rng = np.random.default_rng(77)
    picks = {0, 1, mid - 2, mid - 1, mid, mid + 1, nb - 2, nb - 1}
    picks.update(int(b) for b in rng.integers(0, nb, 24))
    return sorted(picks)


def _slice(t, b, n=N):
    return t[b * B:min((b + 1) * B, n)]


def test_adam_step_beyond_2pow31_elements():
    nb = (N + B - 1) // B
    hp = dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, blocksize=B)
    print(f"\n[large] adam bf16 n={N} blocks={nb}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    p = (torch.randn(N, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    s1 = torch.zeros(N, dtype=torch.uint8, device="cuda")
    s2 = torch.zeros(N, dtype=torch.uint8, device="cuda")
    a1 = torch.zeros(nb, device="cuda")
    a2 = torch.zeros(nb, device="cuda")
    q1 = bitopt.create_dynamic_map(True).cuda()
    q2 = bitopt.create_dynamic_map(False).cuda()
    qh1, qh2 = oracle.dynamic_map(True), oracle.dynamic_map(False)
    blocks = _blocks(nb)
    cmp = Compare()
    for t in (1, 2):
        g = (torch.randn(N, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
        torch.cuda.synchronize()
        pre = {b: dict(p=to_host(_slice(p, b)).copy(), g=to_host(_slice(g, b)).copy(),
                       s1=to_host(_slice(s1, b)).copy(), s2=to_host(_slice(s2, b)).copy(),
                       a1=to_host(a1[b:b + 1]).copy(), a2=to_host(a2[b:b + 1]).copy()) for b in blocks}
        bitopt.step_8bit_blockwise_2state(hp, t, p, g, s1, s2, a1, a2, q1, q2)
        torch.cuda.synchronize()
        del g
        for b in blocks:
            o = pre[b]
            oracle.step_8bit(hp, t, o["p"], o["g"], "bf16", o["s1"], o["a1"], qh1, o["s2"], o["a2"], qh2)
            cmp.codes(to_host(_slice(s1, b)), o["s1"], f"step {t} block {b} state1")
            cmp.codes(to_host(_slice(s2, b)), o["s2"], f"step {t} block {b} state2")
            cmp.values(to_host(a1[b:b + 1]), o["a1"], param_rtol("bf16"), f"step {t} block {b} absmax1", kind="a")
            cmp.values(to_host(a2[b:b + 1]), o["a2"], param_rtol("bf16"), f"step {t} block {b} absmax2", kind="a")
            cmp.values(as_f32(to_host(_slice(p, b)), "bf16"), as_f32(o["p"], "bf16"), param_rtol("bf16"),
                       f"step {t} block {b} p")
    print("  " + cmp.summary(), flush=True)
    # the codec on the same tensor: quantize the parameters, compare sampled blocks
    codes, absmax = bitopt.quantize_blockwise(p, q1, B)
    torch.cuda.synchronize()
    for b in blocks:
        c_ref, a_ref = oracle.quantize_blockwise(to_host(_slice(p, b)).copy(), "bf16", qh1, B)
        np.testing.assert_array_equal(to_host(_slice(codes, b)), c_ref, err_msg=f"codec block {b}")
        np.testing.assert_array_equal(to_host(absmax[b:b + 1]), a_ref, err_msg=f"codec absmax {b}")
