"""GPU parity of the non-block-wise (tensor-wide) 8-bit step: one absmax per state
for the whole tensor, two passes on the device.  The oracle runs the same step as
one block spanning the tensor (blocksize 0).  Bar as for the block-wise step."""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, as_f32, param_rtol, to_dev, to_host

pytestmark = pytest.mark.gpu

OPTS = {
    "adam": dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    "ademamix": dict(optimizer="ademamix", lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0,
                     t_alpha=3, t_beta3=3, eps=1e-8, weight_decay=0.01),
    "momentum": dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01),
    "lion": dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01),
    "rmsprop": dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8, weight_decay=0.01),
    "adagrad": dict(optimizer="adagrad", lr=0.01, eps=1e-10, weight_decay=0.01),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


class TW8:
    def __init__(self, hp, p0, dtype, maps=None):
        self.hp = dict(hp, blocksize=0)
        self.dtype = dtype
        n = self.n = p0.size
        opt = hp["optimizer"]
        k = 2 if opt == "ademamix" else 1
        self.two = oracle.NUM_STATES[opt] >= 2
        q1 = oracle.dynamic_map(opt not in oracle.UNSIGNED_STATE1)
        q2 = oracle.dynamic_map(False)
        if maps is not None:
            q1, q2 = maps
        self.o = dict(p=p0.copy(), s1=np.zeros(k * n, np.uint8), a1=np.zeros(k, np.float32),
                      s2=np.zeros(n, np.uint8) if self.two else None,
                      a2=np.zeros(1, np.float32) if self.two else None, q1=q1, q2=q2)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.d = dict(p=to_dev(p0, dtype), s1=dev(self.o["s1"]), a1=dev(self.o["a1"]), q1=dev(q1),
                      s2=dev(self.o["s2"]) if self.two else None, a2=dev(self.o["a2"]) if self.two else None,
                      q2=dev(q2) if self.two else None)
        self.ws = None

    def step_gpu(self, t, g_dev):
        d = self.d
        self.ws = bitopt.step_8bit_tensorwise(self.hp, t, d["p"], g_dev, d["s1"], d["a1"], d["q1"],
                                              d["s2"], d["a2"], d["q2"], workspace=self.ws)

    def step_oracle(self, t, g):
        o = self.o
        oracle.step_8bit(self.hp, t, o["p"], g, self.dtype, o["s1"], o["a1"], o["q1"],
                         o["s2"], o["a2"], o["q2"] if self.two else None)

    def compare(self, cmp, what):
        torch.cuda.synchronize()
        d, o = self.d, self.o
        cmp.codes(to_host(d["s1"]), o["s1"], what + " state1")
        cmp.values(to_host(d["a1"]), o["a1"], param_rtol(self.dtype), what + " absmax1", kind="a")
        if self.two:
            cmp.codes(to_host(d["s2"]), o["s2"], what + " state2")
            cmp.values(to_host(d["a2"]), o["a2"], param_rtol(self.dtype), what + " absmax2", kind="a")
        cmp.values(as_f32(to_host(d["p"], self.dtype), self.dtype), as_f32(o["p"], self.dtype),
                   param_rtol(self.dtype), what + " p")


def _grad(seed, t, n, dtype, zero_frac=0.0):
    g = W.normal_f32([seed, 2, t], n, 0.01)
    if zero_frac:
        rng = np.random.default_rng([seed, t])
        g[rng.random(n) < zero_frac] = 0.0
    return W.to_dtype(g, dtype)


def _run(name, n, dtype, steps, seed, zero_frac=0.0, maps=None, skip=False, max_unorm=0.0):
    hp = dict(OPTS[name], skip_zeros=skip, max_unorm=max_unorm)
    print(f"\n[tensorwise] {name} {dtype} n={n} steps={steps} skip={skip} max_unorm={max_unorm}", flush=True)
    q = TW8(hp, W.to_dtype(W.normal_f32([seed, 1], n, 0.02), dtype), dtype, maps)
    cmp = Compare()
    for t in range(1, steps + 1):
        g = _grad(seed, t, n, dtype, zero_frac)
        q.step_gpu(t, to_dev(g, dtype))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print("  " + cmp.summary(), flush=True)
    return q


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_tensorwise_step(name, dtype):
    _run(name, 5 * 1024 + 300 + 5 if name != "ademamix" else 5 * 1024 + 304, dtype, 4, 1100)


@pytest.mark.parametrize("name", list(OPTS))
def test_tensorwise_skip_zeros(name):
    _run(name, 3 * 1024 + 77 if name != "ademamix" else 3 * 1024 + 80, "f16", 3, 1200, zero_frac=0.3, skip=True)


@pytest.mark.parametrize("name", list(OPTS))
def test_tensorwise_max_unorm(name):
    """A cap of 0.002 clips every optimizer's first steps here; the clip factor comes
    from norms over the whole tensor."""
    _run(name, 5 * 1024 + 300 + 5 if name != "ademamix" else 5 * 1024 + 304, "f32", 3, 1700, max_unorm=0.002)


def test_tensorwise_max_unorm_skip_f16_and_off():
    _run("adam", 3 * 1024 + 77, "f16", 3, 1710, zero_frac=0.3, skip=True, max_unorm=0.002)
    _run("momentum", 2 * 1024 + 5, "f32", 2, 1720, max_unorm=1e30)      # a cap never reached


def test_tensorwise_max_unorm_many_groups():
    """More tiles than pass-1 groups (each group strides over several tiles) and a
    ragged tail: the partial sums of every group reach the clip factor."""
    _run("adam", 4100 * 1024 + 3, "f32", 1, 1730, max_unorm=0.002)


def test_tensorwise_skip_all_zero_is_noop():
    n = 4096
    q = _run("momentum", n, "f32", 2, 1310)
    q.hp["skip_zeros"] = True
    snap = {k: to_host(v).copy() for k, v in q.d.items() if v is not None}
    q.step_gpu(3, torch.zeros(n, device="cuda"))
    torch.cuda.synchronize()
    for k, v in q.d.items():
        if v is not None:
            np.testing.assert_array_equal(to_host(v), snap[k])


def test_tensorwise_custom_maps_and_unaligned():
    qs = oracle.dynamic_map(True).astype(np.float64)
    rng = np.random.default_rng(3)
    inner = (qs != 0) & (np.abs(qs) != 1)
    qs[inner] *= 1 + 2e-3 * rng.uniform(-1, 1, int(inner.sum()))
    qs = np.sort(qs).astype(np.float32)
    _run("adam", 4 * 1024 + 9, "f32", 3, 1400, maps=(qs, oracle.dynamic_map(False)))
    # misaligned buffers: element-wise path
    n = 2 * 1024 + 33
    hp = dict(OPTS["lion"])
    p0 = W.to_dtype(W.normal_f32([1500, 1], n, 0.02), "bf16")
    q = TW8(hp, p0, "bf16")
    big = torch.zeros(n + 1, dtype=q.d["p"].dtype, device="cuda")
    big[1:].copy_(q.d["p"])
    q.d["p"] = big[1:]
    cmp = Compare()
    for t in range(1, 4):
        g = _grad(1500, t, n, "bf16")
        q.step_gpu(t, to_dev(g, "bf16"))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print("\n[tensorwise unaligned] " + cmp.summary())


def test_tensorwise_4096_squared_fp32():
    """The 4096x4096 shape: the oracle steps the whole tensor as one block."""
    _run("adam", 4096 * 4096, "f32", 2, 1600)
