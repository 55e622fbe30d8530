"""Seeded random configurations of the block-wise 8-bit step against the oracle:
optimizer, parameter dtype, block size, size (ragged), hyper-parameters drawn over
their valid ranges, skip_zeros with scattered zero gradients, max_unorm, gradient
scale and, for some, a misaligned parameter buffer.  Three steps each, compared
after every step to the same bar as the other parity tests."""
import numpy as np
import pytest
import torch

from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, Quant8, to_dev

pytestmark = pytest.mark.gpu

OPTIMIZERS = ["adam", "ademamix", "momentum", "lion", "rmsprop", "adagrad"]
DTYPES = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _config(seed):
    rng = np.random.default_rng([31337, seed])
    opt = OPTIMIZERS[seed % len(OPTIMIZERS)]
    dtype = DTYPES[(seed // len(OPTIMIZERS)) % len(DTYPES)]
    B = int(rng.choice([256, 2048]))
    n = int(rng.integers(1, 12 * B))
    hp = dict(optimizer=opt, blocksize=B,
              lr=float(10 ** rng.uniform(-5, -1.5)),
              eps=float(10 ** rng.uniform(-10, -6)),
              weight_decay=float(rng.choice([0.0, 10 ** rng.uniform(-4, -1)])),
              skip_zeros=bool(rng.random() < 0.4),
              max_unorm=float(rng.choice([0.0, 10 ** rng.uniform(-3, 0)])))
    if opt in ("adam", "ademamix"):
        hp.update(beta1=float(rng.uniform(0.5, 0.99)), beta2=float(rng.uniform(0.9, 0.9999)))
    if opt == "ademamix":
        hp.update(beta3=float(rng.uniform(0.99, 0.99999)), alpha=float(rng.uniform(0, 10)),
                  t_alpha=int(rng.choice([0, 2, 50])), t_beta3=int(rng.choice([0, 3, 50])))
    if opt == "momentum":
        hp.update(beta1=float(rng.uniform(0.0, 0.99)))
    if opt == "lion":
        hp.update(beta1=float(rng.uniform(0.5, 0.99)), beta2=float(rng.uniform(0.9, 0.999)))
    if opt == "rmsprop":
        hp.update(beta1=float(rng.uniform(0.5, 0.999)))
    gscale = float(10 ** rng.uniform(-4, 0))
    zero_frac = float(rng.uniform(0.05, 0.6)) if hp["skip_zeros"] else 0.0
    misaligned = bool(rng.random() < 0.25)
    return hp, dtype, n, gscale, zero_frac, misaligned


@pytest.mark.parametrize("seed", range(36))
def test_random_config(seed):
    hp, dtype, n, gscale, zero_frac, misaligned = _config(seed)
    print(f"\n[random {seed}] {dtype} n={n} misaligned={misaligned} gscale={gscale:.2e} zero_frac={zero_frac:.2f} "
          f"hp={hp}", flush=True)
    p0 = W.to_dtype(W.normal_f32([seed, 9, 1], n, 0.02), dtype)
    q = Quant8(hp, p0, dtype)
    if misaligned:
        big = torch.zeros(n + 1, dtype=q.d["p"].dtype, device="cuda")
        big[1:].copy_(q.d["p"])
        q.d["p"] = big[1:]
    rng = np.random.default_rng([seed, 9, 3])
    cmp = Compare()
    for t in (1, 2, 3):
        g = W.normal_f32([seed, 9, 2, t], n, gscale)
        if zero_frac:
            g[rng.random(n) < zero_frac] = 0.0
        g = W.to_dtype(g, dtype)
        q.step_gpu(t, to_dev(g, dtype))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print("  " + cmp.summary(), flush=True)
