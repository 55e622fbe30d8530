"""GPU parity at the five workload configurations, at their full sizes and in the
launch configuration the benchmark times.

The device runs every tensor in full; the oracle follows a sample of blocks (each
as a one-block tensor; blocks are independent) from the same generated inputs and
runs its own trajectory for the whole step count.  The 256x256 configuration is
checked in full.

  1. Adam 8-bit, 256x256 fp32, block 256, 10 steps (checked in full)
  2. AdamW 8-bit, 4096x4096, fp32 and fp16, blocks 256 and 2048, wd 0.01, 20 steps
  3. AdEMAMix 8-bit, 4096x4096 bf16, alpha 5, t_alpha = t_beta3 = 100, 200 steps
  4. Momentum and Lion 8-bit, 50257x1024 fp16 embedding, 70% zero gradient rows,
     wd 0.01, skip_zeros on and off, 10 steps
  5. GPT-style 1.3B parameter set (146 8-bit bf16 tensors, 146 32-bit fp32 tensors
     below 4096 elements), one multi-tensor Adam step
  and the 1-state RMSprop and Adagrad on the 4096x4096 shape (fp32, bf16), 20 steps.
"""
import numpy as np
import pytest
import torch

from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, SampledTensor, sample_blocks, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _run_single(wl, nsample=48, check_every=1, extra_blocks=()):
    t = wl.tensors[0]
    n, dtype, B = t.numel, t.dtype, wl.hp["blocksize"]
    nb = (n + B - 1) // B
    blocks = np.arange(nb) if nsample is None else sample_blocks(nb, nsample, wl.seed, extra_blocks)
    print(f"\n[config] {wl.name}: n={n} steps={wl.steps} blocks checked={len(blocks)}/{nb}", flush=True)
    st = SampledTensor(wl.hp, n, dtype, blocks, wl.param(0))
    cmp = Compare()
    for step in range(1, wl.steps + 1):
        g = wl.grad(0, step)
        st.step_gpu(step, to_dev(g, dtype))
        st.step_oracle(step, g)
        if step % check_every == 0 or step == wl.steps:
            st.compare(cmp, f"step {step}")
    print("  " + cmp.summary(), flush=True)
    return cmp


def test_config1_adam_256x256_full():
    cmp = _run_single(W.c1_adam_256(), nsample=None)
    assert cmp.code_elems > 0


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_config2_adamw_4096(dtype, bs):
    _run_single(W.c2_adamw_4096(dtype, bs))


def test_config3_ademamix_4096_bf16_200_steps():
    _run_single(W.c3_ademamix_4096(), nsample=32, check_every=10)


@pytest.mark.parametrize("skip", [True, False])
@pytest.mark.parametrize("opt", ["momentum", "lion"])
def test_config4_embedding_fp16(opt, skip):
    wl = W.c4_embedding(opt, skip)
    # blocks of rows that are zero at step 1 and of rows that are not
    rows = wl.tensors[0].shape[0]
    mask = W.zero_row_mask([wl.seed, 3, 0, 1], rows, wl.zero_row_frac)
    zr, nzr = np.nonzero(mask)[0][:8], np.nonzero(~mask)[0][:8]
    extra = np.concatenate([zr * 4, nzr * 4 + 1])          # 1024 columns = 4 blocks of 256 per row
    _run_single(wl, nsample=48, extra_blocks=extra)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opt", ["rmsprop", "adagrad"])
def test_one_state_rmsprop_adagrad_4096(opt, dtype):
    _run_single(W.f2_one_state_4096(opt, dtype))


def test_config5_gpt_1p3b_multi_tensor():
    wl = W.c5_gpt_1p3b()
    hp = wl.hp
    B = hp["blocksize"]
    print(f"\n[config] {wl.name}: {len(wl.tensors)} tensors, "
          f"{sum(t.numel for t in wl.tensors)} parameters, 1 multi-tensor step", flush=True)
    sampled = {"wte", "wpe", "h0.attn.qkv.w", "h5.attn.qkv.b", "h11.mlp.fc.w", "h23.mlp.fc2.w", "h23.mlp.fc.b"}
    sts, descs, grads = [], [], []
    for i, t in enumerate(wl.tensors):
        n = t.numel
        nb = (n + B - 1) // B
        if not t.eightbit:
            blocks = np.arange(nb)                         # small 32-bit tensors: checked in full
        elif t.name in sampled:
            blocks = sample_blocks(nb, 16, wl.seed + i)
        else:
            blocks = []
        st = SampledTensor(hp, n, t.dtype, blocks, wl.param(i), eight=t.eightbit)
        g = wl.grad(i, 1)
        gd = to_dev(g, t.dtype)
        sts.append(st)
        grads.append(g if len(st.blocks) else None)
        descs.append(st.desc(gd))
    q1, q2 = SampledTensor.qdev()
    bitopt.step_multi(hp, 1, descs, q1, q2)
    cmp = Compare()
    for st, g in zip(sts, grads):
        if g is not None:
            st.step_oracle(1, g)
            st.compare(cmp, "step 1")
    print("  " + cmp.summary(), flush=True)
    assert cmp.code_elems > 0
